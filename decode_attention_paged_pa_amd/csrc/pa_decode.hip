// Decode-phase kernels: page-tag validation, split-K attention over pages,
// and the reduce that merges the token partitions.
//
// The decode step revisits every cached K/V token of each sequence ("How we
// built the most efficient inference engine for Cloudflare's network",
// section "Batching to feed the Tensor Cores"), so the attention kernel is a
// stream over the cache: it must move the KV bytes once, at HBM speed.  The
// grouped queries of one KV head (G <= 16) form the N side of 16x16 MFMA
// tiles, the only dense contraction on this path:
//   S^T[t][g] = sum_d K[t][d] Q[g][d]      (mfma 16x16x32 bf16, A = K page)
//   O^T[d][g] += sum_t V^T[d][t] P^T[t][g] (mfma 16x16x16, A = V^T page)
// With this orientation the score tile that comes out of the first MFMA is
// already the B operand of the second, and each lane owns the softmax state
// of exactly one query column, so no data crosses lanes except two swaps per
// page for the column maximum.
#include "pa_block.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// A page maximum may exceed the running maximum by this many log2 units
// before the accumulators are rescaled; weights stay below 2^8, which fp32
// sums and f16/bf16 MFMA operands hold without loss of range.
constexpr float kRescaleSlack = 8.0f;

// FP8 P.V operands are f16: p * (v_scale / v_ref) * kPScale, where v_ref is
// the largest V scale the wave has met so far in its run.  The factor is at
// most 1 and p at most 2^8, so the operand stays below 2^15, inside f16's
// range (65504) whatever the cache's magnitudes, and weights down to 2^-21
// of the largest keep f16's full precision.  O then accumulates in units of
// v_ref / kPScale, and is converted when partials or outputs are written.
constexpr float kPScale = 128.0f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int N> struct IntC { static constexpr int value = N; };   // a compile-time int argument

// Max of four scores that are never NaN (masked ones are -inf), in two
// v_max3_f32.  Written out because fmaxf must quiet NaN inputs first: the
// compiler adds a canonicalising max for each operand it cannot prove
// canonical (all of them after the causal mask's select).
__device__ inline float max4(float a, float b, float c, float d) {
  float t, r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(t) : "v"(a), "v"(b), "v"(c));
  asm("v_max3_f32 %0, %1, %2, %2" : "=v"(r) : "v"(t), "v"(d));
  return r;
}

// Tuning knobs (fixed at build time; the defaults are the measured best).
#ifndef PA_PIPE_DEPTH
#define PA_PIPE_DEPTH 2        // pages held in registers per wave (loads in flight + current)
#endif
#ifndef PA_NT_LOADS
#define PA_NT_LOADS 1          // KV loads marked non-temporal (streamed once)
#endif
#ifndef PA_THROTTLE
#define PA_THROTTLE 1          // each wave waits for its loads before requesting the next page
#endif
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 4      // occupancy hint for the register allocator (0: none)
#endif
#ifndef PA_VAL_PER
#define PA_VAL_PER 8           // table entries per validation thread whose loads are issued together
#endif
// Kernels with several query-column tiles: measured on MI355X, deeper rings
// and dropping the throttle change nothing with two tiles (their time goes to
// compute and to the lower occupancy), so those keep the same defaults; the
// four-tile kernels hold one K buffer instead (PA_MQ_LATE_K), where the
// compiler places the waits.
#ifndef PA_MQ_PIPE_DEPTH
#define PA_MQ_PIPE_DEPTH 2
#endif
#ifndef PA_MQ_THROTTLE
#define PA_MQ_THROTTLE 1
#endif
#ifndef PA_MQ_LATE_K
#define PA_MQ_LATE_K 1         // 4 tiles: one K buffer, next page requested after Q.K
#endif
#ifndef PA_QK_SCHED
#define PA_QK_SCHED 4          // two tiles: Q reads kept this far ahead of Q.K (0: compiler's order)
#endif
#ifndef PA_QK_SCHED4
#define PA_QK_SCHED4 8         // four tiles: the same
#endif
#ifndef PA_IDREGS4
#define PA_IDREGS4 2           // four tiles, BF16: page-id registers (64 pages each)
#endif
#ifndef PA_RED_THREADS
#define PA_RED_THREADS 64      // threads per reduce workgroup (D/4 per query row)
#endif
#ifndef PA_MQ_WAVES2
#define PA_MQ_WAVES2 0         // occupancy hint with 2 column tiles (0: derived below)
#endif
#ifndef PA_MQ_WAVES4
#define PA_MQ_WAVES4 2         // occupancy hint with 4 column tiles
#endif
#ifndef PA_SHARED_WAVES
#define PA_SHARED_WAVES 3      // occupancy hint of the page-sharing kernel
#endif
#ifndef PA_SHARED_STAGES
#define PA_SHARED_STAGES 4     // LDS pages of the page-sharing BF16 kernel's ring (3 in flight)
#endif
static_assert(PA_SHARED_STAGES == 2 || PA_SHARED_STAGES == 4,
              "page-sharing ring: whole ring cycles per 64-page id chunk, within the LDS");
#ifndef PA_SHARED_STAGES_FP8
#define PA_SHARED_STAGES_FP8 4 // FP8 pages of the page-sharing kernel's ring
#endif
#ifndef PA_SHARED_LEAD_FP8
#define PA_SHARED_LEAD_FP8 3   // FP8 pages requested ahead of the one being widened
#endif
static_assert((PA_SHARED_STAGES_FP8 == 4 || PA_SHARED_STAGES_FP8 == 8) &&
              PA_SHARED_LEAD_FP8 >= 1 && PA_SHARED_LEAD_FP8 <= PA_SHARED_STAGES_FP8 - 1,
              "page-sharing FP8 ring: whole ring cycles per 64-page id chunk; a stage is widened before it is reused");
// Word 3 of a raw buffer resource on CDNA: 32-bit data format (any nonzero
// format enables the access; untyped loads ignore it), no swizzle.
constexpr int kBufWord3 = 0x00020000;

// One 1 KiB block from global memory straight into LDS: lane l fetches the
// 16 bytes at src + voff (voff < 1024; the buffer's bounds return zeros past
// the block) and they land at LDS byte lds + 16 l.  Written in asm so that
// the compiler does not track it: its own tracking loses, at a loop's back
// edge, which LDS buffer each load in flight writes, and then waits for every
// load before the loop's first LDS read.  The caller orders the loads
// against the LDS reads itself (s_waitcnt vmcnt, then a barrier).  The asm
// has no destination register; M0 (the LDS base) is restored before it ends,
// and the s_nop is the wait state an M0 write needs before an LDS-DMA load.
__device__ inline void dma_block(const uint8_t* src, uint32_t lds, int voff) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t p = reinterpret_cast<uint64_t>(src);
  const i32x4 rs{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xFFFFu), 1024, kBufWord3};
  int keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds), "v"(voff), "s"(rs)
      : "memory");
}
constexpr int kPipe = PA_PIPE_DEPTH;
static_assert(kPipe == 2 || kPipe == 4, "pipeline depth: whole ring cycles per 64-page id chunk");
static_assert(PA_MQ_PIPE_DEPTH == 2 || PA_MQ_PIPE_DEPTH == 4, "pipeline depth: whole ring cycles per 64-page id chunk");

// BF16 pages hold twice the bytes in the register ring, so that kernel gets
// one wave per SIMD less than the FP8 one instead of spilling; every extra
// tile of query columns adds its O accumulators and Q operands (D/2 + D/4
// registers per lane at D = 128... 48 + 16 at D = 64), paid for in waves.
template <bool FP8, int NQ, bool SHARED = false>
constexpr int waves_per_eu() {
  return SHARED ? PA_SHARED_WAVES
       : NQ == 1 ? (FP8 ? PA_WAVES_PER_EU : PA_WAVES_PER_EU - 1)
       : NQ == 2 ? (PA_MQ_WAVES2 > 0 ? PA_MQ_WAVES2
                                     : (FP8 ? PA_WAVES_PER_EU - 1 : PA_WAVES_PER_EU - 2))
                 : PA_MQ_WAVES4;
}
#if PA_WAVES_PER_EU > 0
#define PA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(waves_per_eu<FP8, NQ, SHARED>())))
#else
#define PA_OCCUPANCY
#endif

__device__ inline u32x4 load16(const uint8_t* p) {
#if PA_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

// 16 bytes at blk + soff + voff, through a buffer resource over the block:
// blk and soff are uniform (scalar registers) and voff is the lane's offset,
// so the address costs no vector instructions.  bytes bounds the access
// (reads past it return zeros).
__device__ inline u32x4 load_blk(const uint8_t* blk, int bytes, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), (short)0, bytes, kBufWord3);
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, PA_NT_LOADS ? 2 : 0));
}

// ------------------------------------------------------------ validation
// Integrity check of the pages a decode will read ("Cloudflare quantizes
// Kimi and GLM caches for 41% faster inference", integrity-check paragraph:
// a separate batch validation before decode reads).  One workgroup per
// sequence writes its flags word; in the HEAD layout with per_unit, one
// workgroup per unit writes a word per unit instead, and the decode ORs a
// sequence's words (a HEAD sequence has Hkv tables of up to table_width
// entries each: spread over Hkv workgroups the check takes one pass, where a
// workgroup per sequence took several, measured 4.5% of the headwise step).
// The table entries of the workgroup's units form one flat index space, 8
// entries per thread per pass with every load of a pass issued before any is
// used: two dependent round trips per 8192 entries.
constexpr int kValUnits = 64;   // units whose entry offsets are held at a time

__device__ void validate_block(const ValidateArgs& a, int x) {
  const int b = a.per_unit ? x / a.num_kv_heads : x;
  const int unit_base = a.per_unit ? x : b * a.num_kv_heads;   // HEAD: first unit
  __shared__ uint32_t s_bits;
  __shared__ int s_off[kValUnits + 1];
  const int tid = threadIdx.x;
  if (tid == 0) s_bits = 0;
  uint32_t bits = 0;
  const int cap = a.table_width * kPageSize;
  const int n_units = (a.head_layout && !a.per_unit) ? a.num_kv_heads : 1;
  for (int u0 = 0; u0 < n_units; u0 += kValUnits) {
    const int nu = min(kValUnits, n_units - u0);
    if (tid < nu) {
      const int row = a.head_layout ? unit_base + u0 + tid : b;
      int L = a.lens[row];
      if (L > cap || L < 0) bits |= 4u;
      L = L < 0 ? 0 : (L > cap ? cap : L);
      s_off[tid + 1] = (L + kPageSize - 1) / kPageSize;
    }
    __syncthreads();
    if (tid == 0) {
      s_off[0] = 0;
      for (int i = 1; i <= nu; ++i) s_off[i] += s_off[i - 1];
    }
    __syncthreads();
    const int total = s_off[nu];
    constexpr int kPer = PA_VAL_PER;
    // With up to 8 units the offsets sit in registers and an entry's unit is a
    // count of compares; more units search the LDS copy.
    constexpr int kRegUnits = 8;
    int offr[kRegUnits + 1];
#pragma unroll
    for (int k = 0; k <= kRegUnits; ++k) offr[k] = k <= nu ? s_off[k] : INT_MAX;
    auto unit_of = [&](int i) {
      int u = 0;
      if (nu <= kRegUnits) {
#pragma unroll
        for (int k = 1; k <= kRegUnits; ++k) u += offr[k] <= i ? 1 : 0;
      } else {
        while (s_off[u + 1] <= i) ++u;
      }
      return u;
    };
    for (int base = 0; base < total; base += kPer * 1024) {
      int pid[kPer];
      uint32_t want[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = base + j * 1024 + tid;
        pid[j] = 0;
        want[j] = 0u;
        if (i < total) {
          const int u = unit_of(i);               // the unit holding flat entry i
          const int row = a.head_layout ? unit_base + u0 + u : b;
          const size_t e = (size_t)row * a.table_width + (i - s_off[u]);
          pid[j] = a.block_table[e];
          if (a.expected_tags) want[j] = a.expected_tags[e];
        }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (base + j * 1024 + tid >= total) continue;
        if ((unsigned)pid[j] >= (unsigned)a.num_pages) {
          bits |= 2u;
        } else if (a.expected_tags && want[j] != a.page_tags[pid[j]]) {
          bits |= 1u;
        }
      }
    }
    __syncthreads();   // s_off is rewritten by the next group of units
  }
  if (bits) atomicOr(&s_bits, bits);  // LDS atomic
  __syncthreads();
  if (tid == 0) a.flags[x] = s_bits;
}

// ----------------------------------------------------------------- plan
// Length-balanced split of the automatic decode: one chunk size for the whole
// batch, chosen from the real lengths, and group g (a sequence, or a unit in
// the HEAD layout) gets ceil(pages_g / chunk) partitions of its pages.  The
// chunk is the smallest (at least min_chunk) for which the partitions, each
// last one of a group rounded up, make at most target_waves waves: every
// wave then has at most `chunk` pages, and no compute unit holds more waves
// than the rest.  With fixed partitions a ragged batch leaves only its
// longest units' waves running at the end (measured: 56-72% of 8 TB/s against
// 82-85% for the same kernels on uniform lengths), and a wave count just
// above target_waves leaves a few compute units with a third wave per SIMD.
// One workgroup; the partition counts are then scanned 1024 groups at a time.
__device__ inline int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

constexpr int kPlanCache = 4096;   // groups whose page counts the planner keeps in LDS

__device__ void plan_block(const PlanArgs& a) {
  __shared__ int s_np[kPlanCache];
  __shared__ long long s_part[2][16];
  __shared__ int s_wave[16];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  if (a.plan == nullptr || a.plan_group == nullptr) return;   // no plan asked of this workgroup
  const int n = a.num_groups;
  const int cap = a.table_width * kPageSize;
  auto pages = [&](int g) {
    int L = a.lens[g];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    return (L + kPageSize - 1) / kPageSize;
  };
  for (int g = tid; g < n && g < kPlanCache; g += 1024) s_np[g] = pages(g);
  if (tid == 0) s_carry = 0;
  __syncthreads();
  auto np_of = [&](int g) { return g < kPlanCache ? s_np[g] : pages(g); };
  // block-wide sum of f(group); double-buffered, one barrier per call
  int buf = 0;
  auto block_sum = [&](auto f) {
    long long v = 0;
    for (int g = tid; g < n; g += 1024) v += f(np_of(g));
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
    if (lane == 0) s_part[buf][wv] = v;
    __syncthreads();
    long long t = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += s_part[buf][i];
    buf ^= 1;
    return t;
  };
  const long long total = block_sum([](int p) { return p; });   // pages of all groups
  const long long hpg = a.heads_per_group, target = a.target_waves;
  const long long W = min(a.max_chunk, a.table_width);   // the largest chunk allowed
  // The smallest chunk in [lo, hi] whose waves fit the target, where lo is
  // the bound from the page total alone and hi fits for sure: pairs <=
  // total / c + groups, so hi = ceil(total / (target / hpg - groups)) (or
  // the whole table).  Each pass, wave w tests candidate lo + (hi - lo) * w / 16
  // on its own (lanes stride over the groups, sums saturate above the
  // target) and the range shrinks to the gap below the first one that fits.
  long long lo = (total * hpg + target - 1) / target;
  if (lo < a.min_chunk) lo = a.min_chunk;
  if (lo > W) lo = W;
  const long long room = target / hpg - n;
  long long hi = room > 0 ? (total + room - 1) / room : W;
  if (hi > W) hi = W;
  if (hi < lo) hi = lo;
  const int cap_sum = (int)(target / hpg) + 1;   // pairs above this already fail
  while (lo < hi) {                               // uniform loop: invariant hi fits (or is W)
    const int c = (int)(lo + (hi - lo) * wv / 16);
    int v = 0;
    for (int g = lane; g < n && v < cap_sum; g += 64) v += (np_of(g) + c - 1) / c;
    v = min(v, cap_sum);
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d);
    if (lane == 0) s_part[buf][wv] = (long long)v * hpg <= target ? 1 : 0;
    __syncthreads();
    // the first candidate that fits (16 if none): all 16 flags read at once
    long long fit[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) fit[i] = s_part[buf][i];
    int w = 16;
#pragma unroll
    for (int i = 15; i >= 0; --i) w = fit[i] != 0 ? i : w;
    buf ^= 1;
    if (w == 0) {
      hi = lo;
    } else {
      const long long below = lo + (hi - lo) * (w - 1) / 16;   // candidate w - 1 fails
      if (w < 16) hi = lo + (hi - lo) * w / 16;
      lo = below + 1;
    }
  }
  const int chunk = (int)hi;
  int32_t* first = a.plan + 2;
  for (int base = 0; base < n; base += 1024) {
    const int g = base + tid;
    const int parts = g < n ? (np_of(g) + chunk - 1) / chunk : 0;
    const int incl = wave_incl_scan(parts, lane);
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    if (wv == 0) {
      const int x = lane < 16 ? s_wave[lane] : 0;
      const int xi = wave_incl_scan(x, lane);
      if (lane < 16) s_wave[lane] = xi - x;
    }
    __syncthreads();
    const int excl = s_carry + s_wave[wv] + incl - parts;
    if (g < n) {
      first[g] = excl;
      int L = a.lens[g];
      L = L < 0 ? 0 : (L > cap ? cap : L);
      for (int p = 0; p < parts && excl + p < a.max_pairs; ++p) {
        a.plan_group[excl + p] = g;
        if (a.plan_rec)
          *reinterpret_cast<int4*>(a.plan_rec + 4 * (excl + p)) = int4{g, p, chunk, L};
      }
    }
    __syncthreads();
    if (tid == 1023) s_carry = excl + parts;
    __syncthreads();
  }
  if (tid == 0) {
    a.plan[0] = chunk;
    a.plan[1] = min(s_carry, a.max_pairs);   // never clipped: max_pairs bounds the count
    first[n] = s_carry;
  }
  if (a.plan_rec)   // slots past the last pair: no work
    for (int p = s_carry + tid; p < a.max_pairs; p += 1024) a.plan_rec[4 * p] = -1;
}

// OR over the 64 lanes of a wave.
__device__ inline uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x |= (uint32_t)__shfl_xor((int)x, d, 64);
  return x;
}

// The validation and the plans share one launch: workgroups 0 .. nval - 1
// validate sequences, and one more per plan asked for (the decode's split,
// the score pass's split) plans; the plans read only the lengths, so they run
// beside the validation.
__global__ __launch_bounds__(1024) void prep_kernel(ValidateArgs v, PlanArgs p0, PlanArgs p1,
                                                    int nval) {
  const int x = blockIdx.x;
  if (x < nval) validate_block(v, x);
  else plan_block(x == nval ? p0 : p1);
}

// A decode step's append in the same launch as its validation and plan: the
// append writes only pages and scales, which neither of them reads, and the
// attention launch that follows sees all three.  Workgroups past the
// validation and plan ones carry four append items each, one per 256 threads.
template <int D, bool FP8>
__global__ __launch_bounds__(1024) void step_prep_kernel(AppendArgs ap, int items,
                                                         ValidateArgs v, PlanArgs p0,
                                                         PlanArgs p1, int nval, int nplan) {
  __shared__ float s_red[4][2][4];
  __shared__ float s_old[4][2];
  const int x = blockIdx.x;
  if (x < nval) {
    validate_block(v, x);
  } else if (x < nval + nplan) {
    plan_block(x == nval ? p0 : p1);
  } else {
    const int qt = threadIdx.x >> 8;
    const int item = (x - nval - nplan) * 4 + qt;
    append_item<D, FP8, 256, false>(ap, item, item < items, threadIdx.x & 255, s_red[qt], s_old[qt]);
  }
}

// ------------------------------------------------------------- attention
// One wave owns one work item = (unit, partition), unit = (sequence, KV
// head), partition = a run of chunk_pages pages of the unit.  The four waves
// of a workgroup are independent (no LDS ring, no barrier): each streams its
// pages through a register ring and writes its own partial (max, sum, O) --
// or, with a single partition, the normalised output -- straight from
// registers.  The exception is the prefill kernel (SHARED): its four waves
// are 32-column blocks of one unit that load each page once, into an LDS
// ring, with a barrier per page (see the page loop).
//
// Query columns: the G query heads of the unit for each of its T query
// tokens, column cc = t * G + g, in NQ tiles of 16.  T > 1 is a multi-query
// step (speculative verification: the drafts are checked in one pass, "Making
// Workers AI faster and more efficient", speculative decoding section): token
// t sits at position L - T + t and sees tokens 0 .. L - T + t, so CAUSAL masks
// the scores of the last page or two per column.  Every K and V fragment is
// converted once and multiplied into all NQ tiles.
//
// With a.row_ml set (scored decode), single-partition rows also keep their
// final (max, sum) there for the eviction score pass (mass_kernel below).
template <int D, bool FP8, bool HEAD, int NQ, bool CAUSAL, bool SHARED>
__global__ __launch_bounds__(256) PA_OCCUPANCY void attention_kernel(AttnArgs a) {
  constexpr int E = FP8 ? 1 : 2;               // bytes per cached element
  constexpr int BLOCK = kPageSize * D * E;     // bytes of one (page, head) block
  constexpr int NSEG = BLOCK / 1024;           // 16-byte loads per lane per block
  constexpr int NT = D / 16;                   // 16-dim output tiles
  constexpr int NSTEP = D / 32;                // QK MFMA steps over d
  constexpr int PIPE = NQ == 1 ? kPipe : PA_MQ_PIPE_DEPTH;
  constexpr bool THROTTLE = NQ == 1 ? PA_THROTTLE : PA_MQ_THROTTLE;
  // Four-tile kernels (prefill, 8 drafts) hold one K buffer instead of two:
  // measured on MI355X, 4-5% faster there, 3% slower with two tiles.
  constexpr bool LATEK = NQ == 4 && PA_MQ_LATE_K;
  static_assert(!LATEK || PIPE == 2, "one K and two V buffers");
  // A wave streams at most two partitions (single-tile kernels only); the
  // state of the first is parked here (O, max, per-lane sum; one column per
  // lane) until the wave ends.
  constexpr int kStash = NQ == 1 ? 4 * NT + 2 : 1;
  __shared__ float s_stash[kWaves][kStash][64];
  // With several column tiles the Q operands live in LDS instead of
  // registers (D/8 registers per tile per lane otherwise): each lane reads
  // back only what it wrote itself, so no barrier is involved.  The
  // page-sharing kernel (SHARED, below) keeps its two tiles' Q in registers
  // and gives LDS to the pages.
  static_assert(!SHARED || (NQ == 2 && CAUSAL), "page sharing: prefill column blocks of 32");
  constexpr bool QLDS = NQ > 1 && !SHARED;
  __shared__ bf16x8 s_q[QLDS ? kWaves : 1][QLDS ? NQ * NSTEP : 1][64];
  // SHARED: a ring of pages (K then V, 1 KiB segments) for the workgroup,
  // one array per stage, so that the compiler tells the stages apart and
  // waits for a stage's loads only where that stage is read.
  constexpr int kStages = SHARED ? (FP8 ? PA_SHARED_STAGES_FP8 : PA_SHARED_STAGES) : 1;
  constexpr int kRingSegs = SHARED ? 2 * NSEG : 1;
  __shared__ u32x4 s_st0[kRingSegs][64], s_st1[kStages > 1 ? kRingSegs : 1][64],
      s_st2[kStages > 2 ? kRingSegs : 1][64], s_st3[kStages > 3 ? kRingSegs : 1][64],
      s_st4[kStages > 4 ? kRingSegs : 1][64], s_st5[kStages > 5 ? kRingSegs : 1][64],
      s_st6[kStages > 6 ? kRingSegs : 1][64], s_st7[kStages > 7 ? kRingSegs : 1][64];
  // SHARED with an FP8 cache (CVT): each wave widens the FP8 segments it
  // loaded, one page ahead, into the bf16 (K) and f16 (V) MFMA operands of
  // every lane, in one of two buffers; the waves then read operands that
  // need no conversion.  Per page: the 2 * NSEG operands of Q.K (one per
  // 32-dim step), then the 2 * NSEG of P.V (one per 32-dim block).
  constexpr bool CVT = SHARED && FP8;
  constexpr int NOP = CVT ? 2 * NSEG : NSEG;   // operand registers per K (or V) of a page
  __shared__ u32x4 s_cv0[CVT ? 2 * NOP : 1][64], s_cv1[CVT ? 2 * NOP : 1][64];

  const int Pn = a.num_parts;
  const bool planned = a.plan != nullptr;      // length-balanced split (see plan_block)
  const int ppw = (NQ == 1 && !planned) ? a.parts_per_wave : 1;
  const int groups = (Pn + ppw - 1) / ppw;     // waves per unit (fixed partitions)
  const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
  const int T = CAUSAL ? a.q_len : 1;
  const int C = G * T;                         // query columns of the unit
  // Long chunks (prefill) split a unit's columns into blocks of 16 * NQ (32:
  // the page-sharing kernel), one wave per block; a block reads (SHARED:
  // computes) only the pages its last column can see.
  const int cblocks = a.col_blocks;
  // readfirstlane: the wave index is uniform, and saying so keeps every
  // per-page index, bound and branch in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < kWaves);   // workgroups of kWaves waves (launch bound)
  int b, h, g, cb = 0;  // sequence, KV head, partition group, column block of this wave
  int chunk = a.chunk_pages;
  bool direct = Pn == 1;   // no reduce follows for this wave's unit: it writes the output rows
  int pslot = 0;           // planned: this wave's partial slot
  int planned_len = 0;     // planned: the group's length (clamped), from its record
  if (planned) {
    // One partition per pair, all of about the same size; the workgroup
    // order (XCD-aware for SEQ, as below) is the same, over the plan's pairs.
    const int hpg = HEAD ? 1 : Hkv;
    int pair, hh;
    if (a.xcd_order) {
      const int hgs = Hkv / kWaves;
      const int x = blockIdx.x;
      pair = (x / (8 * hgs)) * 8 + (x % 8);
      hh = ((x / 8) % hgs) * kWaves + wave;
    } else {
      const int item = blockIdx.x * kWaves + wave;
      pair = item / hpg;
      hh = item - pair * hpg;
    }
    if (pair >= a.max_pairs) return;
    const int4 rec = *reinterpret_cast<const int4*>(a.plan_rec + 4 * pair);
    const int grp = __builtin_amdgcn_readfirstlane(rec.x);
    if (grp < 0) return;
    g = __builtin_amdgcn_readfirstlane(rec.y);
    chunk = __builtin_amdgcn_readfirstlane(rec.z);
    planned_len = __builtin_amdgcn_readfirstlane(rec.w);
    direct = (planned_len + kPageSize - 1) / kPageSize <= chunk;   // the group's only partition
    b = HEAD ? grp / Hkv : grp;
    h = HEAD ? grp - b * Hkv : hh;
    pslot = pair * hpg + hh;
  } else if (a.xcd_order) {
    // Workgroups are dealt to the 8 XCDs in turn (id % 8).  A workgroup holds
    // 4 heads of one (sequence, partition group) pair, and the Hkv/4
    // workgroups of a pair get ids 8 apart -- same XCD, launched together --
    // so all heads of a page meet in one L2 (its scales, its table entries,
    // and the neighbouring head blocks of the SEQ layout).  Pairs are
    // numbered partition-major, so an XCD's share is spread over sequences
    // rather than tied to one partition index (late partitions of short
    // sequences are empty).
    const int hgs = Hkv / kWaves;               // head groups per pair
    const int x = blockIdx.x;
    const int pair = (x / (8 * hgs)) * 8 + (x % 8);
    const int hg = (x / 8) % hgs;
    if (pair >= a.batch * groups) return;
    g = pair / a.batch;
    b = pair - g * a.batch;
    h = hg * kWaves + wave;
  } else if (cblocks > 1) {
    // Prefill: every column block of a unit reads the same pages, so all of
    // a unit's waves go to one XCD (workgroups are dealt to the 8 XCDs in
    // turn, id % 8), where they walk its pages together through one L2.
    // Dealt across XCDs instead, each L2 saw every unit and hit 43% of its
    // requests (measured on the 2048-token chunk).  Within a unit the blocks
    // that see the most pages start first.
    // SHARED: a workgroup is kWaves consecutive column blocks of one (unit,
    // partition group), and all its waves stay to the end (they share the
    // page loads and a barrier per page), also those past the unit's columns.
    const int per = cblocks * groups;               // waves of one unit
    const int cgroups = (cblocks + kWaves - 1) / kWaves;
    const int wgu = SHARED ? cgroups * groups : (per + kWaves - 1) / kWaves;   // workgroups of one unit
    const int x = blockIdx.x;
    const int k = x >> 3;
    const int slot = (k / wgu) * 8 + (x & 7);       // the unit's place in the start order
    const int jw = k - (k / wgu) * wgu;             // workgroup within the unit
    const int j = jw * kWaves + wave;               // wave within the unit
    const int nunits = a.batch * Hkv;
    if (slot >= nunits || (!SHARED && j >= per)) return;   // (SHARED: uniform over the workgroup)
    // The longest units start first: a unit's waves are as long as its
    // cached prefix, and one that starts after the short units have drained
    // ends the launch late (measured on MI355X: 4% on the 2048-token chunk
    // over prefixes of 0-30K tokens, and on the 512-token one).  The order is
    // by length, longest first, ties by index; each wave ranks the lengths
    // itself (one per lane), so batches of up to 64 lengths are ordered and
    // larger ones keep the index order.
    int unit = slot;
    const int nkeys = HEAD ? nunits : a.batch;     // lengths: one per unit (HEAD) or sequence
    if (nkeys <= 64) {
      const int ln = threadIdx.x & 63;
      const int cap = a.table_width * kPageSize;
      const int Li = ln < nkeys ? min(max(a.lens[ln], 0), cap) : -1;
      int rank = 0;
      for (int t = 0; t < nkeys; ++t) {
        const int Lt = __builtin_amdgcn_readlane(Li, t);
        rank += (Lt > Li || (Lt == Li && t < ln)) ? 1 : 0;
      }
      const int want = HEAD ? slot : slot / Hkv;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(ln < nkeys && rank == want);
      if (hit != 0) {   // always exactly one lane: the ranks are a permutation
        const int key = __builtin_ctzll(hit);
        unit = HEAD ? key : key * Hkv + (slot - want * Hkv);
      }
    }
    if constexpr (SHARED) {
      const int jg = jw / groups;
      g = jw - jg * groups;
      cb = (cgroups - 1 - jg) * kWaves + wave;      // may be past the last block: no columns
    } else {
      const int jb = j / groups;
      g = j - jb * groups;
      cb = cblocks - 1 - jb;
    }
    b = unit / Hkv;
    h = unit - b * Hkv;
  } else {
    const int item = blockIdx.x * kWaves + wave;
    if (item >= a.batch * Hkv * cblocks * groups) return;
    const int rest = item / groups;
    g = item - rest * groups;
    const int unit = rest / cblocks;
    cb = rest - unit * cblocks;
    b = unit / Hkv;
    h = unit - b * Hkv;
  }
  const int cbase = cb * 16 * NQ;              // first column of this wave's block
  const int cend = max(min(cbase + 16 * NQ, C), cbase);   // (= cbase: a block past the columns)
  const int unit = b * Hkv + h;
  const int part0 = g * ppw;  // first partition of this wave
  const int row = HEAD ? unit : b;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;      // MFMA row/column index owned by this lane
  const int q4 = lane >> 4;     // which quarter of the MFMA K dimension

  const int cap = a.table_width * kPageSize;
  int L = planned ? planned_len : a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int npages_all = (L + kPageSize - 1) / kPageSize;
  auto pages_to = [&](int ce) {  // pages visible to the column before ce (CAUSAL)
    const int seen = L - T + (ce - 1) / G + 1;  // column ce - 1 sees L - T + t + 1 tokens
    return seen > 0 ? min(npages_all, (seen + kPageSize - 1) / kPageSize) : 0;
  };
  // SHARED: the workgroup walks the pages its last column sees; each wave
  // computes the ones its own columns see (npages_w), none without columns.
  const int wg_cend = SHARED ? min((cb - wave + kWaves) * 16 * NQ, C) : cend;
  int npages = npages_all;
  if (CAUSAL) npages = pages_to(SHARED ? wg_cend : cend);
  const int npages_w = !SHARED ? npages : (cend > cbase ? pages_to(cend) : 0);
  const int p0 = part0 * chunk;
  const int p1 = planned ? min(p0 + chunk, npages) : min(min(part0 + ppw, Pn) * chunk, npages);
  // Fixed partitions: a unit whose pages all lie in its first partition has
  // nothing to merge, so that partition's waves write its output rows and the
  // reduce skips them (as for the planned split's single-partition groups).
  if (!planned && part0 == 0 && npages_all <= chunk) direct = true;
  bool flagged;
  if (a.unit_flags != nullptr) {   // HEAD with the check: the sequence's unit words
    uint32_t word = 0u;
    for (int u = lane; u < Hkv; u += 64) word |= a.unit_flags[(size_t)b * Hkv + u];
    word = wave_or(word);
    flagged = word != 0u;
    if (a.write_flags && h == 0 && part0 == 0 && cb == 0 && lane == 0) a.flags_out[b] = word;
  } else {
    flagged = a.flags != nullptr && a.flags[b] != 0u;
  }
  // query row (in [B][T][Hq]) of column cc of this unit
  auto col_row = [&](int cc) {
    const int t = cc / G;
    return ((size_t)b * T + t) * Hq + h * G + (cc - t * G);
  };
  if (flagged || p0 >= p1) {
    if (direct) {
      for (int i = lane; i < (cend - cbase) * D; i += 64)
        a.out[col_row(cbase + i / D) * D + i % D] = 0;
    }
    return;
  }
  const int n = p1 - p0;
  const int nw = SHARED ? max(min(p1, npages_w) - p0, 0) : n;   // pages this wave computes

  // Q^T as the B operand of S^T = K Q^T: lane (c, q4) of tile nq holds column
  // 16 * nq + c and the 8 dims that the K A-operand places in this lane for
  // each step.  lim: tokens visible to the lane's column.
  bf16x8 qop[QLDS ? 1 : NQ][NSTEP];
  int lim[NQ];
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    const int cc = cbase + 16 * nq + c;
    const bool ok = cc < cend;
    const uint16_t* qrow = a.q + col_row(ok ? cc : 0) * D;
    lim[nq] = CAUSAL ? L - T + (ok ? cc / G : 0) + 1 : L;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      int d0;
      if (FP8) d0 = 64 * (s >> 1) + 16 * q4 + 8 * (s & 1);
      else d0 = 32 * s + 8 * q4;
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      if constexpr (QLDS) s_q[wave][nq * NSTEP + s][lane] = __builtin_bit_cast(bf16x8, v);
      else qop[nq][s] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // first token that some column cannot see: pages at or past it need masks
  const int vis_min = CAUSAL ? L - T + cbase / G + 1 : L;

  // Running max before a column's first visible token.  Causal kernels start
  // from the lowest finite float rather than -inf: a column with nothing
  // visible yet then needs no special case (exp2(-inf - m) = 0 for its masked
  // scores, and a rescale that finds no visible score leaves it at alpha = 1),
  // and the first visible score replaces it with alpha = exp2(-FLT_MAX - m) = 0
  // exactly as from -inf.  Partials of such columns are never merged (the
  // reduce reads only partitions that hold a visible token of the row).
  constexpr float kEmptyMax = CAUSAL ? -3.40282347e38f : -INFINITY;
  // O^T accumulators.  One tile: 16 x 16 tiles (dims x columns), one per 16
  // dims.  Several tiles: 32 x 32 tiles, one per (32 dims, pair of column
  // tiles), for the double-rate 32x32x16 P.V MFMA -- a page's 16 tokens are
  // exactly its K dimension (same register count: D / 2 per column tile).
  // In a 32 x 32 tile lane l holds column 32 p + (l & 31) and the dims
  // 32 J + 8 g + 4 (l >> 5) + r of element 4 g + r (VPERM: g = 1 and 3
  // trade dims).
  constexpr bool WIDE = NQ >= 2;
  constexpr int NP = WIDE ? NQ / 2 : 1;        // column-tile pairs
  constexpr int NJ = WIDE ? NT / 2 : 1;        // 32-dim blocks
  f32x4 o[WIDE ? 1 : NQ][WIDE ? 1 : NT];
  f32x16 ow[NP][NJ];
  float m_run[NQ], l_acc[NQ];
  float thr[NQ];   // m_run + kRescaleSlack: a page rescales when a score exceeds it
#pragma unroll
  for (int nq = 0; nq < NQ; ++nq) {
    if constexpr (!WIDE) {
#pragma unroll
      for (int j = 0; j < NT; ++j) o[nq][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    m_run[nq] = kEmptyMax;
    thr[nq] = kEmptyMax + kRescaleSlack;
    l_acc[nq] = 0.f;
  }
  if constexpr (WIDE) {
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) ow[pp][jj] = f32x16{};
  }

  const int32_t* bt = a.block_table + (size_t)row * a.table_width + p0;
  const size_t page_stride = HEAD ? (size_t)BLOCK : (size_t)Hkv * BLOCK;
  const uint8_t* kpool = a.k_pages + (HEAD ? 0 : (size_t)h * BLOCK);
  // V blocks sit in other slots than their K blocks (v_block_slot): the next
  // head's slot of the same page, or the neighbouring page's slot.
  const bool v_rot = !HEAD && Hkv > 1;
  const uint8_t* vpool = a.v_pages + (HEAD ? 0 : (size_t)(v_rot ? (h + 1) % Hkv : h) * BLOCK);
  const float* kscale = FP8 ? a.k_scale + (HEAD ? 0 : h) : nullptr;
  const float* vscale = FP8 ? a.v_scale + (HEAD ? 0 : h) : nullptr;
  float v_ref = 0.f;   // FP8: the reference V scale of the P.V operands (uniform; see kPScale)
  const int scale_stride = HEAD ? 1 : Hkv;
  const int lane_off = (c * 4 + q4) * 16;
  // The page-sharing BF16 kernel keeps V in its LDS ring in the order of the
  // 32x32x16 A operand (see its ring loads): each lane reads its operand as
  // two 8-byte halves and no row swaps are needed.  Its P.V rows hold the
  // dims in another order: row m = c + 16 b of a 32-dim block holds dim
  // c + 16 (b ^ (c >> 3)), i.e. rows 8-15 and 24-31 trade places, so that
  // the lanes of a 16-lane group read different halves of their LDS slots
  // (emit maps the rows back).
  constexpr bool VPERM = SHARED && !FP8;

  // Page ids, one lane per page, 512 pages (8 registers) at a time.  They are
  // loaded, and waited for, before the page loop of each 512-page segment:
  // a load inside the loop would put a join in front of every use, and the
  // compiler then waits for all outstanding loads there on every page.  The
  // look-ahead page's id is always read from ids[0]; the registers shift down
  // by one when the look-ahead enters the next 64 pages (constant indices
  // only, so the array stays in registers).  Ids out of range (only possible
  // with the tag check off) are read as page 0 so no access leaves the pool.
  //
  // FP8 scales of the segment's pages are gathered the same way, one lane per
  // page, right after the ids: two gathers per 64 pages instead of two loads
  // per page (which measured about 3% of the kernel time).  The segment is
  // then 256 pages, so that ids and scales fit the register budget.  The
  // segment's largest V scale updates the wave's reference scale there.
  constexpr bool SEGSC = FP8;
  // FP8 kernels with several column tiles apply a page's V operand factor
  // inside the exponent, exp2(s - (m - log2 f)) = f exp2(s - m), instead of
  // one multiply per weight; the row sums take the weights back with one
  // multiply-add by 1/f per tile.
  constexpr bool VFOLD = FP8 && NQ >= 2;
  // (four-tile BF16 kernels keep fewer ids, for registers to read Q ahead)
  constexpr int kIdRegs = SEGSC ? 4 : (NQ == 4 ? PA_IDREGS4 : 8);
  constexpr int kSegPages = 64 * kIdRegs;
  int ids[kIdRegs];
  float sks[SEGSC ? kIdRegs : 1], svs[SEGSC ? kIdRegs : 1];
  // The id of page rr of the segment: rr lies in the 64-page chunk that
  // ids[0] holds, or in the next one (nxt).  The loops walk the pages in
  // 64-page chunks and shift the registers down by one after each
  // (shift_ids): a shift under a condition inside the page loop made the
  // compiler copy every id register on every page.  Each loop consumes W
  // pages per iteration and loads W - 1 pages ahead, so only the steps
  // u >= 1 of a chunk's last iteration load from the next chunk, and only
  // when another chunk follows: that iteration runs after the chunk's loop.
  // (nxt is a compile-time choice: the loops know which steps look into the
  // next chunk, so no register is selected at run time)
  auto pid_of = [&](int rr, auto nxt) __attribute__((always_inline)) {
    return __builtin_amdgcn_readlane(ids[decltype(nxt)::value], rr & 63);
  };
  // Byte offset of page pid's block in a pool: ids are non-negative and the
  // page stride is below 2^31 (checked on the host), so one 32 x 32-bit
  // multiply with a 64-bit product.
  auto page_off = [&](int pid) __attribute__((always_inline)) {
    return (uint64_t)(uint32_t)pid * (uint32_t)page_stride;
  };
  auto scale_of = [&](const float (&sv)[SEGSC ? kIdRegs : 1], int rr, auto nxt) __attribute__((always_inline)) {
    constexpr int t = SEGSC ? decltype(nxt)::value : 0;
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv[t]), rr & 63));
  };
  auto shift_ids = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t + 1 < kIdRegs; ++t) {
      ids[t] = ids[t + 1];
      if constexpr (SEGSC) {
        sks[t] = sks[t + 1];
        svs[t] = svs[t + 1];
      }
    }
  };
  static_assert(kIdRegs >= 2, "a look-ahead page may sit in the next chunk");

  // Page r's block: a scalar base address plus this lane's 16-byte chunk, so
  // that every load is one 1 KiB contiguous wave access.  FP8 scales of the
  // page are requested with its data.  nxt: as for pid_of.
  auto load = [&](u32x4 (&kr)[NOP], u32x4 (&vr)[NOP], float& ksc, float& vsc, int r, auto nxt) __attribute__((always_inline)) {
    const int pid = pid_of(r, nxt);
    const uint8_t* kp = kpool + page_off(pid);
    const int vpid = v_rot ? pid : ((pid ^ 1) < a.num_pages ? (pid ^ 1) : pid);
    const uint8_t* vp = vpool + page_off(vpid);
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      kr[i] = load_blk(kp, NSEG * 1024, lane_off, i * 1024);
      vr[i] = load_blk(vp, NSEG * 1024, lane_off, i * 1024);
    }
    if constexpr (SEGSC) {   // vsc: the page's V scale / v_ref * kPScale (VFOLD: its log2)
      ksc = scale_of(sks, r, nxt);
      vsc = scale_of(svs, r, nxt);
    }
  };

  // S^T of one page: acc[nq] = K Q^T for column tile nq (unscaled)
  auto qk = [&](f32x4 (&acc)[NQ], const u32x4 (&kr)[NOP]) __attribute__((always_inline)) {
    // Q operand of tile nq, step st; the LDS address passes through an empty
    // asm on every page, so the compiler cannot tell it is the same and does
    // not hoist the reads out of the page loop (which would put Q back into
    // registers), and the reads use it with immediate offsets
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    lds_bf16x8* qb = (lds_bf16x8*)&s_q[wave][0][lane];
    if constexpr (QLDS) asm volatile("" : "+v"(qb));
    auto qv = [&](int nq, int st) -> bf16x8 {
      if constexpr (QLDS) return qb[(nq * NSTEP + st) * 64];
      else return qop[nq][st];
    };
    // K operand of step st (16 tokens x 32 dims): FP8 codes widened to bf16
    // (CVT: widened already)
    auto kv = [&](int st) -> bf16x8 {
      if constexpr (FP8 && !CVT) {
        const int i = st >> 1, hh = st & 1;
        u32x2 lo = fp8x4_to_bf16x4(kr[i][2 * hh]);
        u32x2 hi = fp8x4_to_bf16x4(kr[i][2 * hh + 1]);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      } else {
        return __builtin_bit_cast(bf16x8, kr[st]);
      }
    };
    // ---- scores S^T (token rows x query columns), one accumulator per tile;
    // the Q operands of step st + 1 are requested before step st's MFMAs
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) acc[nq] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qn[NQ];
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) qn[nq] = qv(nq, 0);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      bf16x8 qc[NQ];
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) qc[nq] = qn[nq];
      if (st + 1 < NSTEP) {
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq) qn[nq] = qv(nq, st + 1);
      }
      const bf16x8 av = kv(st);
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq)
        acc[nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qc[nq], acc[nq], 0, 0, 0);
    }
    constexpr int kAhead = NQ == 4 ? PA_QK_SCHED4 : PA_QK_SCHED;
    if constexpr (QLDS && kAhead > 0) {
      // Keep kAhead LDS reads of Q ahead of the MFMAs that use them.  Left to
      // itself the compiler waited for each read just before its MFMA,
      // exposing the LDS latency 12 times per page (measured on MI355X: 17-19%
      // of the prefill kernel's time at 4 ahead, 9-11% more at 8 ahead with 4
      // tiles).  With 2 tiles, 6 ahead spills in the page loop; with 4 BF16
      // tiles, 8 ahead spills 5 registers that live only outside it.
      constexpr int nr = NQ * NSTEP, ahead = kAhead;
      __builtin_amdgcn_sched_group_barrier(0x100, ahead, 0);
#pragma unroll
      for (int i = 0; i < nr - ahead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, ahead, 0);
    }
  };

  // Softmax update and O^T += V^T P^T for page k of the run, from its scores.
  auto pv = [&](const f32x4 (&acc)[NQ], u32x4 (&vr)[NOP], float ksc, float vsc, int k) __attribute__((always_inline)) {
    const int page = p0 + k;
    float kfac = a.score_scale_log2;
    if (FP8) kfac *= ksc;
    const float vinv = VFOLD ? __builtin_amdgcn_exp2f(-vsc) : 1.f;   // 1/f
    // lane (c, q4) holds the scores of column c of each tile for tokens 4*q4 + r
    const int tok0 = page * kPageSize + q4 * 4;
    const bool tail = page * kPageSize + kPageSize > vis_min;
    f16x4 pbh[NQ];   // FP8: P^T operands (f16); BF16 uses pbb
    i16x4 pbb[NQ];
    // The running max of a column moves only when one of its scores exceeds
    // it by more than the slack.  A lane's own max over its 4 tokens decides
    // that as well as the column max does (the ballot is over the whole wave
    // and the column's 4 lanes share m_run), so the cross-lane column max is
    // only formed on the rare pages that rescale.
    float sc[NQ][4], lmax[NQ];
    bool grow = false;
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[nq][r] = acc[nq][r] * kfac;
    if (tail) {
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[nq][r] = (tok0 + r < lim[nq]) ? sc[nq][r] : -INFINITY;
    }
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      lmax[nq] = max4(sc[nq][0], sc[nq][1], sc[nq][2], sc[nq][3]);
      grow |= lmax[nq] > thr[nq];
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
      float alph[NQ];
      bool moved[NQ];
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
        alph[nq] = 1.f;
        moved[nq] = __builtin_amdgcn_ballot_w64(lmax[nq] > thr[nq]) != 0;
        if (moved[nq]) {
          const float m_new = fmaxf(m_run[nq], col_max(lmax[nq]));
          const float alpha = __builtin_amdgcn_exp2f(m_run[nq] - m_new);
          l_acc[nq] *= alpha;
          if constexpr (!WIDE) {
#pragma unroll
            for (int j = 0; j < NT; ++j) o[nq][j] *= alpha;
          }
          alph[nq] = alpha;
          m_run[nq] = m_new;
          thr[nq] = m_new + kRescaleSlack;
        }
      }
      if constexpr (WIDE) {   // lanes with (l & 16) hold the pair's second tile's column
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if (moved[2 * pp] || moved[2 * pp + 1]) {
            const float f = pick_hi16(alph[2 * pp], alph[2 * pp + 1]);
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) ow[pp][jj] *= f;
          }
        }
      }
    }
#pragma unroll
    for (int nq = 0; nq < NQ; ++nq) {
      float p[4];
      const float mq = VFOLD ? m_run[nq] - vsc : m_run[nq];   // (VFOLD: vsc = log2 f)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[nq][r] - mq);
      // (the page-sharing BF16 kernel sums the rounded weights it multiplies
      // V by, two per dot instruction: its normaliser is then exactly the sum
      // of the P operands)
      if constexpr (VFOLD) l_acc[nq] = __builtin_fmaf((p[0] + p[1]) + (p[2] + p[3]), vinv, l_acc[nq]);
      else if (!(SHARED && !FP8)) l_acc[nq] += (p[0] + p[1]) + (p[2] + p[3]);
      if (FP8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pbh[nq][r] = (_Float16)(VFOLD ? p[r] : p[r] * vsc);
      } else {
        // two values per conversion (round to nearest even, as one by one)
        const bf16x2 lo = __builtin_convertvector(f32x2{p[0], p[1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector(f32x2{p[2], p[3]}, bf16x2);
        pbb[nq] = __builtin_bit_cast(i16x4, u32x2{__builtin_bit_cast(uint32_t, lo),
                                                 __builtin_bit_cast(uint32_t, hi)});
        if constexpr (SHARED) {
          const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
          l_acc[nq] = __builtin_amdgcn_fdot2_f32_bf16(
              hi, one, __builtin_amdgcn_fdot2_f32_bf16(lo, one, l_acc[nq], false), false);
        }
      }
    }

    // ---- O^T += V^T P^T; on the last page zero V of tokens past L (the
    // slots may hold anything, and 0 * NaN would poison the sum; CVT: zeroed
    // when widened)
    if (!CVT && page * kPageSize + kPageSize > L) {   // the last page only, in place
      const int nv = min(max(L - tok0, 0), 4);  // this lane's valid tokens (4 per dword row)
      if constexpr (VPERM) {
        // operand order: tokens 8 h .. 8 h + 3 in dwords 0-1, 8 h + 4 .. 8 h + 7
        // in dwords 2-3 (h = q4 >> 1), two tokens per dword, low half first
        const int t0 = page * kPageSize + 8 * (q4 >> 1);
        const int na = min(max(L - t0, 0), 4), nb = min(max(L - t0 - 4, 0), 4);
        const uint64_t ma = na >= 4 ? ~0ull : ((1ull << (16 * na)) - 1ull);
        const uint64_t mb = nb >= 4 ? ~0ull : ((1ull << (16 * nb)) - 1ull);
        const u32x4 mk{(uint32_t)ma, (uint32_t)(ma >> 32), (uint32_t)mb, (uint32_t)(mb >> 32)};
#pragma unroll
        for (int i = 0; i < NSEG; ++i) vr[i] &= mk;
      } else if (FP8) {
        const uint32_t m = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
#pragma unroll
        for (int i = 0; i < NSEG; ++i) vr[i] &= u32x4{m, m, m, m};
      } else {   // BF16: tokens 0-1 in the even dwords, 2-3 in the odd ones
        const uint64_t m = nv >= 4 ? ~0ull : ((1ull << (16 * nv)) - 1ull);
        const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
#pragma unroll
        for (int i = 0; i < NSEG; ++i) vr[i] &= u32x4{lo, hi, lo, hi};
      }
    }
    if constexpr (WIDE) {
      // 32x32x16: B = P^T of a pair of column tiles, A = V^T of 32 dims; both
      // from the 16 x 16 operands of two tiles by one row swap per dword
      u32x4 pb2[NP];
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        if (FP8) pb2[pp] = pair_rows(__builtin_bit_cast(u32x2, pbh[2 * pp]),
                                     __builtin_bit_cast(u32x2, pbh[2 * pp + 1]));
        else pb2[pp] = pair_rows(__builtin_bit_cast(u32x2, pbb[2 * pp]),
                                 __builtin_bit_cast(u32x2, pbb[2 * pp + 1]));
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        u32x4 av;
        if constexpr (FP8 && !CVT) {
          av = pair_rows(fp8x4_to_f16x4(vr[(2 * jj) >> 2][(2 * jj) & 3]),
                         fp8x4_to_f16x4(vr[(2 * jj + 1) >> 2][(2 * jj + 1) & 3]));
        } else if constexpr (VPERM || CVT) {   // already in operand order
          av = vr[jj];
        } else {   // tiles 2 jj and 2 jj + 1 are the two halves of segment jj
          const u32x4& seg = vr[jj];
          av = pair_rows(u32x2{seg[0], seg[1]}, u32x2{seg[2], seg[3]});
        }
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
          if (FP8)
            ow[pp][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, av), __builtin_bit_cast(f16x8, pb2[pp]), ow[pp][jj], 0, 0, 0);
          else
            ow[pp][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, pb2[pp]), ow[pp][jj], 0, 0, 0);
        }
      }
    } else if (FP8) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint32_t w = vr[j >> 2][j & 3];
        const f16x4 vf = __builtin_bit_cast(f16x4, fp8x4_to_f16x4(w));
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
          o[nq][j] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pbh[nq], o[nq][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x4& seg = vr[j >> 1];
        const uint64_t w = ((uint64_t)seg[2 * (j & 1) + 1] << 32) | seg[2 * (j & 1)];
        const i16x4 vb = __builtin_bit_cast(i16x4, w);
#pragma unroll
        for (int nq = 0; nq < NQ; ++nq)
          o[nq][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb, pbb[nq], o[nq][j], 0, 0, 0);
      }
    }
  };

  auto compute = [&](const u32x4 (&kr)[NOP], u32x4 (&vr)[NOP], float ksc, float vsc, int k) __attribute__((always_inline)) {
    f32x4 acc[NQ];
    qk(acc, kr);
    pv(acc, vr, ksc, vsc, k);
  };

  // This wave's result for partition `part`: the normalised output when the
  // unit has a single partition, else the partial (max, sum, unnormalised O).
  // A column that saw no token (multi-query, L - T + t < 0) has sum 0 and
  // O = 0, and is written as zeros.  vfac converts O to the values' units
  // (FP8: v_ref / kPScale; 1 for BF16 and for a parked partition).
  auto emit = [&](int part, float vfac) __attribute__((always_inline)) {
    if constexpr (WIDE) {
      float lt[NQ];
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) lt[nq] = col_sum(l_acc[nq]);
      const int dq = 4 * (lane >> 5);           // this lane's offset within each 8 dims
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        const float l_tot = pick_hi16(lt[2 * pp], lt[2 * pp + 1]);
        const float m_col = pick_hi16(m_run[2 * pp], m_run[2 * pp + 1]);
        const int cc = cbase + 32 * pp + (lane & 31);
        if (cc >= cend) continue;
        const size_t qrow = col_row(cc);
        if (direct) {
          const float inv = (CAUSAL && !(l_tot > 0.f)) ? 0.f : (FP8 ? vfac / l_tot : 1.f / l_tot);
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16& v = ow[pp][jj];
              const uint32_t lo = (uint32_t)bf16_rne(v[4 * g] * inv) |
                                  ((uint32_t)bf16_rne(v[4 * g + 1] * inv) << 16);
              const uint32_t hi = (uint32_t)bf16_rne(v[4 * g + 2] * inv) |
                                  ((uint32_t)bf16_rne(v[4 * g + 3] * inv) << 16);
              *reinterpret_cast<u32x2*>(a.out + qrow * D + 32 * jj + 8 * (VPERM ? g ^ ((g & 1) << 1) : g) + dq) =
                  u32x2{lo, hi};
            }
        } else {
          const size_t pi = planned ? (size_t)pslot * C + cc : qrow * Pn + part;
          float* po = a.part_o + pi * D;
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x16& v = ow[pp][jj];
              const f32x4 x = f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
              *reinterpret_cast<f32x4*>(po + 32 * jj + 8 * (VPERM ? g ^ ((g & 1) << 1) : g) + dq) =
                  FP8 ? x * vfac : x;
            }
          if (dq == 0) {
            a.part_ml[pi * 2 + 0] = m_col;
            a.part_ml[pi * 2 + 1] = l_tot;
          }
        }
      }
    } else {
#pragma unroll
      for (int nq = 0; nq < NQ; ++nq) {
        const float l_tot = col_sum(l_acc[nq]);
        const int cc = cbase + 16 * nq + c;
        if (cc < cend) {
          const size_t qrow = col_row(cc);
          if (direct) {
            if (a.row_ml != nullptr && q4 == 0) {   // scored decode: the row's final (max, sum)
              a.row_ml[qrow * 2 + 0] = m_run[nq];
              a.row_ml[qrow * 2 + 1] = l_tot;
            }
            const float inv = (CAUSAL && !(l_tot > 0.f)) ? 0.f : (FP8 ? vfac / l_tot : 1.f / l_tot);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              const f32x4 v = o[nq][j];
              uint32_t lo = (uint32_t)bf16_rne(v[0] * inv) | ((uint32_t)bf16_rne(v[1] * inv) << 16);
              uint32_t hi = (uint32_t)bf16_rne(v[2] * inv) | ((uint32_t)bf16_rne(v[3] * inv) << 16);
              *reinterpret_cast<u32x2*>(a.out + qrow * D + 16 * j + 4 * q4) = u32x2{lo, hi};
            }
          } else {
            // fixed partitions: [row][Pn]; planned: [slot][column]
            const size_t pi = planned ? (size_t)pslot * C + cc : qrow * Pn + part;
            float* po = a.part_o + pi * D;
#pragma unroll
            for (int j = 0; j < NT; ++j)
              *reinterpret_cast<f32x4*>(po + 16 * j + 4 * q4) = FP8 ? o[nq][j] * vfac : o[nq][j];
            if (q4 == 0) {
              a.part_ml[pi * 2 + 0] = m_run[nq];
              a.part_ml[pi * 2 + 1] = l_tot;
            }
          }
        }
      }
    }
  };

  // Register ring of PIPE pages: page r+PIPE-1 is requested before page r
  // is consumed.  Past the end of a segment the last page is requested again
  // (an L2 hit) so that every iteration issues the same loads.  At each
  // partition boundary the finished partition is emitted and the state
  // restarts; the ring keeps streaming across it.
  u32x4 kr[PIPE][NOP], vr[PIPE][NOP];   // (NOP = NSEG on these paths)
  float ks[PIPE], vs[PIPE];
  int part = part0;
  int next_boundary = chunk;  // page index (relative to p0) of the next partition
  float (*stash)[64] = s_stash[wave];
  for (int seg = 0; seg < n; seg += kSegPages) {
    const int m = min(kSegPages, n - seg);
#pragma unroll
    for (int j = 0; j < kIdRegs; ++j) {
      const int k = seg + 64 * j + lane;
      ids[j] = k < n ? bt[k] : 0;
    }
    // wait for the ids here, once per segment (see above)
    int last = __builtin_amdgcn_readfirstlane(ids[kIdRegs - 1]);
    asm volatile("" : : "s"(last));
    // ids out of range (only possible with the tag check off) read page 0,
    // so that no access leaves the pool
#pragma unroll
    for (int j = 0; j < kIdRegs; ++j) ids[j] = (unsigned)ids[j] < (unsigned)a.num_pages ? ids[j] : 0;
    if constexpr (SEGSC) {
#pragma unroll
      for (int j = 0; j < kIdRegs; ++j) {
        const int pid = (unsigned)ids[j] < (unsigned)a.num_pages ? ids[j] : 0;
        sks[j] = kscale[(size_t)pid * scale_stride];
        svs[j] = vscale[(size_t)pid * scale_stride];
      }
      // The largest V scale of the segment's pages in this run; when it
      // exceeds the reference, O moves to the new units (a rare rescale:
      // once per wave for caches of one magnitude).  NaN scales are skipped
      // here and still poison their own page's operands, as they should.
      float vmax = 0.f;
#pragma unroll
      for (int j = 0; j < kIdRegs; ++j) vmax = seg + 64 * j + lane < n ? fmaxf(vmax, svs[j]) : vmax;
      vmax = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(vmax))));
      if (vmax > v_ref) {
        if (v_ref > 0.f) {
          const float r = v_ref / vmax;
          if constexpr (WIDE) {
#pragma unroll
            for (int pp = 0; pp < NP; ++pp)
#pragma unroll
              for (int jj = 0; jj < NJ; ++jj) ow[pp][jj] *= r;
          } else {
#pragma unroll
            for (int nq = 0; nq < NQ; ++nq)
#pragma unroll
              for (int j = 0; j < NT; ++j) o[nq][j] *= r;
          }
        }
        v_ref = vmax;
      }
      const float to_op = v_ref > 0.f ? kPScale / v_ref : 0.f;
#pragma unroll
      for (int j = 0; j < kIdRegs; ++j) {
        svs[j] *= to_op;
        // (VFOLD: the exponent offset log2 of the factor, at least -64: a page
        // 2^64 times below the segment's largest V contributes nothing
        // measurable; a NaN factor stays NaN)
        if constexpr (VFOLD) svs[j] = __builtin_amdgcn_logf(fmaxf(svs[j], 0x1p-64f) + (svs[j] - svs[j]));
      }
    }
    if constexpr (SHARED) {
      // The workgroup's waves load each page once, into LDS, for all of
      // them: wave w requests 1 KiB segments w, w + kWaves, ... of the page
      // (K's, then V's) straight into the page's ring stage, kStages - 1
      // pages ahead.  Page r: each wave waits for its own segments of it
      // (the counter runs in order: only later pages' may stay in flight),
      // then a barrier makes the stage whole for all and proves that every
      // wave has read the previous page, whose stage the next request
      // reuses.  Every wave runs all of the workgroup's pages (m: uniform)
      // and computes those its own columns see (mw).
      //
      // FP8 (CVT): the stages hold FP8 codes, and only the wave that loaded
      // a segment reads it.  In page r's step each wave widens its segments
      // of page r + 1 into the operand buffer that no wave reads in this
      // step; the next step's barrier makes that buffer whole.  So a wave
      // waits only for its own loads of page r + 1, a stage can be requested
      // again once its loading wave has widened it (the requests run LEAD + 1
      // pages ahead, up to kStages), and page r's scales are read before the
      // step's request reuses their slot.
      //
      // The loads are buffer loads (dma_block): the segment's address is a
      // scalar resource and the lane's offset a loop-invariant register, so a
      // request costs no vector instructions.  A K lane fetches the chunk
      // that the compute lane of its index reads (linear LDS reads).  A V
      // lane L fetches chunk g = 4 (L & 15) + 2 ((L >> 4) & 1) + (L >> 5):
      // the compute lane (c, q4) then finds its 32x32x16 A operand (chunks
      // (c, 2 h) and (c, 2 h + 1), the 8-byte half e = (q4 & 1) ^ (c >> 3) of
      // each, h = q4 >> 1) as two 8-byte words 512 bytes apart.  Each 16-lane
      // group reads 8 first and 8 second halves of 16 slots: 16 distinct bank
      // pairs in 128 bytes, no bank conflicts.
      //
      // The pages run in 64-page chunks, one register of ids each: inside a
      // chunk the ids stay put (the look-ahead page's id comes from this
      // chunk's register or the next one's) and they shift once per chunk.
      constexpr int SEGS = 2 * NSEG;
      constexpr int MY = (SEGS + kWaves - 1) / kWaves;   // segments per wave and page
      constexpr int R = kStages;
      static_assert(64 % R == 0, "a 64-page chunk holds whole ring cycles");
      // pages requested ahead of the one a step waits for: page r (CVT: page
      // r + 1, which the step widens) may wait while LEAD later pages load.
      // A stage is requested again once every wave (CVT: the wave that loaded
      // it, the only one that reads it) has read it.
      constexpr int LEAD = CVT ? PA_SHARED_LEAD_FP8 : R - 2;
      static_assert(LEAD + (CVT ? 1 : 2) <= R, "a stage is read before it is requested again");
      auto ring = [&](auto st) -> u32x4 (*)[64] {
        constexpr int S = decltype(st)::value;
        if constexpr (S == 0) return s_st0;
        else if constexpr (S == 1) return s_st1;
        else if constexpr (S == 2) return s_st2;
        else if constexpr (S == 3) return s_st3;
        else if constexpr (S == 4) return s_st4;
        else if constexpr (S == 5) return s_st5;
        else if constexpr (S == 6) return s_st6;
        else return s_st7;
      };
      auto cvbuf = [&](auto bc) -> u32x4 (*)[64] {
        if constexpr (decltype(bc)::value == 0) return s_cv0;
        else return s_cv1;
      };
      // CVT: this wave's FP8 segments of page k (in ring stage st) widened
      // into operand buffer bc: a K segment holds the 16-byte halves of two
      // Q.K steps, a V segment the 4-token rows of two 32-dim P.V blocks
      // (one row swap each, as the register path does).  V of tokens past L
      // is zeroed first, on the unit's last page.
      auto widen = [&](auto st, auto bc, int k) __attribute__((always_inline)) {
        u32x4 (*src)[64] = ring(st);
        u32x4 (*dst)[64] = cvbuf(bc);
        const int page = p0 + k;
#pragma unroll
        for (int i = 0; i < MY; ++i) {
          const int sg = wave + i * kWaves;
          if (sg < NSEG) {
            const u32x4 w = src[sg][lane];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const u32x2 lo = fp8x4_to_bf16x4(w[2 * hh]), hi = fp8x4_to_bf16x4(w[2 * hh + 1]);
              dst[2 * sg + hh][lane] = u32x4{lo.x, lo.y, hi.x, hi.y};
            }
          } else if (sg < SEGS) {
            u32x4 w = src[sg][lane];
            if (page * kPageSize + kPageSize > L) {
              const int nv = min(max(L - (page * kPageSize + q4 * 4), 0), 4);
              const uint32_t mk = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
              w &= u32x4{mk, mk, mk, mk};
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
              dst[NOP + 2 * (sg - NSEG) + hh][lane] =
                  pair_rows(fp8x4_to_f16x4(w[2 * hh]), fp8x4_to_f16x4(w[2 * hh + 1]));
          }
        }
      };
      const int v_off = VPERM ? ((lane & 15) * 4 + ((lane >> 4) & 1) * 2 + (lane >> 5)) * 16 : lane_off;
      // 8-byte word of the V operand: half (q4 & 1) ^ (c >> 3) of the slot (see VPERM)
      const int v_rd = ((q4 >> 1) * 16 + c) * 2 + ((q4 & 1) ^ (c >> 3));
      float stk[R], stv[R];   // FP8 scales of the pages in the ring
      // page rr (of this chunk, or of the next one: nxt) into stage st
      auto request = [&](auto st, int rr, auto nxt) __attribute__((always_inline)) {
        constexpr int S = decltype(st)::value;
        const int pid = pid_of(rr, nxt);
        const uint8_t* kp = kpool + page_off(pid);
        const int vpid = v_rot ? pid : ((pid ^ 1) < a.num_pages ? (pid ^ 1) : pid);
        const uint8_t* vp = vpool + page_off(vpid);
        u32x4 (*dst)[64] = ring(st);
#pragma unroll
        for (int i = 0; i < MY; ++i) {
          const int sg = wave + i * kWaves;
          if (sg < SEGS) {
            const uint8_t* sp = sg < NSEG ? kp + sg * 1024 : vp + (sg - NSEG) * 1024;
            dma_block(sp, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&dst[sg][0],
                      sg < NSEG ? lane_off : v_off);
          }
        }
        if constexpr (SEGSC) {
          stk[S] = scale_of(sks, rr, nxt);
          stv[S] = scale_of(svs, rr, nxt);
        }
      };
      // every wave's reads of the ring are done (lgkmcnt), then the barrier;
      // the compiler-only fences keep LDS accesses on their side of it
      auto sync = [&]() __attribute__((always_inline)) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);               // s_waitcnt lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      };
      const int mw = min(max(nw - seg, 0), m);
      sync();                                             // the last segment's reads are done
      // Every step requests a page (past the segment's end, its last page
      // again: an L2 hit into a stage nobody reads), so that the count of
      // loads issued after page r's is always the same and one wait serves.
      auto first = [&](auto jc) __attribute__((always_inline)) {   // pages 0 .. LEAD into stages 0 .. LEAD
        constexpr int J = decltype(jc)::value;
        if constexpr (J <= LEAD) request(IntC<J>{}, min(J, m - 1), IntC<0>{});
      };
      first(IntC<0>{});
      first(IntC<1>{});
      first(IntC<2>{});
      first(IntC<3>{});
      first(IntC<4>{});
      first(IntC<5>{});
      first(IntC<6>{});
      if constexpr (CVT) {
        // page 0 widened before the loop; each step then widens the next
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (LEAD * MY));   // vmcnt: this wave's page 0
        widen(IntC<0>{}, IntC<0>{}, seg);
      }
      for (int c0 = 0; c0 < m; c0 += 64) {
        const int ce = min(c0 + 64, m);
        // iter: the R pages from r0; lc: the last iteration of a chunk that
        // another follows, whose steps u >= 1 load from the next chunk
        auto iter = [&](const int r0, auto lc) __attribute__((always_inline)) {
          auto step = [&](auto uc, auto lc) __attribute__((always_inline)) {
            constexpr int U = decltype(uc)::value;
            const int r = r0 + U;
            if (r >= ce) return;
            constexpr int nxt = (decltype(lc)::value && U + LEAD + 1 >= R) ? 1 : 0;
            if constexpr (CVT) {
              // The widened page r is whole after the barrier.  After page
              // r's compute, this wave widens its FP8 segments of page r + 1
              // (read once the LEAD later pages' loads, the one just
              // requested included, are all that may remain), so that the
              // conversions overlap the compute's last MFMAs.  (At the
              // segment's last page the stage holds a repeat of it, widened
              // into the buffer nobody reads.)  Page r's scales are read
              // first: the request may reuse its stage.
              const float ksc = stk[U], vsc = stv[U];
              sync();
              request(IntC<(U + LEAD + 1) % R>{}, min(r + LEAD + 1, m - 1), IntC<nxt>{});
              if (r < mw) {
                u32x4 (*src)[64] = cvbuf(IntC<U & 1>{});
                u32x4 kp[NOP], vp[NOP];
#pragma unroll
                for (int i = 0; i < NOP; ++i) {
                  kp[i] = src[i][lane];
                  vp[i] = src[NOP + i][lane];
                }
                compute(kp, vp, ksc, vsc, seg + r);
              }
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              __builtin_amdgcn_s_waitcnt(0x0F70 | (LEAD * MY));   // vmcnt
              if (r + 1 < m) widen(IntC<(U + 1) % R>{}, IntC<(U + 1) & 1>{}, seg + r + 1);
            } else {
              // requested after page r: the LEAD steps' worth that follow it
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              __builtin_amdgcn_s_waitcnt(0x0F70 | (LEAD * MY));   // vmcnt
              sync();
              request(IntC<(U + LEAD + 1) % R>{}, min(r + LEAD + 1, m - 1), IntC<nxt>{});
              if (r < mw) {
                u32x4 (*src)[64] = ring(IntC<U>{});
                u32x4 kp[NOP], vp[NOP];
#pragma unroll
                for (int i = 0; i < NSEG; ++i) {
                  kp[i] = src[i][lane];
                  if constexpr (VPERM) {
                    const u32x2* vb = reinterpret_cast<const u32x2*>(&src[NSEG + i][0]) + v_rd;
                    const u32x2 x = vb[0], y = vb[64];
                    vp[i] = u32x4{x.x, x.y, y.x, y.y};
                  } else {
                    vp[i] = src[NSEG + i][lane];
                  }
                }
                compute(kp, vp, stk[U], stv[U], seg + r);
              }
            }
          };
          step(IntC<0>{}, lc);
          step(IntC<1>{}, lc);
          if constexpr (R > 2) step(IntC<2>{}, lc);
          if constexpr (R > 3) step(IntC<3>{}, lc);
          if constexpr (R > 4) step(IntC<4>{}, lc);
          if constexpr (R > 5) step(IntC<5>{}, lc);
          if constexpr (R > 6) step(IntC<6>{}, lc);
          if constexpr (R > 7) step(IntC<7>{}, lc);
        };
        const bool more = c0 + 64 < m;
        int r0 = c0;
        for (; r0 < (more ? ce - R : ce); r0 += R) iter(r0, IntC<0>{});
        if (more) iter(r0, IntC<1>{});
        shift_ids();
      }
      // the last requests (repeats) land before the stages are used again or
      // the workgroup's LDS is released
      __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
      continue;
    }
    if constexpr (LATEK) {
      // One K buffer: page r+1 is requested as soon as page r's Q.K has read
      // K, and the waits are the compiler's (K before Q.K, V before P.V)
      load(kr[0], vr[0], ks[0], vs[0], 0, IntC<0>{});
      for (int c0 = 0; c0 < m; c0 += 64) {
        const int ce = min(c0 + 64, m);
        auto iter = [&](const int r0, auto lc) __attribute__((always_inline)) {
          auto step = [&](auto uc, auto lc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int r = r0 + u;
            if (r < ce) {
              f32x4 acc[NQ];
              qk(acc, kr[0]);
              if (r + 1 < m)
                load(kr[0], vr[1 - u], ks[1 - u], vs[1 - u], r + 1,
                     IntC<(decltype(lc)::value && u >= 1) ? 1 : 0>{});
              pv(acc, vr[u], ks[u], vs[u], seg + r);
            }
          };
          step(IntC<0>{}, lc);
          step(IntC<1>{}, lc);
        };
        const bool more = c0 + 64 < m;
        int r0 = c0;
        for (; r0 < (more ? ce - 2 : ce); r0 += 2) iter(r0, IntC<0>{});
        if (more) iter(r0, IntC<1>{});
        shift_ids();
      }
      continue;
    }
    static_assert(64 % PIPE == 0, "a 64-page chunk holds whole ring cycles");
#pragma unroll
    for (int u = 0; u < PIPE - 1; ++u) load(kr[u], vr[u], ks[u], vs[u], min(u, m - 1), IntC<0>{});
    for (int c0 = 0; c0 < m; c0 += 64) {
      const int ce = min(c0 + 64, m);
      auto iter = [&](const int r0, auto lc) __attribute__((always_inline)) {
        auto step = [&](auto uc, auto lc) __attribute__((always_inline)) {
          constexpr int u = decltype(uc)::value;
          const int r = r0 + u;                      // page within the segment
          const int slot = (u + PIPE - 1) % PIPE;  // a constant once the loop is unrolled
          if constexpr (THROTTLE) {
            // At most one page in flight per wave besides the one being consumed:
            // measured on MI355X, 2048 waves each keeping two or more pages of
            // random 2 KiB blocks outstanding move the cache 2-4% slower.
            __builtin_amdgcn_s_waitcnt(0x0F70);      // s_waitcnt vmcnt(0)
          }
          const int rr = min(r + PIPE - 1, m - 1);
          load(kr[slot], vr[slot], ks[slot], vs[slot], rr, IntC<(decltype(lc)::value && u >= 1) ? 1 : 0>{});
          if (r < ce) {
            const int k = seg + r;                   // page within this wave's run
            if constexpr (NQ == 1) {
              if (k == next_boundary) {
                // Park the finished partition in LDS: a global store now would
                // be waited for by the next page's throttle, and under the full
                // read stream stores take long to complete (measured: 6% of the
                // kernel time on the 32K-token FP8 workload).  FP8 O is parked in
                // the values' units: the reference scale may still grow.
                const float vfac = FP8 ? v_ref / kPScale : 1.f;
#pragma unroll
                for (int j = 0; j < NT; ++j)
#pragma unroll
                  for (int r = 0; r < 4; ++r) stash[4 * j + r][lane] = o[0][j][r] * vfac;
                stash[4 * NT][lane] = m_run[0];
                stash[4 * NT + 1][lane] = l_acc[0];
                ++part;
                next_boundary += chunk;
#pragma unroll
                for (int j = 0; j < NT; ++j) o[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                m_run[0] = -INFINITY;
                thr[0] = -INFINITY;
                l_acc[0] = 0.f;
              }
            }
            compute(kr[u], vr[u], ks[u], vs[u], k);
          }
        };
        step(IntC<0>{}, lc);
        step(IntC<1>{}, lc);
        if constexpr (PIPE > 2) step(IntC<2>{}, lc);
        if constexpr (PIPE > 3) step(IntC<3>{}, lc);
      };
      const bool more = c0 + 64 < m;
      int r0 = c0;
      for (; r0 < (more ? ce - PIPE : ce); r0 += PIPE) iter(r0, IntC<0>{});
      if (more) iter(r0, IntC<1>{});
      shift_ids();
    }
  }
  emit(part, FP8 ? v_ref / kPScale : 1.f);
  if constexpr (NQ == 1) {
    if (part > part0) {  // the parked first partition
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[0][j][r] = stash[4 * j + r][lane];
      m_run[0] = stash[4 * NT][lane];
      l_acc[0] = stash[4 * NT + 1][lane];
      emit(part0, 1.f);
    }
  }
}

// ---------------------------------------------------------------- reduce
// Workgroups of PA_RED_THREADS threads; D/4 lanes per query row (sequence,
// query token, query head), each lane merging 4 consecutive dims with 16-byte
// loads.  Partitions that hold tokens visible to the
// row are merged in partition order (deterministic).  With the
// length-balanced split, rows of single-partition units were written by the
// attention kernel and are left alone.  (One workgroup of D threads per row,
// with 4-byte loads, measured 2-3x slower on the multi-query steps.)
template <int D, bool HEAD>
__global__ __launch_bounds__(PA_RED_THREADS) void reduce_kernel(AttnArgs a) {
  constexpr int LPR = D / 4;                 // lanes per row
  constexpr int RPG = PA_RED_THREADS / LPR;  // rows per workgroup
  const int sub = threadIdx.x / LPR;
  const int d0 = (threadIdx.x - sub * LPR) * 4;
  const int Hq = a.num_q_heads;
  const int T = a.q_len;
  const int qrow = blockIdx.x * RPG + sub;
  if (qrow >= a.batch * T * Hq) return;   // (no barrier in this kernel)
  const int b = qrow / (T * Hq);
  const int rem = qrow - b * T * Hq;
  const int t = rem / Hq;
  const int hq = rem - t * Hq;
  const int h = hq / a.group;
  const int row = HEAD ? b * a.num_kv_heads + h : b;
  const int cap = a.table_width * kPageSize;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int vis = L - T + t + 1;   // tokens this row sees (T = 1: all L)
  const int npages = vis > 0 ? (vis + kPageSize - 1) / kPageSize : 0;
  // partials of this row: fixed partitions [row][Pn]; planned [slot][column],
  // slots first * hpg + h_in_group, stepping by hpg per partition
  int chunk = a.chunk_pages, nparts = a.num_parts;
  size_t pi0 = (size_t)qrow * nparts, step = 1;
  if (a.plan != nullptr) {
    const int hpg = HEAD ? 1 : a.num_kv_heads;
    const int grp = HEAD ? row : b;
    const int first = a.plan[2 + grp];
    chunk = a.plan[0];
    nparts = a.plan[3 + grp] - first;
    const int C = a.group * T;
    pi0 = ((size_t)first * hpg + (HEAD ? 0 : h)) * C + t * a.group + (hq - h * a.group);
    step = (size_t)hpg * C;
  }
  const int nvp = min(nparts, (npages + chunk - 1) / chunk);
  bool flagged;
  if (a.unit_flags != nullptr) {   // HEAD with the check: the sequence's unit words
    uint32_t word = 0u;
    for (int u = 0; u < a.num_kv_heads; ++u) word |= a.unit_flags[(size_t)b * a.num_kv_heads + u];
    flagged = word != 0u;
    if (a.write_flags && rem == 0 && d0 == 0) a.flags_out[b] = word;   // the sequence's first row
  } else {
    flagged = a.flags != nullptr && a.flags[b] != 0u;
  }
  uint16_t* orow = a.out + (size_t)qrow * D + d0;
  if (flagged || nvp == 0) {
    *reinterpret_cast<u32x2*>(orow) = u32x2{0u, 0u};
    return;
  }
  // written by the attention kernel: a planned group's only partition, or a
  // unit whose pages all lie in the first of the fixed partitions
  if (a.plan != nullptr ? nparts == 1 : (L + kPageSize - 1) / kPageSize <= chunk) return;
  const float* ml = a.part_ml + pi0 * 2;
  const float* po = a.part_o + pi0 * D + d0;
  // Partitions in groups of 8 (16 for rows with more than 8), every load of a
  // group issued before use; a running (max, sum, O) merges the groups in
  // partition order.  Measured on MI355X: groups of 16 throughout cost 30% on
  // rows of 4 partitions, groups of 8 cost 12% on rows of about 40.
  float M = -INFINITY, lsum = 0.f;
  f32x4 osum = f32x4{0.f, 0.f, 0.f, 0.f};
  auto merge = [&](auto grp) {
    constexpr int kGrp = decltype(grp)::value;
    for (int p0 = 0; p0 < nvp; p0 += kGrp) {
      float m[kGrp], l[kGrp];
      f32x4 o[kGrp];
#pragma unroll
      for (int j = 0; j < kGrp; ++j) {
        const bool ok = p0 + j < nvp;
        m[j] = ok ? ml[2 * step * (p0 + j)] : -INFINITY;
        l[j] = ok ? ml[2 * step * (p0 + j) + 1] : 0.f;
        o[j] = ok ? *reinterpret_cast<const f32x4*>(po + step * (p0 + j) * D)
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      float Mg = M;
#pragma unroll
      for (int j = 0; j < kGrp; ++j) Mg = fmaxf(Mg, m[j]);
      const float r = __builtin_amdgcn_exp2f(M - Mg);  // M = -inf on the first group: r = 0
      lsum *= r;
#pragma unroll
      for (int c = 0; c < 4; ++c) osum[c] *= r;
#pragma unroll
      for (int j = 0; j < kGrp; ++j) {
        const float f = __builtin_amdgcn_exp2f(m[j] - Mg);  // empty slots: exp2(-inf) = 0
        lsum += l[j] * f;
#pragma unroll
        for (int c = 0; c < 4; ++c) osum[c] += o[j][c] * f;
      }
      M = Mg;
    }
  };
  if (nvp > 8) merge(IntC<16>{});
  else merge(IntC<8>{});
  const uint32_t lo = (uint32_t)bf16_rne(osum[0] / lsum) | ((uint32_t)bf16_rne(osum[1] / lsum) << 16);
  const uint32_t hi = (uint32_t)bf16_rne(osum[2] / lsum) | ((uint32_t)bf16_rne(osum[3] / lsum) << 16);
  *reinterpret_cast<u32x2*>(orow) = u32x2{lo, hi};
  if (a.row_ml != nullptr && d0 == 0) {   // scored decode: the row's final (max, sum)
    a.row_ml[(size_t)qrow * 2 + 0] = M;
    a.row_ml[(size_t)qrow * 2 + 1] = lsum;
  }
}

template <int D, bool FP8, bool HEAD, int NQ, bool CAUSAL, bool SHARED = false>
hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  unsigned grid;
  if (a.plan != nullptr) {  // enough waves for the most pairs a plan can hold; the rest exit
    const unsigned pairs = (unsigned)a.max_pairs;
    if (a.xcd_order) grid = ((pairs + 7) / 8) * 8 * (unsigned)(a.num_kv_heads / kWaves);
    else grid = (pairs * (HEAD ? 1u : (unsigned)a.num_kv_heads) + kWaves - 1) / kWaves;
  } else {
    const int ppw = NQ == 1 ? a.parts_per_wave : 1;
    const unsigned groups = (unsigned)(a.num_parts + ppw - 1) / ppw;
    if (a.xcd_order) {  // see attention_kernel: (Hkv / 4) workgroups per pair, in blocks of 8 pairs
      const unsigned pairs = (unsigned)a.batch * groups;
      grid = ((pairs + 7) / 8) * 8 * (unsigned)(a.num_kv_heads / kWaves);
    } else if (a.col_blocks > 1) {  // see attention_kernel: a unit's workgroups on one XCD
      const unsigned wgu = SHARED ? ((unsigned)(a.col_blocks + kWaves - 1) / kWaves) * groups
                                  : ((unsigned)a.col_blocks * groups + kWaves - 1) / kWaves;
      const unsigned units = (unsigned)a.batch * a.num_kv_heads;
      grid = ((units + 7) / 8) * 8 * wgu;
    } else {
      const unsigned items = (unsigned)a.batch * a.num_kv_heads * a.col_blocks * groups;
      grid = (items + kWaves - 1) / kWaves;
    }
  }
  hipLaunchKernelGGL((attention_kernel<D, FP8, HEAD, NQ, CAUSAL, SHARED>), dim3(grid),
                     dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

// Column tiles: one for plain decode; for T query tokens, ceil(G * T / 16)
// rounded up to 1, 2 or 4.
template <int D, bool FP8, bool HEAD>
hipError_t launch_attention_q(const AttnArgs& a, hipStream_t s) {
  if (a.q_len == 1) return launch_attention_t<D, FP8, HEAD, 1, false>(a, s);
  // prefill column blocks of kPrefillCols: the page-sharing kernel
  if (a.col_blocks > 1 && kPrefillCols == 32) return launch_attention_t<D, FP8, HEAD, 2, true, true>(a, s);
  const int cols = a.group * a.q_len;
  if (cols <= 16) return launch_attention_t<D, FP8, HEAD, 1, true>(a, s);
  if (cols <= 32) return launch_attention_t<D, FP8, HEAD, 2, true>(a, s);
  return launch_attention_t<D, FP8, HEAD, 4, true>(a, s);
}

// ------------------------------------------------------ eviction scores
// Second pass of a scored decode step, for the eviction policy of "Making
// Workers AI faster and more efficient" (KV cache compression section: the
// entries that have drawn the least attention go first).  The weight of token
// j in row (b, query head) is exp2(s_j - M) / L, with (M, L) the row's final
// log2-domain max and sum: they exist only once the decode and its reduce have
// finished.  This kernel reads the K pages again, recomputes the scores with
// the attention kernel's operands and MFMA sequence (so s is bitwise the same),
// and adds each token's weights, summed over the G query heads of its KV head,
// to the paged score array.  Rereading K (half the decode's bytes) costs less
// than writing every score out of the decode and reading it back: G * 64 bytes
// per page and head each way, a write stream that measured about 45% of the
// decode kernel's time when it ran inside it.
//
// One wave per (unit, run of at most 128 pages).  The runs come from a
// length-balanced plan of their own (plan_block; chunk between 16 and 128
// pages, about 4096 waves of equal work): with runs of a fixed length a
// ragged batch left few waves running at the end.  A SEQ pair's heads are
// neighbouring waves, so a workgroup reads neighbouring head blocks of the
// same pages.
// Lane (c, q4) owns query head c and tokens 4*q4 .. 4*q4+3 of each page; the
// sum over heads is a butterfly across the 16 lanes of a DPP row (fixed
// order: deterministic).  The page's 16 sums go to the wave's own LDS rows,
// and the scores are read, added to and written once, after the run's last
// page.  A score access inside the page loop stalls the K stream: vector
// loads and stores share one in-order completion counter, so the next K wait
// also waits for it (measured on the 32K-token FP8 workload: reads or writes
// of the scores every 64 pages each cost about a quarter of the kernel time).
#ifndef PA_MASS_PIPE
#define PA_MASS_PIPE 2         // pages held in registers per wave
#endif
#ifndef PA_MASS_THROTTLE
#define PA_MASS_THROTTLE 1     // wait for a page's loads before requesting the next
#endif
static_assert(PA_MASS_PIPE >= 2 && PA_MASS_PIPE <= 6, "pipeline depth");

// Sum over the 16 lanes of each DPP row; every lane gets the (same) total.
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

template <int D, bool FP8, bool HEAD>
__global__ __launch_bounds__(256) void mass_kernel(AttnArgs a) {
  constexpr int E = FP8 ? 1 : 2;
  constexpr int BLOCK = kPageSize * D * E;
  constexpr int NSEG = BLOCK / 1024;
  constexpr int NSTEP = D / 32;
  constexpr int PIPE = PA_MASS_PIPE;
  const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Runs from the score pass's own length-balanced plan (chunk <= kMassRun
  // pages), heads of a SEQ pair in neighbouring waves.
  const int hpg = HEAD ? 1 : Hkv;
  const int item = blockIdx.x * kWaves + wave;
  const int pair = item / hpg;
  if (pair >= a.plan[1]) return;
  const int chunk = a.plan[0];
  const int grp = a.plan_group[pair];
  const int part = pair - a.plan[2 + grp];
  const int b = HEAD ? grp / Hkv : grp;
  const int h = HEAD ? grp - b * Hkv : item - pair * hpg;
  if (a.flags != nullptr && a.flags[b] != 0u) return;   // aborted request: no update
  const int unit = b * Hkv + h;
  const int row = HEAD ? unit : b;
  const int cap = a.table_width * kPageSize;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int p0 = part * chunk;
  const int p1 = min(p0 + chunk, npages);
  if (p0 >= p1) return;
  const int n = min(p1 - p0, kMassRun);   // the plan's runs are never longer
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, q4 = lane >> 4;
  const bool col = c < G;
  const size_t qrow = (size_t)b * Hq + h * G + (col ? c : 0);

  // Q^T operand and the lane's row (max, 1/sum), as in the attention kernel
  bf16x8 qop[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int d0 = FP8 ? 64 * (s >> 1) + 16 * q4 + 8 * (s & 1) : 32 * s + 8 * q4;
    u32x4 v = *reinterpret_cast<const u32x4*>(a.q + qrow * D + d0);
    if (!col) v = u32x4{0u, 0u, 0u, 0u};
    qop[s] = __builtin_bit_cast(bf16x8, v);
  }
  const float M = a.row_ml[qrow * 2 + 0];
  const float inv = 1.f / a.row_ml[qrow * 2 + 1];

  const int32_t* bt = a.block_table + (size_t)row * a.table_width + p0;
  const size_t page_stride = HEAD ? (size_t)BLOCK : (size_t)Hkv * BLOCK;
  const uint8_t* kpool = a.k_pages + (HEAD ? 0 : (size_t)h * BLOCK);
  const float* kscale = FP8 ? a.k_scale + (HEAD ? 0 : h) : nullptr;
  const int scale_stride = HEAD ? 1 : Hkv;
  const int lane_off = (c * 4 + q4) * 16;

  // The run's page ids (and FP8 scales), one lane per page, loaded and waited
  // for before the page loop (see the attention kernel).
  constexpr int kIdRegs = kMassRun / 64;
  int ids[kIdRegs];
  float sks[FP8 ? kIdRegs : 1];
#pragma unroll
  for (int j = 0; j < kIdRegs; ++j) {
    const int k = 64 * j + lane;
    ids[j] = k < n ? bt[k] : 0;
  }
  int last = __builtin_amdgcn_readfirstlane(ids[kIdRegs - 1]);
  asm volatile("" : : "s"(last));
  if constexpr (FP8) {
#pragma unroll
    for (int j = 0; j < kIdRegs; ++j) {
      const int pid = (unsigned)ids[j] < (unsigned)a.num_pages ? ids[j] : 0;
      sks[j] = kscale[(size_t)pid * scale_stride];
    }
  }
  static_assert(kIdRegs == 2, "one register per 64 pages");
  auto lane_reg = [&](const auto (&v)[kIdRegs], int r) { return r < 64 ? v[0] : v[1]; };

  u32x4 kr[PIPE][NSEG];
  float ks[PIPE];
  auto load = [&](int slot, int r) __attribute__((always_inline)) {   // r: page within the run, uniform
    const int raw = __builtin_amdgcn_readlane(lane_reg(ids, r), r & 63);
    const int pid = (unsigned)raw < (unsigned)a.num_pages ? raw : 0;
    const uint8_t* kp = kpool + (size_t)pid * page_stride;
#pragma unroll
    for (int i = 0; i < NSEG; ++i) kr[slot][i] = load16(kp + lane_off + i * 1024);
    if constexpr (FP8)
      ks[slot] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_reg(sks, r)), r & 63));
  };

  // The run's score sums: row k holds page k's 16 tokens.
  __shared__ f32x4 s_mass[kWaves][kMassRun][4];
  f32x4 (*mass)[4] = s_mass[wave];

  auto compute = [&](int slot, int k) __attribute__((always_inline)) {
    const int page = p0 + k;
    float kfac = a.score_scale_log2;
    if (FP8) kfac *= ks[slot];
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      if (FP8) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x2 lo = fp8x4_to_bf16x4(kr[slot][i][2 * hh]);
          u32x2 hi = fp8x4_to_bf16x4(kr[slot][i][2 * hh + 1]);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qop[2 * i + hh], acc, 0, 0, 0);
        }
      } else {
        const bf16x8 av = __builtin_bit_cast(bf16x8, kr[slot][i]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qop[i], acc, 0, 0, 0);
      }
    }
    const int tok0 = page * kPageSize + q4 * 4;
    f32x4 w;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sc = acc[r] * kfac;
      w[r] = (col && tok0 + r < L) ? __builtin_amdgcn_exp2f(sc - M) * inv : 0.f;
      w[r] = row16_sum(w[r]);
    }
    if (c == 0) mass[k][q4] = w;
  };

  // Register ring of PIPE pages with the attention kernel's throttle (one
  // page in flight besides the one being consumed: measured best here too).
#pragma unroll
  for (int u = 0; u < PIPE - 1; ++u) load(u, min(u, n - 1));
  for (int r0 = 0; r0 < n; r0 += PIPE) {
#pragma unroll
    for (int u = 0; u < PIPE; ++u) {
      const int r = r0 + u;
      if constexpr (PA_MASS_THROTTLE) __builtin_amdgcn_s_waitcnt(0x0F70);   // s_waitcnt vmcnt(0)
      load((u + PIPE - 1) % PIPE, min(r + PIPE - 1, n - 1));
      if (r < n) compute(u, r);
    }
  }

  // The run's scores, 16 pages per instruction: lane (page k = 16 * it +
  // lane / 4, quarter e = lane % 4) reads, adds and writes tokens 4e .. 4e+3
  // of page k, so each page's 64 bytes come from four neighbouring lanes.
  // Ids out of range (tag check off) have no page to credit; slots past L
  // keep their bits.
  constexpr int kIt = kMassRun / 16;
  const int e = lane & 3;
  f32x4 v[kIt];
  float* dst[kIt];
  int valid[kIt];   // tokens of the lane's page below L; <= 0: nothing to do
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    const int k = 16 * it + (lane >> 2);
    const int id = __shfl(ids[it >> 2], k & 63);
    const bool live = k < n && (unsigned)id < (unsigned)a.num_pages;
    valid[it] = live ? L - (p0 + k) * kPageSize : 0;
    const size_t slot0 = HEAD ? (size_t)(live ? id : 0) * kPageSize
                              : ((size_t)(live ? id : 0) * Hkv + h) * kPageSize;
    dst[it] = a.scores + slot0 + 4 * e;
    v[it] = live ? *reinterpret_cast<const f32x4*>(dst[it]) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int it = 0; it < kIt; ++it) {
    if (valid[it] <= 0) continue;
    const f32x4 add = mass[16 * it + (lane >> 2)][e];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (4 * e + t < valid[it]) v[it][t] += add[t];
    *reinterpret_cast<f32x4*>(dst[it]) = v[it];   // each (page, head, slot) belongs to one unit
  }
}

template <int D, bool FP8, bool HEAD>
hipError_t launch_mass_t(const AttnArgs& a, hipStream_t s) {
  const unsigned items = (unsigned)a.max_pairs * (HEAD ? 1u : (unsigned)a.num_kv_heads);
  hipLaunchKernelGGL((mass_kernel<D, FP8, HEAD>), dim3((items + kWaves - 1) / kWaves),
                     dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep(const ValidateArgs* v, const PlanArgs* p0, const PlanArgs* p1,
                       const AppendArgs* app, hipStream_t s) {
  if (!p0 && p1) return launch_prep(v, p1, nullptr, app, s);
  const int nval = v ? v->rows : 0;
  const int nplan = (p0 ? 1 : 0) + (p1 ? 1 : 0);
  const int64_t items = app ? (int64_t)app->batch * app->num_kv_heads * app->pages_per_unit : 0;
  const ValidateArgs va = v ? *v : ValidateArgs{};
  const PlanArgs pa0 = p0 ? *p0 : PlanArgs{}, pa1 = p1 ? *p1 : PlanArgs{};
  if (items > 0) {
    const unsigned grid = (unsigned)(nval + nplan + (items + 3) / 4);
    const int it = (int)items;
    if (app->head_dim == 128) {
      if (app->fp8)
        hipLaunchKernelGGL((step_prep_kernel<128, true>), dim3(grid), dim3(1024), 0, s, *app, it,
                           va, pa0, pa1, nval, nplan);
      else
        hipLaunchKernelGGL((step_prep_kernel<128, false>), dim3(grid), dim3(1024), 0, s, *app, it,
                           va, pa0, pa1, nval, nplan);
    } else {
      if (app->fp8)
        hipLaunchKernelGGL((step_prep_kernel<64, true>), dim3(grid), dim3(1024), 0, s, *app, it,
                           va, pa0, pa1, nval, nplan);
      else
        hipLaunchKernelGGL((step_prep_kernel<64, false>), dim3(grid), dim3(1024), 0, s, *app, it,
                           va, pa0, pa1, nval, nplan);
    }
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)(nval + nplan);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prep_kernel, dim3(grid), dim3(1024), 0, s, va, pa0, pa1, nval);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, bool fp8, bool head_layout,
                            hipStream_t s) {
  if (head_dim == 128) {
    if (fp8) return head_layout ? launch_attention_q<128, true, true>(a, s)
                                : launch_attention_q<128, true, false>(a, s);
    return head_layout ? launch_attention_q<128, false, true>(a, s)
                       : launch_attention_q<128, false, false>(a, s);
  }
  if (fp8) return head_layout ? launch_attention_q<64, true, true>(a, s)
                              : launch_attention_q<64, true, false>(a, s);
  return head_layout ? launch_attention_q<64, false, true>(a, s)
                     : launch_attention_q<64, false, false>(a, s);
}

hipError_t launch_reduce(const AttnArgs& a, int head_dim, bool head_layout, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.q_len * a.num_q_heads;
  const int rpg = PA_RED_THREADS / (head_dim / 4);   // rows per workgroup (reduce_kernel)
  const unsigned grid = (unsigned)((rows + rpg - 1) / rpg);
  const dim3 blk(PA_RED_THREADS);
  if (head_dim == 128) {
    if (head_layout) hipLaunchKernelGGL((reduce_kernel<128, true>), dim3(grid), blk, 0, s, a);
    else hipLaunchKernelGGL((reduce_kernel<128, false>), dim3(grid), blk, 0, s, a);
  } else {
    if (head_layout) hipLaunchKernelGGL((reduce_kernel<64, true>), dim3(grid), blk, 0, s, a);
    else hipLaunchKernelGGL((reduce_kernel<64, false>), dim3(grid), blk, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_mass(const AttnArgs& a, int head_dim, bool fp8, bool head_layout, hipStream_t s) {
  if (head_dim == 128) {
    if (fp8) return head_layout ? launch_mass_t<128, true, true>(a, s) : launch_mass_t<128, true, false>(a, s);
    return head_layout ? launch_mass_t<128, false, true>(a, s) : launch_mass_t<128, false, false>(a, s);
  }
  if (fp8) return head_layout ? launch_mass_t<64, true, true>(a, s) : launch_mass_t<64, true, false>(a, s);
  return head_layout ? launch_mass_t<64, false, true>(a, s) : launch_mass_t<64, false, false>(a, s);
}

}  // namespace pa
