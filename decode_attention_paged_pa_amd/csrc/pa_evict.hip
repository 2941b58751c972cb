// Eviction support ("Making Workers AI faster and more efficient", section
// "KV cache compression goes open source"): the cache drops the KV entries
// that past attention used least, like a least-frequently-used policy, and
// the per-head block table lets each head keep a different number of tokens.
//
//   score_kernel    adds a decode step's attention mass per cached token to
//                   fp32 scores stored like the pages ([P][heads][S]), so a
//                   token's score moves with its page;
//   compact_kernel  rewrites the tokens each unit keeps, in order, into the
//                   pages of a new table (FP8: decoded under the old page
//                   scale, re-quantised under the new page's own scale);
//   compact_flags_kernel  range checks of a compaction, one flags word per
//                   sequence.
#include "pa_block.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#pragma clang fp contract(off)

// --------------------------------------------------------------- scores
// Workgroup (unit, group of 16 pages).  The mass of a token is
// sum_g exp2(s_g - M_g) / L_g over the G query heads of the unit, with
// (M_g, L_g) the row's final log2-domain max and sum, and s_g the score the
// attention kernel wrote for that token.  The 16 pages' scores are one
// contiguous run of 16 * G * 16 floats: they are read in 16-byte chunks by
// consecutive threads, turned into weights in LDS, then summed over g in a
// fixed order (deterministic) by one thread per token.
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ float s_m[kMaxGroup], s_inv[kMaxGroup];
  __shared__ f32x4 s_w[16 * kMaxGroup * 4];
  const int unit = blockIdx.x;
  const int Hkv = a.num_kv_heads, G = a.group;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int row = a.head_layout ? unit : b;
  if (a.flags != nullptr && a.flags[b] != 0u) return;   // aborted request: no update
  const int cap = a.table_width * kPageSize;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int i0 = blockIdx.y * 16;                        // first page of this workgroup
  if (i0 >= npages) return;
  const int np = min(16, npages - i0);
  if (threadIdx.x < G) {
    const size_t qrow = (size_t)b * a.num_q_heads + h * G + threadIdx.x;
    s_m[threadIdx.x] = a.row_ml[qrow * 2 + 0];
    s_inv[threadIdx.x] = 1.f / a.row_ml[qrow * 2 + 1];
  }
  __syncthreads();
  const f32x4* src = reinterpret_cast<const f32x4*>(a.logits + ((size_t)unit * a.table_width + i0) * G * 16);
  for (int i = threadIdx.x; i < np * G * 4; i += blockDim.x) {
    const int g = (i >> 2) % G;
    const f32x4 v = src[i];
    f32x4 wt;
#pragma unroll
    for (int r = 0; r < 4; ++r) wt[r] = __builtin_amdgcn_exp2f(v[r] - s_m[g]) * s_inv[g];
    s_w[i] = wt;
  }
  __syncthreads();
  const int pl = threadIdx.x >> 4, slot = threadIdx.x & 15;
  const int t = (i0 + pl) * kPageSize + slot;
  if (pl >= np || t >= L) return;
  const int pid = a.block_table[(size_t)row * a.table_width + i0 + pl];
  if ((unsigned)pid >= (unsigned)a.num_pages) return;   // no page to credit (unchecked ids)
  const float* w = reinterpret_cast<const float*>(s_w) + pl * G * 16 + slot;
  float mass = 0.f;
  for (int g = 0; g < G; ++g) mass += w[g * 16];
  float* sc = a.scores + ((a.head_layout ? (size_t)pid : (size_t)pid * Hkv + h) * kPageSize + slot);
  *sc = *sc + mass;   // each (page, head, slot) belongs to exactly one unit
}

// ----------------------------------------------------------- compaction
// One workgroup per (unit, destination page).  Token s of destination page j
// is kept token j*16 + s of the unit.  Invalid positions and page ids are
// skipped here (the flags kernel reports them).
template <int D, bool FP8>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  constexpr int E = FP8 ? 1 : 2;
  constexpr int BLOCK_ELEMS = kPageSize * D;
  constexpr int PER = kPageSize * D / 256;     // elements of one block per thread
  __shared__ int s_src_blk[kPageSize];         // old block of each token (-1: skip)
  __shared__ int s_src_vblk[kPageSize];
  __shared__ int s_src_slot[kPageSize];
  __shared__ float s_ksc[kPageSize], s_vsc[kPageSize];
  __shared__ float s_red[2][4];

  const int unit = blockIdx.x / a.pages_per_unit;
  const int j = blockIdx.x - unit * a.pages_per_unit;
  const int Hkv = a.num_kv_heads;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int row = a.head_layout ? unit : b;
  const int cap = a.table_width * kPageSize;
  int n = a.n_keep[row];
  n = min(min(n, a.keep_stride), cap);
  const int cnt = min(kPageSize, n - j * kPageSize);
  if (cnt <= 0) return;
  const int pid_new = a.new_table[(size_t)row * a.table_width + j];
  if ((unsigned)pid_new >= (unsigned)a.num_pages) return;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const size_t blk_new = a.head_layout ? (size_t)pid_new : (size_t)pid_new * Hkv + h;
  const size_t vblk_new = v_block_slot(pid_new, h, Hkv, a.num_pages, a.head_layout);

  if (threadIdx.x < kPageSize) {
    const int s = threadIdx.x;
    int blk = -1, vblk = -1, slot = 0;
    if (s < cnt) {
      const int pos = a.keep[((size_t)unit * a.keep_stride) + j * kPageSize + s];
      if (pos >= 0 && pos < L) {
        const int pid = a.block_table[(size_t)row * a.table_width + pos / kPageSize];
        if ((unsigned)pid < (unsigned)a.num_pages) {
          blk = (int)(a.head_layout ? (size_t)pid : (size_t)pid * Hkv + h);
          vblk = (int)v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout);
          slot = pos % kPageSize;
          if (FP8) {
            s_ksc[s] = a.k_scale[blk];
            s_vsc[s] = a.v_scale[blk];
          }
          if (a.scores != nullptr)
            a.scores[blk_new * kPageSize + s] = a.scores[(size_t)blk * kPageSize + slot];
        }
      }
    }
    s_src_blk[s] = blk;
    s_src_vblk[s] = vblk;
    s_src_slot[s] = slot;
  }
  __syncthreads();

  if (!FP8) {
    const uint16_t* ko = reinterpret_cast<const uint16_t*>(a.k_old);
    const uint16_t* vo = reinterpret_cast<const uint16_t*>(a.v_old);
    uint16_t* kn = reinterpret_cast<uint16_t*>(a.k_new) + blk_new * BLOCK_ELEMS;
    uint16_t* vn = reinterpret_cast<uint16_t*>(a.v_new) + vblk_new * BLOCK_ELEMS;
    for (int e = threadIdx.x; e < cnt * D; e += blockDim.x) {
      const int s = e / D, d = e - s * D;
      if (s_src_blk[s] < 0) continue;
      const int so = s_src_slot[s];
      kn[k_elem<D, E>(s, d)] = ko[(size_t)s_src_blk[s] * BLOCK_ELEMS + k_elem<D, E>(so, d)];
      vn[v_elem<D, E>(s, d)] = vo[(size_t)s_src_vblk[s] * BLOCK_ELEMS + v_elem<D, E>(so, d)];
    }
    return;
  }

  // FP8: x = fl32(dec(c) * s_old) for every kept value, then amax, s_new, codes.
  float xk[PER], xv[PER];
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = r * 256 + threadIdx.x;
    const int s = e / D, d = e - s * D;
    xk[r] = xv[r] = 0.f;
    if (s < cnt && s_src_blk[s] >= 0) {
      const int so = s_src_slot[s];
      xk[r] = __fmul_rn(e4m3_to_f32(a.k_old[(size_t)s_src_blk[s] * BLOCK_ELEMS + k_elem<D, E>(so, d)]),
                        s_ksc[s]);
      xv[r] = __fmul_rn(e4m3_to_f32(a.v_old[(size_t)s_src_vblk[s] * BLOCK_ELEMS + v_elem<D, E>(so, d)]),
                        s_vsc[s]);
      mk = fmaxf(mk, fabsf(xk[r]));
      mv = fmaxf(mv, fabsf(xv[r]));
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    mk = fmaxf(mk, __shfl_xor(mk, off, 64));
    mv = fmaxf(mv, __shfl_xor(mv, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    s_red[0][threadIdx.x >> 6] = mk;
    s_red[1][threadIdx.x >> 6] = mv;
  }
  __syncthreads();
  mk = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  mv = fmaxf(fmaxf(s_red[1][0], s_red[1][1]), fmaxf(s_red[1][2], s_red[1][3]));
  const float sk = __fdiv_rn(mk, 448.0f), sv = __fdiv_rn(mv, 448.0f);
  uint8_t* kn = a.k_new + blk_new * BLOCK_ELEMS;
  uint8_t* vn = a.v_new + vblk_new * BLOCK_ELEMS;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int e = r * 256 + threadIdx.x;
    const int s = e / D, d = e - s * D;
    if (s < cnt && s_src_blk[s] >= 0) {
      kn[k_elem<D, E>(s, d)] = sk == 0.f ? (uint8_t)0 : (uint8_t)e4m3_rne_sat(__fdiv_rn(xk[r], sk));
      vn[v_elem<D, E>(s, d)] = sv == 0.f ? (uint8_t)0 : (uint8_t)e4m3_rne_sat(__fdiv_rn(xv[r], sv));
    }
  }
  if (threadIdx.x == 0) {
    a.k_scale[blk_new] = sk;
    a.v_scale[blk_new] = sv;
  }
}

// One workgroup per sequence: bit 1 an old or new page id out of range for a
// token that would move, bit 2 a length or keep count above the table's
// capacity (or a count above keep_stride), bit 3 a keep position outside
// [0, len).  Overwrites flags[b].
__global__ __launch_bounds__(256) void compact_flags_kernel(CompactArgs a) {
  __shared__ uint32_t s_bits;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_bits = 0;
  __syncthreads();
  uint32_t bits = 0;
  const int cap = a.table_width * kPageSize;
  for (int h = 0; h < a.num_kv_heads; ++h) {
    const int unit = b * a.num_kv_heads + h;
    const int row = a.head_layout ? unit : b;
    int n = a.n_keep[row];
    int L = a.lens[row];
    if (n > cap || n > a.keep_stride || L > cap || L < 0) bits |= 4u;
    n = max(0, min(min(n, a.keep_stride), cap));
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int32_t* kp = a.keep + (size_t)unit * a.keep_stride;
    const int32_t* bt = a.block_table + (size_t)row * a.table_width;
    const int32_t* nt = a.new_table + (size_t)row * a.table_width;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int pos = kp[i];
      if (pos < 0 || pos >= L) {
        bits |= 8u;
        continue;
      }
      if ((unsigned)bt[pos / kPageSize] >= (unsigned)a.num_pages) bits |= 2u;
      if (i % kPageSize == 0 && (unsigned)nt[i / kPageSize] >= (unsigned)a.num_pages) bits |= 2u;
    }
  }
  if (bits) atomicOr(&s_bits, bits);  // LDS atomic
  __syncthreads();
  if (threadIdx.x == 0) a.flags[b] = s_bits;
}

}  // namespace

hipError_t launch_score(const ScoreArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.batch * a.num_kv_heads, (unsigned)(a.table_width + 15) / 16);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.batch * a.num_kv_heads * a.pages_per_unit;
  if (grid > 0) {
    if (a.head_dim == 128) {
      if (a.fp8) hipLaunchKernelGGL((compact_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((compact_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
    } else {
      if (a.fp8) hipLaunchKernelGGL((compact_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
      else hipLaunchKernelGGL((compact_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.flags == nullptr) return hipSuccess;
  hipLaunchKernelGGL(compact_flags_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
