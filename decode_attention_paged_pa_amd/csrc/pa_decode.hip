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
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

// A page maximum may exceed the running maximum by this many log2 units
// before the accumulators are rescaled; weights stay below 2^8, which fp32
// sums and f16/bf16 MFMA operands hold without loss of range.
constexpr float kRescaleSlack = 8.0f;

// ------------------------------------------------------------ validation
// One workgroup per sequence; integrity check of the pages it will read
// ("Cloudflare quantizes Kimi and GLM caches for 41% faster inference",
// integrity-check paragraph: a separate batch validation before decode reads).
__global__ __launch_bounds__(256) void validate_kernel(ValidateArgs a) {
  __shared__ uint32_t s_bits;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_bits = 0;
  __syncthreads();
  uint32_t bits = 0;
  const int cap = a.table_width * kPageSize;
  const int n_units = a.head_layout ? a.num_kv_heads : 1;
  for (int u = 0; u < n_units; ++u) {
    const int row = a.head_layout ? b * a.num_kv_heads + u : b;
    int L = a.lens[row];
    if (L > cap || L < 0) bits |= 4u;
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int n = (L + kPageSize - 1) / kPageSize;
    const int32_t* bt = a.block_table + (size_t)row * a.table_width;
    const uint32_t* ex = a.expected_tags ? a.expected_tags + (size_t)row * a.table_width : nullptr;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const int pid = bt[i];
      if ((unsigned)pid >= (unsigned)a.num_pages) {
        bits |= 2u;
      } else if (ex && ex[i] != a.page_tags[pid]) {
        bits |= 1u;
      }
    }
  }
  if (bits) atomicOr(&s_bits, bits);  // LDS atomic
  __syncthreads();
  if (threadIdx.x == 0) a.flags[b] = s_bits;
}

// ------------------------------------------------------------- attention
// Grid: one workgroup per (unit, partition), unit = (sequence, KV head).
// A partition is a run of chunk_pages pages of the unit; its 4 waves split it
// into contiguous sub-runs, each keeping its own (max, sum, O) and merging
// through LDS at the end.
template <int D, bool FP8, bool HEAD>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  constexpr int E = FP8 ? 1 : 2;               // bytes per cached element
  constexpr int BLOCK = kPageSize * D * E;     // bytes of one (page, head) block
  constexpr int NSEG = BLOCK / 1024;           // 16-byte loads per lane per block
  constexpr int NT = D / 16;                   // 16-dim output tiles
  constexpr int NSTEP = D / 32;                // QK MFMA steps over d

  __shared__ float s_o[kWaves][kMaxGroup][D];
  __shared__ float s_m[kWaves][kMaxGroup];
  __shared__ float s_l[kWaves][kMaxGroup];

  const int Pn = a.num_parts;
  const int unit = blockIdx.x / Pn;
  const int part = blockIdx.x - unit * Pn;
  const int Hkv = a.num_kv_heads, G = a.group, Hq = a.num_q_heads;
  const int b = unit / Hkv;
  const int h = unit - b * Hkv;
  const int row = HEAD ? unit : b;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;      // MFMA row/column index owned by this lane
  const int q4 = lane >> 4;     // which quarter of the MFMA K dimension

  const int cap = a.table_width * kPageSize;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int p0 = part * a.chunk_pages;
  const int p1 = min(p0 + a.chunk_pages, npages);
  const bool flagged = a.flags != nullptr && a.flags[b] != 0u;
  if (flagged || p0 >= p1) {
    if (Pn == 1) {  // no reduce follows: this workgroup owns the output rows
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
        const int g = i / D, d = i - g * D;
        a.out[((size_t)b * Hq + h * G + g) * D + d] = 0;
      }
    }
    return;
  }
  const int np = p1 - p0;
  const int per = (np + kWaves - 1) / kWaves;
  const int w0 = p0 + wave * per;
  const int w1 = min(w0 + per, p1);

  // Q^T as the B operand of S^T = K Q^T: lane (c, q4) holds query g = c and
  // the 8 dims that the K A-operand places in this lane for each step.
  bf16x8 qop[NSTEP];
  {
    const uint16_t* qrow = a.q + ((size_t)b * Hq + h * G + (c < G ? c : 0)) * D;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      int d0;
      if (FP8) d0 = 64 * (s >> 1) + 16 * q4 + 8 * (s & 1);
      else d0 = 32 * s + 8 * q4;
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + d0);
      if (c >= G) v = u32x4{0u, 0u, 0u, 0u};
      qop[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_acc = 0.f;

  const int32_t* bt = a.block_table + (size_t)row * a.table_width;
  const size_t page_stride = HEAD ? (size_t)BLOCK : (size_t)Hkv * BLOCK;
  const size_t head_off = HEAD ? 0 : (size_t)h * BLOCK;
  const int lane_off = (c * 4 + q4) * 16;
  const uint8_t* kbase = a.k_pages + head_off + lane_off;
  const uint8_t* vbase = a.v_pages + head_off + lane_off;

  for (int base = w0; base < w1; base += 64) {
    const int cnt = min(64, w1 - base);
    int pid_l = lane < cnt ? bt[base + lane] : 0;
    pid_l = ((unsigned)pid_l < (unsigned)a.num_pages) ? pid_l : 0;
    float ks_l = 1.f, vs_l = 1.f;
    if (FP8) {
      const size_t si = HEAD ? (size_t)pid_l : (size_t)pid_l * Hkv + h;
      ks_l = a.k_scale[si];
      vs_l = a.v_scale[si];
    }

    auto load = [&](u32x4 (&kr)[NSEG], u32x4 (&vr)[NSEG], int k) {
      const int pid = __builtin_amdgcn_readlane(pid_l, k);
      const uint8_t* kp = kbase + (size_t)pid * page_stride;
      const uint8_t* vp = vbase + (size_t)pid * page_stride;
#pragma unroll
      for (int i = 0; i < NSEG; ++i) {
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + i * 1024));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + i * 1024));
      }
    };

    auto compute = [&](const u32x4 (&kr)[NSEG], const u32x4 (&vr)[NSEG], int k) {
      const int page = base + k;
      float kfac = a.score_scale_log2;
      float vsc = 1.f;
      if (FP8) {
        kfac *= __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ks_l), k));
        vsc = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(vs_l), k));
      }
      // ---- scores S^T (token rows x query columns)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NSEG; ++i) {
        if (FP8) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            u32x2 lo = fp8x4_to_bf16x4(kr[i][2 * hh]);
            u32x2 hi = fp8x4_to_bf16x4(kr[i][2 * hh + 1]);
            u32x4 av = {lo.x, lo.y, hi.x, hi.y};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                          qop[2 * i + hh], acc, 0, 0, 0);
          }
        } else {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[i]), qop[i],
                                                        acc, 0, 0, 0);
        }
      }
      // lane (c, q4) now holds the scores of query c for tokens 4*q4 + r
      const int tok0 = page * kPageSize + q4 * 4;
      const bool tail = page * kPageSize + kPageSize > L;
      float sc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[r] = acc[r] * kfac;
      if (tail) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < L) ? sc[r] : -INFINITY;
      }
      float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mloc = col_max(mloc);
      if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_acc *= alpha;
#pragma unroll
        for (int j = 0; j < NT; ++j) o[j] *= alpha;
        m_run = m_new;
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sc[r] - m_run);
      l_acc += (p[0] + p[1]) + (p[2] + p[3]);

      // ---- O^T += V^T P^T; zero V of tokens past L (poisoned slots)
      uint32_t vmask32 = 0xFFFFFFFFu;
      uint64_t vmask64 = ~0ull;
      if (tail) {
        const int nv = min(max(L - tok0, 0), 4);
        vmask32 = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
        vmask64 = nv >= 4 ? ~0ull : ((1ull << (16 * nv)) - 1ull);
      }
      if (FP8) {
        f16x4 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = (_Float16)(p[r] * vsc);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const uint32_t w = vr[j >> 2][j & 3] & vmask32;
          o[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(fp8x4_to_f16x4(w), pb, o[j], 0, 0, 0);
        }
      } else {
        i16x4 pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[r] = __builtin_bit_cast(short, (__bf16)p[r]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const u32x4& seg = vr[j >> 1];
          uint64_t w = ((uint64_t)seg[2 * (j & 1) + 1] << 32) | seg[2 * (j & 1)];
          w &= vmask64;
          o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, w), pb, o[j],
                                                           0, 0, 0);
        }
      }
    };

    u32x4 kA[NSEG], vA[NSEG], kB[NSEG], vB[NSEG];
    load(kA, vA, 0);
    int k = 0;
    for (; k + 1 < cnt; k += 2) {
      load(kB, vB, k + 1);
      compute(kA, vA, k);
      if (k + 2 < cnt) load(kA, vA, k + 2);
      compute(kB, vB, k + 1);
    }
    if (k < cnt) compute(kA, vA, k);
  }

  // ---- merge the waves of this workgroup
  const float l_tot = col_sum(l_acc);
  if (c < G) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[wave][c][16 * j + 4 * q4 + r] = o[j][r];
    }
    if (q4 == 0) {
      s_m[wave][c] = m_run;
      s_l[wave][c] = l_tot;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
      lsum += s_l[w][g] * f;
      osum += s_o[w][g][d] * f;
    }
    const size_t qrow = (size_t)b * Hq + h * G + g;
    if (Pn == 1) {
      a.out[qrow * D + d] = bf16_rne(osum / lsum);
    } else {
      a.part_o[(qrow * Pn + part) * D + d] = osum;
      if (d == 0) {
        a.part_ml[(qrow * Pn + part) * 2 + 0] = M;
        a.part_ml[(qrow * Pn + part) * 2 + 1] = lsum;
      }
    }
  }
}

// ---------------------------------------------------------------- reduce
// One workgroup per (sequence, query head); thread d merges dim d over the
// partitions that hold tokens, in partition order (deterministic).
template <int D, bool HEAD>
__global__ __launch_bounds__(D) void reduce_kernel(AttnArgs a) {
  const int qrow = blockIdx.x;
  const int Hq = a.num_q_heads;
  const int b = qrow / Hq;
  const int hq = qrow - b * Hq;
  const int h = hq / a.group;
  const int row = HEAD ? b * a.num_kv_heads + h : b;
  const int d = threadIdx.x;
  const int cap = a.table_width * kPageSize;
  int L = a.lens[row];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int nvp = (npages + a.chunk_pages - 1) / a.chunk_pages;
  const bool flagged = a.flags != nullptr && a.flags[b] != 0u;
  if (flagged || nvp == 0) {
    a.out[(size_t)qrow * D + d] = 0;
    return;
  }
  const int Pn = a.num_parts;
  const float* ml = a.part_ml + (size_t)qrow * Pn * 2;
  const float* po = a.part_o + (size_t)qrow * Pn * D + d;
  float M = ml[0];
  for (int p = 1; p < nvp; ++p) M = fmaxf(M, ml[2 * p]);
  float lsum = 0.f, osum = 0.f;
  for (int p = 0; p < nvp; ++p) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * p] - M);
    lsum += ml[2 * p + 1] * f;
    osum += po[(size_t)p * D] * f;
  }
  a.out[(size_t)qrow * D + d] = bf16_rne(osum / lsum);
}

template <int D, bool FP8, bool HEAD>
hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.batch * a.num_kv_heads * a.num_parts;
  hipLaunchKernelGGL((attention_kernel<D, FP8, HEAD>), dim3(grid), dim3(64 * kWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_validate(const ValidateArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(validate_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int head_dim, bool fp8, bool head_layout,
                            hipStream_t s) {
  if (head_dim == 128) {
    if (fp8) return head_layout ? launch_attention_t<128, true, true>(a, s)
                                : launch_attention_t<128, true, false>(a, s);
    return head_layout ? launch_attention_t<128, false, true>(a, s)
                       : launch_attention_t<128, false, false>(a, s);
  }
  if (fp8) return head_layout ? launch_attention_t<64, true, true>(a, s)
                              : launch_attention_t<64, true, false>(a, s);
  return head_layout ? launch_attention_t<64, false, true>(a, s)
                     : launch_attention_t<64, false, false>(a, s);
}

hipError_t launch_reduce(const AttnArgs& a, int head_dim, bool head_layout, hipStream_t s) {
  const unsigned grid = (unsigned)a.batch * a.num_q_heads;
  if (head_dim == 128) {
    if (head_layout) hipLaunchKernelGGL((reduce_kernel<128, true>), dim3(grid), dim3(128), 0, s, a);
    else hipLaunchKernelGGL((reduce_kernel<128, false>), dim3(grid), dim3(128), 0, s, a);
  } else {
    if (head_layout) hipLaunchKernelGGL((reduce_kernel<64, true>), dim3(grid), dim3(64), 0, s, a);
    else hipLaunchKernelGGL((reduce_kernel<64, false>), dim3(grid), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pa
