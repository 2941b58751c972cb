// Append kernels: scatter new K/V tokens into their pages through the block
// table, quantising to OCP FP8 e4m3 with per-(page, head) scales when the
// cache is FP8 ("Cloudflare quantizes Kimi and GLM caches for 41% faster
// inference", KV cache quantization paragraph; pages assigned on demand, "How
// we built the most efficient inference engine for Cloudflare's network",
// section "Batching to feed the Tensor Cores").
//
// The quantisation is bit-exact by construction: every fp32 step is an IEEE
// correctly rounded operation written out explicitly (no contraction), and
// the e4m3 rounding is done on the integer bits.
#include "pa_block.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

#pragma clang fp contract(off)

// One workgroup per (unit, touched page).  Grid slot j of a unit is its j-th
// page counted from the page holding its first new token.
template <int D, bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int E = FP8 ? 1 : 2;
  constexpr int BLOCK_ELEMS = kPageSize * D;
  __shared__ float s_red[2][4];
  __shared__ float s_old[2];

  const int unit = blockIdx.x / a.pages_per_unit;
  const int j = blockIdx.x - unit * a.pages_per_unit;
  const int Hkv = a.num_kv_heads;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int row = a.head_layout ? unit : b;
  const int lo = a.lens_old[row];
  const int n = min(a.n_new[row], a.n_max);  // never read past the n_max inputs
  if (lo < 0 || n <= 0) return;
  const int cap = a.table_width * kPageSize;
  const int i = lo / kPageSize + j;
  const int pos_lo = max(lo, i * kPageSize);
  const int pos_hi = min(min(lo + n, (i + 1) * kPageSize), cap);
  if (pos_lo >= pos_hi) return;
  const int pid = a.block_table[(size_t)row * a.table_width + i];
  if ((unsigned)pid >= (unsigned)a.num_pages) return;
  const int slot0 = pos_lo - i * kPageSize;
  const int cnt = pos_hi - pos_lo;
  const int t0 = pos_lo - lo;  // index of the first token in k_new / v_new

  const size_t blk = a.head_layout ? (size_t)pid : (size_t)pid * Hkv + h;
  const size_t src0 = (((size_t)b * Hkv + h) * a.n_max + t0) * D;
  const uint16_t* ks = a.k_new + src0;
  const uint16_t* vs = a.v_new + src0;

  if (!FP8) {
    uint16_t* kb = reinterpret_cast<uint16_t*>(a.k_pages) + blk * BLOCK_ELEMS;
    uint16_t* vb = reinterpret_cast<uint16_t*>(a.v_pages) +
                   v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout) * BLOCK_ELEMS;
    for (int e = threadIdx.x; e < cnt * D; e += blockDim.x) {
      const int s = e / D, d = e - s * D;
      kb[k_elem<D, E>(slot0 + s, d)] = ks[e];
      vb[v_elem<D, E>(slot0 + s, d)] = vs[e];
    }
    return;
  }

  uint8_t* kb = a.k_pages + blk * BLOCK_ELEMS;
  uint8_t* vb = a.v_pages + v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout) * BLOCK_ELEMS;
  // amax of the new values, K and V separately
  float mk = 0.f, mv = 0.f;
  for (int e = threadIdx.x; e < cnt * D; e += blockDim.x) {
    mk = fmaxf(mk, fabsf(bf16_value(ks[e])));
    mv = fmaxf(mv, fabsf(bf16_value(vs[e])));
  }
  if (threadIdx.x == 0) {
    s_old[0] = slot0 == 0 ? 0.f : a.k_scale[blk];  // a write at slot 0 starts the page afresh
    s_old[1] = slot0 == 0 ? 0.f : a.v_scale[blk];
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

  for (int which = 0; which < 2; ++which) {
    uint8_t* pb = which ? vb : kb;
    const uint16_t* src = which ? vs : ks;
    const float so = s_old[which];
    const float amax = which ? mv : mk;
    const float cand = __fdiv_rn(amax, 448.0f);
    const float sn = so > cand ? so : cand;  // max(s_old, fl32(amax / 448))
    if (sn > so && slot0 > 0) {
      for (int e = threadIdx.x; e < slot0 * D; e += blockDim.x) {
        const int t = e / D, d = e - t * D;
        const int off = which ? v_elem<D, E>(t, d) : k_elem<D, E>(t, d);
        const float back = __fmul_rn(e4m3_to_f32(pb[off]), so);
        pb[off] = (uint8_t)e4m3_rne_sat(__fdiv_rn(back, sn));
      }
    }
    for (int e = threadIdx.x; e < cnt * D; e += blockDim.x) {
      const int s = e / D, d = e - s * D;
      const int off = which ? v_elem<D, E>(slot0 + s, d) : k_elem<D, E>(slot0 + s, d);
      pb[off] = sn == 0.f ? (uint8_t)0 : (uint8_t)e4m3_rne_sat(__fdiv_rn(bf16_value(src[e]), sn));
    }
    if (threadIdx.x == 0) (which ? a.v_scale : a.k_scale)[blk] = sn;
  }
}

// One thread per sequence: range and length bits of this append.
__global__ __launch_bounds__(256) void append_flags_kernel(AppendArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  const int cap = a.table_width * kPageSize;
  const int n_units = a.head_layout ? a.num_kv_heads : 1;
  uint32_t bits = 0;
  for (int u = 0; u < n_units; ++u) {
    const int row = a.head_layout ? b * a.num_kv_heads + u : b;
    const int lo = a.lens_old[row];
    const int n = min(a.n_new[row], a.n_max);
    if (n <= 0) continue;
    if (lo < 0 || lo + n > cap) bits |= 4u;
    if (lo < 0) continue;
    const int hi = min(lo + n, cap);
    const int32_t* bt = a.block_table + (size_t)row * a.table_width;
    for (int i = lo / kPageSize; i * kPageSize < hi; ++i) {
      if ((unsigned)bt[i] >= (unsigned)a.num_pages) bits |= 2u;
    }
  }
  a.flags[b] = bits;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.batch * a.num_kv_heads * a.pages_per_unit;
  if (grid == 0) {
    // nothing to write; only the flags (if asked for) are produced below
  } else if (a.head_dim == 128) {
    if (a.fp8) hipLaunchKernelGGL((append_kernel<128, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((append_kernel<128, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (a.fp8) hipLaunchKernelGGL((append_kernel<64, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((append_kernel<64, false>), dim3(grid), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.flags == nullptr) return e;
  hipLaunchKernelGGL(append_flags_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
