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
  __shared__ float s_red[2][4];
  __shared__ float s_old[2];
  append_item<D, FP8, 256>(a, blockIdx.x, true, threadIdx.x, s_red, s_old);
}

// One thread per sequence: range and length bits of this append, and with
// expected tags, bit 0 for a page it would write whose tag is not the
// expected one (that page is left alone).
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
      const int p = bt[i];
      if ((unsigned)p >= (unsigned)a.num_pages) {
        bits |= 2u;
      } else if (a.expected_tags &&
                 a.expected_tags[(size_t)row * a.table_width + i] != a.page_tags[p]) {
        bits |= 1u;
      }
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
