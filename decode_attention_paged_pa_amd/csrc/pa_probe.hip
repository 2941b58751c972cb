// HBM read-ceiling probes (pa_probe.h): a contiguous stream and a block
// gather, loading with the decode kernel's instructions -- one 16-byte
// non-temporal load per lane, so each wave access is 1 KiB contiguous -- and
// doing nothing else with the data than folding it into one word per wave.
// The decode step's roofline is the HBM read rate ("How we built the most
// efficient inference engine for Cloudflare's network", section "Batching to
// feed the Tensor Cores": every decoded token revisits all cached K/V), and
// these kernels measure what that rate is for the two patterns, on the GPU
// the library runs on.
#include "pa.h"
#include "pa_probe.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#define PA_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWaves = 4;   // waves per workgroup

__device__ inline u32x4 nt_load(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ inline uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ inline uint32_t wave_xor(uint32_t x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d, 64);
  return x;
}

// Wave w reads bytes [w * span, (w + 1) * span), 4 KiB per iteration (four
// loads in flight per lane).  span is a multiple of 1024.
__global__ __launch_bounds__(64 * kProbeWaves) void stream_kernel(const uint8_t* buf, int64_t span,
                                                                  uint32_t* sink) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kProbeWaves + wave;
  const uint8_t* p = buf + w * span + lane * 16;
  uint32_t acc = 0;
  int64_t off = 0;
  for (; off + 4096 <= span; off += 4096) {
    const u32x4 a = nt_load(p + off), b = nt_load(p + off + 1024);
    const u32x4 c = nt_load(p + off + 2048), d = nt_load(p + off + 3072);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; off < span; off += 1024) acc ^= fold(nt_load(p + off));
  acc = wave_xor(acc);
  if (lane == 0) sink[w] = acc;
}

// Wave w reads the blocks its run of ids names, INF blocks per batch (all
// their loads issued, then consumed), the run's ids loaded 64 at a time (one
// per lane) and read with readlane.
template <int NSEG, int INF>
__global__ __launch_bounds__(64 * kProbeWaves) void gather_kernel(const uint8_t* pool,
                                                                  int64_t n_blocks,
                                                                  const int32_t* ids, int ipw,
                                                                  uint32_t* sink) {
  constexpr int64_t kBlock = 1024 * NSEG;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kProbeWaves + wave;
  const int32_t* run = ids + w * ipw;
  const uint8_t* base = pool + lane * 16;
  uint32_t acc = 0;
  for (int b0 = 0; b0 < ipw; b0 += 64) {
    int id = b0 + lane < ipw ? run[b0 + lane] : 0;
    id = (id >= 0 && (int64_t)id < n_blocks) ? id : 0;
    const int m = min(64, ipw - b0);   // a multiple of INF
    for (int r = 0; r < m; r += INF) {
      u32x4 v[INF][NSEG];
#pragma unroll
      for (int i = 0; i < INF; ++i) {
        const int64_t pid = __builtin_amdgcn_readlane(id, r + i);
#pragma unroll
        for (int s = 0; s < NSEG; ++s) v[i][s] = nt_load(base + pid * kBlock + s * 1024);
      }
#pragma unroll
      for (int i = 0; i < INF; ++i)
#pragma unroll
        for (int s = 0; s < NSEG; ++s) acc ^= fold(v[i][s]);
    }
  }
  acc = wave_xor(acc);
  if (lane == 0) sink[w] = acc;
}

template <int NSEG>
hipError_t launch_gather(int inflight, dim3 grid, hipStream_t s, const uint8_t* pool,
                         int64_t n_blocks, const int32_t* ids, int ipw, uint32_t* sink) {
  const dim3 blk(64 * kProbeWaves);
  switch (inflight) {
    case 1: hipLaunchKernelGGL((gather_kernel<NSEG, 1>), grid, blk, 0, s, pool, n_blocks, ids, ipw, sink); break;
    case 2: hipLaunchKernelGGL((gather_kernel<NSEG, 2>), grid, blk, 0, s, pool, n_blocks, ids, ipw, sink); break;
    case 4: hipLaunchKernelGGL((gather_kernel<NSEG, 4>), grid, blk, 0, s, pool, n_blocks, ids, ipw, sink); break;
    default: hipLaunchKernelGGL((gather_kernel<NSEG, 8>), grid, blk, 0, s, pool, n_blocks, ids, ipw, sink); break;
  }
  return hipGetLastError();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

PA_API int pa_probe_stream(const void* buf, size_t bytes, int32_t waves, uint32_t* sink,
                           hipStream_t stream) {
  if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4)) return PA_ERR_INVALID_ARG;
  if (waves <= 0 || waves % kProbeWaves != 0) return PA_ERR_INVALID_ARG;
  if (bytes == 0 || bytes % (1024 * (size_t)waves) != 0) return PA_ERR_INVALID_ARG;
  const int64_t span = (int64_t)(bytes / (size_t)waves);
  hipLaunchKernelGGL(stream_kernel, dim3(waves / kProbeWaves), dim3(64 * kProbeWaves), 0, stream,
                     static_cast<const uint8_t*>(buf), span, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_API int pa_probe_gather(const void* pool, size_t pool_bytes, const int32_t* ids, int32_t waves,
                           int32_t ids_per_wave, int32_t block_bytes, int32_t inflight,
                           uint32_t* sink, hipStream_t stream) {
  if (!pool || !ids || !sink || !aligned(pool, 16) || !aligned(ids, 4) || !aligned(sink, 4))
    return PA_ERR_INVALID_ARG;
  if (waves <= 0 || waves % kProbeWaves != 0) return PA_ERR_INVALID_ARG;
  if (block_bytes != 1024 && block_bytes != 2048 && block_bytes != 4096) return PA_ERR_INVALID_ARG;
  if (inflight != 1 && inflight != 2 && inflight != 4 && inflight != 8) return PA_ERR_INVALID_ARG;
  if (ids_per_wave <= 0 || ids_per_wave % inflight != 0) return PA_ERR_INVALID_ARG;
  if (pool_bytes < (size_t)block_bytes) return PA_ERR_INVALID_ARG;
  const int64_t n_blocks = (int64_t)(pool_bytes / (size_t)block_bytes);
  const dim3 grid(waves / kProbeWaves);
  const uint8_t* p = static_cast<const uint8_t*>(pool);
  hipError_t e;
  if (block_bytes == 1024) e = launch_gather<1>(inflight, grid, stream, p, n_blocks, ids, ids_per_wave, sink);
  else if (block_bytes == 2048) e = launch_gather<2>(inflight, grid, stream, p, n_blocks, ids, ids_per_wave, sink);
  else e = launch_gather<4>(inflight, grid, stream, p, n_blocks, ids, ids_per_wave, sink);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
