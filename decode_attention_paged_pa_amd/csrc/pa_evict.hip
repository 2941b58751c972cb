// Eviction support ("Making Workers AI faster and more efficient", section
// "KV cache compression goes open source"): the cache drops the KV entries
// that past attention used least, like a least-frequently-used policy, and
// the per-head block table lets each head keep a different number of tokens.
// The scores themselves (fp32, stored like the pages, [P][heads][S], so a
// token's score moves with its page) are updated by the decode's second pass
// (mass_kernel, with the decode kernels).
//
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

// ----------------------------------------------------------- compaction
// One wave per (unit, destination page); token s of destination page j is
// kept token j*16 + s of the unit.  Lanes 0..15 look up their token's source
// (old block, slot, FP8 scales) and every chunk reads it from them by lane
// shuffle, so a wave needs no LDS and no barrier, and four independent pages
// share each workgroup.  Work goes by 16-byte chunks of the destination
// blocks (the layout pa.h documents), 2 * BLOCK / 1024 chunks per lane:
//   a K chunk holds 16/E consecutive dims of one token, so it comes whole
//   from one chunk of the token's old block;
//   a V chunk holds, for one dim column c and 4 consecutive tokens, 4/E tiles
//   of 4 tokens; its 4 tokens come from 4 old chunks (possibly 4 old pages),
//   4/E elements each.
// FP8 values are decoded under their old page's scale; the new page's K and
// V amax are reduced over the wave, then every chunk is re-encoded.  Slots
// past the kept count and tokens with an invalid position keep the bytes
// they had (the flags kernel reports the invalid ones).
template <int D, bool FP8>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  constexpr int E = FP8 ? 1 : 2;
  constexpr int CE = 16 / E;                   // elements per 16-byte chunk
  constexpr int TPC = CE / 4;                  // V: tiles (dims) per chunk
  constexpr int BLOCK = kPageSize * D * E;
  constexpr int NCH = BLOCK / 16;              // chunks per block (K or V)
  constexpr int CPL = 2 * NCH / 64;            // chunks per lane

  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = item / a.pages_per_unit;
  if (unit >= a.batch * a.num_kv_heads) return;
  const int j = item - unit * a.pages_per_unit;
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

  // lane s < cnt: the source of destination slot s (blk -1: nothing to write)
  int my_blk = -1, my_vblk = 0, my_slot = 0;
  float my_ksc = 0.f, my_vsc = 0.f;
  if (lane < cnt) {
    const int pos = a.keep[((size_t)unit * a.keep_stride) + j * kPageSize + lane];
    if (pos >= 0 && pos < L) {
      const int pid = a.block_table[(size_t)row * a.table_width + pos / kPageSize];
      if ((unsigned)pid < (unsigned)a.num_pages) {
        my_blk = (int)(a.head_layout ? (size_t)pid : (size_t)pid * Hkv + h);
        my_vblk = (int)v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout);
        my_slot = pos % kPageSize;
        if (FP8) {
          my_ksc = a.k_scale[my_blk];
          my_vsc = a.v_scale[my_blk];
        }
      }
    }
  }
  // The scores move last: a store issued before the gathers would be waited
  // for with them.
  auto move_scores = [&]() {
    if (a.scores != nullptr && my_blk >= 0)
      a.scores[blk_new * kPageSize + lane] = a.scores[(size_t)my_blk * kPageSize + my_slot];
  };

  const u32x4* kold = reinterpret_cast<const u32x4*>(a.k_old);
  const u32x4* vold = reinterpret_cast<const u32x4*>(a.v_old);
  u32x4* knew = reinterpret_cast<u32x4*>(a.k_new) + blk_new * NCH;
  u32x4* vnew = reinterpret_cast<u32x4*>(a.v_new) + vblk_new * NCH;

  // Gather every chunk of this lane first (all loads in flight together).
  // K chunk kc = (seg, t, q): token t, dims seg*4*CE + q*CE ... + CE - 1.
  // V chunk vc = (jh, c, t4): element jl*4 + i is token 4*t4 + i, dim
  // (jh*TPC + jl)*16 + c.
  u32x4 raw[CPL];
  uint32_t valid[CPL];
  float esc[CPL][4];   // FP8: the source scale of the chunk's token(s)
#pragma unroll
  for (int r = 0; r < CPL; ++r) {
    const int ch = r * 64 + lane;
    raw[r] = u32x4{0u, 0u, 0u, 0u};
    valid[r] = 0;
    if (ch < NCH) {
      const int t = (ch >> 2) & 15;
      const int blk = __shfl(my_blk, t, 64);
      const int so = __shfl(my_slot, t, 64);
      esc[r][0] = esc[r][1] = esc[r][2] = esc[r][3] = __shfl(my_ksc, t, 64);
      if (blk >= 0) {
        raw[r] = kold[(size_t)blk * NCH + ((ch >> 6) << 6) + so * 4 + (ch & 3)];
        valid[r] = (1u << CE) - 1u;
      }
    } else {
      const int vc = ch - NCH;
      const int t4 = vc & 3, colbase = vc >> 2;   // colbase = jh * 16 + c
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * t4 + i;
        const int blk = __shfl(my_blk, t, 64);
        const int vblk = __shfl(my_vblk, t, 64);
        const int so = __shfl(my_slot, t, 64);
        esc[r][i] = __shfl(my_vsc, t, 64);
        if (blk < 0) continue;
        const u32x4 sc = vold[(size_t)vblk * NCH + colbase * 4 + (so >> 2)];
        // element jl*4 + i <- element jl*4 + (so & 3) of the source chunk
#pragma unroll
        for (int jl = 0; jl < TPC; ++jl) {
          const int se = jl * 4 + (so & 3), de = jl * 4 + i;
          uint32_t v;
          if (E == 1) v = (sc[se >> 2] >> (8 * (se & 3))) & 0xFFu;
          else v = (sc[se >> 1] >> (16 * (se & 1))) & 0xFFFFu;
          if (E == 1) w[de >> 2] |= v << (8 * (de & 3));
          else w[de >> 1] |= v << (16 * (de & 1));
          valid[r] |= 1u << de;
        }
      }
      raw[r] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }

  // Merge `fresh` into destination chunk ch where `valid` says so.
  auto put = [&](int ch, u32x4 fresh, uint32_t vmask) {
    u32x4* dst = ch < NCH ? knew + ch : vnew + (ch - NCH);
    constexpr uint32_t all = (1u << CE) - 1u;
    if ((vmask & all) == all) {
      *dst = fresh;
      return;
    }
    if (vmask == 0) return;
    u32x4 old = *dst;
#pragma unroll
    for (int e = 0; e < CE; ++e) {
      if (!((vmask >> e) & 1u)) continue;
      const uint32_t m = E == 1 ? (0xFFu << (8 * (e & 3))) : (0xFFFFu << (16 * (e & 1)));
      const int wi = E == 1 ? (e >> 2) : (e >> 1);
      old[wi] = (old[wi] & ~m) | (fresh[wi] & m);
    }
    *dst = old;
  };

  if constexpr (!FP8) {
#pragma unroll
    for (int r = 0; r < CPL; ++r) put(r * 64 + lane, raw[r], valid[r]);
    move_scores();
    return;
  } else {
    // FP8: x = fl32(dec(c) * s_old), decoded with gfx950's pair conversions
    // (four codes per two instructions) once for the amax over the wave and
    // again for the re-encode under s_new, rather than kept: 64 more live
    // registers would cost this latency-bound kernel waves per SIMD.  The
    // encode is the fp32 -> OCP e4m3 pair conversion: round to nearest even,
    // sign kept on underflow, and equal to the saturating definition
    // (e4m3_rne_sat) for every finite |v| <= 464, which holds every quotient
    // here (|x| <= amax, s_new = fl32(amax / 448)); checked exhaustively on
    // MI355X.
    auto decode4 = [&](int r, int w4, float (&x)[4]) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(raw[r][w4], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(raw[r][w4], true);
      const float dec[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = w4 * 4 + i;
        x[i] = ((valid[r] >> e) & 1u) ? __fmul_rn(dec[i], esc[r][e & 3]) : 0.f;
      }
    };
    float mk = 0.f, mv = 0.f;
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      const bool is_k = r * 64 + lane < NCH;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        float x[4];
        decode4(r, w4, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (is_k) mk = fmaxf(mk, fabsf(x[i]));
          else mv = fmaxf(mv, fabsf(x[i]));
        }
      }
    }
    for (int off = 32; off >= 1; off >>= 1) {
      mk = fmaxf(mk, __shfl_xor(mk, off, 64));
      mv = fmaxf(mv, __shfl_xor(mv, off, 64));
    }
    const float sk = __fdiv_rn(mk, 448.0f), sv = __fdiv_rn(mv, 448.0f);
#pragma unroll
    for (int r = 0; r < CPL; ++r) {
      if (valid[r] == 0) continue;
      const bool is_k = r * 64 + lane < NCH;
      const float s_new = is_k ? sk : sv;
      u32x4 enc = u32x4{0u, 0u, 0u, 0u};
      if (s_new != 0.f) {
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          float x[4];
          decode4(r, w4, x);
          int word = 0;
          word = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x[0], s_new), __fdiv_rn(x[1], s_new),
                                                 word, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x[2], s_new), __fdiv_rn(x[3], s_new),
                                                 word, true);
          enc[w4] = (uint32_t)word;
        }
      }
      put(r * 64 + lane, enc, valid[r]);   // only the valid elements are written
    }
    if (lane == 0) {
      a.k_scale[blk_new] = sk;
      a.v_scale[blk_new] = sv;
    }
    move_scores();
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

hipError_t launch_compact(const CompactArgs& a, hipStream_t s) {
  const unsigned items = (unsigned)a.batch * a.num_kv_heads * a.pages_per_unit;
  const unsigned grid = (items + 3) / 4;   // one wave per destination page
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
