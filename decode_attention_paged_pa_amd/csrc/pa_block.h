// Device helpers shared by the kernels that write cache blocks (append and
// compaction): element offsets inside a (page, head) block, the exact
// fp32 -> OCP e4m3 rounding, and the work of one append item.  The layout is
// the one pa.h documents.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Element offset of K(t, d) inside a (page, head) block: 64-byte column
// segments of 4*CE elements, CE = elements per 16-byte chunk.
template <int D, int E>
__device__ __forceinline__ int k_elem(int t, int d) {
  constexpr int SEG = 64 / E;
  return (d / SEG) * (kPageSize * SEG) + t * SEG + (d % SEG);
}

// Element offset of V(t, d): transposed, token-minor 16 x 4 tiles, grouped so
// that each 16-byte chunk holds TPC tiles of 4 tokens for one dim column.
template <int D, int E>
__device__ __forceinline__ int v_elem(int t, int d) {
  constexpr int TPC = 4 / E;
  const int c = d & 15, j = d >> 4;
  return ((((j / TPC) * 16 + c) * 4 + (t >> 2)) * TPC + (j % TPC)) * 4 + (t & 3);
}

// fp32 -> e4m3 code: saturate magnitudes above 448, round to nearest even on
// the integer bits, keep the sign of values that round to zero, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  if (a > 0x43E00000u) a = 0x43E00000u;          // 448.0f
  uint32_t mag;
  if (a < 0x3C800000u) {                          // below 2^-6: subnormal grid of 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
  } else {
    const uint32_t e = (a >> 23) - 120u;          // unbiased + 7
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rest = a & 0xFFFFFu;
    const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    mag = ((e << 3) | keep) + up;                 // a mantissa carry bumps the exponent
  }
  return sign | mag;
}

__device__ __forceinline__ float bf16_value(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

// One append item: unit item / pages_per_unit and the j-th page counted from
// the page holding the unit's first new token (the new tokens of several
// pages of one unit are separate items).  NTH threads (whole waves; tid in
// [0, NTH)) share the item, and s_red / s_old are theirs alone.  The cache is
// stored as FP8 e4m3 ("Cloudflare quantizes Kimi and GLM caches for 41%
// faster inference", KV cache quantization paragraph); that page gives no
// scale formula, and the rule used here is this library's reading: each FP8
// page-head keeps scale = amax / 448 (448 being e4m3's largest finite value)
// over everything written since the page started.  The new tokens' amax may
// raise it, and then the page's earlier codes are re-quantised.
//
// A page is written only through a table entry whose expected tag (when the
// request gives them) is the page's current tag: the integrity check of
// "Cloudflare quantizes Kimi and GLM caches for 41% faster inference"
// (integrity-check paragraph) protects requests that share GPU memory, and a
// stale entry names a page that may now hold another request's tokens.
//
// Every thread passes the FP8 path's one barrier exactly once, whether or not
// its item writes anything (inactive items, items past the unit's last page,
// unwritable pages), so items of different units may share a workgroup.
// WHOLE compiles the FP8 path for whole pages written afresh (below); the
// decode step's appends (a few tokens per unit) leave it out.
template <int D, bool FP8, int NTH, bool WHOLE = true>
__device__ void append_item(const AppendArgs& a, int item, bool active, int tid,
                            float (&s_red)[2][NTH / 64], float (&s_old)[2]) {
#pragma clang fp contract(off)
  constexpr int E = FP8 ? 1 : 2;
  constexpr int NW = NTH / 64;
  constexpr int BLOCK_ELEMS = kPageSize * D;
  const int Hkv = a.num_kv_heads;
  const int unit = active ? item / a.pages_per_unit : 0;
  const int j = item - unit * a.pages_per_unit;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const int row = a.head_layout ? unit : b;
  int cnt = 0, slot0 = 0, t0 = 0, pid = 0;   // cnt = 0: nothing to write
  if (active) {
    const int lo = a.lens_old[row];
    const int n = min(a.n_new[row], a.n_max);  // never read past the n_max inputs
    if (lo >= 0 && n > 0) {
      const int cap = a.table_width * kPageSize;
      const int i = lo / kPageSize + j;
      const int pos_lo = max(lo, i * kPageSize);
      const int pos_hi = min(min(lo + n, (i + 1) * kPageSize), cap);
      if (pos_lo < pos_hi) {
        const size_t e = (size_t)row * a.table_width + i;
        const int p = a.block_table[e];
        if ((unsigned)p < (unsigned)a.num_pages &&
            (a.expected_tags == nullptr || a.expected_tags[e] == a.page_tags[p])) {
          pid = p;
          slot0 = pos_lo - i * kPageSize;
          cnt = pos_hi - pos_lo;
          t0 = pos_lo - lo;   // index of the first token in k_new / v_new
        }
      }
    }
  }
  const size_t blk = a.head_layout ? (size_t)pid : (size_t)pid * Hkv + h;
  const size_t src0 = (((size_t)b * Hkv + h) * a.n_max + t0) * D;
  const uint16_t* ks = a.k_new + src0;
  const uint16_t* vs = a.v_new + src0;

  if constexpr (!FP8) {
    if (cnt == 0) return;
    uint16_t* kb = reinterpret_cast<uint16_t*>(a.k_pages) + blk * BLOCK_ELEMS;
    uint16_t* vb = reinterpret_cast<uint16_t*>(a.v_pages) +
                   v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout) * BLOCK_ELEMS;
    if (cnt == kPageSize && ((reinterpret_cast<uintptr_t>(a.k_new) |
                              reinterpret_cast<uintptr_t>(a.v_new)) & 15) == 0) {
      // A whole page from 16-byte aligned inputs (bulk and chunk appends):
      // K rows keep runs of 32 dims of a token together, so 8 dims move as
      // one 16-byte copy; V is stored token-minor, so a thread reads 4
      // tokens x 8 dims and writes each dim's 4 tokens as 8 bytes.
      for (int e = tid; e < kPageSize * D / 8; e += NTH) {
        const int s = e / (D / 8), d = (e - s * (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(kb + k_elem<D, E>(s, d)) =
            *reinterpret_cast<const u32x4*>(ks + s * D + d);
      }
      for (int e = tid; e < (kPageSize / 4) * (D / 8); e += NTH) {
        const int tq = e / (D / 8), d0 = (e - tq * (D / 8)) * 8;
        u32x4 r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = *reinterpret_cast<const u32x4*>(vs + (4 * tq + i) * D + d0);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int sh = 16 * (dd & 1);
          const uint32_t t0v = (r[0][dd >> 1] >> sh) & 0xFFFFu, t1v = (r[1][dd >> 1] >> sh) & 0xFFFFu;
          const uint32_t t2v = (r[2][dd >> 1] >> sh) & 0xFFFFu, t3v = (r[3][dd >> 1] >> sh) & 0xFFFFu;
          *reinterpret_cast<u32x2*>(vb + v_elem<D, E>(4 * tq, d0 + dd)) =
              u32x2{t0v | (t1v << 16), t2v | (t3v << 16)};
        }
      }
      return;
    }
    for (int e = tid; e < cnt * D; e += NTH) {
      const int s = e / D, d = e - s * D;
      kb[k_elem<D, E>(slot0 + s, d)] = ks[e];
      vb[v_elem<D, E>(slot0 + s, d)] = vs[e];
    }
    return;
  } else {
    uint8_t* kb = a.k_pages + blk * BLOCK_ELEMS;
    uint8_t* vb =
        a.v_pages + v_block_slot(pid, h, Hkv, a.num_pages, a.head_layout) * BLOCK_ELEMS;
    // A whole page written afresh (slot 0, 16 tokens) from 16-byte aligned
    // inputs, as bulk and chunk appends write them: the values are loaded 16
    // bytes at a time and kept in registers across the barrier, and the codes
    // go out as 8-byte K runs (8 dims of a token) and 4-byte V runs (4
    // tokens of a dim).  Each element's arithmetic is the same as below.
    const bool whole = WHOLE && cnt == kPageSize && slot0 == 0 &&
                       ((reinterpret_cast<uintptr_t>(a.k_new) |
                         reinterpret_cast<uintptr_t>(a.v_new)) & 15) == 0;
    constexpr int KC = kPageSize * D / 8;            // K: 8 dims of a token each
    constexpr int VC = (kPageSize / 4) * (D / 8);    // V: 4 tokens x 8 dims each
    constexpr int KPT = (KC + NTH - 1) / NTH, VPT = (VC + NTH - 1) / NTH;
    u32x4 kw[KPT], vw[VPT][4];
    auto elem = [](const u32x4& w, int k) { return bf16_value((uint16_t)(w[k >> 1] >> (16 * (k & 1)))); };
    // amax of the new values, K and V separately
    float mk = 0.f, mv = 0.f;
    if (whole) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int e = tid + i * NTH;
        kw[i] = u32x4{0u, 0u, 0u, 0u};
        if (e < KC) {
          const int s = e / (D / 8), d = (e - s * (D / 8)) * 8;
          kw[i] = *reinterpret_cast<const u32x4*>(ks + s * D + d);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) mk = fmaxf(mk, fabsf(elem(kw[i], k)));
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int e = tid + i * NTH;
#pragma unroll
        for (int r = 0; r < 4; ++r) vw[i][r] = u32x4{0u, 0u, 0u, 0u};
        if (e < VC) {
          const int tq = e / (D / 8), d0 = (e - tq * (D / 8)) * 8;
#pragma unroll
          for (int r = 0; r < 4; ++r) vw[i][r] = *reinterpret_cast<const u32x4*>(vs + (4 * tq + r) * D + d0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int k = 0; k < 8; ++k) mv = fmaxf(mv, fabsf(elem(vw[i][r], k)));
      }
    } else {
      for (int e = tid; e < cnt * D; e += NTH) {
        mk = fmaxf(mk, fabsf(bf16_value(ks[e])));
        mv = fmaxf(mv, fabsf(bf16_value(vs[e])));
      }
    }
    if (tid == 0 && cnt > 0) {
      s_old[0] = slot0 == 0 ? 0.f : a.k_scale[blk];  // a write at slot 0 starts the page afresh
      s_old[1] = slot0 == 0 ? 0.f : a.v_scale[blk];
    }
    for (int off = 32; off >= 1; off >>= 1) {
      mk = fmaxf(mk, __shfl_xor(mk, off, 64));
      mv = fmaxf(mv, __shfl_xor(mv, off, 64));
    }
    if ((tid & 63) == 0) {
      s_red[0][tid >> 6] = mk;
      s_red[1][tid >> 6] = mv;
    }
    __syncthreads();
    if (cnt == 0) return;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      mk = fmaxf(mk, s_red[0][w]);
      mv = fmaxf(mv, s_red[1][w]);
    }
    for (int which = 0; which < 2; ++which) {
      uint8_t* pb = which ? vb : kb;
      const uint16_t* src = which ? vs : ks;
      const float so = s_old[which];
      const float amax = which ? mv : mk;
      const float cand = __fdiv_rn(amax, 448.0f);
      const float sn = so > cand ? so : cand;  // max(s_old, fl32(amax / 448))
      auto code = [&](float x) -> uint32_t {
        return sn == 0.f ? 0u : e4m3_rne_sat(__fdiv_rn(x, sn));
      };
      if (whole) {
        if (which == 0) {
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            const int e = tid + i * NTH;
            if (e >= KC) continue;
            const int s = e / (D / 8), d = (e - s * (D / 8)) * 8;
            uint32_t c[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k >> 2] |= code(elem(kw[i], k)) << (8 * (k & 3));
            *reinterpret_cast<u32x2*>(pb + k_elem<D, E>(s, d)) = u32x2{c[0], c[1]};
          }
        } else {
#pragma unroll
          for (int i = 0; i < VPT; ++i) {
            const int e = tid + i * NTH;
            if (e >= VC) continue;
            const int tq = e / (D / 8), d0 = (e - tq * (D / 8)) * 8;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
              uint32_t c = 0u;
#pragma unroll
              for (int r = 0; r < 4; ++r) c |= code(elem(vw[i][r], k)) << (8 * r);
              *reinterpret_cast<uint32_t*>(pb + v_elem<D, E>(4 * tq, d0 + k)) = c;
            }
          }
        }
        if (tid == 0) (which ? a.v_scale : a.k_scale)[blk] = sn;
        continue;
      }
      if (sn > so && slot0 > 0) {
        for (int e = tid; e < slot0 * D; e += NTH) {
          const int t = e / D, d = e - t * D;
          const int off = which ? v_elem<D, E>(t, d) : k_elem<D, E>(t, d);
          const float back = __fmul_rn(e4m3_to_f32(pb[off]), so);
          pb[off] = (uint8_t)e4m3_rne_sat(__fdiv_rn(back, sn));
        }
      }
      for (int e = tid; e < cnt * D; e += NTH) {
        const int s = e / D, d = e - s * D;
        const int off = which ? v_elem<D, E>(slot0 + s, d) : k_elem<D, E>(slot0 + s, d);
        pb[off] = sn == 0.f ? (uint8_t)0 : (uint8_t)e4m3_rne_sat(__fdiv_rn(bf16_value(src[e]), sn));
      }
      if (tid == 0) (which ? a.v_scale : a.k_scale)[blk] = sn;
    }
  }
}

}  // namespace pa
