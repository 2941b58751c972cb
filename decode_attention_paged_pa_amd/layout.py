"""Element order inside one (page, head) block of the K and V pools.

The order is part of the library's contract (include/pa.h, "Physical cache
layout"); these index maps let a caller read pool bytes back as logical
[page][head][slot][dim] values.  S = 16 tokens per page, D = head dim,
e = bytes per element, CE = 16 / e elements per 16-byte chunk.

  K(t, d) at (d // (4 CE)) * (S * 4 CE) + t * 4 CE + d % (4 CE)
  V(t, d) at ((((j // TPC) * 16 + c) * 4 + t // 4) * TPC + j % TPC) * 4 + t % 4
          with c = d % 16, j = d // 16, TPC = CE // 4
"""
import numpy as np

S = 16


def k_offsets(D, esize):
    seg = 64 // esize
    t = np.arange(S)[:, None]
    d = np.arange(D)[None, :]
    return (d // seg) * (S * seg) + t * seg + (d % seg)


def v_offsets(D, esize):
    tpc = 4 // esize
    t = np.arange(S)[:, None]
    d = np.arange(D)[None, :]
    c, j = d % 16, d // 16
    return ((((j // tpc) * 16 + c) * 4 + t // 4) * tpc + j % tpc) * 4 + t % 4


def pool_to_logical(pool_bytes, which, layout, kv_dtype, num_pages, num_kv_heads, head_dim):
    """Raw pool bytes (numpy uint8, flat) -> [P][H][S][D] (H = Hkv, or 1 for HEAD)."""
    esize = 1 if kv_dtype == "fp8" else 2
    dt = np.uint8 if esize == 1 else np.uint16
    H = num_kv_heads if layout == "seq" else 1
    blocks = np.asarray(pool_bytes).view(dt).reshape(num_pages, H, S * head_dim)
    off = k_offsets(head_dim, esize) if which == "k" else v_offsets(head_dim, esize)
    return blocks[:, :, off]
