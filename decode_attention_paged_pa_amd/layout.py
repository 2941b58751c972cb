"""Element order inside one (page, head) block of the K and V pools.

The order is part of the library's contract (include/pa.h, "Physical cache
layout"); these index maps let a caller read pool bytes back as logical
[page][head][slot][dim] values.  S = 16 tokens per page, D = head dim,
e = bytes per element, CE = 16 / e elements per 16-byte chunk.

  K(t, d) at (d // (4 CE)) * (S * 4 CE) + t * 4 CE + d % (4 CE)
  V(t, d) at ((((j // TPC) * 16 + c) * 4 + t // 4) * TPC + j % TPC) * 4 + t % 4
          with c = d % 16, j = d // 16, TPC = CE // 4
The V block of a logical (page, head) is stored in another pool slot than its
K block (v_block_slots).
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


def v_block_slots(layout, num_pages, num_kv_heads):
    """Pool slot (page, head) holding the V block of each logical (page, head).

    SEQ with several heads: head h's V block is in head (h + 1) % Hkv's slot of
    the same page; otherwise page p's V block is in page p ^ 1's slot (p itself
    when p ^ 1 is past the pool).  Returns (page index [P][H], head index [P][H]).
    """
    H = num_kv_heads if layout == "seq" else 1
    p = np.repeat(np.arange(num_pages)[:, None], H, axis=1)
    h = np.repeat(np.arange(H)[None, :], num_pages, axis=0)
    if layout == "seq" and num_kv_heads > 1:
        return p, (h + 1) % num_kv_heads
    q = p ^ 1
    return np.where(q < num_pages, q, p), h


def pool_to_logical(pool_bytes, which, layout, kv_dtype, num_pages, num_kv_heads, head_dim):
    """Raw pool bytes (numpy uint8, flat) -> [P][H][S][D] (H = Hkv, or 1 for HEAD).

    Both block orders are axis permutations of a block: K is [D / 4CE][S][4CE]
    and V is [D / (16 TPC)][16][S / 4][TPC][4] (dims c, then token groups;
    d = 16 (TPC jh + jl) + c, t = 4 tq + tr), so a reshape and a transpose
    read them back; the V blocks are first moved from their slots
    (v_block_slots).  Equal to indexing with k_offsets / v_offsets."""
    esize = 1 if kv_dtype == "fp8" else 2
    dt = np.uint8 if esize == 1 else np.uint16
    H = num_kv_heads if layout == "seq" else 1
    D = head_dim
    blocks = np.asarray(pool_bytes).view(dt).reshape(num_pages, H, S * D)
    if which == "k":
        seg = 64 // esize
        return np.ascontiguousarray(
            blocks.reshape(num_pages, H, D // seg, S, seg).transpose(0, 1, 3, 2, 4)
        ).reshape(num_pages, H, S, D)
    if layout == "seq" and num_kv_heads > 1:
        slotted = np.roll(blocks, -1, axis=1)          # head h's V sits in head h + 1's slot
    else:
        sp, _ = v_block_slots(layout, num_pages, num_kv_heads)
        slotted = blocks[sp[:, 0]]                     # page p's V sits in page p ^ 1's slot
    tpc = 4 // esize
    v = slotted.reshape(num_pages, H, D // 16 // tpc, 16, S // 4, tpc, 4)
    # axes (p, h, jh, c, tq, jl, tr) -> (p, h, tq, tr, jh, jl, c)
    return np.ascontiguousarray(v.transpose(0, 1, 4, 6, 2, 5, 3)).reshape(num_pages, H, S, D)


def pool_to_logical_by_index(pool_bytes, which, layout, kv_dtype, num_pages, num_kv_heads,
                             head_dim):
    """pool_to_logical written with the element index maps (slow; checks the fast one)."""
    esize = 1 if kv_dtype == "fp8" else 2
    dt = np.uint8 if esize == 1 else np.uint16
    H = num_kv_heads if layout == "seq" else 1
    blocks = np.asarray(pool_bytes).view(dt).reshape(num_pages, H, S * head_dim)
    if which == "k":
        return blocks[:, :, k_offsets(head_dim, esize)]
    sp, sh = v_block_slots(layout, num_pages, num_kv_heads)
    return blocks[sp, sh][:, :, v_offsets(head_dim, esize)]
