"""Put a synthetic workload on the GPU and fill its paged cache through the library.

The cache is filled the way a decode loop fills it: one bulk pa_cache_append of
each sequence's first L-T tokens into empty pages, then the decode step's own
append of its T new tokens per unit (lengths L-T -> L; T = 1 for plain decode,
the draft count for a multi-query step), after which decode attends L tokens.  Draws come from workloads.Workload (numpy, per-sequence child
streams), generated on host threads ahead of the uploads.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

from . import pa


@dataclass
class DeviceWorkload:
    w: object
    cache: pa.PagedKVCache
    block_table: torch.Tensor
    lens: torch.Tensor          # tokens attended (after the step's append)
    lens_old: torch.Tensor      # lengths before the step's append
    n_step: torch.Tensor        # tokens appended by the step (T, 0 for empty units)
    k_step: torch.Tensor        # [B][Hkv][T][D] bf16: the step's new tokens
    v_step: torch.Tensor
    q: torch.Tensor             # [B][Hq][D] bf16
    page_tags: torch.Tensor
    expected_tags: torch.Tensor
    flags: torch.Tensor         # [B] int32 (uint32 bit patterns)

    def step_append(self, flags=None, check=True):
        """The step's append; with check, through the expected tags (a page whose tag
        is stale is left alone), as pa_decode_step does it."""
        pa.append(self.cache, self.block_table, self.lens_old, self.n_step, self.k_step,
                  self.v_step, flags=flags, expected_tags=self.expected_tags if check else None)

    def decode_step(self, check=True, num_partitions=0, out=None, workspace=None, events=None):
        """The step's append and decode (T <= 8) in one library call."""
        return pa.decode_step(self.cache, self.q, self.block_table, self.lens_old, self.n_step,
                              self.k_step, self.v_step, self.lens, self.w.sigma,
                              expected_tags=self.expected_tags if check else None,
                              flags=self.flags if check else None,
                              num_partitions=num_partitions, out=out, workspace=workspace,
                              events=events)

    def decode(self, check=True, num_partitions=0, out=None, workspace=None, events=None):
        run = pa.decode if self.w.q_len == 1 else (pa.decode_multi if self.w.q_len <= 8
                                                   else pa.prefill)
        return run(self.cache, self.q, self.block_table, self.lens, self.w.sigma,
                   expected_tags=self.expected_tags if check else None,
                   flags=self.flags if check else None, num_partitions=num_partitions,
                   out=out, workspace=workspace, events=events)


def _dev(x, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def build_device_workload(w, device="cuda", threads=8, seqs=None, log=None):
    """Upload workload `w` and fill its cache; `seqs` limits the bulk fill (tests)."""
    bt = _dev(w.block_table, device)
    lens = _dev(w.lens, device)
    T = w.q_len
    lens_old = _dev(np.maximum(w.lens.astype(np.int32) - T, 0).astype(np.int32), device)
    n_step = (lens > 0).to(torch.int32) * T
    page_tags = _dev(w.page_tags, device, torch.int32)
    exp = _dev(w.expected_tags, device, torch.int32)
    q = _dev(w.q, device, torch.bfloat16)
    cache = pa.PagedKVCache(w.layout, w.kv_dtype, w.P, w.Hkv, w.D, device=device,
                            page_tags=page_tags)
    k_step = np.zeros((w.B, w.Hkv, T, w.D), np.uint16)
    v_step = np.zeros_like(k_step)
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    zero1 = torch.zeros((1,) + tuple(w.lens.shape[1:]), dtype=torch.int32, device=device)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        for i, (b, draws) in enumerate(zip(seqs, ex.map(w.seq_kv, seqs))):
            k_hist, v_hist, k_new, v_new, n_hist = draws
            k_step[b], v_step[b] = k_new, v_new
            if k_hist.shape[1] > 0:
                n_new = _dev(n_hist if w.layout == "head" else n_hist[:1], device).reshape(zero1.shape)
                kd = _dev(k_hist[None], device, torch.bfloat16)
                vd = _dev(v_hist[None], device, torch.bfloat16)
                pa.append(cache, bt[b:b + 1], zero1, n_new, kd, vd)
                del kd, vd
            if log and (i % 16 == 15 or i == len(seqs) - 1):
                log("filled %d/%d sequences" % (i + 1, len(seqs)))
    dw = DeviceWorkload(w=w, cache=cache, block_table=bt, lens=lens, lens_old=lens_old,
                        n_step=n_step, k_step=_dev(k_step, device, torch.bfloat16),
                        v_step=_dev(v_step, device, torch.bfloat16), q=q, page_tags=page_tags,
                        expected_tags=exp,
                        flags=torch.full((w.B,), -1, dtype=torch.int32, device=device))
    return dw
