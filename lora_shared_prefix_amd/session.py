"""Device-side setup of a batch: upload pools and inputs, replay the pool script through
the library, upload block tables and the decode plan, then launch.

Marshalling only -- the attention itself and the fork bookkeeping run in libforkkv.
"""
from __future__ import annotations

import numpy as np
import torch

from . import forkkv as fk


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy array in storage encoding -> device tensor with the same bytes."""
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(np.uint16) if dtype == "bf16" else a


class DeviceBatch:
    """One decode (or prefill) batch bound to device memory.

    ``geom``: dict with num_bpages, num_rpages, num_kv_heads, num_q_heads, head_dim,
    rank, dtype.  ``arrays``: dict of storage-encoded numpy arrays (bpool, rpool, q,
    Bk, Bv, optional chunk rows).  ``ops``/``agents``: the pool operation script and the
    names of the batch's sequences.
    """

    def __init__(self, geom, arrays, ops, agents, perm_b=None, perm_r=None, device="cuda",
                 kernel=fk.KERNEL_AUTO, pages_per_item=0, max_agents_per_item=0, plan=True,
                 stream=None):
        self.g = dict(geom)
        self.dtype = self.g["dtype"]
        self.device = device
        self.bcache = to_device(arrays["bpool"], device)
        self.rcache = to_device(arrays["rpool"], device)
        self.pool = fk.Pool(self.g["num_bpages"], self.g["num_rpages"], self.g["num_kv_heads"],
                            self.g["head_dim"], self.g["rank"], self.dtype, perm_b, perm_r,
                            self.bcache, self.rcache)
        self.names, self.cows = self.pool.replay(ops)
        if self.cows:
            self.pool.cow_copy(self.cows, stream)
        self.agents = list(agents)
        self.handles = [self.names[a] for a in self.agents]
        self.q = to_device(arrays["q"], device)
        self.Bk = to_device(arrays["Bk"], device)
        self.Bv = to_device(arrays["Bv"], device)
        self.out = torch.empty_like(self.q)
        self.refresh_tables()
        self.plan = None
        if plan:
            self.make_plan(kernel, pages_per_item, max_agents_per_item, stream)

    def refresh_tables(self, extra_pages=0):
        """Upload the block tables and, when a sequence holds a frozen tail, the page start
        table (the slot map; ``pstart`` is None for aligned batches)."""
        pages = [self.pool.pages(h) for h in self.handles]
        self.max_pages = max(1, max(pages, default=1) + extra_pages)
        bt, rt, self.lens = self.pool.tables(self.handles, self.max_pages)
        self.btab_host = np.array(bt, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        self.rtab_host = np.array(rt, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        self.btab = torch.from_numpy(self.btab_host).to(self.device)
        self.rtab = torch.from_numpy(self.rtab_host).to(self.device)
        st, aligned = self.pool.starts(self.handles, self.max_pages)
        self.pstart_host = np.array(st, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        self.pstart = None if aligned else torch.from_numpy(self.pstart_host).to(self.device)

    def make_plan(self, kernel=fk.KERNEL_AUTO, pages_per_item=0, max_agents_per_item=0,
                  stream=None):
        self.plan = fk.Plan(self.pool, self.handles, self.g["num_q_heads"], kernel,
                            max_agents_per_item, pages_per_item).upload(stream)
        self.workspace = self.plan.workspace()
        return self.plan

    def decode(self, lora_scale, sm_scale, rope_theta, stream=None, q=None, out=None):
        fk.residual_attn_decode(self.pool, self.plan, self.q if q is None else q, self.Bk,
                                self.Bv, self.btab, self.rtab, self.out if out is None else out,
                                self.workspace, lora_scale, sm_scale, rope_theta, stream,
                                pstart=self.pstart)
        return self.out if out is None else out

    def decode_append(self, rows, lora_scale, sm_scale, rope_theta, stream=None, out=None):
        """After reserve_chunk(1) and make_plan(): store every agent's new token (rows: dict
        of device tensors k_new [N][Hkv][d], v_new, rk_new [N][r], rv_new), then decode."""
        out = self.out if out is None else out
        fk.residual_attn_decode_append(self.pool, self.plan, self.q, self.Bk, self.Bv, self.btab,
                                       self.rtab, out, self.workspace, lora_scale, sm_scale,
                                       rope_theta, rows["k_new"], rows["v_new"], rows["rk_new"],
                                       rows["rv_new"], stream, pstart=self.pstart)
        return out

    # ---- chunked prefill ---------------------------------------------------------------
    def reserve_chunk(self, chunk_len):
        """Append chunk_len rows to every agent (host bookkeeping) and re-upload the tables."""
        self.start = [self.pool.length(h) for h in self.handles]
        for h in self.handles:
            _, _, cow = self.pool.append(h, chunk_len, want_slots=False)
            if cow:
                self.pool.cow_copy([cow])
        self.refresh_tables()
        self.start_dev = torch.tensor(self.start, dtype=torch.int32, device=self.device)
        return self.start

    def prefill(self, chunk, lora_scale, sm_scale, rope_theta, stream=None, out=None,
                kernel=fk.KERNEL_AUTO):
        """chunk: dict of device tensors q, k_new, v_new, rk_new, rv_new."""
        if out is None:
            out = torch.empty_like(chunk["q"])
        fk.residual_attn_prefill(self.pool, chunk["q"], chunk["k_new"], chunk["v_new"],
                                 chunk["rk_new"], chunk["rv_new"], self.Bk, self.Bv, self.btab,
                                 self.rtab, self.start_dev, self.start, out, lora_scale,
                                 sm_scale, rope_theta, stream, pstart=self.pstart,
                                 kernel=kernel)
        return out


def workload_geom(cfg) -> dict:
    return dict(num_bpages=cfg.num_bpages, num_rpages=cfg.num_rpages,
                num_kv_heads=cfg.num_kv_heads, num_q_heads=cfg.num_q_heads,
                head_dim=cfg.head_dim, rank=cfg.rank, dtype=cfg.dtype)
