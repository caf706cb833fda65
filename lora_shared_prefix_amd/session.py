"""Device-side setup of a batch: upload pools and inputs, replay the pool script through
the library, upload block tables and the decode plan, then launch.

Marshalling only -- the attention itself and the fork bookkeeping run in libforkkv.
"""
from __future__ import annotations

import time

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
        self.lib_host_s = 0.0  # time spent in the library's host calls of next_step
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

    def refresh_tables(self, extra_pages=0, inplace=False):
        """Upload the block tables and, when a sequence holds a frozen tail, the page start
        table (the slot map; ``pstart`` is None for aligned batches).  ``extra_pages`` leaves
        room for later pages; ``inplace`` writes into the device tables already there (same
        width, so that a captured launch keeps their addresses)."""
        self._st = None  # next_step's view of the last pages is recomputed
        pages = [self.pool.pages(h) for h in self.handles]
        width = max(1, max(pages, default=1) + extra_pages)
        if inplace:
            assert width <= self.max_pages, "the tables have no room for the new pages"
            width = self.max_pages
        self.max_pages = width
        bt, rt, self.lens = self.pool.tables(self.handles, self.max_pages)
        self.btab_host = np.array(bt, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        self.rtab_host = np.array(rt, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        st, aligned = self.pool.starts(self.handles, self.max_pages)
        self.pstart_host = np.array(st, dtype=np.int32).reshape(len(self.handles), self.max_pages)
        if inplace:
            self.btab.copy_(torch.from_numpy(self.btab_host))
            self.rtab.copy_(torch.from_numpy(self.rtab_host))
            if self.pstart is not None:
                self.pstart.copy_(torch.from_numpy(self.pstart_host))
            return
        self.btab = torch.from_numpy(self.btab_host).to(self.device)
        self.rtab = torch.from_numpy(self.rtab_host).to(self.device)
        self.pstart = None if aligned else torch.from_numpy(self.pstart_host).to(self.device)

    def next_step(self, stream=None):
        """Decode with append, between two steps: reserve each agent's next token on the host
        (one batched call) and, when that took an agent into a new page or needed a
        copy-on-write, run the copies, update the device tables in place and rebuild and
        re-upload the plan (asynchronously).  Returns (same, cows): ``same`` is True when a
        launch captured earlier stays valid (always, within the plan's capacities and the
        tables' room); ``cows`` the row copies that were run."""
        st = self._step_state()
        t0 = time.perf_counter()
        rc = fk.lib().forkkv_seq_append_batch(self.pool.handle, st["seqs"], st["n"], 1,
                                              st["bslots"], st["rslots"], st["cows"],
                                              fk.C.byref(st["pages"]))
        self.lib_host_s += time.perf_counter() - t0
        if rc != fk.OK:
            raise fk.ForkKVError(rc, "forkkv_seq_append_batch")
        cows = [(c.src_bpage, c.dst_bpage, c.n_rows) for c in st["cows"] if c.n_rows]
        if cows:
            self.pool.cow_copy(cows, stream)
        self.lens = [n + 1 for n in self.lens]
        if not st["pages"].value and not cows:
            return True, cows
        # patch the host tables where a token opened a page (row 0) or the last page was
        # copied, then copy them to the device tables in place -- asynchronously, from pinned
        # mirrors (the previous copy out of them has long finished; it is waited for)
        if st["copied"] is not None:
            st["copied"].synchronize()
        for a in range(st["n"]):
            page, row = divmod(st["bslots"][a], fk.PAGE)
            lp = st["last"][a]
            if row == 0 or lp < 0:
                lp += 1
                st["last"][a] = lp
                if self.pstart is not None:
                    self.pstart_host[a, lp] = self.lens[a] - 1
            assert lp < self.max_pages, "the tables have no room for the new pages"
            self.btab_host[a, lp] = page
            self.rtab_host[a, lp] = st["rslots"][a] // fk.PAGE
        self.btab.copy_(st["btab_pin"], non_blocking=True)
        self.rtab.copy_(st["rtab_pin"], non_blocking=True)
        if self.pstart is not None:
            self.pstart.copy_(st["pstart_pin"], non_blocking=True)
        st["copied"] = torch.cuda.Event()
        st["copied"].record()
        t0 = time.perf_counter()
        same = self.plan.rebuild(self.handles)
        dev = self.plan.dev.data_ptr()
        self.plan.upload(stream)
        self.lib_host_s += time.perf_counter() - t0
        same = same and self.plan.dev.data_ptr() == dev
        if self.plan.info["workspace_bytes"] > self.workspace.numel():
            self.workspace = self.plan.workspace()
            same = False
        return same, cows

    def make_plan(self, kernel=fk.KERNEL_AUTO, pages_per_item=0, max_agents_per_item=0,
                  stream=None, spare_items=0):
        self.plan = fk.Plan(self.pool, self.handles, self.g["num_q_heads"], kernel,
                            max_agents_per_item, pages_per_item, spare_items).upload(stream)
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

    def _step_state(self):
        """ctypes buffers of next_step, made once per batch (and the agents' last pages)."""
        st = getattr(self, "_st", None)
        if st is None or st["n"] != len(self.handles):
            n = len(self.handles)
            last = [int((self.btab_host[a] >= 0).sum()) - 1 for a in range(n)]
            st = dict(n=n, seqs=fk._i32_array(self.handles), bslots=(fk.C.c_int32 * n)(),
                      rslots=(fk.C.c_int32 * n)(), cows=(fk.CowOp * n)(),
                      pages=fk.C.c_int32(), last=last, copied=None)
            # pinned host mirrors of the tables (the host arrays become views of them)
            for name in ("btab", "rtab", "pstart"):
                host = getattr(self, name + "_host")
                pin = torch.from_numpy(host.copy()).pin_memory()
                st[name + "_pin"] = pin
                setattr(self, name + "_host", pin.numpy())
            self._st = st
        return st

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
