"""Thin ctypes binding of libforkkv (include/forkkv.h).

Argument marshalling only: every step of the attention path runs in the HIP
library.  Device buffers are torch tensors (passed by ``data_ptr()``), streams
are torch streams (passed by their raw ``hipStream_t``).  There is no fallback:
if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libforkkv.so")

OK, EINVAL, ENOMEM, EHIP, ESTATE, EUNSUPPORTED, ETOOBIG = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 32 << 20
DTYPE_F32, DTYPE_BF16 = 0, 1
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA = 0, 1, 2
FORK_PACK, FORK_FREEZE, FORK_AUTO = 0, 1, 2
TIMING_OFF, TIMING_EVENTS, TIMING_SPLIT_ONLY = 0, 1, 2
PAGE = 16

_i32p = C.POINTER(C.c_int32)


class PoolDesc(C.Structure):
    _fields_ = [("num_bpages", C.c_int32), ("num_rpages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("rank", C.c_int32),
                ("dtype", C.c_int32), ("bpage_order", _i32p), ("rpage_order", _i32p)]


class CowOp(C.Structure):
    _fields_ = [("src_bpage", C.c_int32), ("dst_bpage", C.c_int32), ("n_rows", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [("live_bpages", C.c_int32), ("live_rpages", C.c_int32),
                ("free_bpages", C.c_int32), ("free_rpages", C.c_int32),
                ("shared_bpages", C.c_int32), ("bpage_refs", C.c_int64),
                ("rpage_refs", C.c_int64), ("live_bytes_b", C.c_int64),
                ("live_bytes_r", C.c_int64)]


class PlanOpts(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("max_agents_per_item", C.c_int32),
                ("pages_per_item", C.c_int32), ("spare_items", C.c_int32)]


class PlanInfo(C.Structure):
    _fields_ = [("n_agents", C.c_int32), ("n_items", C.c_int32), ("n_slots", C.c_int32),
                ("kernel", C.c_int32), ("item_ints", C.c_int32), ("num_q_heads", C.c_int32),
                ("plan_bytes", C.c_size_t), ("workspace_bytes", C.c_size_t),
                ("item_capacity", C.c_int32), ("slot_capacity", C.c_int32)]


class DecodeArgs(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("plan", C.c_void_p), ("q", C.c_void_p),
                ("Bk", C.c_void_p), ("Bv", C.c_void_p), ("btab", C.c_void_p),
                ("rtab", C.c_void_p), ("max_pages", C.c_int32), ("lora_scale", C.c_float),
                ("sm_scale", C.c_float), ("rope_theta", C.c_float), ("out", C.c_void_p),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("pstart", C.c_void_p)]


class DecodeAppendArgs(C.Structure):
    _fields_ = [("decode", DecodeArgs), ("k_new", C.c_void_p), ("v_new", C.c_void_p),
                ("rk_new", C.c_void_p), ("rv_new", C.c_void_p)]


class PrefillArgs(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("n_agents", C.c_int32), ("chunk_len", C.c_int32),
                ("num_q_heads", C.c_int32), ("q", C.c_void_p), ("k_new", C.c_void_p),
                ("v_new", C.c_void_p), ("rk_new", C.c_void_p), ("rv_new", C.c_void_p),
                ("Bk", C.c_void_p), ("Bv", C.c_void_p), ("btab", C.c_void_p),
                ("rtab", C.c_void_p), ("max_pages", C.c_int32), ("start_pos", C.c_void_p),
                ("start_pos_host", _i32p), ("lora_scale", C.c_float), ("sm_scale", C.c_float),
                ("rope_theta", C.c_float), ("out", C.c_void_p), ("positions", C.c_void_p),
                ("positions_host", _i32p), ("pstart", C.c_void_p), ("kernel", C.c_int32)]


class WriteArgs(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("n_seqs", C.c_int32), ("n_rows", C.c_int32),
                ("btab", C.c_void_p), ("rtab", C.c_void_p), ("pstart", C.c_void_p),
                ("max_pages", C.c_int32), ("positions", C.c_void_p), ("positions_host", _i32p),
                ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("rk_new", C.c_void_p),
                ("rv_new", C.c_void_p)]


_SIGS = {
    "forkkv_strerror": (C.c_char_p, [C.c_int]),
    "forkkv_pool_bytes": (C.c_int, [C.POINTER(PoolDesc), C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "forkkv_pool_create": (C.c_int, [C.POINTER(PoolDesc), C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "forkkv_pool_destroy": (C.c_int, [C.c_void_p]),
    "forkkv_seq_create": (C.c_int, [C.c_void_p, C.c_int32, _i32p]),
    "forkkv_seq_append": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, _i32p, _i32p, C.POINTER(CowOp)]),
    "forkkv_fork": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, _i32p, C.POINTER(CowOp)]),
    "forkkv_fork_ex": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _i32p, C.POINTER(CowOp)]),
    "forkkv_export_starts": (C.c_int, [C.c_void_p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p]),
    "forkkv_evict_bpages": (C.c_int, [C.c_void_p, _i32p, C.c_int32]),
    "forkkv_refill_bpages": (C.c_int, [C.c_void_p, _i32p, C.c_int32, C.c_int32, C.c_int32, _i32p]),
    "forkkv_seq_free": (C.c_int, [C.c_void_p, C.c_int32]),
    "forkkv_seq_len": (C.c_int, [C.c_void_p, C.c_int32, _i32p]),
    "forkkv_seq_pages": (C.c_int, [C.c_void_p, C.c_int32, _i32p]),
    "forkkv_export_tables": (C.c_int, [C.c_void_p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, _i32p]),
    "forkkv_pool_stats": (C.c_int, [C.c_void_p, C.POINTER(Stats)]),
    "forkkv_free_list": (C.c_int, [C.c_void_p, C.c_int32, _i32p, C.c_int32, _i32p]),
    "forkkv_refcounts": (C.c_int, [C.c_void_p, C.c_int32, _i32p]),
    "forkkv_cow_copy": (C.c_int, [C.c_void_p, C.POINTER(CowOp), C.c_int32, C.c_void_p]),
    "forkkv_plan_decode": (C.c_int, [C.c_void_p, _i32p, C.c_int32, C.c_int32, C.POINTER(PlanOpts), C.POINTER(C.c_void_p)]),
    "forkkv_plan_rebuild": (C.c_int, [C.c_void_p, C.c_void_p, _i32p, C.c_int32, _i32p]),
    "forkkv_seq_append_batch": (C.c_int, [C.c_void_p, _i32p, C.c_int32, C.c_int32, _i32p, _i32p, C.POINTER(CowOp), _i32p]),
    "forkkv_plan_get_info": (C.c_int, [C.c_void_p, C.POINTER(PlanInfo)]),
    "forkkv_plan_export": (C.c_int, [C.c_void_p, _i32p]),
    "forkkv_plan_upload": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "forkkv_plan_destroy": (C.c_int, [C.c_void_p]),
    "forkkv_plan_set_timing": (C.c_int, [C.c_void_p, C.c_int32]),
    "forkkv_plan_timing": (C.c_int, [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_double), _i32p]),
    "forkkv_residual_attn_decode": (C.c_int, [C.POINTER(DecodeArgs), C.c_void_p]),
    "forkkv_residual_attn_decode_noalloc": (C.c_int, [C.POINTER(DecodeArgs), C.c_void_p]),
    "forkkv_residual_attn_decode_append": (C.c_int, [C.POINTER(DecodeAppendArgs), C.c_void_p]),
    "forkkv_residual_attn_prefill": (C.c_int, [C.POINTER(PrefillArgs), C.c_void_p]),
    "forkkv_write_rows": (C.c_int, [C.POINTER(WriteArgs), C.c_void_p]),
}

_lib = None


def lib():
    """Load libforkkv.so (built in-tree).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m lora_shared_prefix_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class ForkKVError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {lib().forkkv_strerror(code).decode()} ({code})")
        self.code = code


def _check(code, what):
    if code != OK:
        raise ForkKVError(code, what)


def _i32_array(values):
    arr = (C.c_int32 * max(len(values), 1))(*[int(v) for v in values])
    return arr


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


class Pool:
    """Host bookkeeping of one pool; optionally bound to device pool tensors."""

    def __init__(self, num_bpages, num_rpages, num_kv_heads, head_dim, rank, dtype,
                 bpage_order=None, rpage_order=None, bcache=None, rcache=None):
        self._bo = _i32_array(bpage_order) if bpage_order is not None else None
        self._ro = _i32_array(rpage_order) if rpage_order is not None else None
        self.desc = PoolDesc(num_bpages, num_rpages, PAGE, num_kv_heads, head_dim, rank,
                             DTYPE_BF16 if dtype in ("bf16", DTYPE_BF16) else DTYPE_F32,
                             C.cast(self._bo, _i32p) if self._bo is not None else None,
                             C.cast(self._ro, _i32p) if self._ro is not None else None)
        self.bcache, self.rcache = bcache, rcache
        h = C.c_void_p()
        _check(lib().forkkv_pool_create(C.byref(self.desc), _ptr(bcache), _ptr(rcache),
                                        C.byref(h)), "forkkv_pool_create")
        self.handle = h

    @staticmethod
    def nbytes(num_bpages, num_rpages, num_kv_heads, head_dim, rank, dtype):
        d = PoolDesc(num_bpages, num_rpages, PAGE, num_kv_heads, head_dim, rank,
                     DTYPE_BF16 if dtype in ("bf16", DTYPE_BF16) else DTYPE_F32, None, None)
        b, r = C.c_size_t(), C.c_size_t()
        _check(lib().forkkv_pool_bytes(C.byref(d), C.byref(b), C.byref(r)), "forkkv_pool_bytes")
        return b.value, r.value

    def close(self):
        if self.handle:
            lib().forkkv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self, with_residual):
        out = C.c_int32()
        _check(lib().forkkv_seq_create(self.handle, int(bool(with_residual)), C.byref(out)),
               "forkkv_seq_create")
        return out.value

    def append(self, seq, n, want_slots=True):
        bs = (C.c_int32 * max(n, 1))() if want_slots else None
        rs = (C.c_int32 * max(n, 1))() if want_slots else None
        cow = CowOp()
        _check(lib().forkkv_seq_append(self.handle, seq, n, bs, rs, C.byref(cow)),
               "forkkv_seq_append")
        cow_t = (cow.src_bpage, cow.dst_bpage, cow.n_rows) if cow.n_rows else None
        if not want_slots:
            return None, None, cow_t
        return list(bs)[:n], list(rs)[:n], cow_t

    def append_batch(self, seqs, n, want_slots=False):
        """Reserve n rows at the end of each sequence of `seqs` (distinct), all or nothing.
        Returns (new base pages taken, [cow ops], bslots or None, rslots or None); a nonzero
        page count means some sequence entered a new page (a decode plan needs a rebuild)."""
        k = len(seqs)
        bs = (C.c_int32 * max(k * n, 1))() if want_slots else None
        rs = (C.c_int32 * max(k * n, 1))() if want_slots else None
        cows = (CowOp * max(k, 1))()
        pages = C.c_int32()
        _check(lib().forkkv_seq_append_batch(self.handle, _i32_array(seqs), k, n, bs, rs, cows,
                                             C.byref(pages)), "forkkv_seq_append_batch")
        cow_list = [(c.src_bpage, c.dst_bpage, c.n_rows) for c in cows[:k] if c.n_rows]
        return (pages.value, cow_list, list(bs)[:k * n] if want_slots else None,
                list(rs)[:k * n] if want_slots else None)

    def fork(self, parent, alias_len, mode=None, suffix_hint=0):
        """Fork (mode None: forkkv_fork, i.e. pack; else forkkv_fork_ex with FORK_*)."""
        child, cow = C.c_int32(), CowOp()
        if mode is None:
            _check(lib().forkkv_fork(self.handle, parent, alias_len, C.byref(child),
                                     C.byref(cow)), "forkkv_fork")
        else:
            _check(lib().forkkv_fork_ex(self.handle, parent, alias_len, int(mode),
                                        int(suffix_hint), C.byref(child), C.byref(cow)),
                   "forkkv_fork_ex")
        return child.value, ((cow.src_bpage, cow.dst_bpage, cow.n_rows) if cow.n_rows else None)

    def starts(self, seqs, max_pages):
        """Page start positions [n][max_pages] (-1 padded) and whether all are aligned."""
        n = len(seqs)
        out = (C.c_int32 * max(n * max_pages, 1))()
        al = C.c_int32()
        _check(lib().forkkv_export_starts(self.handle, _i32_array(seqs), n, max_pages, out,
                                          C.byref(al)), "forkkv_export_starts")
        out = list(out)
        return [out[i * max_pages:(i + 1) * max_pages] for i in range(n)], bool(al.value)

    def evict_base(self, pages):
        _check(lib().forkkv_evict_bpages(self.handle, _i32_array(pages), len(pages)),
               "forkkv_evict_bpages")

    def refill_base(self, seqs, lp0, lp1):
        out = (C.c_int32 * max(lp1 - lp0, 1))()
        _check(lib().forkkv_refill_bpages(self.handle, _i32_array(seqs), len(seqs), lp0, lp1,
                                          out), "forkkv_refill_bpages")
        return list(out)[:max(lp1 - lp0, 0)]

    def free(self, seq):
        _check(lib().forkkv_seq_free(self.handle, seq), "forkkv_seq_free")

    def length(self, seq):
        out = C.c_int32()
        _check(lib().forkkv_seq_len(self.handle, seq, C.byref(out)), "forkkv_seq_len")
        return out.value

    def pages(self, seq):
        out = C.c_int32()
        _check(lib().forkkv_seq_pages(self.handle, seq, C.byref(out)), "forkkv_seq_pages")
        return out.value

    def tables(self, seqs, max_pages):
        n = len(seqs)
        bt = (C.c_int32 * max(n * max_pages, 1))()
        rt = (C.c_int32 * max(n * max_pages, 1))()
        lens = (C.c_int32 * max(n, 1))()
        _check(lib().forkkv_export_tables(self.handle, _i32_array(seqs), n, max_pages, bt, rt,
                                          lens), "forkkv_export_tables")
        bt, rt = list(bt), list(rt)
        return ([bt[i * max_pages:(i + 1) * max_pages] for i in range(n)],
                [rt[i * max_pages:(i + 1) * max_pages] for i in range(n)], list(lens)[:n])

    def stats(self):
        st = Stats()
        _check(lib().forkkv_pool_stats(self.handle, C.byref(st)), "forkkv_pool_stats")
        return {f: getattr(st, f) for f, _ in Stats._fields_}

    def free_list(self, which):
        n = C.c_int32()
        _check(lib().forkkv_free_list(self.handle, which, None, 0, C.byref(n)), "forkkv_free_list")
        out = (C.c_int32 * max(n.value, 1))()
        _check(lib().forkkv_free_list(self.handle, which, out, n.value, C.byref(n)),
               "forkkv_free_list")
        return list(out)[:n.value]

    def refcounts(self, which):
        size = self.desc.num_bpages if which == 0 else self.desc.num_rpages
        out = (C.c_int32 * size)()
        _check(lib().forkkv_refcounts(self.handle, which, out), "forkkv_refcounts")
        return list(out)

    def cow_copy(self, ops, stream=None):
        arr = (CowOp * max(len(ops), 1))(*[CowOp(*o) for o in ops])
        _check(lib().forkkv_cow_copy(self.handle, arr, len(ops), _stream(stream)),
               "forkkv_cow_copy")

    def replay(self, ops):
        """Apply a workload operation script; returns ({name: handle}, [cow ops])."""
        names, cows = {}, []
        for op in ops:
            if op[0] == "create":
                names[op[1]] = self.create(op[2])
            elif op[0] == "append":
                _, _, cow = self.append(names[op[1]], op[2], want_slots=False)
                if cow:
                    cows.append(cow)
            elif op[0] == "fork":
                names[op[3]], cow = self.fork(names[op[1]], op[2], *op[4:])
                if cow:
                    cows.append(cow)
            else:
                raise ValueError(op)
        return names, cows


class Plan:
    def __init__(self, pool: Pool, seqs, num_q_heads, kernel=KERNEL_AUTO, max_agents_per_item=0,
                 pages_per_item=0, spare_items=0):
        opts = PlanOpts(kernel, max_agents_per_item, pages_per_item, spare_items)
        h = C.c_void_p()
        _check(lib().forkkv_plan_decode(pool.handle, _i32_array(seqs), len(seqs), num_q_heads,
                                        C.byref(opts), C.byref(h)), "forkkv_plan_decode")
        self.handle = h
        self.pool = pool
        info = PlanInfo()
        _check(lib().forkkv_plan_get_info(h, C.byref(info)), "forkkv_plan_get_info")
        self.info = {f: getattr(info, f) for f, _ in PlanInfo._fields_}
        self.dev = None

    def rebuild(self, seqs):
        """Rebuild in place from the pool's current state; returns True when a decode launch
        captured before stays valid once the plan is uploaded to the same buffer."""
        same = C.c_int32()
        _check(lib().forkkv_plan_rebuild(self.handle, self.pool.handle, _i32_array(seqs),
                                         len(seqs), C.byref(same)), "forkkv_plan_rebuild")
        info = PlanInfo()
        _check(lib().forkkv_plan_get_info(self.handle, C.byref(info)), "forkkv_plan_get_info")
        self.info = {f: getattr(info, f) for f, _ in PlanInfo._fields_}
        return bool(same.value)

    def blob(self):
        n = self.info["plan_bytes"] // 4
        out = (C.c_int32 * n)()
        _check(lib().forkkv_plan_export(self.handle, out), "forkkv_plan_export")
        return list(out)

    def upload(self, stream=None):
        """Copy the blob to the device (asynchronously on the stream).  The device buffer is
        kept while it is large enough, so a captured launch keeps its address."""
        import torch
        n = self.info["plan_bytes"] // 4
        if self.dev is None or self.dev.numel() < n:
            self.dev = torch.empty(n, dtype=torch.int32, device="cuda")
        _check(lib().forkkv_plan_upload(self.handle, _ptr(self.dev), _stream(stream)),
               "forkkv_plan_upload")
        return self

    def set_timing(self, enable):
        """0 / False: off; 1 / True: events around each launch; TIMING_SPLIT_ONLY: decode
        calls launch the split kernel alone (measurement only; the output is not written)."""
        _check(lib().forkkv_plan_set_timing(self.handle, int(enable)), "forkkv_plan_set_timing")

    def timing(self):
        s, c, k = C.c_double(), C.c_double(), C.c_int32()
        _check(lib().forkkv_plan_timing(self.handle, C.byref(s), C.byref(c), C.byref(k)),
               "forkkv_plan_timing")
        return s.value, c.value, k.value

    def workspace(self):
        import torch
        return torch.empty(max(self.info["workspace_bytes"], 1), dtype=torch.uint8, device="cuda")

    def close(self):
        if self.handle:
            lib().forkkv_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def residual_attn_decode(pool: Pool, plan: Plan, q, Bk, Bv, btab, rtab, out, workspace,
                         lora_scale, sm_scale, rope_theta, stream=None, pstart=None):
    """Launch decode (async).  All tensors on the device; btab/rtab int32 [N][max_pages];
    pstart (int32 [N][max_pages]) is the page start table of batches with a frozen tail."""
    args = DecodeArgs(pool.handle, plan.handle, q.data_ptr(), Bk.data_ptr(), Bv.data_ptr(),
                      btab.data_ptr(), rtab.data_ptr(), int(btab.shape[1]), float(lora_scale),
                      float(sm_scale), float(rope_theta), out.data_ptr(),
                      workspace.data_ptr() if workspace is not None else None,
                      workspace.numel() * workspace.element_size() if workspace is not None else 0,
                      _ptr(pstart))
    _check(lib().forkkv_residual_attn_decode(C.byref(args), _stream(stream)),
           "forkkv_residual_attn_decode")


def residual_attn_decode_noalloc(pool: Pool, plan: Plan, q, Bk, Bv, btab, rtab, out,
                                 lora_scale, sm_scale, rope_theta, stream=None, pstart=None):
    """Launch decode (async) with the library's static split-K scratch instead of a caller
    workspace: nothing is allocated.  Calls that overlap on one GPU race."""
    args = DecodeArgs(pool.handle, plan.handle, q.data_ptr(), Bk.data_ptr(), Bv.data_ptr(),
                      btab.data_ptr(), rtab.data_ptr(), int(btab.shape[1]), float(lora_scale),
                      float(sm_scale), float(rope_theta), out.data_ptr(), None, 0, _ptr(pstart))
    _check(lib().forkkv_residual_attn_decode_noalloc(C.byref(args), _stream(stream)),
           "forkkv_residual_attn_decode_noalloc")


def residual_attn_decode_append(pool: Pool, plan: Plan, q, Bk, Bv, btab, rtab, out, workspace,
                                lora_scale, sm_scale, rope_theta, k_new, v_new, rk_new, rv_new,
                                stream=None, pstart=None):
    """Store each agent's new token (k_new/v_new [N][Hkv][d], rk_new/rv_new [N][r]) at
    position len - 1, then decode over keys 0 .. len - 1 (async)."""
    d = DecodeArgs(pool.handle, plan.handle, q.data_ptr(), Bk.data_ptr(), Bv.data_ptr(),
                   btab.data_ptr(), rtab.data_ptr(), int(btab.shape[1]), float(lora_scale),
                   float(sm_scale), float(rope_theta), out.data_ptr(),
                   workspace.data_ptr() if workspace is not None else None,
                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                   _ptr(pstart))
    args = DecodeAppendArgs(d, k_new.data_ptr(), v_new.data_ptr(), rk_new.data_ptr(),
                            rv_new.data_ptr())
    _check(lib().forkkv_residual_attn_decode_append(C.byref(args), _stream(stream)),
           "forkkv_residual_attn_decode_append")


def residual_attn_prefill(pool: Pool, q, k_new, v_new, rk_new, rv_new, Bk, Bv, btab, rtab,
                          start_pos, start_pos_host, out, lora_scale, sm_scale, rope_theta,
                          stream=None, positions=None, positions_host=None, pstart=None,
                          kernel=KERNEL_AUTO):
    """Launch prefill (async): store the rows, then attend causally.  Rows sit at
    start_pos[a] + i, or at positions[a][i] when a position list (device int32 [N][C] plus
    the same values on the host) is given.  kernel: KERNEL_AUTO, KERNEL_GENERIC or
    KERNEL_MFMA."""
    N, Cn, Hq = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    sp = _i32_array(start_pos_host) if start_pos_host is not None else None
    ph = (_i32_array([int(x) for row in positions_host for x in row])
          if positions_host is not None else None)
    args = PrefillArgs(pool.handle, N, Cn, Hq, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                       rk_new.data_ptr(), rv_new.data_ptr(), Bk.data_ptr(), Bv.data_ptr(),
                       btab.data_ptr(), rtab.data_ptr(), int(btab.shape[1]),
                       start_pos.data_ptr() if start_pos is not None else None,
                       C.cast(sp, _i32p) if sp is not None else None, float(lora_scale),
                       float(sm_scale), float(rope_theta), out.data_ptr(),
                       positions.data_ptr() if positions is not None else None,
                       C.cast(ph, _i32p) if ph is not None else None, _ptr(pstart),
                       int(kernel))
    _check(lib().forkkv_residual_attn_prefill(C.byref(args), _stream(stream)),
           "forkkv_residual_attn_prefill")


def write_rows(pool: Pool, btab, rtab, positions, positions_host, k_new, v_new, rk_new=None,
               rv_new=None, pstart=None, stream=None):
    """Store rows at positions[a][i] without attention (async); with rk_new = rv_new = None
    only the base pool is written (a partial-hit refill)."""
    N, R = int(k_new.shape[0]), int(k_new.shape[1])
    ph = _i32_array([int(x) for row in positions_host for x in row])
    args = WriteArgs(pool.handle, N, R, btab.data_ptr(), _ptr(rtab) if rtab is not None else None,
                     _ptr(pstart), int(btab.shape[1]), positions.data_ptr(), C.cast(ph, _i32p),
                     k_new.data_ptr(), v_new.data_ptr(), _ptr(rk_new), _ptr(rv_new))
    _check(lib().forkkv_write_rows(C.byref(args), _stream(stream)), "forkkv_write_rows")