"""Bookkeeping model of the forked, disaggregated page pools (oracle side; test infrastructure).

Semantics, from the pages:

* ForkKV study note, "2. Q1 / Q2 / Q3" (Q2) and "3. 架构 / 方法图" (Figure 6):
  a new agent inherits the parent's read-only base pages by mapping them
  (Step 1) and gets its own residual pages (Step 2).
* ForkServe README, "Design vs APC" and "Methods" ("CoW tree"): fork aliases
  the parent's page frames before the child writes anything; a write allocates
  private pages only; freeing a child releases its private pages, not the trunk.
  An unaligned trunk tail is *packed*: the child gets a private copy of the
  ``n_valid`` rows of the parent's partial page (``pages_pack`` formula; the
  "Status" section's row copy of n_valid rows, not P).
* ForkServe README, "Status": extra pins keep the trunk alive when the parent is
  freed -- here every page carries a reference count.

Allocator rules (the pages leave them open; the library implements the same):
free lists are FIFO queues seeded with the pool's page order; allocation takes
from the head, release appends to the tail in the order the freed sequence
lists its pages (base pages first, then residual pages).  Sequence handles are
consecutive integers from 0 and are never reused.  Every operation is
all-or-nothing: on failure nothing changes.
"""
from __future__ import annotations

from collections import deque


class PoolError(Exception):
    def __init__(self, kind: str, msg: str = ""):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind  # "EINVAL" or "ENOMEM"


class _Seq:
    __slots__ = ("alive", "has_res", "length", "bpages", "rpages")

    def __init__(self, has_res: bool):
        self.alive, self.has_res, self.length = True, has_res, 0
        self.bpages, self.rpages = [], []


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class PoolModel:
    def __init__(self, num_bpages, num_rpages, page_size=16, bpage_order=None, rpage_order=None):
        self.P = page_size
        self.nb, self.nr = num_bpages, num_rpages
        self.free_b = deque(range(num_bpages) if bpage_order is None else map(int, bpage_order))
        self.free_r = deque(range(num_rpages) if rpage_order is None else map(int, rpage_order))
        self.ref_b = [0] * num_bpages
        self.ref_r = [0] * num_rpages
        self.seqs: list[_Seq] = []

    # ---- helpers -------------------------------------------------------------------------
    def _seq(self, h) -> _Seq:
        if not (0 <= h < len(self.seqs)) or not self.seqs[h].alive:
            raise PoolError("EINVAL", f"bad sequence handle {h}")
        return self.seqs[h]

    def _take_b(self):
        p = self.free_b.popleft()
        self.ref_b[p] = 1
        return p

    def _take_r(self):
        p = self.free_r.popleft()
        self.ref_r[p] = 1
        return p

    # ---- operations ----------------------------------------------------------------------
    def create(self, with_residual: bool) -> int:
        self.seqs.append(_Seq(bool(with_residual)))
        return len(self.seqs) - 1

    def append(self, h, n):
        """Reserve n new rows at the end of sequence h.

        Returns (bslots, rslots, cow): slot = page * P + row for each new row
        (rslots are -1 for a base-only sequence) and the copy-on-write row copy
        this append needs, as ``(src_page, dst_page, n_rows)`` or None.
        """
        s = self._seq(h)
        if n < 0:
            raise PoolError("EINVAL", "negative length")
        P = self.P
        new_len = s.length + n
        grow = _ceil_div(new_len, P) - len(s.bpages)
        cow = n > 0 and s.length % P != 0 and self.ref_b[s.bpages[-1]] > 1
        need_b = grow + (1 if cow else 0)
        need_r = grow if s.has_res else 0
        if need_b > len(self.free_b) or need_r > len(self.free_r):
            raise PoolError("ENOMEM", "pool exhausted")
        cow_op = None
        if cow:
            old = s.bpages[-1]
            new = self._take_b()
            self.ref_b[old] -= 1
            s.bpages[-1] = new
            cow_op = (old, new, s.length % P)
        for _ in range(grow):
            s.bpages.append(self._take_b())
            if s.has_res:
                s.rpages.append(self._take_r())
        bslots, rslots = [], []
        for t in range(s.length, new_len):
            bslots.append(s.bpages[t // P] * P + t % P)
            rslots.append(s.rpages[t // P] * P + t % P if s.has_res else -1)
        s.length = new_len
        return bslots, rslots, cow_op

    def fork(self, parent, alias_len):
        """New agent sharing the parent's first alias_len rows.

        Full pages are aliased (reference count + 1).  A partial tail is packed:
        a private page receives a copy of its alias_len % P rows.  The child gets
        fresh residual pages for [0, alias_len).  Returns (child, cow) with cow
        as in ``append``.
        """
        p = self._seq(parent)
        if not (0 <= alias_len <= p.length):
            raise PoolError("EINVAL", "alias_len out of range")
        P = self.P
        full, tail = divmod(alias_len, P)
        need_b = 1 if tail else 0
        need_r = _ceil_div(alias_len, P)
        if need_b > len(self.free_b) or need_r > len(self.free_r):
            raise PoolError("ENOMEM", "pool exhausted")
        c = _Seq(True)
        for pg in p.bpages[:full]:
            self.ref_b[pg] += 1
            c.bpages.append(pg)
        cow_op = None
        if tail:
            new = self._take_b()
            c.bpages.append(new)
            cow_op = (p.bpages[full], new, tail)
        for _ in range(need_r):
            c.rpages.append(self._take_r())
        c.length = alias_len
        self.seqs.append(c)
        return len(self.seqs) - 1, cow_op

    def free(self, h):
        s = self._seq(h)
        for pg in s.bpages:
            self.ref_b[pg] -= 1
            if self.ref_b[pg] == 0:
                self.free_b.append(pg)
        for pg in s.rpages:
            self.ref_r[pg] -= 1
            if self.ref_r[pg] == 0:
                self.free_r.append(pg)
        s.alive = False
        s.bpages, s.rpages, s.length = [], [], 0

    # ---- views ---------------------------------------------------------------------------
    def length(self, h) -> int:
        return self._seq(h).length

    def tables(self, handles, max_pages):
        """Block tables [n][max_pages] (-1 padded) and lengths, as nested lists."""
        bt, rt, lens = [], [], []
        for h in handles:
            s = self._seq(h)
            if len(s.bpages) > max_pages:
                raise PoolError("EINVAL", "max_pages too small")
            bt.append(s.bpages + [-1] * (max_pages - len(s.bpages)))
            rt.append(s.rpages + [-1] * (max_pages - len(s.rpages)))
            lens.append(s.length)
        return bt, rt, lens

    def stats(self) -> dict:
        return {
            "live_bpages": self.nb - len(self.free_b),
            "live_rpages": self.nr - len(self.free_r),
            "free_bpages": len(self.free_b),
            "free_rpages": len(self.free_r),
            "shared_bpages": sum(1 for c in self.ref_b if c > 1),
            "bpage_refs": sum(self.ref_b),
            "rpage_refs": sum(self.ref_r),
        }

    def replay(self, ops):
        """Apply a workload operation script; returns {name: handle}."""
        names = {}
        for op in ops:
            if op[0] == "create":
                names[op[1]] = self.create(bool(op[2]))
            elif op[0] == "append":
                self.append(names[op[1]], op[2])
            elif op[0] == "fork":
                names[op[3]], _ = self.fork(names[op[1]], op[2])
            else:
                raise ValueError(op)
        return names
