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
* ForkServe README, "Design vs APC" (the adaptive unaligned tail): instead of
  packing, a fork may *freeze* the trunk's partial tail -- one read-only page
  shared by the trunk and every child (``pages_freeze = 1 + k * ceil(l / P)``);
  rows after it go to fresh pages, so a sequence's pages no longer start at
  multiples of P.  Each logical page therefore carries its start position (the
  slot map); a page holds ``next start - start`` rows (P for a full page, fewer
  for a frozen tail), the last page ``length - start``.  ``AUTO`` packs when the
  trunk tail plus the child's expected suffix fit in one page, else freezes.
* ForkKV study note, "Error / eviction recovery" and trick 1 of the
  implementation details: base and residual caches are evicted independently.
  ``evict_base`` drops base pages from every sequence that maps them (their table
  entries become -1) while the residual pages survive; ``refill_base`` maps fresh
  base pages back into the sequences that lost them (a partial hit), into which the
  caller writes the recomputed base rows.  A sequence with a missing base page can
  be neither appended to nor forked (``ESTATE``) until it is refilled.

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
        self.kind = kind  # "EINVAL", "ENOMEM" or "ESTATE"


PACK, FREEZE, AUTO = 0, 1, 2  # fork modes for an unaligned tail


class _Seq:
    __slots__ = ("alive", "has_res", "length", "bpages", "rpages", "starts", "closed")

    def __init__(self, has_res: bool):
        self.alive, self.has_res, self.length = True, has_res, 0
        self.bpages, self.rpages, self.starts = [], [], []
        self.closed = False  # the last page takes no more rows (a frozen tail)

    def rows(self, j):
        """Rows of logical page j that belong to this sequence."""
        end = self.starts[j + 1] if j + 1 < len(self.starts) else self.length
        return end - self.starts[j]

    def room(self, P):
        """Rows that still fit in the last page."""
        if not self.bpages or self.closed:
            return 0
        return P - self.rows(len(self.bpages) - 1)


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
        this append needs, as ``(src_page, dst_page, n_rows)`` or None.  Rows fill
        the last page while it has room (a frozen tail has none), then fresh pages.
        """
        s = self._seq(h)
        if n < 0:
            raise PoolError("EINVAL", "negative length")
        if -1 in s.bpages:
            raise PoolError("ESTATE", "base pages evicted; refill first")
        P = self.P
        room = s.room(P)
        grow = _ceil_div(max(0, n - room), P)
        last = len(s.bpages) - 1
        cow = n > 0 and room > 0 and s.rows(last) > 0 and self.ref_b[s.bpages[last]] > 1
        need_b = grow + (1 if cow else 0)
        need_r = grow if s.has_res else 0
        if need_b > len(self.free_b) or need_r > len(self.free_r):
            raise PoolError("ENOMEM", "pool exhausted")
        cow_op = None
        if cow:
            old = s.bpages[last]
            new = self._take_b()
            self.ref_b[old] -= 1
            s.bpages[last] = new
            cow_op = (old, new, s.rows(last))
        first_new = len(s.bpages)
        nxt = s.length + room  # start of the first fresh page
        for i in range(grow):
            s.bpages.append(self._take_b())
            s.starts.append(nxt + i * P)
            if s.has_res:
                s.rpages.append(self._take_r())
        bslots, rslots = [], []
        for t in range(s.length, s.length + n):
            if t < nxt:
                j, row = last, t - s.starts[last]
            else:
                j, row = first_new + (t - nxt) // P, (t - nxt) % P
            bslots.append(s.bpages[j] * P + row)
            rslots.append(s.rpages[j] * P + row if s.has_res else -1)
        s.length += n
        if grow:
            s.closed = False
        return bslots, rslots, cow_op

    def fork(self, parent, alias_len, mode=PACK, suffix_hint=0):
        """New agent sharing the parent's first alias_len rows.

        Whole pages (full, or frozen tails) below alias_len are aliased (reference
        count + 1).  A page cut by alias_len -- or the parent's open partial last
        page -- is the unaligned tail: PACK gives the child a private page with a
        copy of its rows; FREEZE (only at the parent's end) makes it a read-only
        page of the parent and the child, whose later rows start fresh pages;
        AUTO packs when tail + suffix_hint <= P (or the cut is not at the parent's
        end), else freezes.  The child gets
        fresh residual pages for each of its logical pages.  Returns (child, cow)
        with cow as in ``append``.
        """
        p = self._seq(parent)
        if not (0 <= alias_len <= p.length) or mode not in (PACK, FREEZE, AUTO) or suffix_hint < 0:
            raise PoolError("EINVAL", "alias_len or mode out of range")
        P = self.P
        n_pg = len(p.bpages)
        whole, tail_j, tail = 0, -1, 0
        for j in range(n_pg):
            st, nr = p.starts[j], p.rows(j)
            if st >= alias_len:
                break
            is_open = j == n_pg - 1 and not p.closed and nr < P
            if st + nr <= alias_len and not is_open:
                whole += 1
            else:
                tail_j, tail = j, alias_len - st
                break
        if -1 in p.bpages[:whole + (1 if tail else 0)]:
            raise PoolError("ESTATE", "base pages evicted; refill first")
        if mode == AUTO:
            mode = PACK if tail + suffix_hint <= P or alias_len != p.length else FREEZE
        if tail and mode == FREEZE and alias_len != p.length:
            raise PoolError("EINVAL", "a tail can only be frozen at the parent's end")
        freeze = bool(tail) and mode == FREEZE
        need_b = 1 if tail and not freeze else 0
        need_r = whole + (1 if tail else 0)
        if need_b > len(self.free_b) or need_r > len(self.free_r):
            raise PoolError("ENOMEM", "pool exhausted")
        c = _Seq(True)
        for pg in p.bpages[:whole]:
            self.ref_b[pg] += 1
        c.bpages = p.bpages[:whole]
        c.starts = p.starts[:whole]
        cow_op = None
        if tail:
            c.starts.append(p.starts[tail_j])
            if freeze:
                pg = p.bpages[tail_j]
                self.ref_b[pg] += 1
                c.bpages.append(pg)
                p.closed = True
                c.closed = True
            else:
                new = self._take_b()
                c.bpages.append(new)
                cow_op = (p.bpages[tail_j], new, tail)
        elif whole and c.starts[-1] + (p.rows(whole - 1)) == alias_len and p.rows(whole - 1) < P:
            c.closed = True  # ends on a frozen tail
        for _ in range(need_r):
            c.rpages.append(self._take_r())
        c.length = alias_len
        self.seqs.append(c)
        return len(self.seqs) - 1, cow_op

    def free(self, h):
        s = self._seq(h)
        for pg in s.bpages:
            if pg < 0:
                continue  # evicted
            self.ref_b[pg] -= 1
            if self.ref_b[pg] == 0:
                self.free_b.append(pg)
        for pg in s.rpages:
            self.ref_r[pg] -= 1
            if self.ref_r[pg] == 0:
                self.free_r.append(pg)
        s.alive = False
        s.bpages, s.rpages, s.starts, s.length, s.closed = [], [], [], 0, False

    def evict_base(self, pages):
        """Evict base pages: every live sequence mapping one loses it (entry -1); the
        pages return to the tail of the free list in the order given.  Residual pages
        are untouched."""
        pages = [int(x) for x in pages]
        if len(set(pages)) != len(pages) or any(
                not (0 <= pg < self.nb) or self.ref_b[pg] == 0 for pg in pages):
            raise PoolError("EINVAL", "not a list of distinct live base pages")
        gone = set(pages)
        for s in self.seqs:
            if s.alive:
                s.bpages = [-1 if pg in gone else pg for pg in s.bpages]
        for pg in pages:
            self.ref_b[pg] = 0
            self.free_b.append(pg)

    def refill_base(self, handles, lp0, lp1):
        """Map fresh base pages into logical pages [lp0, lp1) of every listed sequence,
        all of which must miss exactly those pages and agree on their start positions
        and row counts.  Returns the new pages (one per logical page, shared by all)."""
        ss = [self._seq(h) for h in handles]
        if not ss or len(set(handles)) != len(handles) or not (0 <= lp0 < lp1):
            raise PoolError("EINVAL", "bad refill range")
        for s in ss:
            if lp1 > len(s.bpages) or any(s.bpages[j] != -1 for j in range(lp0, lp1)):
                raise PoolError("EINVAL", "refill range is not evicted in every sequence")
            if any(s.starts[j] != ss[0].starts[j] or s.rows(j) != ss[0].rows(j)
                   for j in range(lp0, lp1)):
                raise PoolError("EINVAL", "sequences disagree on the refilled pages")
        if lp1 - lp0 > len(self.free_b):
            raise PoolError("ENOMEM", "pool exhausted")
        new = []
        for j in range(lp0, lp1):
            pg = self._take_b()
            self.ref_b[pg] = len(ss)
            for s in ss:
                s.bpages[j] = pg
            new.append(pg)
        return new

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

    def starts_table(self, handles, max_pages):
        """Start position of every logical page [n][max_pages] (-1 padded)."""
        out = []
        for h in handles:
            s = self._seq(h)
            if len(s.starts) > max_pages:
                raise PoolError("EINVAL", "max_pages too small")
            out.append(s.starts + [-1] * (max_pages - len(s.starts)))
        return out

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
                names[op[3]], _ = self.fork(names[op[1]], op[2], *op[4:])
            else:
                raise ValueError(op)
        return names
