"""The persistent schedule of the matrix-core backward, checked on the CPU.

`Schedule` and `Run` (attention_fa_bwd_amd/csrc/mfma_common.hpp), the work
items and tile cursors of the two passes (`KeyItem`/`KeyCursor` in bwd_dkdv.hpp,
`QueryItem`/`QueryCursor` in bwd_dq.hpp) and the phase structure of their role
loops (`dkdv_run`, `dq_run`) are restated here in Python, statement for
statement, and run for every workgroup of a grid.  The checks are the ones a
GPU run cannot make without risking a hang: within each workgroup the score
waves and the gradient waves pass the same number of barriers; every work
item of either pass is run by exactly one workgroup, whole; the tile (or key
block) a score wave reads in phase g is the one staged into that buffer
before it, and the gradient waves reduce the same tile, from the same
buffers, one phase later.  The shapes cover both causal modes, ragged N, item
counts with and without the XCD shares (divisible by 8 or not), single-item
and many-item workgroups, and CU counts of 256, 13 and 8.
"""
import pytest

BC, BR = 128, 64        # dK/dV pass: keys per work item, queries per tile
BQ, BK = 256, 32        # dQ pass: queries per work item, keys per block
NKB, NVB = 4, 3         # dQ pass: K and V buffers


def heavy_first(work, nwork, nb):
    """(head, rank) of a causal work item, heaviest first, head pairs
    interleaved when each XCD's share holds whole pairs."""
    if nwork % 8 == 0 and (nwork // 8) % (2 * nb) == 0:
        r = work % (2 * nb)
        return 2 * (work // (2 * nb)) + (r & 1), r >> 1
    return work // nb, work % nb


class Schedule:
    def __init__(self, n0, n1, G, b):
        xcd = n0 % 8 == 0 and n1 % 8 == 0 and G % 8 == 0
        parts = 8 if xcd else 1
        x = b % 8 if xcd else 0
        self.slot = b // 8 if xcd else b
        self.slots = G // parts
        self.share0, self.share1 = n0 // parts, n1 // parts
        self.base0, self.base1 = x * self.share0, x * self.share1

    def pos(self, m):
        return m * self.slots + ((self.slots - 1 - self.slot) if m & 1 else self.slot)

    def first_round(self, v):
        m = v // self.slots
        return m + 1 if self.pos(m) < v else m


class Run:
    def __init__(self, s, kind):
        self.lo = s.share0 if kind else 0
        self.m0 = s.first_round(self.lo)
        self.m1 = s.first_round(s.share0 + s.share1 if kind else s.share0)
        self.base = s.base1 if kind else s.base0

    def item(self, s, m):
        return self.base + s.pos(m) - self.lo


def key_item(work, nwork, nkb, N, causal):
    head, kblk = work // nkb, work % nkb
    if causal:
        head, kblk = heavy_first(work, nwork, nkb)
    q_begin = kblk * BC if causal else 0
    return dict(id=(head, kblk), n=(N - q_begin + BR - 1) // BR)


def query_item(work, nwork, nqb, N, causal):
    head, qblk = work // nqb, work % nqb
    if causal:
        head, qblk = heavy_first(work, nwork, nqb)
        qblk = nqb - 1 - qblk
    kend = min(N, qblk * BQ + BQ) if causal else N
    return dict(id=(head, qblk), n=(kend + BK - 1) // BK)


class Cursor:
    def __init__(self, m, item, make):
        self.m, self.p, self.it, self.make = m, 0, item, make

    def valid(self, r):
        return self.m < r.m1

    def advance(self, s, r):
        self.p += 1
        if self.p == self.it["n"]:
            self.p = 0
            self.m += 1
            if self.m < r.m1:
                self.it = self.make(r.item(s, self.m))

    def tile(self):
        return self.it["id"], self.p


def dkdv_run(s, r, make):
    """(barriers of score waves, barriers of gradient waves, items stored)."""
    if r.m0 >= r.m1:
        return 0, 0, []
    first = make(r.item(s, r.m0))
    staged = {0: ((first["id"], 0), 0)}          # phase -> (tile, Q/dO buffer)
    # score waves
    scored, bars_s, it, qb, pb, g = {}, 0, first, 0, 0, 0
    for m in range(r.m0, r.m1):
        nxt = make(r.item(s, m + 1)) if m + 1 < r.m1 else it
        for p in range(it["n"]):
            scored[g] = ((it["id"], p), qb, pb)
            qb, pb, g, bars_s = (0 if qb == 2 else qb + 1), pb ^ 1, g + 1, bars_s + 1
        it = nxt
    bars_s += 1
    # gradient waves
    stg, grd = Cursor(r.m0, first, make), Cursor(r.m0, first, make)
    acc_item, stored, reduced, bars_g, qb, pb, g = first, [], {}, 0, 0, 0, 0
    while True:
        stg.advance(s, r)
        qbn = 0 if qb == 2 else qb + 1
        if stg.valid(r):
            staged[g + 1] = (stg.tile(), qbn)
        if g >= 1:
            if grd.p == 0 and grd.m > r.m0:
                stored.append(acc_item["id"])
            if grd.p == 0:
                acc_item = grd.it
            reduced[g] = (grd.tile(), 2 if qb == 0 else qb - 1, pb ^ 1)
            grd.advance(s, r)
        bars_g += 1
        if not grd.valid(r):
            break
        qb, pb, g = qbn, pb ^ 1, g + 1
    stored.append(acc_item["id"])
    for g, (t, q, p) in scored.items():
        assert staged[g] == (t, q), ("dK/dV staging", g)
        assert reduced[g + 1] == (t, q, p), ("dK/dV reduction", g)
    return bars_s, bars_g, stored


def dq_run(s, r, make):
    if r.m0 >= r.m1:
        return 0, 0, []
    first = make(r.item(s, r.m0))
    stg = Cursor(r.m0, first, make)
    staged = {0: (stg.tile(), 0, 0)}              # block -> (tile, K buffer, V buffer)
    stg.advance(s, r)
    if stg.valid(r):
        staged[1] = (stg.tile(), 1, 1)
    # score waves
    scored, bars_s, it, g = {}, 0, first, 0
    for m in range(r.m0, r.m1):
        for p in range(it["n"]):
            scored[g] = ((it["id"], p), g % NKB, g % NVB, g & 1)
            g, bars_s = g + 1, bars_s + 1
        if m + 1 < r.m1:
            it = make(r.item(s, m + 1))
    bars_s += 1
    # gradient waves
    grd = Cursor(r.m0, first, make)
    acc_item, stored, reduced, bars_g, g = first, [], {}, 0, 0
    while True:
        stg.advance(s, r)
        if stg.valid(r):
            staged[g + 2] = (stg.tile(), (g + 2) % NKB, (g + 2) % NVB)
        if g >= 1:
            if grd.p == 0 and grd.m > r.m0:
                stored.append(acc_item["id"])
            if grd.p == 0:
                acc_item = grd.it
            reduced[g] = (grd.tile(), (g - 1) % NKB, (g - 1) & 1)
            grd.advance(s, r)
        bars_g += 1
        if not grd.valid(r):
            break
        g += 1
    stored.append(acc_item["id"])
    for g, (t, kb, vb, db) in scored.items():
        assert staged[g] == (t, kb, vb), ("dQ staging", g)
        assert reduced[g + 1] == (t, kb, db), ("dQ reduction", g)
    return bars_s, bars_g, stored


def run_grid(mode, N, nh, causal, cus):
    nqb, nkb = (N + BQ - 1) // BQ, (N + BC - 1) // BC
    nq, nk = nqb * nh, nkb * nh
    mq = lambda w: query_item(w, nq, nqb, N, causal)
    mk = lambda w: key_item(w, nk, nkb, N, causal)
    total = {"fused": nq + nk, "dq": nq, "dkdv": nk}[mode]
    G = min(cus, total)
    done_q, done_k = [], []
    for b in range(G):
        if mode == "fused":
            s = Schedule(nq, nk, G, b)
            runs = [(dq_run, Run(s, 0), mq, done_q), (dkdv_run, Run(s, 1), mk, done_k)]
        elif mode == "dq":
            s = Schedule(nq, 0, G, b)
            runs = [(dq_run, Run(s, 0), mq, done_q)]
        else:
            s = Schedule(nk, 0, G, b)
            runs = [(dkdv_run, Run(s, 0), mk, done_k)]
        for fn, r, make, done in runs:
            bars_score, bars_grad, stored = fn(s, r, make)
            assert bars_score == bars_grad, (mode, N, nh, causal, cus, b)
            done += stored
    if mode in ("fused", "dq"):
        assert sorted(done_q) == sorted({(h, q) for h in range(nh) for q in range(nqb)})
    if mode in ("fused", "dkdv"):
        assert sorted(done_k) == sorted({(h, k) for h in range(nh) for k in range(nkb)})


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 31, 33, 65, 129, 255, 257, 300, 1000, 4000])
def test_schedule_barriers_coverage_handoffs(N, causal):
    for nh in (1, 3, 8, 16, 64):
        for cus in (256, 13, 8):
            for mode in ("fused", "dq", "dkdv"):
                run_grid(mode, N, nh, causal, cus)


def test_one_item_per_workgroup_when_grid_equals_items():
    """The dQ pass that writes 16-bit dQ directly is launched with one
    workgroup per item; the schedule then gives each exactly one."""
    for n in range(1, 1100):
        for b in range(n):
            r = Run(Schedule(n, 0, n, b), 0)
            assert r.m1 - r.m0 == 1, (n, b)


def test_snake_order_balances_causal_work():
    """Heaviest-first items dealt in snake order: on the bench shape's causal
    mode every workgroup's dK/dV tiles are within 4 % of the mean."""
    N, nh = 8192, 32
    nkb = N // BC
    nk = nkb * nh
    loads = []
    for b in range(256):
        s = Schedule(nk, 0, 256, b)
        r = Run(s, 0)
        loads.append(sum(key_item(r.item(s, m), nk, nkb, N, True)["n"] for m in range(r.m0, r.m1)))
    mean = sum(loads) / len(loads)
    assert max(loads) <= 1.04 * mean and min(loads) >= 0.96 * mean
