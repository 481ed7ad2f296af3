"""Multi-query attention: the host planner's work split and the kernel's position arithmetic,
checked on the CPU before any launch.

The planner runs through the host-only driver program.  The kernel's mapping from (wave task,
step, lane element) to a cache position is mirrored here line for line from kv4_mq.hip, and the
test checks that every query row attends exactly positions 0 .. its own position, each once,
from the copy decode reads at length L (INT8 slot when protected, INT4 page otherwise), and that
every page and INT8 tile index the kernel forms stays inside the sequence's buffers.
"""
import math

import pytest

import oracle
from tests.test_host_abi import Planner, driver  # noqa: F401  (fixture)

P = 16


def _plan(pl, target, calls):
    line = "multi %d %d " % (target, len(calls)) + " ".join("%d %d" % c for c in calls)
    first, rows = pl.cmd(line, block=True)
    st = dict(zip(first[0::2], (int(x) for x in first[1::2])))
    return st, rows


def _positions(kind, s, k, L, S, R, n8, fmt):
    """Position of step element k (0..31) of unit step s, or None (kv4_mq.hip: positions())."""
    if kind == "int4":
        p0 = S // P
        p = P * (p0 + 2 * (s - n8)) + k
        return p if S <= p < L - R else None
    if fmt == 1:
        p = 32 * s + k
        return p if p < L else None
    u = 32 * s + k
    if u < S:
        return u if u < L else None
    if u < S + R:
        base = max(S, L - R)
        r = (u - S) - base % R
        if r < 0:
            r += R
        q = base + r
        return q if q < L else None
    return None


def _emulate(st, entries, hq, hkv, S, R, fmt):
    G = hq // hkv
    QT = 16 // G
    spc, n8 = st["spc"], st["n8"]
    seen = {}
    task0s = [e[4] for e in entries]
    for w in range(st["tasks"]):
        ei = max(i for i, t0 in enumerate(task0s) if t0 <= w)
        seq, L, nq, qrow0, task0, grp0, steps, nch = entries[ei]
        nrt = -(-nq * G // 16)
        local = w - task0
        head = local // (nch * nrt)
        local -= head * nch * nrt
        chunk, rt = divmod(local, nrt)
        assert 0 <= head < hkv and 0 <= chunk < nch
        s0 = chunk * spc
        s1 = min(s0 + spc, steps)
        assert s0 < s1
        n8e = steps if fmt == 1 else n8
        kinds = [("int8", s) for s in range(s0, min(s1, n8e))] + [("int4", s) for s in range(max(s0, n8e), s1)]
        if fmt == 1:
            assert all(k == "int8" for k, _ in kinds)
        for kind, s in kinds:
            # buffer indices the kernel forms (clamped second page / tile)
            if kind == "int4":
                p0 = S // P
                p1 = (L - R - 1) // P + 1
                pi = p0 + 2 * (s - n8)
                assert p0 <= pi < p1 <= math.ceil(L / P)
            elif fmt == 1:
                assert 2 * s < math.ceil(L / P)
            else:
                assert 2 * s < math.ceil((S + R) / P)
            for k in range(32):
                pos = _positions(kind, s, k, L, S, R, n8, fmt)
                if pos is None:
                    continue
                if kind == "int8" and fmt == 0:
                    assert oracle.int8_slot(pos, S, R) == 32 * s + k
                for r in range(16):
                    jq = rt * QT + r // G
                    if jq >= nq:
                        continue
                    pos_r = L - nq + jq
                    if pos <= pos_r:
                        key = (seq, head, jq, r % G)
                        seen.setdefault(key, []).append((pos, kind))
    return seen


def _check_plan_order(st, entries, calls, hkv, G, target):
    """Entries longest first; row offsets in call order; first tasks and merge groups contiguous
    along the list; the task count within the target whenever one task per row tile allows it."""
    nq_of = dict(calls)
    rows_before, acc = {}, 0
    for seq, nq in calls:
        rows_before[seq] = acc
        acc += nq
    steps = [e[6] for e in entries]
    assert steps == sorted(steps, reverse=True)
    assert sorted(e[0] for e in entries) == sorted(nq_of)
    t = g = 0
    for seq, L, nq, qrow0, task0, grp0, st_, nch in entries:
        assert nq == nq_of[seq] and qrow0 == rows_before[seq]
        assert (task0, grp0) == (t, g)
        nrt = -(-nq * G // 16)
        t += hkv * nch * nrt
        g += hkv * nrt
        assert nch == -(-st_ // st["spc"])
    assert (t, g) == (st["tasks"], st["groups"])
    if st["groups"] <= target:
        assert st["tasks"] <= target
    else:
        assert st["tasks"] == st["groups"]  # one chunk per (sequence, kv head, row tile)


@pytest.mark.parametrize("hq,hkv,S,R,fmt,lens,nqs,target", [
    (32, 8, 4, 128, 0, [1, 17, 132, 133, 300, 700], [1, 5, 16, 40, 133, 150], 64),
    (32, 8, 4, 128, 0, [700, 2000], [3, 1], 4096),
    (8, 2, 4, 32, 0, [36, 37, 90, 500], [36, 7, 90, 64], 7),
    (4, 4, 0, 0, 0, [1, 15, 16, 17, 400], [1, 15, 2, 17, 33], 16),
    (16, 8, 4, 0, 0, [3, 50, 260], [3, 20, 11], 9),
    (16, 8, 0, 40, 0, [39, 40, 41, 300], [39, 12, 41, 100], 30),
    (8, 4, 0, 0, 1, [1, 31, 32, 33, 500], [1, 31, 5, 33, 77], 12),
])
def test_rows_attend_each_position_once_from_the_right_copy(driver, hq, hkv, S, R, fmt, lens, nqs, target):
    pl = Planner(driver)
    try:
        first, _ = pl.cmd("init %d %d 128 16 4096 16 512 %d %d 128 %d" % (hq, hkv, S, R, fmt))
        assert first == ["status", "0"]
        for i, L in enumerate(lens):
            first, _ = pl.cmd("append 1 %d %d" % (i, L), block=True)
            assert first == ["status", "0"]
        st, entries = _plan(pl, target, list(enumerate(nqs)))
        assert st["status"] == 0
        G = hq // hkv
        assert st["groups"] == sum(hkv * -(-nq * G // 16) for nq in nqs)
        _check_plan_order(st, entries, list(enumerate(nqs)), hkv, G, target)
        seen = _emulate(st, entries, hq, hkv, S, R, fmt)
        for seq, (L, nq) in enumerate(zip(lens, nqs)):
            for h in range(hkv):
                for jq in range(nq):
                    for gi in range(G):
                        got = sorted(seen.get((seq, h, jq, gi), []))
                        pos_r = L - nq + jq
                        assert [p for p, _ in got] == list(range(pos_r + 1)), (seq, h, jq, gi)
                        for p, kind in got:
                            want = "int8" if (fmt == 1 or _prot(p, L, S, R)) else "int4"
                            assert kind == want, (p, L)
    finally:
        pl.close()


def _prot(t, L, S, R):
    return t < min(S, L) or max(S, L - R) <= t < L


def test_multi_plan_errors(driver):
    pl = Planner(driver)
    try:
        assert pl.cmd("init 8 2 64 16 256 8 64 4 32 64 0")[0] == ["status", "0"]
        assert pl.cmd("append 2 0 10 1 40", block=True)[0] == ["status", "0"]
        assert _plan(pl, 100, [(0, 11)])[0]["status"] == 3   # n_q > L
        assert _plan(pl, 100, [(0, 0)])[0]["status"] == 1    # n_q < 1
        assert _plan(pl, 100, [(2, 1)])[0]["status"] == 3    # empty sequence
        assert _plan(pl, 100, [(0, 1), (0, 1)])[0]["status"] == 1
        assert _plan(pl, 100, [(9, 1)])[0]["status"] == 1
        st, rows = _plan(pl, 100, [])
        assert st["status"] == 0 and st["tasks"] == 0 and rows == []
        assert pl.cmd("init 8 2 64 16 256 8 64 4 32 1 2")[0] == ["status", "0"]
        assert pl.cmd("append 1 0 10", block=True)[0] == ["status", "0"]
        assert _plan(pl, 100, [(0, 1)])[0]["status"] == 5    # BF16: unsupported
    finally:
        pl.close()


def _xcd_grouped_block(b, nb):
    """Workgroup b's task block (kv4_mq.hip: xcd_grouped_block())."""
    full = nb // 32 * 32
    if b >= full:
        return b
    xcd, slot = b & 7, b >> 3
    return (slot >> 2) * 32 + xcd * 4 + (slot & 3)


@pytest.mark.parametrize("nb", [1, 5, 31, 32, 33, 64, 95, 257, 1024])
def test_xcd_grouped_block_is_a_bijection(nb):
    got = [_xcd_grouped_block(b, nb) for b in range(nb)]
    assert sorted(got) == list(range(nb))
    full = nb // 32 * 32
    for b in range(full):
        # four consecutive task blocks run on one XCD (b % 8)
        assert _xcd_grouped_block(b, nb) // 4 == (b >> 5) * 8 + (b & 7)


@pytest.mark.parametrize("lens,nqs,target", [
    ([300, 700, 2000, 5000], [16, 13, 64, 61], 64),
    ([300, 700, 2000, 5000], [16, 13, 64, 61], 4096),
    ([4096] * 6, [64] * 6, 100000),
    ([1000 + 256], [256], 512),
])
def test_shared_workgroups_take_four_row_tiles_of_one_chunk(driver, lens, nqs, target):
    """The workgroup-shared multi-query kernel is launched when every entry has a multiple of 4
    row tiles; its four waves (tasks 4k .. 4k + 3) must then be row tiles of one (entry, kv head,
    chunk), so that they stage the same pages and pass the same barriers."""
    hq, hkv = 32, 8
    G = hq // hkv
    pl = Planner(driver)
    try:
        first, _ = pl.cmd("init %d %d 128 16 8192 16 512 4 128 128 0" % (hq, hkv))
        assert first == ["status", "0"]
        for i, L in enumerate(lens):
            assert pl.cmd("append 1 %d %d" % (i, L), block=True)[0] == ["status", "0"]
        st, entries = _plan(pl, target, list(enumerate(nqs)))
        assert st["status"] == 0
        assert all(-(-int(e[2]) * G // 16) % 4 == 0 for e in entries)
        assert st["tasks"] % 4 == 0
        task0s = [int(e[4]) for e in entries]
        where = []
        for w in range(st["tasks"]):
            ei = max(i for i, t0 in enumerate(task0s) if t0 <= w)
            nq, nch = int(entries[ei][2]), int(entries[ei][7])
            nrt = -(-nq * G // 16)
            local = w - task0s[ei]
            head = local // (nch * nrt)
            local -= head * nch * nrt
            chunk, rt = divmod(local, nrt)
            where.append((ei, head, chunk, rt))
        for k in range(0, st["tasks"], 4):
            quad = where[k:k + 4]
            assert len({q[:3] for q in quad}) == 1, quad
            assert [q[3] for q in quad] == list(range(quad[0][3], quad[0][3] + 4)), quad
    finally:
        pl.close()
