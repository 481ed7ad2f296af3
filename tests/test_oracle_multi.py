"""Pins of the oracle's multi-query (causal) attention over the cache (CPU only).

Reading pinned here: the n query rows of a sequence of length L sit at positions L-n .. L-1, row r
attends positions 0 .. L-n+r, and every position is read from the copy decode reads at length L.
Each pin ties the new entry point to something fixed independently of its own loop: the pinned
decode attention, a second cache that holds only a prefix, or a dependence (invariance) that any
causal implementation must show.
"""
import numpy as np
import pytest

import oracle

from tests.test_oracle_cache import _bits, _cache, _kv


def _filled(S, R, b, L, seed, hq=4, hkv=2, d=64, outliers=(3, 17)):
    rng = np.random.default_rng(seed)
    c = _cache(hq=hq, hkv=hkv, d=d, num_pages=256, max_seqs=8, max_pps=64, S=S, R=R, b=b)
    k, v = _kv(rng, L, hkv, d, outliers)
    assert c.append([0], [L], k, v) == oracle.OK
    return c, k, v, rng


@pytest.mark.parametrize("S,R,b", [(4, 32, 64), (0, 0, 1), (2, 5, 16)])
def test_one_row_is_decode(S, R, b):
    """n = 1 for every sequence reduces to decode attention (bit-identical)."""
    rng = np.random.default_rng(1)
    c = _cache(S=S, R=R, b=b)
    lens = [1, 37, 200]
    for i, L in enumerate(lens):
        k, v = _kv(rng, L, 2, 64, (5,))
        assert c.append([i], [L], k, v) == oracle.OK
    q = _bits(rng.standard_normal((3, 4, 64)))
    a, _ = c.attend_multi([2, 0, 1], [1, 1, 1], q)
    d, _ = c.decode([2, 0, 1], q)
    assert np.array_equal(a, d)


@pytest.mark.parametrize("S,R,b,L,n", [(0, 0, 1, 150, 40), (0, 0, 64, 150, 40), (4, 32, 64, 30, 12),
                                       (4, 128, 32, 131, 60)])
def test_rows_equal_decode_of_prefix_caches(S, R, b, L, n):
    """When no position changes copy between length p+1 and length L (no protection, or every
    position protected), row r equals decode of a cache holding only positions 0 .. p, p = L-n+r."""
    assert S + R == 0 or L <= S + R
    c, k, v, rng = _filled(S, R, b, L, seed=L + n)
    q = _bits(rng.standard_normal((n, 4, 64)))
    out, _ = c.attend_multi([0], [n], q)
    for r in (0, 1, n // 2, n - 1):
        p = L - n + r
        c2 = _cache(S=S, R=R, b=b)
        assert c2.append([0], [p + 1], k[:p + 1], v[:p + 1]) == oracle.OK
        ref, _ = c2.decode([0], q[r:r + 1])
        assert np.array_equal(out[r], ref[0]), r


def test_last_row_is_decode_at_full_length():
    """With protection active and L > S + R, the last row attends everything: it equals decode."""
    c, k, v, rng = _filled(4, 32, 64, 300, seed=3)
    q = _bits(rng.standard_normal((50, 4, 64)))
    out, _ = c.attend_multi([0], [50], q)
    ref, _ = c.decode([0], q[49:50])
    assert np.array_equal(out[49], ref[0])


def test_rows_ignore_later_positions_and_see_their_own():
    """Row r depends on positions <= L-n+r only: rewriting later positions (same length, so the same
    copies are read) leaves it unchanged, and rewriting position L-n+r changes it."""
    S, R, b, L, n = 4, 32, 64, 300, 48
    c, k, v, rng = _filled(S, R, b, L, seed=5)
    q = _bits(rng.standard_normal((n, 4, 64)))
    out, _ = c.attend_multi([0], [n], q)
    for r in (0, 10, 47):
        p = L - n + r
        k2, v2 = k.copy(), v.copy()
        k2[p + 1:], v2[p + 1:] = _kv(rng, L - p - 1, 2, 64)
        c2 = _cache(S=S, R=R, b=b)
        assert c2.append([0], [L], k2, v2) == oracle.OK
        out2, _ = c2.attend_multi([0], [n], q)
        assert np.array_equal(out2[:r + 1], out[:r + 1]), r
        k3 = k.copy()
        k3[p], _ = _kv(rng, 1, 2, 64)
        c3 = _cache(S=S, R=R, b=b)
        assert c3.append([0], [L], k3, v) == oracle.OK
        out3, _ = c3.attend_multi([0], [n], q)
        assert not np.array_equal(out3[r], out[r]), r
        assert np.array_equal(out3[:r], out[:r]), r


def test_reads_the_copy_of_length_L():
    """A position that is recent at length p+1 but not at L is read from its INT4 page copy, so row r
    differs from decode of the prefix cache, which reads the INT8 copy of those positions; the two
    caches' dequantized rows (decode's own copy choice, pinned by the decode tests) differ exactly
    in that window."""
    S, R, b, L, n = 4, 32, 64, 300, 100
    c, k, v, rng = _filled(S, R, b, L, seed=9)
    q = _bits(rng.standard_normal((n, 4, 64)))
    out, _ = c.attend_multi([0], [n], q)
    r = 20
    p = L - n + r
    c2 = _cache(S=S, R=R, b=b)
    assert c2.append([0], [p + 1], k[:p + 1], v[:p + 1]) == oracle.OK
    ref_prefix, _ = c2.decode([0], q[r:r + 1])
    assert not np.array_equal(out[r], ref_prefix[0])
    # the prefix cache's last R positions are INT8; at length L they are INT4 in `c`
    Kc, Vc = c.dequant_seq(0, 0)
    K2, V2 = c2.dequant_seq(0, 0)
    assert np.array_equal(Kc[:S], K2[:S])
    assert not np.array_equal(Kc[p + 1 - R:p + 1], K2[p + 1 - R:p + 1])
    assert np.array_equal(Kc[S:p + 1 - R], K2[S:p + 1 - R])


def test_multi_errors():
    c, k, v, rng = _filled(4, 32, 64, 20, seed=11)
    q = _bits(rng.standard_normal((21, 4, 64)))
    with pytest.raises(ValueError):
        c.attend_multi([0], [21], q)           # more rows than positions
    with pytest.raises(ValueError):
        c.attend_multi([0], [0], q[:0])        # a sequence with no rows
    with pytest.raises(ValueError):
        c.attend_multi([1], [1], q[:1])        # empty sequence
    out, _ = c.attend_multi([], [], q[:0])
    assert out.shape == (0, 4, 64)
