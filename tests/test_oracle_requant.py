"""Pins of the oracle's second eviction rule (CPU only): INT4 codes re-quantized from the INT8 copy
instead of the dual write ("KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV
Cache Quantization", Abstract: tokens leaving the recent window move from INT8 to INT4).

Each pin ties the INT4 page of a position to something its own code path does not produce: the
position's INT8 slot (a different store), the quantizer's invariants, a cache built another way,
or the dual-write cache."""
import numpy as np
import pytest

import oracle

from tests.test_oracle_cache import _bits, _kv

HQ, HKV, D = 4, 2, 64


def _cache(S=4, R=32, b=64, eviction=1, fmt=oracle.FMT_INT4_PROT, num_pages=256):
    return oracle.OracleCache(HQ, HKV, D, 16, num_pages, 8, 64, S, R, b, fmt, eviction=eviction)


def _f16(bits):
    return np.float32(oracle.fp16_value(int(bits)))


def _round_trip8(codes, s_bits, z_bits):
    s, z = _f16(s_bits), _f16(z_bits)
    return (s * codes.astype(np.float32)).astype(np.float32) + z


def test_int4_page_quantizes_the_int8_slot():
    """For every protected position, the INT4 page row is a valid INT4 quantization (Q = 15) of the
    INT8 slot's dequantized row: z4 <= min, max <= z4 + 15 s4, |s4 c4 + z4 - x8| <= s4 / 2."""
    rng = np.random.default_rng(1)
    S, R, L = 4, 32, 200
    c = _cache(S=S, R=R)
    k, v = _kv(rng, L, HKV, D, outliers=(3, 40))
    assert c.append([0], [L], k, v) == oracle.OK
    checked = 0
    for t in list(range(S)) + list(range(L - R, L)):
        u = oracle.int8_slot(t, S, R)
        for h in range(HKV):
            for kv in range(2):
                c8, (s8, z8), tok = c.int8_slot_contents(0, u, h, kv)
                assert tok == t
                x8 = _round_trip8(np.asarray(c8), s8, z8).astype(np.float64)
                codes, (s4b, z4b), _ = _page_row(c, 0, t, h, kv)
                s4, z4 = float(_f16(s4b)), float(_f16(z4b))
                assert z4 <= x8.min()
                assert x8.max() <= z4 + 15 * s4 * (1 + 2 ** -22)
                x4 = s4 * codes + z4
                assert np.all(np.abs(x4 - x8) <= s4 / 2 * (1 + 2 ** -20))
                checked += 1
    assert checked == (S + R) * HKV * 2


def _page_row(c, seq, t, h, kv):
    page = c.block_table(seq)[t // 16]
    codes, sz, filled = c.page_contents(page, h)
    assert filled[t % 16]
    return np.asarray(codes[t % 16, kv], dtype=np.float64), (int(sz[t % 16, kv, 0]), int(sz[t % 16, kv, 1])), page


@pytest.mark.parametrize("S,R,b", [(4, 32, 64), (0, 16, 1), (2, 5, 16), (4, 0, 64)])
def test_requant_prefill_equals_incremental(S, R, b):
    rng = np.random.default_rng(S + R + b)
    L = 150
    k, v = _kv(rng, L, HKV, D, outliers=(7,))
    a, i = _cache(S=S, R=R, b=b), _cache(S=S, R=R, b=b)
    assert a.append([0], [L], k, v) == oracle.OK
    for t in range(L):
        assert i.append([0], [1], k[t:t + 1], v[t:t + 1]) == oracle.OK
    for t in range(L):
        for h in range(HKV):
            for kv in range(2):
                ca, sa, _ = _page_row(a, 0, t, h, kv)
                ci, si, _ = _page_row(i, 0, t, h, kv)
                assert np.array_equal(ca, ci) and sa == si, (t, h, kv)


def test_requant_changes_int4_only():
    """Against the dual-write cache on the same input: every INT8 slot is identical, INT4 pages
    differ for some positions, and with every position protected decode is identical."""
    rng = np.random.default_rng(5)
    S, R = 4, 32
    k, v = _kv(rng, 300, HKV, D, outliers=(3,))
    rq, dw = _cache(S=S, R=R), _cache(S=S, R=R, eviction=0)
    for cc in (rq, dw):
        assert cc.append([0], [300], k, v) == oracle.OK
        assert cc.append([1], [30], k[:30], v[:30]) == oracle.OK   # L = 30 <= S + R
    for u in range(S + R):
        for h in range(HKV):
            for kv in range(2):
                a, sa, ta = rq.int8_slot_contents(0, u, h, kv)
                b, sb, tb = dw.int8_slot_contents(0, u, h, kv)
                assert ta == tb and np.array_equal(a, b) and sa == sb
    # some rows change (the INT4 grid of a full-range INT8 row nests in the INT8 grid, s4 = 17 s8,
    # so re-quantization moves a code only near an INT4 rounding boundary)
    differ = sum(not np.array_equal(_page_row(rq, 0, t, 0, 0)[0], _page_row(dw, 0, t, 0, 0)[0]) for t in range(300))
    assert differ >= 10
    q = _bits(rng.standard_normal((1, HQ, D)))
    o1, _ = rq.decode([1], q)
    o2, _ = dw.decode([1], q)
    assert np.array_equal(o1, o2)


def test_requant_error_bound():
    """Two roundings: |x4 - y| <= s4 / 2 + s8 / 2 for every element, with y the rotated input and s8
    the INT8 scale of the same row (the quantizer's own bounds, chained)."""
    rng = np.random.default_rng(9)
    L = 64
    k, v = _kv(rng, L, HKV, D, outliers=(1, 2))
    c = _cache(S=0, R=0)
    assert c.append([0], [L], k, v) == oracle.OK
    for t in range(L):
        for h in range(HKV):
            y = oracle.rotate_bf16(k[t, h], 64).astype(np.float64)
            _, s8b, _ = oracle.quantize(oracle.rotate_bf16(k[t, h], 64), 255)
            codes, (s4b, z4b), _ = _page_row(c, 0, t, h, 0)
            s4, z4, s8 = float(_f16(s4b)), float(_f16(z4b)), float(_f16(s8b))
            err = np.abs(s4 * codes + z4 - y)
            assert np.all(err <= (s4 / 2 + s8 / 2) * (1 + 2 ** -19)), t


def test_eviction_rule_checks():
    with pytest.raises(ValueError):
        _cache(eviction=1, fmt=oracle.FMT_INT8)
    with pytest.raises(ValueError):
        _cache(eviction=2)
    c = _cache(eviction=0)
    assert c.append([0], [3], None, None) == oracle.OK
    assert oracle.lib().kv4o_set_eviction(c._h, 1) == oracle.SEQ_STATE
