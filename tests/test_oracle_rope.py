"""Pins of the oracle's fused RoPE append (CPU only): keys arrive before RoPE, the append applies
it (rotate-half pairs, the caller's cos / sin tables, binary32) and then the Hadamard rotation
("SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving": the transform
is applied to keys after RoPE)."""
import numpy as np
import pytest

import kv4_inputs as W
import oracle

from tests.test_oracle_cache import _bits, _kv

HQ, HKV, D = 4, 2, 64


def _cache(S=4, R=32, b=64):
    return oracle.OracleCache(HQ, HKV, D, 16, 256, 8, 64, S, R, b)


def _same_cache(a, b, seq, L):
    for j, page in enumerate(a.block_table(seq)):
        pb = b.block_table(seq)[j]
        for h in range(HKV):
            ca, sa, fa = a.page_contents(page, h)
            cb, sb, fb = b.page_contents(pb, h)
            n = min(16, L - 16 * j)
            if not (np.array_equal(ca[:n], cb[:n]) and np.array_equal(sa[:n], sb[:n])):
                return False
    for u in range(a.S + a.R):
        for h in range(HKV):
            for kv in range(2):
                x, sx, tx = a.int8_slot_contents(seq, u, h, kv)
                y, sy, ty = b.int8_slot_contents(seq, u, h, kv)
                if tx != ty or (tx >= 0 and not (np.array_equal(x, y) and sx == sy)):
                    return False
    return True


def test_identity_table_is_plain_append():
    rng = np.random.default_rng(2)
    L = 120
    k, v = _kv(rng, L, HKV, D, outliers=(5,))
    cos, sin = np.ones((L, D // 2), np.float32), np.zeros((L, D // 2), np.float32)
    a, b = _cache(), _cache()
    assert a.append_rope([0], [L], k, v, cos, sin) == oracle.OK
    assert b.append([0], [L], k, v) == oracle.OK
    assert _same_cache(a, b, 0, L)


def test_quarter_turn_swaps_halves():
    """cos = 0, sin = 1 maps (x_i, x_{i+D/2}) to (-x_{i+D/2}, x_i) exactly: the cache equals a plain
    append of that permuted row (a check of the pairing and of the signs)."""
    rng = np.random.default_rng(3)
    L = 70
    k, v = _kv(rng, L, HKV, D, outliers=(9,))
    cos, sin = np.zeros((L, D // 2), np.float32), np.ones((L, D // 2), np.float32)
    kq = np.concatenate([k[..., D // 2:] ^ np.uint16(0x8000), k[..., :D // 2]], axis=-1)
    a, b = _cache(), _cache()
    assert a.append_rope([0], [L], k, v, cos, sin) == oracle.OK
    assert b.append([0], [L], kq, v) == oracle.OK
    assert _same_cache(a, b, 0, L)


def test_rope_keeps_pair_norms_and_relative_positions():
    rng = np.random.default_rng(4)
    cos, sin = W.rope_tables(4096, D)
    x = _bits(rng.standard_normal(D))
    q = _bits(rng.standard_normal(D))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in (0, 1, 7, 1000, 4095):
        r = oracle.rope_bf16(x, cos[t], sin[t]).astype(np.float64)
        n_in = xf[:D // 2] ** 2 + xf[D // 2:] ** 2
        n_out = r[:D // 2] ** 2 + r[D // 2:] ** 2
        assert np.all(np.abs(n_out - n_in) <= 1e-6 * n_in + 1e-30)
    # <rope(q, p), rope(k, t)> depends on p - t only (up to the tables' binary32 rounding)
    dots = []
    for p0 in (10, 500, 3000):
        rq = oracle.rope_bf16(q, cos[p0 + 7], sin[p0 + 7]).astype(np.float64)
        rk = oracle.rope_bf16(x, cos[p0], sin[p0]).astype(np.float64)
        dots.append(rq @ rk)
    assert max(dots) - min(dots) <= 1e-4 * max(abs(d) for d in dots)
    assert position_zero_is_identity(x, cos, sin)


def position_zero_is_identity(x, cos, sin):
    r = oracle.rope_bf16(x, cos[0], sin[0])
    return np.array_equal(r, (x.astype(np.uint32) << 16).view(np.float32))


def test_rope_prefill_equals_incremental_and_checks_positions():
    rng = np.random.default_rng(6)
    L = 90
    k, v = _kv(rng, L, HKV, D, outliers=(2,))
    cos, sin = W.rope_tables(128, D)
    a, i = _cache(), _cache()
    assert a.append_rope([0], [L], k, v, cos, sin) == oracle.OK
    for t in range(L):
        assert i.append_rope([0], [1], k[t:t + 1], v[t:t + 1], cos, sin) == oracle.OK
    assert _same_cache(a, i, 0, L)
    c = _cache()
    assert c.append_rope([0], [129], *_kv(rng, 129, HKV, D), cos, sin) == oracle.INVALID_ARGUMENT
    assert c.seq_length(0) == 0
