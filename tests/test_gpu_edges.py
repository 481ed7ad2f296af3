"""GPU parity at the edges of the quantizer and the allocator, through the C ABI.

- fp16-subnormal scales and zero points: rows of magnitude 1e-4 .. 1e-9, so that s and z fall in
  (or below) the binary16 subnormal range, with and without the rotation, through both append
  kernels and both copies (INT4 page, INT8 slot);
- round half to even: rows built at b = 1 so that (y - z) * (1 / s) lands exactly on k + 0.5 for
  the INT4 and the INT8 quantizer, beside rows near +-60000;
- page and INT8-tile reuse: sequences freed, their pages handed out again in FIFO order and their
  sequence ids (and INT8 tiles, with stale contents) used again;
- a recent window of 1 or 2 positions with two positions of one sequence appended across a page
  boundary in one call (two single-position tasks of one sequence in one launch).

Codes, scales, page ids and protected INT8 slots compare bit for bit with the oracle; decode
outputs within max-abs 2e-3 of the fp64 oracle on the same dequantized cache.
"""
import numpy as np
import pytest
import torch

import kv4_inputs as W
import oracle
from tests.pair import Pair, TOL

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print("CASE", name, kw, flush=True)


def _bf16(x):
    """float array -> bf16 cuda tensor (round to nearest even); exact for bf16-representable values."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to("cuda").contiguous()


def _exact_bf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    assert torch.equal(t.to(torch.bfloat16).to(torch.float32), t), "value not representable in bf16"
    return t.to(torch.bfloat16).to("cuda").contiguous()


def _decode_check(p, ids, seed, tol=TOL):
    q = W.queries(len(ids), p.hq, p.d, seed, device="cuda")
    out, ref = p.decode(ids, q)
    err = np.abs(out - ref).max()
    print("  decode", ids, "max-abs", err, flush=True)
    assert np.isfinite(out).all()
    assert err <= tol
    return err


def _scale_bits(p, seqs):
    """All (s, z) fp16 patterns the oracle holds for the given sequences (INT4 pages and INT8 slots)."""
    bits = []
    for s in seqs:
        L = p.ora.seq_length(s)
        for t in range(L):
            for h in range(p.hkv):
                for kv in range(2):
                    _, sz, _ = p.ora.page_token(s, t, h, kv)
                    bits.extend(sz)
                    if p.S + p.R > 0 and oracle.is_protected(t, L, p.S, p.R):
                        _, sz8, tok = p.ora.int8_slot_contents(s, oracle.int8_slot(t, p.S, p.R), h, kv)
                        assert tok == t
                        bits.extend(sz8)
    return np.array(bits, dtype=np.uint16)


@pytest.mark.parametrize("b", [1, 128])
def test_subnormal_scales(b):
    _print_case("subnormal scales", b=b)
    hq, hkv, d = 8, 2, 128
    rng = np.random.default_rng(101 + b)
    mags = [1e-4, 3e-5, 1e-6, 1e-7, 1e-8, 1e-9]
    rows_k, rows_v = [], []
    for m in mags:
        for _ in range(6):
            rows_k.append(rng.standard_normal((hkv, d)) * m)
            rows_v.append(rng.standard_normal((hkv, d)) * m * rng.uniform(0.5, 2.0))
    # constant and one-sided rows in the same range: z subnormal with s = 0, z = 0 with s subnormal
    rows_k.append(np.full((hkv, d), 3e-7))
    rows_v.append(np.abs(rng.standard_normal((hkv, d))) * 1e-6)
    n = len(rows_k)
    k, v = _bf16(np.stack(rows_k)), _bf16(np.stack(rows_v))
    p = Pair(hq, hkv, d, num_pages=64, max_seqs=4, max_pps=16, S=4, R=16, b=b)
    p.append([0], [n], k, v)                        # page kernel
    for t in range(n):                              # per-position kernel
        p.append([1], [1], k[t:t + 1].contiguous(), v[t:t + 1].contiguous())
    assert p.compare_cache([0, 1]) > 0
    bits = _scale_bits(p, [0, 1])
    mag = bits & 0x7FFF
    n_sub = int(((mag != 0) & (mag < 0x0400)).sum())
    print("  subnormal s/z patterns", n_sub, "of", bits.size, flush=True)
    assert n_sub > bits.size // 4
    _decode_check(p, [0, 1], 103)


def test_round_half_even_ties():
    """Exact ties of the INT4 quantizer (z = 0, s = 1 over [0, 15]) and of the INT8 one (z = 0, s = 1
    over [0, 255]), also scaled by powers of two and shifted, beside rows near +-60000.  Every
    position is protected, so each row has both its INT4 and its INT8 codes compared."""
    _print_case("round-half-even ties")
    hq, hkv, d = 8, 2, 64
    rng = np.random.default_rng(7)

    def tie_row4(scale, shift):
        r = rng.integers(0, 16, d).astype(np.float64)
        r[:2] = [0, 15]
        r[2:2 + 16] = np.arange(16) + 0.5         # 0.5 .. 15.5: ties (15.5 clamps to 15)
        r[2:2 + 16] = np.minimum(r[2:2 + 16], 14.5)
        return (rng.permutation(r) * scale + shift)

    def tie_row8(scale):
        r = rng.integers(0, 256, d).astype(np.float64)
        r[:2] = [0, 255]
        r[2:40] = rng.choice(128, 38, replace=False) + 0.5  # x.5 with x < 128 (bf16-exact)
        return rng.permutation(r) * scale

    k_rows, v_rows = [], []
    for scale, shift in ((1, 0), (0.25, 0), (16, 0), (256, 0), (1, -8), (0.5, -4)):
        k_rows.append(np.stack([tie_row4(scale, shift) for _ in range(hkv)]))
        v_rows.append(np.stack([tie_row8(scale) for _ in range(hkv)]))
    for scale in (1, 0.5, 8):
        k_rows.append(np.stack([tie_row8(scale) for _ in range(hkv)]))
        v_rows.append(np.stack([tie_row4(scale, 0) for _ in range(hkv)]))
    # rows near +-60000 (keys; values stay moderate so that outputs keep the absolute tolerance)
    for _ in range(4):
        kb = rng.uniform(-60000, 60000, (hkv, d))
        kb[:, 0], kb[:, 1] = -60000, 60000
        k_rows.append(kb)
        v_rows.append(np.stack([tie_row4(1, 0) for _ in range(hkv)]))
    kt = _bf16(np.stack(k_rows))
    vt = _bf16(np.stack(v_rows))
    n = kt.shape[0]
    # the tie rows are exact bf16 values
    _exact_bf16(np.stack(k_rows[:9]))
    _exact_bf16(np.stack(v_rows))
    p = Pair(hq, hkv, d, num_pages=32, max_seqs=4, max_pps=8, S=4, R=64, b=1)
    p.append([0], [n], kt, vt)
    for t in range(n):
        p.append([1], [1], kt[t:t + 1].contiguous(), vt[t:t + 1].contiguous())
    # the oracle's scales are the intended ones (z = 0 or the shift, s = the power of two)
    _, sz, _ = p.ora.page_token(0, 0, 0, 0)
    assert sz == (oracle.fp16_round_up(1.0), 0)
    _, sz8, _ = p.ora.int8_slot_contents(0, 0, 0, 1)
    assert sz8 == (oracle.fp16_round_up(1.0), 0)
    assert p.compare_cache([0, 1]) > 0
    # the key rows near +-60000 make the softmax one-hot; values are small integers or halves
    _decode_check(p, [0, 1], 9)


def test_seq_free_page_and_tile_reuse():
    """Freed pages return to the back of the free list and are handed out again; a freed sequence
    id is used again with its INT8 tiles still holding the old sequence's bytes."""
    _print_case("seq_free reuse")
    hq, hkv, d = 32, 8, 128
    S, R = 4, 32
    p = Pair(hq, hkv, d, num_pages=50, max_seqs=6, max_pps=50, S=S, R=R, b=128)

    def kv(n, idx):
        ch = W.outlier_channels(hkv, d, 4, 61)
        return W.seq_kv(hkv, d, n, ch, 10.0, 61, 0, idx, "cuda")

    lens = [300, 300, 133]            # 19 + 19 + 9 = 47 of 50 pages
    ks, vs = zip(*[kv(L, i) for i, L in enumerate(lens)])
    p.append([0, 1, 2], lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    _decode_check(p, [0, 1, 2], 63)
    p.seq_free(1)
    p.seq_free(0)
    assert p.gpu.free_pages() == p.ora.free_pages() == 41
    # sequence 3 takes the 3 never-used pages, then freed ones (sequence 1's, in its block order)
    k3, v3 = kv(100, 3)
    p.append([3], [100], k3, v3)
    assert p.gpu.block_table(3)[:3] == [47, 48, 49]
    # sequence 1 again (its INT8 tiles hold the old ring), shorter; sequence 0 by single appends
    k1, v1 = kv(20, 11)
    p.append([1], [20], k1, v1)
    for step in range(40):
        kn, vn = kv(2, 100 + step)
        p.append([0, 1], [1, 1], kn, vn)   # argument-plan path of the per-position kernel
    assert p.compare_cache([0, 1, 2, 3]) > 0
    _decode_check(p, [3, 1, 0, 2], 65)
    # free everything and fill the pool again from the recycled list
    for s in (0, 1, 2, 3):
        p.seq_free(s)
    assert p.gpu.free_pages() == 50
    k4, v4 = kv(50 * 16, 4)
    p.append([4], [50 * 16], k4, v4)
    assert p.gpu.free_pages() == 0 and p.gpu.block_table(4) == list(p.ora.block_table(4))
    assert p.compare_cache([4]) > 0
    _decode_check(p, [4], 67)


@pytest.mark.parametrize("S,R", [(0, 1), (4, 1), (0, 2), (4, 2)])
def test_tiny_recent_window_across_page_boundary(S, R):
    """Two positions of one sequence across a page boundary in one call (two single-position tasks of
    that sequence in one launch), with a recent window of 1 or 2: the tasks must see the length after
    the call, or the older position takes the newest one's ring slot."""
    _print_case("tiny recent window", S=S, R=R)
    hq, hkv, d = 32, 8, 128
    p = Pair(hq, hkv, d, num_pages=64, max_seqs=8, max_pps=12, S=S, R=R, b=128)
    ch = W.outlier_channels(hkv, d, 4, 71)

    def kv(n, idx):
        return W.seq_kv(hkv, d, n, ch, 10.0, 71, 0, idx, "cuda")

    lens = [15, 31, 20, 47, 1]
    ks, vs = zip(*[kv(L, i) for i, L in enumerate(lens)])
    p.append(list(range(5)), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    for step, n_new in enumerate(([2, 2, 1, 2, 1], [1, 1, 1, 1, 1], [1, 2, 2, 1, 2], [2, 0, 1, 2, 1])):
        kn, vn = kv(sum(n_new), 50 + step)
        p.append(list(range(5)), n_new, kn, vn)
        assert p.compare_cache(range(5)) > 0
        _decode_check(p, list(range(5)), 73 + step)
