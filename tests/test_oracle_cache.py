"""Pins of the oracle's cache model (allocator, protection slots, append rule) and of its decode
attention against independent formulations (CPU only)."""
import numpy as np
import pytest
import scipy.linalg

import oracle


def _bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _kv(rng, n, hkv, d, outliers=()):
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    for c in outliers:
        k[:, :, c] *= 10
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    return _bits(k), _bits(v)


def _cache(hq=4, hkv=2, d=64, num_pages=256, max_seqs=8, max_pps=64, S=4, R=32, b=64, fmt=oracle.FMT_INT4_PROT):
    return oracle.OracleCache(hq, hkv, d, 16, num_pages, max_seqs, max_pps, S, R, b, fmt)


# ------------------------------------------------------------------------------------------------
# allocator and append rule
# ------------------------------------------------------------------------------------------------

def test_fifo_pages_round_robin_decode_steps():
    """256 sequences start empty and append one position per step in call order 0..255: block j of
    sequence i is page 256*j + i (the free list is 0, 1, 2, ... and pops from the front)."""
    c = _cache(hq=2, hkv=1, d=64, num_pages=256 * 3, max_seqs=256, max_pps=4, S=4, R=32, b=64)
    ids = list(range(256))
    for _ in range(40):
        assert c.append(ids, [1] * 256, None, None) == oracle.OK
    for i in (0, 1, 77, 255):
        assert c.block_table(i).tolist() == [256 * j + i for j in range(3)]


def test_fifo_prefill_and_free_order():
    c = _cache(num_pages=20, max_pps=20)
    assert c.append([3], [100], None, None) == oracle.OK  # 7 pages: 0..6
    assert c.block_table(3).tolist() == list(range(7))
    assert c.append([1], [17], None, None) == oracle.OK   # pages 7, 8
    assert c.seq_free(3) == oracle.OK                      # 0..6 go to the back
    assert c.free_pages() == 18
    assert c.append([2], [16 * 13], None, None) == oracle.OK  # 9..19 then 0, 1
    assert c.block_table(2).tolist() == list(range(9, 20)) + [0, 1]


def test_out_of_pages_is_all_or_nothing():
    rng = np.random.default_rng(0)
    c = _cache(num_pages=5, max_pps=8)
    k, v = _kv(rng, 40, 2, 64)
    assert c.append([0], [40], k, v) == oracle.OK  # 3 pages
    before = (c.free_pages(), c.seq_length(0), c.block_table(0).tolist())
    k2, v2 = _kv(rng, 9 + 33, 2, 64)
    # seq 0 needs 1 more page (40 -> 49), seq 1 needs 3: 4 > 2 free
    assert c.append([0, 1], [9, 33], k2, v2) == oracle.OUT_OF_PAGES
    assert (c.free_pages(), c.seq_length(0), c.block_table(0).tolist()) == before
    assert c.seq_length(1) == 0


def test_append_argument_errors():
    c = _cache()
    assert c.append([0, 0], [1, 1], None, None) == oracle.INVALID_ARGUMENT
    assert c.append([0], [-1], None, None) == oracle.INVALID_ARGUMENT
    assert c.append([99], [1], None, None) == oracle.INVALID_ARGUMENT
    assert c.append([0], [64 * 16 + 1], None, None) == oracle.SEQ_STATE


@pytest.mark.parametrize("S,R,b", [(4, 32, 64), (4, 128, 64), (0, 0, 1), (2, 5, 16)])
def test_prefill_equals_incremental(S, R, b):
    rng = np.random.default_rng(S + R + b)
    n = 300
    k, v = _kv(rng, n, 2, 64, outliers=(3, 40))
    A = _cache(S=S, R=R, b=b)
    B = _cache(S=S, R=R, b=b)
    assert A.append([0], [n], k, v) == oracle.OK
    for t in range(n):
        assert B.append([0], [1], k[t:t + 1], v[t:t + 1]) == oracle.OK
    assert A.block_table(0).tolist() == B.block_table(0).tolist()
    for t in range(n):
        for h in range(2):
            for kv in range(2):
                ca, sa, _ = A.page_token(0, t, h, kv)
                cb_, sb, _ = B.page_token(0, t, h, kv)
                assert np.array_equal(ca, cb_) and sa == sb
    for u in range(S + R):
        for h in range(2):
            for kv in range(2):
                ca, sa, ta = A.int8_slot_contents(0, u, h, kv)
                cb_, sb, tb = B.int8_slot_contents(0, u, h, kv)
                if ta >= 0 and oracle.is_protected(ta, n, S, R):
                    assert ta == tb and np.array_equal(ca, cb_) and sa == sb
    q = _bits(rng.standard_normal((1, 4, 64)))
    oa, _ = A.decode([0], q)
    ob, _ = B.decode([0], q)
    assert np.array_equal(oa, ob)


def test_ring_after_512_steps():
    """Single-position appends for 512 steps with S=4, R=128: the sinks hold 0..3 and the ring holds
    384..511, each token t >= 4 in ring slot 4 + t mod 128."""
    c = _cache(hq=2, hkv=1, d=64, num_pages=64, max_seqs=1, max_pps=40, S=4, R=128, b=64)
    rng = np.random.default_rng(5)
    k, v = _kv(rng, 512, 1, 64)
    for t in range(512):
        assert c.append([0], [1], k[t:t + 1], v[t:t + 1]) == oracle.OK
    held = sorted(c.int8_slot_contents(0, u, 0, 0)[2] for u in range(132))
    assert held == list(range(4)) + list(range(384, 512))
    for t in range(384, 512):
        assert c.int8_slot_contents(0, 4 + t % 128, 0, 1)[2] == t


def test_int8_copy_is_the_rotated_row_at_8_bits():
    rng = np.random.default_rng(9)
    k, v = _kv(rng, 50, 2, 64, outliers=(5,))
    c = _cache(S=4, R=32, b=64)
    assert c.append([0], [50], k, v) == oracle.OK
    for t in (0, 3, 18, 49):
        u = oracle.int8_slot(t, 4, 32)
        y = oracle.rotate_bf16(v[t, 1], 64)
        codes, s, z = oracle.quantize(y, 255)
        gc, (gs, gz), tok = c.int8_slot_contents(0, u, 1, 1)
        assert tok == t and np.array_equal(gc, codes) and (gs, gz) == (s, z)
        y4 = oracle.rotate_bf16(k[t, 0], 64)
        codes4, s4, z4 = oracle.quantize(y4, 15)
        pc, (ps, pz), _ = c.page_token(0, t, 0, 0)
        assert np.array_equal(pc, codes4) and (ps, pz) == (s4, z4)


# ------------------------------------------------------------------------------------------------
# decode attention
# ------------------------------------------------------------------------------------------------

def _softmax_attend(q, K, V, scale):
    e = scale * (K @ q)
    e = e - e.max()
    p = np.exp(e)
    return (p / p.sum()) @ V


@pytest.mark.parametrize("b", [1, 16, 64])
def test_all_protected_matches_unrotated_brute_force(b):
    """L <= S + R: every position is read from INT8.  Rebuild the keys and values in the unrotated
    domain from the INT8 slot contents (x^ H^T, H from scipy's Sylvester matrix) and attend with
    plain softmax: equals the oracle's rotated-domain decode."""
    S, R, d, hkv, hq = 4, 60, 64, 2, 4
    rng = np.random.default_rng(b)
    L = 50
    k, v = _kv(rng, L, hkv, d, outliers=(1, 2))
    c = _cache(hq=hq, hkv=hkv, d=d, S=S, R=R, b=b)
    assert c.append([0], [L], k, v) == oracle.OK
    qb = _bits(rng.standard_normal((1, hq, d)))
    out, _ = c.decode([0], qb)
    Hb = scipy.linalg.hadamard(b) / np.sqrt(b)
    Hbd = np.kron(np.eye(d // b), Hb)
    G = hq // hkv
    for g in range(hq):
        h = g // G
        K = np.zeros((L, d))
        V = np.zeros((L, d))
        for t in range(L):
            u = oracle.int8_slot(t, S, R)
            for kv, M in ((0, K), (1, V)):
                codes, (s, z), tok = c.int8_slot_contents(0, u, h, kv)
                assert tok == t
                M[t] = oracle.fp16_value(s) * codes + oracle.fp16_value(z)
        K = K @ Hbd.T
        V = V @ Hbd.T
        ref = _softmax_attend(_bf16_value(qb[0, g]), K, V, 1 / np.sqrt(d))
        assert np.abs(out[0, g] - ref).max() <= 1e-12


def test_plain_int4_textbook_attention():
    """b = 1, S = R = 0: token-wise INT4 attention with no rotation and no protection."""
    rng = np.random.default_rng(4)
    L, d, hkv, hq = 200, 64, 2, 4
    k, v = _kv(rng, L, hkv, d)
    c = _cache(hq=hq, hkv=hkv, d=d, S=0, R=0, b=1)
    assert c.append([1], [L], k, v) == oracle.OK
    qb = _bits(rng.standard_normal((1, hq, d)))
    out, _ = c.decode([1], qb, scale=0.3)
    for g in range(hq):
        h = g // 2
        K = np.zeros((L, d))
        V = np.zeros((L, d))
        for t in range(L):
            for kv, M in ((0, K), (1, V)):
                # quantize the raw row directly (rotation is the identity at b = 1)
                codes, s, z = oracle.quantize(_bf16_value((k if kv == 0 else v)[t, h]).astype(np.float32), 15)
                M[t] = oracle.fp16_value(s) * codes + oracle.fp16_value(z)
        ref = _softmax_attend(_bf16_value(qb[0, g]), K, V, 0.3)
        assert np.abs(out[0, g] - ref).max() <= 1e-12


def test_single_position_returns_its_value():
    rng = np.random.default_rng(8)
    k, v = _kv(rng, 1, 2, 64)
    c = _cache(S=4, R=32, b=64)
    assert c.append([0], [1], k, v) == oracle.OK
    qb = _bits(rng.standard_normal((1, 4, 64)))
    out, _ = c.decode([0], qb)
    Hb = scipy.linalg.hadamard(64) / 8.0
    for g in range(4):
        codes, (s, z), _ = c.int8_slot_contents(0, 0, g // 2, 1)
        vh = (oracle.fp16_value(s) * codes + oracle.fp16_value(z)) @ Hb.T
        assert np.abs(out[0, g] - vh).max() <= 1e-13


def test_split_merge_invariance():
    """Softmax attention split into chunks and merged by log-sum-exp equals the single pass."""
    rng = np.random.default_rng(12)
    L = 700
    k, v = _kv(rng, L, 2, 64, outliers=(0,))
    c = _cache(S=4, R=32, b=64)
    assert c.append([0], [L], k, v) == oracle.OK
    qb = _bits(rng.standard_normal((1, 4, 64)))
    out, _ = c.decode([0], qb)
    K, V = c.dequant_seq(0, 0)
    Hb = np.kron(np.eye(1), scipy.linalg.hadamard(64) / 8.0)
    q = _bf16_value(qb[0, 0]) @ Hb
    for n_chunks in (1, 3, 7, 50):
        M, Ls, O = -np.inf, 0.0, np.zeros(64)
        for idx in np.array_split(np.arange(L), n_chunks):
            e = (K[idx] @ q) / 8.0
            m = e.max()
            p = np.exp(e - m)
            Mn = max(M, m)
            Ls = Ls * np.exp(M - Mn) + p.sum() * np.exp(m - Mn)
            O = O * np.exp(M - Mn) + (p @ V[idx]) * np.exp(m - Mn)
            M = Mn
        assert np.abs((O / Ls) @ Hb.T - out[0, 0]).max() <= 1e-12


def test_decode_errors():
    c = _cache()
    qb = np.zeros((1, 4, 64), dtype=np.uint16)
    with pytest.raises(ValueError):
        c.decode([0], qb)  # length 0


def test_quality_rotation_and_protection_help():
    """Diagnostic pin of the pages' qualitative claims on outlier-channel keys: the rotated INT4
    cache errs less than plain INT4 against unquantized attention, and protecting sinks and recent
    positions in INT8 errs less again."""
    rng = np.random.default_rng(21)
    L, d, hkv, hq = 400, 128, 2, 8
    k = rng.standard_normal((L, hkv, d)).astype(np.float32)
    k[:, :, [3, 77, 90, 111]] *= 10
    v = rng.standard_normal((L, hkv, d)).astype(np.float32)
    kb, vb = _bits(k), _bits(v)
    q = _bits(rng.standard_normal((4, hq, d)))
    ref_c = oracle.OracleCache(hq, hkv, d, 16, 64, 4, 32, 0, 0, 1, oracle.FMT_BF16)
    assert ref_c.append([0], [L], kb, vb) == oracle.OK

    def err(S, R, b):
        c = oracle.OracleCache(hq, hkv, d, 16, 64, 4, 32, S, R, b)
        assert c.append([0], [L], kb, vb) == oracle.OK
        e = 0.0
        for i in range(4):
            o, _ = c.decode([0], q[i:i + 1])
            r, _ = ref_c.decode([0], q[i:i + 1])
            e += float(np.sqrt(((o - r) ** 2).mean()))
        return e

    plain = err(0, 0, 1)
    rotated = err(0, 0, 128)
    protected = err(4, 128, 128)
    print("rms error: plain INT4 %.4f, rotated %.4f, rotated+protected %.4f" % (plain, rotated, protected))
    assert rotated < plain
    assert protected < rotated
