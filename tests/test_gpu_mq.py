"""GPU parity of multi-query (causal) attention over the cache, through the C ABI, against the CPU
oracle: max-abs <= 2e-3 on every output (fp32 outputs against the fp64 oracle on the same
dequantized cache).  The n_q query rows of a sequence sit at its last n_q positions; row r attends
positions 0 .. L - n_q + r, each from the copy decode reads at length L."""
import numpy as np
import pytest
import torch

import int4_kv_cache_fwht_amd as kv4
import kv4_inputs as W
from tests.pair import Pair, TOL

pytestmark = pytest.mark.gpu


def _kv(n, hkv, d, seed, layer=0, idx=0, outliers=4, scale=10.0):
    ch = W.outlier_channels(hkv, d, outliers, seed, layer)
    return W.seq_kv(hkv, d, n, ch, scale, seed, layer, idx, device="cuda")


def _q(rows, hq, d, seed, step=0):
    return W.queries(rows, hq, d, seed, step=step, device="cuda")


def _print_case(name, **kw):
    print("CASE", name, kw, flush=True)


def _fill(p, lens, hkv, d, seed):
    ks, vs = zip(*[_kv(L, hkv, d, seed=seed, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())


@pytest.mark.parametrize("fmt,b,S,R", [
    (kv4.FORMAT_INT4_PROT, 128, 4, 128),
    (kv4.FORMAT_INT4_PROT, 1, 0, 0),
    (kv4.FORMAT_INT4_PROT, 32, 4, 32),
    (kv4.FORMAT_INT4_PROT, 128, 4, 0),
    (kv4.FORMAT_INT4_PROT, 128, 0, 128),
    (kv4.FORMAT_INT8, 128, 0, 0),
])
def test_mq_ragged(fmt, b, S, R):
    _print_case("mq_ragged", fmt=fmt, b=b, S=S, R=R)
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 100, 132, 133, 300, 1000]
    nqs = [1, 5, 16, 40, 133, 64, 100]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=128, S=S, R=R, b=b, fmt=fmt)
    _fill(p, lens, hkv, d, seed=3)
    q = _q(sum(nqs), hq, d, seed=4)
    # sequences out of id order, to exercise the row layout
    order = [4, 0, 6, 2, 1, 5, 3]
    out, ref = p.multi(order, [nqs[i] for i in order], _reorder(q, nqs, order))
    err = np.abs(out - ref).max()
    print("mq ragged max-abs", err)
    assert err <= TOL


def _reorder(q, nqs, order):
    starts = np.cumsum([0] + nqs)
    return torch.cat([q[starts[i]:starts[i + 1]] for i in order]).contiguous()


@pytest.mark.parametrize("hq,hkv,d", [(16, 8, 128), (8, 2, 64), (4, 4, 64), (8, 8, 128)])
def test_mq_group_and_dims(hq, hkv, d):
    _print_case("mq_group_dims", hq=hq, hkv=hkv, d=d)
    lens = [7, 140, 611]
    nqs = [7, 33, 90]
    p = Pair(hq, hkv, d, num_pages=512, max_seqs=4, max_pps=64, S=4, R=32, b=min(d, 64))
    _fill(p, lens, hkv, d, seed=8)
    out, ref = p.multi([0, 1, 2], nqs, _q(sum(nqs), hq, d, seed=9))
    err = np.abs(out - ref).max()
    print("mq group/dims max-abs", err)
    assert err <= TOL


def test_mq_one_row_matches_decode():
    """n_q = 1 is decode attention: both GPU paths agree with the oracle and with each other."""
    _print_case("mq_one_row")
    hq, hkv, d = 32, 8, 128
    lens = [1, 40, 133, 500, 2000]
    p = Pair(hq, hkv, d, num_pages=1024, max_seqs=8, max_pps=160, S=4, R=128, b=128)
    _fill(p, lens, hkv, d, seed=12)
    q = _q(len(lens), hq, d, seed=13)
    ids = list(range(len(lens)))
    out, ref = p.multi(ids, [1] * len(lens), q)
    dec, ref2 = p.decode(ids, q)
    assert np.array_equal(ref, ref2)
    assert np.abs(out - ref).max() <= TOL
    assert np.abs(out - dec).max() <= 2 * TOL


def test_mq_chunked_prefill():
    """A prefill chunk: 1000 cached positions, then a chunk of 300 is appended and its 300 rows
    attend causally over the cache (positions beyond the recent window come from INT4)."""
    _print_case("mq_chunk")
    hq, hkv, d = 32, 8, 128
    p = Pair(hq, hkv, d, num_pages=256, max_seqs=2, max_pps=128, S=4, R=128, b=128)
    k, v = _kv(1300, hkv, d, seed=21)
    p.append([1], [1000], k[:1000].contiguous(), v[:1000].contiguous())
    p.append([1], [300], k[1000:].contiguous(), v[1000:].contiguous())
    out, ref = p.multi([1], [300], _q(300, hq, d, seed=22))
    err = np.abs(out - ref).max()
    print("mq chunk max-abs", err)
    assert err <= TOL


@pytest.mark.parametrize("seed", [101, 102, 103])
def test_mq_shared_steps_random(seed):
    """Seeded random calls for the workgroup-shared kernel: 5 sequences of random lengths, each with
    16, 32, 48 or 64 query rows (G 4: 4 to 16 row tiles, a multiple of 4), in a random order."""
    rng = np.random.default_rng(seed)
    nqs = [int(x) for x in rng.choice([16, 32, 48, 64], size=5)]
    lens = [int(rng.integers(nq, 3000)) for nq in nqs]
    _print_case("mq_shared_random", seed=seed, lens=lens, nqs=nqs)
    hq, hkv, d = 32, 8, 128
    p = Pair(hq, hkv, d, num_pages=1024, max_seqs=8, max_pps=200, S=4, R=128, b=128)
    _fill(p, lens, hkv, d, seed=seed)
    q = _q(sum(nqs), hq, d, seed=seed + 1)
    order = [int(i) for i in rng.permutation(5)]
    qo = _reorder(q, nqs, order)
    ids, nq = order, [nqs[i] for i in order]
    p.gpu.set_mq_share(False)
    own = p.gpu.multi_query_attention(ids, nq, qo).cpu().numpy()
    p.gpu.set_mq_share(True)
    out, ref = p.multi(ids, nq, qo)
    assert np.array_equal(out.astype(np.float32), own), "shared and per-wave steps differ"
    err = np.abs(out - ref).max()
    print("mq shared random max-abs", err)
    assert err <= TOL


def test_mq_chunked_prefill_shared():
    """A 256-position prefill chunk after 1000 cached positions: 64 row tiles per kv head, so the
    workgroup-shared kernel runs; the same bits as the per-wave kernel, and the oracle's values."""
    _print_case("mq_chunk_shared")
    hq, hkv, d = 32, 8, 128
    p = Pair(hq, hkv, d, num_pages=256, max_seqs=2, max_pps=128, S=4, R=128, b=128)
    k, v = _kv(1256, hkv, d, seed=51)
    p.append([1], [1000], k[:1000].contiguous(), v[:1000].contiguous())
    p.append([1], [256], k[1000:].contiguous(), v[1000:].contiguous())
    q = _q(256, hq, d, seed=52)
    p.gpu.set_mq_share(False)
    own = p.gpu.multi_query_attention([1], [256], q).cpu().numpy()
    p.gpu.set_mq_share(True)
    out, ref = p.multi([1], [256], q)
    assert np.array_equal(out.astype(np.float32), own), "shared and per-wave steps differ"
    err = np.abs(out - ref).max()
    print("mq chunk (shared) max-abs", err)
    assert err <= TOL


def test_mq_full_size_sampled():
    """Qwen3-8B-shaped layer (64 sequences, lengths uniform in [1024, 8192]) with 4 query rows per
    sequence in one call; the oracle checks a sample of the sequences."""
    _print_case("mq_full_size")
    w = W.WORKLOADS["qwen3_8b_layer"]
    lens = w.lengths()
    nq = 4
    p = Pair(w.num_q_heads, w.num_kv_heads, w.head_dim, num_pages=sum(-(-L // 16) for L in lens) + 8,
             max_seqs=w.batch, max_pps=max(-(-L // 16) for L in lens) + 1, S=w.num_sinks, R=w.num_recent,
             b=w.hadamard_block)
    ch = W.outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
    for i, L in enumerate(lens):
        k, v = W.seq_kv(w.num_kv_heads, w.head_dim, L, ch, w.outlier_scale, w.seed, 0, i, device="cuda")
        p.append([i], [L], k, v)
    ids = list(range(w.batch))
    q = _q(nq * w.batch, w.num_q_heads, w.head_dim, seed=31)
    out = p.gpu.multi_query_attention(ids, [nq] * w.batch, q).cpu().numpy().astype(np.float64)
    for i in (0, 17, 63):
        ref, _ = p.ora.attend_multi([i], [nq], W.bf16_bits(q[nq * i:nq * (i + 1)]))
        err = np.abs(out[nq * i:nq * (i + 1)] - ref).max()
        print("mq full size seq", i, "max-abs", err)
        assert err <= TOL


@pytest.mark.parametrize("hq,hkv,d,b,S,R,unit", [
    (32, 8, 128, 128, 4, 128, 16),   # G 4: a row tile is 4 query positions, 4 tiles per 16 rows
    (32, 8, 128, 1, 0, 0, 16),
    (32, 8, 128, 32, 4, 32, 16),
    (16, 8, 128, 128, 4, 128, 32),   # G 2
    (8, 8, 128, 64, 0, 16, 64),      # G 1
    (8, 2, 64, 64, 4, 32, 16),       # D 64: one copy per wave and step
])
def test_mq_shared_steps(hq, hkv, d, b, S, R, unit):
    """Every sequence with a multiple of 4 row tiles: the four waves of a workgroup share each INT4
    step's staged pages and spread operands.  The output equals the unshared kernel's bit for bit
    and the oracle within the tolerance, over ragged lengths and several chunks per sequence."""
    _print_case("mq_shared", hq=hq, hkv=hkv, d=d, b=b, S=S, R=R)
    lens = [unit + 1, 100, 257, 300, 1000, 2500]
    nqs = [unit, unit * (100 // unit), unit * 2, unit, unit * 4, unit * 3]
    p = Pair(hq, hkv, d, num_pages=1024, max_seqs=8, max_pps=192, S=S, R=R, b=b)
    _fill(p, lens, hkv, d, seed=41)
    q = _q(sum(nqs), hq, d, seed=42)
    order = [3, 0, 5, 1, 4, 2]
    qo = _reorder(q, nqs, order)
    ids, nq = order, [nqs[i] for i in order]
    p.gpu.set_mq_share(False)
    own = p.gpu.multi_query_attention(ids, nq, qo).cpu().numpy()
    p.gpu.set_mq_share(True)
    out, ref = p.multi(ids, nq, qo)
    assert np.array_equal(out.astype(np.float32), own), "shared and per-wave steps differ"
    err = np.abs(out - ref).max()
    print("mq shared max-abs", err)
    assert err <= TOL


def test_mq_errors():
    _print_case("mq_errors")
    p = Pair(8, 2, 64, num_pages=64, max_seqs=4, max_pps=16, S=4, R=16, b=64)
    _fill(p, [10, 20], 2, 64, seed=1)
    q = _q(11, 8, 64, seed=2)
    with pytest.raises(kv4.KV4Error) as e:
        p.gpu.multi_query_attention([0], [11], q)
    assert e.value.name == "KV4_ERR_SEQ_STATE"
    with pytest.raises(kv4.KV4Error) as e:
        p.gpu.multi_query_attention([0], [0], q[:0].contiguous())
    assert e.value.name == "KV4_ERR_INVALID_ARGUMENT"
    with pytest.raises(kv4.KV4Error) as e:
        p.gpu.multi_query_attention([2], [1], q[:1].contiguous())
    assert e.value.name == "KV4_ERR_SEQ_STATE"
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(kv4.KV4Error) as e:
        p.gpu.multi_query_attention([0], [3], q[:3].contiguous(), workspace=ws)
    assert e.value.name == "KV4_ERR_WORKSPACE_TOO_SMALL"
    assert p.gpu.multi_query_attention([], [], q[:0].contiguous()).numel() == 0
    cfg = kv4.Config(num_q_heads=8, num_kv_heads=2, head_dim=64, num_pages=8, max_seqs=2, max_pages_per_seq=4,
                     num_sinks=0, num_recent=0, hadamard_block=1, format=kv4.FORMAT_BF16)
    c = kv4.Cache(cfg, "cuda")
    k, v = _kv(5, 2, 64, seed=3)
    c.append([0], [5], k, v)
    with pytest.raises(kv4.KV4Error) as e:
        c.multi_query_attention([0], [1], q[:1].contiguous())
    assert e.value.name == "KV4_ERR_UNSUPPORTED"
    # nothing above changed the state: the cache still decodes as before
    out, ref = p.multi([0, 1], [10, 20], _q(30, 8, 64, seed=4))
    assert np.abs(out - ref).max() <= TOL


def test_mq_wide_merge_long_entry():
    """Many row tiles, so that the merge takes 4 rows per wave, with one long sequence among short
    ones: the chunk size is set for the whole call, so the long sequence's rows merge over more than
    64 chunks (the merge's general path, in rounds of 64 chunks)."""
    _print_case("mq_wide_merge")
    hq, hkv, d = 32, 8, 128
    lens = [300] * 299 + [60000]
    nqs = [4] * 300
    p = Pair(hq, hkv, d, num_pages=9600, max_seqs=300, max_pps=3800, S=4, R=128, b=128)
    _fill(p, lens, hkv, d, seed=31)
    q = _q(sum(nqs), hq, d, seed=33)
    out, ref = p.multi(list(range(len(lens))), nqs, q)
    err = np.abs(out - ref).max()
    print("mq wide merge max-abs", err, flush=True)
    assert err <= TOL
