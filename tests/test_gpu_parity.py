"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Codes, scales, page ids: bit-exact.  Decode outputs: max-abs <= 2e-3 against the fp64 oracle
evaluated on the same dequantized cache.  Inputs come from kv4_inputs (seeded).
"""
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


def _print_case(name, **kw):
    print("CASE", name, kw, flush=True)


def test_tiny_prefill_and_incremental():
    _print_case("tiny")
    w = W.WORKLOADS["tiny"]
    k, v, q = W.tiny_inputs(device="cuda")
    p = Pair(w.num_q_heads, w.num_kv_heads, w.head_dim, num_pages=64, max_seqs=4, max_pps=32, S=w.num_sinks,
             R=w.num_recent, b=w.hadamard_block)
    p.append([0], [300], k, v)
    for t in range(300):
        p.append([1], [1], k[t:t + 1].contiguous(), v[t:t + 1].contiguous())
    assert p.compare_cache([0, 1]) > 0
    out, ref = p.decode([0, 1], torch.cat([q, q]).contiguous())
    err = np.abs(out - ref).max()
    print("tiny max-abs", err)
    assert err <= TOL
    # prefill and incremental caches decode identically
    assert np.array_equal(out[0], out[1])


@pytest.mark.parametrize("fmt,b,S,R", [
    (kv4.FORMAT_INT4_PROT, 128, 4, 128),
    (kv4.FORMAT_INT4_PROT, 1, 0, 0),
    (kv4.FORMAT_INT4_PROT, 32, 4, 32),
    (kv4.FORMAT_INT4_PROT, 128, 4, 0),    # sinks only
    (kv4.FORMAT_INT4_PROT, 128, 0, 128),  # recent window only
    (kv4.FORMAT_INT4_PROT, 1, 4, 128),    # protection without rotation
    (kv4.FORMAT_INT4_PROT, 64, 4, 16),    # half block: the lane-pair stage, not the last one
    (kv4.FORMAT_INT8, 128, 0, 0),
    (kv4.FORMAT_INT8, 16, 0, 0),          # partial block of the INT8 format
    (kv4.FORMAT_BF16, 1, 0, 0),
])
def test_ragged_batch(fmt, b, S, R):
    _print_case("ragged", fmt=fmt, b=b, S=S, R=R)
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 100, 132, 133, 300, 1000]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=128, S=S, R=R, b=b, fmt=fmt)
    ks, vs = zip(*[_kv(L, hkv, d, seed=3, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    # three decode steps: append one position per sequence, then attend
    for step in range(3):
        kn, vn = _kv(len(lens), hkv, d, seed=5, idx=100 + step)
        p.append(list(range(len(lens))), [1] * len(lens), kn, vn)
        q = W.queries(len(lens), hq, d, seed=11, step=step, device="cuda")
        out, ref = p.decode(list(range(len(lens))), q)
        err = np.abs(out - ref).max()
        print("fmt", fmt, "b", b, "step", step, "max-abs", err)
        assert err <= TOL
    assert p.compare_cache(range(len(lens))) > 0


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 8, 128), (8, 2, 64), (4, 4, 64), (4, 1, 128)])
def test_group_and_dims(hq, hkv, d):
    _print_case("gqa", hq=hq, hkv=hkv, d=d)
    lens = [5, 200, 517]
    p = Pair(hq, hkv, d, num_pages=512, max_seqs=8, max_pps=64, S=4, R=64, b=d)
    ks, vs = zip(*[_kv(L, hkv, d, seed=7, idx=i) for i, L in enumerate(lens)])
    p.append([2, 0, 5], lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    assert p.compare_cache([2, 0, 5]) > 0
    q = W.queries(3, hq, d, seed=13, device="cuda")
    out, ref = p.decode([5, 2, 0], q)
    err = np.abs(out - ref).max()
    print("gqa", hq, hkv, d, "max-abs", err)
    assert err <= TOL


@pytest.mark.parametrize("S,R,b", [(4, 128, 128), (4, 32, 32), (0, 16, 1), (4, 0, 128)])
def test_requant_eviction(S, R, b):
    """INT4 codes re-quantized from the INT8 round trip: bit-exact pages, scales and INT8 slots after a
    ragged prefill, single-position appends (the per-position kernel) and a second prefill; decode and
    multi-query outputs within tolerance."""
    _print_case("requant", S=S, R=R, b=b)
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 100, 132, 133, 300, 1000]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=128, S=S, R=R, b=b, eviction=kv4.EVICT_REQUANT)
    ks, vs = zip(*[_kv(L, hkv, d, seed=13, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    for step in range(3):
        kn, vn = _kv(len(lens), hkv, d, seed=15, idx=100 + step)
        p.append(list(range(len(lens))), [1] * len(lens), kn, vn)
    kb, vb = _kv(77, hkv, d, seed=17, idx=7)
    p.append([9], [77], kb, vb)
    assert p.compare_cache(list(range(len(lens))) + [9]) > 0
    ids = list(range(len(lens))) + [9]
    q = W.queries(len(ids), hq, d, 19, device="cuda")
    out, ref = p.decode(ids, q)
    assert np.abs(out - ref).max() <= TOL
    nqs = [1, 3, 16, 20, 60, 64, 100, 77]
    qm = W.queries(sum(nqs), hq, d, 21, device="cuda")
    out, ref = p.multi(ids, nqs, qm)
    assert np.abs(out - ref).max() <= TOL


@pytest.mark.parametrize("fmt,b,S,R", [
    (kv4.FORMAT_INT4_PROT, 128, 4, 128),
    (kv4.FORMAT_INT4_PROT, 32, 4, 32),
    (kv4.FORMAT_INT8, 128, 0, 0),
])
def test_rope_append(fmt, b, S, R):
    """Fused RoPE append (pre-RoPE keys, Qwen3-style tables): bit-exact pages, scales and INT8 slots
    after a ragged prefill (page kernel), single-position appends (per-position kernel) and a second
    prefill; decode within tolerance."""
    _print_case("rope", fmt=fmt, b=b, S=S, R=R)
    hq, hkv, d = 32, 8, 128
    cos, sin = W.rope_tables(2048, d)
    lens = [1, 17, 100, 132, 133, 300, 1000]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=128, S=S, R=R, b=b, fmt=fmt)
    ks, vs = zip(*[_kv(L, hkv, d, seed=23, idx=i) for i, L in enumerate(lens)])
    p.append_rope(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cos, sin)
    for step in range(3):
        kn, vn = _kv(len(lens), hkv, d, seed=25, idx=100 + step)
        p.append_rope(list(range(len(lens))), [1] * len(lens), kn, vn, cos, sin)
    kb, vb = _kv(45, hkv, d, seed=27, idx=7)
    p.append_rope([9], [45], kb, vb, cos, sin)
    ids = list(range(len(lens))) + [9]
    assert p.compare_cache(ids) > 0
    out, ref = p.decode(ids, W.queries(len(ids), hq, d, 29, device="cuda"))
    assert np.abs(out - ref).max() <= TOL


def test_rope_append_errors():
    _print_case("rope_errors")
    hq, hkv, d = 8, 2, 64
    cos, sin = W.rope_tables(40, d)
    p = Pair(hq, hkv, d, num_pages=64, max_seqs=4, max_pps=8, S=4, R=16, b=64)
    k, v = _kv(30, hkv, d, seed=31)
    p.append_rope([0], [30], k, v, cos, sin)
    ct, st = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    k2, v2 = _kv(11, hkv, d, seed=32)
    with pytest.raises(kv4.KV4Error) as e:
        p.gpu.append_rope([0], [11], k2, v2, ct, st)          # position 40 is beyond the tables
    assert e.value.name == "KV4_ERR_INVALID_ARGUMENT"
    assert p.gpu.seq_length(0) == 30
    cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=8, max_seqs=2, max_pages_per_seq=4,
                     num_sinks=0, num_recent=0, hadamard_block=1, format=kv4.FORMAT_BF16)
    c = kv4.Cache(cfg, "cuda")
    with pytest.raises(kv4.KV4Error) as e:
        c.append_rope([0], [5], k2[:5].contiguous(), v2[:5].contiguous(), ct, st)
    assert e.value.name == "KV4_ERR_UNSUPPORTED"
    assert p.compare_cache([0]) > 0


@pytest.mark.parametrize("fmt,b", [(kv4.FORMAT_INT4_PROT, 128), (kv4.FORMAT_BF16, 1)])
def test_decode_bf16_output(fmt, b):
    """bf16 output = round-to-nearest-even of the fp32 output of the same call, bit for bit; and
    within the tolerance plus half a bf16 ulp of the oracle."""
    _print_case("decode_bf16", fmt=fmt)
    hq, hkv, d = 32, 8, 128
    lens = [1, 40, 133, 700, 2000]
    p = Pair(hq, hkv, d, num_pages=1024, max_seqs=8, max_pps=160, S=4, R=128, b=b, fmt=fmt)
    ks, vs = zip(*[_kv(L, hkv, d, seed=41, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    q = W.queries(len(lens), hq, d, 43, device="cuda")
    ids = list(range(len(lens)))
    o32, ref = p.decode(ids, q)
    o16 = p.gpu.decode_attention_bf16(ids, q)
    torch.cuda.synchronize()
    bits16 = o16.view(torch.int16).cpu().numpy().astype(np.uint16)
    assert np.array_equal(bits16, W.bf16_bits(torch.from_numpy(o32.astype(np.float32)).to(torch.bfloat16)))
    v16 = (bits16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(v16 - ref) <= TOL + np.abs(ref) * 2.0 ** -8)


def test_decode_wave_counts():
    """The split kernel at explicit wave counts: one wave (every unit in one slice), counts that
    leave a workgroup partly empty (7, 13), and counts with slices shorter than a unit.  The
    output must not depend on the partition beyond rounding order.  Units then hold 1 to 64
    partials, so the merge takes each of its paths (up to 4, 8 and 16 partials, and the general
    loop): 500 waves alone give all four."""
    _print_case("wave counts")
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 100, 132, 133, 300, 1000]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=128, S=4, R=128, b=128)
    ks, vs = zip(*[_kv(L, hkv, d, seed=3, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    q = W.queries(len(lens), hq, d, seed=13, step=0, device="cuda")
    for waves in (1, 7, 13, 64, 250, 500, 0):
        p.gpu.set_decode_waves(waves)
        out, ref = p.decode(list(range(len(lens))), q)
        err = np.abs(out - ref).max()
        print("waves", waves, "max-abs", err, flush=True)
        assert err <= TOL


def test_decode_two_rounds():
    """A second round of split waves over the last share of the steps (hardware-balanced tail): the
    partition into rounds changes nothing beyond rounding order; round-2 slices shorter than a unit,
    longer than a unit, and a round 2 with more waves than round 1."""
    _print_case("two rounds")
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 100, 132, 133, 300, 1000, 4000]
    p = Pair(hq, hkv, d, num_pages=2048, max_seqs=16, max_pps=300, S=4, R=128, b=128)
    ks, vs = zip(*[_kv(L, hkv, d, seed=3, idx=i) for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    q = W.queries(len(lens), hq, d, seed=17, step=0, device="cuda")
    ids = list(range(len(lens)))
    for waves, w2, pm in ((13, 7, 500), (64, 256, 850), (0, 512, 900), (0, 2048, 700), (1, 3, 999)):
        p.gpu.set_decode_waves(waves)
        p.gpu.set_decode_rounds(w2, pm)
        out, ref = p.decode(ids, q)
        err = np.abs(out - ref).max()
        print("waves", waves, "round 2", w2, "permille", pm, "max-abs", err, flush=True)
        assert err <= TOL
