"""GPU parity at the full workload sizes, in the launch configuration that bench.py times.

The HIP cache is built exactly as the benchmark builds it (same seeded inputs, one layer cache),
then one benchmark step runs (append one position per sequence, decode the batch with the
automatic split).  The oracle rebuilds only a seeded sample of the sequences -- as many as it can
decode in seconds -- and the sampled outputs must be within max-abs 2e-3; codes and scales of
sampled positions (INT4 page copy and INT8 slot) must match bit for bit.  The append workload
(256 sequences x 512 single-position steps, then a 32768-position prefill) is checked in full
against an oracle cache driven with the same calls.
"""
import math

import numpy as np
import pytest
import torch

import bench
import int4_kv_cache_fwht_amd as kv4
import kv4_inputs as W
import oracle
from kv4_inputs import bf16_bits
from tests import kv4_layout
from tests.pair import Pair, TOL

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print("CASE", name, kw, flush=True)


def _gpu_codes(cache, pool, i8, seq, t, h, kv):
    """(codes, (s, z)) of position t of a HIP-cache sequence: INT4 page copy and INT8 slot."""
    sz = cache.sizes
    page = cache.block_table(seq)[t // 16]
    c4, s4 = kv4_layout.int4_page_block(pool[page, h], cache.cfg.head_dim)
    out = {"int4": (c4[t % 16, kv], tuple(s4[t % 16, kv]))}
    S, R = cache.cfg.num_sinks, cache.cfg.num_recent
    L = cache.seq_length(seq)
    if oracle.is_protected(t, L, S, R):
        u = oracle.int8_slot(t, S, R)
        c8, g8, g8b = kv4_layout.int8_tile(i8[seq, h, u // 16], cache.cfg.head_dim)
        assert (g8[u % 16, kv] == g8b[u % 16, kv]).all()
        out["int8"] = (c8[u % 16, kv], tuple(g8[u % 16, kv]))
    return out


def _check_workload(name, sample_fn, positions_per_seq=12, mq_rows=(4,)):
    w = W.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    b = bench.Bench(w, "int4", 1, 1, 2, dev, 0)
    b.step()                       # append 1 position to every sequence, decode all (auto split)
    torch.cuda.synchronize()
    out = b.out.cpu().numpy().astype(np.float64)
    lens0 = b.lens0
    sample = sample_fn(lens0)
    cache = b.caches[0]
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    ch = W.outlier_channels(hkv, d, w.outlier_channels, w.seed)
    # oracle holding the sampled sequences (prefill from the same seeded draws, then the appended row)
    pages = sum(math.ceil((lens0[i] + 1) / 16) for i in sample) + len(sample)
    max_pps = max(math.ceil((lens0[i] + 1) / 16) for i in sample) + 1
    ora = oracle.OracleCache(hq, hkv, d, 16, pages, len(sample), max_pps, w.num_sinks, w.num_recent,
                             w.hadamard_block)
    for j, i in enumerate(sample):
        k, v = W.seq_kv(hkv, d, lens0[i], ch, w.outlier_scale, w.seed, 0, i, dev)
        assert ora.append([j], [lens0[i]], bf16_bits(k), bf16_bits(v)) == oracle.OK
        assert ora.append([j], [1], bf16_bits(b.kn[0][i:i + 1]), bf16_bits(b.vn[0][i:i + 1])) == oracle.OK
    q = b.q[0][sample].contiguous()
    ref, used = ora.decode(list(range(len(sample))), bf16_bits(q))
    err = np.abs(out[sample] - ref).max()
    print(name, "sampled sequences", sample, "lengths", [lens0[i] + 1 for i in sample], "max-abs", err,
          "oracle threads", used, flush=True)
    assert err <= TOL
    # multi-query attention over the same cache: the last nq positions of every sequence as causal
    # query rows, one call (its own work split); the oracle checks the sampled sequences
    for nq in mq_rows:
        qm = W.queries(nq * len(lens0), hq, d, w.seed, step=99 + nq, device=dev)
        outm = cache.multi_query_attention(list(range(len(lens0))), [nq] * len(lens0), qm).cpu().numpy()
        rows = np.concatenate([np.arange(nq * i, nq * (i + 1)) for i in sample])
        refm, _ = ora.attend_multi(list(range(len(sample))), [nq] * len(sample),
                                   bf16_bits(qm[torch.from_numpy(rows).to(dev)]))
        errm = np.abs(outm[rows].astype(np.float64) - refm).max()
        print(name, "multi-query (%d rows) sampled max-abs" % nq, errm, flush=True)
        assert errm <= TOL
    # codes and scales of sampled positions, bit for bit
    sz = cache.sizes
    pool = cache.page_pool.cpu().numpy()[: sz.page_pool].reshape(cache.cfg.num_pages, hkv, sz.page_block_bytes)
    i8 = cache.int8_pool.cpu().numpy().reshape(cache.cfg.max_seqs, hkv, sz.int8_tiles, sz.int8_tile_bytes)
    rng = np.random.default_rng(123)
    checked = 0
    for j, i in enumerate(sample):
        L = lens0[i] + 1
        ts = {0, w.num_sinks - 1, w.num_sinks, L - w.num_recent - 1, L - w.num_recent, L - 1}
        ts |= set(int(x) for x in rng.integers(0, L, positions_per_seq))
        for t in sorted(x for x in ts if 0 <= x < L):
            h = int(rng.integers(0, hkv))
            for kv in range(2):
                got = _gpu_codes(cache, pool, i8, i, t, h, kv)
                oc, osz, _ = ora.page_token(j, t, h, kv)
                assert (got["int4"][0] == oc).all(), (name, i, t, h, kv)
                assert got["int4"][1] == tuple(osz), (name, i, t, h, kv)
                if "int8" in got:
                    u = oracle.int8_slot(t, w.num_sinks, w.num_recent)
                    c8, (s8, z8), tok = ora.int8_slot_contents(j, u, h, kv)
                    assert tok == t
                    assert (got["int8"][0] == c8).all() and got["int8"][1] == (s8, z8), (name, i, t, h, kv)
                checked += 1
    print(name, "positions checked bit-exact", checked, flush=True)


def test_qwen3_8b_layer_full_size():
    _print_case("qwen3_8b_layer full size")
    _check_workload("qwen3_8b_layer", lambda L: [int(np.argmin(L)), int(np.argmax(L)), 17, 40], mq_rows=(4, 16, 64))


def test_rollout_layer_full_size():
    _print_case("rollout layer full size")
    _check_workload("rollout", lambda L: [int(np.argmin(L)), int(np.argmax(L)), 100])


def test_rollout_tp8_full_size():
    """One GPU's share of the rollout regime under 8-way tensor parallelism by kv head: 256
    sequences with 1 kv head and 4 query heads, split over the bench's 2048 waves (8 per unit)."""
    _print_case("rollout_tp8 full size")
    _check_workload("rollout_tp8", lambda L: [int(np.argmin(L)), int(np.argmax(L)), 100])


def test_long_context_full_size():
    _print_case("long_context full size")
    _check_workload("long_context", lambda L: [0, 3, len(L) - 1])


def test_append_workload_full():
    """256 empty sequences, 512 single-position steps (eviction from INT8 begins at L = 133), then a
    32768-position prefill into one more sequence: page ids, codes and scales of every sequence, and
    decode of all of them."""
    _print_case("append workload")
    w = W.WORKLOADS["append"]
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    B, steps = 256, 512
    p = Pair(hq, hkv, d, num_pages=B * (steps // 16) + 2048 + 16, max_seqs=B + 1, max_pps=2048 + 1,
             S=w.num_sinks, R=w.num_recent, b=w.hadamard_block)
    ch = W.outlier_channels(hkv, d, w.outlier_channels, w.seed)
    ids = list(range(B))
    for s in range(steps):
        k, v = W.seq_kv(hkv, d, B, ch, w.outlier_scale, w.seed, 2000 + s, 0, "cuda")
        p.append(ids, [1] * B, k, v)
    for s in ids:
        assert p.gpu.block_table(s) == list(p.ora.block_table(s))
        assert p.gpu.block_table(s) == [256 * j + s for j in range(steps // 16)]
    n = p.compare_cache([0, 1, 77, 128, 255])
    print("append: compared records", n, flush=True)
    q = W.queries(B, hq, d, w.seed, step=7, device="cuda")
    out, ref = p.decode(ids, q)
    err = np.abs(out - ref).max()
    print("append: decode of 256 x 512 max-abs", err, flush=True)
    assert err <= TOL
    # bulk prefill of 32768 positions into one sequence
    k, v = W.seq_kv(hkv, d, 32768, ch, w.outlier_scale, w.seed, 3000, 0, "cuda")
    p.append([B], [32768], k, v)
    n = p.compare_cache([B])
    print("append: prefill compared records", n, flush=True)
    q1 = W.queries(1, hq, d, w.seed, step=8, device="cuda")
    out, ref = p.decode([B], q1)
    err = np.abs(out - ref).max()
    print("append: decode of the 32768 prefill max-abs", err, flush=True)
    assert err <= TOL


def test_edge_cases():
    """Empty calls, zero-length appends inside a call, all-zero and constant rows (scale 0), large
    magnitudes near the fp16 range, a single position, and b = 1 (no rotation)."""
    _print_case("edge cases")
    hq, hkv, d = 8, 2, 64
    for b, S, R in ((64, 4, 16), (1, 2, 0)):
        p = Pair(hq, hkv, d, num_pages=256, max_seqs=8, max_pps=32, S=S, R=R, b=b)
        empty = torch.empty((0, hkv, d), dtype=torch.bfloat16, device="cuda")
        p.append([], [], empty, empty)
        assert p.gpu.decode_attention([], torch.empty((0, hq, d), dtype=torch.bfloat16, device="cuda")).numel() == 0
        rows = []
        zero = torch.zeros((20, hkv, d), dtype=torch.bfloat16)
        const = torch.full((20, hkv, d), 1.5, dtype=torch.bfloat16)
        big = (torch.randn((20, hkv, d), generator=torch.Generator().manual_seed(5)) * 2000).to(torch.bfloat16)
        ramp = torch.arange(20 * hkv * d, dtype=torch.float32).reshape(20, hkv, d).to(torch.bfloat16) * 0.01
        for blk in (zero, const, big, ramp):
            rows.append(blk)
        kcat = torch.cat(rows).to("cuda").contiguous()
        vcat = torch.cat(rows[::-1]).to("cuda").contiguous()
        # sequence 3 gets 0 positions in this call, sequence 5 one, sequence 1 the rest
        p.append([3, 5, 1], [0, 1, 79], kcat, vcat)
        assert p.compare_cache([5, 1]) > 0
        q = W.queries(2, hq, d, 3, device="cuda")
        out, ref = p.decode([5, 1], q)
        err = np.abs(out - ref).max()
        print("edge b", b, "max-abs", err, "max |out|", np.abs(ref).max(), flush=True)
        assert err <= TOL


def test_host_errors_leave_state_unchanged():
    """Argument errors, OUT_OF_PAGES (all or nothing), decode of an empty sequence and a workspace
    that is too small are rejected on the host; nothing changes and no kernel runs."""
    _print_case("host errors")
    hq, hkv, d = 8, 2, 64
    cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=6, max_seqs=4,
                     max_pages_per_seq=8, num_sinks=4, num_recent=16, hadamard_block=64)
    c = kv4.Cache(cfg, "cuda")
    k, v = W.seq_kv(hkv, d, 120, None, 1.0, 1, 0, 0, "cuda")
    c.append([0], [40], k[:40].contiguous(), v[:40].contiguous())       # 3 pages
    before = (c.free_pages(), c.block_table(0), c.seq_length(0))
    with pytest.raises(kv4.KV4Error) as e:
        c.append([1, 2], [40, 20], k[:60].contiguous(), v[:60].contiguous())  # needs 3 + 2 > 3 free
    assert e.value.status == 2
    assert (c.free_pages(), c.block_table(0), c.seq_length(0)) == before and c.seq_length(1) == 0
    with pytest.raises(kv4.KV4Error) as e:
        c.append([1, 1], [1, 1], k[:2].contiguous(), v[:2].contiguous())
    assert e.value.status == 1
    with pytest.raises(kv4.KV4Error) as e:
        c.append([0], [100], k[:100].contiguous(), v[:100].contiguous())    # > max_pages_per_seq * 16
    assert e.value.status == 3
    q = W.queries(1, hq, d, 1, device="cuda")
    with pytest.raises(kv4.KV4Error) as e:
        c.decode_attention([2], q)
    assert e.value.status == 3
    with pytest.raises(kv4.KV4Error) as e:
        c.decode_attention([0], q, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 4
    assert (c.free_pages(), c.block_table(0), c.seq_length(0)) == before
    c.append([1, 2], [32, 16], k[:48].contiguous(), v[:48].contiguous())    # 2 + 1 pages: fits exactly
    assert c.free_pages() == 0


@pytest.mark.parametrize("n", [300, 1024])
def test_uploaded_plan_path(n):
    """More sequences than the kernel arguments carry (300, 1024 > 256): the decode plan and the
    single-position append tasks are uploaded instead (at 1024 the append grid runs far past the
    argument block's entries).  Ragged lengths, two decode steps."""
    _print_case("uploaded plan", n=n)
    hq, hkv, d = 8, 2, 64
    rng = np.random.default_rng(9)
    lens = [int(x) for x in rng.integers(1, 200, n)]
    p = Pair(hq, hkv, d, num_pages=sum(math.ceil((L + 2) / 16) for L in lens) + n, max_seqs=n, max_pps=16,
             S=4, R=32, b=64)
    ch = W.outlier_channels(hkv, d, 2, 9)
    ks, vs = zip(*[W.seq_kv(hkv, d, L, ch, 10.0, 9, 0, i, "cuda") for i, L in enumerate(lens)])
    p.append(list(range(n)), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    ids = [int(x) for x in rng.permutation(n)]
    for step in range(2):
        kn, vn = W.seq_kv(hkv, d, n, ch, 10.0, 9, 50 + step, 0, "cuda")
        p.append(ids, [1] * n, kn, vn)
        q = W.queries(n, hq, d, 9, step=step, device="cuda")
        out, ref = p.decode(ids, q)
        err = np.abs(out - ref).max()
        print("uploaded plan step", step, "max-abs", err, flush=True)
        assert err <= TOL
    assert p.compare_cache([ids[0], ids[1], 17, n - 1]) > 0
