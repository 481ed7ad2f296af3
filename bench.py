#!/usr/bin/env python3
"""Decode-step benchmark of the INT4 KV cache on one MI355X.

One step = one pass of the hot path over one batch: append one new position to every sequence
(fused rotation + quantization into the paged cache, INT8 protection of the newest positions)
and then GQA decode attention over every sequence's full context.  The timed region holds
exactly --steps steps, bracketed by device synchronization; inputs are resident in HBM.

Prints ONE JSON line.  value = kv-tokens/s = (sum of context lengths attended per step) x steps /
wall time.  roofline = the decode split-KV kernel's algorithmic bytes per launch / its average
duration (HIP events recorded by the library on the call's stream), against the 8 TB/s HBM peak.
cpu_baseline = the CPU oracle's decode on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
METRIC = "INT4-KV decode attention kv-tokens/s and achieved HBM GB/s (% of MI355X peak)"
FORMATS = {"int4": 0, "int8": 1, "bf16": 2}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="qwen3_8b_layer",
                    choices=["qwen3_8b_layer", "rollout", "long_context", "tiny", "append", "multi_query"],
                    help="decode workloads; 'append': the append path alone at Hadamard block 128 vs 1; "
                         "'multi_query': causal multi-query attention on the Qwen3-8B-shaped layer")
    ap.add_argument("--mq-rows", type=int, default=4, help="query rows per sequence of the multi_query workload")
    ap.add_argument("--caches", type=int, default=4, help="distinct layer caches cycled (defeats the 256 MB MALL)")
    ap.add_argument("--baselines", default="int8,bf16", help="comma list of baseline formats ('' for none)")
    ap.add_argument("--baseline-steps", type=int, default=12)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true", help="skip the decode-error diagnostic")
    ap.add_argument("--decode-waves", type=int, default=0)
    ap.add_argument("--hadamard-block", type=int, default=0,
                    help="override the workload's Hadamard block (1 = plain INT4: no q / output rotation)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write the measured decode traffic from two rocprofv3 --pmc output folders")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference kernel for PMC byte counters)")
    return ap.parse_args()


def per_token_bytes(fmt, hkv, d):
    """Algorithmic bytes per cached position (all kv heads, K and V)."""
    if fmt == "int4":
        return hkv * 2 * (d // 2 + 4)
    if fmt == "int8":
        return hkv * 2 * (d + 4)
    return hkv * 2 * d * 2


def decode_bytes(fmt, lens, w):
    """Algorithmic HBM bytes of one decode launch: cached positions read once (INT4 pages for
    unprotected positions, INT8 for the protected ones), block-table entries, q in, out out."""
    hkv, d, hq = w.num_kv_heads, w.head_dim, w.num_q_heads
    b4, b8 = per_token_bytes("int4", hkv, d), per_token_bytes("int8", hkv, d)
    total = 0
    for L in lens:
        if fmt == "int4":
            p = min(L, w.num_sinks + w.num_recent)
            total += (L - p) * b4 + p * b8
        else:
            total += L * per_token_bytes(fmt, hkv, d)
        total += math.ceil(L / 16) * 4 + hq * d * 2 + hq * d * 4
    return total


def kernel_source_hash():
    """Hash of the sources that define the decode kernels: kv4_decode.hip, the device helpers and
    plain structs it includes, and the DecodeArgs struct of kv4_launch.h."""
    csrc = os.path.join(ROOT, "int4_kv_cache_fwht_amd", "csrc")
    h = hashlib.sha256()
    for name in ("kv4_decode.hip", "kv4_common.h", "kv4_device_types.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(csrc, "kv4_launch.h")) as f:
        text = f.read()
    i = text.index("struct DecodeArgs")
    h.update(text[i:text.index("};", i)].encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, fmt):
    """Per-launch HBM bytes of the split kernel from committed rocprofv3 PMC runs, if they were taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_split_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get("%s/%s" % (workload, fmt))
    if not e or e.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


class Bench:
    def __init__(self, w, fmt, n_caches, total_steps, device, decode_waves):
        import torch
        import int4_kv_cache_fwht_amd as kv4
        import kv4_inputs as W
        self.torch, self.kv4, self.W = torch, kv4, W
        self.w, self.fmt, self.device = w, fmt, device
        self.lens0 = w.lengths()
        B = w.batch
        growth = math.ceil(total_steps / n_caches) + 1
        max_len = max(self.lens0) + growth
        pages = sum(math.ceil((L + growth) / 16) for L in self.lens0) + B
        self.channels = W.outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
        self.caches, self.lens = [], []
        for c in range(n_caches):
            cfg = kv4.Config(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                             num_pages=pages, max_seqs=B, max_pages_per_seq=math.ceil(max_len / 16) + 1,
                             num_sinks=w.num_sinks, num_recent=w.num_recent,
                             hadamard_block=w.hadamard_block if fmt != "bf16" else 1, format=FORMATS[fmt])
            cache = kv4.Cache(cfg, device)
            if decode_waves:
                cache.set_decode_waves(decode_waves)
            self._prefill(cache, layer=c)
            self.caches.append(cache)
            self.lens.append(list(self.lens0))
        self.ids = list(range(B))
        # per-step inputs, resident before timing
        self.kn, self.vn, self.q = [], [], []
        for s in range(total_steps):
            k, v = W.seq_kv(w.num_kv_heads, w.head_dim, B, self.channels, w.outlier_scale, w.seed, 1000 + s, 0,
                            device)
            self.kn.append(k)
            self.vn.append(v)
            self.q.append(W.queries(B, w.num_q_heads, w.head_dim, w.seed, step=s, device=device))
        self.out = torch.empty((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device=device)
        self.step_idx = 0
        torch.cuda.synchronize()

    def _prefill(self, cache, layer):
        torch, W, w = self.torch, self.W, self.w
        ids, chunk, rows = [], [], 0
        for i, L in enumerate(self.lens0):
            ids.append(i)
            chunk.append(L)
            rows += L
            if rows >= 65536 or i == len(self.lens0) - 1:
                ks, vs = [], []
                for j, Lj in zip(ids, chunk):
                    k, v = W.seq_kv(w.num_kv_heads, w.head_dim, Lj, self.channels, w.outlier_scale, w.seed, layer, j,
                                    self.device)
                    ks.append(k)
                    vs.append(v)
                cache.append(ids, chunk, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
                ids, chunk, rows = [], [], 0
        torch.cuda.synchronize()

    def step(self):
        """One step on the next cache; returns the kv-tokens attended."""
        s = self.step_idx
        c = s % len(self.caches)
        cache = self.caches[c]
        cache.append(self.ids, [1] * len(self.ids), self.kn[s], self.vn[s])
        cache.decode_attention(self.ids, self.q[s], out=self.out)
        self.lens[c] = [L + 1 for L in self.lens[c]]
        self.step_idx += 1
        return sum(self.lens[c]), self.lens[c]

    def timed(self, steps):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks = 0
        for _ in range(steps):
            toks += self.step()[0]
        torch.cuda.synchronize()
        return time.perf_counter() - t0, toks

    def profiled(self, steps):
        """Steps with the library's kernel events on; returns (split avg s, merge avg s, append avg s,
        algorithmic bytes per split launch averaged)."""
        for c in self.caches:
            c.profile_enable(True)
        nbytes = 0
        for _ in range(steps):
            _, lens = self.step()
            nbytes += decode_bytes(self.fmt, lens, self.w)
        tot = {"split_ms": 0.0, "merge_ms": 0.0, "append_ms": 0.0, "decode_launches": 0, "append_launches": 0}
        for c in self.caches:
            p = c.profile_read()
            for k in tot:
                tot[k] += p[k]
            c.profile_enable(False)
        n = max(tot["decode_launches"], 1)
        return (tot["split_ms"] / n * 1e-3, tot["merge_ms"] / n * 1e-3,
                tot["append_ms"] / max(tot["append_launches"], 1) * 1e-3, nbytes / n)


def cpu_baseline(w, seconds, device):
    """The oracle's decode (fp64, threaded) on a bounded sample of the workload: the first sequences
    of layer 0, decoded repeatedly for about `seconds` of CPU time."""
    import torch
    import kv4_inputs as W
    import oracle
    lens = w.lengths()
    n_s = min(len(lens), 4)
    ids = list(range(n_s))
    ch = W.outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
    ora = oracle.OracleCache(w.num_q_heads, w.num_kv_heads, w.head_dim, 16,
                             sum(math.ceil(L / 16) for L in lens[:n_s]) + 1, n_s,
                             max(math.ceil(L / 16) for L in lens[:n_s]) + 1, w.num_sinks, w.num_recent,
                             w.hadamard_block)
    for i in ids:
        k, v = W.seq_kv(w.num_kv_heads, w.head_dim, lens[i], ch, w.outlier_scale, w.seed, 0, i, device)
        assert ora.append([i], [lens[i]], W.bf16_bits(k), W.bf16_bits(v)) == oracle.OK
    q = W.bf16_bits(W.queries(n_s, w.num_q_heads, w.head_dim, w.seed, device=device))
    threads = min(16, os.cpu_count() or 1)
    reps, used, t0 = 0, 0, time.perf_counter()
    while True:
        _, used = ora.decode(ids, q, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    toks = reps * sum(lens[:n_s])
    return {"value": toks / el, "unit": "kv-tokens/s", "cores": used, "kind": "oracle",
            "sample": "%d sequences (%d positions) of %s, oracle decode in fp64 repeated %d times (%.1f s)" % (
                n_s, sum(lens[:n_s]), w.name, reps, el)}


QUALITY_VARIANTS = [
    # name, format, hadamard block (0 = workload's), sinks, recent (None = workload's), eviction
    ("int4_rot_prot", "int4", 0, None, None, 0),
    ("int4_rot_prot_requant", "int4", 0, None, None, 1),
    ("int4_rot_noprot", "int4", 0, 0, 0, 0),
    ("int4_norot_prot", "int4", 1, None, None, 0),
    ("int4_rot_sinks_only", "int4", 0, None, 0, 0),
    ("int4_rot_recent_only", "int4", 0, 0, None, 0),
    ("int4_plain", "int4", 1, 0, 0, 0),
    ("int8", "int8", 0, 0, 0, 0),
    ("bf16", "bf16", 1, 0, 0, 0),
]


def quality(w, device, n_seqs=4):
    """Diagnostic: decode error of each storage variant against exact attention (fp64, numpy) on the
    unquantized bf16 K / V of a seeded sample of the workload's sequences."""
    import numpy as np
    import torch
    import int4_kv_cache_fwht_amd as kv4
    import kv4_inputs as W
    lens = w.lengths()[:n_seqs]
    ch = W.outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
    kvs = [W.seq_kv(w.num_kv_heads, w.head_dim, L, ch, w.outlier_scale, w.seed, 0, i, device) for i, L in enumerate(lens)]
    q = W.queries(len(lens), w.num_q_heads, w.head_dim, w.seed, device=device)
    G = w.num_q_heads // w.num_kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    qf = q.float().cpu().numpy().astype(np.float64)
    ref = np.zeros(qf.shape)
    for i, (k, v) in enumerate(kvs):
        kf = k.float().cpu().numpy().astype(np.float64)
        vf = v.float().cpu().numpy().astype(np.float64)
        for g in range(w.num_q_heads):
            e = kf[:, g // G, :] @ qf[i, g] * scale
            p_ = np.exp(e - e.max())
            ref[i, g] = (p_ / p_.sum()) @ vf[:, g // G, :]
    res = {}
    for name, fmt, block, S, R, evict in QUALITY_VARIANTS:
        cfg = kv4.Config(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                         num_pages=sum(math.ceil(L / 16) for L in lens) + 4, max_seqs=len(lens),
                         max_pages_per_seq=max(math.ceil(L / 16) for L in lens) + 1,
                         num_sinks=w.num_sinks if S is None else S, num_recent=w.num_recent if R is None else R,
                         hadamard_block=block or w.hadamard_block, format=FORMATS[fmt], eviction=evict)
        cache = kv4.Cache(cfg, device)
        cache.append(list(range(len(lens))), lens, torch.cat([k for k, _ in kvs]).contiguous(),
                     torch.cat([v for _, v in kvs]).contiguous())
        out = cache.decode_attention(list(range(len(lens))), q).cpu().numpy().astype(np.float64)
        err = out - ref
        res[name] = {"max_abs": float(np.abs(err).max()),
                     "rel_rms": float(np.sqrt((err ** 2).mean() / (ref ** 2).mean()))}
        del cache
    return {"reference": "exact fp64 attention on the unquantized bf16 K/V, %d sequences (%d positions)" % (
        len(lens), sum(lens)), "errors": res}


def copy_probe(device):
    """Plain device copy of 1 GiB (the reference kernel for PMC byte counters) -> GB/s moved."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del a, b
    return 2 * n * reps / el / 1e9


def append_workload(device, repeats=7):
    """The append path alone: 256 empty sequences x 512 single-position steps, and a bulk prefill of
    32768 positions into one sequence, timed with the rotation (b = 128), without it (b = 1, plain
    INT4), and with the fused RoPE of pre-RoPE keys (b = 128).  Returns the JSON record."""
    import torch
    import int4_kv_cache_fwht_amd as kv4
    import kv4_inputs as W
    w = W.WORKLOADS["append"]
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    B, steps, bulk = 256, 512, 32768
    ch = W.outlier_channels(hkv, d, w.outlier_channels, w.seed)
    rows = [W.seq_kv(hkv, d, B, ch, w.outlier_scale, w.seed, 2000 + s, 0, device) for s in range(steps)]
    kb, vb = W.seq_kv(hkv, d, bulk, ch, w.outlier_scale, w.seed, 3000, 0, device)
    cos, sin = (torch.from_numpy(t).to(device) for t in W.rope_tables(bulk + 1, d))
    res = {}
    for name, block, rope in (("b128", 128, False), ("b1", 1, False), ("b128_rope", 128, True)):
        cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=B * (steps // 16) + bulk // 16 + 16,
                         max_seqs=B + 1, max_pages_per_seq=bulk // 16 + 1, num_sinks=w.num_sinks,
                         num_recent=w.num_recent, hadamard_block=block, format=0)

        def app(cache, ids, n, k, v):
            if rope:
                cache.append_rope(ids, n, k, v, cos, sin)
            else:
                cache.append(ids, n, k, v)

        best_steps = best_bulk = float("inf")
        for _ in range(repeats):
            cache = kv4.Cache(cfg, device)
            ids = list(range(B))
            app(cache, ids, [1] * B, rows[0][0], rows[0][1])  # warm-up of the launch path
            torch.cuda.synchronize()
            for i in ids:
                cache.seq_free(i)
            cache.profile_enable(True)
            for s in range(steps):
                app(cache, ids, [1] * B, rows[s][0], rows[s][1])
            p = cache.profile_read()
            best_steps = min(best_steps, p["append_ms"] / p["append_launches"] * 1e3)
            cache.profile_enable(True)
            app(cache, [B], [bulk], kb, vb)
            p = cache.profile_read()
            best_bulk = min(best_bulk, p["append_ms"] * 1e3)
            cache.profile_enable(False)
            del cache
        res[name] = (best_steps, best_bulk)
    (s128, b128), (s1, b1), (sr, br) = res["b128"], res["b1"], res["b128_rope"]
    bulk_bytes = bulk * hkv * d * 2 * 2 + bulk * hkv * 2 * (d // 2 + 4)   # bf16 in, INT4 + scales out
    return {"metric": "INT4 KV append (rotation + quantization + pack) tokens/s", "value": B / (s128 * 1e-6),
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 1, "ms_per_step": s128 * 1e-3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "append", "sequences": B, "steps": steps, "bulk_prefill": bulk, "kv_heads": hkv,
                       "head_dim": d, "sinks": w.num_sinks, "recent": w.num_recent},
            "append_step_us": {"b128": s128, "b1": s1, "rotation_overhead": s128 / s1 - 1.0,
                               "b128_fused_rope": sr, "fused_rope_overhead": sr / s128 - 1.0},
            "bulk_prefill_us": {"b128": b128, "b1": b1, "rotation_overhead": b128 / b1 - 1.0,
                                "GBps_b128": bulk_bytes / (b128 * 1e-6) / 1e9, "b128_fused_rope": br,
                                "fused_rope_overhead": br / b128 - 1.0},
            "note": "best of %d repeats; kernel time from HIP events on the call's stream" % repeats}

def mq_workload(device, n_q, steps, warmup, n_caches=4):
    """Multi-query attention on the Qwen3-8B-shaped layer (64 sequences, lengths uniform in
    [1024, 8192]): each step appends n_q positions to every sequence of one of n_caches layer
    caches (cycled, as in the decode bench) and then attends with the n_q new positions as causal
    query rows.  Returns the JSON record."""
    import torch
    import int4_kv_cache_fwht_amd as kv4
    import kv4_inputs as W
    w = W.WORKLOADS["qwen3_8b_layer"]
    hq, hkv, d, B = w.num_q_heads, w.num_kv_heads, w.head_dim, w.batch
    lens0 = w.lengths()
    prof_steps = 12
    total = warmup + steps + prof_steps
    growth = (total // n_caches + 1) * n_q
    pages = sum(math.ceil((L + growth) / 16) for L in lens0) + B
    ch = W.outlier_channels(hkv, d, w.outlier_channels, w.seed)
    caches, lens = [], []
    for c in range(n_caches):
        cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=pages, max_seqs=B,
                         max_pages_per_seq=math.ceil((max(lens0) + growth) / 16) + 1, num_sinks=w.num_sinks,
                         num_recent=w.num_recent, hadamard_block=w.hadamard_block, format=0)
        cache = kv4.Cache(cfg, device)
        for i, L in enumerate(lens0):
            k, v = W.seq_kv(hkv, d, L, ch, w.outlier_scale, w.seed, c, i, device)
            cache.append([i], [L], k, v)
        caches.append(cache)
        lens.append(list(lens0))
    ids = list(range(B))
    kn, qs = [], []
    for st in range(total):
        kn.append(W.seq_kv(hkv, d, B * n_q, ch, w.outlier_scale, w.seed, 5000 + st, 0, device))
        qs.append(W.queries(B * n_q, hq, d, w.seed, step=st, device=device))
    out = torch.empty((B * n_q, hq, d), dtype=torch.float32, device=device)
    state = {"i": 0}

    def one():
        st = state["i"]
        c = st % n_caches
        caches[c].append(ids, [n_q] * B, kn[st][0], kn[st][1])
        caches[c].multi_query_attention(ids, [n_q] * B, qs[st], out=out)
        lens[c] = [L + n_q for L in lens[c]]
        state["i"] += 1
        return lens[c]

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    attended = 0
    for _ in range(steps):
        ls = one()
        attended += sum(n_q * L - n_q * (n_q - 1) // 2 for L in ls)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    for c in caches:
        c.profile_enable(True)
    nbytes = flops = 0
    for _ in range(prof_steps):
        ls = one()
        nbytes += decode_bytes("int4", ls, w) + len(ls) * (n_q - 1) * hq * d * 6
        flops += sum(n_q * L - n_q * (n_q - 1) // 2 for L in ls) * hq * 4 * d
    tot = {"mq_split_ms": 0.0, "mq_merge_ms": 0.0, "append_ms": 0.0, "mq_launches": 0, "append_launches": 0}
    for c in caches:
        p = c.profile_read()
        for k in tot:
            tot[k] += p[k]
        c.profile_enable(False)
    split_s = tot["mq_split_ms"] / tot["mq_launches"] * 1e-3
    bytes_launch, flops_launch = nbytes / prof_steps, flops / prof_steps
    gbps = bytes_launch / split_s / 1e9
    tflops = flops_launch / split_s / 1e12
    intensity = flops_launch / bytes_launch
    ridge = MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / MFMA_F16_PEAK_TFLOPS}
    roof.update({"traffic": None, "kernel": "mq_split_kernel<128,4,INT4_PROT>", "avg_launch_us": split_s * 1e6,
                 "algorithmic_bytes_per_launch": bytes_launch, "algorithmic_flops_per_launch": flops_launch,
                 "achieved_GBps": gbps, "achieved_TFLOPs": tflops, "flops_per_byte": intensity})
    return {"metric": "INT4-KV multi-query attention: attended (query row, position) pairs per s", "value":
            attended / el, "unit": "row-positions/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": el / steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32", "data": "synthetic",
            "config": {"workload": "multi_query", "batch": B, "query_rows_per_seq": n_q, "kv_heads": hkv,
                       "q_heads": hq, "head_dim": d, "context": "uniform[1024, 8192] + growth", "sinks": w.num_sinks,
                       "recent": w.num_recent, "hadamard_block": w.hadamard_block, "distinct_caches": n_caches},
            "roofline": roof,
            "step_breakdown_us": {"append": tot["append_ms"] / max(tot["append_launches"], 1) * 1e3,
                                  "mq_split": split_s * 1e6,
                                  "mq_merge": tot["mq_merge_ms"] / tot["mq_launches"] * 1e3}}


def write_traffic(fetch_dir, write_dir, workload, fmt="int4"):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; both with
    --copy-calibration) into the measured HBM bytes per decode-split launch, each counter scaled by
    what it reads for the plain 1 GiB copy; stores them, keyed by the decode sources' hash, in
    profiles/decode_split_traffic.json."""
    import csv
    import glob

    def per_kernel(root, counter):
        vals = {}
        for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row["Counter_Name"] == counter:
                        vals.setdefault(row.get("Kernel_Name", ""), []).append(float(row["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    kname = "kv4::decode_split_kernel<128, 4, %d>" % FORMATS[fmt]
    pick = lambda vals: next(v for k, v in vals.items() if kname in k)
    copy_f = max(v for k, vs in fetch.items() if "copyBuffer" in k for v in vs)
    copy_w = max(v for k, vs in write.items() if "copyBuffer" in k for v in vs)
    n = 1 << 30
    ff, wf = n / (copy_f * 1024), n / (copy_w * 1024)
    f_kib, w_kib = pick(fetch), pick(write)
    fb = sum(f_kib) / len(f_kib) * 1024 * ff
    wb = sum(w_kib) / len(w_kib) * 1024 * wf
    path = os.path.join(ROOT, "profiles", "decode_split_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    cmd = ("rocprofv3 --pmc %s --kernel-include-regex 'kv4|copyBuffer|copy' --output-format csv -d %s -o run -- "
           "python bench.py --workload %s --steps 4 --warmup 1 --baselines '' --no-cpu-baseline --no-quality "
           "--copy-calibration")
    rec["%s/%s" % (workload, fmt)] = {
        "kernel": "decode_split_kernel<128,4,%s>" % {"int4": "INT4_PROT", "int8": "INT8", "bf16": "BF16"}[fmt],
        "kernel_source_hash": kernel_source_hash(),
        "bytes_per_launch": fb + wb, "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
        "fetch_size_kib_mean": sum(f_kib) / len(f_kib), "write_size_kib_mean": sum(w_kib) / len(w_kib),
        "dispatches": len(f_kib),
        "copy_reference": {"bytes_read": n, "bytes_written": n, "fetch_size_kib": copy_f, "write_size_kib": copy_w,
                           "fetch_factor": ff, "write_factor": wf},
        "commands": [cmd % ("FETCH_SIZE", fetch_dir, workload), cmd % ("WRITE_SIZE", write_dir, workload),
                     "python bench.py --workload %s --traffic-from %s %s" % (workload, fetch_dir, write_dir)],
    }
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec["%s/%s" % (workload, fmt)]


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(write_traffic(args.traffic_from[0], args.traffic_from[1], args.workload)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the decode path is built and measured on one GPU "
              "(multi-GPU sharding is not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import kv4_inputs as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda", 0)
    if args.workload == "append":
        print(json.dumps(append_workload(device)), flush=True)
        return
    if args.workload == "multi_query":
        print(json.dumps(mq_workload(device, args.mq_rows, args.steps, args.warmup)), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    if args.hadamard_block:
        import dataclasses
        w = dataclasses.replace(w, hadamard_block=args.hadamard_block)
    total = args.warmup + args.steps + 12

    print("bench: building %d int4 caches for %s" % (args.caches, w.name), file=sys.stderr, flush=True)
    b = Bench(w, "int4", args.caches, total, device, args.decode_waves)
    for _ in range(args.warmup):
        b.step()
    el, toks = b.timed(args.steps)
    split_s, merge_s, append_s, bytes_per_launch = b.profiled(12)
    achieved = bytes_per_launch / split_s / 1e9
    traffic = measured_traffic(w.name, "int4")
    kvtok_step = toks / args.steps
    result = {
        "metric": METRIC,
        "value": toks / el,
        "unit": "kv-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "kv_heads": w.num_kv_heads, "q_heads": w.num_q_heads,
                   "head_dim": w.head_dim, "context": "%s%s" % (w.lengths_kind, list(w.length_args)),
                   "sinks": w.num_sinks, "recent": w.num_recent, "hadamard_block": w.hadamard_block,
                   "kv_storage": "int4 pages + int8 sink/recent", "distinct_caches": args.caches,
                   "kv_tokens_per_step": kvtok_step},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "decode_split_kernel<128,4,INT4_PROT>", "avg_launch_us": split_s * 1e6,
                     "algorithmic_bytes_per_launch": bytes_per_launch},
        "step_breakdown_us": {"append": append_s * 1e6, "decode_split": split_s * 1e6, "decode_merge": merge_s * 1e6},
    }
    del b
    torch.cuda.empty_cache()

    base = {}
    for fmt in [f for f in args.baselines.split(",") if f]:
        print("bench: baseline %s" % fmt, file=sys.stderr, flush=True)
        bb = Bench(w, fmt, args.caches, args.warmup + 2 * args.baseline_steps, device, args.decode_waves)
        for _ in range(args.warmup):
            bb.step()
        el2, toks2 = bb.timed(args.baseline_steps)
        s2, m2, a2, by2 = bb.profiled(args.baseline_steps)
        ach2 = by2 / s2 / 1e9
        base[fmt] = {"kv_tokens_per_s": toks2 / el2, "ms_per_step": el2 / args.baseline_steps * 1e3,
                     "split_avg_us": s2 * 1e6, "achieved_GBps": ach2, "frac": ach2 / HBM_PEAK_GBPS,
                     "int4_speedup": (toks / el) / (toks2 / el2)}
        del bb
        torch.cuda.empty_cache()
    if base:
        result["baselines"] = base
    if args.copy_calibration:
        result["copy_probe_GBps"] = copy_probe(device)
    if not args.no_quality:
        print("bench: quality diagnostic", file=sys.stderr, flush=True)
        result["quality"] = quality(w, device)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_baseline_seconds, device)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
