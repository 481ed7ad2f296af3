#!/usr/bin/env python3
"""Decode-step benchmark of the INT4 KV cache on one MI355X.

Default workload: the asynchronous-rollout regime -- 256 sequences with lognormal context lengths
(median 4096, clipped to [256, 32768]) at Qwen3-8B attention shapes, where one step is 36
identical-shape layers run in sequence.  Each layer has its own cache (36 distinct caches, about
1.9 GB each, so no layer's reads are served by the 256 MB last-level cache).  Per layer the step
appends one new position to every sequence (fused rotation + quantization into the paged cache,
INT8 protection of the newest positions) and then runs GQA decode attention over every sequence's
full context.  The timed region holds exactly --steps steps bracketed by device
synchronization; inputs are resident in HBM.

Prints ONE JSON line.
- value = kv-tokens/s = (sum of context lengths attended per layer) x layers x steps / wall time.
- roofline = the decode split-KV kernel's algorithmic bytes per launch / its mean duration over
  >= 50 back-to-back decode-only launches (kernel-stamped HIP events on the call's stream), against
  the 8 TB/s HBM peak and against the probed streaming-read ceiling of the device.
- baselines = the same workload with INT8-only and bf16 KV caches (pools of 4 distinct caches).
- workloads = the Qwen3-8B layer (64 sequences, 1K-8K), long context (8 x 131072) and one GPU's
  share of the rollout regime under 8-way tensor parallelism by kv head (1 kv head, 4 q heads).
- append = the append path alone, Hadamard block 128 against 1 (rotation overhead).
- protection_cost = decode split time and bytes at (S, R) = (0, 0), (4, 0), (0, 128), (4, 128).
- cpu_baseline = the CPU oracle's decode on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
METRIC = "INT4-KV decode attention kv-tokens/s and achieved HBM GB/s (% of MI355X peak)"
FORMATS = {"int4": 0, "int8": 1, "bf16": 2}
KERNELS = {"int4": "decode_split_kernel<128,4,INT4_PROT>", "int8": "decode_split_kernel<128,4,INT8>",
           "bf16": "decode_split_kernel<128,4,BF16>"}
DTYPE = "fp16 MFMA operands (u4/u8 codes exact, query hi+lo), fp32 softmax and accumulation"
EXTRAS = ("probe", "baselines", "workloads", "append", "protection", "quality", "cpu")


def log(msg):
    print("bench: " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="rollout",
                    choices=["rollout", "qwen3_8b_layer", "long_context", "rollout_tp8", "tiny", "append",
                             "multi_query"],
                    help="decode workloads; 'append': the append path alone at Hadamard block 128 vs 1; "
                         "'multi_query': causal multi-query attention on the Qwen3-8B-shaped layer")
    ap.add_argument("--layers", type=int, default=0, help="layers per step (0: the workload's, 36 for rollout)")
    ap.add_argument("--caches", type=int, default=0,
                    help="distinct layer caches (0: one per layer, at least 4, so no cache fits the 256 MB MALL)")
    ap.add_argument("--decode-launches", type=int, default=72, help="back-to-back decode-only launches timed")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma list of %s, or 'none'" % ",".join(EXTRAS))
    ap.add_argument("--baselines", default="int8,bf16", help="comma list of baseline formats")
    ap.add_argument("--baseline-caches", type=int, default=4)
    ap.add_argument("--mq-rows", type=int, default=4, help="query rows per sequence of the multi_query workload")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--decode-waves", type=int, default=0)
    ap.add_argument("--hadamard-block", type=int, default=0,
                    help="override the workload's Hadamard block (1 = plain INT4: no q / output rotation)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU run: write the measured decode traffic from two rocprofv3 --pmc output folders")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB probe copy (the reference kernel for PMC byte counters)")
    a = ap.parse_args()
    a.extras = set() if a.extras in ("", "none") else set(a.extras.split(","))
    bad = a.extras - set(EXTRAS)
    if bad:
        ap.error("unknown extras: %s" % ",".join(sorted(bad)))
    return a


def per_token_bytes(fmt, hkv, d):
    """Algorithmic bytes per cached position (all kv heads, K and V)."""
    if fmt == "int4":
        return hkv * 2 * (d // 2 + 4)
    if fmt == "int8":
        return hkv * 2 * (d + 4)
    return hkv * 2 * d * 2


def decode_bytes(fmt, lens, w, sinks=None, recent=None):
    """Algorithmic HBM bytes of one decode launch: cached positions read once (INT4 pages for
    unprotected positions, INT8 for the protected ones), block-table entries, q in, out out."""
    hkv, d, hq = w.num_kv_heads, w.head_dim, w.num_q_heads
    S = w.num_sinks if sinks is None else sinks
    R = w.num_recent if recent is None else recent
    b4, b8 = per_token_bytes("int4", hkv, d), per_token_bytes("int8", hkv, d)
    total = 0
    for L in lens:
        if fmt == "int4":
            p = min(L, S + R)
            total += (L - p) * b4 + p * b8
        else:
            total += L * per_token_bytes(fmt, hkv, d)
        total += math.ceil(L / 16) * 4 + hq * d * 2 + hq * d * 4
    return total


def stats_us(ms_list):
    us = [x * 1e3 for x in ms_list]
    return {"mean": statistics.fmean(us), "median": statistics.median(us), "min": min(us), "max": max(us),
            "launches": len(us)}


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
    """n_caches distinct layer caches of one workload; a step runs `layers` layers, layer j of step s
    on cache (s * layers + j) % n_caches: append one position to every sequence, then decode."""

    def __init__(self, w, fmt, n_caches, layers, total_steps, device, decode_waves, sinks=None, recent=None):
        import torch
        import int4_kv_cache_fwht_amd as kv4
        import kv4_inputs as W
        self.torch, self.kv4, self.W = torch, kv4, W
        self.w, self.fmt, self.device, self.layers = w, fmt, device, layers
        self.S = w.num_sinks if sinks is None else sinks
        self.R = w.num_recent if recent is None else recent
        self.lens0 = w.lengths()
        B = w.batch
        growth = math.ceil(total_steps * layers / n_caches) + 1
        max_len = max(self.lens0) + growth
        pages = sum(math.ceil((L + growth) / 16) for L in self.lens0) + B
        self.channels = W.outlier_channels(w.num_kv_heads, w.head_dim, w.outlier_channels, w.seed)
        self.caches, self.lens = [], []
        for c in range(n_caches):
            cfg = kv4.Config(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                             num_pages=pages, max_seqs=B, max_pages_per_seq=math.ceil(max_len / 16) + 1,
                             num_sinks=self.S if fmt == "int4" else 0, num_recent=self.R if fmt == "int4" else 0,
                             hadamard_block=w.hadamard_block if fmt != "bf16" else 1, format=FORMATS[fmt])
            cache = kv4.Cache(cfg, device)
            if decode_waves:
                cache.set_decode_waves(decode_waves)
            self._prefill(cache, layer=c)
            self.caches.append(cache)
            self.lens.append(list(self.lens0))
        self.ids = list(range(B))
        # per-(step, layer) inputs, resident before timing
        self.kn, self.vn, self.q = [], [], []
        for s in range(total_steps):
            for j in range(layers):
                k, v = W.seq_kv(w.num_kv_heads, w.head_dim, B, self.channels, w.outlier_scale, w.seed,
                                1000 + s * layers + j, 0, device)
                self.kn.append(k)
                self.vn.append(v)
                self.q.append(W.queries(B, w.num_q_heads, w.head_dim, w.seed, layer=j, step=s, device=device))
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
        """One step (all its layers); returns the kv-tokens attended and the per-layer lengths."""
        s = self.step_idx
        toks, lens = 0, []
        for j in range(self.layers):
            c = (s * self.layers + j) % len(self.caches)
            cache = self.caches[c]
            i = s * self.layers + j
            cache.append(self.ids, [1] * len(self.ids), self.kn[i], self.vn[i])
            cache.decode_attention(self.ids, self.q[i], out=self.out)
            self.lens[c] = [L + 1 for L in self.lens[c]]
            toks += sum(self.lens[c])
            lens.append(self.lens[c])
        self.step_idx += 1
        return toks, lens

    def timed(self, steps):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks = 0
        for _ in range(steps):
            toks += self.step()[0]
        torch.cuda.synchronize()
        return time.perf_counter() - t0, toks

    def _profiling(self, on):
        for c in self.caches:
            c.profile_enable(on)

    def _durations(self, kind):
        out = []
        for c in self.caches:
            out += c.profile_durations(kind)
        return out

    def profiled_steps(self, steps):
        """Steps with the library's kernel events on: per-launch append, split and merge durations (ms)."""
        self._profiling(True)
        for _ in range(steps):
            self.step()
        d = {k: self._durations(k) for k in ("append", "split", "merge")}
        self._profiling(False)
        return d

    def decode_only(self, launches):
        """`launches` back-to-back decode calls (no appends), cycling the caches: per-launch split and
        merge durations (ms) and the mean algorithmic bytes per launch."""
        self._profiling(True)
        nbytes = 0
        q = self.q[0]
        for i in range(launches):
            c = i % len(self.caches)
            self.caches[c].decode_attention(self.ids, q, out=self.out)
            nbytes += decode_bytes(self.fmt, self.lens[c], self.w, self.S, self.R)
        d = {k: self._durations(k) for k in ("split", "merge")}
        self._profiling(False)
        return d["split"], d["merge"], nbytes / launches

    def close(self):
        for c in self.caches:
            c.close()
        self.caches = []


def run_decode_workload(w, fmt, n_caches, layers, steps, warmup, launches, device, decode_waves=0, sinks=None,
                        recent=None):
    """Timed steps, then back-to-back decode-only launches.  Returns a record."""
    import torch
    b = Bench(w, fmt, n_caches, layers, warmup + steps + 2, device, decode_waves, sinks, recent)
    for _ in range(warmup):
        b.step()
    el, toks = b.timed(steps)
    prof = b.profiled_steps(2)
    split, merge, bytes_launch = b.decode_only(launches)
    b.close()
    del b
    torch.cuda.empty_cache()
    st = stats_us(split)
    ach = bytes_launch / (st["mean"] * 1e-6) / 1e9
    return {"kv_tokens_per_s": toks / el, "ms_per_step": el / steps * 1e3, "wall_s": el, "kv_tokens": toks,
            "split_us": st, "merge_us": stats_us(merge), "algorithmic_bytes_per_launch": bytes_launch,
            "achieved_GBps": ach, "frac": ach / HBM_PEAK_GBPS,
            "achieved_GBps_median": bytes_launch / (st["median"] * 1e-6) / 1e9,
            "step_kernels_us": {"append": stats_us(prof["append"])["mean"], "split": stats_us(prof["split"])["mean"],
                                "merge": stats_us(prof["merge"])["mean"]}}


def hbm_probe(device, reps=20):
    """Ceiling: hand-written streaming read of a 4 GiB buffer and copy of 2 GiB (median of reps)."""
    import torch
    import int4_kv_cache_fwht_amd as kv4
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=device)
    src.fill_(1)
    dst = torch.empty(n // 2, dtype=torch.uint8, device=device)
    kv4.hbm_probe(0, src, dst, n, 2)  # warm-up
    rd = kv4.hbm_probe(0, src, dst, n, reps)
    cp = kv4.hbm_probe(1, src, dst, n // 2, reps)
    del src, dst
    torch.cuda.empty_cache()
    rmed, cmed = statistics.median(rd), statistics.median(cp)
    return {"read_GBps": n / (rmed * 1e-3) / 1e9, "read_GBps_best": n / (min(rd) * 1e-3) / 1e9,
            "copy_GBps": 2 * (n // 2) / (cmed * 1e-3) / 1e9, "buffer_bytes": n, "reps": reps,
            "kernel": "kv4::probe_read_kernel / probe_copy_kernel (16-byte nontemporal loads, 8 in flight per lane)"}


def cpu_baseline(w, seconds, device):
    """The oracle's decode (fp64, threaded) on a bounded sample of the workload: the first sequences
    of layer 0, decoded repeatedly for about `seconds` of CPU time."""
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
            "sample": "%d sequences (%d positions) of %s layer 0, oracle decode in fp64 repeated %d times (%.1f s); "
                      "the layers are identical in shape, so the rate applies per layer" % (
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
    return {"reference": "exact fp64 attention on the unquantized bf16 K/V of %s, %d sequences (%d positions)" % (
        w.name, len(lens), sum(lens)), "errors": res}


def append_workload(device, repeats=7):
    """The append path alone: 256 empty sequences x 512 single-position steps, and a bulk prefill of
    32768 positions into one sequence (its input rows out of the last-level cache), then the same
    rows into a second sequence (in it), timed with the rotation (b = 128), without it (b = 1,
    plain INT4), and with the fused RoPE of pre-RoPE keys (b = 128); variants interleaved per
    repeat, best (minimum) of the per-repeat means."""
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
    variants = (("b128", 128, False), ("b1", 1, False), ("b128_rope", 128, True))
    res = {name: [[], [], []] for name, _, _ in variants}
    for _ in range(repeats):
        for name, block, rope in variants:
            cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             num_pages=B * (steps // 16) + 2 * (bulk // 16) + 32, max_seqs=B + 2,
                             max_pages_per_seq=bulk // 16 + 1, num_sinks=w.num_sinks, num_recent=w.num_recent,
                             hadamard_block=block, format=0)

            def app(cache, ids, n, k, v):
                if rope:
                    cache.append_rope(ids, n, k, v, cos, sin)
                else:
                    cache.append(ids, n, k, v)

            cache = kv4.Cache(cfg, device)
            ids = list(range(B))
            app(cache, ids, [1] * B, rows[0][0], rows[0][1])  # warm-up of the launch path
            torch.cuda.synchronize()
            for i in ids:
                cache.seq_free(i)
            cache.profile_enable(True)
            for s in range(steps):
                app(cache, ids, [1] * B, rows[s][0], rows[s][1])
            res[name][0].append(statistics.fmean(cache.profile_durations("append")) * 1e3)
            cache.profile_enable(True)
            app(cache, [B], [bulk], kb, vb)
            # the same rows again into another sequence: now they come from the last-level cache, as
            # when a prefill appends the K and V its projection has just written
            app(cache, [B + 1], [bulk], kb, vb)
            dd = cache.profile_durations("append")
            res[name][1].append(dd[0] * 1e3)
            res[name][2].append(dd[1] * 1e3)
            cache.profile_enable(False)
            cache.close()
    best = {k: (min(v[0]), min(v[1]), min(v[2])) for k, v in res.items()}
    (s128, b128, w128), (s1, b1, w1), (sr, br, wr) = best["b128"], best["b1"], best["b128_rope"]
    bulk_bytes = bulk * hkv * d * 2 * 2 + bulk * hkv * 2 * (d // 2 + 4)   # bf16 in, INT4 + scales out
    step_bytes = B * hkv * d * 2 * 2 + B * hkv * 2 * (d // 2 + 4) + B * hkv * 2 * (d + 4)  # + INT8 copy
    return {"config": {"sequences": B, "steps": steps, "bulk_prefill": bulk, "kv_heads": hkv, "head_dim": d,
                       "sinks": w.num_sinks, "recent": w.num_recent},
            "tokens_per_s_b128": B / (s128 * 1e-6),
            "append_step_us": {"b128": s128, "b1": s1, "rotation_overhead": s128 / s1 - 1.0,
                               "b128_fused_rope": sr, "fused_rope_overhead": sr / s128 - 1.0,
                               "GBps_b128": step_bytes / (s128 * 1e-6) / 1e9},
            "bulk_prefill_us": {"b128": b128, "b1": b1, "rotation_overhead": b128 / b1 - 1.0,
                                "GBps_b128": bulk_bytes / (b128 * 1e-6) / 1e9,
                                "frac_b128": bulk_bytes / (b128 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                "b128_fused_rope": br, "fused_rope_overhead": br / b128 - 1.0,
                                "input_rows": "not in the last-level cache (512 steps of other rows since)"},
            "bulk_prefill_warm_us": {"b128": w128, "b1": w1, "rotation_overhead": w128 / w1 - 1.0,
                                     "GBps_b128": bulk_bytes / (w128 * 1e-6) / 1e9,
                                     "frac_b128": bulk_bytes / (w128 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                     "b128_fused_rope": wr, "fused_rope_overhead": wr / w128 - 1.0,
                                     "input_rows": "just read by the cold prefill (134 MB, below the 256 MB "
                                                   "last-level cache), as right after the projection writes them"},
            "algorithmic_bytes": {"bulk_prefill": bulk_bytes, "step": step_bytes},
            "note": "kernel time from kernel-stamped HIP events; per variant the minimum over %d interleaved "
                    "repeats of (mean over the 512 step launches) and of the prefill launch" % repeats}


def protection_cost(device, rounds=6, launches=8, n_caches=4):
    """Decode split time and algorithmic bytes on the Qwen3-8B layer with no protection, sinks only,
    recent window only and both (INT4 + INT8 protection), b = 128.  The four variants' caches are
    built first and their decode-only launches interleaved (rounds x launches each), so that a
    drift of the device's speed during the run falls on all of them alike."""
    import torch
    import kv4_inputs as W
    w = W.WORKLOADS["qwen3_8b_layer"]
    variants = ((0, 0), (4, 0), (0, 128), (4, 128))
    benches = {v: Bench(w, "int4", n_caches, 1, 2, device, 0, sinks=v[0], recent=v[1]) for v in variants}
    split = {v: [] for v in variants}
    nbytes = {}
    for _ in range(rounds):
        for v in variants:
            sp, _, by = benches[v].decode_only(launches)
            split[v] += sp
            nbytes[v] = by
    for b in benches.values():
        b.close()
    torch.cuda.empty_cache()
    out = {}
    for (S, R) in variants:
        st = stats_us(split[(S, R)])
        by = nbytes[(S, R)]
        out["S%d_R%d" % (S, R)] = {"split_us": st["mean"], "split_us_median": st["median"],
                                   "algorithmic_bytes_per_launch": by, "achieved_GBps": by / (st["mean"] * 1e-6) / 1e9,
                                   "frac": by / (st["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBPS}
    base = out["S0_R0"]
    for v in out.values():
        v["time_vs_unprotected"] = v["split_us"] / base["split_us"] - 1.0
        v["bytes_vs_unprotected"] = v["algorithmic_bytes_per_launch"] / base["algorithmic_bytes_per_launch"] - 1.0
    return {"workload": "qwen3_8b_layer", "launches_per_variant": rounds * launches, "order": "interleaved",
            "variants": out}


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
    ab_rounds, ab_steps = 4, 3  # per-wave against workgroup-shared INT4 steps, interleaved
    total = warmup + steps + prof_steps + 2 * ab_rounds * ab_steps
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
    split, merge, app = [], [], []
    for c in caches:
        split += c.profile_durations("mq_split")
        merge += c.profile_durations("mq_merge")
        app += c.profile_durations("append")
        c.profile_enable(False)
    # the same steps with the INT4 steps per wave and shared by the workgroup, in A B B A order
    G = hq // hkv
    shares = -(-n_q * G // 16) % 4 == 0
    ab = {True: [], False: []}
    for r in range(ab_rounds):
        for mode in ((True, False) if r % 2 == 0 else (False, True)):
            for c in caches:
                c.set_mq_share(mode)
                c.profile_enable(True)
            for _ in range(ab_steps):
                one()
            for c in caches:
                ab[mode] += c.profile_durations("mq_split")
                c.profile_enable(False)
    for c in caches:
        c.set_mq_share(True)
    split_s = statistics.fmean(split) * 1e-3
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
    kname = "mq_split_shared_kernel<128,4,INT4_PROT>" if shares else "mq_split_kernel<128,4,INT4_PROT>"
    roof.update({"traffic": None, "kernel": kname, "avg_launch_us": split_s * 1e6,
                 "median_launch_us": statistics.median(split) * 1e3,
                 "algorithmic_bytes_per_launch": bytes_launch, "algorithmic_flops_per_launch": flops_launch,
                 "achieved_GBps": gbps, "achieved_TFLOPs": tflops, "flops_per_byte": intensity})
    return {"metric": "INT4-KV multi-query attention: attended (query row, position) pairs per s", "value":
            attended / el, "unit": "row-positions/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": el / steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": DTYPE, "data": "synthetic",
            "config": {"workload": "multi_query", "batch": B, "query_rows_per_seq": n_q, "kv_heads": hkv,
                       "q_heads": hq, "head_dim": d, "context": "uniform[1024, 8192] + growth", "sinks": w.num_sinks,
                       "recent": w.num_recent, "hadamard_block": w.hadamard_block, "distinct_caches": n_caches},
            "roofline": roof,
            "step_breakdown_us": {"append": statistics.fmean(app) * 1e3, "mq_split": split_s * 1e6,
                                  "mq_merge": statistics.fmean(merge) * 1e3},
            "int4_steps_shared_by_workgroup": shares,
            "split_us_shared_vs_per_wave": {
                "shared": stats_us(ab[True]), "per_wave": stats_us(ab[False]),
                "note": "interleaved A B B A rounds of %d steps; the shared kernel runs only when every "
                        "sequence has a multiple of 4 row tiles, else both are the per-wave kernel" % ab_steps}}


def write_traffic(fetch_dir, write_dir, workload, fmt="int4"):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; both with
    --copy-calibration) into the measured HBM bytes per decode-split launch, each counter scaled by
    what it reads for the 1 GiB probe copy; stores them, keyed by the decode sources' hash, in
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
    copy_f = max(v for k, vs in fetch.items() if "probe_copy_kernel" in k for v in vs)
    copy_w = max(v for k, vs in write.items() if "probe_copy_kernel" in k for v in vs)
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
    cmd = ("rocprofv3 --pmc %s --kernel-include-regex 'decode_split|probe_copy' --output-format csv -d %s -o run -- "
           "python bench.py --workload %s --steps 2 --warmup 1 --decode-launches 8 --extras none --copy-calibration")
    rec["%s/%s" % (workload, fmt)] = {
        "kernel": KERNELS[fmt],
        "kernel_source_hash": kernel_source_hash(),
        "bytes_per_launch": fb + wb, "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
        "fetch_size_kib_mean": sum(f_kib) / len(f_kib), "write_size_kib_mean": sum(w_kib) / len(w_kib),
        "dispatches": len(f_kib),
        "copy_reference": {"kernel": "kv4::probe_copy_kernel", "bytes_read": n, "bytes_written": n,
                           "fetch_size_kib": copy_f, "write_size_kib": copy_w, "fetch_factor": ff,
                           "write_factor": wf},
        "commands": [cmd % ("FETCH_SIZE", fetch_dir, workload), cmd % ("WRITE_SIZE", write_dir, workload),
                     "python bench.py --workload %s --traffic-from %s %s" % (workload, fetch_dir, write_dir)],
    }
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec["%s/%s" % (workload, fmt)]


def copy_calibration(device):
    """One 1 GiB probe copy: the reference dispatch for the PMC byte counters."""
    import torch
    import int4_kv_cache_fwht_amd as kv4
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device=device)
    b = torch.empty_like(a)
    ms = kv4.hbm_probe(1, a, b, n, 1)[0]
    del a, b
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def workload_config(w, layers, n_caches, fmt="int4"):
    return {"workload": w.name, "batch": w.batch, "layers_per_step": layers, "kv_heads": w.num_kv_heads,
            "q_heads": w.num_q_heads, "head_dim": w.head_dim,
            "context": "%s%s" % (w.lengths_kind, list(w.length_args)), "sinks": w.num_sinks,
            "recent": w.num_recent, "hadamard_block": w.hadamard_block,
            "kv_storage": {"int4": "int4 pages + int8 sink/recent", "int8": "int8 pages",
                           "bf16": "bf16 pages"}[fmt],
            "distinct_caches": n_caches, "seed": w.seed}


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(write_traffic(args.traffic_from[0], args.traffic_from[1], args.workload)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: the decode path is built and measured on one GPU "
              "(multi-GPU sharding is not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import dataclasses
    import torch
    import kv4_inputs as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda", 0)
    if args.workload == "append":
        rec = append_workload(device)
        if args.copy_calibration:
            rec["copy_calibration_GBps"] = copy_calibration(device)
        print(json.dumps({"metric": "INT4 KV append (rotation + quantization + pack) tokens/s",
                          "value": rec["tokens_per_s_b128"], "unit": "tokens/s", "n_gpus": 1, "steps": 512,
                          "warmup": 1, "ms_per_step": rec["append_step_us"]["b128"] * 1e-3, "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                          "config": dict(rec["config"], workload="append"), "append": rec}), flush=True)
        return
    if args.workload == "multi_query":
        print(json.dumps(mq_workload(device, args.mq_rows, args.steps, args.warmup)), flush=True)
        return
    w = W.WORKLOADS[args.workload]
    if args.hadamard_block:
        w = dataclasses.replace(w, hadamard_block=args.hadamard_block)
    layers = args.layers or w.layers
    n_caches = args.caches or max(layers, 4)

    log("building %d int4 layer caches for %s (%d layers per step)" % (n_caches, w.name, layers))
    b = Bench(w, "int4", n_caches, layers, args.warmup + args.steps + 2, device, args.decode_waves)
    for _ in range(args.warmup):
        b.step()
    el, toks = b.timed(args.steps)
    log("timed %d steps in %.3f s" % (args.steps, el))
    prof = b.profiled_steps(2)
    split, merge, bytes_launch = b.decode_only(args.decode_launches)
    b.close()
    del b
    torch.cuda.empty_cache()
    st = stats_us(split)
    achieved = bytes_launch / (st["mean"] * 1e-6) / 1e9
    traffic = measured_traffic(w.name, "int4")
    layer_wall_us = el / (args.steps * layers) * 1e6
    kern = {"append": stats_us(prof["append"])["mean"], "decode_split": stats_us(prof["split"])["mean"],
            "decode_merge": stats_us(prof["merge"])["mean"]}
    kern_sum = sum(kern.values())
    # the kernels of one stream cannot take longer than the wall clock around them; a violation
    # means the events over-count (seen under a kernel tracer, which lengthens short kernels)
    events_ok = kern_sum <= layer_wall_us
    if not events_ok:
        log("warning: kernel events per layer (%.1f us) exceed the wall-clock layer step (%.1f us)" % (
            kern_sum, layer_wall_us))
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
        "dtype": DTYPE,
        "data": "synthetic",
        "config": dict(workload_config(w, layers, n_caches), kv_tokens_per_step=toks / args.steps),
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "kernel": KERNELS["int4"],
                     "avg_launch_us": st["mean"], "median_launch_us": st["median"], "min_launch_us": st["min"],
                     "max_launch_us": st["max"], "launches": st["launches"],
                     "timing": "kernel-stamped HIP events of %d back-to-back decode-only launches cycling the %d "
                               "layer caches" % (st["launches"], n_caches),
                     "algorithmic_bytes_per_launch": bytes_launch},
        "step_breakdown_us": {"per_layer": kern, "kernels_sum_per_layer": kern_sum, "wall_per_layer": layer_wall_us,
                              "per_step_kernels": kern_sum * layers, "kernels_within_wall": events_ok},
    }
    ex = args.extras
    if "probe" in ex:
        log("HBM probe")
        pr = hbm_probe(device)
        result["roofline"]["probe"] = pr
        result["roofline"]["frac_of_probe_read"] = achieved / pr["read_GBps"]
    if "baselines" in ex:
        base = {}
        for fmt in [f for f in args.baselines.split(",") if f]:
            log("baseline %s (%d caches cycled)" % (fmt, args.baseline_caches))
            r = run_decode_workload(w, fmt, args.baseline_caches, layers, max(args.steps // 2, 4), 1,
                                    args.decode_launches, device, args.decode_waves)
            r["int4_speedup_kv_tokens"] = result["value"] / r["kv_tokens_per_s"]
            r["int4_split_speedup"] = r["split_us"]["mean"] / st["mean"]
            r["kernel"] = KERNELS[fmt]
            r["distinct_caches"] = args.baseline_caches
            base[fmt] = r
        result["baselines"] = base
    if "workloads" in ex:
        wl = {}
        for name in ("qwen3_8b_layer", "long_context", "rollout_tp8"):
            if name == w.name:
                continue
            log("workload %s" % name)
            w2 = W.WORKLOADS[name]
            r = run_decode_workload(w2, "int4", 4, 1, 12, 2, 64, device, args.decode_waves)
            r["config"] = workload_config(w2, 1, 4)
            r["traffic"] = measured_traffic(name, "int4")
            if "probe" in result["roofline"]:
                r["frac_of_probe_read"] = r["achieved_GBps"] / result["roofline"]["probe"]["read_GBps"]
            wl[name] = r
        result["workloads"] = wl
    if "append" in ex:
        log("append workload")
        result["append"] = append_workload(device)
    if "protection" in ex:
        log("protection cost")
        result["protection_cost"] = protection_cost(device)
    if args.copy_calibration:
        result["copy_calibration_GBps"] = copy_calibration(device)
    if "quality" in ex:
        log("quality diagnostic")
        result["quality"] = quality(W.WORKLOADS["qwen3_8b_layer"], device)
    if "cpu" in ex:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_baseline_seconds, device)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
