"""CPU checks of the host side of libkv4: the C ABI loads and exports every function that
``include/kv4.h`` declares, configuration checks and buffer sizes follow the documented layout, and
the host planner (FIFO page allocator, block tables, append tasks, decode work list) agrees with the
oracle's allocator on seeded random call sequences.  No GPU call is made."""
import ctypes
import glob
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv4.h")
CSRC = os.path.join(ROOT, "int4_kv_cache_fwht_amd", "csrc")
LIB = os.path.join(ROOT, "int4_kv_cache_fwht_amd", "libkv4.so")


@pytest.fixture(scope="module")
def libkv4():
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location("kv4_build", os.path.join(ROOT, "int4_kv_cache_fwht_amd",
                                                                                 "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    import int4_kv_cache_fwht_amd as kv4
    return kv4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return sorted(set(re.findall(r"\b(kv4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("kv4_buffer_sizes_query", "kv4_cache_create", "kv4_cache_destroy", "kv4_append",
                 "kv4_decode_workspace_size", "kv4_decode_attention", "kv4_seq_free", "kv4_seq_length",
                 "kv4_block_table", "kv4_status_string", "kv4_last_error"):
        assert must in names


def test_library_exports_every_declared_function(libkv4):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], check=True, capture_output=True, text=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert getattr(L, n) is not None


def test_status_strings(libkv4):
    L = libkv4.lib()
    for code, name in libkv4.STATUS.items():
        s = L.kv4_status_string(code)
        assert s is not None and name.encode() in s
    assert L.kv4_status_string(99) is not None


def _documented_sizes(hq, hkv, d, num_pages, max_seqs, max_pps, S, R, fmt):
    """Sizes from the layout the header documents: an INT4 page block is 16 slots x (D/2 bytes of K
    codes + D/2 of V codes + 4 fp16 scale/zero); an INT8 tile is two such-shaped blocks (D/2 bytes of
    K + 8 slots x D bytes of V ... per block, scales in both); a bf16 page 16 x 2D bf16; INT8
    protection tiles per (sequence, kv head) = ceil((S + R) / 16)."""
    int8_tile = 2 * (16 * (d // 2 + d // 2 + 8))
    if fmt == 0:
        block = 16 * (d // 2 + d // 2 + 8)
    elif fmt == 1:
        block = int8_tile
    else:
        block = 16 * 2 * d * 2
    tiles = math.ceil((S + R) / 16) if (fmt == 0 and S + R > 0) else 0
    return dict(page_pool=num_pages * hkv * block, int8_pool=max_seqs * hkv * tiles * int8_tile,
                block_table=max_seqs * max_pps * 4, page_block_bytes=block, int8_tiles=tiles)


@pytest.mark.parametrize("hq,hkv,d,S,R,b,fmt", [
    (32, 8, 128, 4, 128, 128, 0), (2, 1, 64, 4, 32, 32, 0), (8, 8, 128, 0, 0, 1, 0), (8, 2, 64, 1, 0, 64, 0),
    (32, 8, 128, 4, 128, 128, 1), (32, 8, 128, 4, 128, 1, 2), (4, 4, 64, 3, 17, 16, 0)])
def test_buffer_sizes_follow_documented_layout(libkv4, hq, hkv, d, S, R, b, fmt):
    cfg = libkv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=1000, max_seqs=17,
                        max_pages_per_seq=33, num_sinks=S, num_recent=R, hadamard_block=b, format=fmt)
    z = libkv4.kv4_buffer_sizes_query(cfg)
    want = _documented_sizes(hq, hkv, d, 1000, 17, 33, S, R, fmt)
    for k, v in want.items():
        assert getattr(z, k) == v, k


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=96, hadamard_block=32), 5), (dict(page_size=32), 5), (dict(num_q_heads=12, num_kv_heads=8), 1),
    (dict(num_q_heads=64, num_kv_heads=8), 5), (dict(hadamard_block=48), 1), (dict(hadamard_block=256), 1),
    (dict(format=3), 1), (dict(num_sinks=-1), 1), (dict(max_seqs=0), 1), (dict(num_kv_heads=0), 1),
    (dict(eviction=2), 1), (dict(eviction=-1), 1), (dict(eviction=1, format=1), 1), (dict(eviction=1, format=2), 1)])
def test_invalid_configs_are_rejected(libkv4, change, status):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, num_pages=64, max_seqs=4, max_pages_per_seq=16,
                num_sinks=4, num_recent=128, hadamard_block=128, format=0)
    base.update(change)
    cfg = libkv4.Config(**base)
    with pytest.raises(libkv4.KV4Error) as e:
        libkv4.kv4_buffer_sizes_query(cfg)
    assert e.value.status == status
    # cache creation checks the same before touching the device
    from int4_kv_cache_fwht_amd._binding import _Buffers
    L = libkv4.lib()
    h = ctypes.c_void_p()
    bufs = _Buffers(256, 256, 256)
    rc = L.kv4_cache_create(ctypes.byref(cfg.to_c()), ctypes.byref(bufs), ctypes.byref(h))
    assert rc == status and not h.value


def test_null_arguments(libkv4):
    L = libkv4.lib()
    assert L.kv4_cache_create(None, None, None) == 1
    assert L.kv4_cache_destroy(None) == 1
    assert L.kv4_buffer_sizes_query(None, None) == 1
    assert L.kv4_last_error(None) is not None


# ------------------------------------------------------------------------------------------------
# the host planner (kv4_plan.hpp) through a small host-only driver program
# ------------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_driver")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-I", CSRC, "-o", exe,
                    os.path.join(ROOT, "tests", "plan_driver.cpp")], check=True)
    return exe


class Planner:
    def __init__(self, exe):
        self.p = subprocess.Popen([exe], stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True, bufsize=1)

    def _line(self):
        return self.p.stdout.readline().split()

    def cmd(self, s, block=False):
        self.p.stdin.write(s + "\n")
        self.p.stdin.flush()
        first = self._line()
        rows = []
        if block:
            while True:
                r = self._line()
                if r[0] == "end":
                    break
                rows.append([int(x) for x in r[1:]])
        return first, rows

    def close(self):
        self.p.stdin.close()
        self.p.wait(timeout=10)


def _protected(t, L, S, R):
    return t < min(S, L) or max(S, L - R) <= t < L


def _check_tasks(tasks, calls, lens_before, P):
    """Tasks cover each appended position once, in call order; rows are consecutive; a task stays in
    one page and is flagged new exactly when it starts a page."""
    row = 0
    it = iter(tasks)
    for sid, n in calls:
        t = lens_before[sid]
        end = t + n
        while t < end:
            seq, page, t0, cnt, row0, len_new, bti, flags = next(it)
            assert (seq, t0, row0, len_new) == (sid, t, row, end)
            assert 1 <= cnt <= P and t0 // P == (t0 + cnt - 1) // P and (t0 + cnt == end or (t0 + cnt) % P == 0)
            assert flags == (1 if t0 % P == 0 else 0)
            t += cnt
            row += cnt
    assert next(it, None) is None


@pytest.mark.parametrize("seed,S,R,fmt", [(0, 4, 128, 0), (1, 4, 32, 0), (2, 0, 0, 0), (3, 4, 128, 1),
                                           (4, 1, 0, 2), (5, 0, 7, 0)])
def test_planner_matches_oracle_allocator(driver, seed, S, R, fmt):
    rng = np.random.default_rng(seed)
    hq, hkv, d, P, num_pages, max_seqs, max_pps = 8, 2, 64, 16, 90, 6, 24
    pl = Planner(driver)
    assert pl.cmd("init %d %d %d %d %d %d %d %d %d %d %d" % (hq, hkv, d, P, num_pages, max_seqs, max_pps, S, R, 64,
                                                           fmt))[0] == ["status", "0"]
    ora = oracle.OracleCache(hq, hkv, d, P, num_pages, max_seqs, max_pps, S, R, 64, fmt)
    lens = [0] * max_seqs
    for step in range(300):
        op = rng.random()
        if op < 0.6:
            k = int(rng.integers(1, max_seqs + 1))
            ids = [int(x) for x in rng.permutation(max_seqs)[:k]]
            nn = [int(rng.choice([0, 1, 1, 1, 5, 16, 17, 40, 100, 300])) for _ in ids]
            if rng.random() < 0.05:
                ids[-1] = ids[0]  # duplicate id: rejected
            (hdr, rows) = pl.cmd("append %d %s" % (len(ids), " ".join("%d %d" % x for x in zip(ids, nn))), True)
            st = int(hdr[1])
            want = ora.append(ids, nn, None, None)
            assert st == want, (step, ids, nn)
            if st == 0:
                _check_tasks(rows, list(zip(ids, nn)), lens, P)
                for i, n in zip(ids, nn):
                    lens[i] += n
        elif op < 0.75:
            sid = int(rng.integers(0, max_seqs))
            assert int(pl.cmd("free %d" % sid)[0][1]) == ora.seq_free(sid) == 0
            lens[sid] = 0
        else:
            ids = [int(x) for x in rng.permutation(max_seqs)[:int(rng.integers(1, max_seqs + 1))]]
            (hdr, units) = pl.cmd("decode %d %s" % (len(ids), " ".join(map(str, ids))), True)
            if any(lens[i] == 0 for i in ids):
                assert int(hdr[1]) == 3
                continue
            assert int(hdr[1]) == 0
            _check_units(units, ids, lens, hkv, S, R, fmt, int(hdr[3]), int(hdr[5]))
        assert int(pl.cmd("freepages")[0][1]) == ora.free_pages()
        for sid in range(max_seqs):
            b = pl.cmd("bt %d" % sid)[0]
            assert int(b[1]) == ora.seq_length(sid) == lens[sid]
            assert [int(x) for x in b[2:]] == ora.block_table(sid).tolist()
    pl.close()


def _check_units(units, ids, lens, hkv, S, R, fmt, total, start):
    """One unit per (entry, kv head), entry-major, with step ranges that tile [0, total).  Each range
    is the start charge (`start` steps without work, a small constant) and then the work steps: the
    INT4 steps of a protected-format unit cover the pages of every unprotected position at 4 pages a
    step; its INT8 steps cover the S + R protection slots at 32 a step."""
    assert 0 <= start <= 8
    assert len(units) == len(ids) * hkv
    pos = 0
    for e, sid in enumerate(ids):
        L = lens[sid]
        if fmt == 0:
            pages = sorted(set(t // 16 for t in range(L) if not _protected(t, L, S, R)))
            if pages:
                assert pages == list(range(pages[0], pages[-1] + 1))
            steps = math.ceil(len(pages) / 4) + (math.ceil((S + R) / 32) if S + R > 0 else 0)
        elif fmt == 1:
            steps = math.ceil(math.ceil(L / 16) / 2)
        else:
            steps = math.ceil(L / 16)
        for h in range(hkv):
            seq, ln, entry, head, begin = units[e * hkv + h]
            assert (seq, ln, entry, head, begin) == (sid, L, e, h, pos)
            pos += start + steps
    assert pos == total


def test_planner_out_of_pages_changes_nothing(driver):
    pl = Planner(driver)
    pl.cmd("init 4 2 64 16 10 4 16 4 32 64 0")
    assert pl.cmd("append 1 0 33", True)[0] == ["status", "0"]          # 3 pages
    assert pl.cmd("append 2 1 80 2 40", True)[0] == ["status", "2"]     # 5 + 3 > 7
    assert pl.cmd("freepages")[0] == ["free", "7"]
    assert pl.cmd("bt 1")[0] == ["bt", "0"]
    assert pl.cmd("append 2 1 80 2 32", True)[0] == ["status", "0"]     # 5 + 2 = 7
    assert pl.cmd("freepages")[0] == ["free", "0"]
    pl.close()


def _resource_reports():
    """Per-kernel (VGPRs, scratch bytes per lane, occupancy) from the compiler's reports that
    int4_kv_cache_fwht_amd/build.py keeps beside each kernel object."""
    out = {}
    for path in glob.glob(os.path.join(ROOT, "int4_kv_cache_fwht_amd", "_build", "*.resources.txt")):
        name = None
        for line in open(path):
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                out[name] = {}
                continue
            for key, pat in (("vgprs", r"\bVGPRs: (\d+)"), ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                             ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)")):
                m = re.search(pat, line)
                if m and name:
                    out[name][key] = int(m.group(1))
    return out


def test_kernels_use_no_scratch(libkv4):
    """No kernel spills registers to scratch (private) memory, and the two hot split kernels keep
    at least 2 waves per SIMD (their latency hiding depends on it)."""
    rep = _resource_reports()
    assert len(rep) >= 40, sorted(rep)[:5]
    spills = {k: v for k, v in rep.items() if v.get("scratch", 0) != 0}
    assert not spills, spills
    for k, v in rep.items():
        if "decode_split_kernel" in k or "mq_split_kernel" in k:
            assert v["occupancy"] >= 2, (k, v)


def test_no_bit_cast_of_vector_element_lvalue():
    """hipcc mistranslates a bit cast whose whole argument is one element of an ext_vector
    (`__builtin_bit_cast(half2_t, q[1])` read element 0 of q).  Device code passes such elements
    through a function parameter or an expression instead; this keeps the pattern out."""
    csrc = os.path.join(ROOT, "int4_kv_cache_fwht_amd", "csrc")
    pat = re.compile(r"__builtin_bit_cast\(\s*[\w:]+\s*,\s*[\w.]+(\[[^\]\[]*\])+\s*\)")
    bad = []
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cuh", ".h", ".hpp")):
            with open(os.path.join(csrc, name)) as f:
                for i, line in enumerate(f, 1):
                    if pat.search(line):
                        bad.append("%s:%d: %s" % (name, i, line.strip()))
    assert not bad, bad


def test_fma_with_unit_factor_is_the_add_or_subtract():
    """The kernels' lane-exchange butterflies compute x' + x and x' - x as fmaf(+-1, x, x'): the
    product by +-1 is exact, so the fma rounds once, like the add or subtract.  Checked here
    bit for bit with the C library's fmaf over random, subnormal, signed-zero and large values."""
    import ctypes
    import ctypes.util
    import numpy as np
    libm = ctypes.CDLL(ctypes.util.find_library("m"))
    libm.fmaf.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
    libm.fmaf.restype = ctypes.c_float
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(2000).astype(np.float32))
    vals += list((rng.standard_normal(500) * 1e-40).astype(np.float32))  # subnormals
    vals += list((rng.standard_normal(500) * 1e37).astype(np.float32))
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(1.0), np.float32(-1.0)]
    vals = np.array(vals, dtype=np.float32)
    a = vals
    b = np.roll(vals, 17)
    with np.errstate(over="ignore", invalid="ignore"):
        for x, y in zip(a, b):
            for sgn, ref in ((1.0, np.float32(y) + np.float32(x)), (-1.0, np.float32(y) - np.float32(x))):
                got = np.float32(libm.fmaf(sgn, float(x), float(y)))
                assert got.tobytes() == np.float32(ref).tobytes() or (np.isnan(got) and np.isnan(ref)), (x, y, sgn)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 ends with a message, before any GPU work."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
