"""The allocation-free decode entry point (kv4_decode_attention_noalloc, device scratch held by the
library) against kv4_decode_attention on the same calls: identical output bits, and within the
tolerance of the fp64 oracle.  Two calls in a row, the second with fewer sequences and shorter
contexts, so that the scratch holds the first call's partials when the second runs."""
import numpy as np
import pytest
import torch

import int4_kv_cache_fwht_amd as kv4
import kv4_inputs as W
from tests.pair import Pair, TOL

pytestmark = pytest.mark.gpu


def test_noalloc_decode_matches_workspace_decode():
    print("CASE noalloc decode", flush=True)
    hq, hkv, d = 32, 8, 128
    lens = [1, 17, 133, 300, 1000, 4000, 2500, 64]
    p = Pair(hq, hkv, d, num_pages=1024, max_seqs=16, max_pps=256, S=4, R=128, b=128)
    ch = W.outlier_channels(hkv, d, 4, 83)
    ks, vs = zip(*[W.seq_kv(hkv, d, L, ch, 10.0, 83, 0, i, "cuda") for i, L in enumerate(lens)])
    p.append(list(range(len(lens))), lens, torch.cat(ks).contiguous(), torch.cat(vs).contiguous())
    calls = [list(range(len(lens))), [2, 0, 7]]      # the second call is smaller
    for step, ids in enumerate(calls):
        q = W.queries(len(ids), hq, d, 85, step=step, device="cuda")
        ref_ws, ref_ora = p.decode(ids, q)
        out = torch.full((len(ids), hq, d), float("nan"), dtype=torch.float32, device="cuda")
        p.gpu.decode_attention_noalloc(ids, q, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        print("  call", step, "sequences", ids, "max-abs vs oracle", np.abs(got - ref_ora).max(), flush=True)
        assert np.array_equal(got, ref_ws)
        assert np.abs(got - ref_ora).max() <= TOL


def test_noalloc_limits():
    print("CASE noalloc limits", flush=True)
    hq, hkv, d = 8, 2, 64
    cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=400, max_seqs=300, max_pages_per_seq=2,
                     num_sinks=0, num_recent=0, hadamard_block=64)
    c = kv4.Cache(cfg, "cuda")
    k, v = W.seq_kv(hkv, d, 300, None, 1.0, 3, 0, 0, "cuda")
    c.append(list(range(300)), [1] * 300, k, v)
    q = W.queries(300, hq, d, 3, device="cuda")
    out = torch.empty((300, hq, d), dtype=torch.float32, device="cuda")
    with pytest.raises(kv4.KV4Error) as e:
        c.decode_attention_noalloc(list(range(300)), q, out)   # more than 256 sequences
    assert e.value.name == "KV4_ERR_UNSUPPORTED"
    # 256 sequences are fine
    ref = c.decode_attention(list(range(256)), q[:256].contiguous())
    o2 = torch.empty((256, hq, d), dtype=torch.float32, device="cuda")
    c.decode_attention_noalloc(list(range(256)), q[:256].contiguous(), o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref)
