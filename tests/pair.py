"""A HIP-path cache and an oracle cache driven with the same calls, plus their comparison."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import int4_kv_cache_fwht_amd as kv4
from kv4_inputs import bf16_bits
from tests import kv4_layout

TOL = 2e-3  # max-abs error of decode outputs against the fp64 oracle on the same dequantized cache


class Pair:
    def __init__(self, hq, hkv, d, num_pages, max_seqs, max_pps, S=4, R=128, b=128, fmt=kv4.FORMAT_INT4_PROT,
                 device="cuda", eviction=kv4.EVICT_DUAL_WRITE):
        self.cfg = kv4.Config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, num_pages=num_pages, max_seqs=max_seqs,
                              max_pages_per_seq=max_pps, num_sinks=S, num_recent=R, hadamard_block=b, format=fmt,
                              eviction=eviction)
        self.gpu = kv4.Cache(self.cfg, device)
        self.ora = oracle.OracleCache(hq, hkv, d, 16, num_pages, max_seqs, max_pps, S, R, b, fmt, eviction=eviction)
        self.hq, self.hkv, self.d, self.S, self.R, self.b, self.fmt = hq, hkv, d, S, R, b, fmt

    def append(self, seq_ids, n_new, k, v):
        self.gpu.append(seq_ids, n_new, k, v)
        rows = int(sum(n_new))
        kb = bf16_bits(k) if rows else None
        vb = bf16_bits(v) if rows else None
        rc = self.ora.append(seq_ids, n_new, kb, vb)
        assert rc == oracle.OK, rc

    def append_rope(self, seq_ids, n_new, k, v, cos, sin):
        """cos, sin: float32 numpy tables [positions, d/2] (copied to the device for the GPU side)."""
        self.gpu.append_rope(seq_ids, n_new, k, v, torch.from_numpy(cos).to(k.device),
                             torch.from_numpy(sin).to(k.device))
        rc = self.ora.append_rope(seq_ids, n_new, bf16_bits(k), bf16_bits(v), cos, sin)
        assert rc == oracle.OK, rc

    def seq_free(self, seq):
        self.gpu.seq_free(seq)
        assert self.ora.seq_free(seq) == oracle.OK

    def decode(self, seq_ids, q, scale=0.0):
        out = self.gpu.decode_attention(seq_ids, q, scale=scale)
        ref, _ = self.ora.decode(seq_ids, bf16_bits(q), scale=scale)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), ref

    def multi(self, seq_ids, n_q, q, scale=0.0):
        out = self.gpu.multi_query_attention(seq_ids, n_q, q, scale=scale)
        ref, _ = self.ora.attend_multi(seq_ids, n_q, bf16_bits(q), scale=scale)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), ref

    def compare_cache(self, seqs):
        """Bit-exact comparison of page ids, codes and scales (valid slots only).  Returns the number
        of compared (slot, kv, head) records."""
        torch.cuda.synchronize()
        sz = self.gpu.sizes
        pool = self.gpu.page_pool.cpu().numpy()[: sz.page_pool].reshape(self.cfg.num_pages, self.hkv,
                                                                       sz.page_block_bytes)
        bt_dev = self.gpu.block_table_dev.cpu().numpy()
        i8 = None
        if self.fmt == kv4.FORMAT_INT4_PROT and sz.int8_pool:
            i8 = self.gpu.int8_pool.cpu().numpy().reshape(self.cfg.max_seqs, self.hkv, sz.int8_tiles,
                                                          sz.int8_tile_bytes)
        compared = 0
        for s in seqs:
            L = self.ora.seq_length(s)
            assert self.gpu.seq_length(s) == L
            bto = list(self.ora.block_table(s))
            assert self.gpu.block_table(s) == bto, (s, self.gpu.block_table(s)[:8], bto[:8])
            assert (bt_dev[s, : len(bto)] == np.array(bto, dtype=np.int32)).all()
            for j, page in enumerate(bto):
                nv = min(16, L - 16 * j)
                for h in range(self.hkv):
                    odata, osz, filled = self.ora.page_contents(page, h)
                    assert filled[:nv].all()
                    blk = pool[page, h]
                    if self.fmt == kv4.FORMAT_INT4_PROT:
                        gc, gs = kv4_layout.int4_page_block(blk, self.d)
                    elif self.fmt == kv4.FORMAT_INT8:
                        gc, gs, gs2 = kv4_layout.int8_tile(blk, self.d)
                        assert (gs2[:nv] == gs[:nv]).all(), ("second scale copy", s, j, h)
                    else:
                        gc, gs = kv4_layout.bf16_page_block(blk, self.d), None
                    bad = np.argwhere(gc[:nv] != odata[:nv])
                    assert bad.size == 0, ("codes", s, j, h, bad[:5].tolist())
                    if gs is not None:
                        bad = np.argwhere(gs[:nv] != osz[:nv])
                        assert bad.size == 0, ("scales", s, j, h, bad[:5].tolist(), gs[:nv][tuple(bad[0][:2])],
                                               osz[:nv][tuple(bad[0][:2])])
                    compared += nv * 2
            if i8 is not None:
                for u in range(self.S + self.R):
                    for h in range(self.hkv):
                        gc, gs, gs2 = kv4_layout.int8_tile(i8[s, h, u // 16], self.d)
                        for kv in range(2):
                            oc, (os_, oz), tok = self.ora.int8_slot_contents(s, u, h, kv)
                            if tok < 0 or not oracle.is_protected(tok, L, self.S, self.R):
                                continue
                            assert (gc[u % 16, kv] == oc).all(), ("int8 codes", s, u, h, kv)
                            assert gs[u % 16, kv, 0] == os_ and gs[u % 16, kv, 1] == oz, ("int8 scales", s, u, h, kv)
                            assert (gs2[u % 16, kv] == gs[u % 16, kv]).all(), ("int8 second scale copy", s, u, h, kv)
                            compared += 1
        return compared
