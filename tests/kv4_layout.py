"""Test-side reader of the device memory layout documented in include/kv4.h.

Written from the header's layout description only; it shares no code with the library or the
oracle.  Turns raw pool bytes into logical codes / scales per (slot, K|V, dim).
"""
from __future__ import annotations

import numpy as np

P = 16


def int4_page_block(block: np.ndarray, D: int):
    """One (page, kv head) block of the INT4_PROT format ->
    codes uint8 [16 slots][2 (K, V)][D], scales uint16 [16][2][2] (s, z)."""
    assert block.dtype == np.uint8 and block.size == 16 * D + 128
    codes = np.zeros((P, 2, D), dtype=np.uint8)
    # K: [D/32 chunks][16 slots][16 B]; byte k of chunk c = dims 32c+2k (low nibble), 32c+2k+1 (high)
    k = block[: 8 * D].reshape(D // 32, P, 16)
    lo, hi = k & 0xF, k >> 4
    kk = np.stack([lo, hi], axis=-1)                 # [c][t][k][2]
    codes[:, 0, :] = kk.transpose(1, 0, 2, 3).reshape(P, D)
    # V: [D dims][8 B]; byte k = slot 2k (low nibble) | slot 2k+1 (high nibble)
    v = block[8 * D: 16 * D].reshape(D, 8)
    vv = np.stack([v & 0xF, v >> 4], axis=-1).reshape(D, P)  # [d][slot]
    codes[:, 1, :] = vv.T
    sz = block[16 * D: 16 * D + 128].view(np.uint16).reshape(P, 2, 2)  # (Ks, Kz), (Vs, Vz)
    return codes, sz


def int8_tile(block: np.ndarray, D: int):
    """One INT8 tile (protection slots or INT8-format page) -> codes [16][2][D], scales [16][2][2].

    The tile is two blocks of 16D + 128 bytes.  Block x holds K dims x*D/2 .. (x+1)*D/2 - 1 of
    all 16 slots as [D/32 chunks][16 slots][16 B] (one byte per dim), V of slots 8x .. 8x+7 as
    [D dims][8 B] (byte j = slot 8x + j), and the scales [16][4 x fp16].  Both blocks carry the
    same scales; the second copy is returned as a third output for comparison."""
    bb = 16 * D + 128
    assert block.dtype == np.uint8 and block.size == 2 * bb
    codes = np.zeros((P, 2, D), dtype=np.uint8)
    sz = []
    for x in range(2):
        b = block[x * bb:(x + 1) * bb]
        k = b[: 8 * D].reshape(D // 32, P, 16)                # [c][t][16 dims]
        codes[:, 0, x * D // 2:(x + 1) * D // 2] = k.transpose(1, 0, 2).reshape(P, D // 2)
        v = b[8 * D: 16 * D].reshape(D, 8)                    # [d][slot 8x + j]
        codes[8 * x: 8 * x + 8, 1, :] = v.T
        sz.append(b[16 * D: 16 * D + 128].view(np.uint16).reshape(P, 2, 2))
    return codes, sz[0], sz[1]


def bf16_page_block(block: np.ndarray, D: int):
    """One (page, kv head) block of the BF16 format -> bf16 bits uint16 [16][2][D]."""
    assert block.dtype == np.uint8 and block.size == 64 * D
    out = np.zeros((P, 2, D), dtype=np.uint16)
    k = block[: 32 * D].view(np.uint16).reshape(D // 8, P, 8)  # [c][t][8 dims]
    out[:, 0, :] = k.transpose(1, 0, 2).reshape(P, D)
    v = block[32 * D: 64 * D].view(np.uint16).reshape(D, P)    # [d][slot]
    out[:, 1, :] = v.T
    return out
