"""CPU oracle for the INT4 KV cache (block-diagonal Hadamard rotation, token-wise INT4, INT8
sink/recent protection): ctypes bindings over ``kv4_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It shares no code with the HIP library and never imports it.

What each function follows is stated in ``kv4_oracle.c`` next to its definition; the sources are
the abstracts of "SAW-INT4: System-Aware 4-Bit KV-Cache Quantization for Real-World LLM Serving"
and "KV4-RL: Unlocking Faster Asynchronous Rollouts for RLVR with INT4 KV Cache Quantization",
and item 5 of the "KV Cache Quantization" topic page.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv4_oracle.c")
_LIB = os.path.join(_HERE, "libkv4_oracle.so")

# Oracle status values (its own numbering).
OK = 0
INVALID_ARGUMENT = 1
OUT_OF_PAGES = 2
SEQ_STATE = 3
PRECONDITION = 7

FMT_INT4_PROT = 0
FMT_INT8 = 1
FMT_BF16 = 2

# gcc flags: binary32 steps stay single IEEE operations (no contraction into FMA, no fast-math,
# SSE arithmetic on x86-64), denormals kept.
CFLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile ``libkv4_oracle.so`` with gcc; returns its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        c_int, c_float, c_double = ctypes.c_int, ctypes.c_float, ctypes.c_double
        P = ctypes.c_void_p
        L.kv4o_fp16_value.argtypes = [ctypes.c_uint16]
        L.kv4o_fp16_value.restype = c_double
        L.kv4o_fp16_round_down.argtypes = [c_float, P]
        L.kv4o_fp16_round_down.restype = c_int
        L.kv4o_fp16_round_up.argtypes = [c_float, P]
        L.kv4o_fp16_round_up.restype = c_int
        L.kv4o_rotation_scale.argtypes = [c_int]
        L.kv4o_rotation_scale.restype = c_float
        L.kv4o_fwht_f32.argtypes = [P, c_int, c_int]
        L.kv4o_fwht_f32.restype = None
        L.kv4o_rotate_bf16.argtypes = [P, c_int, c_int, P]
        L.kv4o_rotate_bf16.restype = None
        L.kv4o_quantize.argtypes = [P, c_int, c_int, P, P, P]
        L.kv4o_quantize.restype = c_int
        L.kv4o_pack_int4.argtypes = [P, c_int, P]
        L.kv4o_pack_int4.restype = None
        L.kv4o_is_protected.argtypes = [c_int, c_int, c_int, c_int]
        L.kv4o_is_protected.restype = c_int
        L.kv4o_int8_slot.argtypes = [c_int, c_int, c_int]
        L.kv4o_int8_slot.restype = c_int
        L.kv4o_create.argtypes = [c_int] * 11
        L.kv4o_create.restype = P
        L.kv4o_destroy.argtypes = [P]
        L.kv4o_destroy.restype = None
        L.kv4o_free_pages.argtypes = [P]
        L.kv4o_free_pages.restype = c_int
        L.kv4o_seq_length.argtypes = [P, c_int]
        L.kv4o_seq_length.restype = c_int
        L.kv4o_block_table.argtypes = [P, c_int, P, c_int]
        L.kv4o_block_table.restype = c_int
        L.kv4o_seq_free.argtypes = [P, c_int]
        L.kv4o_seq_free.restype = c_int
        L.kv4o_append.argtypes = [P, c_int, P, P, P, P]
        L.kv4o_append.restype = c_int
        L.kv4o_get_page_token.argtypes = [P, c_int, c_int, c_int, c_int, P, P, P, P]
        L.kv4o_get_page_token.restype = c_int
        L.kv4o_get_page.argtypes = [P, c_int, c_int, P, P, P, P]
        L.kv4o_get_page.restype = c_int
        L.kv4o_get_int8_slot.argtypes = [P, c_int, c_int, c_int, c_int, P, P, P]
        L.kv4o_get_int8_slot.restype = c_int
        L.kv4o_dequant_seq.argtypes = [P, c_int, c_int, P, P]
        L.kv4o_dequant_seq.restype = c_int
        L.kv4o_decode.argtypes = [P, c_int, P, P, c_double, P, c_int, P]
        L.kv4o_decode.restype = c_int
        L.kv4o_rope_bf16.argtypes = [P, c_int, P, P, P]
        L.kv4o_rope_bf16.restype = None
        L.kv4o_append_rope.argtypes = [P, c_int, P, P, P, P, P, P, c_int]
        L.kv4o_append_rope.restype = c_int
        L.kv4o_set_eviction.argtypes = [P, c_int]
        L.kv4o_set_eviction.restype = c_int
        L.kv4o_attend_multi.argtypes = [P, c_int, P, P, P, c_double, P, c_int, P]
        L.kv4o_attend_multi.restype = c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ------------------------------------------------------------------------------------------------
# Scalar / vector primitives
# ------------------------------------------------------------------------------------------------

def fp16_value(bits: int) -> float:
    """Value of a binary16 bit pattern, from the format's definition."""
    return lib().kv4o_fp16_value(int(bits))


def fp16_round_down(x: float) -> int:
    """Bits of the largest binary16 value <= x (a zero gives +0)."""
    out = ctypes.c_uint16()
    if lib().kv4o_fp16_round_down(float(np.float32(x)), ctypes.byref(out)) != 0:
        raise ValueError("outside the binary16 range")
    return out.value


def fp16_round_up(x: float) -> int:
    """Bits of the smallest binary16 value >= x (a zero gives +0)."""
    out = ctypes.c_uint16()
    if lib().kv4o_fp16_round_up(float(np.float32(x)), ctypes.byref(out)) != 0:
        raise ValueError("outside the binary16 range")
    return out.value


def rotation_scale(b: int) -> np.float32:
    return np.float32(lib().kv4o_rotation_scale(int(b)))


def fwht_f32(y: np.ndarray, b: int) -> np.ndarray:
    """Rotate each row of a float32 array (last axis n, n % b == 0) by the block FWHT."""
    y = np.ascontiguousarray(y, dtype=np.float32).copy()
    n = y.shape[-1]
    flat = y.reshape(-1, n)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib().kv4o_fwht_f32(_ptr(row), n, int(b))
        flat[r] = row
    return flat.reshape(y.shape)


def rotate_bf16(x_bits: np.ndarray, b: int) -> np.ndarray:
    """bf16 bit patterns (uint16, last axis n) -> rotated float32 rows."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    n = x_bits.shape[-1]
    flat = x_bits.reshape(-1, n)
    out = np.empty(flat.shape, dtype=np.float32)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        o = np.empty(n, dtype=np.float32)
        lib().kv4o_rotate_bf16(_ptr(row), n, int(b), _ptr(o))
        out[r] = o
    return out.reshape(x_bits.shape)


def rope_bf16(x_bits: np.ndarray, cos_row: np.ndarray, sin_row: np.ndarray) -> np.ndarray:
    """RoPE (rotate-half pairs) of one bf16 row with one position's table rows -> float32 row."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    c = np.ascontiguousarray(cos_row, dtype=np.float32)
    s = np.ascontiguousarray(sin_row, dtype=np.float32)
    assert c.shape == s.shape == (x_bits.shape[0] // 2,)
    out = np.empty(x_bits.shape[0], dtype=np.float32)
    lib().kv4o_rope_bf16(_ptr(x_bits), x_bits.shape[0], _ptr(c), _ptr(s), _ptr(out))
    return out


def quantize(y: np.ndarray, Q: int) -> Tuple[np.ndarray, int, int]:
    """Token-wise asymmetric quantization of one group -> (codes uint8, s bits, z bits)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    codes = np.empty(y.shape[0], dtype=np.uint8)
    s = ctypes.c_uint16()
    z = ctypes.c_uint16()
    rc = lib().kv4o_quantize(_ptr(y), y.shape[0], int(Q), _ptr(codes), ctypes.byref(s), ctypes.byref(z))
    if rc != 0:
        raise ValueError("quantizer precondition violated (non-finite or outside fp16 range)")
    return codes, s.value, z.value


def pack_int4(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[0] // 2, dtype=np.uint8)
    lib().kv4o_pack_int4(_ptr(codes), codes.shape[0], _ptr(out))
    return out


def is_protected(t: int, L: int, S: int, R: int) -> bool:
    return bool(lib().kv4o_is_protected(int(t), int(L), int(S), int(R)))


def int8_slot(t: int, S: int, R: int) -> int:
    return int(lib().kv4o_int8_slot(int(t), int(S), int(R)))


# ------------------------------------------------------------------------------------------------
# Cache model
# ------------------------------------------------------------------------------------------------

class OracleCache:
    """Paged cache model: FIFO page allocator, block tables, logical INT4 / INT8 / bf16 contents."""

    def __init__(self, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int,
                 max_seqs: int, max_pages_per_seq: int, num_sinks: int, num_recent: int, hadamard_block: int,
                 fmt: int = FMT_INT4_PROT, eviction: int = 0):
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.P, self.num_pages, self.max_seqs, self.max_pps = page_size, num_pages, max_seqs, max_pages_per_seq
        self.S, self.R, self.b, self.fmt = num_sinks, num_recent, hadamard_block, fmt
        h = lib().kv4o_create(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, max_seqs,
                              max_pages_per_seq, num_sinks, num_recent, hadamard_block, fmt)
        if not h:
            raise ValueError("invalid oracle cache configuration")
        self._h = ctypes.c_void_p(h)
        self.eviction = eviction
        if eviction and lib().kv4o_set_eviction(self._h, int(eviction)) != OK:
            raise ValueError("invalid eviction rule for this format")

    def close(self):
        if self._h:
            lib().kv4o_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- state ---------------------------------------------------------------------------------
    def free_pages(self) -> int:
        return lib().kv4o_free_pages(self._h)

    def seq_length(self, seq: int) -> int:
        return lib().kv4o_seq_length(self._h, int(seq))

    def block_table(self, seq: int) -> np.ndarray:
        cap = self.max_pps
        buf = np.empty(cap, dtype=np.int32)
        n = lib().kv4o_block_table(self._h, int(seq), _ptr(buf), cap)
        if n < 0:
            raise ValueError("bad sequence id")
        return buf[:n].copy()

    def seq_free(self, seq: int) -> int:
        return lib().kv4o_seq_free(self._h, int(seq))

    def append(self, seq_ids: Sequence[int], n_new: Sequence[int], k_bits: Optional[np.ndarray],
               v_bits: Optional[np.ndarray]) -> int:
        """k_bits, v_bits: uint16 [sum(n_new), hkv, d] bf16 patterns, or None (allocate only)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        nn = np.ascontiguousarray(n_new, dtype=np.int32)
        kp = vp = None
        if k_bits is not None:
            k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
            v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
            assert k_bits.shape == (int(nn.sum()), self.hkv, self.d) and v_bits.shape == k_bits.shape
            kp, vp = _ptr(k_bits), _ptr(v_bits)
        return lib().kv4o_append(self._h, ids.shape[0], _ptr(ids), _ptr(nn), kp, vp)

    def append_rope(self, seq_ids: Sequence[int], n_new: Sequence[int], k_bits: np.ndarray, v_bits: np.ndarray,
                    rope_cos: np.ndarray, rope_sin: np.ndarray) -> int:
        """Like append with pre-RoPE keys; rope_cos / rope_sin: float32 [positions, d/2]."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        nn = np.ascontiguousarray(n_new, dtype=np.int32)
        k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
        assert k_bits.shape == (int(nn.sum()), self.hkv, self.d) and v_bits.shape == k_bits.shape
        c = np.ascontiguousarray(rope_cos, dtype=np.float32)
        s = np.ascontiguousarray(rope_sin, dtype=np.float32)
        assert c.shape == s.shape and c.shape[1] == self.d // 2
        return lib().kv4o_append_rope(self._h, ids.shape[0], _ptr(ids), _ptr(nn), _ptr(k_bits), _ptr(v_bits), _ptr(c),
                                      _ptr(s), c.shape[0])

    # -- contents ------------------------------------------------------------------------------
    def page_token(self, seq: int, t: int, h: int, kv: int):
        """(codes uint8 [d], (s_bits, z_bits), page) of position t, or bf16 bits [d] for fmt bf16."""
        codes = np.empty(self.d, dtype=np.uint8)
        sz = np.empty(2, dtype=np.uint16)
        bf = np.empty(self.d, dtype=np.uint16)
        page = ctypes.c_int()
        rc = lib().kv4o_get_page_token(self._h, int(seq), int(t), int(h), int(kv), _ptr(codes), _ptr(sz), _ptr(bf),
                                       ctypes.byref(page))
        if rc != 0:
            raise KeyError((seq, t))
        if self.fmt == FMT_BF16:
            return bf, None, page.value
        return codes, (int(sz[0]), int(sz[1])), page.value

    def page_contents(self, page: int, h: int):
        """(codes uint8 [P, 2, d] or bf16 bits uint16 [P, 2, d], scales uint16 [P, 2, 2] or None,
        filled bool [P]) of one page for kv head h."""
        filled = np.zeros(self.P, dtype=np.uint8)
        if self.fmt == FMT_BF16:
            bf = np.zeros((self.P, 2, self.d), dtype=np.uint16)
            rc = lib().kv4o_get_page(self._h, int(page), int(h), None, None, _ptr(bf), _ptr(filled))
            data, sz = bf, None
        else:
            codes = np.zeros((self.P, 2, self.d), dtype=np.uint8)
            sz = np.zeros((self.P, 2, 2), dtype=np.uint16)
            rc = lib().kv4o_get_page(self._h, int(page), int(h), _ptr(codes), _ptr(sz), None, _ptr(filled))
            data = codes
        if rc != 0:
            raise KeyError(page)
        return data, sz, filled.astype(bool)

    def int8_slot_contents(self, seq: int, u: int, h: int, kv: int):
        """(codes uint8 [d], (s_bits, z_bits), token held or -1) of INT8 slot u."""
        codes = np.empty(self.d, dtype=np.uint8)
        sz = np.empty(2, dtype=np.uint16)
        tok = ctypes.c_int()
        rc = lib().kv4o_get_int8_slot(self._h, int(seq), int(u), int(h), int(kv), _ptr(codes), _ptr(sz),
                                      ctypes.byref(tok))
        if rc != 0:
            raise KeyError((seq, u))
        return codes, (int(sz[0]), int(sz[1])), tok.value

    def dequant_seq(self, seq: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
        L = self.seq_length(seq)
        k = np.empty((L, self.d), dtype=np.float64)
        v = np.empty((L, self.d), dtype=np.float64)
        rc = lib().kv4o_dequant_seq(self._h, int(seq), int(h), _ptr(k), _ptr(v))
        if rc != OK:
            raise ValueError("dequant failed (%d)" % rc)
        return k, v

    def decode(self, seq_ids: Sequence[int], q_bits: np.ndarray, scale: float = 0.0,
               threads: int = 0) -> Tuple[np.ndarray, int]:
        """q_bits: uint16 [n, hq, d] bf16 patterns -> (out float64 [n, hq, d], threads used)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        assert q_bits.shape == (ids.shape[0], self.hq, self.d)
        out = np.zeros((ids.shape[0], self.hq, self.d), dtype=np.float64)
        used = ctypes.c_int()
        rc = lib().kv4o_decode(self._h, ids.shape[0], _ptr(ids), _ptr(q_bits), float(scale), _ptr(out), int(threads),
                               ctypes.byref(used))
        if rc != OK:
            raise ValueError("oracle decode failed (%d)" % rc)
        return out, used.value

    def attend_multi(self, seq_ids: Sequence[int], n_q: Sequence[int], q_bits: np.ndarray, scale: float = 0.0,
                     threads: int = 0) -> Tuple[np.ndarray, int]:
        """Causal attention of the last n_q[i] positions of each sequence over its cache.
        q_bits: uint16 [sum n_q, hq, d] bf16 patterns, rows of a sequence consecutive (ascending
        position) -> (out float64 [sum n_q, hq, d], threads used)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int32)
        nq = np.ascontiguousarray(n_q, dtype=np.int32)
        assert nq.shape == ids.shape
        rows = int(nq.sum())
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        assert q_bits.shape == (rows, self.hq, self.d)
        out = np.zeros((rows, self.hq, self.d), dtype=np.float64)
        used = ctypes.c_int()
        rc = lib().kv4o_attend_multi(self._h, ids.shape[0], _ptr(ids), _ptr(nq), _ptr(q_bits), float(scale), _ptr(out),
                                     int(threads), ctypes.byref(used))
        if rc != OK:
            raise ValueError("oracle multi-query attention failed (%d)" % rc)
        return out, used.value
