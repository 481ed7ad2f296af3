"""ctypes binding of libkv4 (names follow ``include/kv4.h``); argument marshalling only."""
from __future__ import annotations

import array
import ctypes
import os
from dataclasses import dataclass, asdict
from typing import Optional, Sequence

import torch  # loaded first so that libkv4 binds to the same HIP runtime as torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libkv4.so")

FORMAT_INT4_PROT = 0
FORMAT_INT8 = 1
FORMAT_BF16 = 2

EVICT_DUAL_WRITE = 0
EVICT_REQUANT = 1

STATUS = {
    0: "KV4_OK",
    1: "KV4_ERR_INVALID_ARGUMENT",
    2: "KV4_ERR_OUT_OF_PAGES",
    3: "KV4_ERR_SEQ_STATE",
    4: "KV4_ERR_WORKSPACE_TOO_SMALL",
    5: "KV4_ERR_UNSUPPORTED",
    6: "KV4_ERR_HIP",
}


class KV4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, "KV4_UNKNOWN")
        super().__init__("%s: %s" % (self.name, detail))


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages", "max_seqs", "max_pages_per_seq",
        "num_sinks", "num_recent", "hadamard_block", "format", "eviction")]


class _BufferSizes(ctypes.Structure):
    _fields_ = [("page_pool", ctypes.c_size_t), ("int8_pool", ctypes.c_size_t), ("block_table", ctypes.c_size_t),
                ("page_block_bytes", ctypes.c_size_t), ("int8_tile_bytes", ctypes.c_size_t),
                ("int8_tiles", ctypes.c_int32)]


class _Profile(ctypes.Structure):
    _fields_ = [("append_launches", ctypes.c_int64), ("append_ms", ctypes.c_double),
                ("decode_launches", ctypes.c_int64), ("split_ms", ctypes.c_double), ("merge_ms", ctypes.c_double),
                ("mq_launches", ctypes.c_int64), ("mq_split_ms", ctypes.c_double), ("mq_merge_ms", ctypes.c_double)]


class _Buffers(ctypes.Structure):
    _fields_ = [("page_pool", ctypes.c_void_p), ("int8_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p)]


@dataclass
class Config:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_pages: int
    max_seqs: int
    max_pages_per_seq: int
    num_sinks: int = 4
    num_recent: int = 128
    hadamard_block: int = 128
    format: int = FORMAT_INT4_PROT
    page_size: int = 16
    eviction: int = 0  # EVICT_DUAL_WRITE or EVICT_REQUANT

    def to_c(self) -> _Config:
        c = _Config()
        for k, v in asdict(self).items():
            setattr(c, k, int(v))
        return c


@dataclass
class BufferSizes:
    page_pool: int
    int8_pool: int
    block_table: int
    page_block_bytes: int
    int8_tile_bytes: int
    int8_tiles: int


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Loads libkv4.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libkv4.so is not built (run __graft_entry__.build() or "
                              "python -m int4_kv_cache_fwht_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.kv4_buffer_sizes_query.argtypes = [P, P]
        L.kv4_cache_create.argtypes = [P, P, P]
        L.kv4_cache_destroy.argtypes = [P]
        L.kv4_append_workspace_size.argtypes = [P, I32, P, P, P]
        L.kv4_append.argtypes = [P, I32, P, P, P, P, P, SZ, P]
        L.kv4_append_rope.argtypes = [P, I32, P, P, P, P, P, P, I32, P, SZ, P]
        L.kv4_seq_free.argtypes = [P, I32]
        L.kv4_decode_workspace_size.argtypes = [P, I32, P]
        L.kv4_decode_attention.argtypes = [P, I32, P, P, ctypes.c_float, P, P, SZ, P]
        L.kv4_decode_attention_bf16.argtypes = [P, I32, P, P, ctypes.c_float, P, P, SZ, P]
        L.kv4_decode_attention_noalloc.argtypes = [P, I32, P, P, ctypes.c_float, P, P]
        L.kv4_multi_query_workspace_size.argtypes = [P, I32, P, P, P]
        L.kv4_multi_query_attention.argtypes = [P, I32, P, P, P, ctypes.c_float, P, P, SZ, P]
        L.kv4_seq_length.argtypes = [P, I32, P]
        L.kv4_block_table.argtypes = [P, I32, P, I32, P]
        L.kv4_free_pages.argtypes = [P, P]
        L.kv4_set_decode_waves.argtypes = [P, I32]
        L.kv4_set_decode_rounds.argtypes = [P, I32, I32]
        L.kv4_set_mq_share.argtypes = [P, I32]
        L.kv4_profile_enable.argtypes = [P, I32]
        L.kv4_profile_read.argtypes = [P, P]
        L.kv4_profile_durations.argtypes = [P, I32, P, I32, P]
        L.kv4_hbm_probe.argtypes = [I32, P, P, SZ, I32, I32, P, P]
        L.kv4_status_string.argtypes = [ctypes.c_int]
        L.kv4_status_string.restype = ctypes.c_char_p
        L.kv4_last_error.argtypes = [P]
        L.kv4_last_error.restype = ctypes.c_char_p
        for name in ("kv4_buffer_sizes_query", "kv4_cache_create", "kv4_cache_destroy", "kv4_append_workspace_size",
                     "kv4_append", "kv4_append_rope", "kv4_seq_free", "kv4_decode_workspace_size", "kv4_decode_attention",
                     "kv4_decode_attention_bf16", "kv4_decode_attention_noalloc",
                     "kv4_multi_query_workspace_size", "kv4_multi_query_attention",
                     "kv4_seq_length", "kv4_block_table", "kv4_free_pages", "kv4_set_decode_waves", "kv4_set_decode_rounds", "kv4_set_mq_share",
                     "kv4_profile_enable", "kv4_profile_read", "kv4_profile_durations", "kv4_hbm_probe"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, handle=None):
    if status != 0:
        detail = lib().kv4_last_error(handle)
        raise KV4Error(status, detail.decode() if detail else "")


def _i32_array(values: Sequence[int]):
    """An int32 C array holding `values`.  The conversion runs in C (array.array); a per-element
    Python loop cost about 15 us for 256 sequence ids, more than a decode launch at small shapes."""
    a = array.array("i", values)
    if a.itemsize != 4:
        raise RuntimeError("C int is not 32 bits on this platform")
    if len(a) == 0:
        return (ctypes.c_int32 * 0)()
    return (ctypes.c_int32 * len(a)).from_buffer(a)  # shares a's memory and keeps it alive


def kv4_buffer_sizes_query(cfg: Config) -> BufferSizes:
    c = cfg.to_c()
    out = _BufferSizes()
    _check(lib().kv4_buffer_sizes_query(ctypes.byref(c), ctypes.byref(out)))
    return BufferSizes(out.page_pool, out.int8_pool, out.block_table, out.page_block_bytes, out.int8_tile_bytes,
                       out.int8_tiles)


def hbm_probe(mode: int, src: torch.Tensor, dst: torch.Tensor, nbytes: int, reps: int, blocks: int = 0,
              stream=None):
    """kv4_hbm_probe: per-launch durations (ms) of `reps` streaming reads (mode 0) or copies (mode 1)
    of `nbytes` from src to dst (device tensors of the current device)."""
    if src.device.type != "cuda" or dst.device.type != "cuda":
        raise ValueError("probe buffers must be device tensors")
    if src.numel() * src.element_size() < nbytes:
        raise ValueError("src smaller than nbytes")
    if blocks <= 0:
        blocks = 8 * torch.cuda.get_device_properties(dst.device).multi_processor_count
    need = nbytes if mode == 1 else blocks * 1024
    if dst.numel() * dst.element_size() < need:
        raise ValueError("dst too small")
    ms = (ctypes.c_float * reps)()
    _check(lib().kv4_hbm_probe(int(mode), src.data_ptr(), dst.data_ptr(), int(nbytes), int(blocks), int(reps), ms,
                               _stream_ptr(stream)))
    return [ms[i] for i in range(reps)]


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Cache:
    """A kv4 cache over torch-allocated device buffers on ``device``.

    Workspaces are cached per instance and grown on demand; calls through one instance must be
    ordered on one stream (the library's own rule for a handle).
    """

    def __init__(self, cfg: Config, device="cuda"):
        self.cfg = cfg
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        self.sizes = kv4_buffer_sizes_query(cfg)
        with torch.cuda.device(self.device):
            self.page_pool = torch.empty(max(self.sizes.page_pool, 256), dtype=torch.uint8, device=self.device)
            self.int8_pool = (torch.empty(self.sizes.int8_pool, dtype=torch.uint8, device=self.device)
                              if self.sizes.int8_pool else None)
            self.block_table_dev = torch.full((cfg.max_seqs, cfg.max_pages_per_seq), -1, dtype=torch.int32,
                                              device=self.device)
            bufs = _Buffers(self.page_pool.data_ptr(), self.int8_pool.data_ptr() if self.int8_pool is not None else None,
                            self.block_table_dev.data_ptr())
            c = cfg.to_c()
            h = ctypes.c_void_p()
            _check(lib().kv4_cache_create(ctypes.byref(c), ctypes.byref(bufs), ctypes.byref(h)))
        self._h = h
        self._ws_append = None
        self._ws_decode = None
        self._ws_mq = None

    # -- lifetime --------------------------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            lib().kv4_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    # -- workspace -------------------------------------------------------------------------------
    def _workspace(self, attr: str, nbytes: int) -> torch.Tensor:
        ws = getattr(self, attr)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            setattr(self, attr, ws)
        return ws

    def append_workspace_size(self, seq_ids: Sequence[int], n_new: Sequence[int]) -> int:
        return self._append_ws_size(_i32_array(seq_ids), _i32_array(n_new))

    def _append_ws_size(self, ids, nn) -> int:
        out = ctypes.c_size_t()
        _check(lib().kv4_append_workspace_size(self._h, len(ids), ids, nn, ctypes.byref(out)), self._h)
        return out.value

    def decode_workspace_size(self, n_seqs: int) -> int:
        out = ctypes.c_size_t()
        _check(lib().kv4_decode_workspace_size(self._h, int(n_seqs), ctypes.byref(out)), self._h)
        return out.value

    # -- calls -------------------------------------------------------------------------------------
    def append(self, seq_ids: Sequence[int], n_new: Sequence[int], k: Optional[torch.Tensor],
               v: Optional[torch.Tensor], stream=None, workspace: Optional[torch.Tensor] = None):
        """k, v: bf16 [sum(n_new), Hkv, D] on the cache's device (rows in call order)."""
        ids, nn = _i32_array(seq_ids), _i32_array(n_new)
        rows = sum(int(x) for x in n_new)
        kp = vp = None
        if rows > 0:
            for t in (k, v):
                if t is None or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != self.device:
                    raise ValueError("k / v must be contiguous bf16 tensors on the cache device")
                if tuple(t.shape) != (rows, self.cfg.num_kv_heads, self.cfg.head_dim):
                    raise ValueError("k / v shape must be [sum(n_new), Hkv, D]")
            kp, vp = k.data_ptr(), v.data_ptr()
        if workspace is None:
            workspace = self._workspace("_ws_append", self._append_ws_size(ids, nn))
        st = _stream_ptr(stream)
        _check(lib().kv4_append(self._h, len(ids), ids, nn, kp, vp, workspace.data_ptr(), workspace.numel(), st),
               self._h)

    def append_rope(self, seq_ids: Sequence[int], n_new: Sequence[int], k: torch.Tensor, v: torch.Tensor,
                    rope_cos: torch.Tensor, rope_sin: torch.Tensor, stream=None,
                    workspace: Optional[torch.Tensor] = None):
        """Append with pre-RoPE keys; rope_cos / rope_sin: float32 [positions, D/2] on the device."""
        ids, nn = _i32_array(seq_ids), _i32_array(n_new)
        rows = sum(int(x) for x in n_new)
        for t in (k, v):
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != self.device:
                raise ValueError("k / v must be contiguous bf16 tensors on the cache device")
            if tuple(t.shape) != (rows, self.cfg.num_kv_heads, self.cfg.head_dim):
                raise ValueError("k / v shape must be [sum(n_new), Hkv, D]")
        for t in (rope_cos, rope_sin):
            if t.dtype != torch.float32 or not t.is_contiguous() or t.device != self.device or t.dim() != 2 \
                    or t.shape[1] != self.cfg.head_dim // 2:
                raise ValueError("RoPE tables must be contiguous float32 [positions, D/2] on the cache device")
        if rope_cos.shape != rope_sin.shape:
            raise ValueError("RoPE tables differ in shape")
        if workspace is None:
            workspace = self._workspace("_ws_append", self._append_ws_size(ids, nn))
        st = _stream_ptr(stream)
        _check(lib().kv4_append_rope(self._h, len(ids), ids, nn, k.data_ptr(), v.data_ptr(), rope_cos.data_ptr(),
                                     rope_sin.data_ptr(), rope_cos.shape[0], workspace.data_ptr(), workspace.numel(),
                                     st), self._h)

    def decode_attention(self, seq_ids: Sequence[int], q: torch.Tensor, scale: float = 0.0,
                         out: Optional[torch.Tensor] = None, stream=None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """q: bf16 [n, Hq, D] -> fp32 [n, Hq, D]."""
        ids = _i32_array(seq_ids)
        n = len(ids)
        shape = (n, self.cfg.num_q_heads, self.cfg.head_dim)
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != shape or q.device != self.device:
            raise ValueError("q must be a contiguous bf16 [n, Hq, D] tensor on the cache device")
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape:
            raise ValueError("out must be a contiguous fp32 [n, Hq, D] tensor")
        if workspace is None:
            workspace = self._workspace("_ws_decode", self.decode_workspace_size(n))
        st = _stream_ptr(stream)
        _check(lib().kv4_decode_attention(self._h, n, ids, q.data_ptr(), float(scale), out.data_ptr(),
                                          workspace.data_ptr(), workspace.numel(), st), self._h)
        return out

    def decode_attention_noalloc(self, seq_ids: Sequence[int], q: torch.Tensor, out: torch.Tensor,
                                 scale: float = 0.0, stream=None) -> torch.Tensor:
        """kv4_decode_attention_noalloc: q bf16 [n, Hq, D] -> out, a caller-given fp32 [n, Hq, D]
        tensor (the call takes no workspace and allocates nothing)."""
        ids = _i32_array(seq_ids)
        n = len(ids)
        shape = (n, self.cfg.num_q_heads, self.cfg.head_dim)
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != shape or q.device != self.device:
            raise ValueError("q must be a contiguous bf16 [n, Hq, D] tensor on the cache device")
        if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape \
                or out.device != self.device:
            raise ValueError("out must be a contiguous fp32 [n, Hq, D] tensor on the cache device")
        st = _stream_ptr(stream)
        _check(lib().kv4_decode_attention_noalloc(self._h, n, ids, q.data_ptr(), float(scale), out.data_ptr(), st),
               self._h)
        return out

    def multi_query_workspace_size(self, seq_ids: Sequence[int], n_q: Sequence[int]) -> int:
        ids, nq = _i32_array(seq_ids), _i32_array(n_q)
        out = ctypes.c_size_t()
        _check(lib().kv4_multi_query_workspace_size(self._h, len(ids), ids, nq, ctypes.byref(out)), self._h)
        return out.value

    def multi_query_attention(self, seq_ids: Sequence[int], n_q: Sequence[int], q: torch.Tensor, scale: float = 0.0,
                              out: Optional[torch.Tensor] = None, stream=None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """q: bf16 [sum(n_q), Hq, D] (each sequence's rows in ascending position) -> fp32, same shape."""
        ids, nq = _i32_array(seq_ids), _i32_array(n_q)
        rows = sum(int(x) for x in n_q)
        shape = (rows, self.cfg.num_q_heads, self.cfg.head_dim)
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != shape or q.device != self.device:
            raise ValueError("q must be a contiguous bf16 [sum(n_q), Hq, D] tensor on the cache device")
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != shape:
            raise ValueError("out must be a contiguous fp32 [sum(n_q), Hq, D] tensor")
        if workspace is None:
            workspace = self._workspace("_ws_mq", self.multi_query_workspace_size(seq_ids, n_q))
        st = _stream_ptr(stream)
        _check(lib().kv4_multi_query_attention(self._h, len(ids), ids, nq, q.data_ptr(), float(scale), out.data_ptr(),
                                               workspace.data_ptr(), workspace.numel(), st), self._h)
        return out

    def decode_attention_bf16(self, seq_ids: Sequence[int], q: torch.Tensor, scale: float = 0.0,
                              out: Optional[torch.Tensor] = None, stream=None,
                              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
        """q: bf16 [n, Hq, D] -> bf16 [n, Hq, D] (the fp32 result rounded to nearest even)."""
        ids = _i32_array(seq_ids)
        n = len(ids)
        shape = (n, self.cfg.num_q_heads, self.cfg.head_dim)
        if q.dtype != torch.bfloat16 or not q.is_contiguous() or tuple(q.shape) != shape or q.device != self.device:
            raise ValueError("q must be a contiguous bf16 [n, Hq, D] tensor on the cache device")
        if out is None:
            out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        elif out.dtype != torch.bfloat16 or not out.is_contiguous() or tuple(out.shape) != shape:
            raise ValueError("out must be a contiguous bf16 [n, Hq, D] tensor")
        if workspace is None:
            workspace = self._workspace("_ws_decode", self.decode_workspace_size(n))
        st = _stream_ptr(stream)
        _check(lib().kv4_decode_attention_bf16(self._h, n, ids, q.data_ptr(), float(scale), out.data_ptr(),
                                               workspace.data_ptr(), workspace.numel(), st), self._h)
        return out

    def seq_free(self, seq_id: int):
        _check(lib().kv4_seq_free(self._h, int(seq_id)), self._h)

    def seq_length(self, seq_id: int) -> int:
        out = ctypes.c_int32()
        _check(lib().kv4_seq_length(self._h, int(seq_id), ctypes.byref(out)), self._h)
        return out.value

    def block_table(self, seq_id: int):
        cap = self.cfg.max_pages_per_seq
        buf = (ctypes.c_int32 * cap)()
        n = ctypes.c_int32()
        _check(lib().kv4_block_table(self._h, int(seq_id), buf, cap, ctypes.byref(n)), self._h)
        return [buf[i] for i in range(min(n.value, cap))]

    def free_pages(self) -> int:
        out = ctypes.c_int32()
        _check(lib().kv4_free_pages(self._h, ctypes.byref(out)), self._h)
        return out.value

    def set_decode_waves(self, waves: int):
        _check(lib().kv4_set_decode_waves(self._h, int(waves)), self._h)

    def set_decode_rounds(self, round2_waves: int, round1_permille: int = 1000):
        _check(lib().kv4_set_decode_rounds(self._h, int(round2_waves), int(round1_permille)), self._h)

    def set_mq_share(self, enable: bool):
        _check(lib().kv4_set_mq_share(self._h, int(bool(enable))), self._h)

    def profile_enable(self, enable: bool = True):
        _check(lib().kv4_profile_enable(self._h, 1 if enable else 0), self._h)

    def profile_durations(self, kind: str) -> list:
        """Per-launch durations (ms) since profile_enable: 'append', 'split', 'merge', 'mq_split', 'mq_merge'."""
        k = ["append", "split", "merge", "mq_split", "mq_merge"].index(kind)
        n = ctypes.c_int32()
        _check(lib().kv4_profile_durations(self._h, k, None, 0, ctypes.byref(n)), self._h)
        buf = (ctypes.c_float * max(n.value, 1))()
        _check(lib().kv4_profile_durations(self._h, k, buf, n.value, ctypes.byref(n)), self._h)
        return [buf[i] for i in range(n.value)]

    def profile_read(self) -> dict:
        p = _Profile()
        _check(lib().kv4_profile_read(self._h, ctypes.byref(p)), self._h)
        return {"append_launches": p.append_launches, "append_ms": p.append_ms,
                "decode_launches": p.decode_launches, "split_ms": p.split_ms, "merge_ms": p.merge_ms,
                "mq_launches": p.mq_launches, "mq_split_ms": p.mq_split_ms, "mq_merge_ms": p.mq_merge_ms}
