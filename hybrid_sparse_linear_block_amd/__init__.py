"""Python binding of libhsla: hybrid sparse-plus-linear decode attention on
MI355X (gfx950).

The functions below carry the C ABI's names (include/hsla.h) and only
marshal arguments: torch tensors become device pointers, the current torch
stream becomes the hipStream_t.  Every step of the computation runs in the
HIP kernels of libhsla.so.  There is no fallback: importing the binding when
the library has not been built raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhsla.so")
# the same library with every entry point checking lengths and block tables
# before it launches (HSLA_DEBUG_CHECKS); open it with open_library()
DEBUG_LIB_PATH = os.path.join(HERE, "libhsla_debug.so")
# the same library with per-workgroup phase timestamps of the decode kernels
# (HSLA_PHASE_TIMESTAMPS; a diagnostic build, read by hsla_phase_timestamps)
PHASES_LIB_PATH = os.path.join(HERE, "libhsla_phases.so")

HSLA_OK = 0
HSLA_ERR_INVALID_ARG = -1
HSLA_ERR_UNSUPPORTED = -2
HSLA_ERR_WORKSPACE = -3
HSLA_ERR_HIP = -4
HSLA_F32 = 0
HSLA_BF16 = 1
HSLA_SEL_PER_HEAD = 0
HSLA_SEL_GROUPED = 1
HSLA_SEL_TOKEN = 2
HSLA_STATE_BLOCKS = 0
HSLA_STATE_TOKENS = 1
HSLA_SPLIT_DEFAULT = 0
HSLA_SPLIT_FIXED = 1
HSLA_SPLIT_DYNAMIC = 2
HSLA_MAX_PROFILE_EVENTS = 8

EXPORTED = ("hsla_status_string", "hsla_version", "hsla_build_workspace_size", "hsla_build_state",
            "hsla_append_token", "hsla_decode_workspace_size", "hsla_decode", "hsla_append_decode",
            "hsla_prefill_chunk_workspace_size", "hsla_prefill_chunk", "hsla_noalloc_scratch_bytes",
            "hsla_append_decode_noalloc", "hsla_check_tables", "hsla_check_tables_host",
            "hsla_phase_timestamp_bytes", "hsla_phase_timestamps")


class hsla_config(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("num_sink", ctypes.c_int32),
                ("window", ctypes.c_int32), ("linear_tail", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("selection", ctypes.c_int32), ("deterministic", ctypes.c_int32),
                ("state_span", ctypes.c_int32)]


class hsla_kv_pool(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("blk_mean", ctypes.c_void_p), ("blk_var", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class hsla_state(ctypes.Structure):
    _fields_ = [("S", ctypes.c_void_p), ("z", ctypes.c_void_p), ("sv", ctypes.c_void_p)]


class hsla_profile(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p * HSLA_MAX_PROFILE_EVENTS), ("capacity", ctypes.c_int32),
                ("recorded", ctypes.c_int32), ("names", ctypes.c_char_p * HSLA_MAX_PROFILE_EVENTS)]


class HslaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhsla.so (built in-tree by hybrid_sparse_linear_block_amd.build).

    torch ships its own HIP runtime (libamdhip64.so, same soname as the
    system one).  torch is imported first so that libhsla binds to that
    runtime: device pointers and streams from torch are then valid in
    libhsla, and the process holds a single HIP runtime.
    """
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def use_library(path: str) -> ctypes.CDLL:
    """Make the build at `path` (the debug or the phase-timestamp library)
    the one every binding function calls from now on."""
    global _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A libhsla build at `path` with every entry point's argument types
    set, independent of the one load() keeps (the debug library, say)."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python hybrid_sparse_linear_block_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    lib.hsla_status_string.argtypes = [ctypes.c_int]
    lib.hsla_status_string.restype = ctypes.c_char_p
    lib.hsla_version.argtypes = []
    lib.hsla_version.restype = ctypes.c_char_p
    lib.hsla_build_workspace_size.argtypes = [P(hsla_config), i32, i32]
    lib.hsla_build_workspace_size.restype = sz
    lib.hsla_build_state.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, i32, i32, vp, sz, vp]
    lib.hsla_build_state.restype = ctypes.c_int
    lib.hsla_append_token.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, vp, vp, vp, i32, i32, vp]
    lib.hsla_append_token.restype = ctypes.c_int
    lib.hsla_decode_workspace_size.argtypes = [P(hsla_config), i32, i32]
    lib.hsla_decode_workspace_size.restype = sz
    lib.hsla_decode.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, vp, i32, i32, vp, vp, vp,
                                sz, vp, P(hsla_profile)]
    lib.hsla_decode.restype = ctypes.c_int
    lib.hsla_append_decode.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, vp, vp, vp, vp, i32,
                                       i32, vp, vp, vp, sz, vp, P(hsla_profile)]
    lib.hsla_append_decode.restype = ctypes.c_int
    lib.hsla_prefill_chunk_workspace_size.argtypes = [P(hsla_config), i32, i32, i32]
    lib.hsla_prefill_chunk_workspace_size.restype = sz
    lib.hsla_prefill_chunk.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, vp, vp, vp, vp, i32,
                                       i32, i32, vp, vp, vp, sz, vp]
    lib.hsla_prefill_chunk.restype = ctypes.c_int
    lib.hsla_noalloc_scratch_bytes.argtypes = []
    lib.hsla_noalloc_scratch_bytes.restype = sz
    lib.hsla_append_decode_noalloc.argtypes = [P(hsla_config), P(hsla_kv_pool), P(hsla_state), vp, vp, vp, vp, vp,
                                               i32, i32, vp, vp, vp]
    lib.hsla_append_decode_noalloc.restype = ctypes.c_int
    lib.hsla_phase_timestamp_bytes.argtypes = []
    lib.hsla_phase_timestamp_bytes.restype = sz
    lib.hsla_phase_timestamps.argtypes = [vp, sz, i32]
    lib.hsla_phase_timestamps.restype = ctypes.c_int
    lib.hsla_check_tables.argtypes = [P(hsla_config), P(hsla_kv_pool), vp, i32, i32, i32, vp, vp]
    lib.hsla_check_tables.restype = ctypes.c_int
    lib.hsla_check_tables_host.argtypes = [P(hsla_config), i32, i32, vp, vp, i32, i32, i32, vp]
    lib.hsla_check_tables_host.restype = ctypes.c_int
    return lib


def status_string(status: int) -> str:
    return load().hsla_status_string(int(status)).decode()


def hsla_version() -> str:
    return load().hsla_version().decode()


# ----------------------------------------------------------------------------
# Argument marshalling
# ----------------------------------------------------------------------------

@dataclass
class Config:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int
    num_sink: int
    window: int
    linear_tail: int = 1
    kv_dtype: int = HSLA_BF16
    scale: float = 0.0
    selection: int = HSLA_SEL_PER_HEAD
    deterministic: int = 0
    state_span: int = HSLA_STATE_BLOCKS

    def c(self) -> hsla_config:
        return hsla_config(self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size, self.top_k,
                           self.num_sink, self.window, self.linear_tail, self.kv_dtype, self.scale,
                           self.selection, self.deterministic, self.state_span)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


@dataclass
class Pool:
    """Device tensors of the paged cache (see hsla_kv_pool)."""
    k_pages: object
    v_pages: object
    blk_mean: object
    blk_var: object
    block_table: object

    def c(self) -> hsla_kv_pool:
        return hsla_kv_pool(_ptr(self.k_pages), _ptr(self.v_pages), _ptr(self.blk_mean), _ptr(self.blk_var),
                            _ptr(self.block_table), int(self.block_table.shape[1]),
                            int(self.k_pages.shape[0]))


@dataclass
class State:
    """Device tensors of the global linear state (see hsla_state)."""
    S: object
    z: object
    sv: object

    def c(self) -> hsla_state:
        return hsla_state(_ptr(self.S), _ptr(self.z), _ptr(self.sv))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int) -> None:
    if status != HSLA_OK:
        raise HslaError(fn, status)


def hsla_build_workspace_size(cfg: Config, batch: int, max_seq_len: int) -> int:
    return int(load().hsla_build_workspace_size(ctypes.byref(cfg.c()), batch, max_seq_len))


def hsla_decode_workspace_size(cfg: Config, batch: int, max_seq_len: int) -> int:
    return int(load().hsla_decode_workspace_size(ctypes.byref(cfg.c()), batch, max_seq_len))


def hsla_build_state(cfg: Config, pool: Pool, state: State, seq_lens, batch: int, max_seq_len: int,
                     workspace, workspace_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check("hsla_build_state", load().hsla_build_state(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), ctypes.byref(state.c()), _ptr(seq_lens), batch,
        max_seq_len, _ptr(workspace), nbytes, _stream(stream)))


def hsla_append_token(cfg: Config, pool: Pool, state: State, k_new, v_new, seq_lens_before, seq_lens_after,
                      batch: int, max_seq_len: int, stream=None) -> None:
    _check("hsla_append_token", load().hsla_append_token(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), ctypes.byref(state.c()), _ptr(k_new), _ptr(v_new),
        _ptr(seq_lens_before), _ptr(seq_lens_after), batch, max_seq_len, _stream(stream)))


def hsla_decode(cfg: Config, pool: Pool, state: Optional[State], q, seq_lens, batch: int, max_seq_len: int,
                out, sel_idx, workspace, workspace_bytes: Optional[int] = None, stream=None,
                prof: Optional[hsla_profile] = None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    st = ctypes.byref(state.c()) if state is not None else None
    _check("hsla_decode", load().hsla_decode(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), st, _ptr(q), _ptr(seq_lens), batch, max_seq_len,
        _ptr(out), _ptr(sel_idx), _ptr(workspace), nbytes, _stream(stream),
        ctypes.byref(prof) if prof is not None else None))



def hsla_append_decode(cfg: Config, pool: Pool, state: State, k_new, v_new, seq_lens_before, seq_lens_after, q,
                       batch: int, max_seq_len: int, out, sel_idx, workspace, workspace_bytes: Optional[int] = None,
                       stream=None, prof: Optional[hsla_profile] = None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check("hsla_append_decode", load().hsla_append_decode(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), ctypes.byref(state.c()), _ptr(k_new), _ptr(v_new),
        _ptr(seq_lens_before), _ptr(seq_lens_after), _ptr(q), batch, max_seq_len, _ptr(out), _ptr(sel_idx),
        _ptr(workspace), nbytes, _stream(stream), ctypes.byref(prof) if prof is not None else None))


def hsla_noalloc_scratch_bytes() -> int:
    return int(load().hsla_noalloc_scratch_bytes())


def hsla_append_decode_noalloc(cfg: Config, pool: Pool, state: State, k_new, v_new, seq_lens_before, seq_lens_after,
                               q, batch: int, max_seq_len: int, out, sel_idx, stream=None) -> None:
    _check("hsla_append_decode_noalloc", load().hsla_append_decode_noalloc(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), ctypes.byref(state.c()), _ptr(k_new), _ptr(v_new),
        _ptr(seq_lens_before), _ptr(seq_lens_after), _ptr(q), batch, max_seq_len, _ptr(out), _ptr(sel_idx),
        _stream(stream)))


def hsla_check_tables(cfg: Config, pool: Pool, seq_lens, batch: int, max_seq_len: int, extra: int, result,
                      stream=None) -> None:
    """Enqueues the length / block-table check; `result` is a device int32[2]
    (violations, key of the first), valid once the stream has synchronised."""
    _check("hsla_check_tables", load().hsla_check_tables(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), _ptr(seq_lens), batch, max_seq_len, extra, _ptr(result),
        _stream(stream)))


def hsla_check_tables_host(cfg: Config, max_blocks_per_seq: int, num_pages: int, block_table, seq_lens,
                           batch: int, max_seq_len: int, extra: int):
    """The same check on host int32 arrays (numpy); no GPU.  Returns
    (status, violations, key of the first)."""
    import numpy as np
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    res = np.zeros(2, dtype=np.int32)
    st = load().hsla_check_tables_host(ctypes.byref(cfg.c()), max_blocks_per_seq, num_pages, bt.ctypes.data,
                                       lens.ctypes.data, batch, max_seq_len, extra, res.ctypes.data)
    return int(st), int(res[0]), int(res[1])


def hsla_prefill_chunk_workspace_size(cfg: Config, batch: int, q_len: int, max_seq_len: int) -> int:
    return int(load().hsla_prefill_chunk_workspace_size(ctypes.byref(cfg.c()), batch, q_len, max_seq_len))


def hsla_prefill_chunk(cfg: Config, pool: Pool, state: State, k_chunk, v_chunk, seq_lens_before, seq_lens_after,
                       q, batch: int, q_len: int, max_seq_len: int, out, sel_idx, workspace,
                       workspace_bytes: Optional[int] = None, stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace_bytes is None else workspace_bytes
    _check("hsla_prefill_chunk", load().hsla_prefill_chunk(
        ctypes.byref(cfg.c()), ctypes.byref(pool.c()), ctypes.byref(state.c()), _ptr(k_chunk), _ptr(v_chunk),
        _ptr(seq_lens_before), _ptr(seq_lens_after), _ptr(q), batch, q_len, max_seq_len, _ptr(out), _ptr(sel_idx),
        _ptr(workspace), nbytes, _stream(stream)))


load()
