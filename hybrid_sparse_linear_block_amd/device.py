"""Device-memory plumbing around the libhsla entry points.

`DeviceCache` owns the torch tensors of one paged KV cache (pages, block
statistics, linear state, block table, lengths, workspaces) and calls the
C ABI through the binding.  torch is used for memory and streams only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (HSLA_BF16, HSLA_F32, HSLA_SEL_GROUPED, HSLA_SEL_PER_HEAD, HSLA_SEL_TOKEN, Config, Pool, State,
               hsla_append_decode, hsla_prefill_chunk, hsla_prefill_chunk_workspace_size,
               hsla_append_token, hsla_build_state, hsla_build_workspace_size, hsla_decode,
               hsla_decode_workspace_size)


def to_device(x: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are taken as bfloat16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy; bfloat16 becomes uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceCache:
    def __init__(self, cfg: Config, k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, capacity_len: Optional[int] = None, device="cuda"):
        self.cfg = cfg
        self.device = device
        self.k_pages = to_device(k_pages, device)
        self.v_pages = to_device(v_pages, device)
        P, Hkv, B, d = self.k_pages.shape
        assert Hkv == cfg.num_kv_heads and B == cfg.block_size and d == cfg.head_dim
        assert (self.k_pages.dtype == torch.bfloat16) == (cfg.kv_dtype == HSLA_BF16)
        self.batch = int(block_table.shape[0])
        f32 = dict(dtype=torch.float32, device=device)
        self.blk_mean = torch.zeros((P, Hkv, d), **f32)
        self.blk_var = torch.zeros((P, Hkv, d), **f32)
        self.S = torch.zeros((self.batch, Hkv, d, d), **f32)
        self.z = torch.zeros((self.batch, Hkv, d), **f32)
        self.sv = torch.zeros((self.batch, Hkv, d), **f32)
        self.block_table = to_device(block_table.astype(np.int32), device)
        self.host_lens = np.asarray(seq_lens, np.int64).copy()
        self.lens = [to_device(self.host_lens.astype(np.int32), device),
                     torch.zeros(self.batch, dtype=torch.int32, device=device)]
        self.cur = 0
        cap = int(capacity_len if capacity_len is not None else self.host_lens.max())
        cap = min(cap, int(block_table.shape[1]) * B)
        self.capacity_len = cap
        self.pool = Pool(self.k_pages, self.v_pages, self.blk_mean, self.blk_var, self.block_table)
        self.state = State(self.S, self.z, self.sv)
        self.build_ws = torch.empty(max(16, hsla_build_workspace_size(cfg, self.batch, cap)),
                                    dtype=torch.uint8, device=device)
        self.decode_ws = torch.empty(max(16, hsla_decode_workspace_size(cfg, self.batch, cap)),
                                     dtype=torch.uint8, device=device)

    @property
    def seq_lens(self) -> torch.Tensor:
        return self.lens[self.cur]

    @property
    def max_seq_len(self) -> int:
        return int(self.host_lens.max())

    def build(self, stream=None) -> None:
        hsla_build_state(self.cfg, self.pool, self.state, self.seq_lens, self.batch, self.max_seq_len,
                         self.build_ws, stream=stream)

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
        assert self.max_seq_len + 1 <= self.capacity_len, "no room mapped for the appended token"
        nxt = 1 - self.cur
        hsla_append_token(self.cfg, self.pool, self.state, k_new, v_new, self.lens[self.cur], self.lens[nxt],
                          self.batch, self.max_seq_len + 1, stream=stream)
        self.cur = nxt
        self.host_lens += 1

    def append_decode(self, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      out: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None, stream=None, prof=None):
        """Append one token per (sequence, kv head), then decode at the grown
        lengths, in one call."""
        cfg = self.cfg
        assert self.max_seq_len + 1 <= self.capacity_len, "no room mapped for the appended token"
        if out is None:
            out = torch.empty((self.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=self.device)
        if sel is None and cfg.top_k > 0:
            sel = torch.empty((self.batch, cfg.num_q_heads, cfg.top_k), dtype=torch.int32, device=self.device)
        nxt = 1 - self.cur
        hsla_append_decode(cfg, self.pool, self.state, k_new, v_new, self.lens[self.cur], self.lens[nxt], q,
                           self.batch, self.max_seq_len + 1, out, sel, self.decode_ws, stream=stream, prof=prof)
        self.cur = nxt
        self.host_lens += 1
        return out, sel

    def prefill_chunk(self, k_chunk: torch.Tensor, v_chunk: torch.Tensor, q: torch.Tensor,
                      out: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None, stream=None):
        """Append a chunk of Q tokens per sequence (k/v [batch, Q, Hkv, D]) and
        decode each of its queries (q [batch, Q, Hq, D]) at its own position."""
        cfg = self.cfg
        Q = int(q.shape[1])
        assert self.max_seq_len + Q <= self.capacity_len, "no room mapped for the chunk"
        if out is None:
            out = torch.empty((self.batch, Q, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=self.device)
        if sel is None and cfg.top_k > 0:
            sel = torch.empty((self.batch, Q, cfg.num_q_heads, cfg.top_k), dtype=torch.int32, device=self.device)
        msl = self.capacity_len   # one workspace for every chunk up to the mapped capacity
        key = (Q, msl)
        if getattr(self, "_chunk_ws_key", None) != key:
            n = hsla_prefill_chunk_workspace_size(cfg, self.batch, Q, msl)
            assert n > 0, "chunk length not supported for this configuration"
            self._chunk_ws = torch.empty(n, dtype=torch.uint8, device=self.device)
            self._chunk_ws_key = key
        nxt = 1 - self.cur
        hsla_prefill_chunk(cfg, self.pool, self.state, k_chunk, v_chunk, self.lens[self.cur], self.lens[nxt], q,
                           self.batch, Q, msl, out, sel, self._chunk_ws, stream=stream)
        self.cur = nxt
        self.host_lens += Q
        return out, sel

    def decode(self, q: torch.Tensor, out: Optional[torch.Tensor] = None, sel: Optional[torch.Tensor] = None,
               want_sel: bool = True, stream=None, prof=None):
        cfg = self.cfg
        if out is None:
            out = torch.empty((self.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=self.device)
        if sel is None and want_sel and cfg.top_k > 0:
            sel = torch.empty((self.batch, cfg.num_q_heads, cfg.top_k), dtype=torch.int32, device=self.device)
        hsla_decode(cfg, self.pool, self.state if cfg.linear_tail else None, q, self.seq_lens, self.batch,
                    self.max_seq_len, out, sel, self.decode_ws, stream=stream, prof=prof)
        return out, sel


def config_for(num_q_heads, num_kv_heads, head_dim, block_size, top_k, num_sink, window, linear_tail,
               kv_dtype: str, scale: float = 0.0, grouped: int = 0, deterministic: int = 0,
               tokens: int = 0, state_span: int = 0) -> Config:
    sel = HSLA_SEL_TOKEN if tokens else (HSLA_SEL_GROUPED if grouped else HSLA_SEL_PER_HEAD)
    return Config(num_q_heads, num_kv_heads, head_dim, block_size, top_k, num_sink, window, linear_tail,
                  HSLA_BF16 if kv_dtype == "bf16" else HSLA_F32, scale, sel, int(deterministic), int(state_span))


class PreparedDecodeStep:
    """One decode step (append + decode) of a DeviceCache with every C
    argument marshalled once, so that repeated calls cost one ctypes call per
    entry point.  Lengths ping-pong between the cache's two length buffers;
    each call advances the cache by one token.

    `fused` makes the step one hsla_append_decode call instead of
    hsla_append_token + hsla_decode.

    `bound`, if set, is passed as max_seq_len to both calls in place of the
    current length: an upper bound that stays valid while the cache grows,
    which a captured HIP graph needs since it replays its arguments as
    captured.  `stream` (a HIP stream handle) may be changed between calls."""

    def __init__(self, dc: DeviceCache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                 out: torch.Tensor, sel: Optional[torch.Tensor], stream=None, fused: bool = False):
        import ctypes

        from . import hsla_profile, load
        self.lib = load()
        self.dc = dc
        self.keep = (q, k_new, v_new, out, sel)
        self.cfg = dc.cfg.c()
        self.pool = dc.pool.c()
        self.state = dc.state.c()
        self.stream = (torch.cuda.current_stream() if stream is None else stream).cuda_stream
        self.q, self.k, self.v = q.data_ptr(), k_new.data_ptr(), v_new.data_ptr()
        self.out = out.data_ptr()
        self.sel = sel.data_ptr() if sel is not None else None
        self.ws = dc.decode_ws.data_ptr()
        self.ws_bytes = dc.decode_ws.numel()
        self.lens = [dc.lens[0].data_ptr(), dc.lens[1].data_ptr()]
        self.byref = ctypes.byref
        self.prof_type = hsla_profile
        self.bound: Optional[int] = None
        self.fused = fused

    def __call__(self, prof=None, between=None) -> None:
        """One step; `between`, if given, is called after the append was
        enqueued and before the decode is."""
        dc = self.dc
        assert dc.max_seq_len + 1 <= dc.capacity_len
        cur, nxt = dc.cur, 1 - dc.cur
        br = self.byref
        bound = self.bound
        if self.fused:
            st = self.lib.hsla_append_decode(br(self.cfg), br(self.pool), br(self.state), self.k, self.v,
                                             self.lens[cur], self.lens[nxt], self.q, dc.batch,
                                             dc.max_seq_len + 1 if bound is None else bound, self.out, self.sel,
                                             self.ws, self.ws_bytes, self.stream,
                                             br(prof) if prof is not None else None)
            if st != 0:
                raise RuntimeError(f"hsla_append_decode failed: {st}")
            dc.cur = nxt
            dc.host_lens += 1
            return
        st = self.lib.hsla_append_token(br(self.cfg), br(self.pool), br(self.state), self.k, self.v,
                                        self.lens[cur], self.lens[nxt], dc.batch,
                                        dc.max_seq_len + 1 if bound is None else bound, self.stream)
        if st != 0:
            raise RuntimeError(f"hsla_append_token failed: {st}")
        dc.cur = nxt
        dc.host_lens += 1
        if between is not None:
            between()
        st = self.lib.hsla_decode(br(self.cfg), br(self.pool), br(self.state), self.q, self.lens[nxt], dc.batch,
                                  dc.max_seq_len if bound is None else bound, self.out, self.sel, self.ws,
                                  self.ws_bytes, self.stream,
                                  br(prof) if prof is not None else None)
        if st != 0:
            raise RuntimeError(f"hsla_decode failed: {st}")

    def decode_only(self) -> None:
        """The decode of the current length, without an append (the cache
        does not change)."""
        dc = self.dc
        st = self.lib.hsla_decode(self.byref(self.cfg), self.byref(self.pool), self.byref(self.state), self.q,
                                  self.lens[dc.cur], dc.batch, dc.max_seq_len, self.out, self.sel, self.ws,
                                  self.ws_bytes, self.stream, None)
        if st != 0:
            raise RuntimeError(f"hsla_decode failed: {st}")
