"""Seeded synthetic inputs for the hybrid sparse-plus-linear decode step.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers, rounds them to the stored precision,
plants needle blocks, draws ragged lengths and lays sequences out in a paged
pool.  It holds none of the method's arithmetic: no block statistics, scores,
selection, attention, linear state or merge.

Storage formats
---------------
* ``bf16`` tensors are numpy ``uint16`` arrays holding bfloat16 bit patterns,
  rounded from float32 with round-to-nearest-even.
* ``f32`` tensors are numpy ``float32`` arrays.

Seeding
-------
Every stream is ``numpy.random.default_rng([1000 + cid, stream, ...])`` (PCG64
through SeedSequence), so one (sequence, kv head) pair can be regenerated
without drawing the others.  Streams: 0 keys, 1 values, 2 queries, 3
per-channel scales, 4 needle placement and noise, 5 ragged lengths, 6 page
permutation, 7 per-layer budgets.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

BF16 = "bf16"
F32 = "f32"

S_KEYS, S_VALUES, S_QUERIES, S_SCALES, S_NEEDLES, S_LENGTHS, S_PAGES, S_BUDGETS = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, budgets and input recipe of one decode workload."""

    name: str
    cid: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int
    num_sink: int
    window: int
    linear_tail: int
    kv_dtype: str
    seq_lens: Tuple[int, ...]
    kv_scale_range: Optional[Tuple[float, float]] = None
    needles_per_pair: int = 0
    needle_gain: float = 3.0
    shuffle_pages: bool = False
    spare_pages: int = 0          # extra unmapped pages in the pool
    append_room: int = 1          # blocks mapped past the end of each sequence
    scale: float = 0.0            # 0 means 1/sqrt(head_dim)
    layer: int = 0
    grouped: int = 0              # one block selection per kv head
    deterministic: int = 0        # attention split: 0 the library's default, 1 fixed (bitwise reproducible), 2 dynamic
    tokens: int = 0               # token-level variant: top_k counts single tokens

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.kv_dtype == BF16 else 4

    @property
    def max_seq_len(self) -> int:
        return int(max(self.seq_lens)) if self.seq_lens else 0

    def blocks_mapped(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.block_size) + self.append_room

    @property
    def max_blocks_per_seq(self) -> int:
        return max(self.blocks_mapped(b) for b in range(self.batch))

    @property
    def num_pages(self) -> int:
        return sum(self.blocks_mapped(b) for b in range(self.batch)) + self.spare_pages


def _rng(wl: Workload, *key: int) -> np.random.Generator:
    return np.random.default_rng([1000 + wl.cid, *[int(k) for k in key]])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact).  Used to build needles."""
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_round(x) if wl.kv_dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def _as_f32(wl: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(x) if wl.kv_dtype == BF16 else x


# ----------------------------------------------------------------------------
# Named workloads
# ----------------------------------------------------------------------------

def _ragged_lengths(cid: int, batch: int, lo: int, hi: int) -> Tuple[int, ...]:
    rng = np.random.default_rng([1000 + cid, S_LENGTHS])
    return tuple(int(t) for t in rng.integers(lo, hi + 1, size=batch))


def tiny_f32() -> Workload:
    """Tiny fp32 decode: 1 kv head, GQA 4, d 64, 2048 tokens, block 64, k 4."""
    return Workload("tiny_f32_2k", 1, batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
                    block_size=64, top_k=4, num_sink=4, window=128, linear_tail=1,
                    kv_dtype=F32, seq_lens=(2048,))


def llama8b_32k() -> Workload:
    """Llama-3.1-8B-shaped layer: batch 8, 32q/8kv, d 128, 32K bf16 tokens, per-channel scales."""
    return Workload("llama8b_32k", 2, batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=64, top_k=16, num_sink=4, window=512, linear_tail=1,
                    kv_dtype=BF16, seq_lens=(32768,) * 8, kv_scale_range=(0.5, 2.0))


def needle_128k() -> Workload:
    """Long-context needles: batch 4, 32q/8kv, d 128, 128K bf16 tokens, block 128, k 32."""
    return Workload("needle_128k", 3, batch=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=128, top_k=32, num_sink=4, window=1024, linear_tail=1,
                    kv_dtype=BF16, seq_lens=(131072,) * 4, needles_per_pair=8, needle_gain=3.0)


def ragged_paged() -> Workload:
    """Ragged batch of 64 sequences, lengths ~U{1024..8192}, shuffled paged pool."""
    return Workload("ragged_paged_64", 4, batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    block_size=64, top_k=8, num_sink=4, window=256, linear_tail=1,
                    kv_dtype=BF16, seq_lens=_ragged_lengths(4, 64, 1024, 8192),
                    shuffle_pages=True, spare_pages=64)


HYBRID_LAYERS = 32


def hybrid_layers(num_layers: int = HYBRID_LAYERS, seq_len: int = 32768, batch: int = 1,
                  q_heads: int = 32, kv_heads: int = 8, cid: int = 5, name: str = "hybrid32_32k"):
    """Per-layer workloads of the build + 32-layer hybrid decode.

    Budgets are drawn per layer from {4, 8, 16, 32}; every fourth layer
    (l % 4 == 3) runs with the linear tail switched off (pure block-sparse).
    """
    rng = np.random.default_rng([1000 + cid, S_BUDGETS])
    budgets = rng.choice(np.array([4, 8, 16, 32]), size=num_layers)
    out = []
    for l in range(num_layers):
        out.append(Workload(f"{name}_l{l}", cid, batch=batch, num_q_heads=q_heads,
                            num_kv_heads=kv_heads, head_dim=128, block_size=64,
                            top_k=int(budgets[l]), num_sink=4, window=512,
                            linear_tail=0 if l % 4 == 3 else 1, kv_dtype=BF16,
                            seq_lens=(seq_len,) * batch, layer=l))
    return out


# Reduced versions that the fp64 oracle finishes in seconds; they still span
# several blocks, splits and a ragged tail.
def small(name: str) -> Workload:
    if name == "tiny_f32_2k":
        return tiny_f32()
    if name == "llama8b_small":
        return Workload(name, 12, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=64, top_k=16, num_sink=4, window=512, linear_tail=1,
                        kv_dtype=BF16, seq_lens=(4133, 3001), kv_scale_range=(0.5, 2.0),
                        shuffle_pages=True, spare_pages=3)
    if name == "needle_small":
        return Workload(name, 13, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=128, top_k=8, num_sink=4, window=1024, linear_tail=1,
                        kv_dtype=BF16, seq_lens=(9000, 8300), needles_per_pair=8,
                        needle_gain=3.0, shuffle_pages=True)
    if name == "ragged_small":
        return Workload(name, 14, batch=6, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        block_size=64, top_k=8, num_sink=4, window=256, linear_tail=1,
                        kv_dtype=BF16, seq_lens=_ragged_lengths(14, 6, 1024, 3000),
                        shuffle_pages=True, spare_pages=6)
    raise KeyError(name)


def hybrid_small():
    return hybrid_layers(num_layers=4, seq_len=4099, batch=1, q_heads=8, kv_heads=2,
                         cid=15, name="hybrid4_small")


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------

def channel_scales(wl: Workload) -> Optional[np.ndarray]:
    """Per (kv head, channel) scales for keys [0] and values [1], shared over batch and tokens."""
    if wl.kv_scale_range is None:
        return None
    lo, hi = wl.kv_scale_range
    return _rng(wl, S_SCALES, wl.layer).uniform(lo, hi, size=(2, wl.num_kv_heads, wl.head_dim)).astype(np.float32)


def gen_queries(wl: Workload, variant: int = 0) -> np.ndarray:
    """Queries [batch, Hq, d] in storage format, N(0,1) before rounding."""
    q = np.empty((wl.batch, wl.num_q_heads, wl.head_dim), np.float32)
    for b in range(wl.batch):
        q[b] = _rng(wl, S_QUERIES, b, variant, wl.layer).standard_normal(
            (wl.num_q_heads, wl.head_dim), dtype=np.float32)
    return _store(wl, q)


def needle_plan(wl: Workload, b: int, g: int):
    """[(block, q head)] of the planted needle blocks of pair (b, g).

    Blocks are distinct, drawn from the full blocks that end before the
    window (block 0, which holds the sinks, is never used); needle i is aimed
    at q head G*g + (i mod G).
    """
    if wl.needles_per_pair == 0:
        return []
    T, B = int(wl.seq_lens[b]), wl.block_size
    hi = (T - wl.window) // B          # blocks [1, hi) end before the window
    pool = np.arange(1, hi)
    rng = _rng(wl, S_NEEDLES, b, g, wl.layer)
    blocks = np.sort(rng.choice(pool, size=min(wl.needles_per_pair, len(pool)), replace=False))
    return [(int(blk), wl.group * g + (i % wl.group)) for i, blk in enumerate(blocks)]


def gen_pair(wl: Workload, b: int, g: int, q: Optional[np.ndarray] = None):
    """Keys and values [T_b, d] (storage format) of sequence b, kv head g.

    Keys and values are N(0,1) (times the per-channel scale when the workload
    has one).  Needle blocks get keys 3 * q_hat + N(0, I), where q_hat is the
    unit-norm query of the head the needle is aimed at.
    """
    T, d = int(wl.seq_lens[b]), wl.head_dim
    K = _rng(wl, S_KEYS, b, g, wl.layer).standard_normal((T, d), dtype=np.float32)
    V = _rng(wl, S_VALUES, b, g, wl.layer).standard_normal((T, d), dtype=np.float32)
    sc = channel_scales(wl)
    if sc is not None:
        K *= sc[0, g][None, :]
        V *= sc[1, g][None, :]
    plan = needle_plan(wl, b, g)
    if plan:
        if q is None:
            q = gen_queries(wl)
        rng = _rng(wl, S_NEEDLES, b, g, wl.layer, 1)
        B = wl.block_size
        for blk, h in plan:
            qf = _as_f32(wl, q[b, h]).astype(np.float32)
            qhat = qf / np.float32(np.sqrt(np.sum(qf.astype(np.float64) ** 2)))
            noise = rng.standard_normal((B, d), dtype=np.float32)
            K[blk * B:(blk + 1) * B] = np.float32(wl.needle_gain) * qhat[None, :] + noise
    return _store(wl, K), _store(wl, V)


def gen_token(wl: Workload, step: int):
    """New (k, v) [batch, Hkv, d] for the append of decode step `step`."""
    k = _rng(wl, S_KEYS, 1 << 20, step, wl.layer).standard_normal(
        (wl.batch, wl.num_kv_heads, wl.head_dim), dtype=np.float32)
    v = _rng(wl, S_VALUES, 1 << 20, step, wl.layer).standard_normal(
        (wl.batch, wl.num_kv_heads, wl.head_dim), dtype=np.float32)
    return _store(wl, k), _store(wl, v)


def page_table(wl: Workload) -> np.ndarray:
    """Block table [batch, max_blocks_per_seq] int32 into a pool of wl.num_pages pages.

    Each sequence maps ceil(T_b / B) + append_room blocks.  Pages are handed
    out in order, or through a seeded random permutation of the pool when the
    workload shuffles pages.  Unmapped slots hold 0.
    """
    P = wl.num_pages
    perm = _rng(wl, S_PAGES).permutation(P) if wl.shuffle_pages else np.arange(P)
    table = np.zeros((wl.batch, wl.max_blocks_per_seq), np.int32)
    nxt = 0
    for b in range(wl.batch):
        nb = wl.blocks_mapped(b)
        table[b, :nb] = perm[nxt:nxt + nb]
        nxt += nb
    return table


def empty_pool(wl: Workload) -> np.ndarray:
    dt = np.uint16 if wl.kv_dtype == BF16 else np.float32
    return np.zeros((wl.num_pages, wl.num_kv_heads, wl.block_size, wl.head_dim), dt)


def scatter_pairs(wl: Workload, table: np.ndarray, pool: np.ndarray, b: int, g: int, X: np.ndarray):
    """Write one pair's contiguous [T, d] tensor into its pages."""
    B = wl.block_size
    T = X.shape[0]
    nb = -(-T // B)
    Xp = np.zeros((nb * B, X.shape[1]), X.dtype)
    Xp[:T] = X
    pool[table[b, :nb], g] = Xp.reshape(nb, B, X.shape[1])


def gather_pair(wl: Workload, table: np.ndarray, pool: np.ndarray, b: int, g: int) -> np.ndarray:
    """Read one pair's contiguous [T_b, d] tensor back out of its pages."""
    B, T = wl.block_size, int(wl.seq_lens[b])
    nb = -(-T // B)
    return pool[table[b, :nb], g].reshape(nb * B, -1)[:T]


def make_inputs(wl: Workload, variant: int = 0, keep_pairs: bool = True):
    """All inputs of one workload: queries, paged pools, block table, lengths.

    Returns a dict with q [batch, Hq, d], k_pages / v_pages
    [num_pages, Hkv, B, d], block_table, seq_lens (int32) and, when
    keep_pairs, the contiguous per-pair tensors under 'pairs'[(b, g)].
    """
    q = gen_queries(wl, variant)
    table = page_table(wl)
    kp, vp = empty_pool(wl), empty_pool(wl)
    pairs = {}
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            K, V = gen_pair(wl, b, g, q)
            scatter_pairs(wl, table, kp, b, g, K)
            scatter_pairs(wl, table, vp, b, g, V)
            if keep_pairs:
                pairs[(b, g)] = (K, V)
    return dict(q=q, k_pages=kp, v_pages=vp, block_table=table,
                seq_lens=np.asarray(wl.seq_lens, np.int32), pairs=pairs)
