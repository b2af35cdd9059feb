"""Plain fp64 CPU oracle of the single-token decode step of hybrid
sparse-plus-linear attention, and of the block statistics / linear state it
reads.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its binding) never does; it shares no code,
table or helper with this file.

Sources (page title, then the part of the page):

* [SPLA] "SPLA: Block Sparse Plus Linear Attention for Long Context Modeling"
  -- TL;DR, Abstract, table of contents (sections "Page Attention and
  Selection", "Principled Block Selection via Taylor Expansion", "Residual
  Linear Attention (RLA)", "Recurrence"), Figure 1.
* [SALSA] "SALSA: Training-Consistent Sparse Caching with Sink Preservation
  for Linearized LLMs" -- abstract (sliding window, sparse global cache,
  linear hidden state, initial sink tokens).
* [SLAKE] "SLAKE: Softmax-Approximated Training-Free Linear Attention with
  KV-Cache Eviction for Long-Sequence LLMs" -- abstract (PTAA: first-order
  Taylor linearisation of the softmax kernel for low-importance tokens).
* [SALS] "SALS: Sparse Attention in Latent Space for KV Cache Compression"
  -- summary, Approach (top-k token selection; here on the plain keys).

Every function is pinned by the CPU tests (hand-derived goldens, closed
forms, brute force on tiny inputs, invariants); none is parity unpinned.

None of the pages prints a formula, so every step below states the reading
it implements.  Everything is float64; stored inputs (bfloat16 bit patterns
or float32) are converted to float64 exactly before any arithmetic.

Notation: T tokens in the cache including the current one, B block size,
d head dim, sigma = 1/sqrt(d) unless a scale is given, ns sink tokens,
W window length, k the per-head block budget.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# Stored formats
# ----------------------------------------------------------------------------

def to_f64(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored tensor -> float64, exactly.  'bf16' arrays hold bit patterns."""
    if kv_dtype == "bf16":
        return (np.ascontiguousarray(x).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


@dataclasses.dataclass(frozen=True)
class Params:
    """The problem statement's parameters (GQA heads, block, budget, sinks, window)."""

    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    top_k: int
    num_sink: int
    window: int
    linear_tail: int = 1
    scale: float = 0.0
    grouped: int = 0   # 1: one selection shared by the G query heads of a kv head
    tokens: int = 0    # 1: top_k counts single tokens, scored by their own keys (token-level variant)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sigma(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.head_dim)


# ----------------------------------------------------------------------------
# O1: GQA grouping -- query head h reads kv head h // G (contiguous groups).
# ----------------------------------------------------------------------------

def kv_head_of(h: int, p: Params) -> int:
    return h // p.group


# ----------------------------------------------------------------------------
# O3: block statistics.  [SPLA TL;DR, Abstract: selection from "block
# statistics"]  Blocks are aligned at token 0; only full blocks have
# statistics.  mean = (1/B) sum_t k_t; var_c = (1/B) sum_t (k_tc - mean_c)^2
# (population variance, diagonal only), computed in two passes.
# ----------------------------------------------------------------------------

def block_statistics(K: np.ndarray, B: int):
    """K [T, d] float64 -> (mean [nb, d], var [nb, d]) over the nb = T // B full blocks."""
    T, d = K.shape
    nb = T // B
    mean = np.zeros((nb, d))
    var = np.zeros((nb, d))
    for b in range(nb):
        blk = K[b * B:(b + 1) * B]
        mu = blk.sum(axis=0) / B
        mean[b] = mu
        var[b] = ((blk - mu) ** 2).sum(axis=0) / B
    return mean, var


# ----------------------------------------------------------------------------
# O4: block score.  [SPLA, section "Principled Block Selection via Taylor
# Expansion"; Abstract: "second-order Taylor expansions"]
# Reading: expand exp(sigma q.k) to second order around k = mean_b and
# average over the block's tokens.  The first-order term averages to zero and
# the second-order term gives (1/2) sigma^2 q^T Cov_b q; with the diagonal
# variance this is exp(sigma q.mean_b) * (1 + sigma^2/2 sum_c q_c^2 var_bc).
# The score is its logarithm (a monotone map, so the ranking is unchanged).
# ----------------------------------------------------------------------------

def block_score(q: np.ndarray, mean: np.ndarray, var: np.ndarray, sigma: float) -> np.ndarray:
    """q [d], mean/var [nb, d] -> score [nb]."""
    first = sigma * (mean @ q)
    second = 0.5 * sigma * sigma * (var @ (q * q))
    return first + np.log1p(second)


# ----------------------------------------------------------------------------
# O5 / O6: sinks, window, candidates.  [SALSA abstract: sliding window plus
# initial sink tokens; SPLA Figure 1(a): block-level selection]
# The query is the current token, already in the cache at position T-1.
# Sinks are [0, ns), the window is [T-W, T) and includes the current token.
# Candidate blocks are those that intersect [ns, T-W); with W >= B they are
# all full blocks.
# ----------------------------------------------------------------------------

def sink_range(T: int, p: Params):
    return 0, min(p.num_sink, T)


def window_range(T: int, p: Params):
    return max(0, T - p.window), T


def candidate_blocks(T: int, p: Params) -> np.ndarray:
    """Block indices b with [bB, (b+1)B) intersecting [ns, T - W), ascending."""
    lo, hi = p.num_sink, T - p.window
    B = p.block_size
    return np.array([b for b in range(-(-T // B))
                     if b * B < hi and (b + 1) * B > lo and lo < hi], dtype=np.int64)


# ----------------------------------------------------------------------------
# Token-level variant.  ["SALS: Sparse Attention in Latent Space for KV
# Cache Compression", summary, Approach: top-k critical tokens picked by a
# score against each key; SALSA abstract: a sparse cache of selected tokens
# beside the window and the linear state.]
# Here the score is taken on the plain key (no latent projection):
# candidates are the tokens of [ns, T - W), a token's score is sigma q.k_t,
# and the top_k tokens by (score descending, index ascending) join the
# exact set; everything else is unchanged.
# ----------------------------------------------------------------------------

def candidate_tokens(T: int, p: Params) -> np.ndarray:
    """Token indices of [ns, T - W), ascending (empty when W covers the rest)."""
    lo, hi = p.num_sink, T - p.window
    return np.arange(lo, hi, dtype=np.int64) if lo < hi else np.zeros(0, np.int64)


def token_scores(q: np.ndarray, K: np.ndarray, cands: np.ndarray, sigma: float) -> np.ndarray:
    return sigma * (K[cands] @ q)


def select_top_k(cands: np.ndarray, scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) best candidates by (score descending, block index ascending),
    returned in ascending block order."""
    if k <= 0 or len(cands) == 0:
        return np.zeros(0, np.int64)
    order = sorted(range(len(cands)), key=lambda i: (-scores[i], cands[i]))
    chosen = [int(cands[i]) for i in order[:k]]
    return np.array(sorted(chosen), dtype=np.int64)


# ----------------------------------------------------------------------------
# Grouped selection (variant): one block selection shared by the G query
# heads of a kv head.  [SPLA table of contents, section "Grouped Sparsity";
# the section's text is not on the page.]
# Reading: a head's block score estimates the log of the head's attention
# mass on the block, so a softmax over the candidates gives the block's share
# of that head's candidate mass.  The group's weight of a block is the sum of
# these shares over its G heads (every head counts equally, whatever its
# score offset), and the k blocks of largest weight are taken, lower index
# first on ties.  With G = 1 this is the per-head selection.
# ----------------------------------------------------------------------------

def group_block_weights(scores_by_head: np.ndarray) -> np.ndarray:
    """scores [G, n] (one row per query head of the group) -> weight [n]."""
    G, n = scores_by_head.shape
    w = np.zeros(n)
    for h in range(G):
        s = scores_by_head[h]
        e = np.exp(s - s.max())
        w += e / e.sum()
    return w


def select_top_k_grouped(cands: np.ndarray, scores_by_head: np.ndarray, k: int) -> np.ndarray:
    """The shared selection of a group: top-k of the group weights, ascending."""
    if len(cands) == 0:
        return np.zeros(0, np.int64)
    return select_top_k(cands, group_block_weights(scores_by_head), k)


def group_selection(qs: np.ndarray, K: np.ndarray, p: Params, stats=None):
    """qs [G, d] (the group's queries), K [T, d] -> (candidates, per-head
    scores [G, n], group weights [n], shared selection)."""
    T = K.shape[0]
    cands = candidate_blocks(T, p)
    if stats is None:
        stats = block_statistics(K, p.block_size)
    mean, var = stats
    if len(cands) == 0:
        return cands, np.zeros((len(qs), 0)), np.zeros(0), np.zeros(0, np.int64)
    scores = np.stack([block_score(q, mean[cands], var[cands], p.sigma) for q in qs])
    w = group_block_weights(scores)
    return cands, scores, w, select_top_k(cands, w, p.top_k)


# ----------------------------------------------------------------------------
# O7: exact set E_h = sinks U window U selected blocks (a set: every token
# once); the residual set is U_h = [0, T) \ E_h.  [SPLA Figure 1(b); SALSA
# abstract: history split into window, sparse cache and linear state]
# ----------------------------------------------------------------------------

def exact_token_mask(T: int, selected: Sequence[int], p: Params) -> np.ndarray:
    E = np.zeros(T, dtype=bool)
    s0, s1 = sink_range(T, p)
    E[s0:s1] = True
    w0, w1 = window_range(T, p)
    E[w0:w1] = True
    B = 1 if p.tokens else p.block_size   # token-level: the selection holds token indices
    for b in selected:
        E[b * B:min((b + 1) * B, T)] = True
    return E


# ----------------------------------------------------------------------------
# O10 state: global linear state over all T tokens.  [SPLA Abstract: residual
# linear attention as "global minus selected"; section "Recurrence"; SLAKE
# abstract: first-order Taylor kernel]  With phi(q).phi(k) = 1 + sigma q.k the
# state is S = sum_t k_t v_t^T (d x d), z = sum_t k_t, sv = sum_t v_t, n = T.
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class LinearState:
    S: np.ndarray
    z: np.ndarray
    sv: np.ndarray
    n: int


def global_state(K: np.ndarray, V: np.ndarray) -> LinearState:
    return LinearState(S=K.T @ V, z=K.sum(axis=0), sv=V.sum(axis=0), n=K.shape[0])


def state_over(K: np.ndarray, V: np.ndarray, mask: np.ndarray) -> LinearState:
    """The same state built directly over the tokens where mask is True."""
    return global_state(K[mask], V[mask])


# ----------------------------------------------------------------------------
# O12: recurrence.  [SPLA section "Recurrence"]  Appending token (k, v) at
# position n updates S += k v^T, z += k, sv += v, n += 1; when the block that
# holds the new token becomes full its statistics are computed.
# ----------------------------------------------------------------------------

def append_token(state: LinearState, k: np.ndarray, v: np.ndarray) -> LinearState:
    return LinearState(S=state.S + np.outer(k, v), z=state.z + k, sv=state.sv + v, n=state.n + 1)


def filled_block_stats(K_after: np.ndarray, B: int):
    """After an append, the (block index, mean, var) of the block the new token
    completed, or None when that block is not full yet."""
    T = K_after.shape[0]
    if T % B != 0:
        return None
    b = T // B - 1
    blk = K_after[b * B:T]
    mu = blk.sum(axis=0) / B
    return b, mu, ((blk - mu) ** 2).sum(axis=0) / B


# ----------------------------------------------------------------------------
# O8-O11: one query head.
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class HeadResult:
    out: np.ndarray            # [d]
    selected: np.ndarray       # ascending block indices
    candidates: np.ndarray
    scores: np.ndarray         # per candidate
    exact: np.ndarray          # bool [T]
    num_u: np.ndarray          # residual numerator [d]
    den_u: float


def decode_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, p: Params, *,
                selected: Optional[Sequence[int]] = None,
                form: str = "subtraction",
                state: Optional[LinearState] = None,
                stats=None) -> HeadResult:
    """Decode output of one query head over one sequence's keys/values.

    q [d], K/V [T, d], all float64.  `selected` forces the block selection
    (used where near-ties allow several correct selections).  `form` picks
    the residual: 'definition' sums over U directly, 'subtraction' takes the
    global state minus the exact tokens' contribution (SPLA Abstract).

    Output (O11, merged in unshifted units since both parts approximate
    exp(s)):  o = (sum_E e^{s_t} v_t + num_U) / (sum_E e^{s_t} + den_U), with
    num_U = sum_U (1 + s_t) v_t and den_U = sum_U (1 + s_t), s_t = sigma q.k_t.
    Both are shifted by m = max_E s_t for range; that factor cancels.
    With the linear tail off, or U empty, num_U and den_U are exactly 0.
    """
    T, d = K.shape
    sig = p.sigma
    B = p.block_size
    if p.tokens:
        cands = candidate_tokens(T, p)
        scores = token_scores(q, K, cands, sig)
    else:
        cands = candidate_blocks(T, p)
        if stats is None:
            stats = block_statistics(K, B)
        mean, var = stats
        if len(cands):
            scores = block_score(q, mean[cands], var[cands], sig)
        else:
            scores = np.zeros(0)
    if selected is None:
        sel = select_top_k(cands, scores, p.top_k)
    else:
        sel = np.array(sorted(int(b) for b in selected), dtype=np.int64)
    E = exact_token_mask(T, sel, p)
    U = ~E

    s = sig * (K @ q)                       # O8
    sE = s[E]
    m = sE.max()
    wE = np.exp(sE - m)                     # O9
    A = wE @ V[E]
    L = wE.sum()

    if p.linear_tail and U.any():           # O10
        if form == "definition":
            num_u = (1.0 + s[U]) @ V[U]
            den_u = float((1.0 + s[U]).sum())
        elif form == "subtraction":
            st = state if state is not None else global_state(K, V)
            num_g = st.sv + sig * (st.S.T @ q)
            den_g = st.n + sig * float(q @ st.z)
            num_u = num_g - (1.0 + sE) @ V[E]
            den_u = den_g - float((1.0 + sE).sum())
        else:
            raise ValueError(form)
    else:
        num_u = np.zeros(d)
        den_u = 0.0

    em = math.exp(-m)                       # O11
    den = L + em * den_u
    assert den > 0, "merged denominator must be positive"
    out = (A + em * num_u) / den
    return HeadResult(out=out, selected=sel, candidates=cands, scores=scores,
                      exact=E, num_u=num_u, den_u=den_u)


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sigma: float) -> np.ndarray:
    """Plain softmax(sigma q K^T) V over all tokens (the k >= n_cand case)."""
    s = sigma * (K @ q)
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def decode_chunk_head(qc: np.ndarray, K: np.ndarray, V: np.ndarray, T0: int, p: Params, *,
                      selected: Optional[Sequence[Optional[Sequence[int]]]] = None,
                      form: str = "subtraction") -> list:
    """A chunk of Q consecutive queries of one head: the multi-query form of
    the decode step (SALSA abstract, training-consistent form over a tile of
    queries; SPLA Figure 1(a) partition per query).

    qc [Q, d]; K/V [T0 + Q, d] hold the cache's T0 tokens followed by the
    chunk's Q tokens.  Reading: query i sits at position T0 + i and sees the
    tokens 0 .. T0 + i (causal), so its output is the decode step at length
    T0 + i + 1 with its own candidates, selection, window, exact set and
    linear tail.  Returns one HeadResult per query.  `selected` may force a
    row's selection (near-ties), as in decode_head.
    """
    Q = qc.shape[0]
    assert K.shape[0] >= T0 + Q and V.shape[0] >= T0 + Q
    rows = []
    for i in range(Q):
        L = T0 + i + 1
        sel = None if selected is None else selected[i]
        rows.append(decode_head(qc[i], K[:L], V[:L], p, selected=sel, form=form))
    return rows


# ----------------------------------------------------------------------------
# Whole batch
# ----------------------------------------------------------------------------

def decode_batch(q: np.ndarray, pairs: dict, p: Params, seq_lens: Sequence[int], *,
                 heads=None, selected: Optional[dict] = None, form: str = "subtraction",
                 states: Optional[dict] = None, stats: Optional[dict] = None):
    """q [batch, Hq, d] and pairs[(b, g)] = (K, V) as float64.

    Returns {(b, h): HeadResult} for the requested (b, h) (all by default).
    `selected`, `states`, `stats` may hold per-(b, h) / per-(b, g) overrides.
    """
    batch, Hq, _ = q.shape
    if heads is None:
        heads = [(b, h) for b in range(batch) for h in range(Hq)]
    res = {}
    shared = {}   # grouped selection per (b, g)
    for b, h in heads:
        g = kv_head_of(h, p)
        K, V = pairs[(b, g)]
        assert K.shape[0] == seq_lens[b]
        sel = None if selected is None else selected.get((b, h))
        if sel is None and p.grouped:
            if (b, g) not in shared:
                G = p.group
                shared[(b, g)] = group_selection(q[b, g * G:(g + 1) * G], K, p,
                                                 stats=None if stats is None else stats.get((b, g)))[3]
            sel = shared[(b, g)]
        res[(b, h)] = decode_head(
            q[b, h], K, V, p,
            selected=sel,
            form=form,
            state=None if states is None else states.get((b, g)),
            stats=None if stats is None else stats.get((b, g)))
    return res
