"""Comparison rules between the HIP path and the fp64 oracle.

* Selections: the spec rule.  Let t_k and t_k1 be the oracle's k-th and
  (k+1)-th best candidate scores.  When t_k - t_k1 > 1e-5 * max(|t_k|, |t_k1|)
  the GPU's selected indices must equal the oracle's exactly.  Otherwise the
  blocks whose score lies within 1e-5 * |t_k| of t_k are interchangeable and
  every other block must match; the oracle is then re-run with the GPU's
  selection before outputs are compared.
* Outputs: row-normwise max relative error, max_row ||o - o_ref||_inf /
  ||o_ref||_inf, at most 2e-3 for bf16 keys/values and 1e-5 for fp32.
"""
from __future__ import annotations

import numpy as np

import oracle as O

SEL_REL = 1e-5
OUT_TOL = {"bf16": 2e-3, "f32": 1e-5}


def gpu_selection(row: np.ndarray) -> list:
    return [int(x) for x in row if x >= 0]


def check_selection(res: "O.HeadResult", gpu_sel: list, k: int):
    """Returns (ok, near_tie_flip, message)."""
    ref = res.selected.tolist()
    if gpu_sel != sorted(gpu_sel):
        return False, False, f"not ascending: {gpu_sel}"
    n = len(res.candidates)
    if k >= n or k == 0:
        return gpu_sel == ref, False, f"gpu {gpu_sel} oracle {ref}"
    order = np.argsort(-res.scores, kind="stable")
    tk = res.scores[order[k - 1]]
    tk1 = res.scores[order[k]]
    if tk - tk1 > SEL_REL * max(abs(tk), abs(tk1)):
        return gpu_sel == ref, False, f"gpu {gpu_sel} oracle {ref}"
    tol = SEL_REL * abs(tk)
    cand = res.candidates.tolist()
    near = {cand[i] for i in range(n) if abs(res.scores[i] - tk) <= tol}
    must = {cand[i] for i in range(n) if res.scores[i] > tk + tol}
    gs = set(gpu_sel)
    ok = len(gpu_sel) == k and must <= gs and gs <= (must | near)
    return ok, gs != set(ref), f"near-tie: gpu {gpu_sel} oracle {ref} near {sorted(near)}"


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(out - ref).max() / np.abs(ref).max())


def assert_stats_close(gpu_mean, gpu_var, ref_mean, ref_var, K, B, what=""):
    """fp32 two-pass block statistics against fp64: |err| <= B * 2^-24 times
    the block's magnitude, with a factor 4 of headroom."""
    nb = ref_mean.shape[0]
    assert gpu_mean.shape == ref_mean.shape and gpu_var.shape == ref_var.shape
    if nb == 0:
        return
    Kb = K[:nb * B].reshape(nb, B, -1)
    mag = np.abs(Kb).mean(axis=1)
    tol_m = 4 * B * 2.0 ** -24 * mag + 1e-30
    tol_v = 4 * B * 2.0 ** -24 * (Kb ** 2).mean(axis=1) + 1e-30
    em = np.abs(gpu_mean - ref_mean)
    ev = np.abs(gpu_var - ref_var)
    assert (em <= tol_m).all(), f"{what} mean err {em.max()} (max ratio {(em / tol_m).max():.2f})"
    assert (ev <= tol_v).all(), f"{what} var err {ev.max()} (max ratio {(ev / tol_v).max():.2f})"


def assert_state_close(gpu: "O.LinearState", ref: "O.LinearState", K, V, depth: int, what=""):
    """fp32 sums of T terms reduced with a tree of depth `depth` against fp64:
    |err| <= depth * 2^-24 * sum |terms| (summation error bound)."""
    u = 2.0 ** -24
    absS = np.abs(K).T @ np.abs(V)
    eS = np.abs(gpu.S - ref.S)
    assert (eS <= depth * u * absS + 1e-30).all(), f"{what} S err ratio {(eS / (depth * u * absS + 1e-30)).max():.2f}"
    ez = np.abs(gpu.z - ref.z)
    assert (ez <= depth * u * np.abs(K).sum(0) + 1e-30).all(), f"{what} z"
    esv = np.abs(gpu.sv - ref.sv)
    assert (esv <= depth * u * np.abs(V).sum(0) + 1e-30).all(), f"{what} sv"
