"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case prints its name, seed and shape before touching the GPU."""
import dataclasses
import math
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import oracle as O
import workloads as W
from parity import (OUT_TOL, assert_state_close, assert_stats_close, check_selection, gpu_selection,
                    row_rel_err)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import hybrid_sparse_linear_block_amd as H  # noqa: E402
from hybrid_sparse_linear_block_amd.device import DeviceCache, config_for, to_device  # noqa: E402


def _announce(wl, extra=""):
    print(f"[case] {wl.name} cid={wl.cid} batch={wl.batch} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
          f"d={wl.head_dim} B={wl.block_size} k={wl.top_k} ns={wl.num_sink} W={wl.window} "
          f"lin={wl.linear_tail} {wl.kv_dtype} T={list(wl.seq_lens)[:8]} {extra}", flush=True)
    sys.stdout.flush()


def cfg_of(wl):
    return config_for(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k, wl.num_sink,
                      wl.window, wl.linear_tail, wl.kv_dtype, wl.scale, grouped=wl.grouped,
                      deterministic=wl.deterministic, tokens=wl.tokens)


def params_of(wl):
    return O.Params(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k, wl.num_sink,
                    wl.window, wl.linear_tail, wl.scale, grouped=wl.grouped, tokens=wl.tokens)


def run_gpu(wl, inp, capacity_len=None):
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                     capacity_len=capacity_len)
    dc.build()
    q = to_device(inp["q"])
    out, sel = dc.decode(q)
    torch.cuda.synchronize()
    return dc, out.cpu().numpy(), (None if sel is None else sel.cpu().numpy())


def state_depth(T):
    return min(T, 4096) + math.ceil(T / 32) + 16


def check_case(wl, inp, dc, out, sel, heads=None, check_build=True, pair_data=None):
    """Compares statistics, state, selections and outputs with the oracle.
    Returns (worst row error, number of near-tie flips)."""
    p = params_of(wl)
    B, G = wl.block_size, wl.group
    q64 = O.to_f64(inp["q"], wl.kv_dtype)
    table = inp["block_table"]
    if heads is None:
        heads = [(b, h) for b in range(wl.batch) for h in range(wl.num_q_heads)]
    pairs = sorted({(b, h // G) for b, h in heads})
    if check_build:
        mean_g, var_g = dc.blk_mean.cpu().numpy(), dc.blk_var.cpu().numpy()
        S_g, z_g, sv_g = dc.S.cpu().numpy(), dc.z.cpu().numpy(), dc.sv.cpu().numpy()
    cache = {}
    for b, g in pairs:
        if pair_data is not None:
            K, V = pair_data(b, g)
        else:
            K, V = inp["pairs"][(b, g)]
        Kf, Vf = O.to_f64(K, wl.kv_dtype), O.to_f64(V, wl.kv_dtype)
        stats = O.block_statistics(Kf, B)
        state = O.global_state(Kf, Vf)
        cache[(b, g)] = (Kf, Vf, stats, state)
        if check_build:
            T = Kf.shape[0]
            nb = T // B
            pages = table[b, :nb]
            assert_stats_close(mean_g[pages, g], var_g[pages, g], stats[0], stats[1], Kf, B, f"pair {(b, g)}")
            # the library's state holds the tokens of complete blocks
            Ts = nb * B
            gs = O.LinearState(S_g[b, g].astype(np.float64), z_g[b, g].astype(np.float64),
                               sv_g[b, g].astype(np.float64), Ts)
            assert_state_close(gs, O.global_state(Kf[:Ts], Vf[:Ts]), Kf[:Ts], Vf[:Ts], state_depth(Ts),
                               f"pair {(b, g)}")
    worst, flips = 0.0, 0
    shared = {}   # grouped selection: (candidates, group weights, selection) per pair
    for b, h in heads:
        g = h // G
        Kf, Vf, stats, state = cache[(b, g)]
        if wl.grouped:
            if (b, g) not in shared:
                cands, _, w, gsel = O.group_selection(q64[b, g * G:(g + 1) * G], Kf, p, stats=stats)
                shared[(b, g)] = SimpleNamespace(candidates=cands, scores=w, selected=gsel)
            ref_sel = shared[(b, g)]
            r = O.decode_head(q64[b, h], Kf, Vf, p, stats=stats, state=state, selected=ref_sel.selected)
        else:
            r = O.decode_head(q64[b, h], Kf, Vf, p, stats=stats, state=state)
            ref_sel = r
        if sel is not None:
            gs = gpu_selection(sel[b, h])
            ok, flip, msg = check_selection(ref_sel, gs, wl.top_k)
            assert ok, f"(b={b}, h={h}) {msg}"
            if flip:
                flips += 1
                r = O.decode_head(q64[b, h], Kf, Vf, p, stats=stats, state=state, selected=gs)
        assert np.isfinite(out[b, h]).all(), f"(b={b}, h={h}) non-finite output"
        err = row_rel_err(out[b, h], r.out)
        assert err <= OUT_TOL[wl.kv_dtype], f"(b={b}, h={h}) row error {err:.3e}"
        worst = max(worst, err)
    return worst, flips


# ----------------------------------------------------------------------------
# Reduced workloads: every head against the oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_f32_2k", "llama8b_small", "needle_small", "ragged_small"])
def test_small_workloads(name):
    wl = W.small(name)
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, flips = check_case(wl, inp, dc, out, sel)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


def test_hybrid_layers_small():
    for wl in W.hybrid_small():
        _announce(wl)
        inp = W.make_inputs(wl)
        dc, out, sel = run_gpu(wl, inp)
        worst, _ = check_case(wl, inp, dc, out, sel)
        print(f"  layer {wl.layer}: worst {worst:.3e}")


def test_needles_recalled_on_gpu():
    wl = W.small("needle_small")
    _announce(wl)
    inp = W.make_inputs(wl)
    _, _, sel = run_gpu(wl, inp)
    for b in range(wl.batch):
        for g in range(wl.num_kv_heads):
            for blk, h in W.needle_plan(wl, b, g):
                assert blk in sel[b, h].tolist(), (b, g, blk, h)


# ----------------------------------------------------------------------------
# Special cases and edge shapes
# ----------------------------------------------------------------------------

def _wl(name, cid, **kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64, top_k=6, num_sink=4,
                window=256, linear_tail=1, kv_dtype=W.BF16, seq_lens=(1500, 1203), shuffle_pages=True,
                spare_pages=2)
    base.update(kw)
    return W.Workload(name, cid, **base)


def test_dense_when_budget_covers_all_candidates():
    wl = _wl("dense_k", 30, top_k=40)          # 40 >= every n_cand here
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel)
    p = params_of(wl)
    for b in range(wl.batch):
        for h in range(wl.num_q_heads):
            K, V = inp["pairs"][(b, h // wl.group)]
            ref = O.dense_attention(O.to_f64(inp["q"][b, h], wl.kv_dtype), O.to_f64(K, wl.kv_dtype),
                                    O.to_f64(V, wl.kv_dtype), p.sigma)
            assert row_rel_err(out[b, h], ref) <= OUT_TOL[wl.kv_dtype]


def test_sinks_and_window_only():
    wl = _wl("sink_window", 31, top_k=0, linear_tail=0)
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel)


@pytest.mark.parametrize("lens", [(1, 5), (64, 260), (300, 261), (255, 320)])
@pytest.mark.parametrize("lin", [1, 0])
def test_short_sequences_have_no_candidates(lens, lin):
    """No candidate block anywhere in the batch; without the linear tail the
    scoring launch then has no work at all."""
    wl = _wl(f"short_{lens[0]}_{lens[1]}", 32, seq_lens=lens, window=256, num_sink=4, linear_tail=lin)
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel)


SHAPES = [
    # (G, d, B, dtype, ns, W, k, lin)
    (1, 128, 64, W.BF16, 4, 512, 8, 1),
    (8, 128, 64, W.BF16, 4, 512, 5, 1),
    (2, 64, 32, W.BF16, 0, 100, 7, 1),
    (4, 128, 16, W.BF16, 20, 48, 12, 1),
    (4, 128, 128, W.F32, 4, 256, 3, 1),
    (4, 64, 256, W.BF16, 300, 600, 2, 1),
    (4, 128, 256, W.BF16, 4, 256, 3, 0),
    (4, 64, 64, W.F32, 70, 130, 4, 1),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "G{}_d{}_B{}_{}_ns{}_W{}_k{}_lin{}".format(*s))
def test_shapes(shape):
    G, d, B, dt, ns, Wn, k, lin = shape
    wl = _wl("shape", 40 + SHAPES.index(shape), num_q_heads=2 * G, num_kv_heads=2, head_dim=d, block_size=B,
             kv_dtype=dt, num_sink=ns, window=Wn, top_k=k, linear_tail=lin, seq_lens=(2311, 1777))
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel)


def test_exact_ties_go_to_the_lower_block():
    """Blocks 5, 9 and 20 are copies of block 2, which is made to score high
    for the first query head of each group: with k = 3 the four-way tie at the
    top straddles the cut and must resolve to blocks 2, 5, 9."""
    wl = _wl("ties", 50, batch=1, seq_lens=(2048,), top_k=3, shuffle_pages=False)
    _announce(wl)
    inp = W.make_inputs(wl)
    B = wl.block_size
    rng = np.random.default_rng(7)
    for g in range(wl.num_kv_heads):
        K, V = inp["pairs"][(0, g)]
        qh = W.bf16_to_f32(inp["q"][0, g * wl.group])
        qhat = qh / np.sqrt((qh.astype(np.float64) ** 2).sum())
        K[2 * B:3 * B] = W.bf16_round(3.0 * qhat[None, :] + rng.standard_normal((B, wl.head_dim)))
        for dst in (5, 9, 20):
            K[dst * B:(dst + 1) * B] = K[2 * B:3 * B]
        W.scatter_pairs(wl, inp["block_table"], inp["k_pages"], 0, g, K)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel)
    for g in range(wl.num_kv_heads):
        assert gpu_selection(sel[0, g * wl.group]) == [2, 5, 9]


def test_page_order_does_not_change_results():
    wl1 = _wl("pages_a", 51, shuffle_pages=False, deterministic=1)
    wl2 = dataclasses.replace(wl1, name="pages_b", shuffle_pages=True, spare_pages=7)
    _announce(wl1)
    inp1, inp2 = W.make_inputs(wl1), W.make_inputs(wl2)
    _, o1, s1 = run_gpu(wl1, inp1)
    _, o2, s2 = run_gpu(wl2, inp2)
    assert np.array_equal(s1, s2)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_runs_are_bitwise_reproducible():
    """With the fixed split every bit repeats; the dynamic split (below)
    only changes the summation order."""
    wl = dataclasses.replace(W.small("llama8b_small"), deterministic=1)
    _announce(wl, "deterministic")
    inp = W.make_inputs(wl)
    dc, o1, s1 = run_gpu(wl, inp)
    S1 = dc.S.cpu().numpy().copy()
    dc.build()
    o2, s2 = dc.decode(to_device(inp["q"]))
    torch.cuda.synchronize()
    assert np.array_equal(S1.view(np.uint32), dc.S.cpu().numpy().view(np.uint32))
    assert np.array_equal(o1.view(np.uint32), o2.cpu().numpy().view(np.uint32))
    assert np.array_equal(s1, s2.cpu().numpy())


def test_dynamic_split_repeats_within_rounding():
    """The dynamic split: selections repeat exactly, outputs to fp32
    summation-order rounding, and both match the fixed split."""
    wl = dataclasses.replace(W.small("llama8b_small"), deterministic=2)
    _announce(wl, "dynamic vs fixed split")
    inp = W.make_inputs(wl)
    dc, o1, s1 = run_gpu(wl, inp)
    outs = [o1]
    for _ in range(3):
        o, s = dc.decode(to_device(inp["q"]))
        torch.cuda.synchronize()
        assert np.array_equal(s1, s.cpu().numpy())
        outs.append(o.cpu().numpy())
    _, od, sd = run_gpu(dataclasses.replace(wl, deterministic=1), inp)
    assert np.array_equal(s1, sd)
    for o in outs:
        for b in range(wl.batch):
            for h in range(wl.num_q_heads):
                assert row_rel_err(o[b, h], od[b, h]) < 1e-5, (b, h)


@pytest.mark.parametrize("name", ["llama8b_small", "needle_small", "ragged_small"])
def test_dynamic_split_workloads(name):
    """The reduced workloads with the dynamic split (HSLA_SPLIT_DYNAMIC;
    the default split is the fixed one) against the oracle."""
    wl = dataclasses.replace(W.small(name), deterministic=2)
    _announce(wl, "dynamic split")
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, flips = check_case(wl, inp, dc, out, sel, check_build=False)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


@pytest.mark.parametrize("dtype,fused", [(W.BF16, False), (W.F32, False), (W.BF16, True), (W.F32, True)])
def test_append_matches_rebuild(dtype, fused):
    """Decode after N appends (crossing block boundaries) equals the oracle on
    the full sequence, and the appended state matches a rebuild.  `fused`:
    every append goes through hsla_append_decode (the last call's output is
    the decode checked)."""
    N = 70
    full = _wl("append_full", 60, kv_dtype=dtype, seq_lens=(1400, 1250), append_room=3)
    start = dataclasses.replace(full, name="append_start", seq_lens=tuple(t - N for t in full.seq_lens))
    _announce(full, f"N={N}")
    inp_full = W.make_inputs(full)
    table = inp_full["block_table"]
    # Start from the first T-N tokens of every pair, laid out in the same pages.
    kp, vp = W.empty_pool(full), W.empty_pool(full)
    for (b, g), (K, V) in inp_full["pairs"].items():
        W.scatter_pairs(full, table, kp, b, g, K[:start.seq_lens[b]])
        W.scatter_pairs(full, table, vp, b, g, V[:start.seq_lens[b]])
    dc = DeviceCache(cfg_of(full), kp, vp, table, np.asarray(start.seq_lens, np.int32),
                     capacity_len=max(full.seq_lens))
    dc.build()
    q_dev = to_device(inp_full["q"])
    for i in range(N):
        kn = np.stack([np.stack([inp_full["pairs"][(b, g)][0][start.seq_lens[b] + i]
                                 for g in range(full.num_kv_heads)]) for b in range(full.batch)])
        vn = np.stack([np.stack([inp_full["pairs"][(b, g)][1][start.seq_lens[b] + i]
                                 for g in range(full.num_kv_heads)]) for b in range(full.batch)])
        if fused:
            out, sel = dc.append_decode(to_device(kn), to_device(vn), q_dev)
        else:
            dc.append(to_device(kn), to_device(vn))
    if not fused:
        out, sel = dc.decode(q_dev)
    torch.cuda.synchronize()
    assert dc.seq_lens.cpu().numpy().tolist() == list(full.seq_lens)
    inp_check = dict(inp_full)
    worst, _ = check_case(full, inp_check, dc, out.cpu().numpy(), sel.cpu().numpy(), check_build=False)
    # statistics and state after appends
    mean_g, var_g = dc.blk_mean.cpu().numpy(), dc.blk_var.cpu().numpy()
    for (b, g), (K, V) in inp_full["pairs"].items():
        Kf, Vf = O.to_f64(K, dtype), O.to_f64(V, dtype)
        Ts = Kf.shape[0] - Kf.shape[0] % full.block_size   # the state holds complete blocks
        st = O.global_state(Kf[:Ts], Vf[:Ts])
        gs = O.LinearState(dc.S[b, g].cpu().numpy().astype(np.float64), dc.z[b, g].cpu().numpy().astype(np.float64),
                           dc.sv[b, g].cpu().numpy().astype(np.float64), Ts)
        assert_state_close(gs, st, Kf[:Ts], Vf[:Ts], state_depth(Ts) + N)
        m, v = O.block_statistics(Kf, full.block_size)
        pages = table[b, :Kf.shape[0] // full.block_size]
        assert_stats_close(mean_g[pages, g], var_g[pages, g], m, v, Kf, full.block_size)


# ----------------------------------------------------------------------------
# Grouped selection: one selection per kv head
# ----------------------------------------------------------------------------

GROUPED = [
    # (name, workload overrides); the last two exceed the register-resident
    # key counts (G x ceil(n_cand / 64) > 64) and take the streaming path
    ("llama8b_small", {}),
    ("needle_small", {}),
    ("ragged_small", {}),
    ("tiny_f32_2k", {}),
    ("G8_B16_long", dict(num_q_heads=16, num_kv_heads=2, block_size=16, window=256, top_k=12,
                         seq_lens=(10017, 9601))),
    ("G4_B16_long", dict(block_size=16, window=256, top_k=20, seq_lens=(20011, 17000))),
]


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: c[0])
def test_grouped_selection(case):
    name, over = case
    if name in ("llama8b_small", "needle_small", "ragged_small", "tiny_f32_2k"):
        wl = dataclasses.replace(W.small(name), grouped=1)
    else:
        wl = dataclasses.replace(_wl("grouped_" + name, 70 + GROUPED.index(case), **over), grouped=1)
    _announce(wl, "grouped selection")
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, flips = check_case(wl, inp, dc, out, sel, check_build=False)
    G = wl.group
    for b in range(wl.batch):   # every head of a group carries the same selection
        for g in range(wl.num_kv_heads):
            for h in range(g * G + 1, (g + 1) * G):
                assert np.array_equal(sel[b, h], sel[b, g * G]), (b, h)
    if wl.needles_per_pair:
        for b in range(wl.batch):
            for g in range(wl.num_kv_heads):
                for blk, h in W.needle_plan(wl, b, g):
                    assert blk in sel[b, h].tolist(), (b, g, blk, h)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


LONG_ROWS = [
    # candidate rows past the register-resident sizes of the per-head
    # selection (n_cand > 1024 and > 2048), a block-table row too long to
    # stage in LDS (> 2048 blocks), and more than 64 chunks of 64 blocks in
    # the union prologue (> 4096 blocks)
    ("B16_20k", dict(block_size=16, window=256, top_k=20, seq_lens=(20011, 17000))),
    ("B16_40k", dict(block_size=16, window=256, top_k=24, seq_lens=(40000, 36999))),
    ("B16_70k", dict(batch=1, block_size=16, window=512, top_k=9, seq_lens=(70001,))),
    # the largest candidate row the attention prologue takes: 8 heads x
    # 256 bitmap words = 16 KB of LDS (16384 candidate blocks of 16 tokens)
    ("max_bitmap_G8", dict(batch=1, num_q_heads=8, num_kv_heads=1, head_dim=64, block_size=16, window=64, top_k=16,
                           seq_lens=(262208,), spare_pages=0)),
]


@pytest.mark.parametrize("case", LONG_ROWS, ids=lambda c: c[0])
def test_long_candidate_rows(case):
    name, over = case
    wl = _wl("long_" + name, 80 + LONG_ROWS.index(case), **over)
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, flips = check_case(wl, inp, dc, out, sel, check_build=False)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


# ----------------------------------------------------------------------------
# Merge by the last attention workgroup of each pair
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("deterministic", [1, 2])
def test_merge_in_last_workgroup(deterministic):
    """128 pairs, so two splits per pair: the attention kernel's last
    workgroup of each pair merges.  Outputs against the oracle, then
    alternating queries on the same cache: every call must match the first
    call with the same queries (a merge reading another call's partials
    would not)."""
    wl = _wl("merge_fused", 90, batch=16, num_q_heads=32, num_kv_heads=8,
             seq_lens=(2100, 1900, 2047, 1500, 1300, 1800, 2200, 1717, 1600, 2000, 1999, 1450, 2050, 1650, 1900, 1333),
             deterministic=deterministic)
    _announce(wl, "merge in the attention kernel")
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, _ = check_case(wl, inp, dc, out, sel, check_build=False)
    print(f"  worst row error {worst:.3e}")
    qs = [to_device(inp["q"]), to_device(W.gen_queries(wl, variant=1))]
    first = []
    for i in range(2):
        o, s = dc.decode(qs[i])
        torch.cuda.synchronize()
        first.append((o.cpu().numpy(), s.cpu().numpy()))
    assert not np.array_equal(first[0][0], first[1][0])
    for it in range(40):
        o, s = dc.decode(qs[it % 2])
        o, s = o.cpu().numpy(), s.cpu().numpy()
        ref_o, ref_s = first[it % 2]
        assert np.array_equal(s, ref_s), it
        if deterministic == 1:
            assert np.array_equal(o, ref_o), it
        else:
            for b in range(wl.batch):
                for h in range(wl.num_q_heads):
                    assert row_rel_err(o[b, h], ref_o[b, h]) < 1e-5, (it, b, h)


# ----------------------------------------------------------------------------
# Token-level variant: top_k single tokens per head, scored by their keys
# ----------------------------------------------------------------------------

TOKEN_CASES = [
    ("bf16_g4", dict(top_k=64, window=512, seq_lens=(4133, 3001))),
    ("bf16_g4_k300", dict(top_k=300, window=256, seq_lens=(2900, 2311), deterministic=1)),
    ("f32_d64", dict(kv_dtype=W.F32, head_dim=64, top_k=40, seq_lens=(1500, 1203))),
    ("g1", dict(num_q_heads=2, num_kv_heads=2, top_k=33, seq_lens=(1500, 977))),
    ("g2_b16", dict(num_q_heads=4, num_kv_heads=2, block_size=16, window=64, top_k=50, seq_lens=(1313, 700))),
    ("g8", dict(num_q_heads=16, num_kv_heads=2, top_k=70, seq_lens=(2600, 1900))),
    ("g8_f32_d64", dict(num_q_heads=16, num_kv_heads=2, kv_dtype=W.F32, head_dim=64, top_k=30, seq_lens=(1500, 900))),
    ("no_tail", dict(linear_tail=0, top_k=25, seq_lens=(1500, 1203))),
    ("dense", dict(top_k=4000, seq_lens=(1500, 1203))),
    ("short", dict(top_k=16, seq_lens=(200, 37))),
    ("batch4", dict(batch=4, top_k=128, seq_lens=(2000, 1999, 1024, 3000))),
]


@pytest.mark.parametrize("case", TOKEN_CASES, ids=lambda c: c[0])
def test_token_level_selection(case):
    name, over = case
    wl = _wl("tokens_" + name, 95 + TOKEN_CASES.index(case), tokens=1, **over)
    _announce(wl)
    inp = W.make_inputs(wl)
    dc, out, sel = run_gpu(wl, inp)
    worst, flips = check_case(wl, inp, dc, out, sel, check_build=False)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


@pytest.mark.parametrize("n", [1500, 2900])   # 1024-candidate register path and the workgroup radix path
def test_token_level_exact_ties_go_to_the_lower_token(n):
    """Tokens 40, 41, 700 and 900 hold copies of token 30's key, which is made
    to score high for the first query head of each group: with k = 3 the
    five-way tie at the top straddles the cut and must resolve to tokens 30,
    40, 41."""
    wl = _wl("token_ties", 110, batch=1, seq_lens=(n,), top_k=3, tokens=1, shuffle_pages=False)
    _announce(wl)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(8)
    for g in range(wl.num_kv_heads):
        K, V = inp["pairs"][(0, g)]
        qh = W.bf16_to_f32(inp["q"][0, g * wl.group])
        qhat = qh / np.sqrt((qh.astype(np.float64) ** 2).sum())
        K[30] = W.bf16_round(6.0 * qhat + 0.1 * rng.standard_normal(wl.head_dim))
        for dst in (40, 41, 700, 900):
            K[dst] = K[30]
        W.scatter_pairs(wl, inp["block_table"], inp["k_pages"], 0, g, K)
    dc, out, sel = run_gpu(wl, inp)
    check_case(wl, inp, dc, out, sel, check_build=False)
    for g in range(wl.num_kv_heads):
        assert gpu_selection(sel[0, g * wl.group]) == [30, 40, 41]
