"""Full-size workloads in the configuration the benchmark times.

Each workload runs at its real shape (batch, context, heads, paging); the
build and one decode step go through the C ABI exactly as in bench.py.  A
sample of (sequence, kv head) pairs -- first, last, a middle one and, for
ragged batches, the shortest and longest sequence -- is checked against the
fp64 oracle (statistics, state, selections, outputs of every query head of
the pair); every head of the batch is checked for the properties that hold
at any size (finite outputs, selections ascending, inside the candidate
range, of the right count).
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from test_gpu_parity import _announce, cfg_of, check_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from hybrid_sparse_linear_block_amd.device import DeviceCache, to_device  # noqa: E402

FULL = {"llama8b_32k": W.llama8b_32k, "needle_128k": W.needle_128k, "ragged_paged": W.ragged_paged,
        "llama8b_32k_grouped": lambda: W.dataclasses.replace(W.llama8b_32k(), grouped=1),
        # token-level variant with the block budget's token count (16 x 64)
        "llama8b_32k_tokens": lambda: W.dataclasses.replace(W.llama8b_32k(), tokens=1, top_k=1024)}


def run_full(wl, inp):
    # room for one appended token, as the benchmark maps it
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                     capacity_len=int(max(wl.seq_lens)) + 1)
    dc.build()
    out, sel = dc.decode(to_device(inp["q"]))
    torch.cuda.synchronize()
    return dc, out.cpu().numpy(), sel.cpu().numpy()


def sampled_pairs(wl):
    lens = np.asarray(wl.seq_lens)
    picks = {(0, 0), (wl.batch - 1, wl.num_kv_heads - 1), (wl.batch // 2, wl.num_kv_heads // 2),
             (int(lens.argmin()), 1 % wl.num_kv_heads), (int(lens.argmax()), 2 % wl.num_kv_heads)}
    return sorted(picks)


def check_properties(wl, out, sel):
    assert np.isfinite(out).all(), "non-finite outputs"
    B, k = (1 if wl.tokens else wl.block_size), wl.top_k   # token-level rows hold token indices
    for b in range(wl.batch):
        T = int(wl.seq_lens[b])
        lo = wl.num_sink // B
        hi_tok = T - wl.window
        nc = 0 if hi_tok <= wl.num_sink else -(-hi_tok // B) - lo
        for h in range(wl.num_q_heads):
            row = sel[b, h]
            got = row[row >= 0]
            assert (row[len(got):] == -1).all(), (b, h, row)
            assert len(got) == min(k, nc), (b, h, row)
            assert (np.diff(got) > 0).all(), (b, h, row)
            if len(got):
                assert got[0] >= lo and got[-1] < lo + nc, (b, h, row)


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_workload(name):
    wl = FULL[name]()
    _announce(wl, "full size, sampled pairs")
    inp = W.make_inputs(wl, keep_pairs=False)
    dc, out, sel = run_full(wl, inp)
    check_properties(wl, out, sel)
    G = wl.group
    pairs = sampled_pairs(wl)
    heads = [(b, h) for b, g in pairs for h in range(g * G, (g + 1) * G)]
    worst, flips = check_case(wl, inp, dc, out, sel, heads=heads,
                              pair_data=lambda b, g: W.gen_pair(wl, b, g, inp["q"]))
    print(f"  pairs {pairs}: worst row error {worst:.3e}, near-tie flips {flips}")
    sys.stdout.flush()
    if wl.needles_per_pair:
        for b in range(wl.batch):
            for g in range(wl.num_kv_heads):
                for blk, h in W.needle_plan(wl, b, g):
                    assert blk in sel[b, h].tolist(), (b, g, blk, h)


@pytest.mark.parametrize("name,split", [("llama8b_32k", 0), ("needle_128k", 0), ("llama8b_32k", 2)])
def test_full_size_append_decode(name, split):
    """The call the benchmark times: one hsla_append_decode with the
    default (fixed) split at full size (and once with the dynamic split,
    split = 2) -- the token's page write, the fold
    of a block it completes with that block's statistics, and the decode at
    T + 1 -- checked against the oracle at T + 1 on sampled pairs.  The
    first sequence is one token shorter, so that its appended token
    completes a block."""
    base = FULL[name]()
    lens = list(base.seq_lens)
    lens[0] -= 1
    wl = W.dataclasses.replace(base, seq_lens=tuple(lens), deterministic=split)
    assert (wl.seq_lens[0] + 1) % wl.block_size == 0
    _announce(wl, f"full size, hsla_append_decode (split {split}), sampled pairs at T + 1")
    inp = W.make_inputs(wl, keep_pairs=False)
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                     capacity_len=int(max(wl.seq_lens)) + 1)
    dc.build()
    k_tok, v_tok = W.gen_token(wl, 0)
    out, sel = dc.append_decode(to_device(k_tok), to_device(v_tok), to_device(inp["q"]))
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    grown = W.dataclasses.replace(wl, seq_lens=tuple(t + 1 for t in wl.seq_lens))
    assert dc.seq_lens.cpu().numpy().tolist() == list(grown.seq_lens)
    check_properties(grown, out, sel)

    def pair_data(b, g):
        K, V = W.gen_pair(wl, b, g, inp["q"])
        return np.concatenate([K, k_tok[b, g][None]]), np.concatenate([V, v_tok[b, g][None]])

    G = wl.group
    pairs = sorted(set(sampled_pairs(grown)) | {(0, 0)})
    heads = [(b, h) for b, g in pairs for h in range(g * G, (g + 1) * G)]
    worst, flips = check_case(grown, inp, dc, out, sel, heads=heads, pair_data=pair_data)
    print(f"  pairs {pairs}: worst row error {worst:.3e}, near-tie flips {flips}")
    sys.stdout.flush()


def test_full_size_hybrid_32_layers():
    """Build + decode of all 32 layers at 32768 tokens (budgets from
    {4, 8, 16, 32}, every fourth layer without the linear tail); one pair
    per layer against the oracle."""
    for wl in W.hybrid_layers():
        _announce(wl, f"layer {wl.layer}")
        inp = W.make_inputs(wl, keep_pairs=False)
        dc, out, sel = run_full(wl, inp)
        check_properties(wl, out, sel)
        g = wl.layer % wl.num_kv_heads
        heads = [(0, h) for h in range(g * wl.group, (g + 1) * wl.group)]
        worst, _ = check_case(wl, inp, dc, out, sel, heads=heads,
                              pair_data=lambda b, gg: W.gen_pair(wl, b, gg, inp["q"]))
        print(f"  layer {wl.layer}: k={wl.top_k} lin={wl.linear_tail} worst {worst:.3e}")
        sys.stdout.flush()
        del dc
        torch.cuda.empty_cache()
