"""Append + decode steps captured in a HIP graph and replayed.

The library enqueues kernels only (no allocation, no memset, no host
synchronisation), so a caller may capture a whole multi-layer step.  Two
identical sets of caches advance side by side: one eagerly, one through
replays of a captured two-step graph (two steps bring the ping-ponged length
buffers back to where the capture started).  Every replay is checked against
the eager outputs and selections of the same step, with eager torch work and
synchronisation between replays.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _announce, cfg_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from hybrid_sparse_linear_block_amd.device import DeviceCache, PreparedDecodeStep, to_device  # noqa: E402
from parity import row_rel_err  # noqa: E402

REPLAYS = 3


def _layer_set(layers, inps, cap, fused):
    preps = []
    for wl, inp in zip(layers, inps):
        dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                         capacity_len=cap)
        dc.build()
        k_tok, v_tok = (to_device(x) for x in W.gen_token(wl, 0))
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        sel = torch.empty((wl.batch, wl.num_q_heads, wl.top_k), dtype=torch.int32, device="cuda")
        preps.append(PreparedDecodeStep(dc, to_device(inp["q"]), k_tok, v_tok, out, sel, fused=fused))
    return preps


def _snapshot(preps):
    torch.cuda.synchronize()
    return [(p.keep[3].cpu().numpy().copy(), p.keep[4].cpu().numpy().copy()) for p in preps]


@pytest.mark.parametrize("fused", [False, True], ids=["two_calls", "append_decode"])
@pytest.mark.parametrize("deterministic", [1, 2])
def test_graph_replays_match_eager_steps(deterministic, fused):
    # 4157 tokens: the third step's token completes block 64, so the replays
    # also fold a block into the state and write its statistics
    layers = [dataclasses.replace(wl, append_room=2, deterministic=deterministic, seq_lens=(4157,))
              for wl in W.hybrid_small()]
    _announce(layers[0], f"graph replays, {len(layers)} layers, deterministic={deterministic}, fused={fused}")
    inps = [W.make_inputs(wl, keep_pairs=False) for wl in layers]
    steps = 2 * REPLAYS
    cap = int(max(layers[0].seq_lens)) + steps + 2
    eager, graphed = _layer_set(layers, inps, cap, fused), _layer_set(layers, inps, cap, fused)
    for p in eager:   # the same length bound as the graph (the split of the work depends on it)
        p.bound = cap

    # eager reference: the outputs after every second step
    want = []
    for s in range(steps):
        for p in eager:
            p()
        if s % 2 == 1:
            want.append(_snapshot(eager))

    gs = torch.cuda.Stream()
    for p in graphed:
        p.bound, p.stream = cap, gs.cuda_stream
    saved = [(p.dc.cur, p.dc.host_lens.copy()) for p in graphed]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=gs):
        for _ in range(2):
            for p in graphed:
                p()
    for p, (cur, lens) in zip(graphed, saved):
        p.dc.cur, p.dc.host_lens[:] = cur, lens

    noise = torch.randn(512, 512, device="cuda")
    for r in range(REPLAYS):
        graph.replay()
        got = _snapshot(graphed)
        noise = noise @ noise.T / 512.0   # eager work between replays
        torch.cuda.synchronize()
        for li, ((go, gsel), (wo, wsel)) in enumerate(zip(got, want[r])):
            assert np.array_equal(gsel, wsel), (r, li)
            if deterministic == 1:
                assert np.array_equal(go, wo), (r, li)
            else:
                for b in range(go.shape[0]):
                    for h in range(go.shape[1]):
                        assert row_rel_err(go[b, h], wo[b, h]) < 1e-5, (r, li, b, h)
    # the caches advanced identically
    for p, q in zip(graphed, eager):
        p.dc.host_lens += steps
        assert np.array_equal(p.dc.host_lens, q.dc.host_lens)
        assert torch.equal(p.dc.lens[p.dc.cur], q.dc.lens[q.dc.cur])
        assert torch.equal(p.dc.S, q.dc.S) and torch.equal(p.dc.blk_mean, q.dc.blk_mean)
