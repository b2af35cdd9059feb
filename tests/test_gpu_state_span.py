"""A caller-kept per-token linear state (state_span = HSLA_STATE_TOKENS),
through the C ABI, against the fp64 oracle.

The state then holds all T tokens ("SPLA: Block Sparse Plus Linear Attention
for Long Context Modeling", Residual Linear Attention (RLA) and Recurrence:
the state summed over every token so far, n = T).  hsla_build_state builds it
over all T tokens and hsla_decode subtracts every exact token from it, so the
residual covers the same unselected tokens as with a state of whole blocks.
Lengths are chosen off the block grid, so that the incomplete last block is
in the state.  Every case prints its shape before touching the GPU."""
import math
import sys

import numpy as np
import pytest

import oracle as O
import workloads as W
from parity import OUT_TOL, assert_state_close, row_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import hybrid_sparse_linear_block_amd as H  # noqa: E402
from hybrid_sparse_linear_block_amd.device import DeviceCache, config_for, to_device  # noqa: E402

from test_gpu_parity import check_case  # noqa: E402

CASES = {
    "bf16_g4": dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64, top_k=6, num_sink=4,
                    window=256, linear_tail=1, kv_dtype=W.BF16, seq_lens=(1500, 1203)),
    "f32_d64_b16": dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16, top_k=5, num_sink=2,
                        window=64, linear_tail=1, kv_dtype=W.F32, seq_lens=(700, 333)),
    "bf16_g8_b128": dict(batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=128, top_k=4,
                         num_sink=4, window=384, linear_tail=1, kv_dtype=W.BF16, seq_lens=(2000,)),
}


def _cfg(wl, span):
    return config_for(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k, wl.num_sink,
                      wl.window, wl.linear_tail, wl.kv_dtype, wl.scale, state_span=span)


def _state_depth(T):
    return min(T, 4096) + math.ceil(T / 32) + 16


@pytest.mark.parametrize("name", sorted(CASES))
def test_per_token_state_decodes_like_the_oracle(name):
    wl = W.Workload(f"span_{name}", 60 + sorted(CASES).index(name), shuffle_pages=True, spare_pages=2,
                    **CASES[name])
    assert any(t % wl.block_size for t in wl.seq_lens)
    print(f"[case] {wl.name} cid={wl.cid} batch={wl.batch} d={wl.head_dim} B={wl.block_size} "
          f"{wl.kv_dtype} T={list(wl.seq_lens)}", flush=True)
    sys.stdout.flush()
    inp = W.make_inputs(wl)
    q = to_device(inp["q"])
    outs = {}
    for span in (H.HSLA_STATE_BLOCKS, H.HSLA_STATE_TOKENS):
        dc = DeviceCache(_cfg(wl, span), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"])
        dc.build()
        out, sel = dc.decode(q)
        torch.cuda.synchronize()
        out, sel = out.cpu().numpy(), sel.cpu().numpy()
        outs[span] = out
        if span == H.HSLA_STATE_TOKENS:
            # the state holds every token
            S_g, z_g, sv_g = dc.S.cpu().numpy(), dc.z.cpu().numpy(), dc.sv.cpu().numpy()
            for (b, g), (K, V) in inp["pairs"].items():
                Kf, Vf = O.to_f64(K, wl.kv_dtype), O.to_f64(V, wl.kv_dtype)
                T = Kf.shape[0]
                gs = O.LinearState(S_g[b, g].astype(np.float64), z_g[b, g].astype(np.float64),
                                   sv_g[b, g].astype(np.float64), T)
                assert_state_close(gs, O.global_state(Kf, Vf), Kf, Vf, _state_depth(T), f"pair {(b, g)}")
        # outputs and selections against the oracle's own statistics and state
        check_case(wl, inp, dc, out, sel, check_build=False)
    # both spans give the same residual, up to rounding
    tol = OUT_TOL[wl.kv_dtype]
    for b in range(wl.batch):
        for h in range(wl.num_q_heads):
            assert row_rel_err(outs[H.HSLA_STATE_TOKENS][b, h], outs[H.HSLA_STATE_BLOCKS][b, h]) <= 2 * tol


@pytest.mark.parametrize("dtype,fused", [(W.BF16, False), (W.F32, False), (W.BF16, True), (W.F32, True)])
def test_per_token_state_through_appends(dtype, fused):
    """Build at T - N, then N appends crossing block boundaries (each adds
    its token to S, z and sv), then a decode: the state holds all T tokens,
    the completed blocks have their statistics, and every head's selection
    and output match the oracle on the full sequence.  `fused`: every append
    is an hsla_append_decode call, and the last call's output is the decode
    checked; else hsla_append_token, then hsla_decode."""
    N = 70
    full = W.Workload("span_append", 64, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=64,
                      top_k=6, num_sink=4, window=256, linear_tail=1, kv_dtype=dtype, seq_lens=(1400, 1250),
                      shuffle_pages=True, spare_pages=2, append_room=3)
    start = tuple(t - N for t in full.seq_lens)
    print(f"[case] {full.name} cid={full.cid} {dtype} fused={fused} T={list(full.seq_lens)} N={N}", flush=True)
    sys.stdout.flush()
    inp = W.make_inputs(full)
    table = inp["block_table"]
    kp, vp = W.empty_pool(full), W.empty_pool(full)
    for (b, g), (K, V) in inp["pairs"].items():
        W.scatter_pairs(full, table, kp, b, g, K[:start[b]])
        W.scatter_pairs(full, table, vp, b, g, V[:start[b]])
    dc = DeviceCache(_cfg(full, H.HSLA_STATE_TOKENS), kp, vp, table, np.asarray(start, np.int32),
                     capacity_len=max(full.seq_lens))
    dc.build()
    q_dev = to_device(inp["q"])
    for i in range(N):
        kn = np.stack([np.stack([inp["pairs"][(b, g)][0][start[b] + i] for g in range(full.num_kv_heads)])
                       for b in range(full.batch)])
        vn = np.stack([np.stack([inp["pairs"][(b, g)][1][start[b] + i] for g in range(full.num_kv_heads)])
                       for b in range(full.batch)])
        if fused:
            out, sel = dc.append_decode(to_device(kn), to_device(vn), q_dev)
        else:
            dc.append(to_device(kn), to_device(vn))
    if not fused:
        out, sel = dc.decode(q_dev)
    torch.cuda.synchronize()
    assert dc.seq_lens.cpu().numpy().tolist() == list(full.seq_lens)
    # statistics of every complete block and the state over all T tokens
    check_case(full, inp, dc, out.cpu().numpy(), sel.cpu().numpy(), check_build=False)
    mean_g, var_g = dc.blk_mean.cpu().numpy(), dc.blk_var.cpu().numpy()
    S_g, z_g, sv_g = dc.S.cpu().numpy(), dc.z.cpu().numpy(), dc.sv.cpu().numpy()
    from parity import assert_stats_close
    for (b, g), (K, V) in inp["pairs"].items():
        Kf, Vf = O.to_f64(K, dtype), O.to_f64(V, dtype)
        T = Kf.shape[0]
        nb = T // full.block_size
        st = O.block_statistics(Kf, full.block_size)
        pages = table[b, :nb]
        assert_stats_close(mean_g[pages, g], var_g[pages, g], st[0], st[1], Kf, full.block_size, f"pair {(b, g)}")
        gs = O.LinearState(S_g[b, g].astype(np.float64), z_g[b, g].astype(np.float64),
                           sv_g[b, g].astype(np.float64), T)
        assert_state_close(gs, O.global_state(Kf, Vf), Kf, Vf, _state_depth(T) + N, f"pair {(b, g)}")
