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
