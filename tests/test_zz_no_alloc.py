"""hsla_append_decode_noalloc (the entry point for callers that cannot
allocate: its workspace is a fixed device array inside the library) against
hsla_append_decode with a caller-owned workspace.

Two caches with the same contents take the same step, one through each
entry point; two calls in a row, the second with a smaller input (fewer
sequences, shorter contexts).  With the fixed split both paths do the same
arithmetic in the same order, so outputs, selections and the whole cache
are bitwise equal; with the dynamic split (one launch) selections and the
cache are bitwise equal and outputs agree within the bf16 tolerance.
"""
import numpy as np
import pytest

import workloads as W
from parity import OUT_TOL, row_rel_err
from test_gpu_parity import _announce, _wl, cfg_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import hybrid_sparse_linear_block_amd as H  # noqa: E402
from hybrid_sparse_linear_block_amd.device import DeviceCache, to_device  # noqa: E402

# the second call's input is the smaller one
CALLS = [dict(batch=4, seq_lens=(1535, 1201, 900, 1377)), dict(batch=2, seq_lens=(767, 640))]


def _noalloc_step(dc, k, v, q, out, sel):
    nxt = 1 - dc.cur
    H.hsla_append_decode_noalloc(dc.cfg, dc.pool, dc.state, k, v, dc.lens[dc.cur], dc.lens[nxt], q, dc.batch,
                                 dc.max_seq_len + 1, out, sel)
    dc.cur = nxt
    dc.host_lens += 1


@pytest.mark.parametrize("deterministic", [1, 2])
def test_noalloc_matches_workspace_entry_point(deterministic):
    assert H.hsla_noalloc_scratch_bytes() == 16 << 20
    for i, shape in enumerate(CALLS):
        wl = _wl(f"noalloc_{i}", 75 + i, append_room=2, deterministic=deterministic, **shape)
        _announce(wl, f"no-allocation entry point, call {i + 1}")
        inp = W.make_inputs(wl, keep_pairs=False)
        cap = int(max(wl.seq_lens)) + 2
        ref, got = (DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                                capacity_len=cap) for _ in range(2))
        ref.build()
        got.build()
        q = to_device(inp["q"])
        k, v = (to_device(x) for x in W.gen_token(wl, i))
        o_ref, s_ref = ref.append_decode(k, v, q)
        o_got = torch.empty_like(o_ref)
        s_got = torch.empty_like(s_ref)
        _noalloc_step(got, k, v, q, o_got, s_got)
        torch.cuda.synchronize()
        assert torch.equal(s_got, s_ref)
        if deterministic == 1:
            assert torch.equal(o_got, o_ref)
        else:
            a, b = o_got.cpu().numpy(), o_ref.cpu().numpy()
            worst = max(row_rel_err(a[bb, h], b[bb, h]) for bb in range(wl.batch) for h in range(wl.num_q_heads))
            assert worst <= OUT_TOL[wl.kv_dtype], worst
        assert torch.equal(got.seq_lens, ref.seq_lens)
        for name in ("k_pages", "v_pages", "blk_mean", "blk_var", "S", "z", "sv"):
            assert torch.equal(getattr(got, name), getattr(ref, name)), name
