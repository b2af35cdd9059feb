"""hsla_append_decode against hsla_append_token followed by hsla_decode.

With the fixed split both paths do the same arithmetic in the same order,
so every output, selection, page, statistic, state entry and length must be
bitwise equal, step after step, including steps whose token completes a
block (the statistics written inside the decode's first kernel) and
configurations without candidates or without the linear tail.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _announce, _wl, cfg_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import hybrid_sparse_linear_block_amd as H  # noqa: E402
from hybrid_sparse_linear_block_amd.device import DeviceCache, to_device  # noqa: E402

STEPS = 4
# (T + 1) % B == 0 at the first append for sequence 0 (1471 + 1 = 23 x 64)
CASES = {
    "bf16_g4": dict(seq_lens=(1471, 1203)),
    "f32_d64": dict(kv_dtype=W.F32, head_dim=64, seq_lens=(1471, 1203)),
    "bf16_g8": dict(num_q_heads=16, num_kv_heads=2, seq_lens=(1471, 1203)),
    "bf16_g1_b1": dict(batch=1, num_q_heads=2, num_kv_heads=2, seq_lens=(2047,)),
    "no_linear_tail": dict(linear_tail=0, seq_lens=(1471, 1203)),
    "grouped": dict(grouped=1, seq_lens=(1471, 1203)),
    "block16": dict(block_size=16, window=64, top_k=12, seq_lens=(1471, 1202)),
    "no_candidates": dict(seq_lens=(200, 37)),
    "token_level": dict(tokens=1, top_k=40, seq_lens=(1471, 1203)),
    # a per-token state (state_span = HSLA_STATE_TOKENS): every append adds
    # its token to S, z and sv
    "per_token_state": dict(seq_lens=(1471, 1203)),
    "per_token_state_f32_d64": dict(kv_dtype=W.F32, head_dim=64, seq_lens=(1471, 1203)),
    "per_token_state_no_tail": dict(linear_tail=0, seq_lens=(1471, 1203)),
}


def _tokens(wl, step):
    rng = np.random.default_rng([4242, step])
    shape = (wl.batch, wl.num_kv_heads, wl.head_dim)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    if wl.kv_dtype == W.BF16:
        return W.bf16_round(k), W.bf16_round(v)
    return k, v


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_decode_equals_append_then_decode(name):
    wl = _wl(f"append_decode_{name}", 70, append_room=2, deterministic=1, **CASES[name])
    _announce(wl, f"append + decode, {STEPS} steps")
    inp = W.make_inputs(wl, keep_pairs=False)
    cap = int(max(wl.seq_lens)) + STEPS + 1
    cfg = cfg_of(wl)
    if name.startswith("per_token_state"):
        cfg = dataclasses.replace(cfg, state_span=H.HSLA_STATE_TOKENS)
    caches = [DeviceCache(cfg, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"],
                          capacity_len=cap) for _ in range(2)]
    for dc in caches:
        dc.build()
    q = to_device(inp["q"])
    for step in range(STEPS):
        k, v = (to_device(x) for x in _tokens(wl, step))
        o_f, s_f = caches[0].append_decode(k, v, q)
        caches[1].append(k, v)
        o_s, s_s = caches[1].decode(q)
        torch.cuda.synchronize()
        assert torch.equal(o_f, o_s), step
        if wl.top_k > 0:
            assert torch.equal(s_f, s_s), step
    a, b = caches
    assert np.array_equal(a.host_lens, b.host_lens)
    assert torch.equal(a.seq_lens, b.seq_lens)
    assert a.seq_lens.cpu().numpy().tolist() == [t + STEPS for t in wl.seq_lens]
    for name_t in ("k_pages", "v_pages", "blk_mean", "blk_var", "S", "z", "sv"):
        assert torch.equal(getattr(a, name_t), getattr(b, name_t)), name_t
