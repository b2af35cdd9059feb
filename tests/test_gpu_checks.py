"""The length / block-table check on the GPU, and the debug library that runs
it inside every entry point.

- hsla_check_tables (device arrays) gives the same count and first
  violation as hsla_check_tables_host on random tables with planted bad
  entries and lengths (the host rule itself is pinned in test_checks.py).
- libhsla_debug.so decodes a valid cache bitwise like libhsla.so (fixed
  split), and refuses a cache whose block table maps a used block outside
  the pool: HSLA_ERR_INVALID_ARG, and nothing written to the outputs (no
  decode kernel ran on the bad table).
"""
import ctypes

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


def _cfg(B):
    return H.Config(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=B, top_k=16, num_sink=4,
                    window=max(B, 64))


def test_device_check_matches_host_check():
    print("[gpu-checks] device table check vs host check, 40 random tables", flush=True)
    lib = H.load()
    rng = np.random.default_rng(11)
    res = torch.empty(2, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for trial in range(40):
        B = int(rng.choice([16, 64, 128]))
        msl = int(rng.integers(B, 300 * B))
        m = -(-msl // B) + int(rng.integers(0, 3))
        batch = int(rng.integers(1, 17))
        num_pages = int(rng.integers(1, 5000))
        extra = int(rng.choice([0, 1, 8]))
        bt = rng.integers(0, num_pages, size=(batch, m)).astype(np.int32)
        planted = rng.random(bt.shape) < (0.0 if trial % 4 == 0 else 0.01)
        bt[planted] = rng.choice([-1, num_pages, -(2**31)], size=int(planted.sum()))
        lens = rng.integers(0, msl + 2, size=batch).astype(np.int32)
        if trial % 4 == 0:   # all valid
            lens = np.clip(lens, 1, msl - extra)
        c = _cfg(B)
        want = H.hsla_check_tables_host(c, m, num_pages, bt, lens, batch, msl, extra)
        bt_d, lens_d = to_device(bt), to_device(lens)
        pool = H.hsla_kv_pool(None, None, None, None, bt_d.data_ptr(), m, num_pages)
        st = lib.hsla_check_tables(ctypes.byref(c.c()), ctypes.byref(pool), lens_d.data_ptr(), batch, msl, extra,
                                   res.data_ptr(), stream)
        assert st == H.HSLA_OK
        torch.cuda.synchronize()
        assert tuple(res.cpu().tolist()) == want[1:], trial


def test_debug_library_checks_the_table_before_decoding():
    wl = _wl("debug_checks", 81, deterministic=1, seq_lens=(1471, 1203))
    _announce(wl, "debug library: valid table, then a bad block-table entry")
    inp = W.make_inputs(wl, keep_pairs=False)
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"])
    dc.build()
    q = to_device(inp["q"])
    o_rel, s_rel = dc.decode(q)
    torch.cuda.synchronize()

    dbg = H.open_library(H.DEBUG_LIB_PATH)
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.full_like(o_rel, float("nan"))
    sel = torch.full_like(s_rel, -7)

    def decode():
        return dbg.hsla_decode(ctypes.byref(dc.cfg.c()), ctypes.byref(dc.pool.c()), ctypes.byref(dc.state.c()),
                               q.data_ptr(), dc.seq_lens.data_ptr(), dc.batch, dc.max_seq_len, out.data_ptr(),
                               sel.data_ptr(), dc.decode_ws.data_ptr(), dc.decode_ws.numel(), stream, None)

    assert decode() == H.HSLA_OK
    torch.cuda.synchronize()
    assert torch.equal(out, o_rel) and torch.equal(sel, s_rel)

    num_pages = int(dc.k_pages.shape[0])
    m = int(dc.block_table.shape[1])
    saved = int(dc.block_table[1, 3].item())
    dc.block_table[1, 3] = num_pages            # block 3 of sequence 1 (in use) now outside the pool
    res = torch.empty(2, dtype=torch.int32, device="cuda")
    H.hsla_check_tables(dc.cfg, dc.pool, dc.seq_lens, dc.batch, dc.max_seq_len, 0, res)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [1, 1 * (m + 1) + 3 + 1]
    out.fill_(float("nan"))
    sel.fill_(-7)
    torch.cuda.synchronize()
    assert decode() == H.HSLA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and (sel == -7).all()
    dc.block_table[1, 3] = saved
    torch.cuda.synchronize()
    assert decode() == H.HSLA_OK
    torch.cuda.synchronize()
    assert torch.equal(out, o_rel)
