"""The phase-timestamp diagnostic build (libhsla_phases.so): its decode is
bitwise the release library's, and the stamps it records are ordered.

The diagnostic library only adds stores of s_memrealtime stamps to the
decode kernels; with the fixed split every reduction has a fixed order, so
outputs and selections must repeat bit for bit across the two libraries."""
import os
import sys

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import hybrid_sparse_linear_block_amd as H  # noqa: E402
from hybrid_sparse_linear_block_amd.device import DeviceCache, config_for, to_device  # noqa: E402

ATT, SLOTS, SCORE, MERGE = 4096, 16, 16384, 8192


def _decode(wl, inp):
    cfg = config_for(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, wl.top_k, wl.num_sink,
                     wl.window, wl.linear_tail, wl.kv_dtype, deterministic=1)
    dc = DeviceCache(cfg, inp["k_pages"], inp["v_pages"], inp["block_table"], inp["seq_lens"])
    dc.build()
    out, sel = dc.decode(to_device(inp["q"]))
    torch.cuda.synchronize()
    return out.cpu().numpy(), sel.cpu().numpy()


def _ordered(row):
    """Non-zero stamps of one workgroup never decrease in slot order."""
    v = row[row > 0]
    return bool(np.all(np.diff(v.astype(np.int64)) >= 0))


def test_phases_build_matches_release_and_stamps_are_ordered():
    if not os.path.exists(H.PHASES_LIB_PATH):
        pytest.skip("libhsla_phases.so not built")
    wl = W.small("llama8b_small")
    print(f"[gpu-test] {wl.name}: phases library against the release library", flush=True)
    inp = W.make_inputs(wl)
    o_rel, s_rel = _decode(wl, inp)
    try:
        lib = H.use_library(H.PHASES_LIB_PATH)
        nbytes = int(lib.hsla_phase_timestamp_bytes())
        assert nbytes == 8 * (ATT * SLOTS + 2 * SCORE + 2 * MERGE)
        buf = np.zeros(nbytes // 8, np.uint64)
        assert lib.hsla_phase_timestamps(buf.ctypes.data, nbytes, 1) == 0   # clear
        o_ph, s_ph = _decode(wl, inp)
        assert lib.hsla_phase_timestamps(buf.ctypes.data, nbytes, 0) == 0
    finally:
        H.use_library(H.LIB_PATH)
    assert np.array_equal(s_rel, s_ph)
    assert np.array_equal(o_rel.view(np.uint32), o_ph.view(np.uint32))
    a = buf[:ATT * SLOTS].reshape(ATT, SLOTS)
    sc = buf[ATT * SLOTS:ATT * SLOTS + 2 * SCORE].reshape(SCORE, 2)
    m = buf[ATT * SLOTS + 2 * SCORE:].reshape(MERGE, 2)
    a, sc, m = a[a[:, 0] > 0], sc[sc[:, 0] > 0], m[m[:, 0] > 0]
    assert len(a) > 0 and len(sc) > 0
    # the merge kernel runs unless the last attention workgroup of each pair merged
    assert len(m) in (0, wl.batch * wl.num_q_heads)
    for row in a:
        # entry, loads staged, selection per wavefront, prologue done, loop
        # done per wavefront, partials written, exit: by phase
        phases = [row[0], row[1], row[2:6].max(), row[6], row[7:11].max(), row[11], row[12]]
        assert _ordered(np.array(phases, np.uint64)), row
        assert row[12] > 0, row   # every workgroup stamps its exit
    assert np.all(sc[:, 1] >= sc[:, 0]) and np.all(m[:, 1] >= m[:, 0])
    # the launches ran in order: scoring, attention, merge
    assert sc[:, 0].min() <= a[:, 0].min()
    if len(m):
        assert a[:, 12].max() <= m[:, 1].max()
    print(f"  {len(a)} attention, {len(sc)} scoring, {len(m)} merge workgroups stamped", flush=True)
    sys.stdout.flush()
