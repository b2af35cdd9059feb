"""Length and block-table checks (hsla_check_tables_host, and the debug
library's exports), on the host: no GPU.

The rule, from the header: row b is valid when min_len <= T_b and
T_b + extra <= max_seq_len (min_len = 1 when extra is 0, else 0), and its
entries j < ceil((T_b + extra) / B) are pages in [0, num_pages); entries past
that are never used as page indices and are not checked.  The reference
below restates that rule in plain Python, row by row.
"""
import ctypes

import numpy as np
import pytest

import hybrid_sparse_linear_block_amd as H
from test_abi import declared_functions

INT_MAX = 2**31 - 1


def cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=64, top_k=16, num_sink=4, window=512)
    base.update(kw)
    return H.Config(**base)


def reference(bt, lens, B, num_pages, max_seq_len, extra):
    min_len = 0 if extra > 0 else 1
    m = bt.shape[1]
    bad, first = 0, INT_MAX
    for b, T in enumerate(lens.tolist()):
        if T < min_len or T + extra > max_seq_len:
            bad += 1
            first = min(first, b * (m + 1))
            continue
        for j in range(-(-(T + extra) // B)):
            if not 0 <= bt[b, j] < num_pages:
                bad += 1
                first = min(first, b * (m + 1) + j + 1)
    return bad, first


def run(c, bt, lens, num_pages, max_seq_len, extra):
    return H.hsla_check_tables_host(c, bt.shape[1], num_pages, bt, lens, len(lens), max_seq_len, extra)


def test_valid_tables_pass():
    c = cfg()
    bt = np.arange(4 * 10, dtype=np.int32).reshape(4, 10)
    lens = np.array([640, 100, 1, 300], np.int32)
    assert run(c, bt, lens, 40, 640, 0) == (H.HSLA_OK, 0, INT_MAX)
    assert run(c, bt, lens - 1, 40, 640, 1) == (H.HSLA_OK, 0, INT_MAX)   # seq_lens_before of an append


def test_entries_past_the_used_blocks_are_not_checked():
    c = cfg()
    bt = np.full((2, 10), -7, np.int32)   # garbage everywhere ...
    bt[0, :2] = [3, 4]                    # ... except the blocks in use
    bt[1, :1] = [5]
    lens = np.array([128, 64], np.int32)
    assert run(c, bt, lens, 40, 640, 0) == (H.HSLA_OK, 0, INT_MAX)
    # the append of one token needs the next block of row 0 (T = 128 -> block 2)
    assert run(c, bt, lens, 40, 640, 1) == (H.HSLA_ERR_INVALID_ARG, 2, 0 * 11 + 2 + 1)


@pytest.mark.parametrize("page", [-1, 40, 2**31 - 1])
def test_out_of_range_page_is_reported_first(page):
    c = cfg()
    bt = np.arange(3 * 10, dtype=np.int32).reshape(3, 10)
    bt[1, 4] = page
    bt[2, 0] = page
    lens = np.array([640, 300, 64], np.int32)
    assert run(c, bt, lens, 40, 640, 0) == (H.HSLA_ERR_INVALID_ARG, 2, 1 * 11 + 4 + 1)


@pytest.mark.parametrize("T,extra", [(0, 0), (-5, 0), (641, 0), (640, 1), (-1, 1), (600, 64)])
def test_bad_lengths(T, extra):
    c = cfg()
    bt = np.zeros((2, 10), np.int32)
    lens = np.array([64, T], np.int32)
    assert run(c, bt, lens, 40, 640, extra) == (H.HSLA_ERR_INVALID_ARG, 1, 1 * 11)


def test_matches_the_rule_on_random_tables():
    rng = np.random.default_rng(7)
    for trial in range(200):
        B = int(rng.choice([16, 32, 64, 128]))
        msl = int(rng.integers(B, 40 * B))
        m = -(-msl // B) + int(rng.integers(0, 3))
        batch = int(rng.integers(1, 9))
        num_pages = int(rng.integers(1, 200))
        extra = int(rng.choice([0, 0, 1, min(B, 8)]))
        bt = rng.integers(0, num_pages, size=(batch, m)).astype(np.int32)
        planted = rng.random(bt.shape) < 0.05
        bt[planted] = rng.choice([-1, num_pages, num_pages + 17, -(2**31)], size=int(planted.sum()))
        lens = rng.integers(0, msl + 2, size=batch).astype(np.int32)
        c = cfg(block_size=B, window=max(B, 64))
        st, bad, first = run(c, bt, lens, num_pages, msl, extra)
        want = reference(bt, lens, B, num_pages, msl, extra)
        assert (bad, first) == want, trial
        assert st == (H.HSLA_OK if bad == 0 else H.HSLA_ERR_INVALID_ARG)


def test_rejects_invalid_arguments():
    c = cfg()
    bt = np.zeros((2, 10), np.int32)
    lens = np.array([64, 64], np.int32)
    assert run(c, bt, lens, 0, 640, 0)[0] == H.HSLA_ERR_INVALID_ARG      # no pages
    assert run(c, bt, lens, 40, 640, -1)[0] == H.HSLA_ERR_INVALID_ARG     # negative extra
    assert run(c, bt[:, :5], lens, 40, 640, 0)[0] == H.HSLA_ERR_INVALID_ARG   # rows shorter than max_seq_len needs
    assert run(cfg(head_dim=96), bt, lens, 40, 640, 0)[0] == H.HSLA_ERR_UNSUPPORTED


def test_debug_library_exports_the_same_entry_points():
    dbg = H.open_library(H.DEBUG_LIB_PATH)
    for n in declared_functions():
        assert hasattr(dbg, n), n
    # the debug build validates its host arguments like the release build
    res = (ctypes.c_int32 * 2)()
    bt = np.zeros((1, 10), np.int32)
    lens = np.array([700], np.int32)
    st = dbg.hsla_check_tables_host(ctypes.byref(cfg().c()), 10, 40, bt.ctypes.data, lens.ctypes.data, 1, 640, 0,
                                    ctypes.cast(res, ctypes.c_void_p))
    assert (st, res[0], res[1]) == (H.HSLA_ERR_INVALID_ARG, 1, 0)
