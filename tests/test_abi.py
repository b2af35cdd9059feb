"""The C ABI library loads, exports every entry point include/hsla.h declares,
and rejects invalid arguments on the host (no GPU needed: every call here
fails validation before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import hybrid_sparse_linear_block_amd as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hsla_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = H.load()
    names = declared_functions()
    assert set(names) == set(H.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4):
        s = H.status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in H.status_string(7)
    assert "gfx950" in H.hsla_version()


def cfg(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=64, top_k=16, num_sink=4,
                window=512, linear_tail=1, kv_dtype=H.HSLA_BF16, scale=0.0)
    base.update(kw)
    return H.Config(**base)


def test_workspace_sizes_are_host_only_and_grow():
    a = H.hsla_decode_workspace_size(cfg(), 8, 32768)
    b = H.hsla_decode_workspace_size(cfg(), 8, 131072)
    assert 0 < a < b
    assert H.hsla_build_workspace_size(cfg(), 1, 32768) > 0
    assert H.hsla_decode_workspace_size(cfg(head_dim=96), 8, 32768) == 0
    assert H.hsla_build_workspace_size(cfg(num_q_heads=30), 8, 32768) == 0


BAD_CONFIGS = [
    (dict(num_q_heads=30), H.HSLA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), H.HSLA_ERR_INVALID_ARG),
    (dict(num_q_heads=48, num_kv_heads=8), H.HSLA_ERR_UNSUPPORTED),   # group 6
    (dict(head_dim=96), H.HSLA_ERR_UNSUPPORTED),
    (dict(block_size=48), H.HSLA_ERR_UNSUPPORTED),
    (dict(top_k=-1), H.HSLA_ERR_INVALID_ARG),
    (dict(num_sink=-2), H.HSLA_ERR_INVALID_ARG),
    (dict(window=32), H.HSLA_ERR_INVALID_ARG),                         # window < block
    (dict(linear_tail=2), H.HSLA_ERR_INVALID_ARG),
    (dict(kv_dtype=7), H.HSLA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), H.HSLA_ERR_INVALID_ARG),
    (dict(scale=-1.0), H.HSLA_ERR_INVALID_ARG),
    (dict(deterministic=3), H.HSLA_ERR_INVALID_ARG),
    (dict(deterministic=-1), H.HSLA_ERR_INVALID_ARG),
    (dict(state_span=2), H.HSLA_ERR_INVALID_ARG),
    (dict(state_span=-1), H.HSLA_ERR_INVALID_ARG),
]

FAKE = 1 << 20   # an aligned non-null address; never dereferenced because validation fails first


def pool(**kw):
    base = dict(k_pages=FAKE, v_pages=FAKE, blk_mean=FAKE, blk_var=FAKE, block_table=FAKE,
                max_blocks_per_seq=1024, num_pages=4096)
    base.update(kw)
    return H.hsla_kv_pool(**base)


def state(**kw):
    base = dict(S=FAKE, z=FAKE, sv=FAKE)
    base.update(kw)
    return H.hsla_state(**base)


def call_decode(c, p=None, st=None, q=FAKE, lens=FAKE, batch=8, max_len=32768, out=FAKE, sel=FAKE,
                ws=FAKE, ws_bytes=1 << 40):
    lib = H.load()
    return lib.hsla_decode(ctypes.byref(c.c()), ctypes.byref(p or pool()), ctypes.byref(st or state()), q, lens,
                           batch, max_len, out, sel, ws, ws_bytes, None, None)


@pytest.mark.parametrize("bad,code", BAD_CONFIGS)
def test_decode_rejects_bad_configs(bad, code):
    assert call_decode(cfg(**bad)) == code


@pytest.mark.parametrize("bad,code", BAD_CONFIGS)
def test_build_and_append_reject_bad_configs(bad, code):
    lib = H.load()
    c = cfg(**bad)
    assert lib.hsla_build_state(ctypes.byref(c.c()), ctypes.byref(pool()), ctypes.byref(state()), FAKE, 8, 32768,
                                FAKE, 1 << 40, None) == code
    assert lib.hsla_append_token(ctypes.byref(c.c()), ctypes.byref(pool()), ctypes.byref(state()), FAKE, FAKE,
                                 FAKE, FAKE + 256, 8, 32768, None) == code


def test_decode_rejects_bad_pointers_and_sizes():
    c = cfg()
    E = H.HSLA_ERR_INVALID_ARG
    assert call_decode(c, q=0) == E
    assert call_decode(c, q=FAKE + 2) == E               # misaligned
    assert call_decode(c, out=0) == E
    assert call_decode(c, lens=0) == E
    assert call_decode(c, sel=FAKE + 2) == E
    assert call_decode(c, batch=0) == E
    assert call_decode(c, max_len=0) == E
    assert call_decode(c, p=pool(k_pages=0)) == E
    assert call_decode(c, p=pool(blk_var=FAKE + 4)) == E
    assert call_decode(c, p=pool(max_blocks_per_seq=100)) == E   # 100 blocks < 32768 / 64
    assert call_decode(c, st=state(S=0)) == E
    assert call_decode(c, ws=0) == H.HSLA_ERR_WORKSPACE
    assert call_decode(c, ws_bytes=16) == H.HSLA_ERR_WORKSPACE
    assert call_decode(c, max_len=(1 << 20) * 64) == H.HSLA_ERR_UNSUPPORTED
    # one block past the largest candidate row whose selection bitmaps fit
    # the attention workgroup's 16 KB (8 heads x 256 words at 16384 blocks)
    big = cfg(num_q_heads=8, num_kv_heads=1, head_dim=64, block_size=16, window=64)
    assert call_decode(big, max_len=262208 + 16, p=pool(max_blocks_per_seq=1 << 15)) == H.HSLA_ERR_UNSUPPORTED
    assert H.hsla_decode_workspace_size(big, 1, 262208 + 16) == 0
    assert H.hsla_decode_workspace_size(big, 1, 262208) > 0
    # token-level variant: lengths below 2^20 (token index field of the list entries)
    assert call_decode(cfg(selection=H.HSLA_SEL_TOKEN), max_len=1 << 20,
                       p=pool(max_blocks_per_seq=1 << 15)) == H.HSLA_ERR_UNSUPPORTED
    assert H.hsla_decode_workspace_size(cfg(selection=H.HSLA_SEL_TOKEN), 8, 32768) > 0
    assert call_decode(cfg(selection=3)) == H.HSLA_ERR_INVALID_ARG


def test_append_rejects_aliased_lengths():
    lib = H.load()
    c = cfg()
    assert lib.hsla_append_token(ctypes.byref(c.c()), ctypes.byref(pool()), ctypes.byref(state()), FAKE, FAKE,
                                 FAKE, FAKE, 8, 32768, None) == H.HSLA_ERR_INVALID_ARG
    assert lib.hsla_append_token(ctypes.byref(c.c()), ctypes.byref(pool()), ctypes.byref(state()), 0, FAKE,
                                 FAKE, None, 8, 32768, None) == H.HSLA_ERR_INVALID_ARG


def test_build_rejects_small_workspace():
    lib = H.load()
    c = cfg()
    assert lib.hsla_build_state(ctypes.byref(c.c()), ctypes.byref(pool()), ctypes.byref(state()), FAKE, 8, 32768,
                                FAKE, 64, None) == H.HSLA_ERR_WORKSPACE


def call_append_decode(c, p=None, st=None, k=FAKE, v=FAKE, before=FAKE, after=FAKE + 256, q=FAKE, batch=8,
                       max_len=32768, out=FAKE, sel=FAKE, ws=FAKE, ws_bytes=1 << 40, null_state=False):
    lib = H.load()
    sp = None if null_state else ctypes.byref(st or state())
    return lib.hsla_append_decode(ctypes.byref(c.c()), ctypes.byref(p or pool()), sp, k, v, before, after, q,
                                  batch, max_len, out, sel, ws, ws_bytes, None, None)


@pytest.mark.parametrize("bad,code", BAD_CONFIGS)
def test_append_decode_rejects_bad_configs(bad, code):
    assert call_append_decode(cfg(**bad)) == code


def test_append_decode_rejects_bad_pointers_and_sizes():
    c = cfg()
    E = H.HSLA_ERR_INVALID_ARG
    assert call_append_decode(c, after=FAKE) == E          # aliases seq_lens_before
    assert call_append_decode(c, after=0) == E             # the decode reads the grown lengths
    assert call_append_decode(c, before=0) == E
    assert call_append_decode(c, k=0) == E
    assert call_append_decode(c, v=FAKE + 2) == E
    assert call_append_decode(c, q=0) == E
    assert call_append_decode(c, out=FAKE + 4) == E
    assert call_append_decode(c, null_state=True) == E
    # the append keeps the state whatever linear_tail says
    assert call_append_decode(cfg(linear_tail=0), st=state(S=0)) == E
    assert call_append_decode(c, p=pool(max_blocks_per_seq=100)) == E
    assert call_append_decode(c, ws_bytes=16) == H.HSLA_ERR_WORKSPACE


def call_prefill_chunk(c, p=None, st=None, k=FAKE, v=FAKE, before=FAKE, after=FAKE + 256, q=FAKE, batch=8,
                       q_len=16, max_len=32768, out=FAKE, sel=FAKE, ws=FAKE, ws_bytes=1 << 40, null_state=False):
    lib = H.load()
    sp = None if null_state else ctypes.byref(st or state())
    return lib.hsla_prefill_chunk(ctypes.byref(c.c()), ctypes.byref(p or pool()), sp, k, v, before, after, q,
                                  batch, q_len, max_len, out, sel, ws, ws_bytes, None)


@pytest.mark.parametrize("bad,code", BAD_CONFIGS)
def test_prefill_chunk_rejects_bad_configs(bad, code):
    assert call_prefill_chunk(cfg(**bad)) == code
    assert H.hsla_prefill_chunk_workspace_size(cfg(**bad), 8, 16, 32768) == 0


def test_prefill_chunk_limits_and_workspace():
    c = cfg()
    E = H.HSLA_ERR_INVALID_ARG
    # the chunk length: 1 .. min(block size, window - block size + 1)
    assert H.hsla_prefill_chunk_workspace_size(c, 8, 0, 32768) == 0
    assert H.hsla_prefill_chunk_workspace_size(c, 8, 65, 32768) == 0                    # > block size
    assert H.hsla_prefill_chunk_workspace_size(cfg(window=96), 8, 34, 32768) == 0       # > W - B + 1 = 33
    assert H.hsla_prefill_chunk_workspace_size(cfg(window=96), 8, 33, 32768) > 0
    assert call_prefill_chunk(c, q_len=0) == E
    assert call_prefill_chunk(c, q_len=65) == E
    assert call_prefill_chunk(cfg(window=96), q_len=34) == E
    # token-level selection has no chunk form here
    assert H.hsla_prefill_chunk_workspace_size(cfg(selection=H.HSLA_SEL_TOKEN), 8, 16, 32768) == 0
    assert call_prefill_chunk(cfg(selection=H.HSLA_SEL_TOKEN)) == H.HSLA_ERR_UNSUPPORTED
    # the chunk's decode covers batch x q_len rows: its workspace exceeds one decode's
    one = H.hsla_decode_workspace_size(c, 8, 32768)
    ws = H.hsla_prefill_chunk_workspace_size(c, 8, 16, 32768)
    assert ws > one and ws >= H.hsla_decode_workspace_size(c, 8 * 16, 32768) + 8 * 16 * 4
    assert call_prefill_chunk(c, ws_bytes=ws - 1) == H.HSLA_ERR_WORKSPACE


def test_prefill_chunk_rejects_bad_pointers():
    c = cfg()
    E = H.HSLA_ERR_INVALID_ARG
    assert call_prefill_chunk(c, after=FAKE) == E          # aliases seq_lens_before
    assert call_prefill_chunk(c, after=0) == E
    assert call_prefill_chunk(c, before=0) == E
    assert call_prefill_chunk(c, k=0) == E
    assert call_prefill_chunk(c, v=FAKE + 2) == E
    assert call_prefill_chunk(c, q=0) == E
    assert call_prefill_chunk(c, out=FAKE + 4) == E
    assert call_prefill_chunk(c, sel=FAKE + 2) == E
    assert call_prefill_chunk(c, null_state=True) == E
    assert call_prefill_chunk(c, p=pool(max_blocks_per_seq=100)) == E
    assert call_prefill_chunk(c, batch=0) == E


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """hsla_append_decode_noalloc refuses a shape whose workspace exceeds its
    fixed scratch before it touches the GPU (no pointer is dereferenced)."""
    assert H.hsla_noalloc_scratch_bytes() == 16 << 20
    c = cfg(top_k=8, window=256)
    batch, msl = 256, 8192
    assert H.hsla_decode_workspace_size(c, batch, msl) > H.hsla_noalloc_scratch_bytes()
    fake = 1 << 20   # 16-byte aligned, never dereferenced
    pool = H.hsla_kv_pool(fake, fake, fake, fake, fake, msl // 64 + 1, 1)
    state = H.hsla_state(fake, fake, fake)
    lib = H.load()
    st = lib.hsla_append_decode_noalloc(ctypes.byref(c.c()), ctypes.byref(pool), ctypes.byref(state), fake, fake,
                                        fake, fake + 4096, fake, batch, msl, fake, None, None)
    assert st == H.HSLA_ERR_WORKSPACE
    # an invalid configuration keeps its own status
    st = lib.hsla_append_decode_noalloc(ctypes.byref(cfg(head_dim=96).c()), ctypes.byref(pool), ctypes.byref(state),
                                        fake, fake, fake, fake + 4096, fake, 1, 1024, fake, None, None)
    assert st == H.HSLA_ERR_UNSUPPORTED


def test_split_choices_are_accepted():
    """deterministic: 0 (the library's default), 1 (fixed) and 2 (dynamic)
    all give a workspace size."""
    for split in (H.HSLA_SPLIT_DEFAULT, H.HSLA_SPLIT_FIXED, H.HSLA_SPLIT_DYNAMIC):
        c = cfg(deterministic=split)
        assert H.hsla_decode_workspace_size(c, 8, 32768) > 0, split


def test_phase_timestamps_only_in_the_diagnostic_build():
    """The release library records no phase stamps; libhsla_phases.so
    reports the documented buffer size and rejects a short buffer (host-side
    checks, no GPU)."""
    lib = H.load()
    assert lib.hsla_phase_timestamp_bytes() == 0
    buf = (ctypes.c_uint64 * 4)()
    assert lib.hsla_phase_timestamps(ctypes.addressof(buf), 32, 0) == H.HSLA_ERR_UNSUPPORTED
    if not os.path.exists(H.PHASES_LIB_PATH):
        pytest.skip("libhsla_phases.so not built")
    ph = H.open_library(H.PHASES_LIB_PATH)
    assert ph.hsla_phase_timestamp_bytes() == 8 * (4096 * 16 + 16384 * 2 + 8192 * 2)
    assert ph.hsla_phase_timestamps(ctypes.addressof(buf), 32, 0) == H.HSLA_ERR_INVALID_ARG
    assert ph.hsla_phase_timestamps(None, 1 << 30, 0) == H.HSLA_ERR_INVALID_ARG


def test_per_token_state_only_where_the_caller_updates_it():
    """state_span = HSLA_STATE_TOKENS: build, decode and the appends accept
    it; the chunk form, which folds whole blocks after its queries, refuses
    it on the host."""
    c = cfg(state_span=H.HSLA_STATE_TOKENS)
    assert H.hsla_decode_workspace_size(c, 8, 32768) == H.hsla_decode_workspace_size(cfg(), 8, 32768) > 0
    assert H.hsla_build_workspace_size(c, 8, 32768) > 0
    lib = H.load()
    U = H.HSLA_ERR_UNSUPPORTED
    assert call_prefill_chunk(c) == U
    assert H.hsla_prefill_chunk_workspace_size(c, 8, 16, 32768) == 0
