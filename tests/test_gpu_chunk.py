"""hsla_prefill_chunk (the multi-query form) against the oracle.

Every query row of the chunk is compared with the oracle's decode at its
own position (decode_chunk_head: query i of sequence b at length T0 + i + 1),
with the selection rule of the decode tests.  The chunk's page slots are
filled with a wrong value before the call, so the rows must come from the
chunk's keys and values.  The cache after the chunk (pages, block statistics,
state, lengths) must be bitwise equal to the one q_len hsla_append_token
calls leave, including chunks that complete a block.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
import workloads as W
from test_gpu_parity import _announce, _wl, cfg_of, check_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

from hybrid_sparse_linear_block_amd.device import DeviceCache, to_device  # noqa: E402

# T0 (the cache's length before the chunk) and the chunk length Q per case;
# sequence 0 completes a block inside the chunk in every case but one
CASES = {
    "bf16_g4": (dict(), (1530, 1137), 16),
    "bf16_g4_q1_completes": (dict(), (1535, 1203), 1),
    "f32_d64_b16": (dict(kv_dtype=W.F32, head_dim=64, block_size=16, window=64, top_k=12), (1471, 1203), 16),
    "bf16_g8": (dict(num_q_heads=16, num_kv_heads=2), (1530, 1203), 8),
    "grouped": (dict(grouped=1), (1530, 1137), 16),
    "no_linear_tail": (dict(linear_tail=0), (1530, 1137), 16),
    "deterministic": (dict(deterministic=1), (1530, 1137), 16),
    "no_candidates": (dict(), (200, 37), 16),
    "ragged_b1": (dict(batch=3, num_q_heads=8, num_kv_heads=8, top_k=8), (2043, 300, 1031), 16),
    "long_window_q64": (dict(window=512), (3000, 1986), 64),
}


def _setup(name):
    kw, t0, Q = CASES[name]
    lens = tuple(t + Q for t in t0)
    wl = _wl(f"chunk_{name}", 80, seq_lens=lens, **kw)
    inp = W.make_inputs(wl)
    Hkv, G, D = wl.num_kv_heads, wl.group, wl.head_dim
    # the chunk's keys/values (the sequences' last Q tokens) and queries
    kc = np.stack([np.stack([np.stack([inp["pairs"][(b, g)][0][t0[b] + i] for g in range(Hkv)])
                             for i in range(Q)]) for b in range(wl.batch)])
    vc = np.stack([np.stack([np.stack([inp["pairs"][(b, g)][1][t0[b] + i] for g in range(Hkv)])
                             for i in range(Q)]) for b in range(wl.batch)])
    rng = np.random.default_rng([777, wl.cid])
    qf = rng.standard_normal((wl.batch, Q, wl.num_q_heads, D)).astype(np.float32)
    qc = W.bf16_round(qf) if wl.kv_dtype == W.BF16 else qf
    # a wrong value in the chunk's page slots
    bad = np.uint16(0x4040) if wl.kv_dtype == W.BF16 else np.float32(3.0)
    for b in range(wl.batch):
        for i in range(Q):
            t = t0[b] + i
            page = inp["block_table"][b, t // wl.block_size]
            inp["k_pages"][page, :, t % wl.block_size, :] = bad
            inp["v_pages"][page, :, t % wl.block_size, :] = bad
    return wl, inp, np.asarray(t0, np.int64), Q, kc, vc, qc


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunk_rows_match_the_oracle(name):
    wl, inp, t0, Q, kc, vc, qc = _setup(name)
    _announce(wl, f"prefill chunk Q={Q} from T0={t0.tolist()}")
    lens = t0 + Q
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0, capacity_len=int(lens.max()))
    dc.build()
    out, sel = dc.prefill_chunk(to_device(kc), to_device(vc), to_device(qc))
    torch.cuda.synchronize()
    assert dc.seq_lens.cpu().numpy().tolist() == lens.tolist()
    out = out.cpu().numpy().reshape(wl.batch * Q, wl.num_q_heads, wl.head_dim)
    sel = None if sel is None else sel.cpu().numpy().reshape(wl.batch * Q, wl.num_q_heads, wl.top_k)

    # query row r = b Q + i is a decode of sequence b at length T0_b + i + 1
    rows = dataclasses.replace(wl, batch=wl.batch * Q, seq_lens=tuple(int(t0[r // Q]) + r % Q + 1
                                                                       for r in range(wl.batch * Q)))
    inp_rows = {"q": qc.reshape(wl.batch * Q, wl.num_q_heads, wl.head_dim), "block_table": None}

    def pair_data(r, g):
        K, V = inp["pairs"][(r // Q, g)]
        L = int(t0[r // Q]) + r % Q + 1
        return K[:L], V[:L]

    heads = [(r, h) for r in range(wl.batch * Q) for h in range(wl.num_q_heads)]
    worst, flips = check_case(rows, inp_rows, None, out, sel, heads=heads, check_build=False, pair_data=pair_data)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


@pytest.mark.parametrize("name", ["bf16_g4", "f32_d64_b16", "bf16_g4_q1_completes", "no_linear_tail"])
def test_chunk_leaves_the_cache_q_appends_leave(name):
    wl, inp, t0, Q, kc, vc, qc = _setup(name)
    _announce(wl, f"prefill chunk Q={Q} vs {Q} appends")
    cap = int((t0 + Q).max())
    a = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0, capacity_len=cap)
    b = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0, capacity_len=cap)
    a.build()
    b.build()
    a.prefill_chunk(to_device(kc), to_device(vc), to_device(qc))
    for i in range(Q):
        b.append(to_device(np.ascontiguousarray(kc[:, i])), to_device(np.ascontiguousarray(vc[:, i])))
    torch.cuda.synchronize()
    assert np.array_equal(a.host_lens, b.host_lens)
    assert torch.equal(a.seq_lens, b.seq_lens)
    for t in ("k_pages", "v_pages", "blk_mean", "blk_var", "S", "z", "sv"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t


def test_chunk_full_size_llama8b_32k():
    # the configuration `bench.py --chunk 16` times: batch 8 at 32768 tokens,
    # 32q/8kv, d 128, B 64, k 16; sampled (sequence, kv head) pairs and three
    # query rows of each against the oracle, every row for the properties
    # that hold at any size
    Q = 16
    wl = W.dataclasses.replace(W.llama8b_32k(), append_room=2)
    _announce(wl, f"full size, prefill chunk Q={Q}, sampled pairs")
    inp = W.make_inputs(wl, keep_pairs=False)
    t0 = np.asarray(wl.seq_lens, np.int64)
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0,
                     capacity_len=int(t0.max()) + Q)
    dc.build()
    rng = np.random.default_rng([99, Q])
    kc, vc = (W.bf16_round(rng.standard_normal((wl.batch, Q, wl.num_kv_heads, wl.head_dim)).astype(np.float32))
              for _ in range(2))
    qc = W.bf16_round(rng.standard_normal((wl.batch, Q, wl.num_q_heads, wl.head_dim)).astype(np.float32))
    out, sel = dc.prefill_chunk(to_device(kc), to_device(vc), to_device(qc))
    torch.cuda.synchronize()
    out, sel = out.cpu().numpy(), sel.cpu().numpy()
    assert np.isfinite(out).all()
    B = wl.block_size
    for b in range(wl.batch):
        for i in range(Q):
            L = int(t0[b]) + i + 1
            n_cand = -(-(L - wl.window) // B) - wl.num_sink // B
            for h in range(wl.num_q_heads):
                row = [x for x in sel[b, i, h].tolist() if x >= 0]
                assert row == sorted(set(row)) and len(row) == min(wl.top_k, n_cand), (b, i, h)
                assert all(wl.num_sink // B <= x < wl.num_sink // B + n_cand for x in row), (b, i, h)

    rows = dataclasses.replace(wl, batch=wl.batch * Q, seq_lens=tuple(int(t0[r // Q]) + r % Q + 1
                                                                       for r in range(wl.batch * Q)))
    full = {}

    def pair_data(r, g):
        b, i = r // Q, r % Q
        if (b, g) not in full:
            K, V = W.gen_pair(wl, b, g, inp["q"])
            full[(b, g)] = (np.concatenate([K[:t0[b]], kc[b, :, g]]), np.concatenate([V[:t0[b]], vc[b, :, g]]))
        K, V = full[(b, g)]
        return K[:int(t0[b]) + i + 1], V[:int(t0[b]) + i + 1]

    G = wl.group
    pairs = [(0, 0), (wl.batch // 2, wl.num_kv_heads // 2), (wl.batch - 1, wl.num_kv_heads - 1)]
    heads = [(b * Q + i, h) for b, g in pairs for i in (0, Q // 2, Q - 1) for h in range(g * G, (g + 1) * G)]
    inp_rows = {"q": qc.reshape(wl.batch * Q, wl.num_q_heads, wl.head_dim), "block_table": None}
    worst, flips = check_case(rows, inp_rows, None, out.reshape(wl.batch * Q, wl.num_q_heads, wl.head_dim),
                              sel.reshape(wl.batch * Q, wl.num_q_heads, wl.top_k), heads=heads,
                              check_build=False, pair_data=pair_data)
    print(f"  worst row error {worst:.3e}, near-tie flips {flips}")


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_prefill_from_empty_in_chunks(kv):
    # a prefill from nothing as chunked calls: T0 = (0, 3), eight chunks of
    # 16 (B 16, W 64), so that later rows have candidates, a selection and a
    # linear tail; every row of every chunk against the oracle
    Q, n_chunks, t_start = 16, 8, (0, 3)
    kw = dict(kv_dtype=W.BF16 if kv == "bf16" else W.F32, head_dim=64, block_size=16, window=64, top_k=2,
              num_sink=4)
    final = tuple(t + Q * n_chunks for t in t_start)
    wl = _wl(f"chunk_from_empty_{kv}", 81, seq_lens=final, **kw)
    _announce(wl, f"prefill from {list(t_start)} in {n_chunks} chunks of {Q}")
    inp = W.make_inputs(wl)
    bad = np.uint16(0x4040) if wl.kv_dtype == W.BF16 else np.float32(3.0)
    for b in range(wl.batch):
        for t in range(t_start[b], final[b]):
            page = inp["block_table"][b, t // wl.block_size]
            inp["k_pages"][page, :, t % wl.block_size, :] = bad
            inp["v_pages"][page, :, t % wl.block_size, :] = bad
    t0 = np.asarray(t_start, np.int64)
    dc = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0,
                     capacity_len=int(max(final)))
    dc.build()
    rng = np.random.default_rng([5150, wl.cid])
    worst_all = 0.0
    for c in range(n_chunks):
        kc = np.stack([np.stack([np.stack([inp["pairs"][(b, g)][0][t0[b] + i] for g in range(wl.num_kv_heads)])
                                 for i in range(Q)]) for b in range(wl.batch)])
        vc = np.stack([np.stack([np.stack([inp["pairs"][(b, g)][1][t0[b] + i] for g in range(wl.num_kv_heads)])
                                 for i in range(Q)]) for b in range(wl.batch)])
        qf = rng.standard_normal((wl.batch, Q, wl.num_q_heads, wl.head_dim)).astype(np.float32)
        qc = W.bf16_round(qf) if wl.kv_dtype == W.BF16 else qf
        out, sel = dc.prefill_chunk(to_device(kc), to_device(vc), to_device(qc))
        torch.cuda.synchronize()
        assert dc.seq_lens.cpu().numpy().tolist() == (t0 + Q).tolist()
        R = wl.batch * Q
        rows = dataclasses.replace(wl, batch=R, seq_lens=tuple(int(t0[r // Q]) + r % Q + 1 for r in range(R)))

        def pair_data(r, g, t0=t0.copy()):
            K, V = inp["pairs"][(r // Q, g)]
            L = int(t0[r // Q]) + r % Q + 1
            return K[:L], V[:L]

        heads = [(r, h) for r in range(R) for h in range(wl.num_q_heads)]
        worst, _ = check_case(rows, {"q": qc.reshape(R, wl.num_q_heads, wl.head_dim), "block_table": None}, None,
                              out.cpu().numpy().reshape(R, wl.num_q_heads, wl.head_dim),
                              sel.cpu().numpy().reshape(R, wl.num_q_heads, wl.top_k), heads=heads,
                              check_build=False, pair_data=pair_data)
        worst_all = max(worst_all, worst)
        t0 = t0 + Q
    print(f"  worst row error over {n_chunks} chunks {worst_all:.3e}")


@pytest.mark.parametrize("deterministic", [1, 2])
def test_chunk_graph_replays_match_eager_chunks(deterministic):
    # two chunks per captured graph (the ping-ponged length buffers return),
    # replayed three times with eager torch work and synchronisation in
    # between; every replay against the eager chunks of the same lengths
    Q, replays = 16, 3
    t_start = (1530, 1137)
    steps = 2 * replays
    wl = _wl("chunk_graph", 82, deterministic=deterministic, append_room=4,
             seq_lens=tuple(t + Q * steps for t in t_start))
    _announce(wl, f"prefill chunk Q={Q} in a HIP graph, deterministic={deterministic}")
    inp = W.make_inputs(wl, keep_pairs=False)
    t0 = np.asarray(t_start, np.int64)
    cap = int(max(wl.seq_lens))
    rng = np.random.default_rng([31, deterministic])
    cvt = W.bf16_round
    kc = to_device(cvt(rng.standard_normal((wl.batch, Q, wl.num_kv_heads, wl.head_dim)).astype(np.float32)))
    vc = to_device(cvt(rng.standard_normal((wl.batch, Q, wl.num_kv_heads, wl.head_dim)).astype(np.float32)))
    qc = to_device(cvt(rng.standard_normal((wl.batch, Q, wl.num_q_heads, wl.head_dim)).astype(np.float32)))
    caches = [DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0, capacity_len=cap)
              for _ in range(2)]
    for dc in caches:
        dc.build()
    eager, graphed = caches
    outs = [torch.empty((wl.batch, Q, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(2)]
    sels = [torch.empty((wl.batch, Q, wl.num_q_heads, wl.top_k), dtype=torch.int32, device="cuda") for _ in range(2)]
    want = []
    for s in range(steps):
        o, sl = eager.prefill_chunk(kc, vc, qc)
        if s % 2 == 1:
            torch.cuda.synchronize()
            want.append((o.cpu().numpy(), sl.cpu().numpy()))

    # the captured cache takes the workspace a call on a third cache
    # allocated outside the capture (same chunk length and capacity), so
    # that nothing is allocated while capturing
    graphed2 = DeviceCache(cfg_of(wl), inp["k_pages"], inp["v_pages"], inp["block_table"], t0, capacity_len=cap)
    graphed2.build()
    graphed2.prefill_chunk(kc, vc, qc, outs[0], sels[0])
    torch.cuda.synchronize()
    graphed.__dict__.update({"_chunk_ws": graphed2._chunk_ws, "_chunk_ws_key": graphed2._chunk_ws_key})
    gs = torch.cuda.Stream()
    saved = (graphed.cur, graphed.host_lens.copy())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    gs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=gs):
        graphed.prefill_chunk(kc, vc, qc, outs[0], sels[0], stream=gs.cuda_stream)
        graphed.prefill_chunk(kc, vc, qc, outs[1], sels[1], stream=gs.cuda_stream)
    graphed.cur, graphed.host_lens[:] = saved
    noise = torch.randn(512, 512, device="cuda")
    for r in range(replays):
        graph.replay()
        torch.cuda.synchronize()
        go, gsel = outs[1].cpu().numpy(), sels[1].cpu().numpy()
        noise = noise @ noise.T / 512.0
        torch.cuda.synchronize()
        wo, wsel = want[r]
        assert np.array_equal(gsel, wsel), r
        if deterministic == 1:
            assert np.array_equal(go, wo), r
        else:
            err = np.abs(go - wo).max(axis=-1) / np.abs(wo).max(axis=-1)
            assert err.max() < 1e-5, (r, float(err.max()))
    graphed.host_lens += steps * Q
    assert np.array_equal(graphed.host_lens, eager.host_lens)
    assert torch.equal(graphed.lens[graphed.cur], eager.lens[eager.cur])
    for t in ("k_pages", "v_pages", "blk_mean", "blk_var", "S", "z", "sv"):
        assert torch.equal(getattr(graphed, t), getattr(eager, t)), t
