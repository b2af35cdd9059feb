"""fp64 CPU oracle of hybrid sparse-plus-linear decode attention.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The product path (the
HIP library under hybrid_sparse_linear_block_amd/ and its binding) never
imports, links or calls it.
"""
from .hsla_oracle import *  # noqa: F401,F403
from .hsla_oracle import (Params, LinearState, HeadResult, to_f64, kv_head_of, block_statistics,
                          block_score, sink_range, window_range, candidate_blocks, select_top_k,
                          exact_token_mask, global_state, state_over, append_token,
                          filled_block_stats, decode_head, dense_attention, decode_batch)
