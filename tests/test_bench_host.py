"""Host-side logic of bench.py (CPU only)."""

import numpy as np
import torch

import bench
import oracle
from block_sparse_causal_mean_amd import workloads as wl


def test_vs_block_counts_match_the_oracle_lists():
    """bench.py's FLOP count for the vertical-slash path uses the same per-tile block counts as
    the oracle's lists, including indices ended early by -1."""
    for w, nv, ns in [(wl.WORKLOADS["llama8b_32k"].resized(seqlen=1536, n_q_heads=4,
                                                           n_kv_heads=2), 6, 5),
                      (wl.WORKLOADS["prefill_128k"].resized(seqlen=8192), 16, 9)]:
        vert, slash = wl.vs_index(w, nv, ns, seed=3)
        vert[0, 1, 3:] = -1
        slash[0, 2, 2:] = -1
        _, cnt = oracle.vs_lists(oracle.make_cfg(w), vert, slash)
        np.testing.assert_array_equal(bench.vs_block_counts(w, vert, slash), cnt)


def test_effective_flops_count_shared_lists_once_per_head():
    """A list shared by a kv head's G query heads is attended by all G of them."""
    per_head = wl.WORKLOADS["llama8b_32k"].resized(seqlen=2048)
    shared = wl.WORKLOADS["llama8b_32k_kvshared"].resized(seqlen=2048)
    n = per_head.n_blocks
    c_head = torch.full((1, per_head.n_q_heads, n), 3, dtype=torch.int32)
    c_shared = torch.full((1, shared.n_kv_heads, n), 3, dtype=torch.int32)
    assert bench.effective_flops(per_head, c_head) == bench.effective_flops(shared, c_shared)
    assert bench.effective_flops(shared, c_shared) == 4.0 * 64 * 64 * 128 * 32 * n * 3


def test_causal_exact_flops_leave_out_the_masked_pairs():
    """Dense causal lists: the exact count is 4 d per (row, key <= row) pair, N (N + 1) / 2
    pairs per head, for tiles equal to blocks and for 128-row tiles over 64-key blocks;
    without the diagonal blocks' masked pairs the count is the effective one."""
    for w in (wl.WORKLOADS["prefill_128k"].resized(seqlen=1024, n_q_heads=2, n_kv_heads=1),
              wl.WORKLOADS["llama8b_32k_t128"].resized(seqlen=1024, n_q_heads=2, n_kv_heads=1)):
        m, nt = w.tile // w.block, w.n_tiles
        W = m * nt
        idx = torch.full((1, 2, nt, W), -1, dtype=torch.int32)
        cnt = torch.zeros((1, 2, nt), dtype=torch.int32)
        for t in range(nt):
            idx[0, :, t, :m * (t + 1)] = torch.arange(m * (t + 1), dtype=torch.int32)
            cnt[0, :, t] = m * (t + 1)
        N = w.seqlen
        assert bench.causal_exact_flops(w, idx, cnt) == 4.0 * w.head_dim * 2 * N * (N + 1) / 2
        diag_masked = 2 * nt * 4.0 * w.head_dim * w.tile * (w.tile - 1) / 2
        assert (bench.effective_flops(w, cnt) - bench.causal_exact_flops(w, idx, cnt)
                == diag_masked)
