"""Host-side logic of bench.py (CPU only)."""

import numpy as np

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
