"""GPU parity of the vertical-slash attention path (sparse_attn_forward_vs) against the oracle.

The kernel merges each tile's vertical and slash indices on the fly (VSPrefill page,
Metodologia B.3); the oracle builds the same lists as plain set unions (oracle.vs_lists) and
computes fp64 attention over them.  Outputs must agree within the bf16-input bar (2e-2 max-abs
with an fp32 output, plus half a bf16 ulp of |O| with a bf16 output).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

from parity import out_tol, say

pytestmark = pytest.mark.gpu

WL = wl.WORKLOADS


def _run_vs(w, inp, vert, slash, out_dtype=api.SA_F32, with_lse=False):
    p = api.problem(w)
    d = {k: v.cuda() for k, v in inp.items()}
    ws = torch.empty(api.forward_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    odt = torch.float32 if out_dtype == api.SA_F32 else torch.bfloat16
    O = torch.full((w.batch, w.seqlen, w.n_q_heads, w.head_dim), float("nan"), dtype=odt,
                   device="cuda")
    lse = (torch.empty((w.batch, w.n_q_heads, w.seqlen), dtype=torch.float32, device="cuda")
           if with_lse else None)
    api.forward_vs(p, d["Q"], d["K"], d["V"], torch.from_numpy(vert).cuda(),
                   torch.from_numpy(slash).cuda(), 1.0 / math.sqrt(w.head_dim), ws, O, out_dtype,
                   lse)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def _rows(w, rng, max_rows=5000):
    total = w.batch * w.seqlen * w.n_q_heads
    if total <= max_rows:
        return None
    fixed = [(0, 0, i) for t in (0, 1, w.n_blocks - 1) for i in range(t * w.block, (t + 1) * w.block)]
    k = max_rows - len(fixed)
    rnd = np.stack([rng.integers(0, w.batch, k), rng.integers(0, w.n_q_heads, k),
                    rng.integers(0, w.seqlen, k)], axis=1)
    return np.concatenate([np.array(fixed, np.int64), rnd.astype(np.int64)])


def _check(w, inp, vert, slash, tag, seed=0):
    cfg = oracle.make_cfg(w)
    idx, cnt = oracle.vs_lists(cfg, vert, slash)
    rows = _rows(w, np.random.default_rng(seed))
    say(f"[{tag}] oracle ({'all' if rows is None else len(rows)} rows) + GPU")
    O_ref, lse_ref = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt,
                                    1.0 / math.sqrt(w.head_dim), rows=rows)
    for out_dtype in (api.SA_F32, api.SA_BF16):
        O, lse = _run_vs(w, inp, vert, slash, out_dtype, with_lse=out_dtype == api.SA_F32)
        if rows is None:
            got = O
            ref = O_ref
        else:
            got = O[rows[:, 0], rows[:, 2], rows[:, 1]]
            ref = O_ref
        err = np.abs(got - ref)
        tol = out_tol(w, out_dtype, ref)
        assert np.isfinite(got).all(), tag
        assert (err <= tol).all(), f"{tag}: max err {err.max():.3e}"
        if lse is not None:
            lg = lse.transpose(0, 2, 1) if rows is None else lse[rows[:, 0], rows[:, 1], rows[:, 2]]
            assert np.abs(lg - lse_ref).max() <= 1e-3, tag
    return idx, cnt


def _planted(seqlen, **kw):
    w = WL["prefill_128k"].resized(seqlen=seqlen, **kw)
    ex = {}
    inp = wl.make_inputs(w, extras=ex)
    return w, inp, ex["anchors"]


def test_vs_planted_standin_index():
    w, inp, anchors = _planted(4096)
    vert, slash = wl.vs_index(w, 16, 8, anchors=anchors)
    _check(w, inp, vert, slash, "planted n32")


@pytest.mark.parametrize("name,w", [
    ("blk64_d128", WL["llama8b_32k"].resized(seqlen=2048, n_q_heads=8, n_kv_heads=2)),
    ("blk128_d64", WL["llama8b_32k"].resized(seqlen=2560, block=128, n_q_heads=4, n_kv_heads=2,
                                             head_dim=64)),
    ("blk64_d64_b2", WL["llama8b_32k"].resized(batch=2, seqlen=1280, n_q_heads=4, n_kv_heads=4,
                                               head_dim=64)),
])
def test_vs_random_index(name, w):
    inp = wl.make_inputs(w)
    vert, slash = wl.vs_index(w, 7, 5, seed=11)
    _check(w, inp, vert, slash, name)


def test_vs_edge_indices():
    """Empty indices (diagonal only), entries past the tile, -1 in mid-row, per-head lengths,
    and vertical blocks that the slash offsets reach too."""
    w = WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2)
    inp = wl.make_inputs(w)
    n = w.n_blocks  # 24
    vert = np.full((1, 4, 6), -1, np.int32)
    slash = np.full((1, 4, 5), -1, np.int32)
    # head 0: nothing but the diagonal
    # head 1: verticals reaching past most tiles, -1 ending the slash list early
    vert[0, 1] = [0, 5, 17, 23, -1, -1]
    slash[0, 1] = [1, 3, -1, 7, 9]
    # head 2: every even block vertical, even offsets: overlaps on even tiles
    vert[0, 2] = [0, 2, 4, 6, 8, 10]
    slash[0, 2] = [0, 2, 4, 6, 8]
    # head 3: offsets beyond most tiles, vertical including the last block
    vert[0, 3] = [3, n - 1, -1, -1, -1, -1]
    slash[0, 3] = [12, 20, 22, 23, -1]
    idx, cnt = _check(w, inp, vert, slash, "edges")
    assert (cnt[0, 0] == 1).all()


def test_vs_empty_index_arrays():
    """n_vertical = n_slash = 0: every tile reads its diagonal block only."""
    w = WL["llama8b_32k"].resized(seqlen=1024, n_q_heads=2, n_kv_heads=1)
    inp = wl.make_inputs(w)
    vert = np.zeros((1, 2, 0), np.int32)
    slash = np.zeros((1, 2, 0), np.int32)
    _check(w, inp, vert, slash, "empty")


def test_vs_all_vertical_is_dense():
    w = WL["llama8b_32k"].resized(seqlen=1024, n_q_heads=4, n_kv_heads=2)
    inp = wl.make_inputs(w)
    vert = np.tile(np.arange(w.n_blocks, dtype=np.int32), (1, 4, 1))
    slash = np.full((1, 4, 1), -1, np.int32)
    idx, cnt = _check(w, inp, vert, slash, "dense")
    assert (cnt[0, :, -1] == w.n_blocks).all()


@pytest.mark.timeout(600)
def test_vs_full_size_128k_sampled():
    """The 128K workload at full size with the stand-in index (64 vertical blocks, 64 slash
    offsets per head), in the launch configuration bench.py times for this path."""
    w = WL["prefill_128k"]
    say("[vs full] generating inputs")
    ex = {}
    inp = wl.make_inputs(w, extras=ex)
    vert, slash = wl.vs_index(w, 64, 64, anchors=ex["anchors"])
    cfg = oracle.make_cfg(w)
    idx, cnt = oracle.vs_lists(cfg, vert, slash)
    rng = np.random.default_rng(5)
    rows = np.stack([np.zeros(1500, np.int64), rng.integers(0, w.n_q_heads, 1500),
                     rng.integers(0, w.seqlen, 1500)], axis=1)
    say("[vs full] GPU")
    O, _ = _run_vs(w, inp, vert, slash, api.SA_BF16)
    got = O[rows[:, 0], rows[:, 2], rows[:, 1]]
    say("[vs full] oracle rows")
    ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt,
                            1.0 / math.sqrt(w.head_dim), rows=rows)
    err = np.abs(got - ref)
    assert (err <= out_tol(w, api.SA_BF16, ref)).all(), f"max err {err.max():.3e}"
    say(f"[vs full] max |O - O_ref| = {err.max():.2e}, mean list length {cnt.mean():.1f}")
