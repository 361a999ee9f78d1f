"""Helpers shared by the GPU parity tests: run the HIP path and the oracle on the same inputs."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

# Output tolerances (max-abs) for the attention output against the fp64 oracle.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    return {k: v.cuda() for k, v in inp.items()}


def run_gpu(w: wl.Workload, inp, out_dtype=None, with_lse=False):
    """Whole pipeline on the GPU; returns host numpy copies of every output."""
    d = to_dev(inp)
    pf = api.Prefill(w, out_dtype=out_dtype, with_lse=with_lse)
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    n = w.n_blocks
    plane = w.batch * n * w.n_kv_heads * w.head_dim
    summ = pf.summ.cpu().numpy()
    out = {
        "kA": summ[:plane].reshape(w.batch, n, w.n_kv_heads, w.head_dim),
        "kB": (summ[plane:2 * plane].reshape(w.batch, n, w.n_kv_heads, w.head_dim)
               if w.score_mode == wl.KMINMAX else None),
        "vn": (summ[plane * (2 if w.score_mode == wl.KMINMAX else 1):][:w.batch * n * w.n_kv_heads]
               .reshape(w.batch, n, w.n_kv_heads) if w.output_aware else None),
        "kv_idx": pf.kv_idx.cpu().numpy(), "kv_cnt": pf.kv_cnt.cpu().numpy(),
        "sigma": pf.sigma.cpu().numpy(), "sigma_bar": pf.sigma_bar.cpu().numpy(),
        "gate": pf.gate.cpu().numpy(), "tau": pf.tau.cpu().numpy(),
        "O": pf.O.float().cpu().numpy(), "W": pf.W, "scale": pf.scale,
    }
    if with_lse:
        out["lse"] = pf.lse.cpu().numpy()
    return out


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_summaries_equal(w, g, o):
    np.testing.assert_array_equal(bits(g["kA"]), bits(o["kA"]))
    if w.score_mode == wl.KMINMAX:
        np.testing.assert_array_equal(bits(g["kB"]), bits(o["kB"]))
    if w.output_aware:
        np.testing.assert_array_equal(bits(g["vn"]), bits(o["vn"]))


def assert_selection_equal(g, o):
    np.testing.assert_array_equal(g["kv_cnt"], o["kv_cnt"])
    np.testing.assert_array_equal(g["kv_idx"], o["kv_idx"])
    np.testing.assert_array_equal(bits(g["sigma"]), bits(o["sigma"]))
    np.testing.assert_array_equal(bits(g["sigma_bar"]), bits(o["sigma_bar"]))
    np.testing.assert_array_equal(g["gate"], o["gate"])
    np.testing.assert_array_equal(bits(g["tau"]), bits(o["tau"]))


def out_tol(w, out_dtype, O_ref):
    """Max-abs bound per element: the fp32 / bf16 bars, plus the bf16 output cast's half ulp."""
    if w.dtype == wl.F32:
        base = TOL_F32
    else:
        base = TOL_BF16
    if out_dtype == api.SA_BF16:
        return base + np.abs(O_ref) * 2.0 ** -8
    return base


def check_structure(w, kv_idx, kv_cnt, gate, sigma, sigma_bar, tau):
    """Properties every selection output has at any size (vectorised over all tiles)."""
    B, Hq, n, W = kv_idx.shape
    assert n == w.n_tiles
    m = max(1, w.tile // w.block)  # diagonal blocks per tile: d0 .. d0 + m - 1
    t = np.arange(n)
    d0 = t * w.tile // w.block     # the tile's first diagonal block
    cnt = kv_cnt
    assert np.all(cnt >= 1) and np.all(cnt <= W)
    col = np.arange(W)
    valid = col[None, None, None, :] < cnt[..., None]
    assert np.all(kv_idx[~valid] == -1)
    last = np.take_along_axis(kv_idx, (cnt - 1)[..., None], axis=-1)[..., 0]
    assert np.all(last == (d0 + m - 1)[None, None, :]), "diagonal block missing or not last"
    if m > 1:
        prev = np.take_along_axis(kv_idx, (cnt - 2)[..., None], axis=-1)[..., 0]
        assert np.all(prev == (d0 + m - 2)[None, None, :]), "first diagonal block missing"
    d = np.diff(kv_idx, axis=-1)
    vd = valid[..., 1:]
    assert np.all(d[vd] > 0), "lists not strictly ascending"
    assert np.all(kv_idx[valid] >= 0)
    for s in range(min(w.n_sink, w.n_blocks)):
        has = (kv_idx == s).any(-1)
        assert np.all(has[:, :, d0 + m - 1 >= s]), "sink missing"
    assert np.all((sigma >= 0) & (sigma <= 1))
    # gate = eligible and sigma_bar <= tau, tau the ceil(q M)-th smallest eligible sigma_bar
    cfg = oracle.make_cfg(w)
    kt = np.array([oracle.budget(cfg, int(x)) for x in t])
    nfree = d0 - np.minimum(d0, w.n_sink)
    elig = nfree > kt
    for b in range(B):
        sb = sigma_bar[b][elig]
        M = len(sb)
        r = min(M, max(0, math.ceil(w.q * M)))
        want_tau = np.float32(np.sort(sb)[r - 1]) if (r > 0 and w.gate_mode == wl.GATE_QUANTILE) \
            else np.float32(-np.inf)
        if w.gate_mode == wl.GATE_QUANTILE:
            assert bits(tau[b]) == bits(want_tau)
        np.testing.assert_array_equal(gate[b], (elig & (sigma_bar[b] <= tau[b])).astype(np.uint8))
        keep = np.where(gate[b] == 1, np.floor(w.rho * kt).astype(int), kt)
        keep = np.minimum(keep, nfree)
        forced = m + np.minimum(d0, w.n_sink)
        np.testing.assert_array_equal(cnt[b], np.broadcast_to(forced + keep, cnt[b].shape))
