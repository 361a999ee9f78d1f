"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The whole pipeline runs on the full input (bf16 output, no lse: exactly what bench.py runs).
The oracle cannot redo every tile at these sizes in test time, so the check is layered:

  * block summaries: every block, bit for bit (the oracle pools the full input cheaply);
  * selection: sampled tiles (first, second, middle, last, tripped ones and random ones), every
    head: sigma, sigma_bar, eligibility, kv_idx and kv_cnt bit for bit against oracle.select_tile;
  * gate and lists everywhere: the properties that hold at any size (check_structure: tau is
    the ceil(q M)-th smallest eligible sigma_bar, gate = eligible and sigma_bar <= tau, counts =
    forced + kept, lists ascending with the diagonal last, sinks present, sigma in [0, 1]);
  * attention: rows of the sampled tiles (all heads' first rows, random heads' rows) against the
    fp64 oracle on the GPU's own lists, to 2e-2 plus the bf16 output cast.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

from parity import bits, check_structure, out_tol, say

pytestmark = pytest.mark.gpu

FULL = ["llama8b_32k", "prefill_128k", "quest_64k", "stem_32k", "stem_additive_32k",
        "llama8b_32k_kvshared", "stem_32k_kvshared", "llama8b_32k_t128", "stem_32k_t128"]


def _sample_tiles(n, gate_row, rng, extra=4):
    tiles = {0, 1, n // 3, n // 2, n - 1}
    tripped = np.nonzero(gate_row)[0]
    if len(tripped):
        tiles.update(int(x) for x in rng.choice(tripped, size=min(3, len(tripped)), replace=False))
    tiles.update(int(x) for x in rng.integers(2, n - 1, size=extra))
    return sorted(tiles)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    w = wl.WORKLOADS[name]
    say(f"[full] {name}: generating inputs")
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w)  # bench configuration: bf16 output, no lse
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    say(f"[full] {name}: GPU pipeline done")
    n, B, Hq, G = w.n_tiles, w.batch, w.n_q_heads, w.n_q_heads // w.n_kv_heads
    kv_idx, kv_cnt = pf.kv_idx.cpu().numpy(), pf.kv_cnt.cpu().numpy()
    sigma, sigma_bar = pf.sigma.cpu().numpy(), pf.sigma_bar.cpu().numpy()
    gate, tau = pf.gate.cpu().numpy(), pf.tau.cpu().numpy()

    # Properties of every tile.
    check_structure(w, kv_idx, kv_cnt, gate, sigma, sigma_bar, tau)
    trips = int(gate.sum())
    say(f"[full] {name}: structure ok, {trips} tripped tiles of {B * n}")

    # Summaries, in full.
    cfg = oracle.make_cfg(w)
    summ = oracle.pool(cfg, inp["K"], inp["V"])
    plane = B * w.n_blocks * w.n_kv_heads * w.head_dim
    g_summ = pf.summ.cpu().numpy()
    np.testing.assert_array_equal(bits(g_summ[:plane]), bits(summ["kA"].reshape(-1)))
    off = plane
    if w.score_mode == wl.KMINMAX:
        np.testing.assert_array_equal(bits(g_summ[plane:2 * plane]), bits(summ["kB"].reshape(-1)))
        off = 2 * plane
    if w.output_aware:
        np.testing.assert_array_equal(bits(g_summ[off:off + B * w.n_blocks * w.n_kv_heads]),
                                      bits(summ["vn"].reshape(-1)))

    # Selection of sampled tiles, every head.
    rng = np.random.default_rng(7)
    rows = []
    for b in range(B):
        tiles = _sample_tiles(n, gate[b], rng)
        for t in tiles:
            one = oracle.select_tile(cfg, inp["Q"], summ, b, t)
            np.testing.assert_array_equal(bits(sigma[b, :, t]), bits(one["sigma"]))
            assert bits(sigma_bar[b, t]) == bits(one["sigma_bar"])
            lists = one["lists"][int(gate[b, t])]
            cnts = one["cnts"][int(gate[b, t])]
            np.testing.assert_array_equal(kv_cnt[b, :, t], cnts)
            np.testing.assert_array_equal(kv_idx[b, :, t, :], lists[:, :kv_idx.shape[-1]])
            # rows to check: first and last row of the tile for every head, plus 16 random
            # (head, row) pairs
            for h in range(Hq):
                rows.append((b, h, t * w.tile))
                rows.append((b, h, t * w.tile + w.tile - 1))
            for _ in range(16):
                rows.append((b, int(rng.integers(Hq)), t * w.tile + int(rng.integers(w.tile))))
        say(f"[full] {name}: batch {b}: tiles {tiles} match the oracle")

    rows = np.array(rows, np.int64)
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], kv_idx, kv_cnt, pf.scale,
                              rows=rows)
    r = torch.as_tensor(rows, device="cuda")
    O = pf.O[r[:, 0], r[:, 2], r[:, 1]].float().cpu().numpy()
    err = np.abs(O.astype(np.float64) - O_ref)
    tol = out_tol(w, api.SA_BF16, O_ref)
    say(f"[full] {name}: {len(rows)} rows, max|O - O_ref| = {err.max():.3e}")
    assert np.all(err <= tol), f"max err {err.max()} at row {rows[err.max(axis=1).argmax()]}"
