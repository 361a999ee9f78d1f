"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times.

The whole pipeline runs on the full input (bf16 output, no lse: exactly what bench.py runs),
and is compared with the oracle in full where the oracle can do it in test time:

  * block summaries: every block, bit for bit;
  * selection: the whole oracle selection (oracle.select) on the same input: sigma, sigma_bar,
    tau, the gate bits, kv_idx and kv_cnt of every tile and selection unit, bit for bit; and the
    properties that hold at any size (check_structure), as a second, independent reading;
  * attention: one row of every tile (a random head and row) plus the first and last rows of
    a few tiles for every head, against the fp64 oracle on the same lists: the bf16 output to
    2e-2 plus half a bf16 ulp of |O| (the output cast), and an fp32 output of the same call to
    the plain 2e-2.
"""

import numpy as np
import pytest
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

from parity import TOL_BF16, assert_selection_equal, bits, check_structure, out_tol, say

pytestmark = pytest.mark.gpu

FULL = ["llama8b_32k", "prefill_128k", "quest_64k", "stem_32k", "stem_additive_32k",
        "llama8b_32k_kvshared", "stem_32k_kvshared", "llama8b_32k_t128", "stem_32k_t128",
        "prefill_128k_t64"]


def _rows(w, rng):
    """One random (head, row) in every tile of every batch element, plus the first and last
    rows of tiles 0, 1, n/2 and n-1 for every head."""
    n, T, Hq = w.n_tiles, w.tile, w.n_q_heads
    rows = []
    for b in range(w.batch):
        heads = rng.integers(Hq, size=n)
        offs = rng.integers(T, size=n)
        rows += [(b, int(heads[t]), t * T + int(offs[t])) for t in range(n)]
        for t in sorted({0, 1, n // 2, n - 1}):
            for h in range(Hq):
                rows += [(b, h, t * T), (b, h, t * T + T - 1)]
    return np.array(rows, np.int64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    w = wl.WORKLOADS[name]
    say(f"[full] {name}: generating inputs")
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w)  # bench configuration: bf16 output, no lse
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    say(f"[full] {name}: GPU pipeline done")
    B = w.batch
    g = {"kv_idx": pf.kv_idx.cpu().numpy(), "kv_cnt": pf.kv_cnt.cpu().numpy(),
         "sigma": pf.sigma.cpu().numpy(), "sigma_bar": pf.sigma_bar.cpu().numpy(),
         "gate": pf.gate.cpu().numpy(), "tau": pf.tau.cpu().numpy()}
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"], g["tau"])
    say(f"[full] {name}: structure ok, {int(g['gate'].sum())} tripped tiles of {B * w.n_tiles}")

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
    say(f"[full] {name}: summaries equal; oracle selection of every tile ({oracle.threads()} "
        f"threads)")

    # The whole selection.
    o_sel = oracle.select(cfg, inp["Q"], summ)
    assert_selection_equal(g, o_sel)
    say(f"[full] {name}: selection equal on every tile (tau {g['tau'].tolist()})")

    # Attention: a row of every tile, bf16 output (the benchmark's) and fp32 output.
    rows = _rows(w, np.random.default_rng(7))
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], g["kv_idx"], g["kv_cnt"],
                              pf.scale, rows=rows)
    r = torch.as_tensor(rows, device="cuda")
    O16 = pf.O[r[:, 0], r[:, 2], r[:, 1]].float().cpu().numpy().astype(np.float64)
    err16 = np.abs(O16 - O_ref)
    O32 = torch.empty(pf.O.shape, dtype=torch.float32, device="cuda")
    api.forward(pf.p, d["Q"], d["K"], d["V"], pf.kv_idx, pf.kv_cnt, pf.W, pf.scale, pf.fws, O32,
                api.SA_F32)
    torch.cuda.synchronize()
    err32 = np.abs(O32[r[:, 0], r[:, 2], r[:, 1]].cpu().numpy().astype(np.float64) - O_ref)
    say(f"[full] {name}: {len(rows)} rows (every tile), max|O - O_ref| = {err32.max():.3e} "
        f"(fp32 out), {err16.max():.3e} (bf16 out)")
    assert np.all(err32 <= TOL_BF16), f"fp32 out: max err {err32.max()}"
    assert np.all(err16 <= out_tol(w, api.SA_BF16, O_ref)), f"bf16 out: max err {err16.max()}"


def _sample_tiles(n, gate_row, rng, extra=4):
    tiles = {0, 1, n // 3, n // 2, n - 1}
    tripped = np.nonzero(gate_row)[0]
    if len(tripped):
        tiles.update(int(x) for x in rng.choice(tripped, size=min(2, len(tripped)), replace=False))
    tiles.update(int(x) for x in rng.integers(2, n - 1, size=extra))
    return sorted(tiles)


@pytest.mark.timeout(900)
def test_one_million_tokens_sampled_parity():
    """The 128K recipe at 2^20 tokens (8192 blocks of 128 keys).  The oracle's whole selection
    would take tens of minutes here, so: every block summary bit for bit; the structure of
    every tile's selection (tau from sigma_bar, gate, counts, lists); sampled tiles (first,
    last, middle, tripped, random) against oracle.select_tile bit for bit, all heads; and
    sampled output rows against the fp64 oracle."""
    w = wl.WORKLOADS["prefill_1m"]
    say("[1m] generating inputs")
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w)
    say("[1m] GPU pipeline")
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    g = {"kv_idx": pf.kv_idx.cpu().numpy(), "kv_cnt": pf.kv_cnt.cpu().numpy(),
         "sigma": pf.sigma.cpu().numpy(), "sigma_bar": pf.sigma_bar.cpu().numpy(),
         "gate": pf.gate.cpu().numpy(), "tau": pf.tau.cpu().numpy()}
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"], g["tau"])
    say(f"[1m] structure ok, {int(g['gate'].sum())} tripped tiles of {w.n_tiles}")
    cfg = oracle.make_cfg(w)
    summ = oracle.pool(cfg, inp["K"], inp["V"])
    plane = w.n_blocks * w.n_kv_heads * w.head_dim
    np.testing.assert_array_equal(bits(pf.summ[:plane].cpu().numpy()), bits(summ["kA"].reshape(-1)))
    say("[1m] summaries equal")
    rng = np.random.default_rng(11)
    tiles = _sample_tiles(w.n_tiles, g["gate"][0], rng)
    rows = []
    for t in tiles:
        one = oracle.select_tile(cfg, inp["Q"], summ, 0, t)
        np.testing.assert_array_equal(bits(g["sigma"][0, :, t]), bits(one["sigma"]))
        assert bits(g["sigma_bar"][0, t]) == bits(one["sigma_bar"])
        tr = int(g["gate"][0, t])
        np.testing.assert_array_equal(g["kv_cnt"][0, :, t], one["cnts"][tr])
        np.testing.assert_array_equal(g["kv_idx"][0, :, t, :], one["lists"][tr][:, :g["kv_idx"].shape[-1]])
        for h in range(w.n_q_heads):
            rows.append((0, h, t * w.tile + int(rng.integers(w.tile))))
        say(f"[1m] tile {t} (tripped {tr}) matches the oracle")
    rows = np.array(rows, np.int64)
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], g["kv_idx"], g["kv_cnt"],
                              pf.scale, rows=rows)
    r = torch.as_tensor(rows, device="cuda")
    O = pf.O[r[:, 0], r[:, 2], r[:, 1]].float().cpu().numpy().astype(np.float64)
    err = np.abs(O - O_ref)
    say(f"[1m] {len(rows)} rows, max|O - O_ref| = {err.max():.3e}")
    assert np.all(err <= out_tol(w, api.SA_BF16, O_ref))


MAX_BLOCKS = {
    # 16384 key blocks of 64 keys (2^20 tokens), the most a problem may have: the mean-pooled
    # and the bound backbone, two query heads on one kv head, d = 64, k = 4
    "kmean": wl.WORKLOADS["llama8b_32k"].resized(seqlen=64 * 16384, n_q_heads=2, n_kv_heads=1,
                                                 head_dim=64, k_max=4, k_min=4),
    "bound": wl.WORKLOADS["quest_64k"].resized(seqlen=64 * 16384, n_q_heads=2, n_kv_heads=1,
                                               head_dim=64, k_max=4, k_min=4),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(MAX_BLOCKS))
def test_most_blocks_a_problem_may_have_sampled_parity(name):
    """16384 blocks of 64 keys, the largest block count the library admits (the selection's
    sort keys and the gate's LDS are sized for it): every block summary bit for bit; the
    structure of every tile's selection; sampled tiles (first, last, middle, tripped, random)
    against oracle.select_tile bit for bit in both heads; output rows (one in every tile, and
    one per head in each sampled tile) against the fp64 oracle."""
    w = MAX_BLOCKS[name]
    assert w.n_blocks == 16384 and w.n_tiles == 16384
    say(f"[max {name}] generating inputs")
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w)
    say(f"[max {name}] GPU pipeline")
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    g = {"kv_idx": pf.kv_idx.cpu().numpy(), "kv_cnt": pf.kv_cnt.cpu().numpy(),
         "sigma": pf.sigma.cpu().numpy(), "sigma_bar": pf.sigma_bar.cpu().numpy(),
         "gate": pf.gate.cpu().numpy(), "tau": pf.tau.cpu().numpy()}
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"], g["tau"])
    say(f"[max {name}] structure ok, {int(g['gate'].sum())} tripped tiles of {w.n_tiles}")
    cfg = oracle.make_cfg(w)
    summ = oracle.pool(cfg, inp["K"], inp["V"])
    planes = 2 if w.score_mode == wl.KMINMAX else 1
    plane = w.n_blocks * w.n_kv_heads * w.head_dim
    got = bits(pf.summ[:planes * plane].cpu().numpy())
    np.testing.assert_array_equal(got[:plane], bits(summ["kA"].reshape(-1)))
    if planes == 2:
        np.testing.assert_array_equal(got[plane:], bits(summ["kB"].reshape(-1)))
    say(f"[max {name}] summaries equal")
    rng = np.random.default_rng(13)
    tiles = _sample_tiles(w.n_tiles, g["gate"][0], rng)
    rows = []
    for t in tiles:
        one = oracle.select_tile(cfg, inp["Q"], summ, 0, t)
        np.testing.assert_array_equal(bits(g["sigma"][0, :, t]), bits(one["sigma"]))
        assert bits(g["sigma_bar"][0, t]) == bits(one["sigma_bar"])
        tr = int(g["gate"][0, t])
        np.testing.assert_array_equal(g["kv_cnt"][0, :, t], one["cnts"][tr])
        np.testing.assert_array_equal(g["kv_idx"][0, :, t, :],
                                      one["lists"][tr][:, :g["kv_idx"].shape[-1]])
        for h in range(w.n_q_heads):
            rows.append((0, h, t * w.tile + int(rng.integers(w.tile))))
        say(f"[max {name}] tile {t} (tripped {tr}) matches the oracle")
    # and one random (head, row) of every tile
    heads = rng.integers(w.n_q_heads, size=w.n_tiles)
    offs = rng.integers(w.tile, size=w.n_tiles)
    rows += [(0, int(heads[t]), t * w.tile + int(offs[t])) for t in range(w.n_tiles)]
    rows = np.array(rows, np.int64)
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], g["kv_idx"], g["kv_cnt"],
                              pf.scale, rows=rows)
    r = torch.as_tensor(rows, device="cuda")
    O = pf.O[r[:, 0], r[:, 2], r[:, 1]].float().cpu().numpy().astype(np.float64)
    err = np.abs(O - O_ref)
    say(f"[max {name}] {len(rows)} rows, max|O - O_ref| = {err.max():.3e}")
    assert np.all(err <= out_tol(w, api.SA_BF16, O_ref))
