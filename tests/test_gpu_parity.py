"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same inputs.

Selections (summaries, kv_idx, kv_cnt, sigma, sigma_bar, gate, tau) must match bit for bit;
attention outputs within max-abs 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs, fp32 accumulation),
plus half a bf16 ulp of |O| when the output itself is stored in bf16.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

from parity import (assert_selection_equal, assert_summaries_equal, check_structure, out_tol,
                    run_gpu, say)

pytestmark = pytest.mark.gpu

WL = wl.WORKLOADS

# Small cases: the five recipes at sizes the oracle finishes in seconds (budgets scaled so
# that many tiles are eligible and some trip), plus shapes with ragged counts and d = 64.
SMALL = {
    "tiny_ref": WL["tiny_ref"],
    "llama8b_n32": WL["llama8b_32k"].resized(seqlen=2048, k_max=8, k_min=8),
    "prefill_n32_planted": WL["prefill_128k"].resized(seqlen=4096, k_max=6, k_min=6),
    "quest_n32": WL["quest_64k"].resized(seqlen=2048, k_max=6, k_min=6),
    "stem_b2_n32": WL["stem_32k"].resized(batch=2, seqlen=2048, k_max=16, k_min=4),
    "ragged_b3_n13_d64": WL["llama8b_32k"].resized(batch=3, seqlen=832, n_q_heads=6,
                                                    n_kv_heads=2, head_dim=64, k_max=3,
                                                    k_min=3, q=0.3),
    "d64_blk128_quest_oam": WL["quest_64k"].resized(seqlen=2560, n_q_heads=4, n_kv_heads=2,
                                                     head_dim=64, block=128, k_max=3, k_min=3,
                                                     output_aware=1, n_sink=1),
    "f32_d128_blk128": WL["tiny_ref"].resized(seqlen=2048, block=128, n_q_heads=4,
                                               n_kv_heads=2, head_dim=128, k_max=3, k_min=3,
                                               output_aware=1, score_mode=wl.KMINMAX),
    # the additive output-aware metric: bf16 (matrix-core prefilter path) and fp32 (VALU path)
    "stem_additive_b2_n32": WL["stem_additive_32k"].resized(batch=2, seqlen=2048, k_max=16,
                                                            k_min=4),
    "f32_additive_d64_quest": WL["tiny_ref"].resized(seqlen=2048, n_q_heads=4, n_kv_heads=2,
                                                      k_max=3, k_min=3, score_mode=wl.KMINMAX,
                                                      output_aware=wl.OAM_ADDITIVE,
                                                      oam_beta=0.3, v_logn_sigma=1.0),
    # one list per kv head, shared by its query heads: two heads per attention workgroup on
    # 64-key blocks with an even group (d = 128 and 64), one head per workgroup otherwise
    # (odd group, 128-key blocks, fp32)
    "llama8b_n32_kvshared": WL["llama8b_32k_kvshared"].resized(seqlen=2048, k_max=8, k_min=8),
    "stem_b2_n32_kvshared": WL["stem_32k_kvshared"].resized(batch=2, seqlen=2048, k_max=16,
                                                            k_min=4),
    "quest_d64_g2_kvshared": WL["quest_64k"].resized(seqlen=1280, n_q_heads=4, n_kv_heads=2,
                                                      head_dim=64, k_max=3, k_min=3,
                                                      select_unit=wl.SELECT_PER_KV_HEAD),
    "ragged_g3_d64_kvshared": WL["llama8b_32k_kvshared"].resized(
        batch=3, seqlen=832, n_q_heads=6, n_kv_heads=2, head_dim=64, k_max=3, k_min=3, q=0.3),
    "prefill_n32_kvshared": WL["prefill_128k_kvshared"].resized(seqlen=4096, k_max=6, k_min=6),
    "f32_kvshared": WL["tiny_ref"].resized(seqlen=1024, n_q_heads=4, n_kv_heads=2, k_max=3,
                                           k_min=3, select_unit=wl.SELECT_PER_KV_HEAD),
    # query tiles of 128 rows over blocks of 64 keys (two diagonal blocks per tile)
    "llama8b_n16_t128": WL["llama8b_32k_t128"].resized(seqlen=2048, k_max=6, k_min=6),
    "stem_b2_t128": WL["stem_32k_t128"].resized(batch=2, seqlen=2560, k_max=12, k_min=3,
                                                n_sink=3),
    "quest_d64_t128": WL["quest_64k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2,
                                              head_dim=64, k_max=3, k_min=3, q_tile=128,
                                              output_aware=1),
    "t128_kvshared": WL["llama8b_32k_t128"].resized(seqlen=2048, k_max=5, k_min=5,
                                                    select_unit=wl.SELECT_PER_KV_HEAD),
    "f32_t128": WL["tiny_ref"].resized(seqlen=1024, n_q_heads=2, n_kv_heads=1, k_max=3,
                                       k_min=3, q_tile=128),
    "f32_t128_d128": WL["tiny_ref"].resized(seqlen=768, n_q_heads=2, n_kv_heads=2,
                                            head_dim=128, k_max=2, k_min=2, q_tile=128,
                                            score_mode=wl.KMINMAX),
}

MAX_ORACLE_ROWS = 6000


def sample_rows(w, rng, max_rows=MAX_ORACLE_ROWS):
    """All rows when cheap, else every row of tiles 0, 1 and n-1 of head 0 plus random rows."""
    total = w.batch * w.seqlen * w.n_q_heads
    if total <= max_rows:
        return None
    T = w.tile
    fixed = []
    for t in (0, 1, w.n_tiles - 1):
        for i in range(t * T, (t + 1) * T):
            fixed.append((0, 0, i))
    k = max_rows - len(fixed)
    rnd = np.stack([rng.integers(0, w.batch, k), rng.integers(0, w.n_q_heads, k),
                    rng.integers(0, w.seqlen, k)], axis=1)
    return np.concatenate([np.array(fixed, np.int64), rnd.astype(np.int64)])


def compare_outputs(w, g, inp, out_dtype, rows, with_lse=False):
    cfg = oracle.make_cfg(w)
    O_ref, lse_ref = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], g["kv_idx"],
                                    g["kv_cnt"], g["scale"], rows=rows)
    if rows is None:
        O = g["O"]
        lse = g.get("lse")
    else:
        O = g["O"][rows[:, 0], rows[:, 2], rows[:, 1]]
        lse = g["lse"][rows[:, 0], rows[:, 1], rows[:, 2]] if with_lse else None
        lse_ref = lse_ref
    tol = out_tol(w, out_dtype, O_ref)
    err = np.abs(O.astype(np.float64) - O_ref)
    say(f"  max|O - O_ref| = {err.max():.3e}")
    assert np.all(err <= tol), f"max err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"
    if with_lse:
        lse_ref_arr = lse_ref if rows is not None else lse_ref.transpose(0, 2, 1)
        np.testing.assert_allclose(lse, lse_ref_arr, atol=1e-3 if w.dtype == wl.BF16 else 1e-5)


@pytest.mark.parametrize("name", list(SMALL))
def test_pipeline_parity_small(name):
    w = SMALL[name]
    inp = wl.make_inputs(w)
    cfg = oracle.make_cfg(w)
    say(f"[{name}] oracle pool/select")
    o_sum = oracle.pool(cfg, inp["K"], inp["V"])
    o_sel = oracle.select(cfg, inp["Q"], o_sum)
    out_dtype = api.SA_F32
    say(f"[{name}] GPU pipeline (score, select, forward) fp32 out")
    g = run_gpu(w, inp, out_dtype=out_dtype, with_lse=True)
    assert_summaries_equal(w, g, o_sum)
    assert_selection_equal(g, o_sel)
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"],
                    g["tau"])
    rows = sample_rows(w, np.random.default_rng(5))
    compare_outputs(w, g, inp, out_dtype, rows, with_lse=True)
    if w.dtype == wl.BF16:
        say(f"[{name}] GPU pipeline bf16 out")
        g2 = run_gpu(w, inp, out_dtype=api.SA_BF16)
        np.testing.assert_array_equal(g2["kv_idx"], g["kv_idx"])
        compare_outputs(w, g2, inp, api.SA_BF16, rows)


def test_trips_happen_in_small_cases():
    # The small cases exercise the gate: some tiles trip and expand.
    w = SMALL["llama8b_n32"]
    g = run_gpu(w, wl.make_inputs(w))
    assert g["gate"].sum() >= 1
    assert (g["kv_cnt"] > 1 + w.k_max).any()


EDGE = {
    "single_tile": WL["llama8b_32k"].resized(seqlen=64, k_max=2, k_min=2),
    "dense_limit": WL["llama8b_32k"].resized(seqlen=1024, n_q_heads=4, n_kv_heads=2, k_max=64,
                                             k_min=64),
    "q0_no_trips": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=4,
                                             k_min=4, q=0.0),
    "q1_all_trip": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=4,
                                             k_min=4, q=1.0),
    "rho1": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=4,
                                      k_min=4, rho=1.0, q=0.5),
    "rho_frac": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=3,
                                          k_min=3, rho=2.5, q=0.5),
    "gate_off": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=4,
                                          k_min=4, gate_mode=wl.GATE_OFF),
    "gate_fixed": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=1, k_max=4,
                                            k_min=4, gate_mode=wl.GATE_FIXED, tau_fixed=0.3),
    "sinks_exceed": WL["stem_32k"].resized(batch=1, seqlen=640, n_q_heads=4, n_kv_heads=2,
                                           n_sink=12, k_max=4, k_min=2),
    "k1": WL["quest_64k"].resized(seqlen=1280, n_q_heads=8, n_kv_heads=8, k_max=1, k_min=1),
    "tied_rows_kmean": WL["prefill_128k"].resized(seqlen=2048, n_q_heads=4, n_kv_heads=2,
                                                  k_max=4, k_min=4, planted=False),
    "tied_rows_quest": WL["quest_64k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2, k_max=4,
                                               k_min=4, near_tie_keys=False),
    "tied_blocks": WL["llama8b_32k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2, k_max=4,
                                             k_min=4),
    # 128-row tiles over 64-key blocks, and lists shared by a kv head's query heads
    "t128_single_tile": WL["llama8b_32k_t128"].resized(seqlen=128, k_max=2, k_min=2),
    "t128_dense_limit": WL["llama8b_32k_t128"].resized(seqlen=1024, n_q_heads=4, n_kv_heads=2,
                                                       k_max=64, k_min=64),
    "t128_q1_all_trip": WL["llama8b_32k_t128"].resized(seqlen=2048, n_q_heads=4, n_kv_heads=1,
                                                       k_max=4, k_min=4, q=1.0),
    "t128_fixed_gate_odd_sinks": WL["stem_32k_t128"].resized(
        batch=1, seqlen=1280, n_q_heads=4, n_kv_heads=2, n_sink=5, k_max=4, k_min=2,
        gate_mode=wl.GATE_FIXED, tau_fixed=0.3),
    "tied_blocks_t128": WL["llama8b_32k_t128"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2,
                                                       k_max=4, k_min=4),
    "kvshared_dense_limit": WL["llama8b_32k_kvshared"].resized(seqlen=1024, n_q_heads=4,
                                                               n_kv_heads=2, k_max=64, k_min=64),
    "tied_rows_kvshared": WL["prefill_128k_kvshared"].resized(seqlen=2048, n_q_heads=4,
                                                              n_kv_heads=2, k_max=4, k_min=4,
                                                              planted=False),
}


def _edge_inputs(name, w):
    """Inputs of an edge case: the recipe's, or a tie-heavy variant of it."""
    inp = wl.make_inputs(w)
    if name.startswith("tied_rows"):
        # every row of a query tile equal: every row ties for each block's maximum, so the
        # prefilter keeps all of them as candidates
        q = inp["Q"].clone()
        T = w.tile
        for t in range(w.n_tiles):
            q[:, t * T:(t + 1) * T] = q[:, t * T:t * T + 1]
        inp["Q"] = q
    if name.startswith("tied_blocks"):
        # every key block identical: all tile scores of a tile tie, ranking falls to the index
        k = inp["K"].clone()
        T = w.block
        for j in range(1, w.n_blocks):
            k[:, j * T:(j + 1) * T] = k[:, :T]
        inp["K"] = k
    return inp


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_cases(name):
    w = EDGE[name]
    inp = _edge_inputs(name, w)
    cfg = oracle.make_cfg(w)
    say(f"[{name}] oracle + GPU")
    o_sum = oracle.pool(cfg, inp["K"], inp["V"])
    o_sel = oracle.select(cfg, inp["Q"], o_sum)
    g = run_gpu(w, inp, out_dtype=api.SA_F32)
    assert_summaries_equal(w, g, o_sum)
    assert_selection_equal(g, o_sel)
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"],
                    g["tau"])
    compare_outputs(w, g, inp, api.SA_F32, sample_rows(w, np.random.default_rng(1)))
    m = w.tile // w.block  # diagonal blocks per tile
    t = np.arange(w.n_tiles)
    if name.endswith("dense_limit"):  # every causal block of every tile
        assert np.all(g["kv_cnt"] == m * (t + 1))
    if name == "q0_no_trips" or name == "gate_off":
        assert g["gate"].sum() == 0
    if name.endswith("q1_all_trip"):  # tau = the largest eligible sigma_bar: every one trips
        nfree = m * t - np.minimum(m * t, w.n_sink)
        assert g["gate"].sum() == int((nfree > w.k_max).sum()) > 0


def test_forward_any_block_order_and_skipped_entries():
    """Order invariance of the online softmax (ART page, section 2.4); entries after the tile,
    and a sentinel that cuts the list short, are honoured.  Every variant must meet the parity
    bar against the oracle on the original lists."""
    w = WL["stem_32k"].resized(batch=1, seqlen=1024, n_q_heads=4, n_kv_heads=2, k_max=4,
                               k_min=2)
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w, out_dtype=api.SA_F32)
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    idx = pf.kv_idx.clone()
    cnt = pf.kv_cnt.clone()
    cfg = oracle.make_cfg(w)
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx.cpu().numpy(),
                              cnt.cpu().numpy(), pf.scale)
    base = pf.O.clone()

    def check(O, label):
        # Each order meets the bf16 bar against the oracle; between orders P is rounded to
        # fp16 against different running maxima, so they agree to a few fp16 ulps of |V|.
        err = np.abs(O.cpu().numpy().astype(np.float64) - O_ref).max()
        say(f"  {label}: max|O - O_ref| = {err:.3e}")
        assert err <= 2e-2
        assert (O - base).abs().max().item() <= 1e-2

    check(base, "ascending")
    rev = idx.clone()
    for b, h, t in np.ndindex(*idx.shape[:3]):
        c = int(cnt[b, h, t])
        rev[b, h, t, :c] = idx[b, h, t, :c].flip(0)
    pf.kv_idx.copy_(rev)
    pf.forward(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    check(pf.O, "reversed")
    # a wider list with a block after the tile first, then the list, then a sentinel before
    # kv_cnt is reached
    n, W = w.n_blocks, pf.W
    W2 = W + 3
    wide = torch.full((1, 4, n, W2), -1, dtype=torch.int32, device="cuda")
    cnt2 = torch.zeros_like(cnt)
    for h in range(4):
        for t in range(n):
            c = int(cnt[0, h, t])
            row = idx[0, h, t, :c].tolist()
            if t + 1 < n:
                row = [t + 1] + row  # after the tile: skipped
            wide[0, h, t, :len(row)] = torch.tensor(row, dtype=torch.int32)
            cnt2[0, h, t] = len(row) + 2  # count runs past the sentinel
    O2 = torch.empty_like(pf.O)
    api.forward(pf.p, d["Q"], d["K"], d["V"], wide, cnt2, W2, pf.scale, pf.fws, O2, api.SA_F32)
    torch.cuda.synchronize()
    check(O2, "skipped entries")


def test_runs_are_deterministic():
    w = SMALL["stem_b2_n32"]
    inp = wl.make_inputs(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for k in ("kA", "vn", "kv_idx", "kv_cnt", "sigma", "sigma_bar", "gate", "tau", "O"):
        np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("name", ["prefill_128k", "llama8b_32k"])
def test_forward_long_lists_in_segments(name):
    """Lists with more usable entries than the kernel stages in LDS at once (512) are consumed
    in segments, with the online softmax carried across them (ART page, section 2.4).  Dense
    causal lists of up to 1100 blocks, in three orders: ascending (diagonal last), descending
    (diagonal first), and with blocks after the tile interleaved (skipped, so segment
    boundaries fall elsewhere).  Sampled rows against the fp64 oracle."""
    base = WL[name]
    n = 1100
    w = base.resized(seqlen=n * base.block, n_q_heads=2, n_kv_heads=1)
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    p = api.problem(w)
    fws = torch.empty(max(api.forward_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    cfg = oracle.make_cfg(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    tiles = [n - 1, 1000, 700, 520, 300]
    rng = np.random.default_rng(11)
    for order in ("ascending", "descending", "with_skipped"):
        W = 2 * n
        idx = np.full((1, 2, n, W), -1, np.int32)
        cnt = np.zeros((1, 2, n), np.int32)
        for h in range(2):
            for t in tiles:
                row = list(range(t + 1))
                if order == "descending":
                    row = row[::-1]
                elif order == "with_skipped":
                    # a block after the tile (skipped) before every third entry
                    out = []
                    for i, j in enumerate(row):
                        if i % 3 == 0:
                            out.append(min(n - 1, t + 1 + (i % 7)) if t + 1 < n else j)
                        out.append(j)
                    row = [j for j in out]
                    if t + 1 >= n:  # the last tile has no block after it: plain order
                        row = list(range(t + 1))
                idx[0, h, t, :len(row)] = row
                cnt[0, h, t] = len(row)
        O = torch.empty(1, w.seqlen, 2, w.head_dim, dtype=torch.float32, device="cuda")
        api.forward(p, d["Q"], d["K"], d["V"], torch.as_tensor(idx).cuda(),
                    torch.as_tensor(cnt).cuda(), W, scale, fws, O, api.SA_F32)
        torch.cuda.synchronize()
        rows = []
        for t in tiles:
            for h in range(2):
                for r in (0, w.block - 1, int(rng.integers(w.block))):
                    rows.append((0, h, t * w.block + r))
        rows = np.array(rows, np.int64)
        O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt, scale, rows=rows)
        r = torch.as_tensor(rows, device="cuda")
        got = O[r[:, 0], r[:, 2], r[:, 1]].cpu().numpy().astype(np.float64)
        err = np.abs(got - O_ref).max()
        say(f"[long lists {name} {order}] {len(rows)} rows, max|O - O_ref| = {err:.3e}")
        assert err <= out_tol(w, api.SA_F32, O_ref)
        # rows of tiles with empty lists are zero
        assert float(O[0, 5 * w.block:6 * w.block].abs().max()) == 0.0


def test_fixed_gate_with_calibrated_tau_reproduces_the_quantile_gate():
    """A fixed threshold calibrated on an input (the per-call quantile's tau) gives that
    input the same gate, lists and counts as the quantile gate; the fixed-gate run also
    matches the oracle with that threshold bit for bit."""
    w = WL["stem_additive_32k"].resized(batch=1, seqlen=2048, k_max=16, k_min=4)
    inp = wl.make_inputs(w)
    say("[calibrated tau] quantile run + calibration")
    q_run = run_gpu(w, inp, out_dtype=api.SA_F32)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    tau = api.Prefill(w).calibrate_tau(dev["Q"], dev["K"], dev["V"])
    assert tau == float(q_run["tau"][0])
    wf = w.resized(gate_mode=wl.GATE_FIXED, tau_fixed=tau)
    f_run = run_gpu(wf, inp, out_dtype=api.SA_F32)
    for key in ("gate", "kv_idx", "kv_cnt", "sigma", "sigma_bar"):
        np.testing.assert_array_equal(f_run[key], q_run[key], err_msg=key)
    cfg = oracle.make_cfg(wf)
    o_sel = oracle.select(cfg, inp["Q"], oracle.pool(cfg, inp["K"], inp["V"]))
    assert_selection_equal(f_run, o_sel)
