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

from parity import (assert_selection_equal, assert_summaries_equal, bits, check_structure,
                    out_tol, run_gpu, say)

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
    # query tiles of 64 rows inside key blocks of 128 (two tiles per diagonal block)
    "t64_blk128_planted": WL["prefill_128k_t64"].resized(seqlen=4096, k_max=6, k_min=6),
    "t64_blk128_d64_sinks_oam": WL["stem_32k"].resized(
        batch=2, seqlen=2560, n_q_heads=4, n_kv_heads=2, head_dim=64, block=128, q_tile=64,
        k_max=8, k_min=2, n_sink=3),
    "t64_blk128_quest_kvshared": WL["quest_64k"].resized(
        seqlen=2048, n_q_heads=8, n_kv_heads=2, block=128, q_tile=64, k_max=4, k_min=4,
        select_unit=wl.SELECT_PER_KV_HEAD),
    "f32_t64_blk128": WL["tiny_ref"].resized(seqlen=1024, n_q_heads=2, n_kv_heads=1,
                                             block=128, q_tile=64, k_max=2, k_min=2),
    "f32_t64_blk128_d128": WL["tiny_ref"].resized(seqlen=768, n_q_heads=2, n_kv_heads=2,
                                                  head_dim=128, block=128, q_tile=64, k_max=2,
                                                  k_min=2, score_mode=wl.KMINMAX,
                                                  output_aware=1),
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
    # a top list longer than the query rows' LDS area can sort as 64-bit keys (k 300, rho 2:
    # 600 ranked blocks; d 64): the selection keeps 64-bit sort keys (tiles of up to 639
    # free blocks) instead of the 32-bit ones
    "wide_sort_keys": WL["llama8b_32k"].resized(seqlen=64 * 640, n_q_heads=2, n_kv_heads=1,
                                                head_dim=64, k_max=300, k_min=300, q=0.3),
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
    # 64-row tiles inside 128-key blocks
    "t64_single_block": WL["prefill_128k_t64"].resized(seqlen=128, k_max=2, k_min=2),
    "t64_dense_limit": WL["prefill_128k_t64"].resized(seqlen=1024, n_q_heads=4, n_kv_heads=2,
                                                      k_max=64, k_min=64),
    "t64_q1_all_trip": WL["prefill_128k_t64"].resized(seqlen=2048, n_q_heads=4, n_kv_heads=1,
                                                      k_max=4, k_min=4, q=1.0),
    "t64_fixed_gate_odd_sinks": WL["prefill_128k_t64"].resized(
        seqlen=1536, n_q_heads=4, n_kv_heads=2, n_sink=3, k_max=4, k_min=2,
        gate_mode=wl.GATE_FIXED, tau_fixed=0.3),
    "tied_blocks_t64": WL["prefill_128k_t64"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2,
                                                      k_max=4, k_min=4),
    # all keys zero: every score is +0, sigma = 0 everywhere, ranking falls to the index
    "zero_keys_kmean_oam": WL["stem_32k"].resized(batch=1, seqlen=1536, n_q_heads=4,
                                                  n_kv_heads=2, k_max=4, k_min=2),
    "zero_keys_quest": WL["quest_64k"].resized(seqlen=1536, n_q_heads=4, n_kv_heads=2, k_max=4,
                                               k_min=4),
    # product output-aware score with all-zero value blocks: tile scores times 0 are -0 for
    # negative maxima and +0 otherwise; both sides compare and subtract the canonical +0
    "zero_value_blocks_oam": WL["stem_32k"].resized(batch=2, seqlen=2048, n_q_heads=4,
                                                    n_kv_heads=2, k_max=6, k_min=3, q=0.3),
    "zero_value_blocks_oam_t128": WL["stem_32k_t128"].resized(batch=1, seqlen=2048,
                                                              n_q_heads=4, n_kv_heads=2,
                                                              k_max=6, k_min=3, q=0.3),
    # threshold pruning of long rows (tiles with at least 16 times as many free blocks as
    # ranked keys): a prefilter pass, survivors above a safe threshold, exact scores for those
    # only.  Small k makes short sequences qualify.
    "prune_kmean": WL["llama8b_32k"].resized(seqlen=64 * 192, n_q_heads=2, n_kv_heads=1,
                                             k_max=2, k_min=2, q=0.3),
    "prune_kmean_d64_batch2": WL["llama8b_32k"].resized(batch=2, seqlen=64 * 160, n_q_heads=2,
                                                        n_kv_heads=1, head_dim=64, k_max=2,
                                                        k_min=2),
    "prune_oam_sinks_decay": WL["stem_32k"].resized(batch=1, seqlen=64 * 256, n_q_heads=2,
                                                    n_kv_heads=1, k_max=8, k_min=2),
    "prune_additive": WL["stem_additive_32k"].resized(batch=1, seqlen=64 * 256, n_q_heads=2,
                                                      n_kv_heads=1, k_max=4, k_min=2),
    "prune_t128": WL["llama8b_32k_t128"].resized(seqlen=64 * 256, n_q_heads=2, n_kv_heads=1,
                                                 k_max=2, k_min=2),
    "prune_t64_in_block128": WL["prefill_128k_t64"].resized(seqlen=128 * 128, n_q_heads=2,
                                                            n_kv_heads=1, k_max=2, k_min=2),
    "prune_block128_planted": WL["prefill_128k"].resized(seqlen=128 * 160, n_q_heads=2,
                                                         n_kv_heads=1, k_max=2, k_min=2),
    "prune_quest_near_ties": WL["quest_64k"].resized(seqlen=64 * 192, n_q_heads=2, n_kv_heads=1,
                                                     k_max=2, k_min=2),
    "tied_blocks_prune": WL["llama8b_32k"].resized(seqlen=64 * 192, n_q_heads=2, n_kv_heads=1,
                                                   k_max=2, k_min=2),
    "tied_rows_prune": WL["prefill_128k"].resized(seqlen=128 * 160, n_q_heads=2, n_kv_heads=1,
                                                  k_max=2, k_min=2, planted=False),
    "zero_value_blocks_prune": WL["stem_32k"].resized(batch=1, seqlen=64 * 256, n_q_heads=2,
                                                      n_kv_heads=1, k_max=6, k_min=2, q=0.3),
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
    if name.startswith("zero_keys"):
        inp["K"] = torch.zeros_like(inp["K"])
    if name.startswith("zero_value_blocks"):
        # every third key block's values are zero; the keys of the first two of each six
        # blocks are shifted down so that some tiles' maxima over them are negative
        v, k = inp["V"].clone(), inp["K"].clone()
        B = w.block
        for j in range(0, w.n_blocks, 3):
            v[:, j * B:(j + 1) * B] = 0
        for j in range(0, w.n_blocks, 6):
            k[:, j * B:(j + 2) * B] -= 6.0
        inp["V"], inp["K"] = v, k
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
    m = max(1, w.tile // w.block)  # diagonal blocks per tile
    t = np.arange(w.n_tiles)
    d0 = t * w.tile // w.block       # first diagonal block
    if name.endswith("dense_limit"):  # every causal block of every tile
        assert np.all(g["kv_cnt"] == d0 + m)
    if name == "q0_no_trips" or name == "gate_off":
        assert g["gate"].sum() == 0
    if name.endswith("q1_all_trip"):  # tau = the largest eligible sigma_bar: every one trips
        nfree = d0 - np.minimum(d0, w.n_sink)
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


@pytest.mark.parametrize("head_dim", [128, 64])
def test_per_head_lists_that_differ_between_heads(head_dim):
    """64-row tiles over 64-key blocks with a list per query head, where the lists of the two
    query heads of each kv head differ in every way tile by tile: identical, disjoint, nested,
    one of them empty, or random with a block after the tile and a sentinel before kv_cnt, in
    shuffled order.  Every row against the fp64 oracle on the same lists (rows of empty lists
    must be zero)."""
    w = WL["llama8b_32k"].resized(seqlen=64 * 40, n_q_heads=4, n_kv_heads=2, head_dim=head_dim)
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    n, W = w.n_blocks, 24
    rng = np.random.default_rng(5)
    idx = np.full((1, 4, n, W), -1, np.int32)
    cnt = np.zeros((1, 4, n), np.int32)

    def put(h, t, row, count=None):
        row = list(row)
        idx[0, h, t, :len(row)] = row
        cnt[0, h, t] = len(row) if count is None else count

    for t in range(n):
        causal = np.arange(t + 1)
        for pair in (0, 2):
            mode = (t + pair) % 6
            pick = rng.permutation(causal)[:min(t + 1, 12)]
            if mode == 0:  # identical
                a = b = pick
            elif mode == 1:  # disjoint
                a, b = causal[0::2], causal[1::2]
                a, b = rng.permutation(a)[:W], rng.permutation(b)[:W]
            elif mode == 2:  # nested
                a, b = pick, pick[:len(pick) // 2]
            elif mode == 3:  # the second head's list is empty
                a, b = pick, []
            elif mode == 4:  # the first head's list is empty
                a, b = [], rng.permutation(causal)[:W]
            else:  # a block after the tile first, then the list, then a sentinel
                extra = [t + 1] if t + 1 < n else []
                a = extra + list(pick)
                b = extra + list(rng.permutation(causal)[:5])
            put(pair, t, a)
            if mode == 5:
                put(pair + 1, t, b, count=min(W, len(b) + 2))
            else:
                put(pair + 1, t, b)
    p = api.problem(w)
    fws = torch.empty(max(api.forward_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    O = torch.empty(1, w.seqlen, 4, w.head_dim, dtype=torch.float32, device="cuda")
    api.forward(p, d["Q"], d["K"], d["V"], torch.as_tensor(idx).cuda(),
                torch.as_tensor(cnt).cuda(), W, scale, fws, O, api.SA_F32)
    torch.cuda.synchronize()
    cfg = oracle.make_cfg(w)
    with np.errstate(invalid="ignore", divide="ignore"):
        O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt, scale)
    got = O.cpu().numpy().astype(np.float64)
    tile_of_row = np.arange(w.seqlen) // w.tile
    empty = (cnt[0] == 0)[:, tile_of_row].T  # [N, Hq]: rows whose list is empty
    err = np.abs(got[0] - O_ref[0])[~empty].max()
    say(f"[per-head lists d={head_dim}] {int((~empty).sum())} rows, max|O - O_ref| = {err:.3e}; "
        f"{int(empty.sum())} rows of empty lists")
    assert err <= out_tol(w, api.SA_F32, O_ref[0][~empty])
    assert float(np.abs(got[0][empty]).max()) == 0.0


@pytest.mark.parametrize("head_dim", [128, 64])
def test_lists_that_differ_between_the_two_tiles_of_a_block(head_dim):
    """64-row tiles inside 128-key blocks: the two tiles of a block have lists of their own,
    which tile pair by tile pair are identical, disjoint, nested, one of them empty, or random
    with a block after the tile and a sentinel before kv_cnt, in shuffled order.  Every row
    against the fp64 oracle on the same lists (rows of empty lists must be zero)."""
    w = WL["prefill_128k_t64"].resized(seqlen=128 * 24, n_q_heads=2, n_kv_heads=1,
                                       head_dim=head_dim)
    assert w.tile == 64 and w.block == 128
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    nt, W = w.n_tiles, 20
    rng = np.random.default_rng(6)
    idx = np.full((1, 2, nt, W), -1, np.int32)
    cnt = np.zeros((1, 2, nt), np.int32)

    def put(h, t, row, count=None):
        row = list(row)
        idx[0, h, t, :len(row)] = row
        cnt[0, h, t] = len(row) if count is None else count

    for h in range(2):
        for blk in range(nt // 2):
            t0, t1 = 2 * blk, 2 * blk + 1
            causal = np.arange(blk + 1)  # the free blocks before the diagonal one, and it
            mode = (blk + h) % 6
            pick = rng.permutation(causal)[:min(blk + 1, 10)]
            extra = [blk + 1] if blk + 1 < nt // 2 else []
            if mode == 0:  # identical
                a = b = pick
            elif mode == 1:  # disjoint
                a, b = causal[0::2], causal[1::2]
            elif mode == 2:  # nested
                a, b = pick, pick[:len(pick) // 2]
            elif mode == 3:  # the second tile's list is empty
                a, b = pick, []
            elif mode == 4:  # the first tile's list is empty
                a, b = [], rng.permutation(causal)[:W]
            else:  # a block after the tiles first, then the list, then a sentinel
                a = extra + list(pick)
                b = extra + list(rng.permutation(causal)[:4])
            put(h, t0, rng.permutation(np.array(a, np.int64)) if len(a) else [])
            if mode == 5:
                put(h, t1, b, count=min(W, len(b) + 2))
            else:
                put(h, t1, rng.permutation(np.array(b, np.int64)) if len(b) else [])
    p = api.problem(w)
    fws = torch.empty(max(api.forward_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    O = torch.empty(1, w.seqlen, 2, w.head_dim, dtype=torch.float32, device="cuda")
    api.forward(p, d["Q"], d["K"], d["V"], torch.as_tensor(idx).cuda(),
                torch.as_tensor(cnt).cuda(), W, scale, fws, O, api.SA_F32)
    torch.cuda.synchronize()
    cfg = oracle.make_cfg(w)
    with np.errstate(invalid="ignore", divide="ignore"):
        O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt, scale)
    got = O.cpu().numpy().astype(np.float64)
    tile_of_row = np.arange(w.seqlen) // w.tile
    empty = (cnt[0] == 0)[:, tile_of_row].T  # [N, Hq]: rows whose list is empty
    err = np.abs(got[0] - O_ref[0])[~empty].max()
    say(f"[tile-pair lists d={head_dim}] {int((~empty).sum())} rows, max|O - O_ref| = "
        f"{err:.3e}; {int(empty.sum())} rows of empty lists")
    assert err <= out_tol(w, api.SA_F32, O_ref[0][~empty])
    assert float(np.abs(got[0][empty]).max()) == 0.0


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


@pytest.mark.parametrize("W", [200, 600])
def test_long_lists_of_64_row_tiles_in_128_key_blocks(W):
    """64-row tiles inside 128-key blocks with long lists: dense causal lists cut to W entries,
    ascending for one head and descending for the other, on both tiles of several blocks.
    W = 200 keeps both tiles' lists within the kernel's staging area, so a block's two tiles
    share one workgroup over the union of their lists; W = 600 does not, so each tile runs
    alone with its list consumed in segments.  Sampled rows against the fp64 oracle."""
    n = 600  # key blocks
    w = WL["prefill_128k_t64"].resized(seqlen=n * 128, n_q_heads=2, n_kv_heads=1)
    assert w.tile == 64 and w.block == 128
    nt = w.n_tiles
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    p = api.problem(w)
    fws = torch.empty(max(api.forward_workspace_bytes(p), 1), dtype=torch.uint8, device="cuda")
    cfg = oracle.make_cfg(w)
    scale = 1.0 / math.sqrt(w.head_dim)
    blocks = [n - 1, 420, 257, 100, 3]
    idx = np.full((1, 2, nt, W), -1, np.int32)
    cnt = np.zeros((1, 2, nt), np.int32)
    for h in range(2):
        for b in blocks:
            row = list(range(b + 1))
            if h == 1:
                row = row[::-1]
            row = row[:W]
            for t in (2 * b, 2 * b + 1):
                idx[0, h, t, :len(row)] = row
                cnt[0, h, t] = len(row)
    O = torch.empty(1, w.seqlen, 2, w.head_dim, dtype=torch.float32, device="cuda")
    api.forward(p, d["Q"], d["K"], d["V"], torch.as_tensor(idx).cuda(),
                torch.as_tensor(cnt).cuda(), W, scale, fws, O, api.SA_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = []
    for b in blocks:
        for t in (2 * b, 2 * b + 1):
            for h in range(2):
                for r in (0, w.tile - 1, int(rng.integers(w.tile))):
                    rows.append((0, h, t * w.tile + r))
    rows = np.array(rows, np.int64)
    O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt, scale, rows=rows)
    r = torch.as_tensor(rows, device="cuda")
    got = O[r[:, 0], r[:, 2], r[:, 1]].cpu().numpy().astype(np.float64)
    err = np.abs(got - O_ref).max()
    say(f"[t64 long lists W={W}] {len(rows)} rows, max|O - O_ref| = {err:.3e}")
    assert err <= out_tol(w, api.SA_F32, O_ref)
    # rows of tiles with empty lists are zero
    assert float(O[0, 5 * w.tile:6 * w.tile].abs().max()) == 0.0


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


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("case", ["non_uniform_norms", "zero_value_blocks"])
def test_oam_product_golden_on_gpu(case, dtype):
    """The hand-worked product output-aware examples (tests/golden/oam_product.json) through
    the C ABI: summaries, sigma, tau, gate and lists equal the golden values bit for bit."""
    import golden_inputs as gi
    g = gi.load("oam_product.json")
    c = next(x for x in g["cases"] if x["name"] == case)
    w = gi.oam_product_workload(g, dtype)
    inp = gi.oam_product_inputs(c, dtype)
    out = run_gpu(w, inp, out_dtype=api.SA_F32)
    np.testing.assert_array_equal(out["vn"][0, :, 0], np.float32(c["vnorm"]))
    want_sigma = np.array([gi.f32(x) for x in c["sigma"]], np.float32)
    np.testing.assert_array_equal(out["sigma"][0, 0].view(np.uint32), want_sigma.view(np.uint32))
    assert out["tau"][0].view(np.uint32) == gi.f32(c["tau"]).view(np.uint32)
    np.testing.assert_array_equal(out["gate"][0], c["gate"])
    np.testing.assert_array_equal(out["kv_idx"][0, 0], c["kv_idx"])
    np.testing.assert_array_equal(out["kv_cnt"][0, 0], c["kv_cnt"])
    compare_outputs(w, out, inp, api.SA_F32, None)


def _prepared_forward(w, d, pf, V, out_dtype=api.SA_F32):
    """Attention over pf's lists with another V: prepare_values, then forward_prepared."""
    O = torch.empty((w.batch, w.seqlen, w.n_q_heads, w.head_dim),
                    dtype=torch.float32 if out_dtype == api.SA_F32 else torch.bfloat16,
                    device="cuda")
    api.prepare_values(pf.p, V, pf.fws)
    api.forward_prepared(pf.p, d["Q"], d["K"], pf.fws, pf.kv_idx, pf.kv_cnt, pf.W, pf.scale, O,
                         out_dtype)
    torch.cuda.synchronize()
    return O


@pytest.mark.parametrize("name", ["llama8b_n32", "prefill_n32_planted", "stem_b2_t128"])
def test_value_magnitudes_beyond_fp16(name):
    """bf16 V far outside fp16's range (about 1e5 and 1e-6 in magnitude): P V runs on fp16
    matrix cores after a per-(batch, kv head) power-of-two scaling, so scaling V by 2^k scales
    every output by exactly 2^k (bit for bit), and V = c Z meets the bf16 bar on O / c against
    the fp64 oracle (attention is linear in V)."""
    w = SMALL[name]
    inp = wl.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    pf = api.Prefill(w, out_dtype=api.SA_F32)
    pf.run(d["Q"], d["K"], d["V"])
    torch.cuda.synchronize()
    base = pf.O.clone()
    for k in (17, -20):
        Vk = (d["V"].float() * 2.0 ** k).to(torch.bfloat16)  # exact: a power-of-two scaling
        Ok = _prepared_forward(w, d, pf, Vk)
        assert torch.equal(Ok, base * 2.0 ** k), f"2^{k}: not an exact scaling"
        # the combined call gives the same bits as the two halves
        O2 = torch.empty_like(Ok)
        api.forward(pf.p, d["Q"], d["K"], Vk, pf.kv_idx, pf.kv_cnt, pf.W, pf.scale, pf.fws, O2,
                    api.SA_F32)
        torch.cuda.synchronize()
        assert torch.equal(O2, Ok)
    rng = np.random.default_rng(3)
    rows = sample_rows(w, rng, max_rows=3000)
    cfg = oracle.make_cfg(w)
    kv_idx, kv_cnt = pf.kv_idx.cpu().numpy(), pf.kv_cnt.cpu().numpy()
    for c in (1.0e5, -1.0e-6):
        Z = torch.from_numpy(rng.standard_normal(tuple(inp["V"].shape)).astype(np.float32))
        Vc = (Z * c).to(torch.bfloat16)
        Oc = _prepared_forward(w, d, pf, Vc.cuda()).cpu().numpy()
        O_ref, _ = oracle.forward(cfg, inp["Q"], inp["K"], Vc, kv_idx, kv_cnt, pf.scale,
                                  rows=rows)
        got = Oc if rows is None else Oc[rows[:, 0], rows[:, 2], rows[:, 1]]
        err = np.abs(got.astype(np.float64) - O_ref).max() / abs(c)
        say(f"[{name}] V = {c:g} Z: max|O - O_ref| / |c| = {err:.3e}")
        assert np.isfinite(got).all() and err <= 2e-2


def test_calibrated_tau_over_several_sequences():
    """sparse_attn_calibrate_tau over per-sequence quantile thresholds equals the oracle's
    mean of the finite thresholds; with one sequence it is that sequence's tau."""
    w = WL["stem_additive_32k"].resized(batch=3, seqlen=2048, k_max=16, k_min=4)
    inp = wl.make_inputs(w)
    cfg = oracle.make_cfg(w)
    o_sel = oracle.select(cfg, inp["Q"], oracle.pool(cfg, inp["K"], inp["V"]))
    dev = {k: v.cuda() for k, v in inp.items()}
    tau = api.Prefill(w).calibrate_tau(dev["Q"], dev["K"], dev["V"])
    want = oracle.calibrated_tau(o_sel["tau"])
    assert np.float32(tau).view(np.uint32) == want.view(np.uint32)
    t = torch.tensor([0.25, -float("inf"), 0.5, 0.125], device="cuda")
    out = torch.empty(1, device="cuda")
    api.calibrate_tau(t, out)
    assert out.item() == oracle.calibrated_tau(t.cpu().numpy())
    api.calibrate_tau(torch.full((2,), -float("inf"), device="cuda"), out)
    assert out.item() == -float("inf")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_tiles_in_blocks_golden_on_gpu(dtype):
    """The hand-worked 64-row tiles inside 128-key blocks (tests/golden/tiles_in_blocks.json)
    through the C ABI: sigma, tau, gate and lists equal the golden values bit for bit."""
    import golden_inputs as gi
    g = gi.load("tiles_in_blocks.json")
    w = WL["tiny_ref"].resized(seqlen=1024, n_q_heads=1, n_kv_heads=1, head_dim=64,
                               block=g["block"], q_tile=g["tile"], k_max=g["k"], k_min=g["k"],
                               rho=g["rho"], q=g["q"], dtype=dtype)
    Q = np.zeros((1, 1024, 1, 64), np.float32)
    Q[0, :, 0, 0] = 1.0
    K = np.zeros((1, 1024, 1, 64), np.float32)
    for j in range(8):
        K[0, j * 128:(j + 1) * 128, 0, 0] = g["c"][j]
    V = np.random.default_rng(4).standard_normal((1, 1024, 1, 64)).astype(np.float32)
    tdt = torch.float32 if dtype == wl.F32 else torch.bfloat16
    inp = {k: torch.from_numpy(v).to(tdt) for k, v in (("Q", Q), ("K", K), ("V", V))}
    out = run_gpu(w, inp, out_dtype=api.SA_F32)
    want = np.array([gi.f32(x) for x in g["sigma"]], np.float32)
    np.testing.assert_array_equal(out["sigma"][0, 0].view(np.uint32), want.view(np.uint32))
    assert out["tau"][0] == np.float32(g["tau"])
    np.testing.assert_array_equal(out["gate"][0], g["gate"])
    np.testing.assert_array_equal(out["kv_idx"][0, 0], g["kv_idx"])
    np.testing.assert_array_equal(out["kv_cnt"][0, 0], g["kv_cnt"])
    compare_outputs(w, out, inp, api.SA_F32, None)


def test_pruning_over_several_survivor_rounds():
    """Tiles with more than 4096 free blocks, pruned, list their survivors in two rounds of
    4096 positions: 4160 blocks of 64 keys, one head pair, k = 2.  The whole structure of
    every tile, and the last tiles (two rounds), the middle ones (one round) and some early,
    unpruned ones, against oracle.select_tile bit for bit."""
    w = WL["llama8b_32k"].resized(seqlen=64 * 4160, n_q_heads=1, n_kv_heads=1, head_dim=64,
                                  k_max=2, k_min=2, q=0.3)
    inp = wl.make_inputs(w)
    say(f"[prune rounds] {w.n_blocks} blocks: GPU pipeline")
    g = run_gpu(w, inp, out_dtype=api.SA_F32)
    check_structure(w, g["kv_idx"], g["kv_cnt"], g["gate"], g["sigma"], g["sigma_bar"],
                    g["tau"])
    cfg = oracle.make_cfg(w)
    summ = oracle.pool(cfg, inp["K"], inp["V"])
    assert_summaries_equal(w, g, summ)
    n = w.n_tiles
    for t in (3, 40, 64, 2000, 4095, 4097, 4120, n - 2, n - 1):
        one = oracle.select_tile(cfg, inp["Q"], summ, 0, t)
        np.testing.assert_array_equal(bits(g["sigma"][0, :, t]), bits(one["sigma"]))
        tr = int(g["gate"][0, t])
        np.testing.assert_array_equal(g["kv_cnt"][0, :, t], one["cnts"][tr])
        np.testing.assert_array_equal(g["kv_idx"][0, :, t, :], one["lists"][tr])
    say("[prune rounds] sampled tiles equal")
