"""GPU parity of decode attention with run-time termination (sparse_attn_decode_art).

The stop decision is an integer taken from floating-point probe metrics.  The kernel takes
it in fp32, the oracle in fp64, so a metric within rounding of a threshold may fall on either
side.  The check therefore accepts any stop between the oracle's stop with slightly
loosened thresholds (the earliest an fp32 evaluation can stop) and its stop with slightly
tightened ones (the latest), and then requires the output to be the oracle's partial output
over exactly the blocks the kernel processed (the bf16-input bar, 2e-2 max-abs).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

from parity import say

pytestmark = pytest.mark.gpu

BASE = wl.WORKLOADS["art_decode_16k"]
PROBE = 16
# fp32 evaluation of the metrics: relative error a few ulps of the probe's norm, well below
# these bands for probe norms <= ~10
BAND_ABS, BAND_REL = 2e-5, 1e-4
TOL = 2e-2


def _run(w, inp, tau, phi, patience, out_dtype=api.SA_F32):
    p = api.problem(w)
    d = {k: v.cuda() for k, v in inp.items()}
    odt = torch.float32 if out_dtype == api.SA_F32 else torch.bfloat16
    O = torch.full((w.batch, w.n_q_heads, w.head_dim), float("nan"), dtype=odt, device="cuda")
    done = torch.full((w.batch, w.n_q_heads), -7, dtype=torch.int32, device="cuda")
    api.decode_art(p, d["Q"], d["K"], d["V"], 1.0 / math.sqrt(w.head_dim), tau, phi, patience,
                   O, out_dtype, done)
    torch.cuda.synchronize()
    return O.float().cpu().numpy(), done.cpu().numpy()


def _check(w, inp, tau, phi, patience, tag, out_dtype=api.SA_F32):
    cfg = oracle.make_cfg(w)
    say(f"[{tag}] oracle + GPU")
    r = oracle.decode_art(cfg, inp["Q"], inp["K"], inp["V"], 1.0 / math.sqrt(w.head_dim), PROBE,
                          tau, phi, patience)
    O, done = _run(w, inp, tau, phi, patience, out_dtype)
    n = w.seqlen // w.block
    lo = oracle.art_stop(r["dscale"], r["ddir"], tau * (1 + BAND_REL) + BAND_ABS,
                         phi * (1 + BAND_REL) + BAND_ABS, patience)
    hi = oracle.art_stop(r["dscale"], r["ddir"], max(tau * (1 - BAND_REL) - BAND_ABS, 0.0),
                         max(phi * (1 - BAND_REL) - BAND_ABS, 0.0), patience)
    assert ((done >= 1) & (done <= n)).all(), tag
    assert ((lo <= done) & (done <= hi)).all(), f"{tag}: stops outside the band"
    B, Hq = done.shape
    ref = r["Opart"][np.arange(B)[:, None], np.arange(Hq)[None, :], done - 1]
    tol = TOL + (np.abs(ref) * 2.0 ** -8 if out_dtype == api.SA_BF16 else 0.0)
    err = np.abs(O - ref)
    assert (err <= tol).all(), f"{tag}: max err {err.max():.3e}"
    return r, done


@pytest.mark.parametrize("name,w", [
    ("g4_d128", BASE.resized(batch=2, seqlen=2048, n_q_heads=8, n_kv_heads=2)),
    ("g1_d64", BASE.resized(batch=3, seqlen=1536, n_q_heads=2, n_kv_heads=2, head_dim=64)),
    ("g2_d128", BASE.resized(batch=1, seqlen=4096, n_q_heads=4, n_kv_heads=2)),
])
@pytest.mark.parametrize("tau,phi,patience", [(5e-3, 5e-3, 4), (2e-2, 1e-2, 2), (1e-3, 1e-3, 8)])
def test_art_stops_within_band_and_outputs_match(name, w, tau, phi, patience):
    inp = wl.make_decode_inputs(w)
    r, done = _check(w, inp, tau, phi, patience, f"{name} tau={tau} phi={phi} p={patience}")
    say(f"  stops: min {done.min()} median {np.median(done)} max {done.max()} of "
        f"{w.seqlen // w.block}")


def test_art_never_stopping_is_full_decode_attention():
    w = BASE.resized(batch=2, seqlen=1024, n_q_heads=8, n_kv_heads=2)
    inp = wl.make_decode_inputs(w)
    r, done = _check(w, inp, 1.0, 1.0, 0, "patience 0", out_dtype=api.SA_BF16)
    assert (done == w.seqlen // w.block).all()


def test_art_constant_values_stop_after_patience():
    w = BASE.resized(batch=2, seqlen=2048, n_q_heads=4, n_kv_heads=1)
    inp = wl.make_decode_inputs(w)
    inp["V"] = torch.full_like(inp["V"], 0.75)
    for p in (1, 3, 6):
        _, done = _check(w, inp, 1e-4, 1e-4, p, f"constant V p={p}")
        assert (done == p + 1).all()


def test_art_single_block_cache():
    w = BASE.resized(batch=2, seqlen=64, n_q_heads=4, n_kv_heads=2)
    inp = wl.make_decode_inputs(w)
    _, done = _check(w, inp, 1.0, 1.0, 1, "one block")
    assert (done == 1).all()


@pytest.mark.timeout(600)
def test_art_full_size_sampled_sequences():
    """The benchmark's configuration (64 sequences x 16K tokens, its thresholds) on the GPU;
    four sequences checked against the oracle (all their heads)."""
    w = BASE
    say("[art full] generating inputs")
    inp = wl.make_decode_inputs(w)
    O, done = _run(w, inp, w.art_tau, w.art_phi, w.art_patience, api.SA_BF16)
    for b in (0, 17, 40, 63):
        wb = w.resized(batch=1)
        sub = {k: v[b:b + 1] for k, v in inp.items()}
        cfg = oracle.make_cfg(wb)
        r = oracle.decode_art(cfg, sub["Q"], sub["K"], sub["V"], 1.0 / math.sqrt(w.head_dim),
                              PROBE, w.art_tau, w.art_phi, w.art_patience)
        lo = oracle.art_stop(r["dscale"], r["ddir"], w.art_tau * (1 + BAND_REL) + BAND_ABS,
                             w.art_phi * (1 + BAND_REL) + BAND_ABS, w.art_patience)
        hi = oracle.art_stop(r["dscale"], r["ddir"], w.art_tau * (1 - BAND_REL) - BAND_ABS,
                             w.art_phi * (1 - BAND_REL) - BAND_ABS, w.art_patience)
        db = done[b:b + 1]
        assert ((lo <= db) & (db <= hi)).all(), b
        ref = r["Opart"][0, np.arange(w.n_q_heads), db[0] - 1]
        err = np.abs(O[b] - ref)
        assert (err <= TOL + np.abs(ref) * 2.0 ** -8).all(), f"seq {b}: {err.max():.3e}"
    say(f"[art full] stops: mean {done.mean():.1f} of {w.seqlen // w.block} blocks")
