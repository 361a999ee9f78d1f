"""Inputs of the hand-worked golden examples under tests/golden/, built from their JSON.

Shared by the oracle pins (CPU) and the GPU parity tests, so that both run the same
constructed inputs.  Only input construction lives here: no step of the method.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

from block_sparse_causal_mean_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(x) -> np.float32:
    """A golden scalar: a number, or the hex bit pattern of an fp32 value."""
    if isinstance(x, str):
        return np.array([int(x, 16)], np.uint32).view(np.float32)[0]
    return np.float32(x)


def oam_product_workload(g: dict, dtype: int = wl.F32) -> wl.Workload:
    p = g["params"]
    return wl.Workload(
        name="oam_product_golden", batch=1, seqlen=512, n_q_heads=1, n_kv_heads=1, head_dim=64,
        block=64, dtype=dtype, score_mode=wl.KMEAN, output_aware=wl.OAM_PRODUCT,
        k_max=p["k"], k_min=p["k"], budget_kind=wl.BUDGET_CONST, n_sink=p["n_sink"],
        rho=p["rho"], q=p["q"], seed=0)


def oam_product_inputs(case: dict, dtype: int = wl.F32):
    """Q, K, V of one case of oam_product.json: keys c_j e0 and queries e0 (exact scores
    c_j), value rows u_j (rows 0..31 of block j) and w_j (rows 32..63) on coordinates 5..7."""
    N, d, blk = 512, 64, 64
    Q = np.zeros((1, N, 1, d), np.float32)
    Q[0, :, 0, 0] = 1.0
    K = np.zeros((1, N, 1, d), np.float32)
    V = np.zeros((1, N, 1, d), np.float32)
    for j in range(N // blk):
        K[0, j * blk:(j + 1) * blk, 0, 0] = case["c"][j]
        V[0, j * blk:j * blk + blk // 2, 0, 5:8] = case["u"][j]
        V[0, j * blk + blk // 2:(j + 1) * blk, 0, 5:8] = case["w"][j]
    dt = torch.float32 if dtype == wl.F32 else torch.bfloat16
    return {k: torch.from_numpy(v).to(dt) for k, v in (("Q", Q), ("K", K), ("V", V))}
