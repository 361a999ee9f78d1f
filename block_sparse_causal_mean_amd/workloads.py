"""Seeded synthetic workloads for block-sparse causal prefill attention.

This module holds the five workload shapes and their input recipes, and nothing of the
method's arithmetic: it only draws Q/K/V.  Both the HIP path and the CPU oracle consume what
it returns, so neither side generates its own inputs.

The shapes follow long-context prefill workloads of Llama/Qwen/Mistral-class models at
32K-128K tokens (the Stem page's LongBench/RULER runs up to 128K; the uncertainty-gated
selection page's 32K-128K runs).  Those datasets and weights are not available, so these
seeded distributions stand in for them:

* ``tiny_ref``       1 x 1024, 1 q / 1 kv head, d=64, fp32; Q,K,V iid N(0,1).
* ``llama8b_32k``    1 x 32768, 32 q / 8 kv heads, d=128, bf16; Q,K ~ N(0,1);
                     V ~ N(0,1) scaled per token by LogNormal(0, 0.5).
* ``prefill_128k``   1 x 131072, 32 q / 8 kv heads, d=128, bf16; as above plus planted
                     vertical (anchor keys) and slash (offset-periodic) structure, the two
                     patterns the vertical-slash prefill page describes.
* ``quest_64k``      1 x 65536, 64 q / 8 kv heads, d=128, bf16; Q,V ~ N(0,1);
                     K = per-(batch, kv head) base + 0.05 N(0,1): near-tied block bounds.
* ``stem_32k``       4 x 32768, 32 q / 8 kv heads, d=128, bf16; Q,K ~ N(0,1);
                     V ~ N(0,1) scaled per token by LogNormal(0, 1.0).

Every tensor is generated in float32 by ``numpy.random.default_rng(seed)`` (PCG64, stable
across platforms) and then rounded to the workload dtype (round-to-nearest-even), so the
values both sides see are exactly representable in that dtype.  The "per token" value scale
is one scalar per (batch, position, kv head).
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import numpy as np
import torch

# Score backbones and budget kinds.  The integers match the C ABI's enumerations.
KMEAN = 0
KMINMAX = 1
BUDGET_CONST = 0
BUDGET_LINEAR_DECAY = 1
GATE_QUANTILE = 0
GATE_FIXED = 1
GATE_OFF = 2
OAM_OFF = 0
OAM_PRODUCT = 1
OAM_ADDITIVE = 2
SELECT_PER_Q_HEAD = 0   # one block list per query head (the pages' per-head selection)
SELECT_PER_KV_HEAD = 1  # one list per kv head, shared by its query heads
F32 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block: int
    dtype: int              # F32 or BF16 for Q, K, V
    score_mode: int         # KMEAN or KMINMAX
    output_aware: int       # OAM_OFF, OAM_PRODUCT (score x mean value-row L2 norm) or
                            # OAM_ADDITIVE (score / sqrt(d) + oam_beta * max(0, ln vnorm^2))
    k_max: int
    k_min: int
    budget_kind: int
    n_sink: int
    rho: float
    q: float
    seed: int
    v_logn_sigma: float = 0.0   # per-token LogNormal(0, sigma) value scale; 0 = none
    planted: bool = False       # vertical + slash structure
    near_tie_keys: bool = False # K = base + 0.05 noise
    gate_mode: int = GATE_QUANTILE
    tau_fixed: float = 0.0
    oam_beta: float = 0.0       # beta of the additive output-aware form
    kind: str = "prefill"       # "prefill", or "decode" (one query token per sequence)
    art_tau: float = 0.0        # decode: run-time termination thresholds and patience
    art_phi: float = 0.0
    art_patience: int = 0
    select_unit: int = SELECT_PER_Q_HEAD
    q_tile: int = 0         # query tile rows; 0 = block (every workload of the pages)

    @property
    def n_units(self) -> int:
        """Selection units per sequence: query heads, or kv heads for shared lists."""
        return self.n_kv_heads if self.select_unit == SELECT_PER_KV_HEAD else self.n_q_heads

    @property
    def tile(self) -> int:
        return self.q_tile or self.block

    @property
    def n_tiles(self) -> int:
        return self.seqlen // self.tile

    @property
    def n_blocks(self) -> int:
        return self.seqlen // self.block

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    def resized(self, **kw) -> "Workload":
        """Same recipe and method parameters at another size (for small parity cases)."""
        return dataclasses.replace(self, **kw)

    def index_width(self) -> int:
        """Entries per sentinel-padded block list: forced blocks (the tile's diagonal blocks
        and the sinks) plus the expanded budget."""
        n_diag = max(1, self.tile // self.block)
        return min(self.n_blocks,
                   n_diag + self.n_sink + int(math.floor(self.rho * self.k_max)))


WORKLOADS: Dict[str, Workload] = {
    "tiny_ref": Workload(
        name="tiny_ref", batch=1, seqlen=1024, n_q_heads=1, n_kv_heads=1, head_dim=64,
        block=64, dtype=F32, score_mode=KMEAN, output_aware=0, k_max=4, k_min=4,
        budget_kind=BUDGET_CONST, n_sink=0, rho=2.0, q=0.25, seed=1000),
    "llama8b_32k": Workload(
        name="llama8b_32k", batch=1, seqlen=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
        block=64, dtype=BF16, score_mode=KMEAN, output_aware=0, k_max=32, k_min=32,
        budget_kind=BUDGET_CONST, n_sink=0, rho=2.0, q=0.1, seed=1001, v_logn_sigma=0.5),
    "prefill_128k": Workload(
        name="prefill_128k", batch=1, seqlen=131072, n_q_heads=32, n_kv_heads=8, head_dim=128,
        block=128, dtype=BF16, score_mode=KMEAN, output_aware=0, k_max=64, k_min=64,
        budget_kind=BUDGET_CONST, n_sink=0, rho=2.0, q=0.1, seed=1002, v_logn_sigma=0.5,
        planted=True),
    "quest_64k": Workload(
        name="quest_64k", batch=1, seqlen=65536, n_q_heads=64, n_kv_heads=8, head_dim=128,
        block=64, dtype=BF16, score_mode=KMINMAX, output_aware=0, k_max=48, k_min=48,
        budget_kind=BUDGET_CONST, n_sink=0, rho=2.0, q=0.2, seed=1003, near_tie_keys=True),
    "stem_32k": Workload(
        name="stem_32k", batch=4, seqlen=32768, n_q_heads=32, n_kv_heads=8, head_dim=128,
        block=64, dtype=BF16, score_mode=KMEAN, output_aware=1, k_max=64, k_min=8,
        budget_kind=BUDGET_LINEAR_DECAY, n_sink=2, rho=2.0, q=0.1, seed=1004,
        v_logn_sigma=1.0),
    # The Stem page's own output-aware form (Metodologia B), additive on the logit scale,
    # on stem_32k's shapes and data.  There, block scores / sqrt(d) spread by about 0.06
    # across blocks and ln(vnorm^2) by about 0.33, so beta = 0.2 gives the two terms a
    # similar say in the ranking.
    "stem_additive_32k": Workload(
        name="stem_additive_32k", batch=4, seqlen=32768, n_q_heads=32, n_kv_heads=8,
        head_dim=128, block=64, dtype=BF16, score_mode=KMEAN, output_aware=2, k_max=64,
        k_min=8, budget_kind=BUDGET_LINEAR_DECAY, n_sink=2, rho=2.0, q=0.1, seed=1005,
        v_logn_sigma=1.0, oam_beta=0.2),
}

# One list per kv head, shared by its query heads (a GQA variant the pages do not describe):
# the same shapes, method parameters and seeds (so the same inputs) as the per-head workloads.
# On 64-key blocks the attention kernel then runs two query heads per workgroup.
for _base in ("llama8b_32k", "prefill_128k", "stem_32k"):
    WORKLOADS[_base + "_kvshared"] = dataclasses.replace(
        WORKLOADS[_base], name=_base + "_kvshared", select_unit=SELECT_PER_KV_HEAD)

# Query tiles of 128 rows over key blocks of 64 (tile != block, not on the pages: a tile's two
# diagonal blocks are both forced).  Same inputs as the per-head workloads; each K/V step then
# feeds the four waves of a 128-row tile.
for _base in ("llama8b_32k", "stem_32k"):
    WORKLOADS[_base + "_t128"] = dataclasses.replace(
        WORKLOADS[_base], name=_base + "_t128", q_tile=128)

# The 128K recipe at one million tokens (the VSPrefill page's range reaches 1M): 8192 blocks
# of 128 keys, the same budget, so each tile keeps under 2% of its causal blocks.
WORKLOADS["prefill_1m"] = dataclasses.replace(
    WORKLOADS["prefill_128k"], name="prefill_1m", seqlen=1 << 20)

# Query tiles of 64 rows inside key blocks of 128 (the other direction of tile != block: two
# tiles share a diagonal block, forced in both).  The 128K inputs, selected per 64-row tile.
WORKLOADS["prefill_128k_t64"] = dataclasses.replace(
    WORKLOADS["prefill_128k"], name="prefill_128k_t64", q_tile=64)

# Decode with run-time termination (ART page): one new token per sequence and head over a
# 16K-token cache, 64 sequences (one workgroup per sequence and kv head: 512, two per CU; the
# sequential traversal needs the second workgroup to keep HBM busy).  The selection fields are
# unused.  tau = phi = 5e-3 and patience 4 stop these inputs' heads after about a third of
# the cache (the pages give no values).
DECODE_WORKLOADS: Dict[str, Workload] = {
    "art_decode_16k": Workload(
        name="art_decode_16k", batch=64, seqlen=16384, n_q_heads=32, n_kv_heads=8,
        head_dim=128, block=64, dtype=BF16, score_mode=KMEAN, output_aware=0, k_max=1, k_min=1,
        budget_kind=BUDGET_CONST, n_sink=0, rho=1.0, q=0.0, seed=1006, v_logn_sigma=0.5,
        kind="decode", art_tau=5e-3, art_phi=5e-3, art_patience=4),
}
WORKLOADS.update(DECODE_WORKLOADS)

# Order used by reports: the small reference case first, the 128K prefill (the headline) third.
WORKLOAD_ORDER = ["tiny_ref", "llama8b_32k", "prefill_128k", "quest_64k", "stem_32k"]
HEADLINE = "prefill_128k"


def _to_dtype(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def _unit(v: np.ndarray) -> np.ndarray:
    return v / np.linalg.norm(v)


def make_inputs(w: Workload, seed: Optional[int] = None,
                extras: Optional[dict] = None) -> Dict[str, torch.Tensor]:
    """Draw Q [B,N,Hq,d], K [B,N,Hkv,d], V [B,N,Hkv,d] (contiguous BSHD, CPU tensors).

    The tensors hold values exactly representable in the workload dtype.  If `extras` is a
    dict, planted workloads also leave their anchor positions there ("anchors": int64
    [B, Hkv, 64]).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, N, Hq, Hkv, d = w.batch, w.seqlen, w.n_q_heads, w.n_kv_heads, w.head_dim
    G = Hq // Hkv
    dt = w.torch_dtype

    q = rng.standard_normal((B, N, Hq, d), dtype=np.float32)
    if w.near_tie_keys:
        base = rng.standard_normal((B, 1, Hkv, d), dtype=np.float32)
        k = base + np.float32(0.05) * rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    else:
        k = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    if w.v_logn_sigma > 0:
        scale = rng.lognormal(0.0, w.v_logn_sigma, size=(B, N, Hkv, 1)).astype(np.float32)
        v *= scale

    anchor_pos = np.zeros((B, Hkv, min(64, N)), np.int64)
    if w.planted:
        # Vertical stripes: per (batch, kv head) a unit direction u and 64 distinct anchor
        # positions; anchors' keys and every query of the group get +4u, which adds +16 to
        # the raw anchor logit.  Slash: two directions orthonormal to u carry a phase of
        # period 256 on both queries and keys, adding 16 cos(2 pi (i - j) / 256) to q_i.k_j.
        pos = np.arange(N, dtype=np.float64)
        theta = 2.0 * math.pi * pos / 256.0
        for b in range(B):
            for g in range(Hkv):
                u = _unit(rng.standard_normal(d))
                e1 = rng.standard_normal(d)
                e1 = _unit(e1 - (e1 @ u) * u)
                e2 = rng.standard_normal(d)
                e2 = e2 - (e2 @ u) * u - (e2 @ e1) * e1
                e2 = _unit(e2)
                anchors = rng.choice(N, size=min(64, N), replace=False)
                anchor_pos[b, g] = anchors
                k[b, anchors, g, :] += (4.0 * u).astype(np.float32)
                slash = (4.0 * (np.cos(theta)[:, None] * e1[None, :]
                                + np.sin(theta)[:, None] * e2[None, :])).astype(np.float32)
                k[b, :, g, :] += slash
                for r in range(G):
                    h = g * G + r
                    q[b, :, h, :] += (4.0 * u).astype(np.float32)[None, :] + slash

    if extras is not None and w.planted:
        extras["anchors"] = anchor_pos
    return {"Q": _to_dtype(q, dt), "K": _to_dtype(k, dt), "V": _to_dtype(v, dt)}


def make_decode_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Decode inputs: Q [B, Hq, d] (the new tokens), K, V [B, N, Hkv, d] (the cache), CPU
    tensors in the workload dtype.  Q, K ~ N(0, 1); V ~ N(0, 1) times a per-token
    LogNormal(0, v_logn_sigma) scale.  Drawn one sequence at a time (the caches are large)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    B, N, Hq, Hkv, d = w.batch, w.seqlen, w.n_q_heads, w.n_kv_heads, w.head_dim
    dt = w.torch_dtype
    q = rng.standard_normal((B, Hq, d), dtype=np.float32)
    K = torch.empty((B, N, Hkv, d), dtype=dt)
    V = torch.empty((B, N, Hkv, d), dtype=dt)
    for b in range(B):
        K[b] = _to_dtype(rng.standard_normal((N, Hkv, d), dtype=np.float32), dt)
        v = rng.standard_normal((N, Hkv, d), dtype=np.float32)
        if w.v_logn_sigma > 0:
            v *= rng.lognormal(0.0, w.v_logn_sigma, size=(N, Hkv, 1)).astype(np.float32)
        V[b] = _to_dtype(v, dt)
    return {"Q": _to_dtype(q, dt), "K": K, "V": V}


SLASH_PERIOD = 256  # tokens: the planted slash pattern's period


def vs_index(w: Workload, n_vertical: int, n_slash: int, anchors: Optional[np.ndarray] = None,
             seed: int = 0):
    """A stand-in for the VSPrefill page's trained indexer (unavailable here): seeded
    vertical-slash indices for the vertical-slash attention path, int32 [B, Hq, n_vertical]
    key blocks and [B, Hq, n_slash] block offsets, each ascending, distinct, -1 padded.

    With the planted workload's anchor positions (make_inputs' extras): a head's vertical
    blocks are the blocks holding its kv group's anchors (the smallest n_vertical of them), and
    its slash offsets are 0 and 1 (the local window) followed by multiples of the planted
    slash period in blocks.  Without: n_vertical distinct blocks drawn per head, and the local
    window 0 .. n_slash - 1.
    """
    B, Hq, n, G = w.batch, w.n_q_heads, w.n_blocks, w.n_q_heads // w.n_kv_heads
    vert = np.full((B, Hq, max(n_vertical, 1)), -1, np.int32)[..., :n_vertical]
    slash = np.full((B, Hq, max(n_slash, 1)), -1, np.int32)[..., :n_slash]
    rng = np.random.default_rng(seed)
    for b in range(B):
        for h in range(Hq):
            if anchors is not None:
                blocks = np.unique(anchors[b, h // G] // w.block)[:n_vertical]
            else:
                blocks = np.sort(rng.choice(n, size=min(n_vertical, n), replace=False))
            vert[b, h, :len(blocks)] = blocks
            if anchors is not None and SLASH_PERIOD % w.block == 0:
                p = SLASH_PERIOD // w.block
                offs = [0, 1] + [p * i for i in range(1, n) if p * i > 1]
            else:
                offs = list(range(n))
            offs = sorted(set(o for o in offs if o < n))[:n_slash]
            slash[b, h, :len(offs)] = offs
    return np.ascontiguousarray(vert), np.ascontiguousarray(slash)


def tensor_digest(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's bytes (records exactly which inputs a result was measured on)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()
