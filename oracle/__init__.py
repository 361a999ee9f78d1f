"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE: only the tests, the package smoke check and the benchmark's CPU-baseline
leg import this module.  It imports nothing from the GPU package; inputs arrive as CPU tensors
or numpy arrays from the shared seeded generators.

Each function here only marshals arguments; all arithmetic is in oracle.c, which documents
the step of the method each part follows.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class OracleCfg(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("score_mode", ctypes.c_int32),
        ("output_aware", ctypes.c_int32), ("k_max", ctypes.c_int32), ("k_min", ctypes.c_int32),
        ("budget_kind", ctypes.c_int32), ("n_sink", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
        ("tau_fixed", ctypes.c_float), ("oam_beta", ctypes.c_float), ("rho", ctypes.c_double),
        ("q", ctypes.c_double), ("width", ctypes.c_int32), ("select_unit", ctypes.c_int32),
        ("tile", ctypes.c_int32), ("pad3_", ctypes.c_int32),
    ]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"oracle library not built: {_LIB_PATH} (run oracle/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    if lib.oracle_cpu_ok() != 1:
        raise RuntimeError("the oracle is built with FMA instructions and this CPU lacks them")
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(OracleCfg)
    lib.oracle_pool.argtypes = [cfgp, P, P, P, P, P]
    lib.oracle_select.argtypes = [cfgp, P, P, P, P, P, P, P, P, P, P]
    lib.oracle_select_tile.argtypes = [cfgp, P, P, P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
    lib.oracle_tile_scores.argtypes = [cfgp, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    lib.oracle_row_score.argtypes = [cfgp, P, P, P, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_int]
    lib.oracle_row_score.restype = ctypes.c_float
    lib.oracle_forward.argtypes = [cfgp, P, P, P, P, P, ctypes.c_int, ctypes.c_float,
                                   ctypes.c_int64, P, P, P]
    lib.oracle_budget.argtypes = [cfgp, ctypes.c_int]
    lib.oracle_n_tiles.argtypes = [cfgp]
    lib.oracle_diag_end.argtypes = [cfgp, ctypes.c_int]
    lib.oracle_vs_lists.argtypes = [cfgp, P, ctypes.c_int, P, ctypes.c_int, P, P, ctypes.c_int]
    lib.oracle_decode_art.argtypes = [cfgp, P, P, P, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_double, ctypes.c_int, P, P, P, P]
    lib.oracle_calibrated_tau.argtypes = [P, ctypes.c_int]
    lib.oracle_calibrated_tau.restype = ctypes.c_float
    _lib = lib
    return lib


def make_cfg(w, **over) -> OracleCfg:
    """Oracle problem description from any object with the workload's attribute names."""
    get = lambda k: over.get(k, getattr(w, k))
    n, blk = get("seqlen") // get("block"), get("block")
    T = int(over.get("tile", getattr(w, "tile", blk)))
    rho, k_max, n_sink = float(get("rho")), int(get("k_max")), int(get("n_sink"))
    n_diag = max(1, T // blk)  # diagonal blocks per tile
    width = over.get("width", min(n, n_diag + n_sink + int(math.floor(rho * k_max))))
    return OracleCfg(
        batch=get("batch"), seqlen=get("seqlen"), n_q_heads=get("n_q_heads"),
        n_kv_heads=get("n_kv_heads"), head_dim=get("head_dim"), block=get("block"),
        in_dtype=get("dtype"), score_mode=get("score_mode"), output_aware=get("output_aware"),
        k_max=k_max, k_min=get("k_min"), budget_kind=get("budget_kind"), n_sink=n_sink,
        gate_mode=get("gate_mode"), tau_fixed=float(get("tau_fixed")),
        oam_beta=float(over.get("oam_beta", getattr(w, "oam_beta", 0.0))), rho=rho,
        q=float(get("q")), width=width,
        select_unit=int(over.get("select_unit", getattr(w, "select_unit", 0))), tile=T)


def n_tiles(cfg: OracleCfg) -> int:
    """Query tiles per sequence: N / T."""
    return cfg.seqlen // (cfg.tile or cfg.block)


def units(cfg: OracleCfg) -> int:
    """Selection units per batch element: query heads, or kv heads for shared lists."""
    return cfg.n_kv_heads if cfg.select_unit else cfg.n_q_heads


def _arr(x, cfg: OracleCfg) -> np.ndarray:
    """Input tensor as the raw array oracle.c reads: float32, or bfloat16 bit patterns."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                if cfg.in_dtype != 1:
                    raise ValueError("bf16 tensor given for a float32 problem")
                return x.view(torch.int16).numpy().view(np.uint16)
            if cfg.in_dtype != 0:
                raise ValueError("bf16 problem needs bf16 tensors")
            return x.to(torch.float32).numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if cfg.in_dtype == 1:
        if x.dtype != np.uint16:
            raise ValueError("bf16 problem needs uint16 bit patterns")
        return x
    return np.ascontiguousarray(x, dtype=np.float32)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(cfg: OracleCfg):
    if cfg.k_min < 1 or cfg.k_min > cfg.k_max:
        raise ValueError("need 1 <= k_min <= k_max")
    if cfg.seqlen % cfg.block or cfg.n_q_heads % cfg.n_kv_heads:
        raise ValueError("seqlen % block and n_q_heads % n_kv_heads must be 0")
    T = cfg.tile or cfg.block
    if cfg.seqlen % T or (T % cfg.block and cfg.block % T):
        raise ValueError("seqlen % tile must be 0, and tile a multiple or divisor of block")


def pool(cfg: OracleCfg, K, V=None) -> dict:
    """Block summaries: kA (kmean or kmin), kB (kmax or None), vn (or None)."""
    lib = _load()
    _check(cfg)
    n = cfg.seqlen // cfg.block
    shape = (cfg.batch, n, cfg.n_kv_heads, cfg.head_dim)
    kA = np.zeros(shape, np.float32)
    kB = np.zeros(shape, np.float32) if cfg.score_mode == 1 else None
    vn = np.zeros(shape[:3], np.float32) if cfg.output_aware else None
    Ka, Va = _arr(K, cfg), _arr(V, cfg) if cfg.output_aware else None
    if lib.oracle_pool(ctypes.byref(cfg), _p(Ka), _p(Va), _p(kA), _p(kB), _p(vn)) != 0:
        raise RuntimeError("oracle_pool failed")
    return {"kA": kA, "kB": kB, "vn": vn}


def select(cfg: OracleCfg, Q, summ: dict) -> dict:
    """Whole selection: kv_idx [B,U,n,W], kv_cnt, sigma [B,U,n], sigma_bar [B,n], gate, tau
    (U = units(cfg))."""
    lib = _load()
    _check(cfg)
    B, Hq, n, W = cfg.batch, units(cfg), n_tiles(cfg), cfg.width
    out = {
        "kv_idx": np.zeros((B, Hq, n, W), np.int32), "kv_cnt": np.zeros((B, Hq, n), np.int32),
        "sigma": np.zeros((B, Hq, n), np.float32), "sigma_bar": np.zeros((B, n), np.float32),
        "gate": np.zeros((B, n), np.uint8), "tau": np.zeros((B,), np.float32),
    }
    Qa = _arr(Q, cfg)
    rc = lib.oracle_select(ctypes.byref(cfg), _p(Qa), _p(summ["kA"]), _p(summ["kB"]),
                           _p(summ["vn"]), _p(out["kv_idx"]), _p(out["kv_cnt"]),
                           _p(out["sigma"]), _p(out["sigma_bar"]), _p(out["gate"]),
                           _p(out["tau"]))
    if rc != 0:
        raise RuntimeError("oracle_select failed")
    return out


def select_tile(cfg: OracleCfg, Q, summ: dict, b: int, t: int) -> dict:
    """One tile: sigma per unit, sigma_bar, eligibility, lists if untripped [0] / tripped [1]."""
    lib = _load()
    _check(cfg)
    Hq, W = units(cfg), cfg.width
    sig = np.zeros((Hq,), np.float32)
    sbar = np.zeros((1,), np.float32)
    elig = np.zeros((1,), np.int32)
    lists = np.zeros((2, Hq, W), np.int32)
    cnts = np.zeros((2, Hq), np.int32)
    Qa = _arr(Q, cfg)
    rc = lib.oracle_select_tile(ctypes.byref(cfg), _p(Qa), _p(summ["kA"]), _p(summ["kB"]),
                                _p(summ["vn"]), b, t, _p(sig), _p(sbar), _p(elig), _p(lists),
                                _p(cnts))
    if rc != 0:
        raise RuntimeError("oracle_select_tile failed")
    return {"sigma": sig, "sigma_bar": sbar[0], "eligible": bool(elig[0]), "lists": lists,
            "cnts": cnts}


def diag_end(cfg: OracleCfg, t: int) -> int:
    """One past tile t's last causal block (its diagonal blocks end there)."""
    return int(_load().oracle_diag_end(ctypes.byref(cfg), t))


def tile_scores(cfg: OracleCfg, Q, summ: dict, b: int, h: int, t: int) -> np.ndarray:
    """Scores of tile t's causal blocks (NaN for its forced ones), for selection unit h."""
    lib = _load()
    S = np.zeros((lib.oracle_diag_end(ctypes.byref(cfg), t),), np.float32)
    Qa = _arr(Q, cfg)
    lib.oracle_tile_scores(ctypes.byref(cfg), _p(Qa), _p(summ["kA"]), _p(summ["kB"]),
                           _p(summ["vn"]), b, h, t, _p(S))
    return S


def row_score(cfg: OracleCfg, Q, summ: dict, b: int, pos: int, h: int, j: int) -> np.float32:
    lib = _load()
    Qa = _arr(Q, cfg)
    return np.float32(lib.oracle_row_score(ctypes.byref(cfg), _p(Qa), _p(summ["kA"]),
                                           _p(summ["kB"]), b, pos, h, j))


def forward(cfg: OracleCfg, Q, K, V, kv_idx, kv_cnt, softmax_scale: float, rows=None):
    """fp64 attention over the listed blocks.

    rows: None for every row (O is [B,N,Hq,d]) or an int64 array [R,3] of (b, h, pos)
    (O is [R,d]).  Returns (O, lse) as float64.
    """
    lib = _load()
    _check(cfg)
    B, N, Hq, d = cfg.batch, cfg.seqlen, cfg.n_q_heads, cfg.head_dim
    idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
    cnt = np.ascontiguousarray(kv_cnt, dtype=np.int32)
    W = idx.shape[-1]
    if rows is None:
        R = B * N * Hq
        r_arr = None
    else:
        r_arr = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        R = r_arr.shape[0]
    O = np.zeros((R, d), np.float64)
    lse = np.zeros((R,), np.float64)
    rc = lib.oracle_forward(ctypes.byref(cfg), _p(_arr(Q, cfg)), _p(_arr(K, cfg)),
                            _p(_arr(V, cfg)), _p(idx), _p(cnt), W, float(softmax_scale), R,
                            _p(r_arr), _p(O), _p(lse))
    if rc != 0:
        raise RuntimeError("oracle_forward failed")
    if rows is None:
        return O.reshape(B, N, Hq, d), lse.reshape(B, N, Hq)
    return O, lse


def vs_lists(cfg: OracleCfg, vert, slash):
    """Per-tile block lists of a vertical-slash index (oracle.c, oracle_vs_lists): vert
    [B, Hq, NV] key blocks and slash [B, Hq, NS] block offsets, each ending at its first
    negative entry.  Returns (kv_idx [B, Hq, n, W], kv_cnt [B, Hq, n]) with W = NV + NS + 1."""
    lib = _load()
    _check(cfg)
    B, Hq, n = cfg.batch, cfg.n_q_heads, cfg.seqlen // cfg.block
    if (cfg.tile or cfg.block) != cfg.block:
        raise ValueError("vertical-slash lists are defined for tile = block")
    v = np.ascontiguousarray(vert, dtype=np.int32).reshape(B, Hq, -1)
    s = np.ascontiguousarray(slash, dtype=np.int32).reshape(B, Hq, -1)
    NV, NS = v.shape[-1], s.shape[-1]
    W = NV + NS + 1
    idx = np.zeros((B, Hq, n, W), np.int32)
    cnt = np.zeros((B, Hq, n), np.int32)
    rc = lib.oracle_vs_lists(ctypes.byref(cfg), _p(v), NV, _p(s), NS, _p(idx), _p(cnt), W)
    if rc != 0:
        raise RuntimeError(f"oracle_vs_lists failed ({rc})")
    return idx, cnt


def decode_art(cfg: OracleCfg, Q, K, V, softmax_scale: float, probe: int, tau: float,
               phi: float, patience: int, keep_partials: bool = True) -> dict:
    """Decode attention with run-time termination (oracle.c, oracle_decode_art), fp64.
    Q [B, Hq, d] (one token per sequence and head), K, V [B, N, Hkv, d].  Returns dscale,
    ddir [B, Hq, n] (the probe's norm and direction changes per step of the traversal order),
    stop [B, Hq] (blocks processed under the rule) and, if keep_partials, Opart
    [B, Hq, n, d] (the normalised partial output after each step)."""
    lib = _load()
    B, Hq, n, d = cfg.batch, cfg.n_q_heads, cfg.seqlen // cfg.block, cfg.head_dim
    Qa = _arr(Q, cfg)
    if Qa.size != B * Hq * d:
        raise ValueError("Q must hold B * Hq * d elements")
    dsc = np.zeros((B, Hq, n), np.float64)
    ddr = np.zeros((B, Hq, n), np.float64)
    Op = np.zeros((B, Hq, n, d), np.float64) if keep_partials else None
    stop = np.zeros((B, Hq), np.int32)
    rc = lib.oracle_decode_art(ctypes.byref(cfg), _p(Qa), _p(_arr(K, cfg)), _p(_arr(V, cfg)),
                               float(softmax_scale), int(probe), float(tau), float(phi),
                               int(patience), _p(dsc), _p(ddr), _p(Op), _p(stop))
    if rc != 0:
        raise RuntimeError(f"oracle_decode_art failed ({rc})")
    return {"dscale": dsc, "ddir": ddr, "stop": stop, "Opart": Op}


def art_stop(dscale, ddir, tau: float, phi: float, patience: int):
    """The stopping rule applied to given per-step metrics (the same rule oracle.c applies):
    blocks processed per (b, h)."""
    B, Hq, n = dscale.shape
    out = np.full((B, Hq), n, np.int32)
    if patience <= 0:
        return out
    stable = (dscale < tau) & (ddir < phi)
    stable[..., 0] = False
    for b in range(B):
        for h in range(Hq):
            run = 0
            for k in range(1, n):
                run = run + 1 if stable[b, h, k] else 0
                if run >= patience:
                    out[b, h] = k + 1
                    break
    return out


def threads() -> int:
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def budget(cfg: OracleCfg, t: int) -> int:
    return int(_load().oracle_budget(ctypes.byref(cfg), t))


def calibrated_tau(tau) -> np.float32:
    """Fixed-gate threshold from per-sequence thresholds: the mean of the finite ones."""
    t = np.ascontiguousarray(tau, dtype=np.float32)
    return np.float32(_load().oracle_calibrated_tau(_p(t), int(t.size)))
