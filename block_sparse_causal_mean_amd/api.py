"""Python binding of libsparse_attn.so (the C ABI in include/sparse_attn.h).

Argument marshalling only: torch tensors supply device memory and the current HIP stream;
every step of the method runs in the library's HIP kernels.  The library must have been
built (``python -m block_sparse_causal_mean_amd.build`` or ``__graft_entry__.build()``);
there is no fallback, so a missing or unloadable library raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

from . import workloads as wl

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID, SA_ERR_UNSUPPORTED, SA_ERR_HIP = 0, -1, -2, -3
SA_F32, SA_BF16 = 0, 1
SA_KMEAN, SA_KMINMAX = 0, 1
SA_K_CONST, SA_K_LINEAR_DECAY = 0, 1
SA_GATE_QUANTILE, SA_GATE_FIXED, SA_GATE_OFF = 0, 1, 2
SA_OAM_OFF, SA_OAM_PRODUCT, SA_OAM_ADDITIVE = 0, 1, 2
SA_SELECT_PER_Q_HEAD, SA_SELECT_PER_KV_HEAD = 0, 1

# Every function the header declares, checked by the tests against the built library.
EXPORTS = ("sparse_attn_summary_bytes", "sparse_attn_select_workspace_bytes",
           "sparse_attn_index_width", "sparse_attn_score", "sparse_attn_select",
           "sparse_attn_forward_workspace_bytes", "sparse_attn_forward",
           "sparse_attn_prepare_values", "sparse_attn_forward_prepared",
           "sparse_attn_calibrate_tau", "sparse_attn_forward_vs", "sparse_attn_decode_art",
           "sparse_attn_select_noalloc", "sparse_attn_last_error")


class Problem(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in (
        "batch", "seqlen", "n_q_heads", "n_kv_heads", "head_dim", "block", "tile", "dtype",
        "score_mode", "output_aware")] + [("oam_beta", ctypes.c_float),
                                          ("select_unit", ctypes.c_int32)]


class Budget(ctypes.Structure):
    _fields_ = [("k_max", ctypes.c_int32), ("k_min", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("gate_mode", ctypes.c_int32),
                ("tau_fixed", ctypes.c_float), ("rho", ctypes.c_double), ("q", ctypes.c_double)]


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"status {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Loads the HIP library (raises if it is missing: there is no other code path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP extension first")
    lib = ctypes.CDLL(LIB_PATH)
    P, PP, PB = ctypes.c_void_p, ctypes.POINTER(Problem), ctypes.POINTER(Budget)
    lib.sparse_attn_summary_bytes.argtypes = [PP]
    lib.sparse_attn_summary_bytes.restype = ctypes.c_size_t
    lib.sparse_attn_select_workspace_bytes.argtypes = [PP, PB]
    lib.sparse_attn_select_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse_attn_index_width.argtypes = [PP, PB]
    lib.sparse_attn_index_width.restype = ctypes.c_int32
    lib.sparse_attn_score.argtypes = [PP, P, P, P, P]
    lib.sparse_attn_select.argtypes = [PP, PB, P, P, P, ctypes.c_size_t, P, P, P, P, P, P, P]
    lib.sparse_attn_forward_workspace_bytes.argtypes = [PP]
    lib.sparse_attn_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.sparse_attn_forward.argtypes = [PP, P, P, P, P, P, ctypes.c_int32, ctypes.c_float, P,
                                        ctypes.c_size_t, P, ctypes.c_int32, P, P]
    lib.sparse_attn_prepare_values.argtypes = [PP, P, P, ctypes.c_size_t, P]
    lib.sparse_attn_forward_prepared.argtypes = [PP, P, P, P, ctypes.c_size_t, P, P,
                                                 ctypes.c_int32, ctypes.c_float, P,
                                                 ctypes.c_int32, P, P]
    lib.sparse_attn_calibrate_tau.argtypes = [P, ctypes.c_int32, P, P]
    lib.sparse_attn_forward_vs.argtypes = [PP, P, P, P, P, ctypes.c_int32, P, ctypes.c_int32,
                                           ctypes.c_float, P, ctypes.c_size_t, P,
                                           ctypes.c_int32, P, P]
    lib.sparse_attn_decode_art.argtypes = [PP, P, P, P, ctypes.c_float, ctypes.c_float,
                                           ctypes.c_float, ctypes.c_int32, P, ctypes.c_int32,
                                           P, P]
    lib.sparse_attn_select_noalloc.argtypes = [PP, PB, P, P, P, P, P, P, P, P, P]
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    for f in ("sparse_attn_score", "sparse_attn_select", "sparse_attn_forward",
              "sparse_attn_prepare_values", "sparse_attn_forward_prepared",
              "sparse_attn_calibrate_tau", "sparse_attn_forward_vs", "sparse_attn_decode_art",
              "sparse_attn_select_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load().sparse_attn_last_error().decode()


def _check(rc: int):
    if rc != SA_OK:
        raise SparseAttnError(rc, last_error())


def problem(w: wl.Workload) -> Problem:
    return Problem(batch=w.batch, seqlen=w.seqlen, n_q_heads=w.n_q_heads,
                   n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, block=w.block, tile=w.tile,
                   dtype=w.dtype, score_mode=w.score_mode, output_aware=w.output_aware,
                   oam_beta=getattr(w, "oam_beta", 0.0),
                   select_unit=getattr(w, "select_unit", SA_SELECT_PER_Q_HEAD))


def units(p: Problem) -> int:
    """Selection units per sequence (lists per batch element and tile): Hq, or Hkv."""
    return p.n_kv_heads if p.select_unit == SA_SELECT_PER_KV_HEAD else p.n_q_heads


def budget(w: wl.Workload) -> Budget:
    return Budget(k_max=w.k_max, k_min=w.k_min, kind=w.budget_kind, n_sink=w.n_sink,
                  gate_mode=w.gate_mode, tau_fixed=w.tau_fixed, rho=w.rho, q=w.q)


def summary_bytes(p: Problem) -> int:
    n = load().sparse_attn_summary_bytes(ctypes.byref(p))
    if n == 0:
        _check(SA_ERR_INVALID)
    return n


def select_workspace_bytes(p: Problem, b: Budget) -> int:
    n = load().sparse_attn_select_workspace_bytes(ctypes.byref(p), ctypes.byref(b))
    if n == 0:
        _check(SA_ERR_INVALID)
    return n


def index_width(p: Problem, b: Budget) -> int:
    w = load().sparse_attn_index_width(ctypes.byref(p), ctypes.byref(b))
    _check(min(w, 0))
    return w


NOALLOC_SCRATCH_BYTES = 64 << 20  # the library's own selection workspace (per GPU)


def select_noalloc(p: Problem, b: Budget, Q: torch.Tensor, summaries: torch.Tensor,
                   kv_idx: torch.Tensor, kv_cnt: torch.Tensor, sigma=None, sigma_bar=None,
                   gate=None, tau=None, stream=None):
    """sparse_attn_select_noalloc: the selection with the library's own workspace."""
    n = p.seqlen // p.tile
    bhn = p.batch * units(p) * n
    W = index_width(p, b)
    _check(load().sparse_attn_select_noalloc(
        ctypes.byref(p), ctypes.byref(b),
        _ptr(Q, "Q", p.batch * p.seqlen * p.n_q_heads * p.head_dim * _elt(p)),
        _ptr(summaries, "summaries", summary_bytes(p)), _ptr(kv_idx, "kv_idx", bhn * W * 4),
        _ptr(kv_cnt, "kv_cnt", bhn * 4), _ptr(sigma, "sigma", bhn * 4),
        _ptr(sigma_bar, "sigma_bar", p.batch * n * 4), _ptr(gate, "gate", p.batch * n),
        _ptr(tau, "tau", p.batch * 4), _stream(stream)))


def forward_workspace_bytes(p: Problem) -> int:
    """Scratch bytes sparse_attn_forward needs (0 for fp32 problems)."""
    return load().sparse_attn_forward_workspace_bytes(ctypes.byref(p))


def _ptr(t: Optional[torch.Tensor], name: str, nbytes: Optional[int] = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _elt(p: Problem) -> int:
    return 4 if p.dtype == SA_F32 else 2


def score(p: Problem, K: torch.Tensor, V: Optional[torch.Tensor], summaries: torch.Tensor,
          stream=None):
    kv = p.batch * p.seqlen * p.n_kv_heads * p.head_dim * _elt(p)
    _check(load().sparse_attn_score(ctypes.byref(p), _ptr(K, "K", kv), _ptr(V, "V", kv),
                                    _ptr(summaries, "summaries", summary_bytes(p)),
                                    _stream(stream)))


def select(p: Problem, b: Budget, Q: torch.Tensor, summaries: torch.Tensor, ws: torch.Tensor,
           kv_idx: torch.Tensor, kv_cnt: torch.Tensor, sigma=None, sigma_bar=None, gate=None,
           tau=None, stream=None):
    n = p.seqlen // p.tile  # query tiles
    bhn = p.batch * units(p) * n
    W = index_width(p, b)
    _check(load().sparse_attn_select(
        ctypes.byref(p), ctypes.byref(b),
        _ptr(Q, "Q", p.batch * p.seqlen * p.n_q_heads * p.head_dim * _elt(p)),
        _ptr(summaries, "summaries", summary_bytes(p)), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _ptr(kv_idx, "kv_idx", bhn * W * 4),
        _ptr(kv_cnt, "kv_cnt", bhn * 4), _ptr(sigma, "sigma", bhn * 4),
        _ptr(sigma_bar, "sigma_bar", p.batch * n * 4), _ptr(gate, "gate", p.batch * n),
        _ptr(tau, "tau", p.batch * 4), _stream(stream)))


def forward(p: Problem, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
            kv_idx: torch.Tensor, kv_cnt: torch.Tensor, W: int, softmax_scale: float,
            ws: Optional[torch.Tensor], O: torch.Tensor, out_dtype: int,
            lse: Optional[torch.Tensor] = None, stream=None):
    n = p.seqlen // p.tile  # query tiles
    q_bytes = p.batch * p.seqlen * p.n_q_heads * p.head_dim
    kv = p.batch * p.seqlen * p.n_kv_heads * p.head_dim * _elt(p)
    need = forward_workspace_bytes(p)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().sparse_attn_forward(
        ctypes.byref(p), _ptr(Q, "Q", q_bytes * _elt(p)), _ptr(K, "K", kv), _ptr(V, "V", kv),
        _ptr(kv_idx, "kv_idx", p.batch * units(p) * n * W * 4),
        _ptr(kv_cnt, "kv_cnt", p.batch * units(p) * n * 4), W, softmax_scale,
        _ptr(ws, "ws", need), ws_bytes,
        _ptr(O, "O", q_bytes * (4 if out_dtype == SA_F32 else 2)), out_dtype,
        _ptr(lse, "lse", p.batch * p.n_q_heads * p.seqlen * 4), _stream(stream)))


def prepare_values(p: Problem, V: torch.Tensor, ws: torch.Tensor, stream=None):
    """sparse_attn_prepare_values: V (bf16) into the forward workspace."""
    kv = p.batch * p.seqlen * p.n_kv_heads * p.head_dim * _elt(p)
    need = forward_workspace_bytes(p)
    _check(load().sparse_attn_prepare_values(
        ctypes.byref(p), _ptr(V, "V", kv), _ptr(ws, "ws", need),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def forward_prepared(p: Problem, Q: torch.Tensor, K: torch.Tensor, ws: torch.Tensor,
                     kv_idx: torch.Tensor, kv_cnt: torch.Tensor, W: int, softmax_scale: float,
                     O: torch.Tensor, out_dtype: int, lse: Optional[torch.Tensor] = None,
                     stream=None):
    """sparse_attn_forward_prepared: attention with V from prepare_values' workspace."""
    n = p.seqlen // p.tile
    q_bytes = p.batch * p.seqlen * p.n_q_heads * p.head_dim
    kv = p.batch * p.seqlen * p.n_kv_heads * p.head_dim * _elt(p)
    need = forward_workspace_bytes(p)
    _check(load().sparse_attn_forward_prepared(
        ctypes.byref(p), _ptr(Q, "Q", q_bytes * _elt(p)), _ptr(K, "K", kv),
        _ptr(ws, "ws", need), 0 if ws is None else ws.numel() * ws.element_size(),
        _ptr(kv_idx, "kv_idx", p.batch * units(p) * n * W * 4),
        _ptr(kv_cnt, "kv_cnt", p.batch * units(p) * n * 4), W, softmax_scale,
        _ptr(O, "O", q_bytes * (4 if out_dtype == SA_F32 else 2)), out_dtype,
        _ptr(lse, "lse", p.batch * p.n_q_heads * p.seqlen * 4), _stream(stream)))


def calibrate_tau(tau: torch.Tensor, tau_out: torch.Tensor, stream=None):
    """sparse_attn_calibrate_tau: tau_out[0] = mean of the finite entries of tau (fp32 [B])."""
    if tau.dtype != torch.float32 or tau_out.dtype != torch.float32:
        raise ValueError("tau and tau_out must be float32")
    _check(load().sparse_attn_calibrate_tau(_ptr(tau, "tau"), tau.numel(),
                                            _ptr(tau_out, "tau_out", 4), _stream(stream)))


def forward_vs(p: Problem, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
               vertical: torch.Tensor, slash: torch.Tensor, softmax_scale: float,
               ws: torch.Tensor, O: torch.Tensor, out_dtype: int,
               lse: Optional[torch.Tensor] = None, stream=None):
    """Sparse attention over a vertical-slash index (sparse_attn_forward_vs): vertical int32
    [B, Hq, NV] key blocks and slash int32 [B, Hq, NS] block offsets, ascending, distinct,
    ending at the first negative entry."""
    B, Hq = p.batch, p.n_q_heads
    for name, t in (("vertical", vertical), ("slash", slash)):
        if t.dtype != torch.int32 or t.dim() != 3 or tuple(t.shape[:2]) != (B, Hq):
            raise ValueError(f"{name} must be int32 [B, Hq, n]")
    nv, ns = vertical.shape[2], slash.shape[2]
    q_bytes = p.batch * p.seqlen * p.n_q_heads * p.head_dim
    kv = p.batch * p.seqlen * p.n_kv_heads * p.head_dim * _elt(p)
    need = forward_workspace_bytes(p)
    osz = 4 if out_dtype == SA_F32 else 2
    _check(load().sparse_attn_forward_vs(
        ctypes.byref(p), _ptr(Q, "Q", q_bytes * _elt(p)), _ptr(K, "K", kv), _ptr(V, "V", kv),
        _ptr(vertical, "vertical", B * Hq * nv * 4) if nv else None, nv,
        _ptr(slash, "slash", B * Hq * ns * 4) if ns else None, ns, float(softmax_scale),
        _ptr(ws, "ws", need), 0 if ws is None else ws.numel() * ws.element_size(),
        _ptr(O, "O", q_bytes * osz), out_dtype,
        _ptr(lse, "lse", p.batch * p.n_q_heads * p.seqlen * 4), _stream(stream)))


def decode_art(p: Problem, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
               softmax_scale: float, tau: float, phi: float, patience: int, O: torch.Tensor,
               out_dtype: int, blocks_done: torch.Tensor, stream=None):
    """Decode attention with run-time termination (sparse_attn_decode_art): Q [B, Hq, d],
    K, V [B, N, Hkv, d]; writes O [B, Hq, d] and blocks_done int32 [B, Hq]."""
    B, Hq, d = p.batch, p.n_q_heads, p.head_dim
    kv = p.batch * p.seqlen * p.n_kv_heads * d * _elt(p)
    osz = 4 if out_dtype == SA_F32 else 2
    if blocks_done.dtype != torch.int32:
        raise ValueError("blocks_done must be int32")
    _check(load().sparse_attn_decode_art(
        ctypes.byref(p), _ptr(Q, "Q", B * Hq * d * _elt(p)), _ptr(K, "K", kv),
        _ptr(V, "V", kv), float(softmax_scale), float(tau), float(phi), int(patience),
        _ptr(O, "O", B * Hq * d * osz), out_dtype, _ptr(blocks_done, "blocks_done", B * Hq * 4),
        _stream(stream)))


class Prefill:
    """Device buffers for one workload shape and the three calls of a prefill layer.

    Allocation (torch) happens once here; ``run`` only enqueues the three library calls.
    """

    def __init__(self, w: wl.Workload, device="cuda", out_dtype: Optional[int] = None,
                 keep_stats: bool = True, with_lse: bool = False):
        self.w = w
        self.p = problem(w)
        self.b = budget(w)
        self.W = index_width(self.p, self.b)
        n = w.n_tiles
        dev = torch.device(device)
        self.out_dtype = w.dtype if out_dtype is None else out_dtype
        self.summ = torch.empty(summary_bytes(self.p) // 4, dtype=torch.float32, device=dev)
        self.ws = torch.empty(select_workspace_bytes(self.p, self.b), dtype=torch.uint8,
                              device=dev)
        fwb = forward_workspace_bytes(self.p)
        self.fws = torch.empty(max(fwb, 1), dtype=torch.uint8, device=dev) if fwb else None
        U = units(self.p)
        self.kv_idx = torch.empty((w.batch, U, n, self.W), dtype=torch.int32, device=dev)
        self.kv_cnt = torch.empty((w.batch, U, n), dtype=torch.int32, device=dev)
        if keep_stats:
            self.sigma = torch.empty((w.batch, U, n), dtype=torch.float32, device=dev)
            self.sigma_bar = torch.empty((w.batch, n), dtype=torch.float32, device=dev)
            self.gate = torch.empty((w.batch, n), dtype=torch.uint8, device=dev)
            self.tau = torch.empty((w.batch,), dtype=torch.float32, device=dev)
        else:
            self.sigma = self.sigma_bar = self.gate = self.tau = None
        odt = torch.float32 if self.out_dtype == SA_F32 else torch.bfloat16
        self.O = torch.empty((w.batch, w.seqlen, w.n_q_heads, w.head_dim), dtype=odt,
                             device=dev)
        self.lse = (torch.empty((w.batch, w.n_q_heads, w.seqlen), dtype=torch.float32,
                                device=dev) if with_lse else None)
        self.scale = 1.0 / math.sqrt(w.head_dim)

    def score(self, K, V, stream=None):
        score(self.p, K, V if self.w.output_aware else None, self.summ, stream)

    def select(self, Q, stream=None):
        select(self.p, self.b, Q, self.summ, self.ws, self.kv_idx, self.kv_cnt, self.sigma,
               self.sigma_bar, self.gate, self.tau, stream)

    def forward(self, Q, K, V, stream=None):
        forward(self.p, Q, K, V, self.kv_idx, self.kv_cnt, self.W, self.scale, self.fws,
                self.O, self.out_dtype, self.lse, stream)

    def prepare_values(self, V, stream=None):
        """First half of forward (bf16): V into this object's forward workspace."""
        prepare_values(self.p, V, self.fws, stream)

    def forward_prepared(self, Q, K, stream=None):
        """Second half of forward (bf16): the attention kernel over the prepared V."""
        forward_prepared(self.p, Q, K, self.fws, self.kv_idx, self.kv_cnt, self.W, self.scale,
                         self.O, self.out_dtype, self.lse, stream)

    def run(self, Q, K, V, stream=None):
        self.score(K, V, stream)
        self.select(Q, stream)
        self.forward(Q, K, V, stream)
        return self.O

    def calibrate_tau(self, Q, K, V=None) -> float:
        """A per-layer threshold for SA_GATE_FIXED from calibration inputs (gated-selection
        page, Metodologia step 4: a per-layer empirical quantile of sigma_bar): runs the
        summaries and the selection with the quantile gate, whatever this object's gate mode,
        then sparse_attn_calibrate_tau on the per-sequence thresholds.  Overwrites this
        object's lists and statistics; synchronizes to return the value.
        """
        b = budget(self.w)
        b.gate_mode = SA_GATE_QUANTILE
        dev = self.summ.device
        tau = torch.empty((self.w.batch,), dtype=torch.float32, device=dev)
        out = torch.empty((1,), dtype=torch.float32, device=dev)
        self.score(K, V)
        select(self.p, b, Q, self.summ, self.ws, self.kv_idx, self.kv_cnt, self.sigma,
               self.sigma_bar, self.gate, tau, None)
        calibrate_tau(tau, out)
        return float(out.cpu()[0])
