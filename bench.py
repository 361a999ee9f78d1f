"""Throughput of one block-sparse prefill attention layer on one MI355X.

A step is one pass of the whole hot path over one batch: sparse_attn_score (block
summaries), sparse_attn_select (scores, top-k, cut margin, gate, lists) and
sparse_attn_forward (online-softmax attention over the selected blocks), on inputs already
resident in HBM.  The workload is the 128K-token prefill (1 x 131072 tokens, 32 q / 8 kv
heads, d = 128, bf16, block = tile = 128, k = 64, rho = 2, q = 0.1) unless --workload names
another.  Prints ONE JSON line on stdout; progress goes to stderr.

  value         tokens/s = B * N * steps / timed seconds
  roofline      the attention kernel (the dominant one) against bf16 matrix-core peak, on
                effective FLOPs (4 * tile * block * d per listed block), timed on its own
                with HIP events on the stream it runs on: the forward pass runs as its two
                halves, sparse_attn_prepare_values (V to fp16 images) and
                sparse_attn_forward_prepared (the attention kernel alone); the causal-exact
                FLOP count (masked pairs of the diagonal blocks left out) is reported beside
  score_roofline  the block-summary kernel against HBM peak on its algorithmic bytes (keys,
                and values when output-aware, read once; the public summary planes written
                once), timed on launches back to back over three copies of the inputs so
                that no cache holds what a launch reads (a single launch timed right after a
                cache eviction, which also counts the dispatch latency, is reported beside
                it); the selection's private copies of the summaries, written by the same
                kernel, are reported separately
  cpu_baseline  the CPU oracle on a bounded sample of the same workload (see "sample")
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from block_sparse_causal_mean_amd import api  # noqa: E402
from block_sparse_causal_mean_amd import workloads as wl  # noqa: E402

METRIC = "sparse prefill attn tokens/s at 128k (1 GPU); % bf16 MFMA peak; HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def traffic_from_profiles(name: str):
    """HBM bytes per launch measured by rocprofv3 counters, if recorded for this kernel
    source (profiles/<name>.json carries the source digest it was measured on)."""
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "block_sparse_causal_mean_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src):
        return None
    import hashlib
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if digest != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


def effective_flops(w: wl.Workload, kv_cnt: torch.Tensor) -> float:
    """4 T blk d per listed block and query head (a list shared by a kv head's query heads
    counts once per head)."""
    heads_per_list = w.n_q_heads // w.n_units
    return 4.0 * w.tile * w.block * w.head_dim * heads_per_list * float(kv_cnt.sum().item())


def causal_exact_flops(w: wl.Workload, kv_idx: torch.Tensor, kv_cnt: torch.Tensor) -> float:
    """4 d per (query row, key) pair the attention actually computes: every pair of a listed
    block with the key at or before the row (the masked half of the diagonal blocks left
    out), per query head."""
    idx = kv_idx.cpu().numpy().astype(np.int64)
    cnt = kv_cnt.cpu().numpy()
    T, Bk = w.tile, w.block
    valid = np.arange(idx.shape[-1])[None, None, None, :] < cnt[..., None]
    t = np.broadcast_to(np.arange(idx.shape[2])[None, None, :, None], idx.shape)
    j = idx[valid]
    t = t[valid]
    # rows i = tT .. tT+T-1, keys p = jB .. jB+B-1: pairs with p <= i
    i0, p0 = t * T, j * Bk
    full = p0 + Bk - 1 <= i0
    pairs = np.where(full, T * Bk, 0).astype(np.float64)
    part = ~full
    if part.any():
        r = np.arange(T)[None, :]
        c = np.clip(i0[part][:, None] + r - p0[part][:, None] + 1, 0, Bk)
        pairs[part] = c.sum(axis=1)
    heads_per_list = w.n_q_heads // w.n_units
    return 4.0 * w.head_dim * heads_per_list * float(pairs.sum())


def vs_block_counts(w: wl.Workload, vert: np.ndarray, slash: np.ndarray) -> np.ndarray:
    """Blocks per (b, h, t) that the vertical-slash path reads (for its FLOP count): the
    vertical blocks <= t, the blocks t - delta for the offsets delta <= t, and t."""
    n = w.n_blocks
    t = np.arange(n)[:, None]
    cnt = np.zeros(vert.shape[:2] + (n,), np.int64)
    for b in range(vert.shape[0]):
        for h in range(vert.shape[1]):
            m = np.zeros((n, n), bool)
            m[np.arange(n), np.arange(n)] = True
            v = vert[b, h]
            v = v[:np.argmax(v < 0)] if (v < 0).any() else v
            isv = np.zeros(n, bool)
            isv[v[(v >= 0) & (v < n)]] = True
            m |= isv[None, :] & (np.arange(n)[None, :] <= t)
            s = slash[b, h]
            s = s[:np.argmax(s < 0)] if (s < 0).any() else s
            for dl in s:
                r = np.arange(dl, n)
                m[r, r - dl] = True
            cnt[b, h] = m.sum(axis=1)
    return cnt


def bench_vs(args, w: wl.Workload, nv: int, ns: int):
    """The vertical-slash path alone (sparse_attn_forward_vs), index given: the VSPrefill
    page's fused kernel fed by the stand-in index of workloads.vs_index (the trained indexer
    is not available).  One step = one call on inputs resident in HBM."""
    log(f"[bench vs] workload {w.name}: generating inputs")
    ex = {}
    inp = wl.make_inputs(w, extras=ex)
    vert, slash = wl.vs_index(w, nv, ns, anchors=ex.get("anchors"))
    torch.cuda.set_device(0)
    dev = {k: v.cuda() for k, v in inp.items()}
    p = api.problem(w)
    ws = torch.empty(api.forward_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    O = torch.empty((w.batch, w.seqlen, w.n_q_heads, w.head_dim), dtype=torch.bfloat16,
                    device="cuda")
    vt, st = torch.from_numpy(vert).cuda(), torch.from_numpy(slash).cuda()
    scale = 1.0 / math.sqrt(w.head_dim)
    call = lambda: api.forward_vs(p, dev["Q"], dev["K"], dev["V"], vt, st, scale, ws, O,
                                  api.SA_BF16)
    for _ in range(args.warmup):
        call()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in ev:
        e0.record(s)
        call()
        e1.record(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    cnt = vs_block_counts(w, vert, slash)
    flops = 4.0 * w.tile * w.block * w.head_dim * float(cnt.sum())
    achieved = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "vertical-slash sparse attention tokens/s (1 GPU, index given)",
        "value": w.batch * w.seqlen * args.steps / elapsed, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block": w.block, "index": "vertical-slash",
                   "n_vertical": nv, "n_slash": ns,
                   "index_source": "planted anchors + slash period" if "anchors" in ex
                   else "seeded random columns + local window",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel": "attn_bf16 (sparse_attn_forward_vs)",
                     "flops_per_launch": flops, "ms_per_launch": ms},
        "selection": {"mean_blocks_per_tile": float(cnt.mean()),
                      "density_of_causal": float(cnt.sum()) / (w.batch * w.n_q_heads *
                                                               w.n_blocks * (w.n_blocks + 1) / 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_decode(args, w: wl.Workload):
    """Decode with run-time termination (ART page), one step = one decode token per sequence
    and query head over the resident K/V cache.  Times the rule's run and, for comparison, the
    full traversal (patience 0).  HBM traffic = the K/V blocks each (sequence, kv head)
    workgroup streams: up to the last of its query heads to stop."""
    log(f"[bench decode] workload {w.name}: generating inputs")
    t0 = time.perf_counter()
    inp = wl.make_decode_inputs(w)
    log(f"[bench decode] inputs ready in {time.perf_counter() - t0:.1f}s")
    torch.cuda.set_device(0)
    dev = {k: v.cuda() for k, v in inp.items()}
    p = api.problem(w)
    O = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    done = torch.empty((w.batch, w.n_q_heads), dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)
    s = torch.cuda.current_stream()

    def timed(patience):
        call = lambda: api.decode_art(p, dev["Q"], dev["K"], dev["V"], scale, w.art_tau,
                                      w.art_phi, patience, O, api.SA_BF16, done)
        for _ in range(args.warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for e0, e1 in ev:
            e0.record(s)
            call()
            e1.record(s)
        torch.cuda.synchronize()
        return (time.perf_counter() - t_start,
                float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])))

    el_full, ms_full = timed(0)
    el, ms = timed(w.art_patience)
    d = done.cpu().numpy()
    G = w.n_q_heads // w.n_kv_heads
    streamed = d.reshape(w.batch, w.n_kv_heads, G).max(axis=2)
    n = w.seqlen // w.block
    kv_block = w.block * w.head_dim * 2 * 2
    bytes_art = float(streamed.sum()) * kv_block + 2 * w.batch * w.n_q_heads * w.head_dim * 2
    bytes_full = float(w.batch * w.n_kv_heads * n) * kv_block + 2 * w.batch * w.n_q_heads * w.head_dim * 2
    gbs = bytes_art / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode tokens/s with run-time termination (1 GPU)",
        "value": w.batch * args.steps / el, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": el * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "cached_tokens": w.seqlen,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block": w.block, "tau": w.art_tau, "phi": w.art_phi,
                   "patience": w.art_patience, "probe": 16, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "art_decode (sparse_attn_decode_art)", "bytes_per_launch": bytes_art,
                     "ms_per_launch": ms},
        "full_traversal": {"ms_per_launch": ms_full, "bytes_per_launch": bytes_full,
                           "achieved_GBs": bytes_full / (ms_full * 1e-3) / 1e9,
                           "tokens_per_s": w.batch * args.steps / el_full},
        "termination": {"mean_blocks_per_head": float(d.mean()), "blocks": n,
                        "mean_blocks_streamed_per_kv_head": float(streamed.mean()),
                        "speedup_vs_full": ms_full / ms},
    }
    if not args.no_cpu_baseline:
        import oracle
        nb = w.batch
        wb = w.resized(batch=nb)
        t0 = time.perf_counter()
        oracle.decode_art(oracle.make_cfg(wb), inp["Q"][:nb], inp["K"][:nb], inp["V"][:nb], scale,
                          16, w.art_tau, w.art_phi, w.art_patience, keep_partials=False)
        sec = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": nb / sec, "unit": "tokens/s", "cores": oracle.threads(),
                               "kind": "oracle",
                               "sample": f"{nb} of {w.batch} sequences, all {w.n_q_heads} heads, "
                                         f"the whole traversal in fp64 ({sec:.1f}s)"}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def time_score_cold(pf: api.Prefill, K, V, reps: int = 10) -> float:
    """Mean duration (ms) of the summary kernel(s) with the caches evicted before each run.

    The eviction READS a 1 GiB buffer (4x the last-level cache), so K cannot be served from any
    cache and no dirty lines are left behind: evicting by writing leaves write-backs that share
    HBM with the timed kernel and measured at half the read bandwidth of a clean eviction.
    Eviction, start event, kernel and end event are enqueued back to back, so the start event
    completes when the eviction does and the kernel is already queued behind it: the interval
    holds the kernel, not the host's launch latency."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    total = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.sum(flush, dim=0, out=sink)
        e0.record(s)
        pf.score(K, V)
        e1.record(s)
        e1.synchronize()
        total += e0.elapsed_time(e1)
    del flush
    return total / reps


def time_score_stream(pf: api.Prefill, K, V, output_aware: bool, copies: int = 3,
                      rounds: int = 4) -> float:
    """Mean duration (ms) of the summary kernel(s) launched back to back over `copies` copies
    of the keys (and values when output-aware), cycling through them: each launch reads a copy
    after the other copies (over twice the last-level cache) have been streamed, so no cache
    holds its input, and the launches follow each other as a model's layers would, with no
    eviction kernel or host round trip between them. One untimed cycle first."""
    Ks = [K] + [K.clone() for _ in range(copies - 1)]
    Vs = [V] + [V.clone() if output_aware else V for _ in range(copies - 1)]
    for i in range(copies):
        pf.score(Ks[i], Vs[i])
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(rounds):
        for i in range(copies):
            pf.score(Ks[i], Vs[i])
    e1.record(s)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / (rounds * copies)
    pf.score(K, V)  # leave the summaries of the benchmark's own inputs in place
    torch.cuda.synchronize()
    del Ks, Vs
    return ms


def cpu_baseline(w: wl.Workload, inp, budget_s: float = 15.0, max_tiles: int = 48) -> dict:
    """The oracle on a bounded sample: block summaries of the whole sequence, then the
    selection and the attention of every row of query tiles spread evenly over the second
    half-plus of the sequence (all heads, untripped budget), until about `budget_s` seconds
    of CPU work are spent."""
    import oracle
    cfg = oracle.make_cfg(w)
    threads = oracle.threads()
    t0 = time.perf_counter()
    summ = oracle.pool(cfg, inp["K"], inp["V"])
    t_pool = time.perf_counter() - t0
    n = w.n_tiles
    order = [int(x) for x in np.linspace(n // 4, n - 1, max_tiles)]
    rng = np.random.default_rng(0)
    order = list(rng.permutation(sorted(set(order))))
    tiles = []
    t_sel = t_fwd = 0.0
    for t in order:
        if t_sel + t_fwd + t_pool >= budget_s:
            break
        tiles.append(int(t))
        b = 0
        t1 = time.perf_counter()
        one = oracle.select_tile(cfg, inp["Q"], summ, b, t)
        t_sel += time.perf_counter() - t1
        rows = np.array([(b, h, p) for h in range(w.n_q_heads)
                         for p in range(t * w.tile, (t + 1) * w.tile)], np.int64)
        idx = np.zeros((w.batch, w.n_units, n, cfg.width), np.int32)
        cnt = np.zeros((w.batch, w.n_units, n), np.int32)
        idx[b, :, t] = one["lists"][0]
        cnt[b, :, t] = one["cnts"][0]
        t1 = time.perf_counter()
        oracle.forward(cfg, inp["Q"], inp["K"], inp["V"], idx, cnt, 1.0 / math.sqrt(w.head_dim),
                       rows=rows)
        t_fwd += time.perf_counter() - t1
        log(f"  cpu oracle tile {t}: select {t_sel:.1f}s forward {t_fwd:.1f}s (cumulative)")
    tok = len(tiles) * w.tile
    tiles = sorted(tiles)
    per_token = t_pool / (w.batch * w.seqlen) + (t_sel + t_fwd) / tok
    return {
        "value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "sample": (f"block summaries of all {w.batch * w.seqlen} tokens ({t_pool:.2f}s), then "
                   f"selection + attention of every row of {len(tiles)} query tiles "
                   f"{tiles} x {w.n_q_heads} heads ({tok} tokens, {t_sel:.2f}s + {t_fwd:.2f}s); "
                   f"tokens/s = 1 / (pool s per token + tile s per token)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=wl.HEADLINE, choices=list(wl.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--vs", default=None, metavar="NV,NS",
                    help="time the vertical-slash path instead (NV vertical blocks and NS slash "
                         "offsets per head from the stand-in index)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB, so a "
                         "counter profile of this command can scale its byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    w = wl.WORKLOADS[args.workload]
    if args.vs:
        nv, ns = (int(x) for x in args.vs.split(","))
        bench_vs(args, w, nv, ns)
        return
    if w.kind == "decode":
        bench_decode(args, w)
        return
    log(f"[bench] workload {w.name}: generating inputs")
    t0 = time.perf_counter()
    inp = wl.make_inputs(w)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s; copying to the GPU")
    torch.cuda.set_device(0)
    dev = {k: v.cuda() for k, v in inp.items()}
    Q, K, V = dev["Q"], dev["K"], dev["V"]
    pf = api.Prefill(w, keep_stats=True)
    s = torch.cuda.current_stream()
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done")
        del src, dst

    for i in range(args.warmup):
        pf.run(Q, K, V)
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    # One step: score, select, then the forward pass as its two halves (V prepared, then the
    # attention kernel), with an event between each so the attention kernel is timed alone.
    bf16 = w.dtype == wl.BF16
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(s)
        pf.score(K, V)
        ev[i][1].record(s)
        pf.select(Q)
        ev[i][2].record(s)
        if bf16:
            pf.prepare_values(V)
            ev[i][3].record(s)
            pf.forward_prepared(Q, K)
        else:
            ev[i][3].record(s)
            pf.forward(Q, K, V)
        ev[i][4].record(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    stage = np.array([[ev[i][k].elapsed_time(ev[i][k + 1]) for k in range(4)]
                      for i in range(args.steps)])
    ms_score, ms_select, ms_prep, ms_attn = stage.mean(axis=0)
    ms_fwd = ms_prep + ms_attn
    log(f"[bench] {args.steps} steps in {elapsed:.3f}s: score {ms_score:.3f} ms, select "
        f"{ms_select:.3f} ms, forward {ms_fwd:.3f} ms (values {ms_prep:.3f} + attention "
        f"{ms_attn:.3f})")

    tokens = w.batch * w.seqlen
    value = tokens * args.steps / elapsed
    flops = effective_flops(w, pf.kv_cnt)
    exact_flops = causal_exact_flops(w, pf.kv_idx, pf.kv_cnt)
    achieved = flops / (ms_attn * 1e-3) / 1e12
    dense = 4.0 * w.head_dim * w.seqlen * (w.seqlen + 1) / 2 * w.batch * w.n_q_heads
    traffic = traffic_from_profiles("attn_fwd_" + w.name)

    ms_single = time_score_cold(pf, K, V)
    ms_cold = time_score_stream(pf, K, V, bool(w.output_aware))
    elt = 2 if bf16 else 4
    kv_bytes = w.batch * w.seqlen * w.n_kv_heads * w.head_dim * elt
    planes = 2 if w.score_mode == wl.KMINMAX else 1
    blocks = w.batch * w.n_blocks * w.n_kv_heads
    public = 4 * (blocks * w.head_dim * planes + (blocks if w.output_aware else 0))
    score_bytes = kv_bytes * (2 if w.output_aware else 1) + public
    private_bytes = pf.summ.numel() * 4 - public
    score_gbs = score_bytes / (ms_cold * 1e-3) / 1e9

    gate = pf.gate.float().mean().item()
    # causal (tile, block) pairs: tile t has (t + 1) T / blk causal blocks, rounded up
    causal = sum(((t + 1) * w.tile + w.block - 1) // w.block for t in range(w.n_tiles))
    density = float(pf.kv_cnt.sum().item()) / (w.batch * w.n_units * causal)
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "block": w.block, "tile": w.tile,
                   "score_mode": "kminmax" if w.score_mode == wl.KMINMAX else "kmean",
                   "output_aware": ["off", "product", "additive"][w.output_aware],
                   **({"oam_beta": w.oam_beta} if w.output_aware == wl.OAM_ADDITIVE else {}),
                   "k_max": w.k_max, "k_min": w.k_min,
                   "budget": "linear_decay" if w.budget_kind else "const", "n_sink": w.n_sink,
                   "rho": w.rho, "q": w.q,
                   "lists": "per kv head" if w.select_unit else "per query head",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": ("attn_bf16 (sparse_attn_forward_prepared)" if bf16
                                else "attn_f32 (sparse_attn_forward)"),
                     "flops_per_launch": flops, "ms_per_launch": ms_attn,
                     "causal_exact_flops_per_launch": exact_flops,
                     "causal_exact_frac": exact_flops / (ms_attn * 1e-3) / 1e12
                     / PEAK_BF16_TFLOPS},
        "score_roofline": {"bound": "hbm", "achieved": score_gbs, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": score_gbs / PEAK_HBM_GBS,
                           "traffic": traffic_from_profiles("pool_keys_" + w.name),
                           "bytes_per_launch": score_bytes,
                           "private_copy_bytes_per_launch": private_bytes,
                           "ms_per_launch_cold": ms_cold,
                           "ms_single_launch_after_eviction": ms_single,
                           "kernel": "pool_keys (sparse_attn_score)"},
        "stages_ms": {"score": ms_score, "select": ms_select, "forward": ms_fwd,
                      "forward_values": ms_prep, "forward_attention": ms_attn},
        "selection": {"density_of_causal": density, "trip_fraction": gate,
                      "dense_causal_flops": dense, "effective_flops": flops,
                      "causal_exact_flops": exact_flops},
    }
    if not args.no_cpu_baseline and rank == 0:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, inp)
    else:
        out["cpu_baseline"] = None
    if rank == 0:
        print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
