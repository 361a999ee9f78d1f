"""sparse_attn_select_noalloc (the selection with the library's own device workspace, for
callers that cannot allocate) against sparse_attn_select with a caller workspace: two calls
in a row on one GPU, the second on a smaller problem, every output bit for bit."""

import numpy as np
import pytest
import torch

from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    # larger first: a stale workspace from it would show in the second call
    wl.WORKLOADS["stem_32k"].resized(batch=2, seqlen=8192, k_max=24, k_min=6),
    wl.WORKLOADS["quest_64k"].resized(seqlen=2048, n_q_heads=8, k_max=6, k_min=6),
]


def _outputs(w, p, b):
    n, U = w.n_tiles, api.units(p)
    W = api.index_width(p, b)
    dev = "cuda"
    return {"kv_idx": torch.full((w.batch, U, n, W), -7, dtype=torch.int32, device=dev),
            "kv_cnt": torch.full((w.batch, U, n), -7, dtype=torch.int32, device=dev),
            "sigma": torch.full((w.batch, U, n), -7.0, device=dev),
            "sigma_bar": torch.full((w.batch, n), -7.0, device=dev),
            "gate": torch.full((w.batch, n), 7, dtype=torch.uint8, device=dev),
            "tau": torch.full((w.batch,), -7.0, device=dev)}


def test_select_noalloc_matches_select_twice():
    for i, w in enumerate(CASES):
        print(f"[noalloc] call {i}: {w.name} B={w.batch} N={w.seqlen} Hq={w.n_q_heads}",
              flush=True)
        inp = {k: v.cuda() for k, v in wl.make_inputs(w).items()}
        p, b = api.problem(w), api.budget(w)
        assert api.select_workspace_bytes(p, b) <= api.NOALLOC_SCRATCH_BYTES
        summ = torch.empty(api.summary_bytes(p) // 4, dtype=torch.float32, device="cuda")
        api.score(p, inp["K"], inp["V"] if w.output_aware else None, summ)
        ws = torch.empty(api.select_workspace_bytes(p, b), dtype=torch.uint8, device="cuda")
        ref, got = _outputs(w, p, b), _outputs(w, p, b)
        api.select(p, b, inp["Q"], summ, ws, ref["kv_idx"], ref["kv_cnt"], ref["sigma"],
                   ref["sigma_bar"], ref["gate"], ref["tau"])
        api.select_noalloc(p, b, inp["Q"], summ, got["kv_idx"], got["kv_cnt"], got["sigma"],
                           got["sigma_bar"], got["gate"], got["tau"])
        torch.cuda.synchronize()
        for k in ref:
            a, c = ref[k].cpu().numpy(), got[k].cpu().numpy()
            if a.dtype == np.float32:
                a, c = a.view(np.uint32), c.view(np.uint32)
            np.testing.assert_array_equal(c, a, err_msg=f"call {i}: {k}")
        # without the optional statistics (they then live in the library's array too)
        lists = _outputs(w, p, b)
        api.select_noalloc(p, b, inp["Q"], summ, lists["kv_idx"], lists["kv_cnt"])
        torch.cuda.synchronize()
        np.testing.assert_array_equal(lists["kv_idx"].cpu().numpy(), ref["kv_idx"].cpu().numpy())
        np.testing.assert_array_equal(lists["kv_cnt"].cpu().numpy(), ref["kv_cnt"].cpu().numpy())
