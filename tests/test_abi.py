"""The C-ABI library on the CPU: it loads, exports what the header declares, its structs have
the layout the binding assumes, and invalid arguments are rejected before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_causal_mean_amd import api
from block_sparse_causal_mean_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.LIB_PATH):
        from block_sparse_causal_mean_amd import build
        build.build()
    return api.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert _declared() == sorted(api.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in syms, name
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "sparse_attn.h"\n'
        "int main(void){\n"
        'printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(sa_problem), sizeof(sa_budget),'
        " offsetof(sa_budget, tau_fixed), offsetof(sa_budget, rho), offsetof(sa_budget, q),"
        " offsetof(sa_problem, oam_beta), offsetof(sa_problem, select_unit));\n"
        "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(api.Problem), ctypes.sizeof(api.Budget),
            api.Budget.tau_fixed.offset, api.Budget.rho.offset, api.Budget.q.offset,
            api.Problem.oam_beta.offset, api.Problem.select_unit.offset]
    assert got == want


def _ok_problem():
    return api.problem(wl.WORKLOADS["llama8b_32k"])


def _ok_budget():
    return api.budget(wl.WORKLOADS["llama8b_32k"])


def test_sizes(lib):
    p, b = _ok_problem(), _ok_budget()
    assert api.index_width(p, b) == 65
    assert api.select_workspace_bytes(p, b) >= 32 * 512 * 64 * 4

    def expect(B, n, Hkv, d, nplanes, oam):
        # public fp32 planes (+ vnorm), then knorm and dnorm, then 256-aligned private copies
        # in 32-block chunks: bf16 of every plane, then fp32 of every plane
        plane = B * n * Hkv * d
        head = plane * nplanes * 4 + (B * n * Hkv * 4 if oam else 0) + 2 * B * n * Hkv * 4
        head = (head + 255) // 256 * 256
        chunks = B * Hkv * ((n + 31) // 32)
        bfc = chunks * nplanes * d * 32 * 2
        xc_off = (head + bfc + 255) // 256 * 256
        return xc_off + chunks * nplanes * d * 32 * 4

    assert api.summary_bytes(p) == expect(1, 512, 8, 128, 1, False)
    p5, b5 = api.problem(wl.WORKLOADS["stem_32k"]), api.budget(wl.WORKLOADS["stem_32k"])
    assert api.summary_bytes(p5) == expect(4, 512, 8, 128, 1, True)
    assert api.index_width(p5, b5) == 131
    p4 = api.problem(wl.WORKLOADS["quest_64k"])
    assert api.summary_bytes(p4) == expect(1, 1024, 8, 128, 2, False)


BAD_PROBLEMS = [
    (dict(head_dim=96), api.SA_ERR_UNSUPPORTED),
    (dict(block=32, tile=32), api.SA_ERR_UNSUPPORTED),
    (dict(tile=256), api.SA_ERR_UNSUPPORTED),
    (dict(block=128, tile=32), api.SA_ERR_UNSUPPORTED),
    (dict(block=64, tile=32), api.SA_ERR_UNSUPPORTED),
    (dict(seqlen=64 * 511, tile=128), api.SA_ERR_INVALID),
    (dict(seqlen=1000), api.SA_ERR_INVALID),
    (dict(n_q_heads=30), api.SA_ERR_INVALID),
    (dict(batch=0), api.SA_ERR_INVALID),
    (dict(dtype=7), api.SA_ERR_INVALID),
    (dict(score_mode=2), api.SA_ERR_INVALID),
    (dict(output_aware=3), api.SA_ERR_INVALID),
    (dict(output_aware=2, oam_beta=-0.5), api.SA_ERR_INVALID),
    (dict(output_aware=2, oam_beta=float("nan")), api.SA_ERR_INVALID),
    (dict(select_unit=2), api.SA_ERR_INVALID),
    (dict(select_unit=-1), api.SA_ERR_INVALID),
    (dict(seqlen=64 * 16385), api.SA_ERR_UNSUPPORTED),
]

BAD_BUDGETS = [
    dict(k_min=0), dict(k_max=3, k_min=5), dict(kind=5), dict(n_sink=-1), dict(gate_mode=9),
    dict(rho=0.5), dict(rho=float("inf")), dict(q=1.5), dict(q=-0.1), dict(q=float("nan")),
]

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


@pytest.mark.parametrize("over,code", BAD_PROBLEMS)
def test_invalid_problem_rejected_before_hip(lib, over, code):
    p = _ok_problem()
    for k, v in over.items():
        setattr(p, k, v)
    b = _ok_budget()
    assert lib.sparse_attn_summary_bytes(ctypes.byref(p)) == 0
    assert lib.sparse_attn_score(ctypes.byref(p), FAKE, FAKE, FAKE, None) == code
    assert api.last_error()
    assert lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, FAKE, 1 << 40,
                                  FAKE, FAKE, None, None, None, None, None) == code
    assert lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65, 0.1, FAKE,
                                   1 << 40, FAKE, api.SA_BF16, None, None) == code


@pytest.mark.parametrize("over", BAD_BUDGETS)
def test_invalid_budget_rejected_before_hip(lib, over):
    p, b = _ok_problem(), _ok_budget()
    for k, v in over.items():
        setattr(b, k, v)
    assert lib.sparse_attn_index_width(ctypes.byref(p), ctypes.byref(b)) == api.SA_ERR_INVALID
    assert lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, FAKE, 1 << 40,
                                  FAKE, FAKE, None, None, None, None, None) == api.SA_ERR_INVALID


def test_null_pointers_and_small_buffers_rejected(lib):
    p, b = _ok_problem(), _ok_budget()
    r = lib.sparse_attn_score(ctypes.byref(p), None, FAKE, FAKE, None)
    assert r == api.SA_ERR_INVALID and "non-NULL" in api.last_error()
    p5 = api.problem(wl.WORKLOADS["stem_32k"])
    assert lib.sparse_attn_score(ctypes.byref(p5), FAKE, None, FAKE, None) == api.SA_ERR_INVALID
    need = api.select_workspace_bytes(p, b)
    r = lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, FAKE, need - 1,
                               FAKE, FAKE, None, None, None, None, None)
    assert r == api.SA_ERR_INVALID and "workspace" in api.last_error()
    r = lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, FAKE, need, None,
                               FAKE, None, None, None, None, None)
    assert r == api.SA_ERR_INVALID
    big = 1 << 40
    assert lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.1, FAKE,
                                   big, FAKE, api.SA_BF16, None, None) == api.SA_ERR_INVALID
    assert lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65, 0.1, FAKE,
                                   big, FAKE, 5, None, None) == api.SA_ERR_INVALID
    assert lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65,
                                   float("inf"), FAKE, big, FAKE, api.SA_BF16, None,
                                   None) == api.SA_ERR_INVALID
    need = api.forward_workspace_bytes(p)
    vbytes = 1 * 32768 * 8 * 128 * 2  # fp16 V images, then 64 partial maxima and one exponent
    assert need == vbytes + ((8 * 64 * 4 + 255) // 256) * 256 + 256  # per (batch, kv head)
    r = lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65, 0.1, FAKE,
                                need - 1, FAKE, api.SA_BF16, None, None)
    assert r == api.SA_ERR_INVALID and "workspace" in api.last_error()
    assert api.forward_workspace_bytes(api.problem(wl.WORKLOADS["tiny_ref"])) == 0
    assert lib.sparse_attn_score(None, FAKE, FAKE, FAKE, None) == api.SA_ERR_INVALID


def test_bf16_forward_rejects_more_than_4gib_of_keys_per_batch_element(lib):
    # 1M tokens x 16 kv heads x 128 x 2 bytes = 4 GiB of K in one batch element: the bf16 kernel
    # addresses a batch element's keys with 32-bit byte offsets, so the call must refuse it
    # before any HIP call (FAKE pointers are never touched).
    p = _ok_problem()
    p.seqlen, p.n_q_heads, p.n_kv_heads = 1 << 20, 16, 16
    big = 1 << 60
    r = lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65, 0.1, FAKE,
                                big, FAKE, api.SA_BF16, None, None)
    assert r == api.SA_ERR_UNSUPPORTED and "32-bit" in api.last_error()


def test_binding_refuses_host_tensors(lib):
    import torch
    w = wl.WORKLOADS["tiny_ref"]
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        api.score(api.problem(w), x, None, x)


def test_forward_vs_validation(lib):
    p = _ok_problem()
    big = 1 << 40
    ok_ws = api.forward_workspace_bytes(p)

    def call(prob=p, vert=FAKE, nv=4, slash=FAKE, ns=4, ws_bytes=ok_ws, out=api.SA_BF16):
        return lib.sparse_attn_forward_vs(ctypes.byref(prob), FAKE, FAKE, FAKE, vert, nv, slash,
                                          ns, 0.1, FAKE, ws_bytes, FAKE, out, None, None)

    f32 = api.problem(wl.WORKLOADS["tiny_ref"])
    assert call(prob=f32, ws_bytes=big) == api.SA_ERR_UNSUPPORTED
    assert "bf16" in api.last_error()
    assert call(nv=300, ns=212) == api.SA_ERR_UNSUPPORTED
    assert call(nv=-1) == api.SA_ERR_INVALID
    assert call(vert=None) == api.SA_ERR_INVALID
    assert call(slash=None, ns=2) == api.SA_ERR_INVALID
    assert call(ws_bytes=ok_ws - 1) == api.SA_ERR_INVALID
    assert call(out=7) == api.SA_ERR_INVALID


def test_sizes_per_kv_head_lists_and_wide_tiles(lib):
    """Lists per kv head shrink the selection workspace by the group size; 128-row tiles over
    64-key blocks add a second forced diagonal block to each list and halve the tile count."""
    w = wl.WORKLOADS["llama8b_32k"]
    p, b = api.problem(w), api.budget(w)
    pk = api.problem(wl.WORKLOADS["llama8b_32k_kvshared"])
    pt = api.problem(wl.WORKLOADS["llama8b_32k_t128"])
    assert api.units(p) == 32 and api.units(pk) == 8
    ws, wsk = api.select_workspace_bytes(p, b), api.select_workspace_bytes(pk, b)
    assert wsk < ws and wsk >= 8 * 512 * 64 * 4  # ranked keys per (kv head, tile)
    assert api.index_width(pt, b) == 2 + 0 + 64 == wl.WORKLOADS["llama8b_32k_t128"].index_width()
    assert api.select_workspace_bytes(pt, b) < ws  # 256 tiles instead of 512
    # the block summaries do not depend on the tile or the selection unit
    assert api.summary_bytes(pk) == api.summary_bytes(pt) == api.summary_bytes(p)


def test_wide_tiles_rejected_where_unsupported(lib):
    """128-row tiles over 64-key blocks are a selection-and-prefill variant: the vertical-slash
    path and decode reject them before any HIP call."""
    pt = api.problem(wl.WORKLOADS["llama8b_32k_t128"])
    ws = api.forward_workspace_bytes(pt)
    rc = lib.sparse_attn_forward_vs(ctypes.byref(pt), FAKE, FAKE, FAKE, FAKE, 4, FAKE, 4, 0.1,
                                    FAKE, ws, FAKE, api.SA_BF16, None, None)
    assert rc == api.SA_ERR_UNSUPPORTED and "tile" in api.last_error()
    rc = lib.sparse_attn_decode_art(ctypes.byref(pt), FAKE, FAKE, FAKE, 0.1, 0.01, 0.01, 2, FAKE,
                                    api.SA_BF16, FAKE, None)
    assert rc == api.SA_ERR_UNSUPPORTED and "tile" in api.last_error()


def test_bench_refuses_more_than_one_gpu():
    import subprocess, sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)


def test_selection_lds_limit_rejected_before_hip(lib):
    """The selection keeps a sort key per block and the tile's query rows in LDS: problems
    whose need exceeds a CU's LDS are refused with SA_ERR_UNSUPPORTED before any HIP call,
    and the workspace query returns 0 for them.  Keys take 4 bytes while the query rows'
    area can hold the final sort's 64-bit keys, else 8."""
    p, b = _ok_problem(), _ok_budget()  # d 128, 64-row tiles: query rows 17408 B (34816 B
    #                                     with two planes or 128-row tiles); k 32, rho 2

    def fits(q, bb):
        return lib.sparse_attn_select_workspace_bytes(ctypes.byref(q), ctypes.byref(bb)) > 0

    def refused(q, bb):
        assert lib.sparse_attn_select_workspace_bytes(ctypes.byref(q), ctypes.byref(bb)) == 0
        rc = lib.sparse_attn_select(ctypes.byref(q), ctypes.byref(bb), FAKE, FAKE, FAKE,
                                    1 << 50, FAKE, FAKE, None, None, None, None, None)
        return rc == api.SA_ERR_UNSUPPORTED and "LDS" in api.last_error()

    p.seqlen = 64 * 16384  # 16384 blocks, the most a problem may have
    for over in (dict(), dict(score_mode=api.SA_KMINMAX), dict(tile=128),
                 dict(score_mode=api.SA_KMINMAX, tile=128)):
        q = api.Problem.from_buffer_copy(p)
        for k, v in over.items():
            setattr(q, k, v)
        assert fits(q, b), over  # 64 KiB of 4-byte keys + at most 69632 B of query rows
    # a budget whose final sort needs more than the query rows' area: 8-byte keys
    wide = api.Budget.from_buffer_copy(b)
    wide.k_max = wide.k_min = 2048  # Rn = 4096: 16 * 4096 > 34816
    assert fits(p, wide)  # 128 KiB of keys + 17408 B
    for over in (dict(score_mode=api.SA_KMINMAX), dict(tile=128)):
        q = api.Problem.from_buffer_copy(p)
        for k, v in over.items():
            setattr(q, k, v)
        assert refused(q, wide), over  # 128 KiB + 34816 B


def test_value_norm_lds_limit_rejected_before_hip(lib):
    """Output-aware scoring holds block x n_kv_heads norms in LDS."""
    p = api.problem(wl.WORKLOADS["stem_32k"])
    p.block = p.tile = 128
    p.n_q_heads = p.n_kv_heads = 320  # 128 x 320 x 4 bytes = 160 KiB
    rc = lib.sparse_attn_score(ctypes.byref(p), FAKE, FAKE, FAKE, None)
    assert rc == api.SA_ERR_UNSUPPORTED and "LDS" in api.last_error()


def test_prepared_forward_validation(lib):
    p = _ok_problem()
    ws = api.forward_workspace_bytes(p)
    assert lib.sparse_attn_prepare_values(ctypes.byref(p), FAKE, FAKE, ws - 1,
                                          None) == api.SA_ERR_INVALID
    assert lib.sparse_attn_prepare_values(ctypes.byref(p), None, FAKE, ws,
                                          None) == api.SA_ERR_INVALID

    def fwd(prob=p, ws_ptr=FAKE, ws_bytes=ws, W=65, out=api.SA_BF16, scale=0.1):
        return lib.sparse_attn_forward_prepared(ctypes.byref(prob), FAKE, FAKE, ws_ptr, ws_bytes,
                                                FAKE, FAKE, W, scale, FAKE, out, None, None)

    assert fwd(ws_bytes=ws - 1) == api.SA_ERR_INVALID
    assert fwd(ws_ptr=None) == api.SA_ERR_INVALID
    assert fwd(W=0) == api.SA_ERR_INVALID
    assert fwd(out=3) == api.SA_ERR_INVALID
    assert fwd(scale=float("nan")) == api.SA_ERR_INVALID
    f32 = api.problem(wl.WORKLOADS["tiny_ref"])
    assert fwd(prob=f32, ws_bytes=1 << 40) == api.SA_ERR_UNSUPPORTED
    assert "fp32" in api.last_error()
    assert lib.sparse_attn_prepare_values(ctypes.byref(f32), FAKE, FAKE, 1 << 40,
                                          None) == api.SA_ERR_UNSUPPORTED


def test_calibrate_tau_validation(lib):
    assert lib.sparse_attn_calibrate_tau(None, 2, FAKE, None) == api.SA_ERR_INVALID
    assert lib.sparse_attn_calibrate_tau(FAKE, 0, FAKE, None) == api.SA_ERR_INVALID
    assert lib.sparse_attn_calibrate_tau(FAKE, 2, None, None) == api.SA_ERR_INVALID


def test_select_noalloc_validation(lib):
    """The no-allocation selection validates as sparse_attn_select does and refuses problems
    whose workspace exceeds its fixed 64 MiB, all before any HIP call."""
    p, b = _ok_problem(), _ok_budget()

    def call(prob=p, bud=b, Q=FAKE, kv_idx=FAKE):
        return lib.sparse_attn_select_noalloc(ctypes.byref(prob), ctypes.byref(bud), Q, FAKE,
                                              kv_idx, FAKE, None, None, None, None, None)

    assert call(Q=None) == api.SA_ERR_INVALID
    assert call(kv_idx=None) == api.SA_ERR_INVALID
    bad = _ok_budget()
    bad.k_min = 0
    assert call(bud=bad) == api.SA_ERR_INVALID
    big = api.problem(wl.WORKLOADS["quest_64k"].resized(batch=8))
    bq = api.budget(wl.WORKLOADS["quest_64k"])
    assert api.select_workspace_bytes(big, bq) > api.NOALLOC_SCRATCH_BYTES
    assert call(prob=big, bud=bq) == api.SA_ERR_UNSUPPORTED
    assert "67108864" in api.last_error()
    # every benchmark workload fits
    for name in wl.WORKLOAD_ORDER:
        w = wl.WORKLOADS[name]
        assert api.select_workspace_bytes(api.problem(w), api.budget(w)) <= api.NOALLOC_SCRATCH_BYTES


def test_tiles_inside_blocks_sizes(lib):
    """64-row tiles inside 128-key blocks: one diagonal block per tile (W = 1 + n_sink +
    floor(rho k_max)), twice the tiles of the 128-row case, the same summaries."""
    w = wl.WORKLOADS["prefill_128k_t64"]
    p, b = api.problem(w), api.budget(w)
    p128 = api.problem(wl.WORKLOADS["prefill_128k"])
    assert api.index_width(p, b) == 1 + 0 + 128 == w.index_width()
    assert api.summary_bytes(p) == api.summary_bytes(p128)
    assert api.select_workspace_bytes(p, b) > api.select_workspace_bytes(p128, b)


def test_forward_rejects_non_positive_scale(lib):
    p = _ok_problem()
    big = 1 << 40
    for scale in (0.0, -0.1):
        assert lib.sparse_attn_forward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 65, scale,
                                       FAKE, big, FAKE, api.SA_BF16, None,
                                       None) == api.SA_ERR_INVALID
        assert "> 0" in api.last_error()
