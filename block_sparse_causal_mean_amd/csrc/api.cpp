// C ABI of the block-sparse causal prefill library: argument validation, buffer sizes and
// kernel dispatch.  Every check runs on the host before any HIP call, so an invalid call
// enqueues nothing and touches no device.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "common.h"

// Selection workspace of sparse_attn_select_noalloc: a fixed device array instead of a caller
// buffer (each GPU the library runs on holds its own copy until the process ends).  Host code
// never uses this name as an address: it keeps the address hipGetSymbolAddress returns, per
// device.
constexpr size_t kScratchBytes = 64u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int kMaxTiles = 16384;  // LDS sizing of the ranking and gate kernels

int check_problem(const sa_problem* p, sa::Dims* D) {
  if (!p) return fail(SA_ERR_INVALID, "problem is NULL");
  if (p->batch < 1 || p->seqlen < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1)
    return fail(SA_ERR_INVALID, "batch, seqlen and head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads)
    return fail(SA_ERR_INVALID, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->dtype != SA_BF16 && p->dtype != SA_F32)
    return fail(SA_ERR_INVALID, "dtype must be SA_BF16 or SA_F32");
  if (p->score_mode != SA_KMEAN && p->score_mode != SA_KMINMAX)
    return fail(SA_ERR_INVALID, "score_mode must be SA_KMEAN or SA_KMINMAX");
  if (p->output_aware != SA_OAM_OFF && p->output_aware != SA_OAM_PRODUCT &&
      p->output_aware != SA_OAM_ADDITIVE)
    return fail(SA_ERR_INVALID, "output_aware must be SA_OAM_OFF, SA_OAM_PRODUCT or SA_OAM_ADDITIVE");
  if (p->output_aware == SA_OAM_ADDITIVE && !(isfinite(p->oam_beta) && p->oam_beta >= 0.0f))
    return fail(SA_ERR_INVALID, "oam_beta must be finite and >= 0 for SA_OAM_ADDITIVE");
  if (p->select_unit != SA_SELECT_PER_Q_HEAD && p->select_unit != SA_SELECT_PER_KV_HEAD)
    return fail(SA_ERR_INVALID, "select_unit must be SA_SELECT_PER_Q_HEAD or SA_SELECT_PER_KV_HEAD");
  if (p->block < 1 || p->tile < 1) return fail(SA_ERR_INVALID, "block and tile must be >= 1");
  if (p->seqlen % p->block)
    return fail(SA_ERR_INVALID, "seqlen (%d) must be a multiple of block (%d)", p->seqlen,
                p->block);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", p->head_dim);
  if (p->block != 64 && p->block != 128)
    return fail(SA_ERR_UNSUPPORTED, "block %d unsupported (64 or 128)", p->block);
  if (p->tile != p->block && !(p->tile == 128 && p->block == 64) &&
      !(p->tile == 64 && p->block == 128))
    return fail(SA_ERR_UNSUPPORTED,
                "tile (%d) must equal block (%d), or be 128 over block 64, or 64 over block 128",
                p->tile, p->block);
  const long long n = p->seqlen / p->block;
  if (n > kMaxTiles)
    return fail(SA_ERR_UNSUPPORTED, "seqlen / block = %lld tiles exceeds %d", n, kMaxTiles);
  if (p->seqlen % p->tile)
    return fail(SA_ERR_INVALID, "seqlen (%d) must be a multiple of tile (%d)", p->seqlen, p->tile);
  if ((long long)p->batch * p->n_q_heads * n > 0x7fffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "batch * n_q_heads * tiles exceeds the launch grid");
  if (D) {
    D->B = p->batch;
    D->N = p->seqlen;
    D->Hq = p->n_q_heads;
    D->Hkv = p->n_kv_heads;
    D->G = p->n_q_heads / p->n_kv_heads;
    D->d = p->head_dim;
    D->blk = p->block;
    D->n = (int)n;
    D->T = p->tile;
    D->nt = p->seqlen / p->tile;
    D->m = p->tile >= p->block ? p->tile / p->block : 1;
    D->tpb = p->tile >= p->block ? 1 : p->block / p->tile;
    D->dtype = p->dtype;
    D->score_mode = p->score_mode;
    D->oam = p->output_aware;
    D->oam_beta = p->output_aware == SA_OAM_ADDITIVE ? p->oam_beta : 0.0f;
    D->oam_scale = (float)(1.0 / sqrt((double)p->head_dim));
    D->gs = p->select_unit == SA_SELECT_PER_KV_HEAD ? D->G : 1;
    D->Hu = D->Hq / D->gs;
  }
  return SA_OK;
}

int check_budget(const sa_budget* b, const sa::Dims& D, sa::BudgetDev* bd) {
  if (!b) return fail(SA_ERR_INVALID, "budget is NULL");
  if (b->k_min < 1 || b->k_max < b->k_min)
    return fail(SA_ERR_INVALID, "need 1 <= k_min (%d) <= k_max (%d)", b->k_min, b->k_max);
  if (b->kind != SA_K_CONST && b->kind != SA_K_LINEAR_DECAY)
    return fail(SA_ERR_INVALID, "kind must be SA_K_CONST or SA_K_LINEAR_DECAY");
  if (b->n_sink < 0) return fail(SA_ERR_INVALID, "n_sink must be >= 0");
  if (b->gate_mode != SA_GATE_QUANTILE && b->gate_mode != SA_GATE_FIXED &&
      b->gate_mode != SA_GATE_OFF)
    return fail(SA_ERR_INVALID, "gate_mode must be QUANTILE, FIXED or OFF");
  if (!(b->rho >= 1.0) || !isfinite(b->rho) || b->rho * b->k_max > 1e9)
    return fail(SA_ERR_INVALID, "rho must be finite and >= 1");
  if (b->gate_mode == SA_GATE_QUANTILE && !(b->q >= 0.0 && b->q <= 1.0))
    return fail(SA_ERR_INVALID, "q must lie in [0, 1]");
  if (b->gate_mode == SA_GATE_FIXED && isnan(b->tau_fixed))
    return fail(SA_ERR_INVALID, "tau_fixed is NaN");
  if (bd) {
    bd->k_max = b->k_max;
    bd->k_min = b->k_min;
    bd->kind = b->kind;
    bd->n_sink = b->n_sink;
    bd->gate_mode = b->gate_mode;
    bd->tau_fixed = b->tau_fixed;
    bd->rho = b->rho;
    bd->q = b->q;
    const long long ex = (long long)floor(b->rho * (double)b->k_max);
    long long r = ex > b->k_max ? ex : b->k_max;
    if (r > D.n) r = D.n;
    bd->R = (int)(r > 0 ? r : 1);
    long long w = D.m + (long long)b->n_sink + ex;
    if (w > D.n) w = D.n;
    bd->W = (int)w;
    bd->m = D.m;
    bd->tpb = D.tpb;
  }
  return SA_OK;
}

// LDS the selection kernels need grows with the number of blocks (one sort key each) and the
// tile's staged query rows; refused here rather than failing at launch.
int check_select_lds(const sa::Dims& D, const sa::BudgetDev& bd) {
  const size_t need = sa::score_rank_lds(D, bd);
  if (need > sa::kMaxDynLds)
    return fail(SA_ERR_UNSUPPORTED,
                "selection needs %zu bytes of LDS per workgroup (at most %zu): %d blocks of %d "
                "keys, %d-row tiles, head_dim %d%s",
                need, sa::kMaxDynLds, D.n, D.blk, D.T, D.d,
                D.score_mode == SA_KMINMAX ? ", K-min/K-max bound" : "");
  if (sa::gate_lds(D) > sa::kMaxDynLds)
    return fail(SA_ERR_UNSUPPORTED, "the gate needs %zu bytes of LDS (at most %zu)",
                sa::gate_lds(D), sa::kMaxDynLds);
  return SA_OK;
}

// The output-aware summaries hold one norm per (row, kv head) of a block in LDS.
int check_score_lds(const sa::Dims& D) {
  if (D.oam && sa::value_norms_lds(D) > sa::kMaxDynLds)
    return fail(SA_ERR_UNSUPPORTED,
                "output-aware scoring needs %zu bytes of LDS (block %d x %d kv heads x 4; at "
                "most %zu)",
                sa::value_norms_lds(D), D.blk, D.Hkv, sa::kMaxDynLds);
  return SA_OK;
}

size_t summary_bytes(const sa::Dims& D) { return sa::summary_layout(D).bytes; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SA_OK;
  return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t sparse_attn_summary_bytes(const sa_problem* p) {
  sa::Dims D;
  if (check_problem(p, &D) != SA_OK) return 0;
  return summary_bytes(D);
}

size_t sparse_attn_select_workspace_bytes(const sa_problem* p, const sa_budget* b) {
  sa::Dims D;
  sa::BudgetDev bd;
  if (check_problem(p, &D) != SA_OK || check_budget(b, D, &bd) != SA_OK ||
      check_select_lds(D, bd) != SA_OK)
    return 0;
  return sa::select_ws_layout(D, bd).total;
}

int32_t sparse_attn_index_width(const sa_problem* p, const sa_budget* b) {
  sa::Dims D;
  sa::BudgetDev bd;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if ((rc = check_budget(b, D, &bd)) != SA_OK) return rc;
  return bd.W;
}

int sparse_attn_score(const sa_problem* p, const void* K, const void* V, void* summaries,
                      void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (!K || !summaries) return fail(SA_ERR_INVALID, "K and summaries must be non-NULL");
  if (D.oam && !V) return fail(SA_ERR_INVALID, "V is required when output_aware is set");
  if ((rc = check_score_lds(D)) != SA_OK) return rc;
  g_err.clear();
  return hip_status(sa::launch_pool(D, K, V, static_cast<float*>(summaries),
                                    static_cast<hipStream_t>(stream)),
                    "sparse_attn_score launch");
}

int sparse_attn_select(const sa_problem* p, const sa_budget* b, const void* Q,
                       const void* summaries, void* ws, size_t ws_bytes, int32_t* kv_idx,
                       int32_t* kv_cnt, float* sigma, float* sigma_bar, uint8_t* gate,
                       float* tau, void* stream) {
  sa::Dims D;
  sa::BudgetDev bd;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if ((rc = check_budget(b, D, &bd)) != SA_OK) return rc;
  if ((rc = check_select_lds(D, bd)) != SA_OK) return rc;
  if (!Q || !summaries || !ws || !kv_idx || !kv_cnt)
    return fail(SA_ERR_INVALID, "Q, summaries, ws, kv_idx and kv_cnt must be non-NULL");
  const size_t need = sa::select_ws_layout(D, bd).total;
  if (ws_bytes < need)
    return fail(SA_ERR_INVALID, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  g_err.clear();
  return hip_status(sa::launch_select(D, bd, Q, static_cast<const float*>(summaries),
                                      static_cast<char*>(ws), kv_idx, kv_cnt, sigma, sigma_bar,
                                      gate, tau, static_cast<hipStream_t>(stream)),
                    "sparse_attn_select launch");
}

size_t sparse_attn_forward_workspace_bytes(const sa_problem* p) {
  sa::Dims D;
  if (check_problem(p, &D) != SA_OK) return 0;
  return sa::forward_ws_bytes(D);
}

int sparse_attn_forward(const sa_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* kv_idx, const int32_t* kv_cnt, int32_t W,
                        float softmax_scale, void* ws, size_t ws_bytes, void* O,
                        int32_t out_dtype, float* lse, void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (!Q || !K || !V || !kv_idx || !kv_cnt || !O)
    return fail(SA_ERR_INVALID, "Q, K, V, kv_idx, kv_cnt and O must be non-NULL");
  const size_t need = sa::forward_ws_bytes(D);
  if (need && (!ws || ws_bytes < need))
    return fail(SA_ERR_INVALID, "forward workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (W < 1) return fail(SA_ERR_INVALID, "W must be >= 1");
  if (out_dtype != SA_F32 && out_dtype != SA_BF16)
    return fail(SA_ERR_INVALID, "out_dtype must be SA_F32 or SA_BF16");
  if (!(isfinite(softmax_scale) && softmax_scale > 0.0f))
    return fail(SA_ERR_INVALID, "softmax_scale must be finite and > 0");
  if (D.dtype == SA_BF16 && (unsigned long long)D.N * D.Hkv * D.d * 2 >= (1ull << 32))
    return fail(SA_ERR_UNSUPPORTED,
                "seqlen * n_kv_heads * head_dim * 2 = %llu bytes of K per batch element: the "
                "bf16 kernel addresses a batch element's keys with 32-bit offsets (< 2^32)",
                (unsigned long long)D.N * D.Hkv * D.d * 2);
  g_err.clear();
  return hip_status(sa::launch_forward(D, Q, K, V, kv_idx, kv_cnt, W, softmax_scale, ws, O,
                                       out_dtype, lse, static_cast<hipStream_t>(stream)),
                    "sparse_attn_forward launch");
}

int sparse_attn_prepare_values(const sa_problem* p, const void* V, void* ws, size_t ws_bytes,
                               void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (D.dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED,
                "fp32 problems read V directly: call sparse_attn_forward (no prepared values)");
  if (!V || !ws) return fail(SA_ERR_INVALID, "V and ws must be non-NULL");
  const size_t need = sa::forward_ws_bytes(D);
  if (ws_bytes < need)
    return fail(SA_ERR_INVALID, "forward workspace too small: %zu < %zu bytes", ws_bytes, need);
  g_err.clear();
  return hip_status(sa::launch_prepare_values(D, V, ws, static_cast<hipStream_t>(stream)),
                    "sparse_attn_prepare_values launch");
}

int sparse_attn_forward_prepared(const sa_problem* p, const void* Q, const void* K,
                                 const void* ws, size_t ws_bytes, const int32_t* kv_idx,
                                 const int32_t* kv_cnt, int32_t W, float softmax_scale, void* O,
                                 int32_t out_dtype, float* lse, void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (D.dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED,
                "fp32 problems read V directly: call sparse_attn_forward (no prepared values)");
  if (!Q || !K || !ws || !kv_idx || !kv_cnt || !O)
    return fail(SA_ERR_INVALID, "Q, K, ws, kv_idx, kv_cnt and O must be non-NULL");
  const size_t need = sa::forward_ws_bytes(D);
  if (ws_bytes < need)
    return fail(SA_ERR_INVALID, "forward workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (W < 1) return fail(SA_ERR_INVALID, "W must be >= 1");
  if (out_dtype != SA_F32 && out_dtype != SA_BF16)
    return fail(SA_ERR_INVALID, "out_dtype must be SA_F32 or SA_BF16");
  if (!(isfinite(softmax_scale) && softmax_scale > 0.0f))
    return fail(SA_ERR_INVALID, "softmax_scale must be finite and > 0");
  if ((unsigned long long)D.N * D.Hkv * D.d * 2 >= (1ull << 32))
    return fail(SA_ERR_UNSUPPORTED,
                "seqlen * n_kv_heads * head_dim * 2 = %llu bytes of K per batch element: the "
                "bf16 kernel addresses a batch element's keys with 32-bit offsets (< 2^32)",
                (unsigned long long)D.N * D.Hkv * D.d * 2);
  g_err.clear();
  return hip_status(sa::launch_forward_prepared(D, Q, K, ws, kv_idx, kv_cnt, W, softmax_scale, O,
                                                out_dtype, lse, static_cast<hipStream_t>(stream)),
                    "sparse_attn_forward_prepared launch");
}

int sparse_attn_calibrate_tau(const float* tau, int32_t batch, float* tau_out, void* stream) {
  if (!tau || !tau_out) return fail(SA_ERR_INVALID, "tau and tau_out must be non-NULL");
  if (batch < 1) return fail(SA_ERR_INVALID, "batch must be >= 1");
  g_err.clear();
  return hip_status(sa::launch_tau_mean(tau, batch, tau_out, static_cast<hipStream_t>(stream)),
                    "sparse_attn_calibrate_tau launch");
}

int sparse_attn_forward_vs(const sa_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* vertical, int32_t n_vertical, const int32_t* slash,
                           int32_t n_slash, float softmax_scale, void* ws, size_t ws_bytes,
                           void* O, int32_t out_dtype, float* lse, void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (D.dtype != SA_BF16)
    return fail(SA_ERR_UNSUPPORTED, "the vertical-slash path takes bf16 inputs");
  if (D.m != 1) return fail(SA_ERR_UNSUPPORTED, "the vertical-slash path needs tile = block");
  if (!Q || !K || !V || !O) return fail(SA_ERR_INVALID, "Q, K, V and O must be non-NULL");
  if (n_vertical < 0 || n_slash < 0)
    return fail(SA_ERR_INVALID, "n_vertical and n_slash must be >= 0");
  if ((n_vertical > 0 && !vertical) || (n_slash > 0 && !slash))
    return fail(SA_ERR_INVALID, "a non-empty index needs a non-NULL pointer");
  if (n_vertical + n_slash > sa::kVsMaxEntries)
    return fail(SA_ERR_UNSUPPORTED, "n_vertical + n_slash = %d exceeds %d",
                n_vertical + n_slash, sa::kVsMaxEntries);
  const size_t need = sa::forward_ws_bytes(D);
  if (!ws || ws_bytes < need)
    return fail(SA_ERR_INVALID, "forward workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (out_dtype != SA_F32 && out_dtype != SA_BF16)
    return fail(SA_ERR_INVALID, "out_dtype must be SA_F32 or SA_BF16");
  if (!(isfinite(softmax_scale) && softmax_scale > 0.0f))
    return fail(SA_ERR_INVALID, "softmax_scale must be finite and > 0");
  if ((unsigned long long)D.N * D.Hkv * D.d * 2 >= (1ull << 32))
    return fail(SA_ERR_UNSUPPORTED,
                "seqlen * n_kv_heads * head_dim * 2 = %llu bytes of K per batch element: the "
                "bf16 kernel addresses a batch element's keys with 32-bit offsets (< 2^32)",
                (unsigned long long)D.N * D.Hkv * D.d * 2);
  g_err.clear();
  sa::VsIndex vs;
  vs.vert = vertical;
  vs.slash = slash;
  vs.nv = n_vertical;
  vs.ns = n_slash;
  return hip_status(sa::launch_forward_vs(D, Q, K, V, vs, softmax_scale, ws, O, out_dtype, lse,
                                          static_cast<hipStream_t>(stream)),
                    "sparse_attn_forward_vs launch");
}

int sparse_attn_decode_art(const sa_problem* p, const void* Q, const void* K, const void* V,
                           float softmax_scale, float tau, float phi, int32_t patience, void* O,
                           int32_t out_dtype, int32_t* blocks_done, void* stream) {
  sa::Dims D;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if (D.dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "the decode path takes bf16 inputs");
  if (D.blk != 64 || D.m != 1)
    return fail(SA_ERR_UNSUPPORTED, "the decode path uses blocks (and tiles) of 64 keys");
  if (D.G > sa::kArtMaxHeadsPerKv)
    return fail(SA_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads = %d exceeds %d", D.G,
                sa::kArtMaxHeadsPerKv);
  if (!Q || !K || !V || !O || !blocks_done)
    return fail(SA_ERR_INVALID, "Q, K, V, O and blocks_done must be non-NULL");
  if (!(isfinite(tau) && tau >= 0.0f) || !(isfinite(phi) && phi >= 0.0f))
    return fail(SA_ERR_INVALID, "tau and phi must be finite and >= 0");
  if (patience < 0) return fail(SA_ERR_INVALID, "patience must be >= 0");
  if (out_dtype != SA_F32 && out_dtype != SA_BF16)
    return fail(SA_ERR_INVALID, "out_dtype must be SA_F32 or SA_BF16");
  if (!isfinite(softmax_scale)) return fail(SA_ERR_INVALID, "softmax_scale is not finite");
  g_err.clear();
  return hip_status(sa::launch_decode_art(D, Q, K, V, softmax_scale, tau, phi, patience, O,
                                          out_dtype, blocks_done,
                                          static_cast<hipStream_t>(stream)),
                    "sparse_attn_decode_art launch");
}

int sparse_attn_select_noalloc(const sa_problem* p, const sa_budget* b, const void* Q,
                               const void* summaries, int32_t* kv_idx, int32_t* kv_cnt,
                               float* sigma, float* sigma_bar, uint8_t* gate, float* tau,
                               void* stream) {
  sa::Dims D;
  sa::BudgetDev bd;
  int rc = check_problem(p, &D);
  if (rc != SA_OK) return rc;
  if ((rc = check_budget(b, D, &bd)) != SA_OK) return rc;
  if ((rc = check_select_lds(D, bd)) != SA_OK) return rc;
  if (!Q || !summaries || !kv_idx || !kv_cnt)
    return fail(SA_ERR_INVALID, "Q, summaries, kv_idx and kv_cnt must be non-NULL");
  const size_t need = sa::select_ws_layout(D, bd).total;
  if (need > kScratchBytes)
    return fail(SA_ERR_UNSUPPORTED,
                "the selection needs %zu bytes of workspace; sparse_attn_select_noalloc holds "
                "%zu (use sparse_attn_select with a caller workspace)",
                need, kScratchBytes);
  // The device array's address on the current device, looked up once per device.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if ((rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) != SA_OK) return rc;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_ERR_UNSUPPORTED, "device %d beyond the %d this entry point tracks", dev,
                kMaxDevices);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
      void* ptr = nullptr;
      if ((rc = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)),
                           "hipGetSymbolAddress(scratch)")) != SA_OK)
        return rc;
      addr[dev] = ptr;
    }
    ws = addr[dev];
  }
  g_err.clear();
  return hip_status(sa::launch_select(D, bd, Q, static_cast<const float*>(summaries),
                                      static_cast<char*>(ws), kv_idx, kv_cnt, sigma, sigma_bar,
                                      gate, tau, static_cast<hipStream_t>(stream)),
                    "sparse_attn_select_noalloc launch");
}

const char* sparse_attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
