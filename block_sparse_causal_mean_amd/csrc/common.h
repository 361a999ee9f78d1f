// Internal declarations shared by the library's HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// ------------------------------------------------------------------ element conversion

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}
// Low and high bf16 halves of a packed 32-bit word, converted exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// 16-byte global load marked non-temporal: for data a kernel streams once (its lines are not
// worth keeping in the caches).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

// x + 0.0f: maps -0 to +0, leaves every other value unchanged.
__device__ __forceinline__ float canon(float x) { return x + 0.0f; }

// Monotone map of a non-NaN float to an unsigned key (larger float <-> larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ derived sizes

struct Dims {
  int B, N, Hq, Hkv, G, d, blk, n;  // n = N / blk key blocks
  int T, nt, m;  // query tile rows, tiles N / T, diagonal blocks per tile (T / blk, or 1)
  int tpb;       // query tiles per key block (blk / T when a block holds several tiles, or 1)
  int gs, Hu;  // query heads per selection unit (1, or G when lists are per kv head); units
  int dtype, score_mode, oam;     // oam: SA_OAM_OFF, SA_OAM_PRODUCT or SA_OAM_ADDITIVE
  float oam_beta, oam_scale;      // additive form: beta and (float)(1 / sqrt(d))
};

struct BudgetDev {
  int k_max, k_min, kind, n_sink, gate_mode;
  float tau_fixed;
  double rho, q;
  int R;    // ranked entries stored per (b, unit, t)
  int W;    // entries per padded list
  int m;    // diagonal blocks per tile: tile t's are first_diag(t) .. + m - 1, its free ones
  int tpb;  // before first_diag(t); tiles per block (see Dims)
};

// First diagonal block of query tile t, the block holding the tile's first row: t T / blk,
// i.e. m t for tiles of m blocks, t / tpb for tpb tiles per block.
__host__ __device__ __forceinline__ int first_diag(int m, int tpb, int t) { return m * t / tpb; }

// Layout of the block-summary buffer.  The public part (documented in the header) comes
// first: the fp32 planes [B, n, Hkv, d] (kmean, or kmin then kmax) and, when output-aware,
// vnorm [B, n, Hkv].  The library-private part follows: knorm [B, n, Hkv] (fp32 L2 norm of
// each block's scoring vector), dnorm [B, n, Hkv] (L2 norm of the scoring vector's bf16
// rounding residual x - bf16(x): per coordinate the larger of the two planes' for the bound),
// then two copies of the planes in "chunk-major" order, grouped by 32-block chunks per (batch,
// kv head), for the selection kernel:
//   bfc  each plane rounded to bf16 (round to nearest even), the matrix-core prefilter's B
//        operands: per chunk [plane][d/16 steps][64 lanes][8], lane (i, u) holding
//        coordinates 16 step + 8u .. +7 of block 32 chunk + i, so every operand load of a
//        wave reads 1 KiB contiguous;
//   xc   fp32 values for the exact score chains: per chunk [plane][d/8 groups][32 blocks][8],
//        so a wave reading coordinates 8g .. 8g+7 of its 32 blocks reads 1 KiB contiguous.
// Both private copies are 256-byte aligned; chunks past n are padding.
struct SummaryLayout {
  size_t plane;      // elements of one [B, n, Hkv, d] plane
  int nplanes;       // 1 (kmean) or 2 (kmin, kmax)
  size_t vn;         // float offset of vnorm (valid when output-aware)
  size_t kn;         // float offset of knorm
  size_t dn;         // float offset of dnorm
  int ncb;           // 32-block chunks per (batch, kv head)
  size_t bfc_byte;   // byte offset of the bf16 chunk-major copy
  size_t bfc_chunk;  // bf16 elements per (batch, kv head, chunk)
  size_t xc_byte;    // byte offset of the fp32 chunk-major copy
  size_t xc_chunk;   // floats per (batch, kv head, chunk)
  size_t bytes;      // total
};
inline SummaryLayout summary_layout(const Dims& D) {
  SummaryLayout L;
  L.plane = (size_t)D.B * D.n * D.Hkv * D.d;
  L.nplanes = D.score_mode == SA_KMINMAX ? 2 : 1;
  const size_t blocks = (size_t)D.B * D.n * D.Hkv;
  L.vn = L.plane * L.nplanes;
  L.kn = L.vn + (D.oam ? blocks : 0);
  L.dn = L.kn + blocks;
  L.ncb = (D.n + 31) / 32;
  const size_t chunks = (size_t)D.B * D.Hkv * L.ncb;
  L.bfc_chunk = (size_t)L.nplanes * D.d * 32;  // [plane][d/16][64][8]
  L.xc_chunk = (size_t)L.nplanes * D.d * 32;       // [plane][d/8][32][8]
  L.bfc_byte = ((L.dn + blocks) * sizeof(float) + 255) & ~(size_t)255;
  L.xc_byte = (L.bfc_byte + chunks * L.bfc_chunk * sizeof(uint16_t) + 255) & ~(size_t)255;
  L.bytes = L.xc_byte + chunks * L.xc_chunk * sizeof(float);
  return L;
}

// Maps a workgroup id to (b, h, t).  Logical order: (batch, kv head) outermost, then tiles
// latest first (late tiles carry the most blocks), then the q heads of the kv head.  The
// hardware deals consecutive ids to the 8 XCDs in turn, so at any moment every XCD works on the
// same kv head's nearby tiles: the blocks they share are then fetched once into the last-level
// cache that all XCDs see, rather than each XCD streaming a different head.  (Giving each XCD
// its own kv head instead was measured slower: the concurrent working set of 8 heads does not
// fit in that cache.)
__device__ __forceinline__ void decode_tile(const Dims& dm, int& b, int& h, int& t) {
  const int id = (int)blockIdx.x;
  const int per_pair = dm.nt * dm.G;  // tiles x q heads of one (batch, kv head)
  const int pair = id / per_pair;
  const int rest = id - pair * per_pair;
  t = dm.nt - 1 - rest / dm.G;
  const int r = rest - (rest / dm.G) * dm.G;
  b = pair / dm.Hkv;
  h = (pair - b * dm.Hkv) * dm.G + r;
}

// decode_tile over selection units instead of query heads: u is the unit (the query head,
// or the kv head when one list serves all of a kv head's query heads).
__device__ __forceinline__ void decode_unit(const Dims& dm, int& b, int& u, int& t) {
  const int id = (int)blockIdx.x;
  const int Gu = dm.G / dm.gs;  // units per kv head
  const int per_pair = dm.nt * Gu;
  const int pair = id / per_pair;
  const int rest = id - pair * per_pair;
  t = dm.nt - 1 - rest / Gu;
  const int r = rest - (rest / Gu) * Gu;
  b = pair / dm.Hkv;
  u = (pair - b * dm.Hkv) * Gu + r;
}

// The attention kernel's order: as decode_tile, but the G query heads of one tile are dealt
// to the same XCD (consecutive tiles still go to consecutive XCDs).  Those G workgroups run
// together and read the same kv head; with their lists ordered so that blocks shared by
// more heads come first, they request the shared blocks at the same steps and all but the
// first find them in that XCD's L2.  Falls back to decode_tile's order when the counts do
// not divide evenly.
__device__ __forceinline__ void decode_tile_grouped(const Dims& dm, int& b, int& h, int& t) {
  const int U = dm.B * dm.Hq * dm.nt;
  const int p = (int)blockIdx.x;
  int id = p;
  if (U % (8 * dm.G) == 0) {
    const int x = p & 7, y = p >> 3;
    const int z = y / dm.G, hq = y - z * dm.G;
    id = (8 * z + x) * dm.G + hq;
  }
  const int per_pair = dm.nt * dm.G;
  const int pair = id / per_pair;
  const int rest = id - pair * per_pair;
  t = dm.nt - 1 - rest / dm.G;
  const int r = rest - (rest / dm.G) * dm.G;
  b = pair / dm.Hkv;
  h = (pair - b * dm.Hkv) * dm.G + r;
}

// Dynamic LDS of the kernels whose need grows with the problem.  The host checks these
// against kMaxDynLds before any launch (a CU has 160 KiB of LDS; the margin covers each
// kernel's static LDS), so an oversized problem is refused, never launched.
constexpr size_t kMaxDynLds = 160 * 1024 - 4096;
inline size_t pow2_ceil(size_t x) {
  size_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
// Selection's score-and-rank kernels.  fp32: one 64-bit order key per block (score bits,
// then the block index), rounded up to a power of two for the sort.  bf16: the tile's Q rows
// staged as bf16 (two planes for the K-min/K-max bound, rows padded by 8 elements) after the
// keys; the keys are 32-bit (score bits only: a key's block index is its position) whenever
// the Q area can hold the 64-bit keys the final sort needs (2 pow2_ceil(ranked entries) of
// them), else 64-bit as for fp32.  Halving the keys keeps long sequences at two or three
// workgroups per CU (at 2^20 tokens, 8192 blocks: 32 instead of 64 KiB of keys).
inline size_t score_q_lds(const Dims& D) {
  const size_t npl = D.score_mode == SA_KMINMAX ? 2 : 1;
  return sizeof(uint16_t) * npl * D.T * (D.d + 8);
}
inline bool score_keys_compact(const Dims& D, const BudgetDev& bd) {
  if (D.dtype != SA_BF16) return false;
  size_t rn = (size_t)(bd.R > bd.k_max + 1 ? bd.R : bd.k_max + 1);
  if (rn > (size_t)D.n) rn = (size_t)D.n;
  return 2 * pow2_ceil(rn) * sizeof(unsigned long long) <= score_q_lds(D);
}
inline size_t score_keys_lds(const Dims& D, const BudgetDev& bd) {
  const size_t p = pow2_ceil((size_t)D.n);
  return score_keys_compact(D, bd) ? (sizeof(unsigned) * p + 15) / 16 * 16
                                   : sizeof(unsigned long long) * p;
}
// Threshold pruning of the bf16 selection (select.hip): a tile prunes when it has at least
// kPruneRatio times as many free blocks as keys it ranks; survivors are listed kPruneListCap
// positions at a time (uint16 each, after the keys).  Offered for compact keys and one query
// head per unit, when some tile can qualify (its ranked keys are at least
// max(floor(rho k_min), k_min + 1)) and the list fits the LDS.
constexpr int kPruneRatio = 16;
constexpr int kPruneListCap = 4096;
inline bool score_prune_ok(const Dims& D, const BudgetDev& bd) {
  if (!score_keys_compact(D, bd) || D.gs != 1) return false;
  const long long ex = (long long)floor(bd.rho * (double)bd.k_min);
  const long long rn = ex > bd.k_min + 1 ? ex : bd.k_min + 1;
  if ((long long)D.n < (long long)kPruneRatio * rn) return false;
  return score_keys_lds(D, bd) + sizeof(uint16_t) * kPruneListCap + score_q_lds(D) <=
         kMaxDynLds;
}
inline size_t score_rank_lds(const Dims& D, const BudgetDev& bd) {
  return score_keys_lds(D, bd) + (score_prune_ok(D, bd) ? sizeof(uint16_t) * kPruneListCap : 0) +
         (D.dtype == SA_BF16 ? score_q_lds(D) : 0);
}
// Gate kernel: sigma_bar of every tile, then a power-of-two sort buffer.
inline size_t gate_lds(const Dims& D) {
  return sizeof(float) * ((size_t)D.nt + pow2_ceil((size_t)D.nt));
}
// value_norms: the L2 norm of every (row, kv head) of one block.
inline size_t value_norms_lds(const Dims& D) { return sizeof(float) * (size_t)D.blk * D.Hkv; }

// Workspace layout of sparse_attn_select (byte offsets, 256-byte aligned).
struct SelectWs {
  size_t ranked, sigma, sigma_bar, gate, tau, total;
};
SelectWs select_ws_layout(const Dims& D, const BudgetDev& bd);

// ------------------------------------------------------------------ launchers

// Raises a kernel's dynamic-LDS limit when it needs more than the default 64 KiB.
template <typename K>
inline hipError_t allow_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_pool(const Dims& D, const void* K, const void* V, float* summ,
                       hipStream_t s);
hipError_t launch_select(const Dims& D, const BudgetDev& bd, const void* Q, const float* summ,
                         char* ws, int32_t* kv_idx, int32_t* kv_cnt, float* sigma,
                         float* sigma_bar, uint8_t* gate, float* tau, hipStream_t s);
// Mean of the finite entries of tau[0 .. B) (fp32 sum in index order, one IEEE division by
// their count), or -inf if none is finite; one thread.
hipError_t launch_tau_mean(const float* tau, int B, float* out, hipStream_t s);
// Vertical-slash index of the forward pass (per query head: vertical key blocks, ascending;
// slash block offsets, ascending; each list ends at its first negative entry).
struct VsIndex {
  const int32_t* vert = nullptr;
  const int32_t* slash = nullptr;
  int nv = 0, ns = 0;
};
constexpr int kVsMaxEntries = 511;  // nv + ns: the merged list plus the diagonal fit in LDS

// Workspace of the bf16 forward pass (byte offsets, 256-byte aligned): the fp16 V^T step
// images (the size of V), the partial maxima of |V| (kVmaxParts per batch and kv head,
// uint32), and each (batch, kv head)'s power-of-two exponent (int32).
constexpr int kVmaxParts = 64;  // partial maxima of |V| per (batch, kv head)
struct ForwardWs {
  size_t vp, part, vexp, total;
};
inline ForwardWs forward_ws_layout(const Dims& D) {
  auto a256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  ForwardWs w;
  w.vp = 0;
  w.part = a256((size_t)D.B * D.N * D.Hkv * D.d * sizeof(uint16_t));
  w.vexp = a256(w.part + (size_t)D.B * D.Hkv * kVmaxParts * sizeof(uint32_t));
  w.total = a256(w.vexp + (size_t)D.B * D.Hkv * sizeof(int32_t));
  return w;
}
inline size_t forward_ws_bytes(const Dims& D) {
  return D.dtype == SA_BF16 ? forward_ws_layout(D).total : 0;
}
hipError_t launch_prepare_values(const Dims& D, const void* V, void* ws, hipStream_t s);
hipError_t launch_forward_prepared(const Dims& D, const void* Q, const void* K, const void* ws,
                                   const int32_t* kv_idx, const int32_t* kv_cnt, int W,
                                   float scale, void* O, int out_dtype, float* lse,
                                   hipStream_t s);
hipError_t launch_forward(const Dims& D, const void* Q, const void* K, const void* V,
                          const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                          void* ws, void* O, int out_dtype, float* lse, hipStream_t s);
hipError_t launch_forward_vs(const Dims& D, const void* Q, const void* K, const void* V,
                             const VsIndex& vs, float scale, void* ws, void* O, int out_dtype,
                             float* lse, hipStream_t s);

// Decode with run-time termination (decode.hip): blocks of 64 keys, probe of the first
// kArtProbe output coordinates, at most kArtMaxHeadsPerKv query heads per kv head.
constexpr int kArtProbe = 16;
constexpr int kArtMaxHeadsPerKv = 4;
hipError_t launch_decode_art(const Dims& D, const void* Q, const void* K, const void* V,
                             float scale, float tau, float phi, int patience, void* O,
                             int out_dtype, int32_t* done, hipStream_t s);

}  // namespace sa
