// Block selection for block-sparse causal prefill: tile scores, top-k, cut margin, quantile
// gate, expansion and sentinel-padded lists.
//
// "Uncertainty-Gated Selection for Block-Sparse Attention" page, Metodologia:
//   step 2  per query tile, a block's score is the maximum over the tile's query rows; a
//           top-k over blocks gives the initial kv_idx;
//   step 3  the normalised cut margin sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k)) over the
//           sorted scores, per tile and head;
//   step 4  sigma averaged over heads and compared with a per-layer empirical quantile q;
//   step 5  tiles that trip keep the top floor(rho * k) blocks, the others k, and the lists
//           are padded with sentinels so every tile has the same shape.
// Stem page, Metodologia A: the budget k_t may decay linearly with the tile's position, and
// early blocks act as anchors (here: n_sink blocks always kept).
//
// Selection runs per (batch, unit, tile): the unit is a query head, or a kv head whose query
// heads share one list (the tile score then being the maximum over all of their rows).  A
// tile of 128 rows over 64-key blocks has two diagonal blocks, both forced.
//
// Three stream-ordered launches, no host synchronisation:
//   score_rank  one workgroup per (b, unit, t), tiles launched latest-first (they carry the most
//               blocks).  One wave per 64 query rows; lane = query row, with the row held in
//               registers as fp32.  Each block summary is read by the whole wave at one
//               uniform address (scalar loads), so every fused multiply-add takes one operand
//               from a scalar register and the row scores run as independent per-lane
//               chains in coordinate order.  The wave's maximum over rows goes to LDS as an
//               order-preserving 64-bit key (score, then lower index first), merged across
//               the tile's waves with an LDS atomic max, then sorted by a bitonic network.
//   gate        one workgroup per batch element: mean over units, eligible count, the
//               quantile's order statistic (bitonic sort of the eligible sigma_bar), gate bits.
//   emit        one wave per (b, unit, t): forced blocks and the kept ranked blocks marked in
//               an LDS bitmap, then written out in ascending order with a wave prefix sum.
//
// The arithmetic that decides selections is IEEE fp32 with a fixed order (compiled without
// contraction): row score = fused multiply-add chain over coordinates in order, starting at
// +0; tile score = maximum over rows, with -0 mapped to +0, times the value norm when the
// score is output-aware; sigma = two subtractions and a correctly rounded division;
// sigma_bar = sum over units in order divided by their count; the quantile rank
// ceil(q * M) in fp64.

#include <type_traits>

#include "common.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int budget_at(const BudgetDev& bd, int t, int n) {
  if (bd.kind == SA_K_CONST) return bd.k_max;
  const long long k = (long long)bd.k_max * (n - t) / n;
  return k > bd.k_min ? (int)k : bd.k_min;
}
// Free blocks of tile t: the blocks before its diagonal ones, minus the sinks.
__device__ __forceinline__ int n_free(const BudgetDev& bd, int t) {
  const int d0 = first_diag(bd.m, bd.tpb, t);
  return d0 - (d0 < bd.n_sink ? d0 : bd.n_sink);
}
__device__ __forceinline__ int expanded(const BudgetDev& bd, int k) {
  return (int)floor(bd.rho * (double)k);
}
__device__ __forceinline__ int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// LDS scratch of the radix selections below (one per workgroup, reused).
struct RadixLds {
  unsigned int hist[256];
  unsigned long long prefix;
  int need, done;
  unsigned int cnt;
};

// Bitonic sort of P (a power of two) 64-bit keys in LDS, descending, by NT threads.
template <int NT>
__device__ void bitonic_desc(unsigned long long* keys, int P) {
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < (P >> 1); i += NT) {
        const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
        const int hi = lo + jj;
        const unsigned long long a = keys[lo], b = keys[hi];
        const bool desc = (lo & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          keys[lo] = b;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// The Rn largest of the nf distinct 64-bit keys key_at(0 .. nf), sorted descending, by NT
// threads.  A radix select over 8-bit digits from the top finds the Rn-th largest key (a
// 256-bin LDS histogram per digit); the keys at or above it, exactly Rn of them, are gathered
// into `small` and only those are sorted.  When that would not shrink the sort at least
// fourfold, all P keys are sorted instead: in place when `inplace` holds them as 64-bit keys
// (inplace[nf .. P) = 0), else copied into `small`, which the caller sizes for that (P <=
// small_cap whenever the radix path is not taken).  Returns where the sorted top keys are.
// Every thread of the workgroup must call it.
template <int NT, typename KeyAt>
__device__ const unsigned long long* top_desc(KeyAt key_at, unsigned long long* inplace, int nf,
                                              int P, int Rn, unsigned long long* small,
                                              int small_cap, RadixLds& rl) {
  unsigned int* hist = rl.hist;
  unsigned long long& s_prefix = rl.prefix;
  int& s_need = rl.need;
  int& s_done = rl.done;
  unsigned int& s_cnt = rl.cnt;
  int P2 = 1;
  while (P2 < Rn) P2 <<= 1;
  if (nf <= Rn || 4 * P2 > P || P2 > small_cap) {
    if (inplace) {
      bitonic_desc<NT>(inplace, P);
      return inplace;
    }
    for (int f = threadIdx.x; f < P; f += NT) small[f] = f < nf ? key_at(f) : 0ull;
    __syncthreads();
    bitonic_desc<NT>(small, P);
    return small;
  }
  unsigned long long prefix = 0ull;
  int need = Rn, shift = 56;
  for (;;) {
    for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0u;
    __syncthreads();
    const int hs = shift + 8;  // the digits above this one must match the prefix
    for (int f = threadIdx.x; f < nf; f += NT) {
      const unsigned long long key = key_at(f);
      if (hs == 64 || (key >> hs) == (prefix >> hs))
        atomicAdd(&hist[(unsigned)(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds digits 255 - 4l .. 252 - 4l; `above` counts the keys with a larger digit
      const int lane = threadIdx.x;
      unsigned c[4], tot = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        tot += c[e];
      }
      unsigned incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      unsigned above = incl - tot;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < (unsigned)need && above + c[e] >= (unsigned)need) {
          s_prefix = prefix | ((unsigned long long)(255 - 4 * lane - e) << shift);
          s_need = need - (int)above;
          // done when this digit's whole bucket lies within the top Rn
          s_done = above + c[e] == (unsigned)need || shift == 0;
        }
        above += c[e];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    if (s_done) break;
    shift -= 8;
  }
  // exactly Rn keys have (key >> shift) >= (prefix >> shift)
  if (threadIdx.x == 0) s_cnt = 0u;
  for (int i = threadIdx.x; i < P2; i += NT) small[i] = 0ull;
  __syncthreads();
  for (int f = threadIdx.x; f < nf; f += NT) {
    const unsigned long long key = key_at(f);
    if ((key >> shift) >= (prefix >> shift)) small[atomicAdd(&s_cnt, 1u)] = key;
  }
  __syncthreads();
  bitonic_desc<NT>(small, P2);
  return small;
}

// A threshold u with at least Rn of the 32-bit keys k[0 .. nf) at or above it (Rn <= nf), as
// large as two histogram passes find: the keys' range [lo, hi] is cut into 256 bins of 2^s
// keys; the bin holding the Rn-th largest key is cut again into 256, and u is the lower edge
// of the bin holding it there.  (Binning the range spreads the keys over the bins, where an
// 8-bit digit of keys that share their top bits would send them all to one bin.)  Every
// thread must call it.
template <int NT>
__device__ unsigned rank_threshold_u32(const unsigned* k, int nf, int Rn, RadixLds& rl) {
  unsigned lo = 0xffffffffu, hi = 0u;
  for (int f = threadIdx.x; f < nf; f += NT) {
    lo = min(lo, k[f]);
    hi = max(hi, k[f]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (unsigned)__shfl_xor((int)lo, off));
    hi = max(hi, (unsigned)__shfl_xor((int)hi, off));
  }
  if (threadIdx.x == 0) {
    rl.prefix = 0xffffffffull;  // low word: running minimum, high word: running maximum
    rl.need = Rn;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    atomicMin(reinterpret_cast<unsigned*>(&rl.prefix), lo);
    atomicMax(reinterpret_cast<unsigned*>(&rl.prefix) + 1, hi);
  }
  __syncthreads();
  lo = (unsigned)rl.prefix;
  hi = (unsigned)(rl.prefix >> 32);
  int need = Rn;
  for (int pass = 0; pass < 2; ++pass) {
    const unsigned span = hi - lo;
    const int s = span >> 8 ? 32 - __builtin_clz(span >> 8) : 0;  // (hi - lo) >> s < 256
    for (int i = threadIdx.x; i < 256; i += NT) rl.hist[i] = 0u;
    __syncthreads();
    for (int f = threadIdx.x; f < nf; f += NT) {
      const unsigned key = k[f];
      if (key >= lo && key <= hi) atomicAdd(&rl.hist[(key - lo) >> s], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 255 - 4l .. 252 - 4l; `above` counts the keys in higher bins
      const int lane = threadIdx.x;
      unsigned c[4], tot = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = rl.hist[255 - 4 * lane - e];
        tot += c[e];
      }
      unsigned incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      unsigned above = incl - tot;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < (unsigned)need && above + c[e] >= (unsigned)need) {
          rl.cnt = (unsigned)(255 - 4 * lane - e);
          rl.need = need - (int)above;
        }
        above += c[e];
      }
    }
    __syncthreads();
    const unsigned bin = rl.cnt;
    need = rl.need;
    const unsigned new_lo = lo + (bin << s);
    hi = (unsigned)min((unsigned long long)hi, (unsigned long long)new_lo + (1ull << s) - 1ull);
    lo = new_lo;
    __syncthreads();  // every thread has read rl before the next pass rewrites it
    if (s == 0) break;
  }
  return lo;
}

template <typename T, int D>
struct QRow;
template <int D>
struct QRow<uint16_t, D> {
  __device__ __forceinline__ static void load(const uint16_t* p, float* q) {
#pragma unroll
    for (int c = 0; c < D; c += 8) {
      uint4 v = *reinterpret_cast<const uint4*>(p + c);
      q[c + 0] = bf16_lo(v.x); q[c + 1] = bf16_hi(v.x);
      q[c + 2] = bf16_lo(v.y); q[c + 3] = bf16_hi(v.y);
      q[c + 4] = bf16_lo(v.z); q[c + 5] = bf16_hi(v.z);
      q[c + 6] = bf16_lo(v.w); q[c + 7] = bf16_hi(v.w);
    }
  }
};
template <int D>
struct QRow<float, D> {
  __device__ __forceinline__ static void load(const float* p, float* q) {
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float4 v = *reinterpret_cast<const float4*>(p + c);
      q[c] = v.x; q[c + 1] = v.y; q[c + 2] = v.z; q[c + 3] = v.w;
    }
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Output-aware tile score from the canonical tile score m and the block's mean value-row norm
// v.  Product form: m * v.  Additive form (Stem page, Metodologia B: the score plus
// beta * max(0, log ||V_j||^2)): the score on the logit scale, fmaf(m, 1/sqrt(d), bonus),
// with bonus = beta * max(0, ln v^2) evaluated in fp64 and rounded once to fp32.
template <int OAM>
__device__ __forceinline__ float oam_combine(float m, float v, const Dims& dm) {
  if (OAM == SA_OAM_PRODUCT) return canon(m * v);
  if (OAM == SA_OAM_ADDITIVE) {
    const double l = log((double)v * (double)v);
    const float bonus = (float)((double)dm.oam_beta * (l > 0.0 ? l : 0.0));
    return canon(__builtin_fmaf(m, dm.oam_scale, bonus));
  }
  return m;
}

// ----------------------------------------------------------------------- score_rank

template <typename T, int MODE, int OAM, int D, int TILE>
__global__ __launch_bounds__(TILE) void score_rank(Dims dm, BudgetDev bd,
                                                   const T* __restrict__ Q,
                                                   const float* __restrict__ summ,
                                                   int* __restrict__ ranked,
                                                   float* __restrict__ sigma) {
  extern __shared__ unsigned long long keys[];
  constexpr int NT = TILE;  // one lane per query row
  const int n = dm.n, nt = dm.nt;  // blocks, tiles
  const int BH = dm.B * dm.Hu;  // (batch, selection unit) pairs
  const int t = nt - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / dm.Hu, u = bh - b * dm.Hu;
  const int g = u * dm.gs / dm.G;
  const size_t bht = (size_t)bh * nt + t;

  const int kt = budget_at(bd, t, nt);
  const int nf = n_free(bd, t);
  if (nf <= kt) {  // not eligible: every free block is kept, nothing to rank
    if (threadIdx.x == 0) sigma[bht] = 1.0f;
    return;
  }
  const int d0 = first_diag(bd.m, bd.tpb, t);      // first diagonal block
  const int j0 = d0 < bd.n_sink ? d0 : bd.n_sink;  // first free block
  const int P = next_pow2(nf);
  for (int f = threadIdx.x; f < P; f += NT)
    keys[f] = f < nf ? (unsigned long long)(0xffffffffu - (unsigned)(j0 + f)) : 0ull;
  __syncthreads();

  const int row = t * TILE + threadIdx.x;
  const size_t plane = (size_t)dm.B * n * dm.Hkv * D;
  const float* kbase = summ + (((size_t)b * n) * dm.Hkv + g) * D;
  const size_t kstride = (size_t)dm.Hkv * D;
  const float* vn = summ + plane * (MODE == SA_KMINMAX ? 2 : 1) + ((size_t)b * n) * dm.Hkv + g;
  const bool lead = (threadIdx.x & 63) == 0;

  // The unit's query heads in turn; a block's key keeps the maximum over all of their rows
  // (the output-aware combine and the order key are monotone, so the maximum commutes).
  for (int h = u * dm.gs; h < (u + 1) * dm.gs; ++h) {
  float q[D];
  QRow<T, D>::load(Q + (((size_t)b * dm.N + row) * dm.Hq + h) * D, q);
  for (int j = j0; j < d0; ++j) {
    const float* kb = kbase + (size_t)j * kstride;
    float s = 0.0f;
    if (MODE == SA_KMEAN) {
#pragma unroll
      for (int c = 0; c < D; ++c) s = __builtin_fmaf(q[c], kb[c], s);
    } else {
      const float* kx = kb + plane;
#pragma unroll
      for (int c = 0; c < D; ++c) s = __builtin_fmaf(q[c], q[c] >= 0.0f ? kx[c] : kb[c], s);
    }
    float m = canon(wave_max(s));
    m = oam_combine<OAM>(m, OAM ? vn[(size_t)j * dm.Hkv] : 0.0f, dm);
    if (lead) {
      const unsigned long long key =
          ((unsigned long long)order_key(m) << 32) | (0xffffffffu - (unsigned)j);
      atomicMax(&keys[j - j0], key);
    }
  }
  }
  __syncthreads();
  bitonic_desc<NT>(keys, P);

  const int R = min(max(expanded(bd, kt), kt), nf);
  int* out = ranked + bht * bd.R;
  for (int r = threadIdx.x; r < R; r += NT) out[r] = (int)(0xffffffffu - (unsigned)keys[r]);
  if (threadIdx.x == 0) {
    const float s0 = order_key_inv((unsigned)(keys[0] >> 32));
    const float sk1 = order_key_inv((unsigned)(keys[kt - 1] >> 32));
    const float sk = order_key_inv((unsigned)(keys[kt] >> 32));
    const float num = sk1 - sk;
    const float den = s0 - sk;
    sigma[bht] = den == 0.0f ? 0.0f : __fdiv_rn(num, den);
  }
}

// ------------------------------------------------------------- score_rank (bf16 inputs)
//
// Same canonical scores as score_rank, computed where they matter.  For a block j the tile
// score is max_i s_ij over the tile's rows; only the row that attains it needs the canonical
// fp32 chain.  A matrix-core pass computes approximate scores for every (row, block):
//   shat_ij = q_i . bf16(x_j)   (bf16 MFMA, fp32 accumulation; bf16(x) is the fp32 summary
//                                 rounded to nearest, r_j = x_j - bf16(x_j) its residual)
// with |shat_ij - s_ij| <= E_j.  The rounding moves the product by |q_i . r_j|, at most
// |q_i| |r_j| (Cauchy-Schwarz; for the bound backbone the residual takes per coordinate the
// larger of the two planes'); the products q_c bf16(x_c) are exact in fp32, and the MFMA's
// accumulation and the canonical chain's own rounding each stay below d 2^-24 sum_c |q_c x_c|
// <= 2^-17 |q_i| |x_j| for d <= 128.  So E_j = max_i |q_i| (1.001 |r_j| + 2^-12 |x_j|), where
// the factor 1.001 and the 2^-12 (far above 2 x 2^-17) absorb the fp32 rounding of the
// norms themselves.  The row attaining
// max_i s_ij then satisfies shat_ij >= max_i shat_ij - 2 E_j, so recomputing the canonical
// chain for exactly those rows and taking their maximum gives the canonical tile score.
// Usually one row per block qualifies, so the fp32 chain work falls by about the tile height.
//
// One workgroup (4 waves) per (b, unit, t); a unit of several query heads takes one pass per
// head, each block keeping its largest score.  The tile's Q rows are staged in LDS as bf16 (for
// the bound backbone as its positive and negative parts, so q+ . kmax + q- . kmin gives
// the per-coordinate maximum); each wave takes aligned 32-block chunks covering the free
// blocks, holds a 32-block x all-rows score tile in accumulators (lane = block, 16 rows per
// 32-row tile), finds each block's candidate rows lane-locally, runs their canonical chains
// (q from LDS, the fp32 summary from L2) and writes the block's order key.  Both the bf16
// operands and the fp32 summaries come from the chunk-major copies the summary kernel writes
// (common.h), so every one of these loads reads 1 KiB contiguous instead of 16-32 bytes from
// each of 32 blocks.

constexpr int kScoreThreads = 256;
constexpr float kResidualC = 1.001f;   // |q . r| <= |q| |r|, with the norms' own rounding
constexpr float kAccumC = 0x1p-12f;    // MFMA accumulation plus canonical chain rounding

// Threshold pruning for long rows of free blocks.  Only the top Rn = max(R, k + 1) order keys
// are ever read, so a block that provably ranks below Rn others needs no canonical score.  A
// first pass runs the prefilter alone: it brackets every block's (combined) tile score between
// LB_j = combine(M_j - E_j) and UB_j = combine(M_j + E_j) (M_j the largest approximate row
// score; combine is the monotone output-aware step or the identity) and keeps UB_j as the
// block's key.  With U a value that at least Rn of the UB_j reach (rank_threshold_u32 finds it
// at or just below the Rn-th largest) and D the largest UB_j - LB_j, at least Rn blocks have
// an exact score >= U - D >= T, so every block with UB_j < T ranks strictly below them and
// is dropped (key 0, below every real key); the surviving blocks get their canonical scores as
// usual (a second prefilter over lists of 32 survivors, then the candidate rows' chains), and
// the ranking over those keys is the ranking of the full row.  The rounding of M +- E is covered
// by E's margin (kAccumC is 16 times the accumulation bound); D and T are widened by 2^-22
// relative.  Used when a tile has at least kPruneRatio * Rn free blocks (where the survivors
// are few; near-tied rows simply keep more of them) and one query head per selection unit
// (common.h, score_prune_ok).
constexpr int kListCap = kPruneListCap;  // survivors gathered per round (positions, uint16)

// GRP: selection units of several query heads (one list per kv head).  A separate
// instantiation, because the loop over the unit's heads costs the one-head case registers.
// PRUNE: the threshold pruning above may run (compact keys, GRP false; the survivor list sits
// after the keys).  Also separate: its extra state costs the other instantiations registers.
template <int MODE, int OAM, int D, int TILE, bool GRP, bool PRUNE>
// Three waves per SIMD (at most 168 registers): as many workgroups as the LDS allows (three
// per CU), measured 23% faster than the compiler's default of two waves per SIMD.
__global__ __launch_bounds__(kScoreThreads, 3) void score_rank_mfma(
    Dims dm, BudgetDev bd, const uint16_t* __restrict__ Q, const float* __restrict__ summ,
    const uint16_t* __restrict__ bfc, const float* __restrict__ xc, int* __restrict__ ranked,
    float* __restrict__ sigma, size_t vn_off, size_t kn_off, size_t dn_off, int ncb,
    int compact) {
  static_assert(!(GRP && PRUNE), "pruning serves one query head per unit");
  constexpr int NPL = MODE == SA_KMINMAX ? 2 : 1;  // staged Q planes (q, or q+ and q-)
  constexpr int QS = D + 8;                        // LDS row stride (bf16 elements)
  constexpr int RT = TILE / 32;                    // 32-row tiles
  constexpr int KS = D / 16;                       // 16-coordinate MFMA steps
  extern __shared__ __attribute__((aligned(16))) unsigned long long keys[];
  __shared__ float qmax_w[kScoreThreads / 64];
  __shared__ RadixLds rl;
  __shared__ unsigned s_dmax;

  int b, u, t;
  decode_unit(dm, b, u, t);
  const int n = dm.n;  // blocks
  const int g = u * dm.gs / dm.G;
  const size_t bht = ((size_t)b * dm.Hu + u) * dm.nt + t;
  const int kt = budget_at(bd, t, dm.nt);
  const int nf = n_free(bd, t);
  if (nf <= kt) {
    if (threadIdx.x == 0) sigma[bht] = 1.0f;
    return;
  }
  const int d0 = first_diag(bd.m, bd.tpb, t);  // first diagonal block: free ones [j0, d0)
  const int j0 = d0 < bd.n_sink ? d0 : bd.n_sink;
  int P = 1;
  while (P < nf) P <<= 1;
  int Palloc = 1;
  while (Palloc < n) Palloc <<= 1;
  const int R = min(max(expanded(bd, kt), kt), nf);  // ranked entries written
  const int Rn = min(max(R, kt + 1), nf);            // keys read (key kt gives sigma)
  const bool prune = PRUNE && compact && nf >= kPruneRatio * Rn;
  // Keys: 64-bit (score bits, then 0xffffffff - block), or with `compact` only the 32-bit
  // score part, the block being j0 + the key's position.  Then, with PRUNE, the survivor
  // list; then the Q rows.
  unsigned* kq = reinterpret_cast<unsigned*>(keys);
  char* after_keys = compact ? reinterpret_cast<char*>(keys) + (4 * Palloc + 15) / 16 * 16
                             : reinterpret_cast<char*>(keys + Palloc);
  uint16_t* list = reinterpret_cast<uint16_t*>(after_keys);  // [kListCap]
  uint16_t* qs = reinterpret_cast<uint16_t*>(
      after_keys + (PRUNE ? kListCap * sizeof(uint16_t) : 0));  // [NPL][TILE][QS]

  for (int f = threadIdx.x; f < P; f += kScoreThreads) {
    if (compact)
      kq[f] = 0u;
    else
      keys[f] = f < nf ? (unsigned long long)(0xffffffffu - (unsigned)(j0 + f)) : 0ull;
  }
  if (threadIdx.x == 0) s_dmax = 0u;

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  // Blocks of this (batch, kv head) in 32-block chunks: block j sits in chunk j / 32 at slot
  // j % 32 of the chunk-major copies.
  const size_t chunk0 = ((size_t)b * dm.Hkv + g) * ncb;
  constexpr size_t BFC = (size_t)NPL * D * 32, XC = (size_t)NPL * D * 32;
  float qmax = 0.0f;

  // Approximate scores of the tile's rows against the lane pair's block j = 32 c + sl (bf16
  // MFMA; c is uniform over the wave when it walks whole chunks, which keeps the chunk's base
  // address scalar).  Lane (l32, hi) gets rows 32rt + 8i + 4hi + r of its block.
  auto approx = [&](int c, int sl, f32x16 (&acc)[RT]) {
    const uint16_t* bc = bfc + (chunk0 + c) * BFC + (sl + 32 * hi) * 8;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = (f32x16){};
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) {
      // q . x with x = kmean; or q+ . kmax + q- . kmin (kmax is plane 1, kmin plane 0)
      const int xp = MODE == SA_KMINMAX ? 1 - pl : 0;
      const uint16_t* bh_ = bc + (size_t)xp * (KS * 512);
      const uint16_t* ap = qs + (size_t)(pl * TILE + l32) * QS + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bhv = *reinterpret_cast<const bf16x8*>(bh_ + 512 * ks);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(ap + rt * 32 * QS + 16 * ks);
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bhv, acc[rt], 0, 0, 0);
        }
      }
    }
  };
  // Prefilter error bound of block j (valid lanes).
  auto err_bound = [&](int j, bool valid) {
    const size_t bj = ((size_t)b * n + j) * dm.Hkv + g;
    const float kn = valid ? summ[kn_off + bj] : 0.0f;
    const float dn = valid ? summ[dn_off + bj] : 0.0f;
    return qmax * (kResidualC * dn + kAccumC * kn);
  };
  auto value_norm = [&](int j) {
    return OAM ? summ[vn_off + ((size_t)b * n + j) * dm.Hkv + g] : 0.0f;
  };

  // Canonical chain of query row `row` against the bound backbone's block whose fp32 planes
  // start at xk (kmin plane 0, kmax plane 1, chunk-major): x_c = (q_c >= 0 ? kmax_c : kmin_c),
  // one fused multiply-add per coordinate in order.
  auto chain_bound = [&](const float* xk, int row) -> float {
    const uint16_t* qr = qs + (size_t)row * QS;
    const uint16_t* qn = qs + (size_t)(TILE + row) * QS;
    float sv = 0.0f;
#pragma unroll 2
    for (int c0 = 0; c0 < D; c0 += 8) {
      uint4 qv = *reinterpret_cast<const uint4*>(qr + c0);
      const uint4 q2 = *reinterpret_cast<const uint4*>(qn + c0);
      qv.x |= q2.x; qv.y |= q2.y; qv.z |= q2.z; qv.w |= q2.w;
      const float4 x0 = *reinterpret_cast<const float4*>(xk + (c0 / 8) * 256);
      const float4 x1 = *reinterpret_cast<const float4*>(xk + (c0 / 8) * 256 + 4);
      const float4 y0 = *reinterpret_cast<const float4*>(xk + (D / 8 + c0 / 8) * 256);
      const float4 y1 = *reinterpret_cast<const float4*>(xk + (D / 8 + c0 / 8) * 256 + 4);
      const float q8[8] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y),
                           bf16_lo(qv.z), bf16_hi(qv.z), bf16_lo(qv.w), bf16_hi(qv.w)};
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float xb[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) sv = __builtin_fmaf(q8[k], q8[k] >= 0.0f ? xb[k] : xa[k], sv);
    }
    return sv;
  };
  // Canonical chain of query row `row` against the mean-pooled block whose fp32 summary starts
  // at xk (chunk-major): one fused multiply-add per coordinate in order.
  auto chain_mean = [&](const float* xk, int row) -> float {
    const uint16_t* qr = qs + (size_t)row * QS;
    float sv = 0.0f;
#pragma unroll 2
    for (int c0 = 0; c0 < D; c0 += 8) {
      const uint4 qv = *reinterpret_cast<const uint4*>(qr + c0);
      const float4 x0 = *reinterpret_cast<const float4*>(xk + (c0 / 8) * 256);
      const float4 x1 = *reinterpret_cast<const float4*>(xk + (c0 / 8) * 256 + 4);
      const float q8[8] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y),
                           bf16_lo(qv.z), bf16_hi(qv.z), bf16_lo(qv.w), bf16_hi(qv.w)};
      const float xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int k = 0; k < 8; ++k) sv = __builtin_fmaf(q8[k], xa[k], sv);
    }
    return sv;
  };
  // The order key of block j = 32 c + sl's canonical (combined) tile score, on lanes hi == 0
  // of valid blocks: the prefilter's candidate rows, then their canonical fp32 chains.
  auto exact_key = [&](int c, int sl, bool valid) -> unsigned {
    const int j = 32 * c + sl;
    // kmean, or kmin (plane 0) / kmax (plane 1): coordinates 8c .. 8c+7 of this lane's block
    // at xk + (plane * D/8 + c) * 256
    const float* xk = xc + (chunk0 + c) * XC + sl * 8;
    // Mean-pooled backbone: this lane's half of the block's fp32 summary (coordinates
    // D/2 * hi .. +D/2), requested now so it arrives while the matrix products run.
    float xh[MODE == SA_KMEAN ? D / 2 : 1];
    if constexpr (MODE == SA_KMEAN) {
#pragma unroll
      for (int c8 = 0; c8 < D / 16; ++c8) {
        const float4 x0 = *reinterpret_cast<const float4*>(xk + (hi * (D / 16) + c8) * 256);
        const float4 x1 = *reinterpret_cast<const float4*>(xk + (hi * (D / 16) + c8) * 256 + 4);
        xh[8 * c8 + 0] = x0.x; xh[8 * c8 + 1] = x0.y; xh[8 * c8 + 2] = x0.z; xh[8 * c8 + 3] = x0.w;
        xh[8 * c8 + 4] = x1.x; xh[8 * c8 + 5] = x1.y; xh[8 * c8 + 6] = x1.z; xh[8 * c8 + 7] = x1.w;
      }
    }
    f32x16 acc[RT];
    approx(c, sl, acc);
    float mloc = -INFINITY;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, acc[rt][v]);
    const float M = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float thr = M - 2.0f * err_bound(j, valid);
    unsigned long long cand = 0ull;
    if (valid) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (acc[rt][v] >= thr) cand |= 1ull << (rt * 16 + v);
    }
    // Canonical chains of the candidate rows.
    float best = -INFINITY;
    if constexpr (MODE == SA_KMEAN) {
      // The two lanes of block j run each candidate's chain as a two-stage pipeline: lane
      // hi = 0 does coordinates 0 .. D/2-1 of candidate k while lane hi = 1 finishes
      // coordinates D/2 .. D-1 of candidate k-1 from the partial sum handed over by
      // v_permlane32_swap.  Same fused multiply-adds in the same order as one lane's chain.
      // The pair's candidates are lane 0's rows, then lane 1's.
      // v_permlane32_swap(x, x): the first result holds the partner's value in lanes 32-63,
      // the second in lanes 0-31.
      const auto swl = __builtin_amdgcn_permlane32_swap((unsigned)cand, (unsigned)cand, false,
                                                        false);
      const auto swh = __builtin_amdgcn_permlane32_swap((unsigned)(cand >> 32),
                                                        (unsigned)(cand >> 32), false, false);
      const unsigned long long other =
          ((unsigned long long)(hi ? swh[0] : swh[1]) << 32) | (unsigned)(hi ? swl[0] : swl[1]);
      const unsigned long long c0m = hi ? other : cand;  // lane 0's candidates
      const unsigned long long c1m = hi ? cand : other;  // lane 1's candidates
      const int n0 = __builtin_popcountll(c0m), ncand = n0 + __builtin_popcountll(c1m);
      unsigned long long rem0 = c0m, rem1 = c1m;
      int prow = 0;        // row whose second half this lane (hi = 1) finishes next
      float part = 0.0f;   // partial sum handed from lane 0 to lane 1
      for (int k = 0; k <= ncand; ++k) {
        // row of candidate k (lane 0 starts it) and of candidate k-1 (lane 1 finishes it)
        int row = 0;
        if (k < ncand) {
          unsigned long long& rm = k < n0 ? rem0 : rem1;
          const int bit = __builtin_ctzll(rm);
          rm &= rm - 1;
          row = 32 * (bit >> 4) + 8 * ((bit & 15) >> 2) + 4 * (k < n0 ? 0 : 1) + (bit & 3);
        }
        const int r_here = hi ? prow : row;
        const bool active = hi ? (k >= 1) : (k < ncand);
        float sv = hi ? part : 0.0f;
        if (active) {
          const uint16_t* qr = qs + (size_t)r_here * QS + hi * (D / 2);
#pragma unroll
          for (int c0 = 0; c0 < D / 2; c0 += 8) {
            const uint4 qv = *reinterpret_cast<const uint4*>(qr + c0);
            const float q8[8] = {bf16_lo(qv.x), bf16_hi(qv.x), bf16_lo(qv.y), bf16_hi(qv.y),
                                 bf16_lo(qv.z), bf16_hi(qv.z), bf16_lo(qv.w), bf16_hi(qv.w)};
#pragma unroll
            for (int e = 0; e < 8; ++e) sv = __builtin_fmaf(q8[e], xh[c0 + e], sv);
          }
          if (hi) best = fmaxf(best, sv);
        }
        // hand lane 0's partial to lane 1; lane 1 remembers the row it belongs to
        const auto ps = __builtin_amdgcn_permlane32_swap(__float_as_uint(sv),
                                                         __float_as_uint(sv), false, false);
        part = __uint_as_float(hi ? ps[0] : ps[1]);  // lane 1 receives lane 0's partial
        prow = row;
      }
      (void)prow;
    } else {
    while (cand) {
      const int bit = __builtin_ctzll(cand);
      cand &= cand - 1;
      const int row = 32 * (bit >> 4) + 8 * ((bit & 15) >> 2) + 4 * hi + (bit & 3);
      best = fmaxf(best, chain_bound(xk, row));
    }
    }
    best = fmaxf(best, __shfl_xor(best, 32));
    unsigned key = 0u;
    if (valid && hi == 0) key = order_key(oam_combine<OAM>(canon(best), value_norm(j), dm));
    return key;
  };

  // The unit's query heads in turn (one pass per head).  Each free block's key holds the
  // largest tile score over the passes so far: the output-aware combine and the order key are
  // monotone, so the maximum over all of the unit's rows is exact.
  const int h_end = GRP ? (u + 1) * dm.gs : u + 1;
  for (int h = GRP ? u * dm.gs : u; h < h_end; ++h) {
  __syncthreads();  // the previous pass has finished reading qs and qmax_w

  // Stage the tile's Q rows; row norms (any order: they only scale the bound) -> max.  Each
  // thread takes a contiguous piece of one row (PPR pieces per row, all loads issued at
  // once), so a row's sum of squares needs only PPR - 1 neighbouring-lane exchanges.
  {
    constexpr int EPT = TILE * D / kScoreThreads;  // elements per thread
    constexpr int NV = EPT / 8;                    // 16-byte loads per thread
    constexpr int PPR = D / EPT;                   // threads per row
    static_assert(PPR == 2 || PPR == 4, "row pieces must pair within a lane quad");
    const int r = threadIdx.x / PPR, piece = threadIdx.x % PPR;
    const uint16_t* qsrc =
        Q + (((size_t)b * dm.N + (size_t)t * TILE + r) * dm.Hq + h) * D + piece * EPT;
    uint4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = *reinterpret_cast<const uint4*>(qsrc + 8 * i);
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float lo = bf16_lo(w[k]), hi = bf16_hi(w[k]);
        ss = __builtin_fmaf(lo, lo, ss);
        ss = __builtin_fmaf(hi, hi, ss);
      }
      uint16_t* dst = qs + r * QS + piece * EPT + 8 * i;
      if (MODE == SA_KMEAN) {
        *reinterpret_cast<uint4*>(dst) = v[i];
      } else {
        uint32_t pw[4], nw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t neg = ((w[k] >> 15) & 0x00010001u) * 0xffffu;  // negative halves
          pw[k] = w[k] & ~neg;
          nw[k] = w[k] & neg;
        }
        *reinterpret_cast<uint4*>(dst) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        *reinterpret_cast<uint4*>(dst + TILE * QS) = make_uint4(nw[0], nw[1], nw[2], nw[3]);
      }
    }
#pragma unroll
    for (int off = 1; off < PPR; off <<= 1) ss += __shfl_xor(ss, off);
    float rmax = ss;
#pragma unroll
    for (int off = PPR; off < 64; off <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, off));
    if ((threadIdx.x & 63) == 0) qmax_w[threadIdx.x >> 6] = rmax;
  }
  __syncthreads();
  float qmax2 = qmax_w[0];
#pragma unroll
  for (int k = 1; k < kScoreThreads / 64; ++k) qmax2 = fmaxf(qmax2, qmax_w[k]);
  // uniform over the workgroup: kept in a scalar register
  qmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(__builtin_sqrtf(qmax2))));

  if constexpr (!PRUNE && !GRP) {
    // Pairs of aligned 32-block chunks covering [j0, d0), dealt to the waves.  Both lanes of a
    // block hold half of its rows' approximate scores, and nearly every block has a single
    // candidate row, so one chunk at a time would leave one lane of each pair idle through the
    // canonical chains.  With two chunks per pass, lane hi = 0 runs the chains of its block in
    // the first chunk and lane hi = 1 those of its block in the second, each over the
    // candidate rows of both halves (the same rows and the same chains as one chunk at a time).
    using Mask = std::conditional_t<RT <= 2, unsigned, unsigned long long>;
    auto partner = [&](Mask m) -> Mask {  // the value of lane l ^ 32 (v_permlane32_swap)
      const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)m, (unsigned)m, false, false);
      const unsigned plo = hi ? lo[0] : lo[1];
      if constexpr (RT <= 2) {
        return plo;
      } else {
        const unsigned mh = (unsigned)(m >> 32);
        const auto up = __builtin_amdgcn_permlane32_swap(mh, mh, false, false);
        return ((unsigned long long)(hi ? up[0] : up[1]) << 32) | plo;
      }
    };
    for (int ch = (j0 >> 5) + 2 * wv; ch * 32 < d0; ch += 2 * (kScoreThreads / 64)) {
      const bool has_b = (ch + 1) * 32 < d0;  // wave-uniform: the second chunk has free blocks
      // Candidate rows of chunk c's block l32 among this lane's half (bit 16 rt + v: row
      // 32 rt + 8 (v >> 2) + 4 hi + (v & 3)).
      auto cand_mask = [&](int c) -> Mask {
        const int jj = 32 * c + l32;
        const bool vv = jj >= j0 && jj < d0;
        f32x16 acc[RT];
        approx(c, l32, acc);
        float mloc = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, acc[rt][v]);
        const float M = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float thr = M - 2.0f * err_bound(jj, vv);
        Mask m = 0;
        if (vv) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (acc[rt][v] >= thr) m |= (Mask)1 << (rt * 16 + v);
        }
        return m;
      };
      const Mask ma = cand_mask(ch);
      __builtin_amdgcn_sched_barrier(0);
      const Mask mb = has_b ? cand_mask(ch + 1) : (Mask)0;
      __builtin_amdgcn_sched_barrier(0);
      const Mask pa = partner(ma), pb = partner(mb);
      Mask r0 = hi ? pb : ma;  // this lane's block: candidates among the rows of half 0
      Mask r1 = hi ? mb : pa;  // and of half 1
      const int cm = ch + hi;
      const int j = 32 * cm + l32;
      const bool valid = j >= j0 && j < d0;
      const float* xk = xc + (chunk0 + cm) * XC + l32 * 8;
      float best = -INFINITY;
      while (r0 | r1) {
        int bit, half;
        if (r0) {
          bit = (int)__builtin_ctzll((unsigned long long)r0);
          r0 &= r0 - 1;
          half = 0;
        } else {
          bit = (int)__builtin_ctzll((unsigned long long)r1);
          r1 &= r1 - 1;
          half = 1;
        }
        const int row = 32 * (bit >> 4) + 8 * ((bit & 15) >> 2) + 4 * half + (bit & 3);
        if constexpr (MODE == SA_KMINMAX)
          best = fmaxf(best, chain_bound(xk, row));
        else
          best = fmaxf(best, chain_mean(xk, row));
      }
      if (valid) {
        const unsigned ok = order_key(oam_combine<OAM>(canon(best), value_norm(j), dm));
        if (compact) {
          kq[j - j0] = ok;
        } else {
          keys[j - j0] = ((unsigned long long)ok << 32) | (0xffffffffu - (unsigned)j);
        }
      }
    }
  } else if constexpr (!PRUNE) {
    // Every free block: aligned 32-block chunks covering [j0, d0), dealt to the waves.
    for (int ch = (j0 >> 5) + wv; ch * 32 < d0; ch += kScoreThreads / 64) {
      const int j = ch * 32 + l32;  // this lane's block
      const bool valid = j >= j0 && j < d0;
      const unsigned ok = exact_key(ch, l32, valid);
      if (valid && hi == 0) {
        // one lane per block and pass, passes separated by barriers: a plain maximum (the
        // block part of a 64-bit key is the same in every pass)
        if (compact) {
          kq[j - j0] = ok > kq[j - j0] ? ok : kq[j - j0];
        } else {
          const unsigned long long key =
              ((unsigned long long)ok << 32) | (0xffffffffu - (unsigned)j);
          keys[j - j0] = key > keys[j - j0] ? key : keys[j - j0];
        }
      }
    }
  } else {
    if constexpr (PRUNE) {
      if (prune) {
        // First pass of the pruning: the prefilter alone, UB_j as the key, max of UB_j - LB_j.
        // The next chunk's operands are requested while this chunk's products run.
        constexpr int NB = NPL * KS;
        auto load_ops = [&](int c, bf16x8 (&bo)[NB]) {
          const uint16_t* bc = bfc + (chunk0 + c) * BFC + (l32 + 32 * hi) * 8;
#pragma unroll
          for (int pl = 0; pl < NPL; ++pl) {
            const int xp = MODE == SA_KMINMAX ? 1 - pl : 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              bo[pl * KS + ks] =
                  *reinterpret_cast<const bf16x8*>(bc + (size_t)xp * (KS * 512) + 512 * ks);
          }
        };
        float dmax = 0.0f;
        bf16x8 bnext[NB];
        int ch = (j0 >> 5) + wv;
        if (ch * 32 < d0) load_ops(ch, bnext);
        for (; ch * 32 < d0; ch += kScoreThreads / 64) {
          const int j = ch * 32 + l32;
          const bool valid = j >= j0 && j < d0;
          bf16x8 bcur[NB];
#pragma unroll
          for (int i = 0; i < NB; ++i) bcur[i] = bnext[i];
          if ((ch + kScoreThreads / 64) * 32 < d0) load_ops(ch + kScoreThreads / 64, bnext);
          const size_t bj = ((size_t)b * n + (valid ? j : j0)) * dm.Hkv + g;
          const float kn = summ[kn_off + bj], dn = summ[dn_off + bj];
          const float vn = OAM ? summ[vn_off + bj] : 0.0f;
          // Products in (plane, 16-coordinate step) order, each step's four row tiles
          // together; the next step's Q fragments are read from LDS before this step's
          // products, and the order is pinned so that the reads stay ahead.
          f32x16 acc[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = (f32x16){};
          const uint16_t* ap = qs + (size_t)l32 * QS + 8 * hi;
          auto a_frag = [&](int i, int rt) {
            return *reinterpret_cast<const bf16x8*>(ap + (size_t)((i / KS) * TILE + rt * 32) * QS +
                                                    16 * (i % KS));
          };
          bf16x8 acur[RT], anxt[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acur[rt] = a_frag(0, rt);
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            if (i + 1 < NB) {
#pragma unroll
              for (int rt = 0; rt < RT; ++rt) anxt[rt] = a_frag(i + 1, rt);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(acur[rt], bcur[i], acc[rt], 0, 0, 0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acur[rt] = anxt[rt];
            __builtin_amdgcn_sched_barrier(0);
          }
          float mloc = -INFINITY;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, acc[rt][v]);
          const float M = fmaxf(mloc, __shfl_xor(mloc, 32));
          if (valid && hi == 0) {
            const float E = qmax * (kResidualC * dn + kAccumC * kn);
            const float ub = oam_combine<OAM>(canon(M + E), vn, dm);
            const float lb = oam_combine<OAM>(canon(M - E), vn, dm);
            kq[j - j0] = order_key(ub);
            dmax = fmaxf(dmax, ub - lb);
          }
        }
        dmax = wave_max(dmax);
        if (lane == 0) atomicMax(&s_dmax, __float_as_uint(dmax));  // >= 0: bits order as values
        __syncthreads();
      }
    }
    // Blocks to score exactly: without pruning every free block, in aligned 32-block chunks
    // covering [j0, d0) dealt to the waves (one round); with it the survivors of each round of
    // kListCap positions, listed, 32 per wave pass (the others' keys become 0).  A listed
    // position is read and written by one thread of the scan, then by the lane that scores it,
    // after a barrier.
    unsigned Tk = 0u;
    if constexpr (PRUNE) {
      if (prune) {
        const float U = order_key_inv(rank_threshold_u32<kScoreThreads>(kq, nf, Rn, rl));
        const float dm_ = __uint_as_float(s_dmax) * (1.0f + 0x1p-22f);
        float T = U - dm_;
        T = T - fabsf(T) * 0x1p-22f;
        Tk = order_key(T);
      }
    }
    for (int base = 0; base < (prune ? nf : 1); base += kListCap) {
      int items = ((d0 + 31) >> 5) - (j0 >> 5);  // chunks
      if (prune) {
        const int end = min(nf, base + kListCap);
        if (threadIdx.x == 0) rl.cnt = 0u;
        __syncthreads();
        for (int f = base + (int)threadIdx.x; f < end; f += kScoreThreads) {
          if (kq[f] >= Tk)
            list[atomicAdd(&rl.cnt, 1u)] = (uint16_t)(f - base);
          else
            kq[f] = 0u;
        }
        __syncthreads();
        items = ((int)rl.cnt + 31) >> 5;
      }
      const int cnt = prune ? (int)rl.cnt : 0;
      for (int it = wv; it < items; it += kScoreThreads / 64) {
        int j;
        bool valid;
        if (prune) {
          valid = 32 * it + l32 < cnt;
          j = j0 + base + (valid ? (int)list[32 * it + l32] : 0);
        } else {
          j = ((j0 >> 5) + it) * 32 + l32;  // this lane's block
          valid = j >= j0 && j < d0;
        }
        const unsigned ok = exact_key(j >> 5, j & 31, valid);
        if (valid && hi == 0) {
          // one lane per block and pass, passes separated by barriers: a plain maximum (the
          // block part of a 64-bit key is the same in every pass)
          if (compact) {
            kq[j - j0] = prune || ok > kq[j - j0] ? ok : kq[j - j0];
          } else {
            const unsigned long long key =
                ((unsigned long long)ok << 32) | (0xffffffffu - (unsigned)j);
            keys[j - j0] = key > keys[j - j0] ? key : keys[j - j0];
          }
        }
      }
      if (prune) __syncthreads();  // the list is rebuilt by the next round
    }
  }
  }
  __syncthreads();
  // Only the top R keys (and key kt, for sigma) are used: select them, then sort those.  The
  // Q staging area is free by now and holds the selected keys.
  const auto key_at = [&](int f) -> unsigned long long {
    return compact ? ((unsigned long long)kq[f] << 32) | (0xffffffffu - (unsigned)(j0 + f))
                   : keys[f];
  };
  unsigned long long* small = reinterpret_cast<unsigned long long*>(qs);
  const int small_cap = NPL * TILE * QS * (int)sizeof(uint16_t) / (int)sizeof(unsigned long long);
  const unsigned long long* top = nullptr;
  if constexpr (PRUNE) {
    if (prune) {
      // The survivors' keys (the only nonzero ones) gathered into the list area as 64-bit
      // keys, when they fit, so that the ranking reads those alone.
      constexpr int kSurvCap = kListCap * (int)sizeof(uint16_t) / (int)sizeof(unsigned long long);
      unsigned long long* surv = reinterpret_cast<unsigned long long*>(list);
      if (threadIdx.x == 0) rl.cnt = 0u;
      __syncthreads();
      for (int f = threadIdx.x; f < nf; f += kScoreThreads) {
        if (kq[f]) {
          const unsigned slot = atomicAdd(&rl.cnt, 1u);
          if (slot < (unsigned)kSurvCap) surv[slot] = key_at(f);
        }
      }
      __syncthreads();
      const int S = (int)rl.cnt;
      if (S <= kSurvCap) {
        int PS = 1;
        while (PS < S) PS <<= 1;
        for (int f = S + (int)threadIdx.x; f < PS; f += kScoreThreads) surv[f] = 0ull;
        __syncthreads();
        top = top_desc<kScoreThreads>([&](int f) { return surv[f]; }, surv, S, PS, Rn, small,
                                      small_cap, rl);
      }
    }
  }
  if (!top)
    top = top_desc<kScoreThreads>(key_at, compact ? nullptr : keys, nf, P, Rn, small,
                                  small_cap, rl);
  int* out = ranked + bht * bd.R;
  for (int r = threadIdx.x; r < R; r += kScoreThreads)
    out[r] = (int)(0xffffffffu - (unsigned)top[r]);
  if (threadIdx.x == 0) {
    const float s0 = order_key_inv((unsigned)(top[0] >> 32));
    const float sk1 = order_key_inv((unsigned)(top[kt - 1] >> 32));
    const float sk = order_key_inv((unsigned)(top[kt] >> 32));
    const float num = sk1 - sk;
    const float den = s0 - sk;
    sigma[bht] = den == 0.0f ? 0.0f : __fdiv_rn(num, den);
  }
}

// ----------------------------------------------------------------------------- gate

constexpr int kGateThreads = 1024;

__global__ __launch_bounds__(kGateThreads) void gate_kernel(Dims dm, BudgetDev bd,
                                                            const float* __restrict__ sigma,
                                                            float* __restrict__ sigma_bar,
                                                            uint8_t* __restrict__ gate,
                                                            float* __restrict__ tau) {
  extern __shared__ float gsh[];  // sbar[n], then sort buffer [P]
  __shared__ int M;
  const int n = dm.nt, b = blockIdx.x;  // tiles
  float* sbar = gsh;
  float* buf = gsh + n;
  if (threadIdx.x == 0) M = 0;
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += kGateThreads) {
    float acc = 0.0f;
    for (int u = 0; u < dm.Hu; ++u) acc = acc + sigma[((size_t)b * dm.Hu + u) * n + t];
    const float sb = __fdiv_rn(acc, (float)dm.Hu);
    sbar[t] = sb;
    sigma_bar[(size_t)b * n + t] = sb;
    if (n_free(bd, t) > budget_at(bd, t, n)) buf[atomicAdd(&M, 1)] = sb;
  }
  __syncthreads();
  const int m = M;
  float tb = -INFINITY;
  if (bd.gate_mode == SA_GATE_QUANTILE) {
    const int P = next_pow2(m > 0 ? m : 1);
    for (int i = m + threadIdx.x; i < P; i += kGateThreads) buf[i] = INFINITY;
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = threadIdx.x; i < (P >> 1); i += kGateThreads) {
          const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
          const int hi = lo + jj;
          const float a = buf[lo], c = buf[hi];
          const bool asc = (lo & k) == 0;
          if (asc ? (a > c) : (a < c)) {
            buf[lo] = c;
            buf[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    double rq = ceil(bd.q * (double)m);
    const int r = rq < 0.0 ? 0 : (rq > (double)m ? m : (int)rq);
    if (r > 0) tb = buf[r - 1];
  } else if (bd.gate_mode == SA_GATE_FIXED) {
    tb = bd.tau_fixed;
  }
  for (int t = threadIdx.x; t < n; t += kGateThreads) {
    const bool elig = n_free(bd, t) > budget_at(bd, t, n);
    gate[(size_t)b * n + t] =
        (uint8_t)(bd.gate_mode != SA_GATE_OFF && elig && sbar[t] <= tb);
  }
  if (threadIdx.x == 0) tau[b] = tb;
}

// ----------------------------------------------------------------------------- emit

constexpr int kEmitWaves = 4;

__global__ __launch_bounds__(64 * kEmitWaves) void emit_kernel(Dims dm, BudgetDev bd,
                                                               const int* __restrict__ ranked,
                                                               const uint8_t* __restrict__ gate,
                                                               int32_t* __restrict__ kv_idx,
                                                               int32_t* __restrict__ kv_cnt) {
  extern __shared__ unsigned int bits[];  // [kEmitWaves][nwords]
  const int n = dm.nt;                 // tiles
  const int nwords = (dm.n + 31) >> 5;  // bitmap words over the blocks
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t item = (size_t)blockIdx.x * kEmitWaves + w;
  const size_t total = (size_t)dm.B * dm.Hu * n;
  const bool live = item < total;
  const int t = live ? (int)(item % n) : 0;
  const int b = live ? (int)(item / ((size_t)dm.Hu * n)) : 0;
  unsigned int* bm = bits + w * nwords;

  const int kt = budget_at(bd, t, n);
  const int nf = n_free(bd, t);
  const bool elig = live && nf > kt;
  const int d0 = first_diag(bd.m, bd.tpb, t), dend = d0 + bd.m;  // diagonal blocks [d0, dend)
  int keep = 0;
  if (elig) {
    const bool tripped = gate[(size_t)b * n + t] != 0;
    keep = min(tripped ? expanded(bd, kt) : kt, nf);
    for (int i = lane; i <= ((dend - 1) >> 5); i += 64) bm[i] = 0u;
  }
  __syncthreads();
  if (elig) {
    const int* rk = ranked + item * bd.R;
    for (int e = lane; e < keep; e += 64) {
      const int j = rk[e];
      atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
    if (lane < bd.m) atomicOr(&bm[(d0 + lane) >> 5], 1u << ((d0 + lane) & 31));
    for (int j = lane; j < bd.n_sink; j += 64) atomicOr(&bm[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (!live) return;
  int32_t* out = kv_idx + item * bd.W;
  int cnt;
  if (!elig) {  // every causal block 0 .. dend-1 is kept
    cnt = dend;
    for (int e = lane; e < cnt; e += 64) out[e] = e;
  } else {
    const int nw = ((dend - 1) >> 5) + 1;
    int base = 0;
    for (int w0 = 0; w0 < nw; w0 += 64) {
      const unsigned int word = (w0 + lane < nw) ? bm[w0 + lane] : 0u;
      const int pc = __popc(word);
      int incl = pc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      int pos = base + incl - pc;
      unsigned int rest = word;
      while (rest) {
        const int bit = __ffs(rest) - 1;
        rest &= rest - 1;
        out[pos++] = ((w0 + lane) << 5) + bit;
      }
      base += __shfl(incl, 63);
    }
    cnt = base;
  }
  for (int e = cnt + lane; e < bd.W; e += 64) out[e] = -1;
  if (lane == 0) kv_cnt[item] = cnt;
}

template <typename T, int MODE, int OAM, int D, int TILE>
hipError_t launch_score(const Dims& dm, const BudgetDev& bd, const void* Q, const float* summ,
                        int* ranked, float* sigma, hipStream_t s) {
  const size_t lds = score_rank_lds(dm, bd);
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hu * dm.nt);
  hipError_t e = allow_lds(score_rank<T, MODE, OAM, D, TILE>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_rank<T, MODE, OAM, D, TILE>), dim3(grid), dim3(TILE), lds, s, dm,
                     bd, static_cast<const T*>(Q), summ, ranked, sigma);
  return hipGetLastError();
}

template <typename T, int MODE, int OAM>
hipError_t score_by_shape(const Dims& dm, const BudgetDev& bd, const void* Q, const float* summ,
                          int* ranked, float* sigma, hipStream_t s) {
  if (dm.d == 64)
    return dm.T == 64 ? launch_score<T, MODE, OAM, 64, 64>(dm, bd, Q, summ, ranked, sigma, s)
                        : launch_score<T, MODE, OAM, 64, 128>(dm, bd, Q, summ, ranked, sigma, s);
  return dm.T == 64 ? launch_score<T, MODE, OAM, 128, 64>(dm, bd, Q, summ, ranked, sigma, s)
                      : launch_score<T, MODE, OAM, 128, 128>(dm, bd, Q, summ, ranked, sigma, s);
}

template <typename T, int MODE>
hipError_t score_by_oam(const Dims& dm, const BudgetDev& bd, const void* Q, const float* summ,
                        int* ranked, float* sigma, hipStream_t s) {
  if (dm.oam == SA_OAM_PRODUCT)
    return score_by_shape<T, MODE, SA_OAM_PRODUCT>(dm, bd, Q, summ, ranked, sigma, s);
  if (dm.oam == SA_OAM_ADDITIVE)
    return score_by_shape<T, MODE, SA_OAM_ADDITIVE>(dm, bd, Q, summ, ranked, sigma, s);
  return score_by_shape<T, MODE, SA_OAM_OFF>(dm, bd, Q, summ, ranked, sigma, s);
}

template <typename T>
hipError_t score_dispatch(const Dims& dm, const BudgetDev& bd, const void* Q, const float* summ,
                          int* ranked, float* sigma, hipStream_t s) {
  if (dm.score_mode == SA_KMEAN)
    return score_by_oam<T, SA_KMEAN>(dm, bd, Q, summ, ranked, sigma, s);
  return score_by_oam<T, SA_KMINMAX>(dm, bd, Q, summ, ranked, sigma, s);
}

template <int MODE, int OAM, int D, int TILE, bool GRP, bool PRUNE>
hipError_t launch_score_mfma_g(const Dims& dm, const BudgetDev& bd, const void* Q,
                             const float* summ, int* ranked, float* sigma, hipStream_t s) {
  const SummaryLayout L = summary_layout(dm);
  const size_t lds = score_rank_lds(dm, bd);
  hipError_t e = allow_lds(score_rank_mfma<MODE, OAM, D, TILE, GRP, PRUNE>, lds);
  if (e != hipSuccess) return e;
  const char* base = reinterpret_cast<const char*>(summ);
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hu * dm.nt);
  hipLaunchKernelGGL((score_rank_mfma<MODE, OAM, D, TILE, GRP, PRUNE>), dim3(grid), dim3(kScoreThreads),
                     lds, s, dm, bd, static_cast<const uint16_t*>(Q), summ,
                     reinterpret_cast<const uint16_t*>(base + L.bfc_byte),
                     reinterpret_cast<const float*>(base + L.xc_byte), ranked, sigma, L.vn, L.kn,
                     L.dn, L.ncb, score_keys_compact(dm, bd) ? 1 : 0);
  return hipGetLastError();
}

template <int MODE, int OAM, int D, int TILE>
hipError_t launch_score_mfma(const Dims& dm, const BudgetDev& bd, const void* Q,
                             const float* summ, int* ranked, float* sigma, hipStream_t s) {
  if (dm.gs > 1)
    return launch_score_mfma_g<MODE, OAM, D, TILE, true, false>(dm, bd, Q, summ, ranked, sigma, s);
  if (score_prune_ok(dm, bd))
    return launch_score_mfma_g<MODE, OAM, D, TILE, false, true>(dm, bd, Q, summ, ranked, sigma, s);
  return launch_score_mfma_g<MODE, OAM, D, TILE, false, false>(dm, bd, Q, summ, ranked, sigma, s);
}

template <int MODE, int OAM>
hipError_t score_mfma_shape(const Dims& dm, const BudgetDev& bd, const void* Q,
                            const float* summ, int* ranked, float* sigma, hipStream_t s) {
  if (dm.d == 64)
    return dm.T == 64 ? launch_score_mfma<MODE, OAM, 64, 64>(dm, bd, Q, summ, ranked, sigma, s)
                        : launch_score_mfma<MODE, OAM, 64, 128>(dm, bd, Q, summ, ranked, sigma, s);
  return dm.T == 64 ? launch_score_mfma<MODE, OAM, 128, 64>(dm, bd, Q, summ, ranked, sigma, s)
                      : launch_score_mfma<MODE, OAM, 128, 128>(dm, bd, Q, summ, ranked, sigma, s);
}

template <int MODE>
hipError_t score_mfma_oam(const Dims& dm, const BudgetDev& bd, const void* Q,
                          const float* summ, int* ranked, float* sigma, hipStream_t s) {
  if (dm.oam == SA_OAM_PRODUCT)
    return score_mfma_shape<MODE, SA_OAM_PRODUCT>(dm, bd, Q, summ, ranked, sigma, s);
  if (dm.oam == SA_OAM_ADDITIVE)
    return score_mfma_shape<MODE, SA_OAM_ADDITIVE>(dm, bd, Q, summ, ranked, sigma, s);
  return score_mfma_shape<MODE, SA_OAM_OFF>(dm, bd, Q, summ, ranked, sigma, s);
}

hipError_t score_mfma_dispatch(const Dims& dm, const BudgetDev& bd, const void* Q,
                               const float* summ, int* ranked, float* sigma, hipStream_t s) {
  if (dm.score_mode == SA_KMEAN)
    return score_mfma_oam<SA_KMEAN>(dm, bd, Q, summ, ranked, sigma, s);
  return score_mfma_oam<SA_KMINMAX>(dm, bd, Q, summ, ranked, sigma, s);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A fixed gate threshold from the per-sequence quantile thresholds of calibration inputs:
// their mean over the sequences where a tile can trip (a finite tau).
__global__ void tau_mean_kernel(const float* __restrict__ tau, int B, float* __restrict__ out) {
  if (threadIdx.x != 0) return;
  float acc = 0.0f;
  int c = 0;
  for (int b = 0; b < B; ++b) {
    const float x = tau[b];
    if (isfinite(x)) {
      acc = acc + x;
      ++c;
    }
  }
  *out = c > 0 ? acc / (float)c : -INFINITY;
}

}  // namespace

hipError_t launch_tau_mean(const float* tau, int B, float* out, hipStream_t s) {
  hipLaunchKernelGGL(tau_mean_kernel, dim3(1), dim3(64), 0, s, tau, B, out);
  return hipGetLastError();
}

SelectWs select_ws_layout(const Dims& dm, const BudgetDev& bd) {
  SelectWs w;
  const size_t bhn = (size_t)dm.B * dm.Hu * dm.nt;
  w.ranked = 0;
  w.sigma = align256(w.ranked + sizeof(int) * bhn * bd.R);
  w.sigma_bar = align256(w.sigma + sizeof(float) * bhn);
  w.gate = align256(w.sigma_bar + sizeof(float) * (size_t)dm.B * dm.nt);
  w.tau = align256(w.gate + (size_t)dm.B * dm.nt);
  w.total = align256(w.tau + sizeof(float) * dm.B);
  return w;
}

hipError_t launch_select(const Dims& dm, const BudgetDev& bd, const void* Q, const float* summ,
                         char* ws, int32_t* kv_idx, int32_t* kv_cnt, float* sigma,
                         float* sigma_bar, uint8_t* gate, float* tau, hipStream_t s) {
  const SelectWs L = select_ws_layout(dm, bd);
  int* ranked = reinterpret_cast<int*>(ws + L.ranked);
  if (!sigma) sigma = reinterpret_cast<float*>(ws + L.sigma);
  if (!sigma_bar) sigma_bar = reinterpret_cast<float*>(ws + L.sigma_bar);
  if (!gate) gate = reinterpret_cast<uint8_t*>(ws + L.gate);
  if (!tau) tau = reinterpret_cast<float*>(ws + L.tau);

  hipError_t e = dm.dtype == SA_BF16 ? score_mfma_dispatch(dm, bd, Q, summ, ranked, sigma, s)
                                     : score_dispatch<float>(dm, bd, Q, summ, ranked, sigma, s);
  if (e != hipSuccess) return e;

  const size_t glds = gate_lds(dm);
  if ((e = allow_lds(gate_kernel, glds)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)dm.B), dim3(kGateThreads), glds, s, dm, bd,
                     sigma, sigma_bar, gate, tau);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  const size_t total = (size_t)dm.B * dm.Hu * dm.nt;
  const unsigned grid = (unsigned)((total + kEmitWaves - 1) / kEmitWaves);
  const size_t elds = sizeof(unsigned int) * kEmitWaves * (size_t)((dm.n + 31) / 32);
  hipLaunchKernelGGL(emit_kernel, dim3(grid), dim3(64 * kEmitWaves), elds, s, dm, bd, ranked,
                     gate, kv_idx, kv_cnt);
  return hipGetLastError();
}

}  // namespace sa
