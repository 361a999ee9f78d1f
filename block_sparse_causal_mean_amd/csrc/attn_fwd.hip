// Sparse attention over the selected KV blocks: a FlashAttention-style online-softmax pass.
//
// Stem page, implementation note: the method runs block-sparse attention kernels over the
// chosen blocks after block-level scoring; gated-selection page, Metodologia step 5: every
// tile's list has the same padded shape (sentinel -1).  ART page, section 2.4: the online
// softmax is invariant to the order of the KV blocks, and the causal mask is applied before
// accumulation.
//
// bf16 inputs (pack_v + attn_bf16):
//   pack_v      once per call, V [B, N, Hkv, d] bf16 -> fp16 blocks [B, Hkv, n, d, BLK]:
//               each block transposed (V^T, keys contiguous) and XOR-swizzled in 4-key
//               granules, i.e. exactly the LDS image attn_bf16 wants.  Each V block is read
//               by hundreds of tiles, so converting and transposing it once here takes that
//               work out of the attention loop.  bf16 -> fp16 is exact for |v| in
//               [2^-14, 65504]; smaller magnitudes keep an absolute error below 2^-25.
//   attn_bf16   one workgroup per (batch, q head, query tile): BLK/32 query groups of 32 rows
//               x 2 key halves, one wave each (two waves per SIMD).  Per listed block:
//               S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 coordinates from
//               LDS, B = the wave's Q fragment held in registers), so each lane's
//               accumulator holds logits of ONE query row: row max and sum are lane-local
//               plus one swap with the lane 32 apart, and P^T is already laid out as the B
//               operand of O^T += V^T P^T (v_mfma_f32_32x32x16_f16; the key index is
//               permuted consistently in the V^T operand instead of moving P through LDS).
//               K and V^T blocks go from global memory straight into LDS (global_load_lds,
//               no registers), double-buffered so the next block streams in while the
//               current one is computed, with one workgroup barrier per block.  Both LDS
//               images are XOR-swizzled so the operand reads are free of bank conflicts.
//               The two key halves of a query group keep separate online-softmax states and
//               merge once at the end.  fp32 accumulation throughout; P is rounded to fp16
//               (11 significant bits) for the second product.
// fp32 inputs (attn_f32): one thread per query row, fp32 VALU arithmetic, same online softmax.
//
// Launch order (decode_tile): one kv head's tiles, latest first, per XCD.

#include "common.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Index of the next usable list entry at or after e, or -1: the list ends at cnt or at the
// first negative entry; entries after the tile (j > t) are skipped.
__device__ __forceinline__ int next_entry(const int32_t* __restrict__ list, int cnt, int e,
                                          int t) {
  for (; e < cnt; ++e) {
    const int j = list[e];
    if (j < 0) return -1;
    if (j <= t) return e;
  }
  return -1;
}

// ------------------------------------------------------------------ swizzled block images
//
// K block in LDS: BLK rows of D bf16 (16-byte chunks); V^T block (LDS and the packed global
// copy): D rows of BLK fp16 (8-byte granules of 4 keys).  Within a row, chunk/granule c sits
// at c ^ key(row).  The keys make the 16 (b128 reads) or 32 (b64 reads) lanes of one LDS
// phase, which read the same column of consecutive rows, land on distinct banks: rows are
// 256 bytes (one full bank sweep) or 128 bytes (two rows per sweep) long.
template <int D>
__device__ __forceinline__ int k_key(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int k_chunk_pos(int r, int c) { return r * (D / 8) + (c ^ k_key<D>(r)); }
template <int BLK>
__device__ __forceinline__ int v_key(int d) { return BLK == 128 ? (d & 31) : ((d >> 1) & 15); }
template <int BLK>
__device__ __forceinline__ int v_gran_pos(int d, int g) {
  return d * (BLK / 4) + (g ^ v_key<BLK>(d));
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap, no LDS traffic).  The swap
// hands each lane its own value and its partner's, one in each result; both lanes of a pair
// combine the same two values, so they get bit-identical results.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------------ pack_v

constexpr int kPackThreads = 256;

template <int D, int BLK>
__global__ __launch_bounds__(kPackThreads) void pack_v(Dims dm, const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ Vp) {
  constexpr int RS = D + 2;  // LDS row stride (elements)
  __shared__ uint16_t sv[BLK * RS];
  const int id = (int)blockIdx.x;  // ((b * Hkv + g) * n + j)
  const int j = id % dm.n;
  const int bg = id / dm.n;
  const int g = bg % dm.Hkv, b = bg / dm.Hkv;
  const uint16_t* src = V + (((size_t)b * dm.N + (size_t)j * BLK) * dm.Hkv + g) * D;
  for (int c = threadIdx.x; c < BLK * D / 8; c += kPackThreads) {
    const int r = c / (D / 8), col = c - r * (D / 8);
    const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)r * dm.Hkv * D + col * 8);
    uint32_t* dst = reinterpret_cast<uint32_t*>(sv + r * RS + col * 8);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();
  uint2* out = reinterpret_cast<uint2*>(Vp + (size_t)id * D * BLK);
  for (int i = threadIdx.x; i < D * BLK / 4; i += kPackThreads) {
    const int d = i / (BLK / 4), p = i - d * (BLK / 4);
    const int gk = p ^ v_key<BLK>(d);  // granule stored at position p
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = bf16_bits_to_f32(sv[(4 * gk + k) * RS + d]);
    const f16x2 a = __builtin_convertvector((f32x2){x[0], x[1]}, f16x2);
    const f16x2 c = __builtin_convertvector((f32x2){x[2], x[3]}, f16x2);
    out[i] = make_uint2(*reinterpret_cast<const uint32_t*>(&a), *reinterpret_cast<const uint32_t*>(&c));
  }
}

// --------------------------------------------------------------------------- attn_bf16

template <int D, int BLK>
struct Tiles {
  static constexpr int QG = BLK / 32;          // query groups
  static constexpr int NW = QG * 2;            // waves
  static constexpr int NT = 64 * NW;           // threads (= 4 * BLK)
  static constexpr int HK = BLK / 2;           // keys per wave per block
  static constexpr int KT = HK / 32;           // 32-key tiles per wave per block
  static constexpr int CHUNKS = BLK * D / 8;   // 16-byte chunks of one K (or V^T) block
  static constexpr int LPT = CHUNKS / NT;      // direct loads per thread per block image
  static constexpr size_t IMG = (size_t)BLK * D * 2;  // bytes of one block image
  static constexpr size_t STAGE = 2 * IMG;            // K image + V^T image
  static constexpr size_t MERGE = sizeof(float) * (size_t)QG * 64 * (D / 32 * 16 + 2);
  static constexpr size_t LDS = 2 * STAGE > MERGE ? 2 * STAGE : MERGE;
  static_assert(CHUNKS % NT == 0, "load split");
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// Issues the direct global->LDS loads of block j's K and V^T images into one stage.
template <int D, int BLK>
__device__ __forceinline__ void issue_block(const uint16_t* __restrict__ Kg,
                                            const uint16_t* __restrict__ Vpg, int rstride,
                                            int j, char* stage) {
  using TL = Tiles<D, BLK>;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint16_t* kb = Kg + (size_t)j * BLK * rstride;
  const uint16_t* vb = Vpg + (size_t)j * D * BLK;
#pragma unroll
  for (int i = 0; i < TL::LPT; ++i) {
    const int region = wv + TL::NW * i;  // 64-chunk (1 KiB) LDS region
    const int P = region * 64 + lane;    // LDS chunk this lane fills
    const int r = P / (D / 8), pos = P - r * (D / 8);
    const int c = pos ^ k_key<D>(r);     // global chunk that belongs there
    __builtin_amdgcn_global_load_lds(kb + (size_t)r * rstride + c * 8,
                                     (lds_ptr)(stage + region * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + (size_t)P * 8,
                                     (lds_ptr)(stage + TL::IMG + region * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A row's running maximum is only raised when a new logit exceeds it by more than this many
// powers of two; until then probabilities may reach 2^kLazy, which fp16 P and the fp32
// accumulators hold exactly enough, and the rescale of O is skipped.
constexpr float kLazy = 8.0f;

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 4) void attn_bf16(  // BLK * 4 == Tiles<D, BLK>::NT
    Dims dm, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vp, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, int W, float scale_log2, void* __restrict__ O,
    int out_f32, float* __restrict__ lse) {
  using TL = Tiles<D, BLK>;
  constexpr int KT = TL::KT;
  constexpr int DT = D / 32;  // 32-coordinate tiles of the output
  constexpr int DC = D / 16;  // 16-coordinate chunks of the QK^T contraction
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  int b, h, t;
  decode_tile(dm, b, h, t);
  const int g = h / dm.G;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int qg = wv % TL::QG, kh = wv / TL::QG;  // query group, key half
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t bht = ((size_t)b * dm.Hq + h) * dm.n + t;
  const int32_t* list = kv_idx + bht * W;
  const int cnt = min(kv_cnt[bht], W);
  const int qloc = qg * 32 + l32;  // this lane's query row within the tile
  const int qrow = t * BLK + qloc;
  const int rstride = dm.Hkv * D;
  const uint16_t* Kg = K + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const uint16_t* Vpg = Vp + ((size_t)b * dm.Hkv + g) * dm.n * D * BLK;

  // Q fragment (B operand of S^T = K Q^T): lane holds coordinates 16c + 8*hi .. +7 of its row.
  bf16x8 qf[DC];
  {
    const uint16_t* qp = Q + (((size_t)b * dm.N + qrow) * dm.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < DC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  }

  f32x16 acc_o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) acc_o[i] = (f32x16){};
  float m_run = -INFINITY;  // running max of raw logits (before scaling) for this lane's row
  float l_run = 0.0f;       // this lane's share of the row's softmax denominator

  int e = next_entry(list, cnt, 0, t);
  int st = 0;
  if (e >= 0) issue_block<D, BLK>(Kg, Vpg, rstride, list[e], smem);
  while (e >= 0) {
    const int j = list[e];
    const int e2 = next_entry(list, cnt, e + 1, t);
    wait_loads();     // this wave's share of block j has landed
    __syncthreads();  // everyone's share has; stage st^1 is no longer read by anyone
    if (e2 >= 0) issue_block<D, BLK>(Kg, Vpg, rstride, list[e2], smem + (st ^ 1) * TL::STAGE);
    const char* Kst = smem + st * TL::STAGE;
    const char* Vst = Kst + TL::IMG;

    // S^T = K Q^T over this wave's key half: KT tiles of 32 keys x 32 queries.  The two
    // waves sharing a SIMD (same query group, both key halves) leave each barrier in step;
    // the first key half issues its products at raised priority so it reaches its softmax
    // while the other half's products still run, and the two then alternate between matrix
    // and vector work instead of competing for the same unit.
    if (kh == 0) __builtin_amdgcn_s_setprio(2);
    f32x16 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = (f32x16){};
      const int r = kh * TL::HK + kt * 32 + l32;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(Kst + k_chunk_pos<D>(r, 2 * c + hi) * 16);
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kt], 0, 0, 0);
      }
    }
    if (kh == 0) __builtin_amdgcn_s_setprio(0);

    // Online softmax.  Lane value (kt, i, r) is key kh*HK + kt*32 + 8i + 4*hi + r of the
    // block; the causal mask only touches the diagonal block.
    if (j >= t) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kloc = kh * TL::HK + kt * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
          if (j > t || kloc > qloc) s[kt][v] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[kt][v]);
    mloc = pair_max(mloc);
    const bool raise =
        mloc > m_run && (m_run == -INFINITY || (mloc - m_run) * scale_log2 > kLazy);
    if (__any(raise)) {
      const float m_new = raise ? mloc : m_run;
      const float alpha =
          m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc_o[dt] *= alpha;
    }
    const float mc = m_run == -INFINITY ? 0.0f : -m_run * scale_log2;

    float psum = 0.0f;
    f16x8 pf[KT][2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][v], scale_log2, mc));
        psum += p;
        pf[kt][v >> 3][v & 7] = (_Float16)p;
      }
    l_run += psum;

    // O^T += V^T P^T.  B operand slot 8*hi + 4i' + r of pf[kt][half] is key
    // kh*HK + kt*32 + 16*half + 8i' + 4*hi + r; the A operand reads V^T at the same keys.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + l32;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int g0 = (kh * TL::HK + kt * 32 + 16 * half) / 4 + hi;
          const uint2 lo = *reinterpret_cast<const uint2*>(Vst + v_gran_pos<BLK>(d, g0) * 8);
          const uint2 up = *reinterpret_cast<const uint2*>(Vst + v_gran_pos<BLK>(d, g0 + 2) * 8);
          const uint4 raw = make_uint4(lo.x, lo.y, up.x, up.y);
          const f16x8 a = *reinterpret_cast<const f16x8*>(&raw);
          acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[kt][half], acc_o[dt], 0, 0, 0);
        }
    }
    st ^= 1;
    e = e2;
  }
  __syncthreads();  // every wave is done with the K/V stages before they hold merge data

  // Merge the two key halves of each query group through LDS.
  float* mO = reinterpret_cast<float*>(smem) + (size_t)qg * 64 * (DT * 16 + 2);
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mO[(dt * 16 + v) * 64 + lane] = acc_o[dt][v];
    mO[DT * 16 * 64 + lane] = m_run;
    mO[(DT * 16 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = mO[DT * 16 * 64 + lane];
  const float l1 = mO[(DT * 16 + 1) * 64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
  const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
  const float l_lane = l_run * a0 + l1 * a1;
  const float l_tot = pair_sum(l_lane);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const size_t orow = (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * hi;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = 4 * i + r;
        o[r] = (acc_o[dt][v] * a0 + mO[(dt * 16 + v) * 64 + lane] * a1) * inv;
      }
      if (out_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(O) + orow + d0) =
            make_float4(o[0], o[1], o[2], o[3]);
      } else {
        uint2 pk;
        pk.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
        pk.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(O) + orow + d0) = pk;
      }
    }
  if (lse && hi == 0)
    lse[((size_t)b * dm.Hq + h) * dm.N + qrow] =
        l_tot > 0.0f ? (m * scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------- fp32 (VALU) path

template <int D, int BLK>
__global__ __launch_bounds__(BLK) void attn_f32(Dims dm, const float* __restrict__ Q,
                                                const float* __restrict__ K,
                                                const float* __restrict__ V,
                                                const int32_t* __restrict__ kv_idx,
                                                const int32_t* __restrict__ kv_cnt, int W,
                                                float scale, void* __restrict__ O, int out_f32,
                                                float* __restrict__ lse) {
  extern __shared__ float fsm[];
  float* Kb = fsm;            // [BLK][D]
  float* Vb = fsm + BLK * D;  // [BLK][D]
  int b, h, t;
  decode_tile(dm, b, h, t);
  const int g = h / dm.G;
  const size_t bht = ((size_t)b * dm.Hq + h) * dm.n + t;
  const int32_t* list = kv_idx + bht * W;
  const int cnt = min(kv_cnt[bht], W);
  const int qrow = t * BLK + threadIdx.x;
  const int rstride = dm.Hkv * D;

  float q[D], o[D];
  const float* qp = Q + (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qp[c];
    o[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int e = next_entry(list, cnt, 0, t); e >= 0; e = next_entry(list, cnt, e + 1, t)) {
    const int j = list[e];
    const size_t row0 = (size_t)b * dm.N + (size_t)j * BLK;
    for (int x = threadIdx.x; x < BLK * D; x += BLK) {
      const int r = x / D, c = x - r * D;
      Kb[x] = K[(row0 + r) * rstride + (size_t)g * D + c];
      Vb[x] = V[(row0 + r) * rstride + (size_t)g * D + c];
    }
    __syncthreads();
    for (int r = 0; r < BLK; ++r) {
      if ((size_t)j * BLK + r > (size_t)qrow) break;
      float sdot = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) sdot = __builtin_fmaf(q[c], Kb[r * D + c], sdot);
      const float z = sdot * scale;
      const float mn = fmaxf(m, z);
      const float a = __expf(m - mn), p = __expf(z - mn);
      l = l * a + p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, Vb[r * D + c], o[c] * a);
      m = mn;
    }
    __syncthreads();
  }
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const size_t orow = (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    if (out_f32)
      static_cast<float*>(O)[orow + c] = o[c] * inv;
    else
      static_cast<uint16_t*>(O)[orow + c] = (uint16_t)f32_to_bf16_bits(o[c] * inv);
  }
  if (lse)
    lse[((size_t)b * dm.Hq + h) * dm.N + qrow] = l > 0.0f ? m + __logf(l) : -INFINITY;
}

template <int D, int BLK>
hipError_t launch_bf16(const Dims& dm, const void* Q, const void* K, const void* V,
                       const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                       void* ws, void* O, int out_dtype, float* lse, hipStream_t s) {
  using TL = Tiles<D, BLK>;
  uint16_t* Vp = static_cast<uint16_t*>(ws);
  const unsigned nblk = (unsigned)((size_t)dm.B * dm.Hkv * dm.n);
  hipLaunchKernelGGL((pack_v<D, BLK>), dim3(nblk), dim3(kPackThreads), 0, s, dm,
                     static_cast<const uint16_t*>(V), Vp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = allow_lds(attn_bf16<D, BLK>, TL::LDS)) != hipSuccess) return e;
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hq * dm.n);
  hipLaunchKernelGGL((attn_bf16<D, BLK>), dim3(grid), dim3(TL::NT), TL::LDS, s, dm,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K), Vp,
                     kv_idx, kv_cnt, W, scale * kLog2e, O, out_dtype == SA_F32 ? 1 : 0, lse);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_f32(const Dims& dm, const void* Q, const void* K, const void* V,
                      const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                      void* O, int out_dtype, float* lse, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hq * dm.n);
  const size_t lds = sizeof(float) * 2 * BLK * D;
  hipError_t e = allow_lds(attn_f32<D, BLK>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_f32<D, BLK>), dim3(grid), dim3(BLK), lds, s, dm,
                     static_cast<const float*>(Q), static_cast<const float*>(K),
                     static_cast<const float*>(V), kv_idx, kv_cnt, W, scale, O,
                     out_dtype == SA_F32 ? 1 : 0, lse);
  return hipGetLastError();
}

}  // namespace

size_t forward_ws_bytes(const Dims& dm) {
  if (dm.dtype != SA_BF16) return 0;
  return (size_t)dm.B * dm.Hkv * dm.n * dm.d * dm.blk * sizeof(uint16_t);
}

hipError_t launch_forward(const Dims& dm, const void* Q, const void* K, const void* V,
                          const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                          void* ws, void* O, int out_dtype, float* lse, hipStream_t s) {
  if (dm.dtype == SA_BF16) {
    if (dm.d == 64)
      return dm.blk == 64 ? launch_bf16<64, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, ws, O,
                                                out_dtype, lse, s)
                          : launch_bf16<64, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, ws, O,
                                                 out_dtype, lse, s);
    return dm.blk == 64 ? launch_bf16<128, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, ws, O,
                                               out_dtype, lse, s)
                        : launch_bf16<128, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, ws, O,
                                                out_dtype, lse, s);
  }
  if (dm.d == 64)
    return dm.blk == 64
               ? launch_f32<64, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
               : launch_f32<64, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s);
  return dm.blk == 64
             ? launch_f32<128, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
             : launch_f32<128, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s);
}

}  // namespace sa
