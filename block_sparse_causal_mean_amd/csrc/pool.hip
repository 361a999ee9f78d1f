// Block summaries of the keys (and value norms): the first stage of block-sparse prefill.
//
// "Uncertainty-Gated Selection for Block-Sparse Attention" page, Metodologia step 1: keys are
// grouped in blocks and summarised by a backbone, either the SSA-style mean-pooled key or
// Quest's per-coordinate K-min/K-max.  Stem page, Metodologia B (output-aware metric) and its
// implementation note (block downsampling to compute the metric cheaply): the value
// magnitude enters the block score; here as the mean over the block's rows of each value
// row's L2 norm.
//
// Both kernels stream their input exactly once and are bound by HBM bandwidth.
//
// pool_keys: one workgroup per (batch, block, slice of the Hkv*d row span).  A key row
//   [Hkv, d] is contiguous, so each thread owns 16 bytes of the span and walks the block's
//   rows in order: every load instruction of a wave reads 1 KiB contiguous, and the fp32
//   accumulation per coordinate runs in row order (the fixed reduction order the selection
//   relies on for reproducible results).  It also writes, for the selection's matrix-core
//   prefilter, each summary's bf16 hi/lo split and the block's L2 norm (an upper bound
//   ingredient only: it never decides a selection by itself).
// value_norms: one workgroup per (batch, block).  Each (row, kv head) pair's squared norm is
//   a fused multiply-add chain over the d coordinates in order, by one thread; the square
//   roots go to LDS and one thread per kv head sums them in row order.

#include "common.h"

namespace sa {
namespace {

constexpr int kPoolThreads = 256;

template <typename T>
struct Vec16;  // 16 bytes of elements, converted exactly to fp32
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const uint16_t* p, float* x) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
};

// Splits x into bf16 hi = RN(x) and lo = RN(x - hi) (x - hi is exact in fp32), packed as
// bf16 bits into the low halves of the returned pair.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - __uint_as_float(hi << 16));
}

template <typename T, int MODE, int BLK, int HD>
__global__ __launch_bounds__(kPoolThreads) void pool_keys(const T* __restrict__ K,
                                                          float* __restrict__ summ,
                                                          uint16_t* __restrict__ bfp, int N,
                                                          int n, int span, size_t plane,
                                                          size_t kn_off) {
  constexpr int E = Vec16<T>::N;
  constexpr int LPH = HD / E;  // lanes per head (consecutive lanes of one wave)
  const int bj = blockIdx.x;   // b * n + j
  const int b = bj / n, j = bj - b * n;
  const int e0 = (blockIdx.y * kPoolThreads + threadIdx.x) * E;
  if (e0 >= span) return;  // whole heads drop out together: span is a multiple of HD
  const T* src = K + ((size_t)b * N + (size_t)j * BLK) * span + e0;

  float a[E], c[E];
  float x[E];
  Vec16<T>::load(src, x);
  if (MODE == SA_KMEAN) {
#pragma unroll
    for (int i = 0; i < E; ++i) a[i] = 0.0f + x[i];
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) a[i] = c[i] = x[i];
  }
#pragma unroll 16
  for (int r = 1; r < BLK; ++r) {
    Vec16<T>::load(src + (size_t)r * span, x);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if (MODE == SA_KMEAN) {
        a[i] = a[i] + x[i];
      } else {
        a[i] = x[i] < a[i] ? x[i] : a[i];
        c[i] = x[i] > c[i] ? x[i] : c[i];
      }
    }
  }
  const size_t o = (size_t)bj * span + e0;
  float ss = 0.0f;  // squared norm share of the block's scoring vector (for the prefilter bound)
  if (MODE == SA_KMEAN) {
    const float inv = 1.0f / (float)BLK;  // exact: BLK is a power of two
#pragma unroll
    for (int i = 0; i < E; ++i) {
      a[i] = a[i] * inv;
      summ[o + i] = a[i];
      ss = __builtin_fmaf(a[i], a[i], ss);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      a[i] = canon(a[i]);
      c[i] = canon(c[i]);
      summ[o + i] = a[i];
      summ[plane + o + i] = c[i];
      ss = __builtin_fmaf(fmaxf(a[i] * a[i], c[i] * c[i]), 1.0f, ss);
    }
  }
  // bf16 hi/lo planes: plane p's hi at bfp + 2p*plane, lo at bfp + (2p+1)*plane.
#pragma unroll
  for (int p = 0; p < (MODE == SA_KMEAN ? 1 : 2); ++p) {
    const float* v = p == 0 ? a : c;
    uint32_t hw[E / 2], lw[E / 2];
#pragma unroll
    for (int i = 0; i < E; i += 2) {
      uint32_t h0, l0, h1, l1;
      split_bf16(v[i], h0, l0);
      split_bf16(v[i + 1], h1, l1);
      hw[i / 2] = h0 | (h1 << 16);
      lw[i / 2] = l0 | (l1 << 16);
    }
    uint16_t* hp = bfp + (size_t)(2 * p) * plane + o;
    uint16_t* lp = bfp + (size_t)(2 * p + 1) * plane + o;
    if (E == 8) {
      *reinterpret_cast<uint4*>(hp) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(lp) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    } else {
      *reinterpret_cast<uint2*>(hp) = make_uint2(hw[0], hw[1]);
      *reinterpret_cast<uint2*>(lp) = make_uint2(lw[0], lw[1]);
    }
  }
#pragma unroll
  for (int off = 1; off < LPH; off <<= 1) ss += __shfl_xor(ss, off);
  if (e0 % HD == 0) summ[kn_off + (size_t)bj * (span / HD) + e0 / HD] = __builtin_sqrtf(ss);
}

template <typename T, int BLK, int D>
__global__ __launch_bounds__(kPoolThreads) void value_norms(const T* __restrict__ V,
                                                            float* __restrict__ vn, int N,
                                                            int n, int Hkv) {
  extern __shared__ float nrm[];  // [BLK][Hkv]
  constexpr int E = Vec16<T>::N;
  const int bj = blockIdx.x;
  const int b = bj / n, j = bj - b * n;
  const int span = Hkv * D;
  const T* base = V + ((size_t)b * N + (size_t)j * BLK) * span;
  for (int p = threadIdx.x; p < BLK * Hkv; p += kPoolThreads) {
    const int r = p / Hkv, g = p - r * Hkv;
    const T* row = base + (size_t)r * span + g * D;
    float ss = 0.0f;
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += E) {
      float x[E];
      Vec16<T>::load(row + c0, x);
#pragma unroll
      for (int i = 0; i < E; ++i) ss = __builtin_fmaf(x[i], x[i], ss);
    }
    nrm[p] = __builtin_sqrtf(ss);  // correctly rounded (IEEE) with the build flags
  }
  __syncthreads();
  if (threadIdx.x < Hkv) {
    const int g = threadIdx.x;
    float acc = 0.0f;
    for (int r = 0; r < BLK; ++r) acc = acc + nrm[r * Hkv + g];
    vn[(size_t)bj * Hkv + g] = acc * (1.0f / (float)BLK);
  }
}

template <typename T, int MODE, int BLK, int HD>
hipError_t launch_keys(const Dims& D, const void* K, float* summ, hipStream_t s) {
  const SummaryLayout L = summary_layout(D);
  const int span = D.Hkv * D.d;
  const int per_wg = kPoolThreads * Vec16<T>::N;
  dim3 grid((unsigned)(D.B * D.n), (unsigned)((span + per_wg - 1) / per_wg));
  uint16_t* bfp = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(summ) + L.bf_byte);
  hipLaunchKernelGGL((pool_keys<T, MODE, BLK, HD>), grid, dim3(kPoolThreads), 0, s,
                     static_cast<const T*>(K), summ, bfp, D.N, D.n, span, L.plane, L.kn);
  return hipGetLastError();
}

template <typename T, int MODE, int BLK>
hipError_t launch_keys_d(const Dims& D, const void* K, float* summ, hipStream_t s) {
  return D.d == 64 ? launch_keys<T, MODE, BLK, 64>(D, K, summ, s)
                   : launch_keys<T, MODE, BLK, 128>(D, K, summ, s);
}

template <typename T, int BLK, int HD>
hipError_t launch_vn(const Dims& D, const void* V, float* vn, hipStream_t s) {
  const size_t lds = sizeof(float) * BLK * D.Hkv;
  hipLaunchKernelGGL((value_norms<T, BLK, HD>), dim3((unsigned)(D.B * D.n)),
                     dim3(kPoolThreads), lds, s, static_cast<const T*>(V), vn, D.N, D.n,
                     D.Hkv);
  return hipGetLastError();
}

template <typename T>
hipError_t pool_dispatch(const Dims& D, const void* K, const void* V, float* summ,
                         hipStream_t s) {
  hipError_t e;
  if (D.score_mode == SA_KMEAN)
    e = D.blk == 64 ? launch_keys_d<T, SA_KMEAN, 64>(D, K, summ, s)
                    : launch_keys_d<T, SA_KMEAN, 128>(D, K, summ, s);
  else
    e = D.blk == 64 ? launch_keys_d<T, SA_KMINMAX, 64>(D, K, summ, s)
                    : launch_keys_d<T, SA_KMINMAX, 128>(D, K, summ, s);
  if (e != hipSuccess || !D.oam) return e;
  float* vn = summ + summary_layout(D).vn;
  if (D.blk == 64)
    return D.d == 64 ? launch_vn<T, 64, 64>(D, V, vn, s) : launch_vn<T, 64, 128>(D, V, vn, s);
  return D.d == 64 ? launch_vn<T, 128, 64>(D, V, vn, s) : launch_vn<T, 128, 128>(D, V, vn, s);
}

}  // namespace

hipError_t launch_pool(const Dims& D, const void* K, const void* V, float* summ,
                       hipStream_t s) {
  return D.dtype == SA_BF16 ? pool_dispatch<uint16_t>(D, K, V, summ, s)
                            : pool_dispatch<float>(D, K, V, summ, s);
}

}  // namespace sa
