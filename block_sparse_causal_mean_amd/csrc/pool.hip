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
//   relies on for reproducible results).
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

template <typename T, int MODE, int BLK>
__global__ __launch_bounds__(kPoolThreads) void pool_keys(const T* __restrict__ K,
                                                          float* __restrict__ out, int N,
                                                          int n, int span, size_t plane) {
  constexpr int E = Vec16<T>::N;
  const int bj = blockIdx.x;  // b * n + j
  const int b = bj / n, j = bj - b * n;
  const int e0 = (blockIdx.y * kPoolThreads + threadIdx.x) * E;
  if (e0 >= span) return;
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
  float* dst = out + (size_t)bj * span + e0;
  if (MODE == SA_KMEAN) {
    const float inv = 1.0f / (float)BLK;  // exact: BLK is a power of two
#pragma unroll
    for (int i = 0; i < E; ++i) dst[i] = a[i] * inv;
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      dst[i] = canon(a[i]);
      dst[plane + i] = canon(c[i]);
    }
  }
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

template <typename T, int MODE, int BLK>
hipError_t launch_keys(const Dims& D, const void* K, float* summ, hipStream_t s) {
  const int span = D.Hkv * D.d;
  const int per_wg = kPoolThreads * Vec16<T>::N;
  dim3 grid((unsigned)(D.B * D.n), (unsigned)((span + per_wg - 1) / per_wg));
  const size_t plane = (size_t)D.B * D.n * span;
  hipLaunchKernelGGL((pool_keys<T, MODE, BLK>), grid, dim3(kPoolThreads), 0, s,
                     static_cast<const T*>(K), summ, D.N, D.n, span, plane);
  return hipGetLastError();
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
    e = D.blk == 64 ? launch_keys<T, SA_KMEAN, 64>(D, K, summ, s)
                    : launch_keys<T, SA_KMEAN, 128>(D, K, summ, s);
  else
    e = D.blk == 64 ? launch_keys<T, SA_KMINMAX, 64>(D, K, summ, s)
                    : launch_keys<T, SA_KMINMAX, 128>(D, K, summ, s);
  if (e != hipSuccess || !D.oam) return e;
  const size_t plane = (size_t)D.B * D.n * D.Hkv * D.d;
  float* vn = summ + plane * (D.score_mode == SA_KMINMAX ? 2 : 1);
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
