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
// pool_keys: one workgroup per (batch, block, kv head).  The block's key tile is copied to
//   LDS with all of its loads in flight at once, then one thread per coordinate accumulates
//   the rows in order (the fixed reduction order the selection relies on for reproducible
//   results).  It also writes the selection kernel's private copies of the summaries (bf16
//   and fp32, in chunk-major order: see common.h) and the block's L2 norm (an
//   upper-bound ingredient only: it never decides a selection by itself).
// value_norms: one workgroup per (batch, block).  Each (row, kv head) pair's squared norm is
//   a fused multiply-add chain over the d coordinates in order, by one thread; the square
//   roots go to LDS (block x Hkv floats, checked against the LDS size on the host) and one
//   thread per kv head sums them in row order.

#include "common.h"

namespace sa {
namespace {

constexpr int kPoolThreads = 256;

template <typename T>
struct Vec16;  // 16 bytes of elements, converted exactly to fp32
template <>
struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void cvt(const uint4& v, float* x) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float* x) {
    cvt(*reinterpret_cast<const uint4*>(p), x);
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void cvt(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static void load(const float* p, float* x) {
    cvt(*reinterpret_cast<const uint4*>(p), x);
  }
};

// pool_keys: one workgroup per (batch, block, kv head).  The block's BLK x HD key tile is
// first copied into LDS with every 16-byte load issued at once (8 per thread for bf16 at
// BLK = HD = 128), so the memory system sees the whole tile in flight; then thread c sums
// coordinate c over the rows in order from LDS (the fixed reduction order), writes the
// summary, its bf16 rounding, the block's L2 norm and the L2 norm of the bf16 rounding
// residual (workgroup reductions in any order: they only scale the prefilter's error bound).
template <typename T, int MODE, int BLK, int HD>
__global__ __launch_bounds__(kPoolThreads) void pool_keys(const T* __restrict__ K,
                                                          float* __restrict__ summ,
                                                          uint16_t* __restrict__ bfc,
                                                          float* __restrict__ xc, int N, int n,
                                                          int Hkv, size_t plane, size_t kn_off,
                                                          size_t dn_off, int ncb) {
  constexpr int E = Vec16<T>::N;   // elements per 16-byte chunk
  constexpr int CPR = HD / E;      // chunks per row
  constexpr int NCH = BLK * CPR;   // chunks in the tile
  constexpr int NPL = MODE == SA_KMINMAX ? 2 : 1;
  static_assert(NCH % kPoolThreads == 0, "tile chunks must split evenly over the threads");
  static_assert(HD <= kPoolThreads, "one thread per coordinate");
  __shared__ uint4 tile[NCH];
  __shared__ float red[2][kPoolThreads / 64];
  const int id = (int)blockIdx.x;  // (b * n + j) * Hkv + g
  const int g = id % Hkv;
  const int bj = id / Hkv;
  const int b = bj / n, j = bj - b * n;
  const int span = Hkv * HD;
  const T* src = K + ((size_t)b * N + (size_t)j * BLK) * span + (size_t)g * HD;
  {
    uint4 v[NCH / kPoolThreads];
#pragma unroll
    for (int k = 0; k < NCH / kPoolThreads; ++k) {
      const int c = threadIdx.x + k * kPoolThreads;
      v[k] = load_nt16(src + (size_t)(c / CPR) * span + (c % CPR) * E);  // K is read once
    }
#pragma unroll
    for (int k = 0; k < NCH / kPoolThreads; ++k) tile[threadIdx.x + k * kPoolThreads] = v[k];
  }
  __syncthreads();
  float ss = 0.0f, dd = 0.0f;  // this coordinate's |x|^2 and bf16 rounding residual^2
  const int c = threadIdx.x;
  if (c < HD) {
    const T* tv = reinterpret_cast<const T*>(tile);
    float v[NPL];
    float& a = v[0];
    float mx = 0.0f;
    a = 0.0f;
#pragma unroll 16
    for (int r = 0; r < BLK; ++r) {
      float x;
      if constexpr (sizeof(T) == 2) x = bf16_bits_to_f32(tv[r * HD + c]);
      else x = tv[r * HD + c];
      if (MODE == SA_KMEAN) {
        a = (r == 0 ? 0.0f : a) + x;
      } else if (r == 0) {
        a = mx = x;
      } else {
        a = x < a ? x : a;
        mx = x > mx ? x : mx;
      }
    }
    const size_t o = ((size_t)bj * Hkv + g) * HD + c;
    if (MODE == SA_KMEAN) {
      a = a * (1.0f / (float)BLK);  // exact: BLK is a power of two
      summ[o] = a;
      ss = a * a;
    } else {
      a = canon(a);
      v[NPL - 1] = canon(mx);
      summ[o] = a;
      summ[plane + o] = v[NPL - 1];
      ss = fmaxf(a * a, v[NPL - 1] * v[NPL - 1]);
    }
    // Chunk-major copies for the selection kernel (layout in common.h).
    const int cb = j >> 5, jl = j & 31;
    const size_t chunk = ((size_t)b * Hkv + g) * ncb + cb;
    uint16_t* bc = bfc + chunk * (size_t)(NPL * HD * 32);
    float* xcp = xc + chunk * (size_t)(NPL * HD * 32);
    const int ks = c >> 4, u = (c >> 3) & 1, e = c & 7;
    const int lane = jl + 32 * u;
#pragma unroll
    for (int p = 0; p < NPL; ++p) {
      const uint32_t h16 = f32_to_bf16_bits(v[p]);
      bc[(p * (HD / 16) + ks) * 512 + lane * 8 + e] = (uint16_t)h16;
      xcp[(p * (HD / 8) + (c >> 3)) * 256 + jl * 8 + e] = v[p];
      const float r = v[p] - bf16_bits_to_f32(h16);  // exact (Sterbenz)
      dd = fmaxf(dd, r * r);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off);
    dd += __shfl_xor(dd, off);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = ss;
    red[1][threadIdx.x >> 6] = dd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f, td = 0.0f;
#pragma unroll
    for (int w = 0; w < kPoolThreads / 64; ++w) {
      t += red[0][w];
      td += red[1][w];
    }
    summ[kn_off + (size_t)bj * Hkv + g] = __builtin_sqrtf(t);
    summ[dn_off + (size_t)bj * Hkv + g] = __builtin_sqrtf(td);
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
  for (int g = threadIdx.x; g < Hkv; g += kPoolThreads) {
    float acc = 0.0f;
    for (int r = 0; r < BLK; ++r) acc = acc + nrm[r * Hkv + g];
    vn[(size_t)bj * Hkv + g] = acc * (1.0f / (float)BLK);
  }
}

template <typename T, int MODE, int BLK, int HD>
hipError_t launch_keys(const Dims& D, const void* K, float* summ, hipStream_t s) {
  const SummaryLayout L = summary_layout(D);
  char* base = reinterpret_cast<char*>(summ);
  hipLaunchKernelGGL((pool_keys<T, MODE, BLK, HD>), dim3((unsigned)(D.B * D.n * D.Hkv)),
                     dim3(kPoolThreads), 0, s, static_cast<const T*>(K), summ,
                     reinterpret_cast<uint16_t*>(base + L.bfc_byte),
                     reinterpret_cast<float*>(base + L.xc_byte), D.N, D.n, D.Hkv, L.plane, L.kn,
                     L.dn, L.ncb);
  return hipGetLastError();
}

template <typename T, int MODE, int BLK>
hipError_t launch_keys_d(const Dims& D, const void* K, float* summ, hipStream_t s) {
  return D.d == 64 ? launch_keys<T, MODE, BLK, 64>(D, K, summ, s)
                   : launch_keys<T, MODE, BLK, 128>(D, K, summ, s);
}

template <typename T, int BLK, int HD>
hipError_t launch_vn(const Dims& D, const void* V, float* vn, hipStream_t s) {
  const size_t lds = value_norms_lds(D);
  const hipError_t e = allow_lds(value_norms<T, BLK, HD>, lds);
  if (e != hipSuccess) return e;
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
