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
  int B, N, Hq, Hkv, G, d, blk, n;  // n = N / blk tiles (= blocks)
  int dtype, score_mode, oam;
};

struct BudgetDev {
  int k_max, k_min, kind, n_sink, gate_mode;
  float tau_fixed;
  double rho, q;
  int R;  // ranked entries stored per (b, h, t)
  int W;  // entries per padded list
};

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
hipError_t launch_forward(const Dims& D, const void* Q, const void* K, const void* V,
                          const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                          void* O, int out_dtype, float* lse, hipStream_t s);

}  // namespace sa
