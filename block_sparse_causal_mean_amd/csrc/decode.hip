// Decode attention with run-time termination (ART page, sections 2.1-2.4).
//
// A decode query attends to its sequence's K/V cache block by block with an online softmax.
// After each block the partial output's probe vector (its first kArtProbe coordinates) is
// compared with the previous one: the change of its L2 norm and its change of direction
// (1 - cosine similarity).  Once both have stayed below their thresholds (tau, phi) for
// `patience` consecutive blocks, the traversal stops and the partial output is the result.
// Block 0 (the attention sink) is always evaluated first; the other blocks follow
// recency-first (n-1, n-2, ..., 1), an order the online softmax is invariant to (section 2.4).
//
// art_decode: one workgroup per (batch, kv head); wave h computes query head h of the kv
// head's group (at most four), so each K/V block is read from memory once for all of them.
// A head that stops freezes its output; the workgroup stops streaming when all have.  Each
// block's K and V arrive in registers kArtPrefetch blocks ahead of their use (one register
// slot per block in flight; the step loop is unrolled that many times so that the slots are
// compile-time; the sequential traversal needs the depth to cover memory latency), are
// stored to one of two LDS tile sets (alternating, so that one barrier per block suffices),
// and are read from there: K rows padded by 16 bytes so that 64 lanes reading 64 rows hit
// distinct banks.  Scores: lane r = key r of the block, a dot product over d with
// v_dot2_f32_bf16 (two exact bf16 products per instruction, fp32 sums); softmax in
// the log2 domain with exact rescaling; P V: lane i holds output coordinates E i .. E i + E-1.
// Bound: HBM (the whole traversal streams K and V once); early termination is the saving.

#include <type_traits>

#include "common.h"

namespace sa {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kArtBlk = 64;
constexpr int kArtThreads = 256;
constexpr int kArtPrefetch = 4;  // blocks in flight per workgroup
constexpr int kArtMaxG = 4;

template <int D>
struct ArtCfg {
  static constexpr int CH = D / 8;                  // 16-byte chunks per K or V row
  static constexpr int NCH = kArtBlk * CH;          // chunks per block of K (or V)
  static constexpr int CPT = NCH / kArtThreads;     // chunks per thread per tensor
  static constexpr int RS = D * 2 + 16;             // K tile row stride (bytes)
  static constexpr int E = D / 64;                  // output coordinates per lane
  static_assert(NCH % kArtThreads == 0, "block chunks must split evenly");
  static_assert(kArtProbe % E == 0 && kArtProbe / E <= 64, "probe lanes");
};

// Wave-wide sum and max without the LDS crossbar: lanes pair up within quads (DPP quad
// permutes: lane ^ 1, lane ^ 2), within 8- and 16-lane rows (DPP half-row and row mirrors),
// then across 16- and 32-lane groups (v_permlane16_swap, v_permlane32_swap).  At each level
// two partners combine the same two values, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xf, 0xf, false));
}
template <typename OP>
__device__ __forceinline__ float wreduce(float v, OP op) {
  v = op(v, dpp<0xB1>(v));   // quad_perm [1, 0, 3, 2]: lane ^ 1
  v = op(v, dpp<0x4E>(v));   // quad_perm [2, 3, 0, 1]: lane ^ 2
  v = op(v, dpp<0x141>(v));  // row_half_mirror: the other quad of the 8-lane half-row
  v = op(v, dpp<0x140>(v));  // row_mirror: the other half of the 16-lane row
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
  v = op(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
  return op(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ __forceinline__ float wsum(float v) {
  return wreduce(v, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ float wmax(float v) {
  return wreduce(v, [](float a, float b) { return fmaxf(a, b); });
}

template <int D>
__global__ __launch_bounds__(kArtThreads) void art_decode(
    Dims dm, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float scale_log2, float tau, float phi, int patience,
    void* __restrict__ O, int out_f32, int32_t* __restrict__ done) {
  using C = ArtCfg<D>;
  constexpr int CH = C::CH, CPT = C::CPT, RS = C::RS, E = C::E;
  __shared__ __attribute__((aligned(16))) char ktiles[2][kArtBlk * RS];
  __shared__ __attribute__((aligned(16))) uint16_t vtiles[2][kArtBlk * D];
  __shared__ __attribute__((aligned(16))) uint32_t qs[kArtMaxG][D / 2];  // bf16 pairs
  __shared__ __attribute__((aligned(16))) float ps[kArtMaxG][kArtBlk];
  // Stop flags, double-buffered by step parity: step k reads live[k & 1] (every decision
  // up to step k - 1) and each wave posts its own state for step k + 1 to live[(k + 1) & 1].
  // A wave can only write live[k & 1] again in step k + 1, after the barrier that every wave
  // passes once its reads of step k are done, so all waves read the same flags.
  __shared__ int live[2][kArtMaxG];

  const int g = (int)blockIdx.x % dm.Hkv, b = (int)blockIdx.x / dm.Hkv;
  const int G = dm.G;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = dm.N / kArtBlk;
  const size_t rstride = (size_t)dm.Hkv * D;
  const uint16_t* Kb = K + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const uint16_t* Vb = V + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const bool active = w < G;  // this wave computes query head g * G + w
  const int h = g * G + w;

  for (int i = threadIdx.x; i < G * D / 2; i += kArtThreads) {
    const int hh = i / (D / 2), c2 = i - hh * (D / 2);
    qs[hh][c2] = reinterpret_cast<const uint32_t*>(Q + ((size_t)b * dm.Hq + g * G + hh) * D)[c2];
  }
  if (threadIdx.x < 2 * kArtMaxG)
    live[threadIdx.x / kArtMaxG][threadIdx.x % kArtMaxG] = (int)threadIdx.x % kArtMaxG < G ? 1 : 0;

  // Block k of the traversal: block 0, then n-1, n-2, ..., 1.
  auto block_of = [n](int k) { return k == 0 ? 0 : n - k; };
  // This thread's chunks of a block: chunk i is row r, 16-byte column cc, at a fixed element
  // offset from the block's first row; the block's base is uniform, so a load's address is a
  // scalar base plus that offset.
  uint32_t coff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int q = (int)threadIdx.x + i * kArtThreads;
    const int r = q / CH, cc = q - r * CH;
    coff[i] = (uint32_t)(r * rstride + cc * 8);
  }
  auto chunk_src = [&](const uint16_t* base, int j, int i) {
    const uint16_t* blk = base + (size_t)__builtin_amdgcn_readfirstlane(j) * kArtBlk * rstride;
    return load_nt16(blk + coff[i]);  // read once
  };
  uint4 kr[kArtPrefetch][CPT], vr[kArtPrefetch][CPT];
#pragma unroll
  for (int sl = 0; sl < kArtPrefetch; ++sl) {
    const int j = block_of(sl < n ? sl : 0);  // past the end: a valid block, never used
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      kr[sl][i] = chunk_src(Kb, j, i);
      vr[sl][i] = chunk_src(Vb, j, i);
    }
  }

  float m_run = -INFINITY, l_run = 0.0f, nprev = 0.0f;  // nprev: the previous probe's norm
  float acc[E], prev[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = prev[e] = 0.0f;
  int run = 0, stopped = 0;  // stopped: blocks processed when this head stopped (0: running)

  // One step of the traversal on the block whose chunks are in (kr, vr), in tile set k & 1;
  // refills the registers with block k + kArtPrefetch.  The barrier after the stores also
  // means every wave is done with step k - 1 (whose tile set step k + 1 overwrites) and has
  // posted its stop state to live[k & 1].  Stores, barrier and refill happen on every step,
  // also past the end and after every head stopped (valid blocks, never used), so that each
  // step's memory operations are the same and the compiler's waits stay partial: a step waits
  // for its own block only, with the later blocks still in flight.  Returns whether any head
  // was still running after step k - 1 (the same value in every wave).
  auto step = [&](int k, uint4 (&kr)[CPT], uint4 (&vr)[CPT]) -> bool {
    char* ktile = ktiles[k & 1];
    uint16_t* vtile = vtiles[k & 1];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int q = (int)threadIdx.x + i * kArtThreads;
      const int r = q / CH, cc = q - r * CH;
      *reinterpret_cast<uint4*>(ktile + r * RS + cc * 16) = kr[i];
      *reinterpret_cast<uint4*>(vtile + r * D + cc * 8) = vr[i];
    }
    __syncthreads();
    bool any = false;
    for (int i = 0; i < G; ++i) any |= live[k & 1][i] != 0;
    {
      const int jn = block_of(min(k + kArtPrefetch, n - 1));
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        kr[i] = chunk_src(Kb, jn, i);
        vr[i] = chunk_src(Vb, jn, i);
      }
    }
    if (k < n && active && stopped == 0) {
      // scores of key `lane`
      float s = 0.0f;
      auto d2 = [](uint32_t a, uint32_t b2, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b2), c, false);
      };
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
        const uint4 kv = *reinterpret_cast<const uint4*>(ktile + lane * RS + cc * 16);
        const uint4 q4 = *reinterpret_cast<const uint4*>(&qs[w][cc * 4]);
        s = d2(kv.x, q4.x, s);
        s = d2(kv.y, q4.y, s);
        s = d2(kv.z, q4.z, s);
        s = d2(kv.w, q4.w, s);
      }
      s *= scale_log2;
      const float m_new = fmaxf(m_run, wmax(s));
      const float alpha = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float p = __builtin_amdgcn_exp2f(s - m_new);
      l_run = l_run * alpha + wsum(p);
      m_run = m_new;
      ps[w][lane] = p;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= alpha;
      for (int r4 = 0; r4 < kArtBlk; r4 += 4) {
        const float4 p4 = *reinterpret_cast<const float4*>(&ps[w][r4]);
        const float pr[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint16_t* vrow = vtile + (r4 + u) * D + E * lane;
          if constexpr (E == 2) {
            const uint32_t v2 = *reinterpret_cast<const uint32_t*>(vrow);
            acc[0] = __builtin_fmaf(pr[u], bf16_lo(v2), acc[0]);
            acc[1] = __builtin_fmaf(pr[u], bf16_hi(v2), acc[1]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
              acc[e] = __builtin_fmaf(pr[u], bf16_bits_to_f32(vrow[e]), acc[e]);
          }
        }
      }
      // probe: output coordinates 0 .. kArtProbe-1 (lanes 0 .. kArtProbe/E - 1)
      const float inv = 1.0f / l_run;
      float nx = 0.0f, dp = 0.0f;
      if (lane < kArtProbe / E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float x = acc[e] * inv;
          nx = __builtin_fmaf(x, x, nx);
          dp = __builtin_fmaf(x, prev[e], dp);
          prev[e] = x;
        }
      }
      nx = __builtin_sqrtf(wsum(nx));
      dp = wsum(dp);
      const float np = nprev;
      nprev = nx;
      if (k > 0 && patience > 0) {
        const float dsc = fabsf(nx - np);
        const float ddr = (nx > 0.0f && np > 0.0f) ? 1.0f - dp / (nx * np) : 1.0f;
        run = (dsc < tau && ddr < phi) ? run + 1 : 0;
        if (run >= patience) stopped = k + 1;
      }
    }
    if (active && lane == 0) live[(k + 1) & 1][w] = stopped == 0 ? 1 : 0;
    return any;
  };

  // Rounds of kArtPrefetch steps; the traversal ends after the round in which the last head
  // stopped (at most kArtPrefetch steps of loads later: no compute is spent on them).
  for (int k = 0;; k += kArtPrefetch) {
    bool any = true;
#pragma unroll
    for (int sl = 0; sl < kArtPrefetch; ++sl) any = step(k + sl, kr[sl], vr[sl]);
    if (!any || k + kArtPrefetch >= n) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // refills issued before the exit
  if (active) {
    const int blocks = stopped ? stopped : n;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const size_t orow = ((size_t)b * dm.Hq + h) * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o = acc[e] * inv;
      if (out_f32) static_cast<float*>(O)[orow + e] = o;
      else static_cast<uint16_t*>(O)[orow + e] = (uint16_t)f32_to_bf16_bits(o);
    }
    if (lane == 0) done[(size_t)b * dm.Hq + h] = blocks;
  }
}

template <int D>
hipError_t launch_art(const Dims& dm, const void* Q, const void* K, const void* V, float scale,
                      float tau, float phi, int patience, void* O, int out_dtype, int32_t* done,
                      hipStream_t s) {
  hipLaunchKernelGGL((art_decode<D>), dim3((unsigned)(dm.B * dm.Hkv)), dim3(kArtThreads), 0, s,
                     dm, static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), scale * 1.4426950408889634f, tau, phi,
                     patience, O, out_dtype == SA_F32 ? 1 : 0, done);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_art(const Dims& dm, const void* Q, const void* K, const void* V,
                             float scale, float tau, float phi, int patience, void* O,
                             int out_dtype, int32_t* done, hipStream_t s) {
  return dm.d == 64 ? launch_art<64>(dm, Q, K, V, scale, tau, phi, patience, O, out_dtype, done, s)
                    : launch_art<128>(dm, Q, K, V, scale, tau, phi, patience, O, out_dtype, done,
                                      s);
}

}  // namespace sa
