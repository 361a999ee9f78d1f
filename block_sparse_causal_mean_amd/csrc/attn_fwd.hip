// Sparse attention over the selected KV blocks: a FlashAttention-style online-softmax pass.
//
// Stem page, implementation note: the method runs block-sparse attention kernels over the
// chosen blocks after block-level scoring; gated-selection page, Metodologia step 5: every
// tile's list has the same padded shape (sentinel -1).  ART page, section 2.4: the online
// softmax is invariant to the order of the KV blocks, and the causal mask is applied before
// accumulation.
//
// bf16 inputs (pack_v + attn_bf16):
//   pack_v      once per call, V [B, N, Hkv, d] bf16 -> fp16 sub-block images (V^T, keys
//               contiguous, rows padded): exactly the LDS image attn_bf16 wants.  Each V block is read
//               by hundreds of tiles, so converting and transposing it once here takes that
//               work out of the attention loop.  bf16 -> fp16 is exact for |v| in
//               [2^-14, 65504]; smaller magnitudes keep an absolute error below 2^-25.
//   attn_bf16   one workgroup per (batch, q head, query tile): one wave per 32-row query
//               group, two workgroups per CU (independent barriers, so one computes while
//               the other waits for memory).  Per 64-key (or 32-key) sub-block of a listed
//               block:
//               S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 coordinates from
//               LDS, B = the wave's Q fragment held in registers), so each lane's
//               accumulator holds logits of ONE query row: row max and sum are lane-local
//               plus one swap with the lane 32 apart, and P^T is already laid out as the B
//               operand of O^T += V^T P^T (v_mfma_f32_32x32x16_f16; the key index is
//               permuted consistently in the V^T operand instead of moving P through LDS).
//               K and V^T sub-blocks go from global memory straight into LDS
//               (global_load_lds, no registers), double-buffered so the next one streams in
//               while the current one is computed, with one barrier per sub-block.  Both LDS
//               images have padded rows, which keeps the operand reads free of bank
//               conflicts at per-lane base + constant offsets.
//               fp32 accumulation throughout; P is rounded to fp16 (11 significant bits)
//               for the second product.
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

// A tile's block list held in registers, 64 entries at a time (lane i holds entry base + i),
// read with readlane.  Keeping list reads off the scalar-memory path matters: a scalar load
// in flight shares the LDS wait counter and would force every operand wait in the compute
// loop to drain completely.
struct ListWindow {
  const int32_t* list;
  int cnt, t, base, val;
  __device__ __forceinline__ ListWindow(const int32_t* l, int c, int tt)
      : list(l), cnt(c), t(tt), base(-64), val(-1) {}
  __device__ __forceinline__ int get(int e) {  // e uniform, 0 <= e < cnt
    if (e < base || e >= base + 64) {
      base = e & ~63;
      const int i = base + (int)(threadIdx.x & 63);
      val = i < cnt ? list[i] : -1;
    }
    return __builtin_amdgcn_readlane(val, e - base);
  }
  // Next usable entry at or after e (same rules as next_entry), or -1.
  __device__ __forceinline__ int next(int e) {
    for (; e < cnt; ++e) {
      const int j = get(e);
      if (j < 0) return -1;
      if (j <= t) return e;
    }
    return -1;
  }
};

// ------------------------------------------------------------------ padded block images
//
// The attention loop streams each listed block in sub-blocks of SB = BLK/2 keys.  In LDS a K
// sub-block is SB rows of D bf16 and a V^T sub-block is D rows of SB fp16, each row padded
// (K by 16 bytes, V^T by 8) so that the lanes of one LDS phase, which read the same column
// of consecutive rows, fall on distinct banks: the row strides are odd multiples of the read
// width modulo the 256-byte bank sweep.  Padding rather than an address swizzle keeps every
// operand read at a per-lane base plus a compile-time offset.
template <int D>
struct KImg {
  static constexpr int RB = D * 2 + 16;  // row bytes
  static constexpr int CPR = RB / 16;    // 16-byte chunks per row (last one is padding)
};
template <int SB>
struct VImg {
  static constexpr int RB = SB * 2 + 8;  // row bytes
};

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

// V [B, N, Hkv, D] bf16 -> fp16 sub-block images [B, Hkv, n, BLK/SB] x (D rows of
// VImg<SB>::RB bytes: SB keys then zero padding) -- exactly the LDS image attn_bf16 uses.
template <int D, int BLK>
__global__ __launch_bounds__(kPackThreads) void pack_v(Dims dm, const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ Vp) {
  constexpr int SB = BLK / 2;
  constexpr int RS = D + 2;                 // LDS row stride (elements)
  constexpr int GR = VImg<SB>::RB / 8;      // 8-byte granules per image row (last: padding)
  constexpr int IMG = D * VImg<SB>::RB / 2; // fp16 elements per sub-block image
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
  uint2* out = reinterpret_cast<uint2*>(Vp + (size_t)id * (BLK / SB) * IMG);
  for (int i = threadIdx.x; i < (BLK / SB) * D * GR; i += kPackThreads) {
    const int sub = i / (D * GR);
    const int w = i - sub * (D * GR);
    const int d = w / GR, gk = w - d * GR;  // granule gk of row d
    if (gk == GR - 1) {
      out[i] = make_uint2(0u, 0u);
      continue;
    }
    const int key0 = sub * SB + 4 * gk;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = bf16_bits_to_f32(sv[(key0 + k) * RS + d]);
    const f16x2 a = __builtin_convertvector((f32x2){x[0], x[1]}, f16x2);
    const f16x2 c = __builtin_convertvector((f32x2){x[2], x[3]}, f16x2);
    out[i] = make_uint2(*reinterpret_cast<const uint32_t*>(&a), *reinterpret_cast<const uint32_t*>(&c));
  }
}

// --------------------------------------------------------------------------- attn_bf16

template <int D, int BLK>
struct Tiles {
  static constexpr int NW = BLK / 32;          // waves = query groups of 32 rows
  static constexpr int NT = 64 * NW;           // threads (= 2 * BLK)
  static constexpr int SB = BLK / 2;           // keys per pipeline step (sub-block)
  static constexpr int NSB = BLK / SB;         // sub-blocks per block
  static constexpr int KT = SB / 32;           // 32-key tiles per step
  static constexpr int KB = SB * KImg<D>::RB;  // bytes of a K image
  static constexpr int VB = D * VImg<SB>::RB;  // bytes of a V^T image
  static constexpr int KCH = KB / 16, VCH = VB / 16;  // 16-byte chunks
  static constexpr int STAGE = KB + VB;
  static constexpr int VSUB = VB / 2;          // fp16 elements per packed V^T image
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// Issues the direct global->LDS loads of sub-block `sub` of block j into one stage: lane i
// of a wave's load lands at the 1 KiB region base + 16 i, so each lane fetches the global
// chunk that belongs at its slot (K padding slots refetch the row's first chunk).
template <int D, int BLK>
__device__ __forceinline__ void issue_step(const uint16_t* __restrict__ Kg,
                                           const uint16_t* __restrict__ Vpg, int rstride,
                                           int j, int sub, char* kst, char* vst) {
  using TL = Tiles<D, BLK>;
  constexpr int CPR = KImg<D>::CPR;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint16_t* kb = Kg + ((size_t)j * BLK + (size_t)sub * TL::SB) * rstride;
  const uint16_t* vb = Vpg + ((size_t)j * TL::NSB + sub) * TL::VSUB;
#pragma unroll
  for (int region = wv; region * 64 < TL::KCH; region += TL::NW) {
    const int P = region * 64 + lane;
    const int r = P / CPR, c = P - r * CPR;
    if (P < TL::KCH)
      __builtin_amdgcn_global_load_lds(kb + (size_t)r * rstride + (c < CPR - 1 ? c : 0) * 8,
                                       (lds_ptr)(kst + region * 1024), 16, 0, 0);
  }
#pragma unroll
  for (int region = wv; region * 64 < TL::VCH; region += TL::NW) {
    const int P = region * 64 + lane;
    if (P < TL::VCH)
      __builtin_amdgcn_global_load_lds(vb + (size_t)P * 8, (lds_ptr)(vst + region * 1024), 16,
                                       0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A row's running maximum is only raised when a new logit exceeds it by more than this many
// powers of two; until then probabilities may reach 2^kLazy, which fp16 P and the fp32
// accumulators hold exactly enough, and the rescale of O is skipped.
constexpr float kLazy = 8.0f;

// Online-softmax state of one wave (32 query rows; each lane pair shares a row).
template <int D>
struct RowState {
  f32x16 acc_o[D / 32];
  float m_run, l_run;
};

// One pipeline step: S^T = K Q^T for SB keys, online softmax, O^T += V^T P^T.
template <int D, int BLK>
__device__ __forceinline__ void compute_step(const char* __restrict__ kst,
                                             const char* __restrict__ vst, const bf16x8 (&qf)[D / 16],
                                             RowState<D>& rs, bool diag, int k0, int qloc,
                                             int l32, int hi, float scale_log2) {
  using TL = Tiles<D, BLK>;
  constexpr int KT = TL::KT, SB = TL::SB, DT = D / 32, DC = D / 16;
  constexpr int KRB = KImg<D>::RB, VRB = VImg<SB>::RB;
  // S^T = K Q^T: KT tiles x DC coordinate chunks = NS products, their A operands read from
  // LDS PD products ahead (scheduling fences keep the reads where they are written, so the
  // matrix unit never waits on the full LDS latency).
  constexpr int NS = KT * DC, PD = 4;
  f32x16 s[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) s[kt] = (f32x16){};
  const char* kp = kst + l32 * KRB + hi * 16;  // row l32 (+32 kt), coordinates 8*hi + 16c
  auto kaddr = [&](int i) { return kp + (i / DC) * 32 * KRB + (i % DC) * 32; };
  bf16x8 ka[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(kaddr(i));
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    s[i / DC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i % PD], qf[i % DC], s[i / DC], 0, 0, 0);
    if (i + PD < NS) ka[i % PD] = *reinterpret_cast<const bf16x8*>(kaddr(i + PD));
  }
  __builtin_amdgcn_sched_barrier(0);
  // Lane value (kt, i, r) is key k0 + kt*32 + 8i + 4*hi + r of the block.
  if (diag) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kloc = k0 + kt * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (kloc > qloc) s[kt][v] = -INFINITY;
      }
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int v = 0; v < 16; ++v) mloc = fmaxf(mloc, s[kt][v]);
  mloc = pair_max(mloc);
  const bool raise =
      mloc > rs.m_run && (rs.m_run == -INFINITY || (mloc - rs.m_run) * scale_log2 > kLazy);
  if (__any(raise)) {
    const float m_new = raise ? mloc : rs.m_run;
    const float alpha =
        rs.m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((rs.m_run - m_new) * scale_log2);
    rs.m_run = m_new;
    rs.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) rs.acc_o[dt] *= alpha;
  }
  const float mc = rs.m_run == -INFINITY ? 0.0f : -rs.m_run * scale_log2;
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
  rs.l_run += psum;
  // O^T += V^T P^T.  B operand slot 8*hi + 4i' + r of pf[kt][half] is key
  // kt*32 + 16*half + 8i' + 4*hi + r of the step; the A operand reads V^T at those keys.
  // Products are ordered (dt, kt, half); operands are read PD products ahead.
  constexpr int NP = DT * KT * 2;
  const char* vp = vst + l32 * VRB + hi * 8;  // row d = dt*32 + l32, keys 4*hi + ...
  auto vaddr = [&](int i) {
    const int dt = i / (KT * 2), kt = (i / 2) % KT, half = i % 2;
    return vp + dt * 32 * VRB + (kt * 32 + 16 * half) * 2;
  };
  auto vload = [&](int i) {
    const char* q = vaddr(i);
    const uint2 lo = *reinterpret_cast<const uint2*>(q);
    const uint2 up = *reinterpret_cast<const uint2*>(q + 16);
    const uint4 raw = make_uint4(lo.x, lo.y, up.x, up.y);
    return *reinterpret_cast<const f16x8*>(&raw);
  };
  f16x8 va[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) va[i] = vload(i);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int dt = i / (KT * 2), kt = (i / 2) % KT, half = i % 2;
    rs.acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i % PD], pf[kt][half], rs.acc_o[dt], 0, 0, 0);
    if (i + PD < NP) va[i % PD] = vload(i + PD);
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void attn_bf16(  // BLK*2 == Tiles::NT; 2 waves/SIMD
    Dims dm, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vp, const int32_t* __restrict__ kv_idx,
    const int32_t* __restrict__ kv_cnt, int W, float scale_log2, void* __restrict__ O,
    int out_f32, float* __restrict__ lse) {
  using TL = Tiles<D, BLK>;
  constexpr int SB = TL::SB, DT = D / 32, DC = D / 16;
  // Two separate stage buffers: the loads in flight into one are then provably disjoint from
  // the reads of the other, so reads never wait for them.
  __shared__ __attribute__((aligned(1024))) char k0s[TL::KB], v0s[TL::VB];
  __shared__ __attribute__((aligned(1024))) char k1s[TL::KB], v1s[TL::VB];

  int b, h, t;
  decode_tile(dm, b, h, t);
  const int g = h / dm.G;
  const int lane = threadIdx.x & 63, qg = threadIdx.x >> 6;  // wave = query group
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t bht = ((size_t)b * dm.Hq + h) * dm.n + t;
  const int32_t* list = kv_idx + bht * W;
  const int cnt = min(kv_cnt[bht], W);
  const int qloc = qg * 32 + l32;  // this lane's query row within the tile
  const int qrow = t * BLK + qloc;
  const int rstride = dm.Hkv * D;
  const uint16_t* Kg = K + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const uint16_t* Vpg = Vp + ((size_t)b * dm.Hkv + g) * dm.n * TL::NSB * TL::VSUB;

  // Q fragment (B operand of S^T = K Q^T): lane holds coordinates 16c + 8*hi .. +7 of its row.
  bf16x8 qf[DC];
  {
    const uint16_t* qp = Q + (((size_t)b * dm.N + qrow) * dm.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < DC; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  }
  RowState<D> rs;
#pragma unroll
  for (int i = 0; i < DT; ++i) rs.acc_o[i] = (f32x16){};
  rs.m_run = -INFINITY;
  rs.l_run = 0.0f;

  // Steps are (list entry, sub-block); stage 0 holds even steps, stage 1 odd ones.
  ListWindow lw(list, cnt, t);
  int e = lw.next(0), sub = 0;
  int j = e >= 0 ? lw.get(e) : 0;
  if (e >= 0) issue_step<D, BLK>(Kg, Vpg, rstride, j, 0, k0s, v0s);
  while (e >= 0) {
    // even step: compute from stage 0, prefetch the next step into stage 1
    {
      int e2 = e, sub2 = sub + 1, j2 = j;
      if (sub2 == TL::NSB) {
        e2 = lw.next(e + 1);
        sub2 = 0;
        if (e2 >= 0) j2 = lw.get(e2);
      }
      wait_loads();
      __syncthreads();
      if (e2 >= 0) issue_step<D, BLK>(Kg, Vpg, rstride, j2, sub2, k1s, v1s);
      const int k0 = sub * SB;
      if (!(j == t && k0 > qg * 32 + 31))
        compute_step<D, BLK>(k0s, v0s, qf, rs, j == t, k0, qloc, l32, hi, scale_log2);
      e = e2;
      sub = sub2;
      j = j2;
    }
    if (e < 0) break;
    // odd step: compute from stage 1, prefetch into stage 0
    {
      int e2 = e, sub2 = sub + 1, j2 = j;
      if (sub2 == TL::NSB) {
        e2 = lw.next(e + 1);
        sub2 = 0;
        if (e2 >= 0) j2 = lw.get(e2);
      }
      wait_loads();
      __syncthreads();
      if (e2 >= 0) issue_step<D, BLK>(Kg, Vpg, rstride, j2, sub2, k0s, v0s);
      const int k0 = sub * SB;
      if (!(j == t && k0 > qg * 32 + 31))
        compute_step<D, BLK>(k1s, v1s, qf, rs, j == t, k0, qloc, l32, hi, scale_log2);
      e = e2;
      sub = sub2;
      j = j2;
    }
  }

  const float l_tot = pair_sum(rs.l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  const size_t orow = (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * hi;
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = rs.acc_o[dt][4 * i + r] * inv;
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
        l_tot > 0.0f ? (rs.m_run * scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
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
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hq * dm.n);
  hipLaunchKernelGGL((attn_bf16<D, BLK>), dim3(grid), dim3(TL::NT), 0, s, dm,
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
  // packed V^T images: per block, 2 sub-blocks of d rows x (blk/2 keys + 4 padding) fp16
  return (size_t)dm.B * dm.Hkv * dm.n * 2 * dm.d * (dm.blk / 2 + 4) * sizeof(uint16_t);
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
