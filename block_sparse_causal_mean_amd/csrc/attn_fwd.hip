// Sparse attention over the selected KV blocks: a FlashAttention-style online-softmax pass.
//
// Stem page, implementation note: the method runs block-sparse attention kernels over the
// chosen blocks after block-level scoring; gated-selection page, Metodologia step 5: every
// tile's list has the same padded shape (sentinel -1).  ART page, section 2.4: the online
// softmax is invariant to the order of the KV blocks, and the causal mask is applied before
// accumulation.
//
// bf16 inputs (value_absmax + pack_v, then attn_bf16):
//   value_absmax  partial maxima of |v| per (batch, kv head): bf16 magnitudes compared as
//               integers (their bit patterns order like the values), kVmaxParts per head.
//   pack_v      V [B, N, Hkv, d] bf16 -> fp16 V^T step images (32 keys each, dense,
//               swizzled): exactly the LDS image attn_bf16 wants.  Each V block is read by
//               hundreds of tiles, so converting and transposing it once here takes that work
//               out of the attention loop.  fp16 holds less range than bf16, so every value
//               of a (batch, kv head) is first multiplied by the power of two 2^e that brings
//               its largest magnitude into [2^14, 2^15) (exact; e comes from value_absmax's
//               partial maxima), and attn_bf16 multiplies that head's outputs by 2^-e.  Any
//               finite bf16 V is then represented: values within a factor 2^29 of the head's
//               largest magnitude exactly (bf16 -> fp16 is exact in fp16's normal range), the
//               smaller ones with an absolute error below 2^-25 in scaled units.
//   attn_bf16   one workgroup per (batch, q head, query tile), one wave per 32 query rows
//               (4 waves for 128-row tiles, 2 for 64-row tiles), three workgroups per CU.  The
//               tile's blocks are consumed in steps of 32 keys:
//               S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 coordinates from
//               LDS, B = the wave's Q fragment held in registers), so each lane's accumulator
//               holds logits of ONE query row: row max and sum are lane-local plus one swap
//               with the lane 32 apart, and P^T is already laid out as the B operand of
//               O^T += V^T P^T (v_mfma_f32_32x32x16_f16; the V^T image stores each lane's eight
//               keys in exactly that order, so one 16-byte read feeds one product and P never
//               moves through LDS).  fp32 accumulation throughout; P is rounded to fp16
//               (11 significant bits) for the second product.
//               K and V^T steps go from global memory straight into a ring of LDS slots
//               (global_load_lds, no registers), each refilled NR - 1 steps ahead of use,
//               with partial vector-memory waits so a step never waits for later steps'
//               loads.  (For 128-row tiles a 3-slot ring fits three workgroups per CU,
//               three waves per SIMD: measured 5% faster than a 4-slot ring at two
//               workgroups per CU; 2-wave workgroups for 64-row tiles use a split ring of
//               three single K or V^T images instead, which fits six of them per CU, see Cfg.)
//               The template also builds 64-row waves (QH = 2: one K read feeds two products),
//               which halves LDS operand traffic but needs over 256 registers, i.e. one wave
//               per SIMD; on gfx950 it measured slower, so the launcher uses QH = 1.
//               64-row tiles inside 128-key blocks run two to a workgroup (TPW = 2): the
//               block's two tiles form one 128-row tile whose K/V steps stream the union of
//               the two tiles' lists once (stage_union), and each tile's waves skip the
//               blocks their own list lacks.  Adjacent tiles' lists overlap heavily (their
//               union is about 1.15 times one list), so this halves the refills per product
//               and gives three waves per SIMD instead of two: 5% faster than one 2-wave
//               workgroup per tile.
// fp32 inputs (attn_f32): one thread per query row, fp32 VALU arithmetic, same online softmax.
//
// Launch order (decode_tile_grouped): one kv head at a time, its tiles latest first, the
// query heads of a tile on one XCD; each tile's blocks are visited shared-first
// (reorder_shared) so that those heads hit each other's blocks in L2.

#include <type_traits>

#include "common.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Index of the next usable list entry at or after e, or -1: the list ends at cnt or at the
// first negative entry; entries after the tile's last causal block (j > t) are skipped.
__device__ __forceinline__ int next_entry(const int32_t* __restrict__ list, int cnt, int e,
                                          int t) {
  for (; e < cnt; ++e) {
    const int j = list[e];
    if (j < 0) return -1;
    if (j <= t) return e;
  }
  return -1;
}

// Sum of x over lanes l and l ^ 32 (v_permlane32_swap, no LDS traffic).  The swap hands each
// lane its own value and its partner's, one in each result; both lanes of a pair combine the
// same two values, so they get bit-identical results (pair_max_num below likewise).
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------ step images
//
// A step is 32 consecutive keys of one block.  In LDS (and, for V, in the packed workspace):
//   K image    32 key rows x D bf16, rows of 2D bytes, dense.  The 16-byte chunk q of row r
//              (coordinates 8q .. 8q+7) sits at chunk position q ^ kswz(r).
//   V^T image  D coordinate rows x 32 keys fp16, rows of 64 bytes, dense.  Row d holds four
//              16-byte chunks; logical chunk c = 2h + u holds keys 16h + 4u + (0..3) followed
//              by keys 16h + 8 + 4u + (0..3) (the eight keys one lane feeds to one P V^T
//              product) and sits at chunk position c ^ vswz(d).
// The swizzles make the 16-byte operand reads conflict-free: in a K read (chunk q of rows
// 0..31, 256-byte rows) any 16 consecutive lanes hit 16 distinct 16-byte bank groups; in a V^T
// read (chunk c of rows 0..31, 64-byte rows) any 8 consecutive lanes hit distinct groups of a
// 128-byte bank sweep and any 16 consecutive lanes distinct groups of a 256-byte one.
// Swizzling instead of padding keeps the images dense, so no padding bytes are streamed.
constexpr int kStep = 32;

#ifndef ATTN_QH
#define ATTN_QH 1
#endif

template <int D>
__device__ __forceinline__ int kswz(int r) {
  return (r / (128 / D)) & (D / 8 - 1);
}
__device__ __forceinline__ int vswz(int d) { return (((d >> 1) ^ (d >> 3)) & 1) | (d & 4) >> 1; }

// ------------------------------------------------------------------------------ pack_v

constexpr int kPackThreads = 256;

// Largest bf16 magnitude among the eight values of v, as its 15-bit pattern.
__device__ __forceinline__ uint32_t absmax8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7fffu, (w[i] >> 16) & 0x7fffu));
  return m;
}

// Partial maxima of |v|: workgroup (b, g, c) covers rows [c R, (c + 1) R) of (batch b, kv
// head g), R = ceil(N / kVmaxParts), and writes one 15-bit magnitude pattern to
// part[(b Hkv + g) kVmaxParts + c].
template <int D>
__global__ __launch_bounds__(kPackThreads) void value_absmax(Dims dm,
                                                             const uint16_t* __restrict__ V,
                                                             uint32_t* __restrict__ part) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int U = 8;        // loads in flight per thread
  __shared__ uint32_t red[kPackThreads / 64];
  const int id = (int)blockIdx.x;
  const int c = id % kVmaxParts, bg = id / kVmaxParts;
  const int g = bg % dm.Hkv, b = bg / dm.Hkv;
  const int R = (dm.N + kVmaxParts - 1) / kVmaxParts;
  const int q0 = min(dm.N, c * R) * CPR, q1 = min(dm.N, (c + 1) * R) * CPR;
  const uint16_t* base = V + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const size_t rstride = (size_t)dm.Hkv * D;
  uint32_t mx = 0;
  for (int q = q0 + (int)threadIdx.x; q < q1; q += U * kPackThreads) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int qq = min(q + u * kPackThreads, q1 - 1);  // a repeated chunk changes no maximum
      v[u] = load_nt16(base + (size_t)(qq / CPR) * rstride + (qq % CPR) * 8);  // read once
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mx = max(mx, absmax8(v[u]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
#pragma unroll
    for (int w = 1; w < kPackThreads / 64; ++w) m = max(m, red[w]);
    part[id] = m;
  }
}

// The power-of-two exponent e of a (batch, kv head) from its largest magnitude (15-bit bf16
// pattern): |v|max * 2^e lies in [2^14, 2^15); 0 when every value is zero.
__device__ __forceinline__ int value_exponent(uint32_t mbits) {
  if (mbits == 0) return 0;
  int ex;
  (void)frexpf(bf16_bits_to_f32(mbits), &ex);  // |v|max = f 2^ex, f in [0.5, 1)
  return 15 - ex;
}

// V [B, N, Hkv, D] bf16 -> fp16 V^T step images [B, Hkv, N / 32] x (D x 32), each value
// multiplied by its head's 2^e, one workgroup per step; the head's first step also writes e to
// vexp[b Hkv + g].
template <int D>
__global__ __launch_bounds__(kPackThreads) void pack_v(Dims dm, const uint16_t* __restrict__ V,
                                                       const uint32_t* __restrict__ part,
                                                       uint16_t* __restrict__ Vp,
                                                       int32_t* __restrict__ vexp) {
  constexpr int RS = D + 2;  // LDS row stride (elements)
  __shared__ uint16_t sv[kStep * RS];
  __shared__ int s_e;
  const int steps = dm.N / kStep;
  const int id = (int)blockIdx.x;  // (b * Hkv + g) * steps + s
  const int s = id % steps;
  const int bg = id / steps;
  const int g = bg % dm.Hkv, b = bg / dm.Hkv;
  if (threadIdx.x < 64) {
    static_assert(kVmaxParts == 64, "one partial maximum per lane");
    uint32_t m = part[(size_t)bg * kVmaxParts + threadIdx.x];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (threadIdx.x == 0) {
      const int e = value_exponent(m);
      s_e = e;
      if (s == 0) vexp[bg] = e;
    }
  }
  const uint16_t* src = V + (((size_t)b * dm.N + (size_t)s * kStep) * dm.Hkv + g) * D;
  for (int c = threadIdx.x; c < kStep * D / 8; c += kPackThreads) {
    const int r = c / (D / 8), col = c - r * (D / 8);
    const uint4 v = load_nt16(src + (size_t)r * dm.Hkv * D + col * 8);  // V is read once
    uint32_t* dst = reinterpret_cast<uint32_t*>(sv + r * RS + col * 8);
    dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
  }
  __syncthreads();
  const int e = s_e;
  uint4* out = reinterpret_cast<uint4*>(Vp + (size_t)id * D * kStep);
  for (int i = threadIdx.x; i < D * 4; i += kPackThreads) {
    const int d = i >> 2, pos = i & 3;
    const int c = pos ^ vswz(d);
    const int key0 = 16 * (c >> 1) + 4 * (c & 1);  // keys key0 + (0..3), key0 + 8 + (0..3)
    float x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // exact: a power-of-two scaling that stays below 2^15
      x[k] = ldexpf(bf16_bits_to_f32(sv[(key0 + k) * RS + d]), e);
      x[4 + k] = ldexpf(bf16_bits_to_f32(sv[(key0 + 8 + k) * RS + d]), e);
    }
    uint32_t wv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f16x2 h2 = __builtin_convertvector((f32x2){x[2 * k], x[2 * k + 1]}, f16x2);
      wv[k] = __builtin_bit_cast(uint32_t, h2);
    }
    out[i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// --------------------------------------------------------------------------- attn_bf16

// D head dim, QH 32-row query groups per wave, NW waves per workgroup, HPW query heads per
// workgroup (two only with lists shared by a kv head's query heads: then one K/V stream feeds
// both heads' waves).
template <int D, int QH, int NW, int HPW = 1, int KB = 0>
struct Cfg {
  static constexpr int ROWS = 32 * QH * NW / HPW;  // query tile rows
  static constexpr int BLK = KB ? KB : ROWS;       // keys per block: the tile rows, or half or twice
  static constexpr int WPH = NW / HPW;             // waves per query head
  static constexpr int NSUB = BLK / kStep;     // steps per block
  static constexpr int DC = D / 16;            // 16-coordinate chunks of the S^T products
  static constexpr int DT = D / 32;            // 32-coordinate tiles of O^T
  static constexpr int KSLOT = kStep * D * 2;  // bytes of a K step image
  static constexpr int VSLOT = D * kStep * 2;  // bytes of a V^T step image
  // 4-wave workgroups: a ring of NR = 3 slots, each a K and a V^T image, refilled a whole
  // slot at a time (three workgroups per CU).
  // 2-wave workgroups (SPLIT): a ring of three single images, K and V^T of consecutive steps
  // in turn (image 2i is step i's K, image 2i + 1 its V^T, image m in buffer m % 3).  Step i's
  // K buffer is refilled with step i + 1's V^T once every wave's S products are done, and
  // step i's V^T buffer with step i + 2's K once its P V^T products are, so each image still
  // has a whole step to land, in 24 KiB instead of the 32 KiB of two full slots: six such
  // workgroups share a CU (three waves per SIMD) instead of four.
  static constexpr bool SPLIT = NW == 2;
  static constexpr int NR = 3;  // slots of the 4-wave ring (a split ring is three images)
  static constexpr int RING = SPLIT ? 3 * KSLOT : NR * (KSLOT + VSLOT);  // bytes
  static constexpr int KREG = KSLOT / 1024;    // 1 KiB load regions per image
  static constexpr int VREG = VSLOT / 1024;
  static constexpr int LPW = (KREG + VREG) / NW;  // loads per wave per refill group
  static constexpr int LPI = KREG / NW;           // loads per wave per image (SPLIT)
  static_assert(KREG % NW == 0 && VREG % NW == 0, "load regions must split evenly");
  static_assert(!SPLIT || KSLOT == VSLOT, "split-ring buffers hold either image");
  static constexpr int LCAP = 512;             // list entries staged in LDS per segment
  // Waves per SIMD the register allocation must allow: three for 32-row waves (168
  // registers), two for 64-row waves (256).
  static constexpr int WPE = QH == 1 ? 3 : 2;
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS byte address of a pointer into a __shared__ object, and reads at a raw LDS address
// (one address register per read, any constant offset folded into the instruction).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr)p;
}
template <typename T>
__device__ __forceinline__ T lds_read(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>((uintptr_t)addr);
}

// Direct global -> LDS load: lane i's 16 bytes at gbase + voff (bytes) land at LDS address
// m0 + 16 i.  gbase and lds are wave-uniform.  Inline asm keeps these loads out of the
// compiler's own wait insertion, which cannot tell which ring slot a later LDS read touches
// and would drain every load in flight before it; each wait for them is explicit (wait_vm
// followed by a barrier).  The s_nop is the one wait state an LDS-DMA load needs after M0
// is written.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone), as the builtin so that the compiler's
// own wait insertion knows which earlier loads have completed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Workgroup barrier without the full memory drain __syncthreads() implies: loads still in
// flight into other ring slots stay in flight.  Every LDS read before it has been consumed
// by then (its value fed a product that precedes the barrier).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// A row's running maximum is only raised when a new logit exceeds it by more than this many
// powers of two; until then probabilities may reach 2^kLazy, which fp16 P and the fp32
// accumulators hold exactly enough, and the rescale of O is skipped.
constexpr float kLazy = 8.0f;

// Per query row (lane-local, QH rows per lane): the running maximum m of the raw logits is
// kept as two derived values, with c = scale log2 e:
//   thr = m + kLazy / c  the raw logit above which m is raised (-inf while no key was seen),
//   mc  = -m c           the exponent offset of P = 2^(s c + mc) (0 while no key was seen).
template <int D, int QH>
struct WaveState {
  f32x16 acc_o[QH][D / 32];
  float l_run[QH];
  float thr[QH];
  float mc[QH];
};

// max of x over lanes l and l ^ 32 for values that are never NaN (logits, or -inf): a compare
// and a select, without the quieting fmaxf adds for values it cannot see the origin of.
__device__ __forceinline__ float pair_max_num(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return a > b ? a : b;
}

// Operand reads issued ahead of the products that use them: four when a read feeds one
// product, two when it feeds two (fewer registers held for 64-row waves).
template <int QH>
constexpr int kReadAhead = QH == 1 ? 4 : 2;

// S^T for one step: QH accumulators of 32 keys x 32 query rows.  Each K chunk read from LDS
// feeds QH products.  ka_addr[c] is this lane's address of chunk 2c + hi in ring slot 0 (kept
// in registers for the whole kernel) and slotoff the step's slot offset, a compile-time
// constant in the unrolled step loop that the read instruction takes as its immediate.
template <int D, int QH>
__device__ __forceinline__ void step_scores(const uint32_t (&ka_addr)[D / 16], uint32_t slotoff,
                                            const bf16x8 (&qf)[QH][D / 16], f32x16 (&s)[QH]) {
  constexpr int DC = D / 16, PD = kReadAhead<QH>;
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) s[qh] = (f32x16){};
  bf16x8 ka[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) ka[i] = lds_read<bf16x8>(ka_addr[i] + slotoff);
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
      s[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c % PD], qf[qh][c], s[qh], 0, 0, 0);
    if (c + PD < DC) ka[c % PD] = lds_read<bf16x8>(ka_addr[c + PD] + slotoff);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Online softmax of one step's logits (masked on the diagonal block) and O^T += V^T P^T.
// va_addr as ka_addr in step_scores (slot 0, loop-invariant), slotoff the offset of the step's
// V^T image from there.  pre_pv() runs between the softmax and the first V^T operand read
// (a split ring's wait for that image).
template <int D, int QH, typename PrePv>
__device__ __forceinline__ void step_softmax_pv(f32x16 (&s)[QH], const uint32_t (&va_addr)[2],
                                                uint32_t slotoff, WaveState<D, QH>& st,
                                                bool diag, int kbase, int qbase, int hi,
                                                float scale_log2, float lazy_raw,
                                                PrePv&& pre_pv) {
  constexpr int DT = D / 32;
  // Lane value v of s[qh] is key kbase + 8 (v >> 2) + 4 hi + (v & 3) of the tile, query row
  // qbase + 32 qh (+ lane % 32).
  if (diag) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kloc = kbase + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (kloc > qbase + 32 * qh) s[qh][v] = -INFINITY;
      }
  }
  // The row maximum is raised only when a logit passes thr (lazy rescaling, rare once the
  // first blocks are in); the common path is the maximum, one compare and one vote.
  float mloc[QH];
  bool any_raise = false;
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[qh][v]);
    mloc[qh] = pair_max_num(mx);
    any_raise |= mloc[qh] > st.thr[qh];
  }
  if (__any(any_raise)) {
#pragma unroll
    for (int qh = 0; qh < QH; ++qh) {
      const bool raise = mloc[qh] > st.thr[qh];
      const float mc_new = raise ? -mloc[qh] * scale_log2 : st.mc[qh];
      // O and l scale by 2^((m - m_new) c) = 2^(mc_new - mc); nothing was accumulated yet
      // while thr is -inf
      const float alpha = !raise ? 1.0f
                          : st.thr[qh] == -INFINITY
                              ? 0.0f
                              : __builtin_amdgcn_exp2f(mc_new - st.mc[qh]);
      st.l_run[qh] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st.acc_o[qh][dt] *= alpha;
      if (raise) {
        st.thr[qh] = mloc[qh] + lazy_raw;
        st.mc[qh] = mc_new;
      }
    }
  }
  f16x8 pf[QH][2];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    const float mc = st.mc[qh];
#pragma unroll
    for (int v = 0; v < 16; ++v)
      pf[qh][v >> 3][v & 7] =
          (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qh][v], scale_log2, mc));
    // Row sum of the fp16 probabilities the P V^T product uses, two per v_dot2_f32_f16 (the
    // products by 1 are exact; the sum is accumulated in fp32).
    float psum = st.l_run[qh];
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const f16x2 pp = {pf[qh][v >> 3][v & 7], pf[qh][v >> 3][(v & 7) + 1]};
      psum = __builtin_amdgcn_fdot2(pp, one, psum, false);
    }
    st.l_run[qh] = psum;
  }
  // O^T += V^T P^T.  B operand slot 8 hi + 4 i' + r of pf[qh][half] is key
  // 16 half + 8 i' + 4 hi + r of the step; the A operand is chunk 2 half + hi of V^T row d,
  // which holds exactly those keys in that order (read through va_addr[half]).
  constexpr int NP = DT * 2, PD = kReadAhead<QH>;
  auto vload = [&](int i) {
    const int dt = i >> 1, half = i & 1;
    return lds_read<f16x8>(va_addr[half] + slotoff + dt * 2048);
  };
  pre_pv();
  f16x8 va[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) va[i] = vload(i);
  // The P V^T products issue at raised wave priority: a wave that has finished its softmax
  // gets its products onto the matrix core ahead of the other waves' vector work, which then
  // fills the issue slots while those products run (1-3% faster on every 128-row-tile
  // workload; raising it for the S products too, or for the softmax instead, gained nothing).
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int dt = i >> 1, half = i & 1;
#pragma unroll
    for (int qh = 0; qh < QH; ++qh)
      st.acc_o[qh][dt] =
          __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i % PD], pf[qh][half], st.acc_o[qh][dt], 0, 0, 0);
    if (i + PD < NP) va[i % PD] = vload(i + PD);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
}

// Run by one wave.  lst[0 .. U) holds this tile's usable blocks (U = seg_info[0] <= 256);
// reorders them by (number of the kv head's query heads whose list for this tile contains the
// block) descending, then block index ascending, and updates the diagonal's position
// (seg_info[1]).  The other heads' lists are copied to `scratch` first; membership is a binary
// search, which assumes ascending lists (as sparse_attn_select writes them): other orders give
// another, still valid, order.
__device__ void reorder_shared(const int32_t* __restrict__ list, const int32_t* __restrict__ kv_cnt,
                               size_t bht, const Dims& dm, int h, int t, int W, int* lst,
                               int* seg_info, int* scratch) {
  const int lane = threadIdx.x & 63;
  const int U = seg_info[0];
  const int g0 = (h / dm.G) * dm.G;
  // other heads' lists: scratch[k * W ..], lengths in cl[k]
  int cl[8];
  int no = 0;
  for (int hh = g0; hh < g0 + dm.G && no < 8; ++hh) {
    if (hh == h) continue;
    const long long d = ((long long)hh - h) * dm.nt * W;  // same (b, t), other head
    const int c = max(0, min(kv_cnt[(size_t)((long long)bht + ((long long)hh - h) * dm.nt)], W));
    for (int e = lane; e < c; e += 64) scratch[no * W + e] = list[d + e];
    cl[no++] = c;
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  int P = 1;
  while (P < U) P <<= 1;
  unsigned* key = reinterpret_cast<unsigned*>(scratch + no * W);
  for (int i = lane; i < P; i += 64) {
    unsigned k = 0xffffffffu;  // padding sorts last
    if (i < U) {
      const int x = lst[i];
      int count = 1;
      for (int o = 0; o < no; ++o) {
        const int* sl = scratch + o * W;
        int lo = 0, hi = cl[o];
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (sl[mid] < x) lo = mid + 1; else hi = mid;
        }
        count += lo < cl[o] && sl[lo] == x;
      }
      k = ((unsigned)(dm.G - count) << 24) | (unsigned)x;
    }
    key[i] = k;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  // ascending bitonic sort of key[0 .. P) by this wave (its LDS accesses execute in order)
  for (int k = 2; k <= P; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = lane; i < (P >> 1); i += 64) {
        const int lo = ((i & ~(jj - 1)) << 1) | (i & (jj - 1));
        const int hi = lo + jj;
        const unsigned a = key[lo], b = key[hi];
        const bool up = (lo & k) == 0;
        if (up ? (a > b) : (a < b)) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  int diag = -1, diag2 = -1;
  const int d0 = first_diag(dm.m, dm.tpb, t);  // the tile's diagonal blocks d0 (and d0 + 1)
  for (int i = lane; i < U; i += 64) {
    const int x = (int)(key[i] & 0xffffffu);
    lst[i] = x;
    const unsigned long long dm_ = __ballot(x == d0);
    if (dm_) diag = (i - lane) + __builtin_ctzll(dm_);
    const unsigned long long dm2 = __ballot(dm.m > 1 && x == d0 + 1);
    if (dm2) diag2 = (i - lane) + __builtin_ctzll(dm2);
  }
  if (lane == 0) {
    seg_info[1] = diag;
    seg_info[4] = diag2;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Stages the next segment of a tile's list in LDS and orders it; run by the whole workgroup.
// Usable entries are the tile's causal blocks (0 <= j < d0 + m, d0 = first_diag(t), m = 1 or 2
// diagonal blocks per tile) before the first negative entry; at most LCAP of them per segment
// (wave 0 compacts, the workgroup waits).  seg_info receives: usable entries, position of the
// first diagonal block d0 (-1 if absent), the list position the next segment starts at, whether
// this segment ends the list, and the position of the second diagonal block m t + 1.
//
// Single-segment lists are then ordered so that blocks listed by more of the kv head's query
// heads come first (ties by index): the G workgroups of the tile run together on one XCD and
// request their shared blocks at the same steps.  Attention does not depend on the order.
// `scratch` (scratch_ints ints of LDS, free at this point) holds the other heads' lists.
template <int LCAP>
__device__ __forceinline__ void stage_segment(const int32_t* __restrict__ list,
                                              const int32_t* __restrict__ kv_cnt, int cnt,
                                              size_t bht, const Dims& dm, int h, int t, int W,
                                              int seg_start, int w, int lane, int* lst,
                                              int* seg_info, int* scratch, int scratch_ints) {
  // the tile's diagonal blocks: d0 (and d0 + 1 for tiles of two blocks); causal ones < dend
  const int d0 = first_diag(dm.m, dm.tpb, t), dend = d0 + dm.m;
  if (w == 0) {
    int u = 0, base = seg_start, diag = -1, diag2 = -1, next = cnt, done = 1;
    while (base < cnt) {
      const int e = base + lane;
      const int x = e < cnt ? list[e] : 0;
      const unsigned long long negm = __ballot(e < cnt && x < 0);
      const int first_neg = negm ? __builtin_ctzll(negm) : 64;
      const bool valid = e < cnt && lane < first_neg && x < dend;
      const unsigned long long vm = __ballot(valid);
      const int pre = __builtin_popcountll(vm & ((1ull << lane) - 1ull));
      const int nv = __builtin_popcountll(vm);
      const int fit = min(nv, LCAP - u);
      if (valid && pre < fit) lst[u + pre] = x;
      // entries are distinct, so at most one lane holds each diagonal block
      const unsigned long long dm_ = __ballot(valid && pre < fit && x == d0);
      if (dm_) diag = u + (int)__builtin_popcountll(vm & ((1ull << __builtin_ctzll(dm_)) - 1ull));
      const unsigned long long dm2 = __ballot(valid && pre < fit && x == d0 + 1);
      if (dm2) diag2 = u + (int)__builtin_popcountll(vm & ((1ull << __builtin_ctzll(dm2)) - 1ull));
      u += fit;
      if (fit < nv) {  // LDS full: continue from the first entry that did not fit
        const unsigned long long om = __ballot(valid && pre == fit);
        next = base + __builtin_ctzll(om);
        done = 0;
        break;
      }
      if (negm) break;
      base += 64;
    }
    if (lane == 0) {
      seg_info[0] = u;
      seg_info[1] = diag;
      seg_info[2] = next;
      seg_info[3] = done;
      seg_info[4] = diag2;
    }
  }
  __syncthreads();
  if (dm.G > 1 && dm.gs == 1 && seg_start == 0 && seg_info[3] && seg_info[0] > 1 &&
      seg_info[0] <= 256 &&
      (dm.G - 1) * W + 256 <= scratch_ints) {
    if (w == 0) reorder_shared(list, kv_cnt, bht, dm, h, t, W, lst, seg_info, scratch);
    __syncthreads();
  }
}

// Stages the union of two lists for one workgroup, run by the whole workgroup: the lists of
// the two 64-row query tiles t and t + 1 of one 128-key block (one query head), which share
// that diagonal block and the free blocks before it.  Usable entries are as in stage_segment
// (before the first negative entry, below the tiles' causal end, at most cnt of them); a
// block in both lists appears once.  Each staged entry is the block index with a membership
// mask in bits 16-17 (bit 16 + k: list k has it), in ascending block order; the waves of a
// tile skip the products of the blocks their tile's list does not have, so each tile attends
// to exactly its own blocks.  Built as a bitmap of the causal blocks per list in `scratch`
// (2 * ceil(dend / 32) + 2 ints, just over 4 KiB at 16384 blocks), then compacted by wave 0.  seg_info as
// stage_segment's, one segment.  The host uses this only when both lists together fit in
// LCAP entries (2 W <= LCAP).
template <int LCAP>
__device__ __attribute__((noinline)) void stage_union(const int32_t* __restrict__ list0,
                                                      int cnt0, const int32_t* __restrict__ list1,
                                                      int cnt1, const Dims& dm, int t, int w,
                                                      int lane, int* lst, int* seg_info,
                                                      int* scratch) {
  const int d0 = first_diag(dm.m, dm.tpb, t), dend = d0 + dm.m;
  const int nwords = (dend + 31) >> 5;
  unsigned* bm = reinterpret_cast<unsigned*>(scratch);  // [2][nwords]
  int* fneg = scratch + 2 * nwords;                      // first negative entry per list
  const int nthr = (int)blockDim.x;
  for (int i = (int)threadIdx.x; i < 2 * nwords; i += nthr) bm[i] = 0u;
  if (threadIdx.x < 2) fneg[threadIdx.x] = 0x7fffffff;
  __syncthreads();
  for (int e = (int)threadIdx.x; e < cnt0; e += nthr)
    if (list0[e] < 0) atomicMin(&fneg[0], e);
  for (int e = (int)threadIdx.x; e < cnt1; e += nthr)
    if (list1[e] < 0) atomicMin(&fneg[1], e);
  __syncthreads();
  const int u0 = min(cnt0, fneg[0]), u1 = min(cnt1, fneg[1]);
  for (int e = (int)threadIdx.x; e < u0; e += nthr) {
    const int x = list0[e];
    if (x < dend) atomicOr(&bm[x >> 5], 1u << (x & 31));
  }
  for (int e = (int)threadIdx.x; e < u1; e += nthr) {
    const int x = list1[e];
    if (x < dend) atomicOr(&bm[nwords + (x >> 5)], 1u << (x & 31));
  }
  __syncthreads();
  if (w == 0) {
    int base_pos = 0, diag = -1;
    for (int base = 0; base < nwords; base += 64) {
      const int i = base + lane;
      const unsigned a = i < nwords ? bm[i] : 0u, c = i < nwords ? bm[nwords + i] : 0u;
      unsigned u = a | c;
      // exclusive prefix of the per-lane counts over the wave
      const int cntl = __builtin_popcount(u);
      int incl = cntl;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int pos = base_pos + incl - cntl;
      while (u) {
        const int bit = __builtin_ctz(u);
        u &= u - 1u;
        const int j = 32 * i + bit;
        const int mk = (int)((a >> bit) & 1u) | (int)(((c >> bit) & 1u) << 1);
        lst[pos] = j | (mk << 16);
        if (j == d0) diag = pos;
        ++pos;
      }
      base_pos += __shfl(incl, 63);
    }
    // at most one lane found the diagonal block
    const unsigned long long dmask = __ballot(diag >= 0);
    if (dmask) diag = __shfl(diag, __builtin_ctzll(dmask));
    if (lane == 0) {
      seg_info[0] = base_pos;
      seg_info[1] = diag;
      seg_info[2] = 0;
      seg_info[3] = 1;
      seg_info[4] = -1;
    }
  }
  __syncthreads();
}

// Appends to out the entries of row[0 .. len) before its first negative one that lie in
// [0, t], mapped by f, in row order; returns their number.  Run by one wave.
template <typename F>
__device__ __forceinline__ int compact_row(const int32_t* __restrict__ row, int len, int t,
                                           int* out, int lane, F f) {
  int n = 0;
  for (int base = 0; base < len; base += 64) {
    const int e = base + lane;
    const int x = e < len ? row[e] : -1;
    const unsigned long long negm = __ballot(e < len && x < 0);
    const int first_neg = negm ? __builtin_ctzll(negm) : 64;
    const bool valid = e < len && lane < first_neg && x <= t;
    const unsigned long long vm = __ballot(valid);
    if (valid) out[n + __builtin_popcountll(vm & ((1ull << lane) - 1ull))] = f(x);
    n += __builtin_popcountll(vm);
    if (negm) break;
  }
  return n;
}

// Stages query tile t's list from a vertical-slash index (VSPrefill page, Metodologia B.3:
// the fused kernel merges the vertical and the slash indices on the fly, with Merge Path, and
// never materialises per-tile lists).  Run by wave 0; the workgroup waits afterwards.
//   A = the vertical blocks <= t, ascending (vrow is ascending);
//   B = t - delta for the slash offsets delta <= t, kept in descending order (srow is
//       ascending);
// each element's place in the merged order is its index plus its co-rank (the number of
// smaller elements of the other list, a binary search), so a block present in both lists
// lands on two adjacent places; those and any entry outside [0, t] (only possible when the
// inputs break the ascending-and-distinct contract) are dropped, and the diagonal block t is
// appended when neither list holds it.  `scratch` holds 2 (nv + ns) ints.
__device__ void stage_vs(const int32_t* __restrict__ vrow, int nv,
                         const int32_t* __restrict__ srow, int ns, int t, int w, int lane,
                         int* lst, int* seg_info, int* scratch) {
  if (w == 0) {
    int* A = scratch;
    int* Bd = scratch + nv;
    int* M = scratch + nv + ns;
    const int na = compact_row(vrow, nv, t, A, lane, [](int x) { return x; });
    const int nb = compact_row(srow, ns, t, Bd, lane, [t](int x) { return t - x; });
    for (int p = lane; p < na + nb; p += 64) M[p] = -1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    for (int i = lane; i < na; i += 64) {  // A[i]: i + #{B < a}
      const int a = A[i];
      int lo = 0, hi = nb;  // first k with Bd[k] < a (Bd descending)
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (Bd[mid] < a) hi = mid; else lo = mid + 1;
      }
      M[i + (nb - lo)] = a;
    }
    for (int k = lane; k < nb; k += 64) {  // Bd[k] (ascending place nb-1-k): + #{A <= b}
      const int b = Bd[k];
      int lo = 0, hi = na;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (A[mid] <= b) lo = mid + 1; else hi = mid;
      }
      M[(nb - 1 - k) + lo] = b;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    int u = 0;
    for (int base = 0; base < na + nb; base += 64) {
      const int p = base + lane;
      const int x = p < na + nb ? M[p] : -1;
      const int prev = p > 0 && p < na + nb ? M[p - 1] : -1;
      const bool keep = x >= 0 && x <= t && x != prev;
      const unsigned long long km = __ballot(keep);
      if (keep) lst[u + __builtin_popcountll(km & ((1ull << lane) - 1ull))] = x;
      u += __builtin_popcountll(km);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int lastv = u > 0 ? lst[u - 1] : -1;
    if (lastv != t) {
      if (lane == 0) lst[u] = t;
      ++u;
    }
    if (lane == 0) {
      seg_info[0] = u;
      seg_info[1] = u - 1;  // the diagonal is the last (largest) block
      seg_info[2] = 0;
      seg_info[3] = 1;
      seg_info[4] = -1;
    }
  }
  __syncthreads();
}

// D head dim, QH 32-row query groups per wave, NW waves per workgroup; VS: the tile's list
// comes from a vertical-slash index (stage_vs) instead of kv_idx / kv_cnt; HPW query heads
// per workgroup (2: consecutive query heads of one kv head, which share their lists); TPW
// 64-row tiles per workgroup (2: the two tiles of a 128-key block, streamed as the union of
// their lists, stage_union).
template <int D, int QH, int NW, bool VS, int HPW, int KB, int TPW>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(Cfg<D, QH, NW, HPW, KB>::WPE))) void attn_bf16(
    Dims dm, const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ Vp, const int32_t* __restrict__ vexp,
    const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt, int W, VsIndex vs,
    float scale_log2, void* __restrict__ O, int out_f32, float* __restrict__ lse) {
  using C = Cfg<D, QH, NW, HPW, KB>;
  static_assert(HPW == 1 || !VS, "vertical-slash lists are per query head");
  static_assert(TPW == 1 || (HPW == 1 && KB == 0 && !VS && NW == 4 && QH == 1),
                "two 64-row tiles per workgroup run as one 128-row tile over its 128-key block");
  static_assert(KB == 0 || !VS, "vertical-slash lists need tile = block");
  static_assert(KB == 0 || KB == C::ROWS / 2 || KB == 2 * C::ROWS,
                "key blocks of half or twice the tile");
  constexpr int BLK = C::BLK, ROWS = C::ROWS, NSUB = C::NSUB, DC = C::DC, DT = C::DT;
  constexpr int LPW = C::LPW;
  // Ring of NR slots, each a K step image followed by a V^T step image; for 2-wave
  // workgroups three single images (Cfg::SPLIT).
  constexpr int SLOT = C::KSLOT + C::VSLOT;
  __shared__ __attribute__((aligned(1024))) char ring[C::RING];
  __shared__ int lst[C::LCAP];
  // usable entries, position of diagonal block d0, next entry, done, position of d0 + 1
  __shared__ int seg_info[5];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int wr = w % C::WPH;  // the wave's place among its head's waves
  int b, h, t;  // t: the workgroup's tile of ROWS rows
  if constexpr (HPW == 1 && TPW == 1) {
    decode_tile_grouped(dm, b, h, t);
  } else if constexpr (TPW == 2) {
    // workgroups over (batch, query head, pair of 64-row tiles) in the same order
    Dims dp = dm;
    dp.nt = dm.nt / 2;
    decode_tile_grouped(dp, b, h, t);
  } else {
    // workgroups over (batch, pair of query heads, tile) in the same order
    Dims dp = dm;
    dp.G = dm.G / HPW;
    dp.Hq = dm.Hq / HPW;
    int hp;
    decode_tile_grouped(dp, b, hp, t);
    h = hp * HPW + w / C::WPH;
  }
  const int g = h / dm.G;
  const int l32 = lane & 31, hi = lane >> 5;
  // With two lists per workgroup (two 64-row tiles, TPW), the wave's tile within the pair.
  const int pb = TPW == 2 ? w / 2 : 0;
  const int tl = TPW == 2 ? 2 * t + pb : t;  // the wave's tile in the list arrays
  const size_t bht = ((size_t)b * dm.Hu + h / dm.gs) * dm.nt + tl;  // the list's (b, unit, t)
  const int32_t* list = VS ? nullptr : kv_idx + bht * W;
  const int cnt = VS ? 0 : max(0, min(kv_cnt[bht], W));
  const int qbase = wr * 32 * QH + l32;  // this lane's first query row within the tile
  // tiles smaller than the key block: the tile's first row is rowoff keys into its diagonal
  // block
  const int rowoff = KB > ROWS ? (t % dm.tpb) * ROWS : 0;
  const int rstride = dm.Hkv * D;
  const uint16_t* Kg = K + ((size_t)b * dm.N * dm.Hkv + g) * D;
  const uint16_t* Vpg = Vp + ((size_t)b * dm.Hkv + g) * (size_t)dm.N * D;

  // Q fragments (B operand of S^T = K Q^T): lane holds coordinates 16c + 8 hi .. +7 of row
  // qbase + 32 qh.
  bf16x8 qf[QH][DC];
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    const uint16_t* qp =
        Q + (((size_t)b * dm.N + (size_t)t * ROWS + qbase + 32 * qh) * dm.Hq + h) * D + 8 * hi;
#pragma unroll
    for (int c = 0; c < DC; ++c) qf[qh][c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c);
  }
  // Use the fragments once here so that the compiler waits for them now, before the K/V
  // stream is in flight, rather than draining that stream at the first product.
#pragma unroll
  for (int qh = 0; qh < QH; ++qh)
#pragma unroll
    for (int c = 0; c < DC; ++c) asm volatile("" ::"v"(qf[qh][c]));
  WaveState<D, QH> st;
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc_o[qh][dt] = (f32x16){};
    st.l_run[qh] = 0.0f;
    st.thr[qh] = -INFINITY;
    st.mc[qh] = 0.0f;
  }
  const float lazy_raw = kLazy / scale_log2;  // kLazy in raw logit units (scale > 0)

  // Per-lane LDS read offsets within a slot: K chunk hi of row l32 and V^T chunk hi of row l32.
  // Chunk positions are chunk indices XOR a per-row value (kswz, vswz), so chunk 2c + hi sits
  // at koff ^ 32 c, and V^T chunk 2 + hi at voff ^ 32; slots are 1 KiB aligned, so the same
  // holds for the LDS addresses.  The addresses in ring slot 0 stay in registers for the whole
  // kernel; a step adds its slot's offset as the read instruction's immediate.
  const int koff = l32 * 2 * D + 16 * (hi ^ kswz<D>(l32));
  const int voff = l32 * 64 + 16 * (hi ^ vswz(l32));
  uint32_t ka_addr[DC], va_addr[2];
  {
    const uint32_t ring0 = lds_addr(ring);
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      ka_addr[c] = ring0 + ((uint32_t)koff ^ (32u * c));
      asm volatile("" : "+v"(ka_addr[c]));
    }
    // (a split ring's buffers hold either image: V^T offsets then start at the ring's base)
    const uint32_t vbase0 = ring0 + (C::SPLIT ? 0u : (uint32_t)C::KSLOT);
    va_addr[0] = vbase0 + (uint32_t)voff;
    va_addr[1] = vbase0 + ((uint32_t)voff ^ 32u);
    asm volatile("" : "+v"(va_addr[0]), "+v"(va_addr[1]));
  }
  // Per-lane source offsets (elements, relative to a step's first key row) of this wave's K
  // regions: region w + NW k, lane i lands at image byte 1024 (w + NW k) + 16 i.
  int kgo[C::KREG / NW];
#pragma unroll
  for (int k = 0; k < C::KREG / NW; ++k) {
    const int off = (w + NW * k) * 1024 + 16 * lane;
    const int r = off / (2 * D), p = (off % (2 * D)) / 16;
    kgo[k] = 2 * (r * rstride + 8 * (p ^ kswz<D>(r)));  // bytes
  }
  const uint32_t vlo = 16 * lane;  // V^T images are copied verbatim

  int seg_start = 0;
  for (;;) {
    if constexpr (VS) {
      const size_t bh = (size_t)b * dm.Hq + h;
      stage_vs(vs.vert + bh * vs.nv, vs.nv, vs.slash + bh * vs.ns, vs.ns, t, w, lane, lst,
               seg_info, reinterpret_cast<int*>(ring));
    } else if constexpr (TPW == 2) {
      const size_t bht0 = bht - pb;  // the pair's first tile
      stage_union<C::LCAP>(kv_idx + bht0 * W, max(0, min(kv_cnt[bht0], W)),
                           kv_idx + (bht0 + 1) * W, max(0, min(kv_cnt[bht0 + 1], W)), dm,
                           2 * t, w, lane, lst, seg_info, reinterpret_cast<int*>(ring));
    } else {
      stage_segment<C::LCAP>(list, kv_cnt, cnt, bht, dm, h, t, W, seg_start, w, lane, lst,
                             seg_info, reinterpret_cast<int*>(ring), C::RING / 4);
    }
    const int U = seg_info[0], diag_e = seg_info[1], next_start = seg_info[2];
    const int diag_e2 = KB ? seg_info[4] : -1;  // second diagonal block (128-row tiles)
    const int seg_done = seg_info[3];
    const int nsteps = U * NSUB;

    if (nsteps > 0) {
      // Refills: steps past the end reload the last step (valid memory, into a slot or buffer
      // nobody reads again) so that every refill issues the same loads per wave, which the
      // partial waits below count on.
      // Scalar address arithmetic is kept to 32-bit unsigned sums and shifts: byte offsets
      // within this (batch, kv head)'s K rows and V^T images are below 2^32 (the host checks
      // N * Hkv * d * 2 < 2^32), and the ring slots of a step are carried, not divided out.
      const uint32_t ring_lds = lds_addr(ring);
      const uint32_t last = (uint32_t)nsteps - 1;
      const uint32_t kblk_bytes = (uint32_t)(BLK * rstride * 2);
      const uint32_t kstep_bytes = (uint32_t)(kStep * rstride * 2);
      const char* kbase = reinterpret_cast<const char*>(Kg);
      const char* vbase = reinterpret_cast<const char*>(Vpg) + 1024 * w;
      // (union entries carry a membership mask above bit 15; block indices stay below 2^15)
      auto entry_of = [&](uint32_t m) {
        const int x = lst[min(m, last) / NSUB];
        return TPW == 2 ? x & 0xffff : x;
      };
      // K step m's and V^T step m's global sources (scalar bases) for block jv
      auto k_src = [&](uint32_t m, int jv) {
        const uint32_t a = min(m, last);
        const uint32_t j = (uint32_t)__builtin_amdgcn_readfirstlane(jv);  // uniform: SGPR
        return kbase + (j * kblk_bytes + (a % NSUB) * kstep_bytes);
      };
      auto v_src = [&](uint32_t m, int jv) {
        const uint32_t a = min(m, last);
        const uint32_t j = (uint32_t)__builtin_amdgcn_readfirstlane(jv);
        return vbase + (j * NSUB + a % NSUB) * (uint32_t)C::VSLOT;
      };
      // LDS byte offset of this wave's first region in the ring at `off`; the ring base is
      // re-derived here rather than kept per slot in scalar registers across the unrolled loop
      auto ring_dst = [&](uint32_t off) {
        uint32_t rb = ring_lds;
        asm volatile("" : "+s"(rb));
        return rb + off + w * 1024;
      };
      auto issue_k = [&](uint32_t m, int jv, uint32_t off) {
        const char* kb = k_src(m, jv);
        const uint32_t dst = ring_dst(off);
#pragma unroll
        for (int k = 0; k < C::KREG / NW; ++k) dma16(kb, kgo[k], dst + NW * k * 1024);
      };
      auto issue_v = [&](uint32_t m, int jv, uint32_t off) {
        const char* vb = v_src(m, jv);
        const uint32_t dst = ring_dst(off);
#pragma unroll
        for (int k = 0; k < C::VREG / NW; ++k) dma16(vb + NW * k * 1024, vlo, dst + NW * k * 1024);
      };
      // Step i's geometry for this wave: whether it computes the step at all, whether the step
      // lies on a diagonal block (masked), and its key offset from the tile's first row there.
      struct StepGeo {
        bool run, diag;
        int kofs;
      };
      auto geometry = [&](uint32_t i) {
        const int e = (int)(i / NSUB), sub = (int)(i % NSUB);
        // key offset of the step from the tile's first row, on the diagonal blocks (the
        // second one starts BLK keys in); -1 elsewhere
        int kofs;
        bool diag;
        if constexpr (KB == 0) {
          diag = e == diag_e;
          kofs = sub * kStep;
        } else if constexpr (KB < ROWS) {
          kofs = e == diag_e ? sub * kStep : (e == diag_e2 ? BLK + sub * kStep : -1);
          diag = kofs >= 0;
        } else {  // the tile's rows lie inside its diagonal block, rowoff keys in: steps
                  // wholly before them need no mask
          kofs = sub * kStep - rowoff;
          diag = e == diag_e && kofs > -kStep;
        }
        // On a diagonal block, a step whose first key lies after this wave's last row is
        // fully masked for the wave: skip it.
        // With the union of two tiles' lists, a block the wave's tile did not select.
        const bool other =
            TPW == 2 && !((__builtin_amdgcn_readfirstlane(lst[e]) >> (16 + pb)) & 1);
        return StepGeo{!other && (!diag || kofs < kStep * QH * (wr + 1)), diag, kofs};
      };

      if constexpr (C::SPLIT) {
        // Image m in buffer m % 3 (2i: step i's K, 2i + 1: its V^T).  Step i: wait for its K
        // (its V^T may still be in flight), barrier (every wave's part of the K image is in,
        // and every wave is done with step i-1's P V^T products, whose buffer the next K
        // overwrites), issue step i+1's K, S products and softmax; then wait for its V^T
        // (step i+1's K may still be in flight), barrier (every wave is done with step i's S
        // products), issue step i+1's V^T into step i's K buffer, P V^T products.  A wave that
        // skips the step still takes part in both barriers and issues.  Unrolled by 3, so
        // every buffer is a compile-time constant.
        constexpr uint32_t IB = (uint32_t)C::KSLOT;
        issue_k(0, entry_of(0), 0);
        issue_v(0, entry_of(0), IB);
        int jn = entry_of(1);  // block of step i + 1
        for (uint32_t i0 = 0; i0 <= last; i0 += 3) {
#pragma unroll
          for (int r = 0; r < 3; ++r) {
            const uint32_t i = i0 + r;
            if (i > last) break;
            wait_vm<C::LPI>();
            barrier_only();
            issue_k(i + 1, jn, (uint32_t)((2 * r + 2) % 3) * IB);
            auto pre_pv = [&] {
              wait_vm<C::LPI>();
              barrier_only();
              issue_v(i + 1, jn, (uint32_t)((2 * r) % 3) * IB);
              jn = entry_of(i + 2);
            };
            const StepGeo gs = geometry(i);
            if (gs.run) {
              f32x16 sc[QH];
              step_scores<D, QH>(ka_addr, (uint32_t)((2 * r) % 3) * IB, qf, sc);
              step_softmax_pv<D, QH>(sc, va_addr, (uint32_t)((2 * r + 1) % 3) * IB, st, gs.diag,
                                     gs.kofs, qbase, hi, scale_log2, lazy_raw, pre_pv);
            } else {
              pre_pv();
            }
          }
        }
      } else {
        // Refill group m: K step m and V step m into ring slot m % NR.
        auto issue = [&](uint32_t m, int jv, uint32_t slot_idx) {
          issue_k(m, jv, slot_idx * SLOT);
          issue_v(m, jv, slot_idx * SLOT + C::KSLOT);
        };
#pragma unroll
        for (int m = 0; m < C::NR - 1; ++m) issue(m, entry_of(m), m);
        int jn = entry_of(C::NR - 1);  // block of the next group, read one step early

        // Step i (slot i % NR): wait until group i has landed (groups i+1 .. i+NR-2 may still
        // be in flight), barrier (every wave's part of group i is in, and every wave is done
        // with step i-1, whose slot the new group overwrites), issue group i+NR-1, then
        // compute step i.  The loop is unrolled by NR, so each step's slot (read and refilled)
        // is a compile-time constant.
        for (uint32_t i0 = 0; i0 <= last; i0 += C::NR) {
#pragma unroll
          for (int r = 0; r < C::NR; ++r) {
            const uint32_t i = i0 + r;
            if (i > last) break;
            wait_vm<(C::NR - 2) * LPW>();
            barrier_only();
            issue(i + C::NR - 1, jn, (uint32_t)((r + C::NR - 1) % C::NR));
            jn = entry_of(i + C::NR);
            const uint32_t slotoff = (uint32_t)(r * SLOT);
            const StepGeo gs = geometry(i);
            if (gs.run) {
              f32x16 sc[QH];
              step_scores<D, QH>(ka_addr, slotoff, qf, sc);
              step_softmax_pv<D, QH>(sc, va_addr, slotoff, st, gs.diag, gs.kofs, qbase, hi,
                                     scale_log2, lazy_raw, [] {});
            }
          }
        }
      }
      wait_vm<0>();  // dummy refills still in flight must land before the slots are reused
    }
    __syncthreads();
    if (seg_done) break;
    seg_start = next_start;
  }

  const int ve = -vexp[(size_t)b * dm.Hkv + g];  // undoes pack_v's 2^e of this kv head
#pragma unroll
  for (int qh = 0; qh < QH; ++qh) {
    const float l_tot = pair_sum(st.l_run[qh]);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    const int qrow = t * ROWS + qbase + 32 * qh;
    const size_t orow = (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = dt * 32 + 8 * i + 4 * hi;
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = ldexpf(st.acc_o[qh][dt][4 * i + r] * inv, ve);
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
          l_tot > 0.0f ? (__log2f(l_tot) - st.mc[qh]) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------- fp32 (VALU) path

// One thread per query row of a TR-row tile; blocks of KB keys staged in LDS.
template <int D, int TR, int KB>
__global__ __launch_bounds__(TR) void attn_f32(Dims dm, const float* __restrict__ Q,
                                                const float* __restrict__ K,
                                                const float* __restrict__ V,
                                                const int32_t* __restrict__ kv_idx,
                                                const int32_t* __restrict__ kv_cnt, int W,
                                                float scale, void* __restrict__ O, int out_f32,
                                                float* __restrict__ lse) {
  extern __shared__ float fsm[];
  float* Kb = fsm;           // [KB][D]
  float* Vb = fsm + KB * D;  // [KB][D]
  int b, h, t;
  decode_tile(dm, b, h, t);
  const int g = h / dm.G;
  const size_t bht = ((size_t)b * dm.Hu + h / dm.gs) * dm.nt + t;  // the list's (b, unit, t)
  const int32_t* list = kv_idx + bht * W;
  const int cnt = min(kv_cnt[bht], W);
  const int qrow = t * TR + threadIdx.x;
  const int jmax = first_diag(dm.m, dm.tpb, t) + dm.m - 1;  // the tile's last causal block
  const int rstride = dm.Hkv * D;

  float q[D], o[D];
  const float* qp = Q + (((size_t)b * dm.N + qrow) * dm.Hq + h) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = qp[c];
    o[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int e = next_entry(list, cnt, 0, jmax); e >= 0; e = next_entry(list, cnt, e + 1, jmax)) {
    const int j = list[e];
    const size_t row0 = (size_t)b * dm.N + (size_t)j * KB;
    for (int x = threadIdx.x; x < KB * D; x += TR) {
      const int r = x / D, c = x - r * D;
      Kb[x] = K[(row0 + r) * rstride + (size_t)g * D + c];
      Vb[x] = V[(row0 + r) * rstride + (size_t)g * D + c];
    }
    __syncthreads();
    for (int r = 0; r < KB; ++r) {
      if ((size_t)j * KB + r > (size_t)qrow) break;
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

template <int D>
hipError_t launch_prepare(const Dims& dm, const void* V, void* ws, hipStream_t s) {
  const ForwardWs L = forward_ws_layout(dm);
  char* base = static_cast<char*>(ws);
  uint32_t* part = reinterpret_cast<uint32_t*>(base + L.part);
  hipLaunchKernelGGL((value_absmax<D>), dim3((unsigned)((size_t)dm.B * dm.Hkv * kVmaxParts)),
                     dim3(kPackThreads), 0, s, dm, static_cast<const uint16_t*>(V), part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nsteps = (unsigned)((size_t)dm.B * dm.Hkv * (dm.N / kStep));
  hipLaunchKernelGGL((pack_v<D>), dim3(nsteps), dim3(kPackThreads), 0, s, dm,
                     static_cast<const uint16_t*>(V), part,
                     reinterpret_cast<uint16_t*>(base + L.vp),
                     reinterpret_cast<int32_t*>(base + L.vexp));
  return hipGetLastError();
}

template <int D, int QH, int NW, bool VS, int HPW = 1, int KB = 0, int TPW = 1>
hipError_t launch_bf16(const Dims& dm, const void* Q, const void* K, const int32_t* kv_idx,
                       const int32_t* kv_cnt, int W, const VsIndex& vs, float scale,
                       const void* ws, void* O, int out_dtype, float* lse, hipStream_t s) {
  const ForwardWs L = forward_ws_layout(dm);
  const char* base = static_cast<const char*>(ws);
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hq / HPW * dm.nt / TPW);
  hipLaunchKernelGGL((attn_bf16<D, QH, NW, VS, HPW, KB, TPW>), dim3(grid), dim3(64 * NW), 0, s, dm,
                     static_cast<const uint16_t*>(Q), static_cast<const uint16_t*>(K),
                     reinterpret_cast<const uint16_t*>(base + L.vp),
                     reinterpret_cast<const int32_t*>(base + L.vexp), kv_idx, kv_cnt, W, vs,
                     scale * kLog2e, O, out_dtype == SA_F32 ? 1 : 0, lse);
  return hipGetLastError();
}

template <int D, int TR, int KB>
hipError_t launch_f32(const Dims& dm, const void* Q, const void* K, const void* V,
                      const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                      void* O, int out_dtype, float* lse, hipStream_t s) {
  const unsigned grid = (unsigned)((size_t)dm.B * dm.Hq * dm.nt);
  const size_t lds = sizeof(float) * 2 * KB * D;
  hipError_t e = allow_lds(attn_f32<D, TR, KB>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_f32<D, TR, KB>), dim3(grid), dim3(TR), lds, s, dm,
                     static_cast<const float*>(Q), static_cast<const float*>(K),
                     static_cast<const float*>(V), kv_idx, kv_cnt, W, scale, O,
                     out_dtype == SA_F32 ? 1 : 0, lse);
  return hipGetLastError();
}

template <bool VS>
hipError_t launch_bf16_shape(const Dims& dm, const void* Q, const void* K, const int32_t* kv_idx,
                             const int32_t* kv_cnt, int W, const VsIndex& vs, float scale,
                             const void* ws, void* O, int out_dtype, float* lse, hipStream_t s) {
  if constexpr (!VS) {
    // 64-row tiles inside 128-key blocks, both lists of a block's two tiles fitting the
    // staging area together: one 4-wave workgroup per block streams the union of the two
    // lists (each tile's waves skip the other's blocks), as a 128-row tile would.
    if (dm.tpb == 2 && dm.nt % 2 == 0 && 2 * W <= Cfg<128, 1, 4>::LCAP)
      return dm.d == 64 ? launch_bf16<64, 1, 4, false, 1, 0, 2>(dm, Q, K, kv_idx, kv_cnt, W, vs,
                                                                scale, ws, O, out_dtype, lse, s)
                        : launch_bf16<128, 1, 4, false, 1, 0, 2>(dm, Q, K, kv_idx, kv_cnt, W,
                                                                 vs, scale, ws, O, out_dtype,
                                                                 lse, s);
    // Otherwise two waves per tile, four steps per block.
    if (dm.tpb == 2)
      return dm.d == 64 ? launch_bf16<64, 1, 2, false, 1, 128>(dm, Q, K, kv_idx, kv_cnt, W, vs,
                                                               scale, ws, O, out_dtype, lse, s)
                        : launch_bf16<128, 1, 2, false, 1, 128>(dm, Q, K, kv_idx, kv_cnt, W, vs,
                                                                scale, ws, O, out_dtype, lse, s);
    // 128-row tiles over 64-key blocks: four waves per tile, two steps per block.
    if (dm.m == 2)
      return dm.d == 64 ? launch_bf16<64, 1, 4, false, 1, 64>(dm, Q, K, kv_idx, kv_cnt, W, vs,
                                                              scale, ws, O, out_dtype, lse, s)
                        : launch_bf16<128, 1, 4, false, 1, 64>(dm, Q, K, kv_idx, kv_cnt, W, vs,
                                                               scale, ws, O, out_dtype, lse, s);
    // 64-row tiles whose lists a kv head's query heads share (an even number of them): two
    // heads per workgroup, so each K/V step in LDS feeds four waves instead of two.
    if (dm.blk == 64 && dm.gs > 1 && dm.gs % 2 == 0)
      return dm.d == 64 ? launch_bf16<64, 1, 4, false, 2>(dm, Q, K, kv_idx, kv_cnt, W, vs, scale,
                                                          ws, O, out_dtype, lse, s)
                        : launch_bf16<128, 1, 4, false, 2>(dm, Q, K, kv_idx, kv_cnt, W, vs, scale,
                                                           ws, O, out_dtype, lse, s);
  }
  if (dm.d == 64)
    return dm.blk == 64 ? launch_bf16<64, 1, 2, VS>(dm, Q, K, kv_idx, kv_cnt, W, vs, scale, ws, O,
                                                    out_dtype, lse, s)
                        : launch_bf16<64, ATTN_QH, 4 / ATTN_QH, VS>(dm, Q, K, kv_idx, kv_cnt, W,
                                                                    vs, scale, ws, O, out_dtype,
                                                                    lse, s);
  if (dm.blk == 64)
    return launch_bf16<128, 1, 2, VS>(dm, Q, K, kv_idx, kv_cnt, W, vs, scale, ws, O, out_dtype,
                                      lse, s);
  return launch_bf16<128, ATTN_QH, 4 / ATTN_QH, VS>(dm, Q, K, kv_idx, kv_cnt, W, vs, scale, ws, O,
                                                    out_dtype, lse, s);
}

}  // namespace

hipError_t launch_prepare_values(const Dims& dm, const void* V, void* ws, hipStream_t s) {
  return dm.d == 64 ? launch_prepare<64>(dm, V, ws, s) : launch_prepare<128>(dm, V, ws, s);
}

hipError_t launch_forward_prepared(const Dims& dm, const void* Q, const void* K,
                                   const void* ws, const int32_t* kv_idx,
                                   const int32_t* kv_cnt, int W, float scale, void* O,
                                   int out_dtype, float* lse, hipStream_t s) {
  return launch_bf16_shape<false>(dm, Q, K, kv_idx, kv_cnt, W, VsIndex{}, scale, ws, O,
                                  out_dtype, lse, s);
}

hipError_t launch_forward(const Dims& dm, const void* Q, const void* K, const void* V,
                          const int32_t* kv_idx, const int32_t* kv_cnt, int W, float scale,
                          void* ws, void* O, int out_dtype, float* lse, hipStream_t s) {
  if (dm.dtype == SA_BF16) {
    const hipError_t e = launch_prepare_values(dm, V, ws, s);
    if (e != hipSuccess) return e;
    return launch_forward_prepared(dm, Q, K, ws, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s);
  }
  if (dm.tpb == 2)  // 64-row tiles inside 128-key blocks
    return dm.d == 64
               ? launch_f32<64, 64, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
               : launch_f32<128, 64, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse,
                                          s);
  if (dm.m == 2)  // 128-row tiles over 64-key blocks
    return dm.d == 64
               ? launch_f32<64, 128, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
               : launch_f32<128, 128, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse,
                                          s);
  if (dm.d == 64)
    return dm.blk == 64
               ? launch_f32<64, 64, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
               : launch_f32<64, 128, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse,
                                          s);
  return dm.blk == 64
             ? launch_f32<128, 64, 64>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse, s)
             : launch_f32<128, 128, 128>(dm, Q, K, V, kv_idx, kv_cnt, W, scale, O, out_dtype, lse,
                                         s);
}

hipError_t launch_forward_vs(const Dims& dm, const void* Q, const void* K, const void* V,
                             const VsIndex& vs, float scale, void* ws, void* O, int out_dtype,
                             float* lse, hipStream_t s) {
  const hipError_t e = launch_prepare_values(dm, V, ws, s);
  if (e != hipSuccess) return e;
  return launch_bf16_shape<true>(dm, Q, K, nullptr, nullptr, 1, vs, scale, ws, O, out_dtype, lse,
                                 s);
}

}  // namespace sa
