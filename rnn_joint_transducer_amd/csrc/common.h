// Shared device-side definitions for the fused RNN-T joint + transducer loss
// kernels (gfx950 / CDNA4, wave64).
//
// Lattice notation follows the "Flash RNN-T" page (Abstract: joint network and
// transducer loss over the full alignment space and vocabulary) and the RNN
// transducer definition on the "Daily Papers" page (abstract on sequence
// transduction with recurrent networks): a cell is (b, t, u) with t < T'_b and
// u <= U'_b; pred row u is the prediction state after u labels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnntj {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Cell tile of the joint kernels: 16 frames x 8 label positions = 128 cells,
// processed by 4 waves that own 4 frames x 8 label positions (32 rows) each.
// Training criterion of a forward (word 3 of the state header): the full sum
// over alignments, or its maximum approximation (the best alignment).
constexpr int kCritSum = 0, kCritMax = 1;
// Token-and-duration transducer: the token head's transition posteriors are
// precomputed per cell (summed over durations) and handed over in place of
// alpha (blank) and beta (label).
constexpr int kCritTdt = 2;

constexpr int kTileT = 16;
constexpr int kTileU = 8;
constexpr int kTileCells = kTileT * kTileU;
constexpr int kVocabTile = 128;  // vocabulary columns per pass of one wave
// Largest vocabulary: keeps the 32-bit element offsets inside one 16 x 8
// cell tile of logit rows (at most (15 x 1024 + 7) x V + V, below 2^32) and
// a label + 1 inside 30 bits.
constexpr int kMaxV = 262144;
constexpr int kMaxProj = 65536;  // largest input / output width of a joint input projection

// Shapes shared by every kernel.
struct Dims {
  int B, T, U, H, V, blank;
  int U1;     // U + 1 (prediction rows)
  int DG;     // T + U: anti-diagonals t+u of the padded lattice
  int Tpad;   // T rounded up to kTileT
  int U1pad;  // U1 rounded up to kTileU
};

// Per-cell scalars (lse, LB, LE, alpha, beta) are stored diagonal-skewed:
// diagonal d = t + u is contiguous in u, so the lattice recursion reads and
// writes whole anti-diagonals with unit stride.
__device__ __forceinline__ size_t skew_idx(const Dims& d, int b, int t, int u) {
  return ((size_t)b * d.DG + (size_t)(t + u)) * d.U1 + u;
}

// ---------------------------------------------------------------- bf16 / f32

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// round-to-nearest-even float -> bf16 (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> bf16 bits with the hardware round-to-nearest-even conversion
// (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two floats to two bf16 (round to nearest even) in one 32-bit word, lo in
// the low half: one packed conversion instead of two conversions and a merge.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f32(float x) { return x; }
  static __device__ __forceinline__ float from_f32(float x) { return x; }
};
template <> struct ElemTraits<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16_hw(x); }
};

// Eight consecutive elements along the contraction axis: one MFMA operand
// fragment of one lane for a 16-wide k-step (bf16: 16 bytes; fp32: 32 bytes).
template <typename T> struct Frag8;
template <> struct Frag8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = v[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Frag8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ float get(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
};

__device__ __forceinline__ Frag8<uint16_t> load_frag(const uint16_t* p) {
  Frag8<uint16_t> f;
  f.v = *reinterpret_cast<const u32x4*>(p);
  return f;
}
__device__ __forceinline__ Frag8<float> load_frag(const float* p) {
  Frag8<float> f;
  f.lo = *reinterpret_cast<const f32x4*>(p);
  f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f;
}
__device__ __forceinline__ void store_frag(uint16_t* p, const Frag8<uint16_t>& f) {
  *reinterpret_cast<u32x4*>(p) = f.v;
}
__device__ __forceinline__ void store_frag(float* p, const Frag8<float>& f) {
  *reinterpret_cast<f32x4*>(p) = f.lo;
  *reinterpret_cast<f32x4*>(p + 4) = f.hi;
}
__device__ __forceinline__ void zero_frag(Frag8<uint16_t>& f) { f.v = u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void zero_frag(Frag8<float>& f) {
  f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
  f.hi = f.lo;
}
// Build a fragment from 8 floats (bf16: round to nearest even).
__device__ __forceinline__ void pack_frag(Frag8<uint16_t>& f, const float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.v[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
}
__device__ __forceinline__ void pack_frag(Frag8<float>& f, const float* x) {
  f.lo = f32x4{x[0], x[1], x[2], x[3]};
  f.hi = f32x4{x[4], x[5], x[6], x[7]};
}

// One 16-wide k-step of a 32x32 output block: C += A(32x16) * B(16x32).
// Lane l supplies A row (l % 32) and B column (l % 32), elements
// k = 8*(l/32) .. 8*(l/32)+7 of the step.  bf16 uses one 32x32x16 MFMA; fp32
// uses eight 32x32x2 MFMAs, the s-th pairing element s of both lane halves
// (the same k permutation on both operands leaves the sum unchanged).
__device__ __forceinline__ void mma_step(f32x16& acc, const Frag8<uint16_t>& a,
                                         const Frag8<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_step(f32x16& acc, const Frag8<float>& a,
                                         const Frag8<float>& b) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
}

// Fragment of 8 consecutive rows (the contraction axis) of one column of a
// row-major LDS tile with leading dimension ld (elements): lane l receives
// tile[row0 + 8*(l/32) + e][col0 + l%32], e = 0..7 -- the operand layout that
// mma_step expects, read from a tile stored [k][n].
// bf16 uses two ds_read_tr16_b64: within each 16-lane group, lane i receives
// element i%4 of the 8-byte words addressed by lanes 4j + i/4 (j = 0..3), so a
// lane that points at tile[kb + i/4][cb + 4*(i%4)] hands every lane i of the
// group four consecutive rows kb..kb+3 of column cb + i.  A lane's result
// depends on addresses held by other lanes, so the call must be made with
// every lane of the wave active.  fp32 uses eight scalar reads.
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// the four 16-bit values of a transposing read, as the two 32-bit words they
// occupy (element 2i in the low half of word i)
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
__device__ __forceinline__ Frag8<uint16_t> load_frag_T(const uint16_t* tile, int ld, int row0,
                                                       int col0) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, i = l & 15;
  const int kb = row0 + 8 * (g >> 1);
  const int cb = col0 + 16 * (g & 1);
  const uint16_t* p0 = tile + (kb + (i >> 2)) * ld + cb + 4 * (i & 3);
  const uint16_t* p1 = p0 + 4 * ld;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  Frag8<uint16_t> f;
  const u32x2_t a2 = __builtin_bit_cast(u32x2_t, a), b2 = __builtin_bit_cast(u32x2_t, b);
  f.v = u32x4{a2[0], a2[1], b2[0], b2[1]};
  return f;
}
__device__ __forceinline__ Frag8<float> load_frag_T(const float* tile, int ld, int row0,
                                                    int col0) {
  const int l = threadIdx.x & 63;
  const float* p = tile + (row0 + 8 * (l >> 5)) * ld + col0 + (l & 31);
  Frag8<float> f;
  f.lo = f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
  f.hi = f32x4{p[4 * ld], p[5 * ld], p[6 * ld], p[7 * ld]};
  return f;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds_base + 16 l.  lds_base must be the
// same in every lane of the wave.  Issued as inline assembly, so the
// compiler does not track it: the caller waits for it with wait_vm<N>()
// (vmcnt counts these copies like any other vector memory access) and makes
// it visible to the other waves with a barrier.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc),
               "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// As dma16, addressed as a wave-uniform base plus a per-lane 32-bit byte
// offset (the scalar-base form of the global load): a copy pattern repeated
// from many bases keeps its per-lane part in one register.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint64_t p = reinterpret_cast<uint64_t>(sbase);
  const uint64_t up = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(up), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// wait until at most N vector memory accesses of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Orders the current scheduling region as NM repetitions of (one MFMA, up to
// NDS LDS reads, up to NV other vector ALU instructions), so that with one
// wave per SIMD the operand reads and arithmetic of the next k-step issue in
// the shadow of this k-step's MFMAs instead of after them.
template <int NM, int NDS, int NV>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (NDS > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
    if (NV > 0) __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
}
// wait until this wave's LDS reads (and scalar loads) have completed
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Load of a value the kernel never writes, through the constant address
// space: with a wave-uniform address it becomes a scalar load, which neither
// waits for nor is waited on by the vector-memory counter.
template <typename P>
__device__ __forceinline__ P ld_const(const P* p) {
  return *(const __attribute__((address_space(4))) P*)p;
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Row of accumulator register r of a 32x32 block for lane-half kh = l/32
// (column is l % 32): rows 8*(r/4) + 4*kh + (r%4).
__device__ __forceinline__ int acc_row(int r, int kh) { return 8 * (r >> 2) + 4 * kh + (r & 3); }

// tanh(x) = 1 - 2 / (1 + e^{2x}); saturates correctly at +-inf, absolute
// error a few 1e-8.  NaN propagates (the clamp is a compare, not fminf).
__device__ __forceinline__ float fast_tanh(float x) {
  float y = x * (2.0f * kLog2e);
  y = y > 126.0f ? 126.0f : y;
  float e = __builtin_amdgcn_exp2f(y);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Transition posteriors of cell (t,u) from the float64 forward / backward
// variables (all diagonal-skewed):
//   gB(t,u) = exp(alpha(t,u) + LB(t,u) + beta(t+1,u) - logP)  (t < T'-1)
//   gB(T'-1,U') = exp(alpha + LB - logP),  gB(T'-1,u<U') = 0
//   gE(t,u) = exp(alpha(t,u) + LE(t,u) + beta(t,u+1) - logP)  (u < U'), else 0
// Maximum approximation: the lattice pass leaves in `beta` the marks of the
// best alignment's steps (kPathBlank / kPathLabel on the cell a step leaves;
// other cells hold their predecessor decision, a positive value).
constexpr double kPathBlank = -1.0, kPathLabel = -2.0;

// The per-cell inputs of the posteriors, loaded in one go so that a caller
// can issue the loads well before it needs the result.
struct CellPostIn {
  double a, bt, bu, m;  // alpha(t,u), beta(t+1,u), beta(t,u+1); max: the mark
  float lb, le;
};
__device__ __forceinline__ CellPostIn cell_post_load(const Dims& d,
                                                    const double* __restrict__ alpha,
                                                    const double* __restrict__ beta,
                                                    const float* __restrict__ LB,
                                                    const float* __restrict__ LE, int b, int t,
                                                    int u, int Tl, int Ul, int crit) {
  const size_t ix = skew_idx(d, b, t, u);
  CellPostIn c{0.0, 0.0, 0.0, 0.0, 0.f, 0.f};
  if (crit == kCritMax) {
    c.m = beta[ix];
    return c;
  }
  if (crit == kCritTdt) {
    c.a = alpha[ix];
    c.m = beta[ix];
    return c;
  }
  c.a = alpha[ix];
  c.lb = LB[ix];
  c.le = LE[ix];
  if (t < Tl - 1) c.bt = beta[skew_idx(d, b, t + 1, u)];
  if (u < Ul) c.bu = beta[skew_idx(d, b, t, u + 1)];
  return c;
}
__device__ __forceinline__ void cell_post_eval(const CellPostIn& c, double logP, int t, int u,
                                               int Tl, int Ul, double& gB, double& gE,
                                               int crit) {
  if (crit == kCritMax) {  // 0/1 indicators of the best alignment's steps
    gB = c.m == kPathBlank ? 1.0 : 0.0;
    gE = c.m == kPathLabel ? 1.0 : 0.0;
    return;
  }
  if (crit == kCritTdt) {  // precomputed, summed over the durations
    gB = c.a;
    gE = c.m;
    return;
  }
  if (t < Tl - 1)
    gB = exp(c.a + (double)c.lb + c.bt - logP);
  else
    gB = (u == Ul) ? exp(c.a + (double)c.lb - logP) : 0.0;
  gE = (u < Ul) ? exp(c.a + (double)c.le + c.bu - logP) : 0.0;
}
__device__ __forceinline__ void cell_posteriors(const Dims& d, const double* __restrict__ alpha,
                                                const double* __restrict__ beta,
                                                const float* __restrict__ LB,
                                                const float* __restrict__ LE, double logP,
                                                int b, int t, int u, int Tl, int Ul,
                                                double& gB, double& gE, int crit) {
  cell_post_eval(cell_post_load(d, alpha, beta, LB, LE, b, t, u, Tl, Ul, crit), logP, t, u, Tl,
                 Ul, gB, gE, crit);
}

}  // namespace rnntj
