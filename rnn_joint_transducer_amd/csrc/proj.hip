// Joint input projections: the affine maps that take each encoding into the
// joint's hidden size ahead of the add.
//
// "Daily Papers" page, Transformer-Transducer abstract: the audio and label
// encodings are combined by a feed-forward layer into one label distribution
// per (frame, label history); read as one affine map per encoding,
//     enc_p = enc @ W_enc + b_enc,   pred_p = pred @ W_pred + b_pred,
// whose gradients chain from the joint's gradients of enc_p and pred_p:
//     dx = dy @ W^T,   dW = x^T @ dy,   db = sum over rows of dy.
//
// The products run on one kernel (plus a bf16 MFMA variant of y = x W + b
// when x and W are bf16): a 64 x 64 output tile per workgroup
// (four waves, each a 32 x 32 fp32 MFMA block), 32-deep k-steps staged in LDS
// as fp32 (bf16 operands are widened on the way in, so every product is
// exact and accumulates in fp32), the next k-step's global loads issued
// before the current one's MFMAs.  An operand is read either with its k
// index contiguous (x, dy, W in dx = dy W^T) or with its other index
// contiguous (W in y = x W, x^T in dW = x^T dy); either way a thread loads
// 8 consecutive elements.  dW splits its k range (the rows of x) over
// workgroups and adds the partial sums with fp32 atomics into a zeroed
// output; the workgroups of its first row tile also sum the dy rows they
// stage (db), so dy is read once for both.
#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr int kPT = 64;   // output tile edge
constexpr int kPK = 32;   // k-step
constexpr int kLdA = 36;  // LDS row strides (floats): 16-byte aligned rows,
constexpr int kLdB = 68;  // conflict-free fragment reads

template <typename X>
__device__ __forceinline__ void load8(const X* p, bool ok, float (&v)[8]) {
  if constexpr (sizeof(X) == 2) {
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (ok) w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
    if (ok) {
      a = *reinterpret_cast<const f32x4*>(p);
      b = *reinterpret_cast<const f32x4*>(p + 4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// C[i][j] = sum_k A(i,k) B(k,j) over k in [k0, k1) of this workgroup's
// split: A(i,k) = a[i*sai + k] (AK) or a[k*sak + i] (!AK); B(k,j) =
// b[k*sbk + j] (BJ) or b[j*sbj + k] (!BJ).  OUT: 0 store fp32, 1 atomic add
// fp32, 2 add bias[j] and store as the operand type TO.  With OUT == 1 and
// colsum set, workgroups with blockIdx.x == 0 also add the column sums of
// their B rows (k range) into colsum[j].
struct GemmArgs {
  const void* a;
  long long sa;  // row stride of a
  const void* b;
  long long sb;  // row stride of b
  const void* bias;
  void* c;
  long long ldc;
  int M, N, K, kchunk;
  float* colsum;
  int zbase;  // k split of blockIdx.z == 0 (launches of one split at a time)
};

template <typename TA, typename TB, bool AK, bool BJ, int OUT, typename TO>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  __shared__ __align__(16) float As[kPT * kLdA];  // [i][k]
  __shared__ __align__(16) float Bs[kPK * kLdB];  // [k][j]; also the column-sum reduction
  const TA* __restrict__ A = static_cast<const TA*>(g.a);
  const TB* __restrict__ Bm = static_cast<const TB*>(g.b);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = blockIdx.x * kPT, j0 = blockIdx.y * kPT;
  const int kb = (g.zbase + (int)blockIdx.z) * g.kchunk;
  const int ke = min(g.K, kb + g.kchunk);
  // this thread's 8-element piece of the A and B tiles
  const int ai = AK ? tid >> 2 : (tid & 7) * 8, ak = AK ? (tid & 3) * 8 : tid >> 3;
  const int bk = BJ ? tid >> 3 : (tid & 3) * 8, bj = BJ ? (tid & 7) * 8 : tid >> 2;
  float av[8], bv[8];
  auto fetch = [&](int k0) {
    const int gi = i0 + ai, gk = k0 + ak;
    if constexpr (AK)
      load8(A + (size_t)gi * g.sa + gk, gi < g.M && gk < ke, av);
    else
      load8(A + (size_t)gk * g.sa + gi, gi < g.M && gk < ke, av);
    const int hk = k0 + bk, hj = j0 + bj;
    if constexpr (BJ)
      load8(Bm + (size_t)hk * g.sb + hj, hk < ke && hj < g.N, bv);
    else
      load8(Bm + (size_t)hj * g.sb + hk, hk < ke && hj < g.N, bv);
  };
  auto stash = [&]() {
    if constexpr (AK) {
      *reinterpret_cast<f32x4*>(&As[ai * kLdA + ak]) = f32x4{av[0], av[1], av[2], av[3]};
      *reinterpret_cast<f32x4*>(&As[ai * kLdA + ak + 4]) = f32x4{av[4], av[5], av[6], av[7]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) As[(ai + e) * kLdA + ak] = av[e];
    }
    if constexpr (BJ) {
      *reinterpret_cast<f32x4*>(&Bs[bk * kLdB + bj]) = f32x4{bv[0], bv[1], bv[2], bv[3]};
      *reinterpret_cast<f32x4*>(&Bs[bk * kLdB + bj + 4]) = f32x4{bv[4], bv[5], bv[6], bv[7]};
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) Bs[(bk + e) * kLdB + bj] = bv[e];
    }
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  constexpr bool kColsum = OUT == 1 && BJ;
  const bool do_cs = kColsum && g.colsum != nullptr && blockIdx.x == 0;
  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int wi = (w >> 1) * 32, wj = (w & 1) * 32;
  if (kb < ke) fetch(kb);
  for (int k0 = kb; k0 < ke; k0 += kPK) {
    __syncthreads();  // the previous k-step's fragment reads are done
    stash();
    if (do_cs) {  // bv: 8 columns of one staged row (zero outside the k range)
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] += bv[e];
    }
    __syncthreads();
    if (k0 + kPK < ke) fetch(k0 + kPK);
#pragma unroll
    for (int ks = 0; ks < kPK; ks += 16) {
      const float* ap = &As[(wi + (lane & 31)) * kLdA + ks + 8 * (lane >> 5)];
      Frag8<float> fa, fb;
      fa.lo = *reinterpret_cast<const f32x4*>(ap);
      fa.hi = *reinterpret_cast<const f32x4*>(ap + 4);
      fb = load_frag_T(Bs, kLdB, ks, wj);
      mma_step(acc, fa, fb);
    }
  }
  if (do_cs) {  // uniform: reduce the 32 threads of each column group
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) Bs[bk * kLdB + bj + e] = cs[e];
    __syncthreads();
    if (tid < kPT && j0 + tid < g.N) {
      float s = 0.f;
      for (int r = 0; r < kPK; ++r) s += Bs[r * kLdB + tid];
      atomicAdd(&g.colsum[j0 + tid], s);
    }
  }
  const int kh = lane >> 5, col = j0 + wj + (lane & 31);
  if (col >= g.N) return;
  float bias = 0.f;
  if constexpr (OUT == 2)
    if (g.bias) bias = ElemTraits<TO>::to_f32(static_cast<const TO*>(g.bias)[col]);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = i0 + wi + acc_row(r, kh);
    if (row >= g.M) continue;
    const size_t o = (size_t)row * g.ldc + col;
    if constexpr (OUT == 0) {
      static_cast<float*>(g.c)[o] = acc[r];
    } else if constexpr (OUT == 1) {
      atomicAdd(static_cast<float*>(g.c) + o, acc[r]);
    } else {
      static_cast<TO*>(g.c)[o] = ElemTraits<TO>::from_f32(acc[r] + bias);
    }
  }
}

// y = x W + b with x, W (and y) bf16: the same 64 x 64 tiles and 32-deep
// k-steps, staged in LDS as bf16 and multiplied by v_mfma_f32_32x32x16_bf16
// (bf16 products are exact, the sums accumulate in fp32): 16 times the
// widened fp32 MFMA rate.  x's fragments are 16-byte row reads; W's, with
// the output column contiguous, come from transposing LDS reads.
constexpr int kLdA16 = kPK + 8;  // bf16 row strides: 16-byte aligned rows
constexpr int kLdB16 = kPT + 8;
__global__ __launch_bounds__(256) void proj_fwd_bf16_kernel(GemmArgs g) {
  __shared__ __align__(16) uint16_t As[kPT * kLdA16];  // [i][k]
  __shared__ __align__(16) uint16_t Bs[kPK * kLdB16];  // [k][j]
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.a);
  const uint16_t* __restrict__ Bm = static_cast<const uint16_t*>(g.b);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i0 = blockIdx.x * kPT, j0 = blockIdx.y * kPT;
  const int ai = tid >> 2, ak = (tid & 3) * 8;  // 8 consecutive k of row ai
  const int bk = tid >> 3, bj = (tid & 7) * 8;  // 8 consecutive j of k-row bk
  u32x4 av, bv;
  auto fetch = [&](int k0) {
    const int gi = i0 + ai, gk = k0 + ak, hk = k0 + bk, hj = j0 + bj;
    av = u32x4{0u, 0u, 0u, 0u};
    bv = av;
    if (gi < g.M && gk < g.K) av = *reinterpret_cast<const u32x4*>(A + (size_t)gi * g.sa + gk);
    if (hk < g.K && hj < g.N) bv = *reinterpret_cast<const u32x4*>(Bm + (size_t)hk * g.sb + hj);
  };
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int wi = (w >> 1) * 32, wj = (w & 1) * 32;
  fetch(0);
  for (int k0 = 0; k0 < g.K; k0 += kPK) {
    __syncthreads();  // the previous k-step's fragment reads are done
    *reinterpret_cast<u32x4*>(&As[ai * kLdA16 + ak]) = av;
    *reinterpret_cast<u32x4*>(&Bs[bk * kLdB16 + bj]) = bv;
    __syncthreads();
    if (k0 + kPK < g.K) fetch(k0 + kPK);
#pragma unroll
    for (int ks = 0; ks < kPK; ks += 16) {
      Frag8<uint16_t> fa;
      fa.v = *reinterpret_cast<const u32x4*>(&As[(wi + (lane & 31)) * kLdA16 + ks + 8 * (lane >> 5)]);
      const Frag8<uint16_t> fb = load_frag_T(Bs, kLdB16, ks, wj);
      mma_step(acc, fa, fb);
    }
  }
  const int kh = lane >> 5, col = j0 + wj + (lane & 31);
  if (col >= g.N) return;
  const float bias = g.bias ? bf16_to_f32(static_cast<const uint16_t*>(g.bias)[col]) : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = i0 + wi + acc_row(r, kh);
    if (row < g.M)
      static_cast<uint16_t*>(g.c)[(size_t)row * g.ldc + col] = f32_to_bf16_hw(acc[r] + bias);
  }
}

// (in_order: the k splits as consecutive launches, so that the atomic sums
// of each output element come in split order)
template <typename TA, typename TB, bool AK, bool BJ, int OUT, typename TO>
hipError_t gemm(const GemmArgs& g, int splits, hipStream_t st, bool in_order = false) {
  const dim3 grid((g.M + kPT - 1) / kPT, (g.N + kPT - 1) / kPT, in_order ? 1 : splits);
  if (!in_order) {
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AK, BJ, OUT, TO>), grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  GemmArgs gs = g;
  for (int z = 0; z < splits; ++z) {
    gs.zbase = z;
    hipLaunchKernelGGL((gemm_kernel<TA, TB, AK, BJ, OUT, TO>), grid, dim3(256), 0, st, gs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_fwd(const void* x, const void* W, const void* b, bool bf16, int M, int K,
                           int N, void* y, hipStream_t st) {
  GemmArgs g{x, K, W, N, b, y, N, M, N, K, K, nullptr};
  if (bf16) {
    const dim3 grid((M + kPT - 1) / kPT, (N + kPT - 1) / kPT, 1);
    hipLaunchKernelGGL(proj_fwd_bf16_kernel, grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  return gemm<float, float, true, true, 2, float>(g, 1, st);
}

hipError_t launch_proj_dx(const float* dy, const void* W, bool bf16, int M, int K, int N,
                          float* dx, hipStream_t st) {
  // dx[M,K] = dy[M,N] W[K,N]^T: k runs over N
  GemmArgs g{dy, N, W, N, nullptr, dx, K, M, K, N, N, nullptr};
  if (bf16) return gemm<float, uint16_t, true, false, 0, float>(g, 1, st);
  return gemm<float, float, true, false, 0, float>(g, 1, st);
}

hipError_t launch_proj_dw(const void* x, const float* dy, bool bf16, int M, int K, int N,
                          float* dW, float* db, int cus, bool in_order, hipStream_t st) {
  // dW[K,N] += x[M,K]^T dy[M,N] and db[N] += column sums of dy: k runs over
  // the M rows, split so that the grid holds about four workgroups per
  // compute unit (in_order: the splits run one launch after another, so the
  // atomic sums of each element come in a fixed order)
  const int tiles = ((K + kPT - 1) / kPT) * ((N + kPT - 1) / kPT);
  int splits = (4 * cus + tiles - 1) / tiles;
  const int max_splits = (M + kPK - 1) / kPK;
  splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
  int kchunk = (M + splits - 1) / splits;
  kchunk = (kchunk + kPK - 1) / kPK * kPK;
  splits = (M + kchunk - 1) / kchunk;
  GemmArgs g{x, K, dy, N, nullptr, dW, N, K, N, M, kchunk, db, 0};
  if (bf16) return gemm<uint16_t, float, false, true, 1, float>(g, splits, st, in_order);
  return gemm<float, float, false, true, 1, float>(g, splits, st, in_order);
}


}  // namespace rnntj
