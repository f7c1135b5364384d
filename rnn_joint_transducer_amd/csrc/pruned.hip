// Pruning bounds of the pruned transducer loss ("Pruned RNN-T for fast,
// memory-efficient ASR training", Abstract): a simple joiner, linear in the
// two embeddings, is evaluated over the whole lattice without a [T, U+1, V]
// tensor; its lattice gives each frame a window of S label positions, and the
// full joiner is then evaluated only inside those windows (the joint, lattice
// and backward kernels of the fused path, restricted to the band).
//
// The simple joiner is the fused path's joiner without its tanh and with the
// same weights: zs(t,u) = (enc[t] + pred[u]) W_out + b_out = am[t] + lm[u],
// am = enc W_out, lm = pred W_out + b_out.  Its normaliser factorises:
//   lse_s(t,u) = ma[t] + ml[u] + log sum_v EA[t,v] EL[u,v],
//   EA = exp(am - ma), EL = exp(lm - ml), ma / ml the row maxima,
// an (T x V) by (V x U+1) product per utterance.  Everything on this side is
// float64: the window of a frame is an integer decided by rounding the
// frame's occupancy centre, and float64 keeps that decision where a float64
// reference takes it (a centre would have to fall within ~1e-10 of a
// rounding boundary for the two to differ).
//
// Kernels (in launch order):
//   f64_gemm_kernel<kProj>   am, lm: [rows, H] x [H, V] products (+ bias)
//   simple_rows_kernel       row maxima, blank / label gathers, EA / EL in place
//   f64_gemm_kernel<kScore>  per utterance EA EL^T -> LBs, LEs (diagonal-skewed)
//   simple_lattice_kernel    alpha_s, beta_s (float64 log-add-exp), simple cost
//   centres_kernel           c_t = sum_u u occ(t,u) / sum_u occ(t,u)
//   bounds_kernel            window starts s_t (rounded centres made to hold an
//                            alignment), infeasible utterances flagged
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr double kNegInfD = -__builtin_inf();

// float64 log(e^a + e^b); -inf if both are -inf, NaN if either is NaN
__device__ __forceinline__ double lae(double a, double b) {
  const double m = a > b ? a : b;
  if (m == kNegInfD) return kNegInfD;
  return m + log1p(exp(-fabs(a - b)));
}

template <typename T>
__device__ __forceinline__ double to_f64(T x) {
  if constexpr (std::is_same<T, float>::value) return (double)x;
  else if constexpr (std::is_same<T, double>::value) return x;
  else return (double)bf16_to_f32(x);
}

// ------------------------------------------------------------ float64 GEMM
//
// One 64 x 64 output tile per workgroup of 4 waves; wave w computes rows
// 32 (w / 2) .. +31 and columns 32 (w % 2) .. +31 as 2 x 2 blocks of
// v_mfma_f64_16x16x4_f64.  k-steps of 16 are staged in LDS as float64
// (operands converted as they are written); the next step's global loads
// are in flight while the current step's MFMAs run.  A is row-major [M, K];
// B is row-major [K, N] (kProj) or [N, K] (kScore, the product with B
// transposed).  MFMA operand layout (lane l): A[l % 16][l / 16] of a 16 x 4
// block, B[l / 16][l % 16] of a 4 x 16 block; output value i of lane l is
// D[4 i + l / 16][l % 16].
constexpr int kProj = 0, kScore = 1;

struct F64GemmArgs {
  // kProj: C[M, N] = A[M, K] B[K, N] + bias[N]
  const void* A;
  const void* B;
  const void* bias;  // dtype [N] or null
  double* C;
  int M, N, K;
  // kScore (per utterance blockIdx.z): A = EA [B, T, V], B = EL [B, U+1, V]
  Dims d;
  const int32_t* Teff;
  const int32_t* Ueff;
  const double* ma;   // [B, T]
  const double* ml;   // [B, U+1]
  const double* amB;  // [B, T]      am[t, blank]
  const double* amY;  // [B, T, U]   am[t, labels[u]]
  const double* lmB;  // [B, U+1]    lm[u, blank]
  const double* lmY;  // [B, U+1]    lm[u, labels[u]]
  double* LBs;        // diagonal-skewed [B, T+U, U+1]
  double* LEs;
};

typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename TA, typename TB, int MODE>
__global__ __launch_bounds__(256) void f64_gemm_kernel(F64GemmArgs g) {
  __shared__ __align__(16) double As[2][16][64];
  __shared__ __align__(16) double Bs[2][16][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = 32 * (w >> 1), c0 = 32 * (w & 1);
  const int lm = lane & 15, lk4 = lane >> 4;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  int M = g.M, N = g.N, K = g.K;
  const TA* A = static_cast<const TA*>(g.A);
  const TB* B = static_cast<const TB*>(g.B);
  int b = 0, Tl = 0, Ul = 0;
  if constexpr (MODE == kScore) {
    b = blockIdx.z;
    Tl = g.Teff[b];
    Ul = g.Ueff[b];
    if (m0 >= Tl || n0 > Ul) return;  // uniform
    M = Tl;
    N = Ul + 1;
    K = g.d.V;
    A += (size_t)b * g.d.T * K;
    B += (size_t)b * g.d.U1 * K;
  }
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  // loader roles: A (and B of kScore) 4 consecutive k of row tid / 4;
  // B of kProj 4 consecutive n of k-row tid / 16.  Raw values are held
  // across the MFMAs and converted as they are written to LDS.
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const int bk = tid >> 4, bn = (tid & 15) * 4;
  TA xa[4];
  TB xb[4];
  // (sources clamped into the operands, the values outside them zeroed:
  // no branches around the loads; K and N are multiples of 4)
  auto load = [&](int k0) {
    {
      const bool ok = m0 + lr < M && k0 + lk < K;
      const TA* p = A + (size_t)min(m0 + lr, M - 1) * K + min(k0 + lk, K - 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const TA v = p[i];
        xa[i] = ok ? v : TA(0);
      }
    }
    if constexpr (MODE == kProj) {
      const bool ok = k0 + bk < K && n0 + bn < N;
      const TB* p = B + (size_t)min(k0 + bk, K - 1) * N + min(n0 + bn, N - 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const TB v = p[i];
        xb[i] = ok ? v : TB(0);
      }
    } else {
      const bool ok = n0 + lr < N && k0 + lk < K;
      const TB* p = B + (size_t)min(n0 + lr, N - 1) * K + min(k0 + lk, K - 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const TB v = p[i];
        xb[i] = ok ? v : TB(0);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) As[buf][lk + i][lr] = to_f64(xa[i]);
    if constexpr (MODE == kProj) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Bs[buf][bk][bn + i] = to_f64(xb[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) Bs[buf][lk + i][lr] = to_f64(xb[i]);
    }
  };
  // two LDS stages: step s computes from buffer s % 2 while step s + 1's
  // operands load and are then written to the other buffer, whose last
  // reader (step s - 1) finished before the previous barrier
  load(0);
  store(0);
  __syncthreads();
  int k0 = 0, buf = 0;
  do {  // K >= 4: at least one step
    // (the last step reloads its own operands into the idle buffer)
    load(k0 + 16 < K ? k0 + 16 : k0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = As[buf][4 * kk + lk4][r0 + 16 * i + lm];
        bb[i] = Bs[buf][4 * kk + lk4][c0 + 16 * i + lm];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    store(buf ^ 1);
    __syncthreads();
    k0 += 16;
    buf ^= 1;
  } while (k0 < K);

  if constexpr (MODE == kProj) {
    const TB* bias = static_cast<const TB*>(g.bias);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + c0 + 16 * j + lm;
      if (n >= N) continue;
      const double bn_ = bias ? to_f64(bias[n]) : 0.0;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + r0 + 16 * i + 4 * q + lk4;
          if (m < M) g.C[(size_t)m * N + n] = acc[i][j][q] + bn_;
        }
    }
  } else {
    const Dims d = g.d;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int u = n0 + c0 + 16 * j + lm;
      if (u > Ul) continue;
      const size_t ru = (size_t)b * d.U1 + u;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = m0 + r0 + 16 * i + 4 * q + lk4;
          if (t >= Tl) continue;
          const size_t rt = (size_t)b * d.T + t;
          const double lse = g.ma[rt] + g.ml[ru] + log(acc[i][j][q]);
          const size_t ix = skew_idx(d, b, t, u);
          g.LBs[ix] = g.amB[rt] + g.lmB[ru] - lse;
          g.LEs[ix] = u < Ul ? g.amY[rt * d.U + u] + g.lmY[ru] - lse : 0.0;
        }
    }
  }
}

// ------------------------------------------------------------ row pass
//
// Row r < B*T is am row (b, t), else lm row (b, u): the row maximum, the blank
// (and label) entries, then the row replaced by exp(row - max).  Rows outside
// the lattice are skipped.
__global__ __launch_bounds__(256) void simple_rows_kernel(double* am, double* lm,
                                                          const int32_t* __restrict__ labels,
                                                          const int32_t* __restrict__ Teff,
                                                          const int32_t* __restrict__ Ueff,
                                                          Dims d, double* ma, double* ml,
                                                          double* amB, double* amY, double* lmB,
                                                          double* lmY) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const long long r = blockIdx.x;
  const long long nA = (long long)d.B * d.T;
  const bool isA = r < nA;
  int b, i;
  if (isA) {
    b = (int)(r / d.T);
    i = (int)(r % d.T);
  } else {
    b = (int)((r - nA) / d.U1);
    i = (int)((r - nA) % d.U1);
  }
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0 || (isA ? i >= Tl : i > Ul)) return;  // uniform
  const size_t row = isA ? (size_t)r : (size_t)(r - nA);
  double* x = (isA ? am : lm) + row * d.V;
  double m = kNegInfD;
  for (int v = tid; v < d.V; v += 256) m = fmax(m, x[v]);
  red[tid] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
    __syncthreads();
  }
  m = red[0];
  const int32_t* y = labels + (size_t)b * d.U;
  if (isA) {
    if (tid == 0) {
      ma[row] = m;
      amB[row] = x[d.blank];
    }
    for (int u = tid; u < Ul; u += 256) amY[row * d.U + u] = x[y[u]];
  } else if (tid == 0) {
    ml[row] = m;
    lmB[row] = x[d.blank];
    lmY[row] = i < Ul ? x[y[i]] : 0.0;
  }
  __syncthreads();  // the gathers have read the row
  for (int v = tid; v < d.V; v += 256) x[v] = exp(x[v] - m);
}

// ------------------------------------------------------------ simple lattice
//
// alpha_s (blockIdx.y == 0) and beta_s (== 1) of one utterance in float64
// with the exact log-add-exp, one anti-diagonal per step, label position u on
// thread u (U+1 <= 512).  A step needs its own cell's value on the previous
// diagonal (kept in a register) and the neighbour's (u-1 for alpha, u+1 for
// beta) through LDS; the step weights of the next diagonal load during the
// current one.
__global__ __launch_bounds__(512) void simple_lattice_kernel(const double* __restrict__ LBs,
                                                             const double* __restrict__ LEs,
                                                             const int32_t* __restrict__ Teff,
                                                             const int32_t* __restrict__ Ueff,
                                                             Dims d, double* alpha, double* beta,
                                                             double* logPs, float* simple_costs) {
  __shared__ double nb[2][513];
  const int b = blockIdx.x, u = threadIdx.x;
  const bool fwd = blockIdx.y == 0;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0) {
    if (fwd && u == 0 && simple_costs) simple_costs[b] = __builtin_nanf("");
    return;
  }
  nb[0][u] = kNegInfD;
  nb[1][u] = kNegInfD;
  if (u == 0) {
    nb[0][512] = kNegInfD;
    nb[1][512] = kNegInfD;
  }
  __syncthreads();
  const int nd = Tl + Ul;
  const bool lane_on = u <= Ul;
  auto cell = [&](int dg, int& t) {  // is (dg - u, u) a lattice cell?
    t = dg - u;
    return lane_on && t >= 0 && t < Tl;
  };
  if (fwd) {
    // x: alpha(t-1,u) + LB(t-1,u) carried from the previous step
    double x = kNegInfD;
    double lb = 0.0, le = 0.0;
    int t;
    if (cell(0, t)) {
      const size_t ix = skew_idx(d, b, t, u);
      lb = LBs[ix];
      le = LEs[ix];
    }
    for (int dg = 0; dg < nd; ++dg) {
      int tn;
      double lbn = 0.0, len = 0.0;
      if (cell(dg + 1, tn)) {  // prefetch the next diagonal's weights
        const size_t ix = skew_idx(d, b, tn, u);
        lbn = LBs[ix];
        len = LEs[ix];
      }
      const bool on = cell(dg, t);
      // label step into (t,u) from (t,u-1): written by thread u-1 last step
      const double y = u > 0 ? nb[(dg & 1) ^ 1][u - 1] : kNegInfD;
      double a = kNegInfD;
      if (on) a = (dg == 0) ? 0.0 : lae(x, y);
      if (on) alpha[skew_idx(d, b, t, u)] = a;
      x = on ? a + lb : kNegInfD;
      nb[dg & 1][u] = (on && u < Ul) ? a + le : kNegInfD;
      if (on && t == Tl - 1 && u == Ul) {
        const double lp = a + lb;
        logPs[b] = lp;
        if (simple_costs) simple_costs[b] = (float)(-lp);
      }
      lb = lbn;
      le = len;
      __syncthreads();
    }
  } else {
    // x: beta(t+1,u) carried from the previous (later) diagonal
    double x = kNegInfD;
    int t;
    double lb = 0.0, le = 0.0;
    if (cell(nd - 1, t)) {
      const size_t ix = skew_idx(d, b, t, u);
      lb = LBs[ix];
      le = LEs[ix];
    }
    for (int dg = nd - 1; dg >= 0; --dg) {
      int tn;
      double lbn = 0.0, len = 0.0;
      if (dg > 0 && cell(dg - 1, tn)) {
        const size_t ix = skew_idx(d, b, tn, u);
        lbn = LBs[ix];
        len = LEs[ix];
      }
      const bool on = cell(dg, t);
      // label step (t,u) -> (t,u+1): beta(t,u+1) written by thread u+1 last step
      const double y = nb[(dg & 1) ^ 1][u + 1];
      double bt = kNegInfD;
      if (on) {
        if (t == Tl - 1 && u == Ul) bt = lb;
        else bt = lae(x + lb, u < Ul ? y + le : kNegInfD);
        beta[skew_idx(d, b, t, u)] = bt;
      }
      x = on ? bt : kNegInfD;
      nb[dg & 1][u] = on ? bt : kNegInfD;
      lb = lbn;
      le = len;
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ bounds
//
// Occupancy centre of every frame: c_t = sum_u u occ(t,u) / sum_u occ(t,u),
// occ = exp(alpha_s + beta_s - logPs).  One thread per frame.
__global__ __launch_bounds__(64) void centres_kernel(const double* __restrict__ alpha,
                                                     const double* __restrict__ beta,
                                                     const double* __restrict__ logPs,
                                                     const int32_t* __restrict__ Teff,
                                                     const int32_t* __restrict__ Ueff, Dims d,
                                                     double* centres) {
  const int b = blockIdx.y, t = blockIdx.x * 64 + threadIdx.x;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (t >= Tl) return;
  const double lp = logPs[b];
  double num = 0.0, den = 0.0;
  for (int u = 0; u <= Ul; ++u) {
    const size_t ix = skew_idx(d, b, t, u);
    const double o = exp(alpha[ix] + beta[ix] - lp);
    num = fma((double)u, o, num);
    den += o;
  }
  centres[(size_t)b * d.T + t] = num / den;
}

// Window starts of one utterance: s0_t = clamp(floor(c_t - (S-1)/2 + 1/2),
// 0, smax) in parallel; then, on one thread, the forward pass (start at 0,
// non-decreasing, at most S-1 apart) and the backward pass (end at smax, at
// most S-1 apart looking back).  If the first window then starts above 0 no
// alignment fits: the utterance is marked invalid (lengths zeroed) and
// kErrPruneInfeasible set.  Bounds past T' repeat the last window.  s is
// kept in LDS as 16-bit integers (s <= U <= 511), 2 T bytes.
__global__ __launch_bounds__(256) void bounds_kernel(const double* __restrict__ centres,
                                                     int32_t* Teff, int32_t* Ueff, Dims d, int S,
                                                     int32_t* bounds, int32_t* status) {
  extern __shared__ short sw[];
  __shared__ int s_last;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0) return;
  const int smax = Ul + 1 - S > 0 ? Ul + 1 - S : 0;
  const double half = 0.5 * (double)(S - 1);
  for (int t = tid; t < Tl; t += 256) {
    double x = floor(centres[(size_t)b * d.T + t] - half + 0.5);
    x = x >= 0.0 ? x : 0.0;  // NaN -> 0
    x = x <= (double)smax ? x : (double)smax;
    sw[t] = (short)x;
  }
  __syncthreads();
  if (tid == 0) {
    int prev = 0;
    sw[0] = 0;
    for (int t = 1; t < Tl; ++t) {
      int s = sw[t];
      s = s > prev ? s : prev;
      s = s < prev + S - 1 ? s : prev + S - 1;
      sw[t] = (short)s;
      prev = s;
    }
    int next = smax;
    sw[Tl - 1] = (short)smax;
    for (int t = Tl - 2; t >= 0; --t) {
      int s = sw[t];
      s = s > next - (S - 1) ? s : next - (S - 1);
      sw[t] = (short)s;
      next = s;
    }
    s_last = sw[Tl - 1];
    if (sw[0] != 0) {  // no band of these windows holds an alignment
      Teff[b] = 0;
      Ueff[b] = 0;
      atomicOr(status, kErrPruneInfeasible);
    }
  }
  __syncthreads();
  for (int t = tid; t < d.T; t += 256)
    bounds[(size_t)b * d.T + t] = t < Tl ? (int32_t)sw[t] : s_last;
}

__global__ void fill_kernel(float* p, size_t n, float v) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

}  // namespace

hipError_t launch_pruning_bounds(const PruneArgs& p, hipStream_t st) {
  const Dims d = p.d;
  F64GemmArgs g = {};
  // am = enc W_out, lm = pred W_out + b_out  (float64)
  g.B = p.W;
  g.N = d.V;
  g.K = d.H;
  auto proj = [&](const void* X, int rows, const void* bias, double* C) {
    g.A = X;
    g.M = rows;
    g.bias = bias;
    g.C = C;
    dim3 grid((rows + 63) / 64, (d.V + 63) / 64);
    if (p.bf16)
      hipLaunchKernelGGL((f64_gemm_kernel<uint16_t, uint16_t, kProj>), grid, dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((f64_gemm_kernel<float, float, kProj>), grid, dim3(256), 0, st, g);
  };
  proj(p.enc, d.B * d.T, nullptr, p.am);
  proj(p.pred, d.B * d.U1, p.bias, p.lm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned rows = (unsigned)(d.B * d.T + d.B * d.U1);
  hipLaunchKernelGGL(simple_rows_kernel, dim3(rows), dim3(256), 0, st, p.am, p.lm, p.labels,
                     p.Teff, p.Ueff, d, p.ma, p.ml, p.amB, p.amY, p.lmB, p.lmY);
  F64GemmArgs s = {};
  s.A = p.am;
  s.B = p.lm;
  s.d = d;
  s.Teff = p.Teff;
  s.Ueff = p.Ueff;
  s.ma = p.ma;
  s.ml = p.ml;
  s.amB = p.amB;
  s.amY = p.amY;
  s.lmB = p.lmB;
  s.lmY = p.lmY;
  s.LBs = p.LBs;
  s.LEs = p.LEs;
  hipLaunchKernelGGL((f64_gemm_kernel<double, double, kScore>),
                     dim3((d.T + 63) / 64, (d.U1 + 63) / 64, d.B), dim3(256), 0, st, s);
  hipLaunchKernelGGL(simple_lattice_kernel, dim3(d.B, 2), dim3(512), 0, st, p.LBs, p.LEs, p.Teff,
                     p.Ueff, d, p.alpha, p.beta, p.logPs, p.simple_costs);
  hipLaunchKernelGGL(centres_kernel, dim3((d.T + 63) / 64, d.B), dim3(64), 0, st, p.alpha,
                     p.beta, p.logPs, p.Teff, p.Ueff, d, p.centres);
  hipLaunchKernelGGL(bounds_kernel, dim3(d.B), dim3(256), (size_t)2 * d.T, st, p.centres, p.Teff,
                     p.Ueff, d, p.S, p.bounds, p.status);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  blocks = blocks < 4096 ? blocks : 4096;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace rnntj
