// Token-and-duration transducer ("Daily Papers" page, Token-and-Duration
// Transducer abstract): the joint has two outputs, normalised independently,
// over tokens and over durations (the frames a token covers).
//
// The token head is the fused path's joint + vocabulary projection + online
// log-sum-exp, unchanged (LB, LE per cell).  This file holds what the
// durations add:
//   dur_head_kernel      LD(t,u,k) = log_softmax(h W_dur + b_dur)[k] per cell,
//                        h = tanh(enc[t] + pred[u]) rebuilt from the e^{2x} rows
//   tdt_lattice_kernel   alpha / beta over the lattice whose steps jump d_k
//                        frames (blank d_k >= 1: (t,u) -> (t+d,u); label:
//                        (t,u) -> (t+d,u+1)); float64, exact log-add-exp
//   tdt_post_kernel      per cell the summed blank / label step posteriors
//                        (the token head's backward reads them in place of
//                        alpha / beta) and the duration-logit gradient
//                        dzd(t,u,k) = gc ((gB + gE) q_k - (gB_k + gE_k))
//   dur_bwd_kernel       the duration head's share of d_enc and d_pred,
//                        (1 - h^2) (W_dur dzd) summed over label positions
//                        and over frames, from one pass over blocks of
//                        frames, plus d_W_dur = sum h dzd^T, d_b_dur = sum dzd.
// The lattice runs in float64 with one anti-diagonal per step: every
// predecessor of a cell lies on one of the dmax + 1 previous diagonals, which
// a ring of diagonals in LDS holds.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr double kNegInfD = -__builtin_inf();
constexpr int kRing = kTdtMaxDur + 2;  // diagonals kept: dmax + 1 back, plus the current

__device__ __forceinline__ double lae(double a, double b) {
  const double m = a > b ? a : b;
  if (m == kNegInfD) return kNegInfD;
  return m + log1p(exp(-fabs(a - b)));
}

// h of cell (t,u) for hidden unit k from the e^{2x} rows (or directly)
__device__ __forceinline__ float h_of(const TdtArgs& a, int b, int t, int u, int k, bool use_ep) {
  const Dims& d = a.d;
  if (use_ep) {
    const float e = a.Eexp[((size_t)b * d.T + t) * d.H + k];
    const float p = a.Pexp[((size_t)b * d.U1 + u) * d.H + k];
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e * p);
  }
  float x;
  if (a.bf16) {
    x = bf16_to_f32(static_cast<const uint16_t*>(a.enc)[((size_t)b * d.T + t) * d.H + k]) +
        bf16_to_f32(static_cast<const uint16_t*>(a.pred)[((size_t)b * d.U1 + u) * d.H + k]);
  } else {
    x = static_cast<const float*>(a.enc)[((size_t)b * d.T + t) * d.H + k] +
        static_cast<const float*>(a.pred)[((size_t)b * d.U1 + u) * d.H + k];
  }
  return fast_tanh(x);
}

// the h the MFMA path multiplies: rounded to the input type
__device__ __forceinline__ float h_round(const TdtArgs& a, float h) {
  return a.bf16 ? bf16_to_f32(f32_to_bf16_hw(h)) : h;
}

__device__ __forceinline__ float wdur(const TdtArgs& a, int k, int j) {
  const size_t i = (size_t)k * a.K + j;
  return a.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.Wd)[i])
                : static_cast<const float*>(a.Wd)[i];
}
__device__ __forceinline__ float bdur(const TdtArgs& a, int j) {
  return a.bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.bd)[j])
                : static_cast<const float*>(a.bd)[j];
}

// ------------------------------------------------------------ duration head
//
// One workgroup per (b, t); wave w takes the cells u = w, w + 4, ...; the 64
// lanes of a wave split the hidden units (lane l: l, l + 64, ...), so each
// e^{2 pred} row is read in coalesced 256-byte pieces, and the K partial
// sums of the lanes meet in a butterfly.  W_dur (float32, [K][H]) and the
// frame's e^{2 enc} row are in LDS.
// (KK = the number of durations, a.K)
template <int KK>
__global__ __launch_bounds__(256) void dur_head_kernel(TdtArgs a) {
  extern __shared__ float sm[];  // W_dur [K][H], then the e^{2 enc} row [H]
  const Dims d = a.d;
  const int b = blockIdx.y, t = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t >= Tl) return;  // uniform
  const int H = d.H;
  constexpr int K = KK;
  float* w = sm;
  float* er = sm + H * K;
  const bool use_ep = (a.hdr[1] & kFlagEpBad) == 0;
  for (int i = tid; i < H * K; i += 256) w[(i % K) * H + i / K] = wdur(a, i / K, i % K);
  for (int k = tid; k < H; k += 256) er[k] = a.Eexp[((size_t)b * d.T + t) * H + k];
  __syncthreads();
  for (int u = wv; u <= Ul; u += 4) {
    float z[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) z[j] = 0.f;
    const float* pr = a.Pexp + ((size_t)b * d.U1 + u) * H;
    for (int k = lane; k < H; k += 64) {
      const float h = h_round(a, use_ep ? 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + er[k] * pr[k])
                                        : h_of(a, b, t, u, k, false));
#pragma unroll
      for (int j = 0; j < KK; ++j)
        z[j] = fmaf(h, w[j * H + k], z[j]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int j = 0; j < KK; ++j)
        z[j] += __shfl_xor(z[j], off);
    if (lane == 0) {
      float m = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j < K) {
          z[j] += bdur(a, j);
          m = fmaxf(m, z[j]);
        }
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j < K) s += __expf(z[j] - m);
      const float lse = m + __logf(s);
      float* ld = a.LD + skew_idx(d, b, t, u) * K;
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j < K) ld[j] = z[j] - lse;
    }
  }
}

// ------------------------------------------------------------ lattice
//
// blockIdx.y == 0: alpha, == 1: beta; thread u owns label position u.
//
// A cell's value is the log of a sum over up to 2K incoming (alpha) or
// outgoing (beta) steps.  It is formed as the largest term, in float64, plus
// the natural log of the sum of exp(term - largest) taken in float32: every
// difference is <= 0 and the sum lies in [1, 2K], so the float32 part adds a
// few 1e-8 of absolute error per cell to a float64 state (no difference is
// rounded before it is taken).  A NaN term makes the cell NaN.
//
// The step weights a diagonal needs (float32 LB, LE, LD of the source cells)
// do not depend on the recursion: each lane loads the next diagonal's while
// the current one is computed.  The loads are a fixed set of K per kind
// (a source outside the lattice reads a valid cell and is masked), so the
// wait before their use never has to cover the loads issued after them.
// The kernel is instantiated for each duration count, so no work is spent on
// unused duration slots.
// (absent steps hold -inf)
template <int N>
__device__ __forceinline__ double lse_terms(const double (&x)[N]) {
  double m = kNegInfD;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    nan |= x[i] != x[i];
    m = x[i] > m ? x[i] : m;
  }
  if (nan) return __builtin_nan("");
  if (m == kNegInfD) return kNegInfD;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) sum += exp2_fast((float)(x[i] - m) * kLog2e);
  return m + (double)(__builtin_amdgcn_logf(sum) * kLn2);
}

// (KK = the number of durations, a.K)
template <int KK>
__global__ __launch_bounds__(512) void tdt_lattice_kernel(TdtArgs a) {
  __shared__ double ring[kRing][513];
  const Dims d = a.d;
  const int b = blockIdx.x, u = threadIdx.x;
  constexpr int K = KK;
  const bool fwd = blockIdx.y == 0;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (Tl == 0) {
    if (fwd && u == 0) {
      a.costs[b] = __builtin_nanf("");
      a.logP[b] = __builtin_nan("");
    }
    return;
  }
  for (int r = 0; r < kRing; ++r) {
    ring[r][u] = kNegInfD;
    if (u == 0) ring[r][512] = kNegInfD;
  }
  __syncthreads();
  const bool lane_on = u <= Ul;
  const int nd = Tl + Ul;  // diagonals 0 .. Tl-1+Ul
  int dur[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) dur[j] = a.dur[j];
  const size_t base = (size_t)b * d.DG * d.U1;
  // cell (t, uu) of this utterance, t + uu <= DG - 1 and uu <= U1 - 1
  auto idx = [&](int t, int uu) { return base + (size_t)(t + uu) * d.U1 + uu; };
  if (fwd) {
    // weights of the cell this lane computes on diagonal k: blank from
    // (t - d_j, u), label from (t - d_j, u - 1); invalid sources read (0, 0)
    float wlb[KK], wlbd[KK], wle[KK], wled[KK];
    auto load_w = [&](int k) {
      const int t = k - u;
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        const int s = t - dur[j];
        const bool okb = lane_on && t < Tl && s >= 0;
        const bool oke = okb && u >= 1;
        const size_t ib = okb ? idx(s, u) : base, ie = oke ? idx(s, u - 1) : base;
        wlb[j] = a.LB[ib];
        wlbd[j] = a.LD[ib * K + j];
        wle[j] = a.LE[ie];
        wled[j] = a.LD[ie * K + j];
      }
    };
    load_w(0);
    for (int k = 0; k < nd; ++k) {
      float clb[KK], clbd[KK], cle[KK], cled[KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        clb[j] = wlb[j];
        clbd[j] = wlbd[j];
        cle[j] = wle[j];
        cled[j] = wled[j];
      }
      if (k + 1 < nd) load_w(k + 1);
      const int t = k - u;
      const bool on = lane_on && t >= 0 && t < Tl;
      double v = kNegInfD;
      if (on) {
        if (k == 0) {
          v = 0.0;
        } else {
          double x[2 * KK];
#pragma unroll
          for (int j = 0; j < KK; ++j) {
            const int dj = dur[j], s = t - dj;
            const bool ok = j < K && s >= 0;
            // blank (s,u) -> (t,u), on diagonal k - dj
            x[2 * j] = ok && dj >= 1 ? ring[(k - dj) % kRing][u] + ((double)clb[j] + (double)clbd[j])
                                     : kNegInfD;
            // label (s,u-1) -> (t,u), on diagonal k - dj - 1
            x[2 * j + 1] = ok && u >= 1
                               ? ring[(k - dj - 1) % kRing][u - 1] + ((double)cle[j] + (double)cled[j])
                               : kNegInfD;
          }
          v = lse_terms(x);
        }
        a.alpha[idx(t, u)] = v;
      }
      ring[k % kRing][u] = on ? v : kNegInfD;
      __syncthreads();
    }
    if (u == Ul) {  // the final blank lands exactly on frame T'
      double x[2 * KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        const int dj = dur[j], s = Tl - dj;
        x[2 * j] = j < K && dj >= 1 && s >= 0
                       ? a.alpha[idx(s, Ul)] + ((double)a.LB[idx(s, Ul)] + (double)a.LD[idx(s, Ul) * K + j])
                       : kNegInfD;
        x[2 * j + 1] = kNegInfD;
      }
      const double lp = lse_terms(x);
      a.logP[b] = lp;
      a.costs[b] = (float)(-lp);
    }
  } else {
    // the weights of a cell's outgoing steps are its own LB, LE, LD
    float wlb = 0.f, wle = 0.f, wld[KK];
    auto load_w = [&](int k) {
      const int t = k - u;
      const bool ok = lane_on && t >= 0 && t < Tl;
      const size_t i = ok ? idx(t, u) : base;
      wlb = a.LB[i];
      wle = a.LE[i];
#pragma unroll
      for (int j = 0; j < KK; ++j) wld[j] = a.LD[i * K + j];
    };
    load_w(nd - 1);
    for (int k = nd - 1; k >= 0; --k) {
      const float clb = wlb, cle = wle;
      float cld[KK];
#pragma unroll
      for (int j = 0; j < KK; ++j) cld[j] = wld[j];
      if (k > 0) load_w(k - 1);
      const int t = k - u;
      const bool on = lane_on && t >= 0 && t < Tl;
      double v = kNegInfD;
      if (on) {
        const double lb = clb, le = u < Ul ? (double)cle : 0.0;
        double x[2 * KK];
#pragma unroll
        for (int j = 0; j < KK; ++j) {
          const int dj = dur[j];
          const double ldj = cld[j];
          double xb = kNegInfD, xe = kNegInfD;
          if (j < K && dj >= 1) {
            if (t + dj == Tl && u == Ul) xb = lb + ldj;
            else if (t + dj < Tl) xb = lb + ldj + ring[(k + dj) % kRing][u];
          }
          if (j < K && u < Ul && t + dj < Tl) xe = le + ldj + ring[(k + dj + 1) % kRing][u + 1];
          x[2 * j] = xb;
          x[2 * j + 1] = xe;
        }
        v = lse_terms(x);
        a.beta[idx(t, u)] = v;
      }
      ring[k % kRing][u] = on ? v : kNegInfD;
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ posteriors
//
// One thread per cell: gbt = sum_k gB, get = sum_k gE (float64; the token
// head's backward reads them as its transition posteriors), dzd (float32,
// the grad_costs weight included).
// (KK = the number of durations, a.K)
template <int KK>
__global__ __launch_bounds__(256) void tdt_post_kernel(TdtArgs a) {
  const Dims d = a.d;
  const int b = blockIdx.y, t = blockIdx.x;
  constexpr int K = KK;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t >= Tl) return;
  const double lp = a.logP[b];
  const double gc = a.gcost ? (double)a.gcost[b] : 1.0;
  // no alignment reaches the end (logP = -inf): cost +inf, gradients zero
  const bool dead = lp == kNegInfD;
  for (int u = threadIdx.x; u <= Ul; u += blockDim.x) {
    const size_t ix = skew_idx(d, b, t, u);
    if (dead) {
      a.gB[ix] = 0.0;
      a.gE[ix] = 0.0;
      for (int j = 0; j < K; ++j) a.dzd[ix * K + j] = 0.f;
      continue;
    }
    const double al = a.alpha[ix];
    const double lb = a.LB[ix], le = u < Ul ? (double)a.LE[ix] : 0.0;
    double sB = 0.0, sE = 0.0, g[KK];
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      g[j] = 0.0;
      if (j >= K) continue;
      const int dj = a.dur[j];
      const double ldj = a.LD[ix * K + j];
      double gb = 0.0, ge = 0.0;
      if (dj >= 1) {
        if (t + dj == Tl && u == Ul) gb = exp(al + lb + ldj - lp);
        else if (t + dj < Tl) gb = exp(al + lb + ldj + a.beta[skew_idx(d, b, t + dj, u)] - lp);
      }
      if (u < Ul && t + dj < Tl) ge = exp(al + le + ldj + a.beta[skew_idx(d, b, t + dj, u + 1)] - lp);
      sB += gb;
      sE += ge;
      g[j] = gb + ge;
    }
    a.gB[ix] = sB;
    a.gE[ix] = sE;
    const double occ = sB + sE;
#pragma unroll
    for (int j = 0; j < KK; ++j)
      if (j < K) a.dzd[ix * K + j] = (float)(gc * (occ * exp((double)a.LD[ix * K + j]) - g[j]));
  }
}

// ------------------------------------------------------------ duration head backward
//
// One workgroup per (b, block of kFrames frames); thread k0 owns the hidden
// units k0, k0 + 256, k0 + 512 (H <= 768), with those units' W_dur entries
// and the block's e^{2 enc} values in registers.  The duration-logit
// gradients of the block go through LDS in chunks of kUChunk label
// positions.  Per cell and unit, h is formed once and
//   dp = (1 - h^2) sum_j W_dur[k][j] dzd(t,u,j)
// is summed over the block's frames into the d_pred row of u (one float32
// atomic per unit and label position) and over the label positions into
// the frames' d_enc rows (atomics at the end); d_W_dur += h dzd and
// d_b_dur += dzd are summed over the block's cells.
constexpr int kFrames = kTdtFrames;
constexpr int kHPer = 3;  // hidden units per thread (H <= 768)
constexpr int kUChunk = 32;

// (KK = the number of durations, a.K)
template <int KK>
__global__ __launch_bounds__(256) void dur_bwd_kernel(TdtArgs a) {
  __shared__ float zs[kUChunk][kFrames][KK];
  const Dims d = a.d;
  const int b = blockIdx.y, tid = threadIdx.x;
  constexpr int K = KK;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  const int H = d.H;
  const bool use_ep = (a.hdr[1] & kFlagEpBad) == 0;
  const bool det = a.part_w != nullptr;
  const int t_lo = blockIdx.x * kFrames;
  if (t_lo >= Tl) return;  // uniform
  const int nt = min(kFrames, Tl - t_lo);
  float w[kHPer][KK], dw[kHPer][KK], db[KK];
  float e[kFrames][kHPer], ae[kFrames][kHPer];
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {
    const int k = tid + 256 * i;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      w[i][j] = (k < H && j < K) ? wdur(a, k, j) : 0.f;
      dw[i][j] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < kFrames; ++q) {
      const int t = t_lo + (q < nt ? q : 0);
      e[q][i] = (use_ep && k < H) ? a.Eexp[((size_t)b * d.T + t) * H + k] : 0.f;
      ae[q][i] = 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < KK; ++j) db[j] = 0.f;

  for (int u0 = 0; u0 <= Ul; u0 += kUChunk) {
    const int nu = min(kUChunk, Ul + 1 - u0);
    __syncthreads();  // the previous chunk's reads are done
    for (int i = tid; i < kUChunk * kFrames * KK; i += 256) {
      const int j = i % KK, q = (i / KK) % kFrames, uu = i / (KK * kFrames);
      float v = 0.f;
      if (uu < nu && q < nt && j < K) v = a.dzd[skew_idx(d, b, t_lo + q, u0 + uu) * K + j];
      zs[uu][q][j] = v;
    }
    __syncthreads();
    for (int uu = 0; uu < nu; ++uu) {
      const int u = u0 + uu;
      float p[kHPer], ap[kHPer];
#pragma unroll
      for (int i = 0; i < kHPer; ++i) {
        const int k = tid + 256 * i;
        p[i] = (use_ep && k < H) ? a.Pexp[((size_t)b * d.U1 + u) * H + k] : 0.f;
        ap[i] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < kFrames; ++q) {
        if (q >= nt) continue;  // uniform
        float z[KK];
#pragma unroll
        for (int j = 0; j < KK; ++j) {
          z[j] = zs[uu][q][j];
          db[j] += tid == 0 ? z[j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kHPer; ++i) {
          const int k = tid + 256 * i;
          if (k >= H) continue;
          const float h = use_ep ? 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e[q][i] * p[i])
                                 : h_of(a, b, t_lo + q, u, k, false);
          float sacc = 0.f;
#pragma unroll
          for (int j = 0; j < KK; ++j) sacc = fmaf(w[i][j], z[j], sacc);
          const float dp = (1.0f - h * h) * sacc;
          ae[q][i] += dp;
          ap[i] += dp;
          const float hr = h_round(a, h);
#pragma unroll
          for (int j = 0; j < KK; ++j) dw[i][j] = fmaf(hr, z[j], dw[i][j]);
        }
      }
      if (!det) {
#pragma unroll
        for (int i = 0; i < kHPer; ++i) {
          const int k = tid + 256 * i;
          if (k < H) atomicAdd(&a.d_pred[((size_t)b * d.U1 + u) * H + k], ap[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {
    const int k = tid + 256 * i;
    if (k >= H) continue;
#pragma unroll
    for (int q = 0; q < kFrames; ++q)
      if (q < nt) atomicAdd(&a.d_enc[((size_t)b * d.T + t_lo + q) * H + k], ae[q][i]);
    const size_t blk = (size_t)b * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      if (det) a.part_w[(blk * H + k) * K + j] = dw[i][j];
      else atomicAdd(&a.d_Wd[(size_t)k * K + j], dw[i][j]);
    }
  }
  if (tid == 0) {
    const size_t blk = (size_t)b * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < KK; ++j) {
      if (det) a.part_b[blk * K + j] = db[j];
      else atomicAdd(&a.d_bd[j], db[j]);
    }
  }
}

// Deterministic mode: d_pred's share of the duration head, one writer per
// element.  Workgroup (u block, b): thread k0 owns hidden units k0, k0 + 256,
// k0 + 512; for kUPer label positions it sums
//   dp = (1 - h^2) sum_j W_dur[k][j] dzd(t,u,j)
// over the frames in order and adds the sums to d_pred.
constexpr int kUPer = 4;
template <int KK>
__global__ __launch_bounds__(256) void dur_pred_kernel(TdtArgs a) {
  const Dims d = a.d;
  const int b = blockIdx.y, tid = threadIdx.x;
  constexpr int K = KK;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  const int H = d.H;
  const int u0 = blockIdx.x * kUPer;
  if (Tl == 0 || u0 > Ul) return;  // uniform
  const bool use_ep = (a.hdr[1] & kFlagEpBad) == 0;
  float w[kHPer][KK], ap[kUPer][kHPer], p[kUPer][kHPer];
#pragma unroll
  for (int i = 0; i < kHPer; ++i) {
    const int k = tid + 256 * i;
#pragma unroll
    for (int j = 0; j < KK; ++j) w[i][j] = k < H ? wdur(a, k, j) : 0.f;
#pragma unroll
    for (int q = 0; q < kUPer; ++q) {
      const int u = min(u0 + q, Ul);
      ap[q][i] = 0.f;
      p[q][i] = (use_ep && k < H) ? a.Pexp[((size_t)b * d.U1 + u) * H + k] : 0.f;
    }
  }
  for (int t = 0; t < Tl; ++t) {
    float e[kHPer];
#pragma unroll
    for (int i = 0; i < kHPer; ++i) {
      const int k = tid + 256 * i;
      e[i] = (use_ep && k < H) ? a.Eexp[((size_t)b * d.T + t) * H + k] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kUPer; ++q) {
      const int u = u0 + q;
      if (u > Ul) continue;  // uniform
      float z[KK];
      const float* zp = a.dzd + skew_idx(d, b, t, u) * K;
#pragma unroll
      for (int j = 0; j < KK; ++j) z[j] = zp[j];
#pragma unroll
      for (int i = 0; i < kHPer; ++i) {
        const int k = tid + 256 * i;
        if (k >= H) continue;
        const float h = use_ep ? 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e[i] * p[q][i])
                               : h_of(a, b, t, u, k, false);
        float sacc = 0.f;
#pragma unroll
        for (int j = 0; j < KK; ++j) sacc = fmaf(w[i][j], z[j], sacc);
        ap[q][i] += (1.0f - h * h) * sacc;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kUPer; ++q) {
    const int u = u0 + q;
    if (u > Ul) continue;
#pragma unroll
    for (int i = 0; i < kHPer; ++i) {
      const int k = tid + 256 * i;
      if (k < H) a.d_pred[((size_t)b * d.U1 + u) * H + k] += ap[q][i];
    }
  }
}

// Deterministic mode: d_W_dur and d_b_dur from the frame blocks' partial
// sums, added in block order (blocks past an utterance's length hold none).
__global__ __launch_bounds__(256) void dur_reduce_kernel(TdtArgs a, int nfb) {
  const int H = a.d.H, K = a.K;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < H * K) {
    float s = 0.f;
    for (int b = 0; b < a.d.B; ++b) {
      const int nb = (a.Teff[b] + kFrames - 1) / kFrames;
      for (int f = 0; f < nb; ++f) s += a.part_w[((size_t)b * nfb + f) * H * K + i];
    }
    a.d_Wd[i] += s;
  }
  if (i < K) {
    float s = 0.f;
    for (int b = 0; b < a.d.B; ++b) {
      const int nb = (a.Teff[b] + kFrames - 1) / kFrames;
      for (int f = 0; f < nb; ++f) s += a.part_b[((size_t)b * nfb + f) * K + i];
    }
    a.d_bd[i] += s;
  }
}

}  // namespace

hipError_t launch_tdt_dur_head(const TdtArgs& a, hipStream_t st) {
  const size_t lds = sizeof(float) * (size_t)a.d.H * (a.K + 1);
  const dim3 g(a.d.T, a.d.B), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL(dur_head_kernel<1>, g, blk, lds, st, a); break;
    case 2: hipLaunchKernelGGL(dur_head_kernel<2>, g, blk, lds, st, a); break;
    case 3: hipLaunchKernelGGL(dur_head_kernel<3>, g, blk, lds, st, a); break;
    case 4: hipLaunchKernelGGL(dur_head_kernel<4>, g, blk, lds, st, a); break;
    case 5: hipLaunchKernelGGL(dur_head_kernel<5>, g, blk, lds, st, a); break;
    case 6: hipLaunchKernelGGL(dur_head_kernel<6>, g, blk, lds, st, a); break;
    case 7: hipLaunchKernelGGL(dur_head_kernel<7>, g, blk, lds, st, a); break;
    case 8: hipLaunchKernelGGL(dur_head_kernel<8>, g, blk, lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tdt_lattice(const TdtArgs& a, hipStream_t st) {
  const dim3 g(a.d.B, 2), blk(512);
  switch (a.K) {
    case 1: hipLaunchKernelGGL(tdt_lattice_kernel<1>, g, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL(tdt_lattice_kernel<2>, g, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL(tdt_lattice_kernel<3>, g, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL(tdt_lattice_kernel<4>, g, blk, 0, st, a); break;
    case 5: hipLaunchKernelGGL(tdt_lattice_kernel<5>, g, blk, 0, st, a); break;
    case 6: hipLaunchKernelGGL(tdt_lattice_kernel<6>, g, blk, 0, st, a); break;
    case 7: hipLaunchKernelGGL(tdt_lattice_kernel<7>, g, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL(tdt_lattice_kernel<8>, g, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tdt_post(const TdtArgs& a, hipStream_t st) {
  const dim3 g(a.d.T, a.d.B), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL(tdt_post_kernel<1>, g, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL(tdt_post_kernel<2>, g, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL(tdt_post_kernel<3>, g, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL(tdt_post_kernel<4>, g, blk, 0, st, a); break;
    case 5: hipLaunchKernelGGL(tdt_post_kernel<5>, g, blk, 0, st, a); break;
    case 6: hipLaunchKernelGGL(tdt_post_kernel<6>, g, blk, 0, st, a); break;
    case 7: hipLaunchKernelGGL(tdt_post_kernel<7>, g, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL(tdt_post_kernel<8>, g, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_tdt_dur_bwd(const TdtArgs& a, hipStream_t st) {
  const int nfb = (a.d.T + kFrames - 1) / kFrames;
  const dim3 g(nfb, a.d.B), blk(256);
  switch (a.K) {
    case 1: hipLaunchKernelGGL(dur_bwd_kernel<1>, g, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL(dur_bwd_kernel<2>, g, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL(dur_bwd_kernel<3>, g, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL(dur_bwd_kernel<4>, g, blk, 0, st, a); break;
    case 5: hipLaunchKernelGGL(dur_bwd_kernel<5>, g, blk, 0, st, a); break;
    case 6: hipLaunchKernelGGL(dur_bwd_kernel<6>, g, blk, 0, st, a); break;
    case 7: hipLaunchKernelGGL(dur_bwd_kernel<7>, g, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL(dur_bwd_kernel<8>, g, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  if (!a.part_w) return hipGetLastError();
  // deterministic mode: d_pred by its own pass, then the ordered reduction
  const dim3 gp((a.d.U1 + kUPer - 1) / kUPer, a.d.B);
  switch (a.K) {
    case 1: hipLaunchKernelGGL(dur_pred_kernel<1>, gp, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL(dur_pred_kernel<2>, gp, blk, 0, st, a); break;
    case 3: hipLaunchKernelGGL(dur_pred_kernel<3>, gp, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL(dur_pred_kernel<4>, gp, blk, 0, st, a); break;
    case 5: hipLaunchKernelGGL(dur_pred_kernel<5>, gp, blk, 0, st, a); break;
    case 6: hipLaunchKernelGGL(dur_pred_kernel<6>, gp, blk, 0, st, a); break;
    case 7: hipLaunchKernelGGL(dur_pred_kernel<7>, gp, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL(dur_pred_kernel<8>, gp, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(dur_reduce_kernel, dim3((a.d.H * a.K + 255) / 256), blk, 0, st, a, nfb);
  return hipGetLastError();
}

}  // namespace rnntj
