// Lattice recursions and small helper kernels.
//
// Alpha / beta over the transducer lattice (RNN transducer definition on the
// "Daily Papers" page, abstract on sequence transduction with recurrent
// networks; the full sum over alignments, as opposed to the maximum
// approximation discussed in the abstract comparing the two criteria):
//   alpha(0,0) = 0
//   alpha(t,u) = logaddexp(alpha(t-1,u) + LB(t-1,u), alpha(t,u-1) + LE(t,u-1))
//   logP = alpha(T'-1,U') + LB(T'-1,U')
//   beta(T'-1,U') = LB(T'-1,U')
//   beta(t,u) = logaddexp(beta(t+1,u) + LB(t,u), beta(t,u+1) + LE(t,u))
//
// One wave64 per (utterance, direction): cells of one anti-diagonal t+u are
// independent, so the wave sweeps the T'+U' anti-diagonals with label
// position u = 64*j + lane held in register slot j.  The u-1 / u+1
// neighbour on the previous diagonal comes from the adjacent lane by a
// cross-lane shuffle.  State is float64 (the posteriors later take
// exp(alpha + beta - logP) of numbers of size ~1e4); the logaddexp
// correction log(1 + e^-|x-y|) lies in [0, ln 2] and is evaluated in float32.
// LB / LE of upcoming diagonals are loaded kPrefetch steps ahead.
#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr double kNegInfD = -__builtin_inf();
constexpr int kPrefetch = 4;

__device__ __forceinline__ double log_add_exp(double x, double y) {
  // comparisons (not fmax) so that a NaN operand propagates
  const bool xg = x > y;
  const double hi = xg ? x : y;
  const double lo = xg ? y : x;
  if (hi == kNegInfD) return kNegInfD;
  const float dl = (float)(lo - hi);
  const float c = __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(dl * kLog2e)) * kLn2;
  return hi + (double)c;
}

template <int NU>
__global__ __launch_bounds__(64) void lattice_kernel(const float* __restrict__ LB,
                                                     const float* __restrict__ LE,
                                                     const int32_t* __restrict__ Teff,
                                                     const int32_t* __restrict__ Ueff, Dims d,
                                                     double* __restrict__ alpha,
                                                     double* __restrict__ beta,
                                                     double* __restrict__ logP,
                                                     float* __restrict__ costs) {
  const int b = blockIdx.x, dir = blockIdx.y, l = threadIdx.x;
  const int Tl = Teff[b], Ul = Ueff[b];
  if (Tl == 0) {  // invalid utterance
    if (dir == 0 && l == 0) {
      costs[b] = __builtin_nanf("");
      logP[b] = __builtin_nan("");
    }
    return;
  }
  const int nd = Tl + Ul;  // number of anti-diagonals of this lattice
  const size_t base = (size_t)b * d.DG * d.U1;
  const float* lb = LB + base;
  const float* le = LE + base;
  double* out = (dir == 0 ? alpha : beta) + base;

  double prev[NU];
#pragma unroll
  for (int j = 0; j < NU; ++j) prev[j] = kNegInfD;

  // operands of step s (anti-diagonal dg(s)) for slot j:
  //   alpha: LB(t-1,u), LE(t,u-1) (both on diagonal dg-1)
  //   beta : LB(t,u),   LE(t,u)   (on diagonal dg)
  auto diag_of = [&](int s) { return dir == 0 ? s : nd - 1 - s; };
  auto fetch = [&](int s, float (&fb)[NU], float (&fe)[NU]) {
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      fb[j] = 0.f;
      fe[j] = 0.f;
    }
    if (s >= nd) return;
    const int dg = diag_of(s);
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int u = 64 * j + l;
      const int t = dg - u;
      if (u > Ul || t < 0 || t >= Tl) continue;
      if (dir == 0) {
        if (t >= 1) fb[j] = lb[(size_t)(dg - 1) * d.U1 + u];
        if (u >= 1) fe[j] = le[(size_t)(dg - 1) * d.U1 + u - 1];
      } else {
        fb[j] = lb[(size_t)dg * d.U1 + u];
        if (u < Ul) fe[j] = le[(size_t)dg * d.U1 + u];
      }
    }
  };

  float rb[kPrefetch][NU], re[kPrefetch][NU];
#pragma unroll
  for (int p = 0; p < kPrefetch; ++p) fetch(p, rb[p], re[p]);

  for (int s0 = 0; s0 < nd; s0 += kPrefetch) {
#pragma unroll
    for (int p = 0; p < kPrefetch; ++p) {
      const int s = s0 + p;
      if (s < nd) {  // uniform across the wave
        float cb[NU], ce[NU];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
          cb[j] = rb[p][j];
          ce[j] = re[p][j];
        }
        fetch(s + kPrefetch, rb[p], re[p]);
        const int dg = diag_of(s);
        double nb[NU];
        if (dir == 0) {
          // alpha(t, u-1) on the previous diagonal: lane l-1 (slot j), or
          // lane 63 of slot j-1 for lane 0
#pragma unroll
          for (int j = 0; j < NU; ++j) {
            const double up = __shfl_up(prev[j], 1);
            const double wrap = __shfl(j > 0 ? prev[j > 0 ? j - 1 : 0] : kNegInfD, 63);
            nb[j] = (l == 0) ? (j > 0 ? wrap : kNegInfD) : up;
          }
        } else {
          // beta(t, u+1) on the previous (later) diagonal: lane l+1 (slot j),
          // or lane 0 of slot j+1 for lane 63
#pragma unroll
          for (int j = 0; j < NU; ++j) {
            const double dn = __shfl_down(prev[j], 1);
            const double wrap = __shfl(j + 1 < NU ? prev[j + 1 < NU ? j + 1 : 0] : kNegInfD, 0);
            nb[j] = (l == 63) ? (j + 1 < NU ? wrap : kNegInfD) : dn;
          }
        }
        double cur[NU];
#pragma unroll
        for (int j = 0; j < NU; ++j) {
          const int u = 64 * j + l;
          const int t = dg - u;
          const bool valid = (u <= Ul) && (t >= 0) && (t < Tl);
          double v = kNegInfD;
          if (valid) {
            if (dir == 0) {
              if (dg == 0) {
                v = 0.0;
              } else {
                const double ft = (t >= 1) ? prev[j] + (double)cb[j] : kNegInfD;
                const double fu = (u >= 1) ? nb[j] + (double)ce[j] : kNegInfD;
                v = log_add_exp(ft, fu);
              }
            } else {
              if (t == Tl - 1 && u == Ul) {
                v = (double)cb[j];
              } else {
                const double ft = (t + 1 < Tl) ? prev[j] + (double)cb[j] : kNegInfD;
                const double fu = (u < Ul) ? nb[j] + (double)ce[j] : kNegInfD;
                v = log_add_exp(ft, fu);
              }
            }
            out[(size_t)dg * d.U1 + u] = v;
          }
          cur[j] = v;
        }
#pragma unroll
        for (int j = 0; j < NU; ++j) prev[j] = cur[j];
        if (dir == 0 && s == nd - 1) {
          // final cell (T'-1, U') lies on the last diagonal
#pragma unroll
          for (int j = 0; j < NU; ++j) {
            if (64 * j + l == Ul) {
              const double lp = cur[j] + (double)lb[(size_t)dg * d.U1 + Ul];
              logP[b] = lp;
              costs[b] = (float)(-lp);
            }
          }
        }
      }
    }
  }
}

__global__ void validate_kernel(const int32_t* __restrict__ T_lens,
                                const int32_t* __restrict__ U_lens,
                                const int32_t* __restrict__ labels, Dims d,
                                int32_t* __restrict__ Teff, int32_t* __restrict__ Ueff,
                                int32_t* __restrict__ status) {
  __shared__ int sbad;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) sbad = 0;
  __syncthreads();
  const int Tl = T_lens[b], Ul = U_lens[b];
  int bad = 0;
  if (Tl < 1 || Tl > d.T || Ul < 0 || Ul > d.U) {
    bad = 1;
  } else {
    for (int u = threadIdx.x; u < Ul; u += blockDim.x) {
      const int y = labels[(size_t)b * d.U + u];
      if (y < 0 || y >= d.V || y == d.blank) bad |= 2;
    }
  }
  if (bad) atomicOr(&sbad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    Teff[b] = sbad ? 0 : Tl;
    Ueff[b] = sbad ? 0 : Ul;
    if (sbad) atomicOr(status, sbad);
  }
}

template <typename E>
__global__ void transpose_kernel(const E* __restrict__ src, E* __restrict__ dst, int H, int V) {
  __shared__ E tile[32][33];
  const int v0 = blockIdx.x * 32, h0 = blockIdx.y * 32;
  const int tx = threadIdx.x, ty = threadIdx.y;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int h = h0 + i, v = v0 + tx;
    if (h < H && v < V) tile[i][tx] = src[(size_t)h * V + v];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int v = v0 + i, h = h0 + tx;
    if (v < V && h < H) dst[(size_t)v * H + h] = tile[tx][i];
  }
}

// e^{2x} of every enc and pred element (accurate expf), and the flag that
// some finite |x| exceeds 40, where e^{2x} alone could overflow although the
// joint's sum enc + pred is moderate.
template <typename E>
__global__ void ep_kernel(const E* __restrict__ enc, const E* __restrict__ pred, Dims d,
                          float* __restrict__ Eexp, float* __restrict__ Pexp,
                          int32_t* __restrict__ hdr) {
  const size_t ne = (size_t)d.B * d.T * d.H, np = (size_t)d.B * d.U1 * d.H;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < ne + np; i += stride) {
    const float x = i < ne ? ElemTraits<E>::to_f32(enc[i]) : ElemTraits<E>::to_f32(pred[i - ne]);
    const float ax = fabsf(x);
    if (ax > 40.0f && ax != __builtin_inff()) bad = true;
    const float e = expf(2.0f * x);
    if (i < ne)
      Eexp[i] = e;
    else
      Pexp[i - ne] = e;
  }
  if (bad) atomicOr(&hdr[1], kFlagEpBad);
}

// hdr[2] = max_v (|b[v]| + sum_k |W[k,v]|) as float bits (non-negative, so
// integer max orders them; a NaN column bound wins and disables the bound).
template <typename E>
__global__ void colbound_kernel(const E* __restrict__ W, const E* __restrict__ bias, Dims d,
                                int32_t* __restrict__ hdr) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= d.V) return;
  float s = fabsf(ElemTraits<E>::to_f32(bias[v]));
  for (int k = 0; k < d.H; ++k) s += fabsf(ElemTraits<E>::to_f32(W[(size_t)k * d.V + v]));
  atomicMax(&hdr[2], __float_as_int(s));
}

__global__ void zero_kernel(uint32_t* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

hipError_t launch_lattice(const float* LB, const float* LE, const int32_t* Teff,
                          const int32_t* Ueff, const Dims& d, double* alpha, double* beta,
                          double* logP, float* costs, hipStream_t st) {
  const int nu = (d.U1 + 63) / 64;
  dim3 grid(d.B, 2), block(64);
#define RNNTJ_LAT(N)                                                                        \
  case N:                                                                                   \
    hipLaunchKernelGGL(lattice_kernel<N>, grid, block, 0, st, LB, LE, Teff, Ueff, d, alpha, \
                       beta, logP, costs);                                                  \
    break;
  switch (nu) {
    RNNTJ_LAT(1)
    RNNTJ_LAT(2)
    RNNTJ_LAT(3)
    RNNTJ_LAT(4)
    RNNTJ_LAT(5)
    RNNTJ_LAT(6)
    RNNTJ_LAT(7)
    RNNTJ_LAT(8)
    default:
      return hipErrorInvalidValue;
  }
#undef RNNTJ_LAT
  return hipGetLastError();
}

hipError_t launch_validate(const int32_t* T_lens, const int32_t* U_lens,
                           const int32_t* labels, const Dims& d, int32_t* Teff,
                           int32_t* Ueff, int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(d.B), dim3(256), 0, st, T_lens, U_lens, labels, d,
                     Teff, Ueff, status);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int H, int V, bool bf16,
                            hipStream_t st) {
  dim3 grid((V + 31) / 32, (H + 31) / 32), block(32, 8);
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, block, 0, st,
                       static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), H, V);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, st,
                       static_cast<const float*>(src), static_cast<float*>(dst), H, V);
  return hipGetLastError();
}

hipError_t launch_prep(const void* enc, const void* pred, const void* W, const void* bias,
                       bool bf16, const Dims& d, float* Eexp, float* Pexp, int32_t* hdr,
                       hipStream_t st) {
  const size_t n = (size_t)d.B * (d.T + d.U1) * d.H;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 gb((d.V + 255) / 256);
  if (bf16) {
    hipLaunchKernelGGL(ep_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(enc), static_cast<const uint16_t*>(pred), d,
                       Eexp, Pexp, hdr);
    hipLaunchKernelGGL(colbound_kernel<uint16_t>, gb, dim3(256), 0, st,
                       static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(bias), d, hdr);
  } else {
    hipLaunchKernelGGL(ep_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const float*>(enc), static_cast<const float*>(pred), d, Eexp,
                       Pexp, hdr);
    hipLaunchKernelGGL(colbound_kernel<float>, gb, dim3(256), 0, st,
                       static_cast<const float*>(W), static_cast<const float*>(bias), d, hdr);
  }
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t n_words, hipStream_t st) {
  if (n_words == 0) return hipSuccess;
  size_t blocks = (n_words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<uint32_t*>(p), n_words);
  return hipGetLastError();
}

}  // namespace rnntj
