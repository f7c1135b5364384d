// Backward kernels of the fused RNN-T joint + transducer loss.
//
// Gradient of sum_b gc_b * cost_b (transducer lattice as defined on the
// "Daily Papers" page, abstract on sequence transduction with recurrent
// networks; joint and loss of the "Flash RNN-T" page, Abstract):
//   dz(t,u)[v] = gc * (occ * softmax(z)[v] - gB [v=blank] - gE [v=y_u])
//   dW_out = sum_cells h^T dz,   db_out = sum_cells dz
//   dh = dz @ W_out^T,  dpre = (1 - h^2) * dh,
//   d_enc[t] = sum_u dpre(t,u),  d_pred[u] = sum_t dpre(t,u)
//
// Kernels here:
//   grad_inplace_kernel : untiled mode, stored logits -> dz in place.
//   dh_kernel           : MFMA GEMM dz[cells, V] x W_out^T -> [cells, H] for
//                         one 16x8 cell tile and 128 hidden columns, with the
//                         (1 - h^2) epilogue and the two lattice reductions
//                         done in registers before float32 atomics.
//   dw_kernel           : MFMA GEMM h^T[H, cells] x dz[cells, V] split over
//                         utterances (split-K); h and dz rows are staged
//                         row-major and read with transposing LDS loads; the
//                         hidden-row-0 workgroups also sum dz columns into
//                         db_out (float64).
//   hrow_kernel         : untiled mode, h = tanh(enc + pred) rows for dw.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr float kInf = __builtin_inff();

// ------------------------------------------------------------ untiled dz

template <typename T>
__global__ __launch_bounds__(256) void grad_inplace_kernel(T* __restrict__ z, JointArgs a) {
  __shared__ float row_c[kTileCells], row_b[kTileCells], row_e[kTileCells];
  __shared__ int row_y[kTileCells];
  const Dims d = a.d;
  const int b = blockIdx.y;
  const int n_tu = d.U1pad / kTileU;
  const int t0 = (blockIdx.x / n_tu) * kTileT;
  const int u0 = (blockIdx.x % n_tu) * kTileU;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t0 >= Tl || u0 > Ul) return;
  const int tid = threadIdx.x;
  if (tid < kTileCells) {
    const int t = t0 + (tid >> 3), u = u0 + (tid & 7);
    float c = kInf, gb = 0.f, ge = 0.f;
    int y = -1;
    if (t < Tl && u <= Ul) {
      const double g = a.gcost ? (double)a.gcost[b] : 1.0;
      double gB, gE;
      cell_posteriors(d, a.alpha, a.beta, a.LB, a.LE, a.logP[b], b, t, u, Tl, Ul, gB, gE);
      const double occ = gB + gE;
      const double lse = (double)a.lse[skew_idx(d, b, t, u)];
      c = occ > 0.0 ? (float)(lse - log(occ)) : kInf;
      gb = (float)(g * gB);
      ge = (float)(g * gE);
      if (u < Ul) y = a.labels[(size_t)b * d.U + u];
    }
    row_c[tid] = c;
    row_b[tid] = gb;
    row_e[tid] = ge;
    row_y[tid] = y;
  }
  __syncthreads();
  const float gc = a.gcost ? a.gcost[b] : 1.0f;
  const int V = d.V;
  const int cpr = V / 8;  // 8-element chunks per row
  for (int c = tid; c < kTileCells * cpr; c += 256) {
    const int row = c / cpr, v0 = (c % cpr) * 8;
    const int t = t0 + (row >> 3), u = u0 + (row & 7);
    T* zp = z + (((size_t)b * d.Tpad + t) * d.U1pad + u) * V + v0;
    Frag8<T> f;
    if (t < Tl && u <= Ul) {
      f = load_frag(zp);
      float x[8];
      const float cr = row_c[row];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float g = gc * __expf(f.get(i) - cr);
        if (v0 + i == d.blank) g -= row_b[row];
        if (v0 + i == row_y[row]) g -= row_e[row];
        x[i] = g;
      }
      pack_frag(f, x);
    } else {
      zero_frag(f);
    }
    store_frag(zp, f);
  }
}

// ------------------------------------------------------------ staging config

template <typename T>
struct Cfg {
  static constexpr int BK = std::is_same<T, float>::value ? 32 : 64;  // dh: k (vocab) per stage
  static constexpr int CE = 16 / (int)sizeof(T);
  static constexpr int LDK = BK + CE;
  static constexpr int CH = 128 * BK / CE / 256;  // 16 B chunks per thread per operand
};

// ------------------------------------------------------------ dh GEMM

template <typename T>
__device__ __forceinline__ void dh_load(const DhArgs& a, int b, int t0, int u0, int Tl, int Ul,
                                        int n0, int k0, u32x4 (&ra)[Cfg<T>::CH],
                                        u32x4 (&rb)[Cfg<T>::CH]) {
  using C = Cfg<T>;
  const T* g = static_cast<const T*>(a.g);
  const T* W = static_cast<const T*>(a.W);
  const Dims& d = a.d;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < C::CH; ++q) {
    const int c = tid + 256 * q;
    const int row = c / (C::BK / C::CE);
    const int col = (c % (C::BK / C::CE)) * C::CE;
    const int k = k0 + col;
    // A: dz rows of the cell tile, row = 8*tt + uu
    const int t = t0 + (row >> 3), u = u0 + (row & 7);
    if (t < Tl && u <= Ul && k < d.V)
      ra[q] = *reinterpret_cast<const u32x4*>(
          g + (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * d.V + k);
    else
      ra[q] = u32x4{0u, 0u, 0u, 0u};
    // B: W_out rows n0 + row (hidden index), contiguous in the vocabulary
    const int n = n0 + row;
    if (n < d.H && k < d.V)
      rb[q] = *reinterpret_cast<const u32x4*>(W + (size_t)n * d.V + k);
    else
      rb[q] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T>
__device__ __forceinline__ void stage_store(T* lds, const u32x4 (&r)[Cfg<T>::CH]) {
  using C = Cfg<T>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < C::CH; ++q) {
    const int c = tid + 256 * q;
    const int row = c / (C::BK / C::CE);
    const int col = (c % (C::BK / C::CE)) * C::CE;
    *reinterpret_cast<u32x4*>(lds + row * C::LDK + col) = r[q];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void dh_kernel(DhArgs a) {
  using C = Cfg<T>;
  __shared__ __align__(16) T As[2][128 * C::LDK];
  __shared__ __align__(16) T Bs[2][128 * C::LDK];
  const Dims d = a.d;
  const int b = blockIdx.z;
  const int t0 = a.ct0 + (blockIdx.x / a.n_tu) * kTileT;
  const int u0 = a.cu0 + (blockIdx.x % a.n_tu) * kTileU;
  const int n0 = blockIdx.y * 128;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t0 >= Tl || u0 > Ul) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kh = lane >> 5, lc = lane & 31;
  const int wm = w >> 1, wn = w & 1;  // 64 rows x 64 cols per wave

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[C::CH], rb[C::CH];
  const int nk = (d.V + C::BK - 1) / C::BK;
  dh_load<T>(a, b, t0, u0, Tl, Ul, n0, 0, ra, rb);
  stage_store<T>(As[0], ra);
  stage_store<T>(Bs[0], rb);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    const bool has_next = kb + 1 < nk;
    if (has_next) dh_load<T>(a, b, t0, u0, Tl, Ul, n0, (kb + 1) * C::BK, ra, rb);
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      Frag8<T> fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = load_frag(&As[cur][(64 * wm + 32 * i + lc) * C::LDK + kk * 16 + 8 * kh]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = load_frag(&Bs[cur][(64 * wn + 32 * j + lc) * C::LDK + kk * 16 + 8 * kh]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma_step(acc[i][j], fa[i], fb[j]);
    }
    if (has_next) {
      stage_store<T>(As[cur ^ 1], ra);
      stage_store<T>(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }

  // ---- epilogue: dpre = (1 - h^2) * dh, h rebuilt from enc / pred
  const T* enc = static_cast<const T*>(a.enc);
  const T* pred = static_cast<const T*>(a.pred);
  const bool use_ep = (a.hdr[1] & kFlagEpBad) == 0;
  // wave rows: 64*wm + 32*i + acc_row(r, kh)  <->  tt = 8*wm + 4*i + r/4, uu = 4*kh + r%4
  float pred_sum[2][4];  // [j][r%4]: sum over this wave's frames, per label position
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) pred_sum[j][q] = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + lc;
    const bool nvalid = n < d.H;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {  // frame within the 32-row block
        const int t = t0 + 8 * wm + 4 * i + q4;
        float enc_sum = 0.f;
        const bool tn = nvalid && t < Tl;
        const size_t ie = ((size_t)b * d.T + t) * d.H + n;
        const float ev = tn ? (use_ep ? a.Eexp[ie] : ElemTraits<T>::to_f32(enc[ie])) : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // label position within the half
          const int r = 4 * q4 + q;
          const int u = u0 + 4 * kh + q;
          float v = 0.f;
          if (tn && u <= Ul) {
            const size_t ip = ((size_t)b * d.U1 + u) * d.H + n;
            const float h = use_ep
                                ? 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + ev * a.Pexp[ip])
                                : fast_tanh(ev + ElemTraits<T>::to_f32(pred[ip]));
            v = (1.0f - h * h) * acc[i][j][r];
          }
          enc_sum += v;
          pred_sum[j][q] += v;
        }
        // the other 4 label positions of this frame live in lane l ^ 32
        enc_sum += __shfl_xor(enc_sum, 32);
        if (kh == 0 && nvalid && t < Tl)
          atomicAdd(&a.d_enc[((size_t)b * d.T + t) * d.H + n], enc_sum);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + lc;
    if (n < d.H) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = u0 + 4 * kh + q;
        if (u <= Ul) atomicAdd(&a.d_pred[((size_t)b * d.U1 + u) * d.H + n], pred_sum[j][q]);
      }
    }
  }
}

// ------------------------------------------------------------ dW GEMM

// d_W_out[m0:m0+128, n0:n0+128] += h^T dz over the valid cells of one
// utterance in the chunk.  h rows [cell][H] and dz rows [cell][V] are staged
// row-major (16-byte copies) and read as MFMA operands with load_frag_T, so
// neither operand is transposed in memory.  K block = 8 frames x 8 label
// positions (bf16) or 4 x 8 (fp32) of one 16x8 cell tile.
template <typename T>
struct DwCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int KB = kBf16 ? 64 : 32;           // cells per stage
  static constexpr int LD = 128 + (kBf16 ? 16 : 4);    // LDS row (elements): 288 B / 528 B
  static constexpr int CE = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  static constexpr int CPR = 128 / CE;                 // chunks per staged row
  static constexpr int CH = KB * CPR / 256;            // chunks per thread per operand
  static constexpr int SPT = kTileCells / KB;          // stages per cell tile
};

template <typename T>
__global__ __launch_bounds__(256) void dw_kernel(DwArgs a) {
  using C = DwCfg<T>;
  __shared__ __align__(16) T As[2][C::KB * C::LD];  // h  [cell][hidden]
  __shared__ __align__(16) T Bs[2][C::KB * C::LD];  // dz [cell][vocab]
  __shared__ double dbw[4][128];
  const Dims d = a.d;
  const int n0 = blockIdx.x * 128, m0 = blockIdx.y * 128;
  const int b = blockIdx.z / a.ksplit, kpart = blockIdx.z % a.ksplit;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  // valid cell tiles of this utterance inside the chunk form a rectangle;
  // this workgroup takes the kpart-th of ksplit equal runs of their stages
  const int tv = min(a.CT, Tl - a.ct0), uv = min(a.CU, Ul + 1 - a.cu0);
  if (tv <= 0 || uv <= 0) return;
  const int ntt = (tv + kTileT - 1) / kTileT, ntu = (uv + kTileU - 1) / kTileU;
  const int nall = ntt * ntu * C::SPT;
  const int s_begin = (int)(((long long)nall * kpart) / a.ksplit);
  const int s_end = (int)(((long long)nall * (kpart + 1)) / a.ksplit);
  const int nstage = s_end - s_begin;
  if (nstage <= 0) return;
  const int n_tu = a.CU / kTileU;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const bool do_db = (blockIdx.y == 0);
  const T* hsrc = static_cast<const T*>(a.h);
  const T* gsrc = static_cast<const T*>(a.g);
  // this thread's staging chunks: row = c / CPR, column chunk = c % CPR
  // (c = tid + 256 q, so the column chunk is the same for every q)
  const int ccol = (tid % C::CPR) * C::CE;
  const bool mok = m0 + ccol < d.H, nok = n0 + ccol < d.V;
  double dbacc[C::CE];
#pragma unroll
  for (int i = 0; i < C::CE; ++i) dbacc[i] = 0.0;

  u32x4 ra[C::CH], rb[C::CH];
  auto load_stage = [&](int sl) {
    const int s = s_begin + sl;
    const int tile = s / C::SPT, part = s % C::SPT;
    const int t0 = a.ct0 + (tile / ntu) * kTileT + part * (C::KB / kTileU);
    const int u0 = a.cu0 + (tile % ntu) * kTileU;
#pragma unroll
    for (int q = 0; q < C::CH; ++q) {
      const int row = (tid + 256 * q) / C::CPR;
      const int t = t0 + row / kTileU, u = u0 + row % kTileU;
      const bool ok = t < Tl && u <= Ul;
      const size_t crow = ((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0);
      ra[q] = (ok && mok) ? *reinterpret_cast<const u32x4*>(hsrc + crow * d.H + m0 + ccol)
                          : u32x4{0u, 0u, 0u, 0u};
      rb[q] = (ok && nok) ? *reinterpret_cast<const u32x4*>(gsrc + crow * d.V + n0 + ccol)
                          : u32x4{0u, 0u, 0u, 0u};
    }
    (void)n_tu;
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int q = 0; q < C::CH; ++q) {
      const int row = (tid + 256 * q) / C::CPR;
      *reinterpret_cast<u32x4*>(&As[buf][row * C::LD + ccol]) = ra[q];
      *reinterpret_cast<u32x4*>(&Bs[buf][row * C::LD + ccol]) = rb[q];
      if (do_db) {
        Frag8<T> f;
        if constexpr (C::kBf16) {
          f.v = rb[q];
        } else {
          f.lo = __builtin_bit_cast(f32x4, rb[q]);
        }
#pragma unroll
        for (int i = 0; i < C::CE; ++i) dbacc[i] += (double)f.get(i);
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    const bool has_next = s + 1 < nstage;
    if (has_next) load_stage(s + 1);
#pragma unroll
    for (int kk = 0; kk < C::KB / 16; ++kk) {
      Frag8<T> fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = load_frag_T(As[cur], C::LD, kk * 16, 64 * wm + 32 * i);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = load_frag_T(Bs[cur], C::LD, kk * 16, 64 * wn + 32 * j);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma_step(acc[i][j], fa[i], fb[j]);
    }
    if (has_next) store_stage(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wn + 32 * j + (lane & 31);
      if (n < d.V) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 64 * wm + 32 * i + acc_row(r, kh);
          if (m < d.H) atomicAdd(&a.d_W[(size_t)m * d.V + n], acc[i][j][r]);
        }
      }
    }

  if (do_db) {
    // threads with equal tid % CPR share columns: 4 per wave for bf16
    // (CPR = 16), 2 per wave for fp32 (CPR = 32); then across the 4 waves
#pragma unroll
    for (int i = 0; i < C::CE; ++i) {
      double v = dbacc[i];
      for (int off = C::CPR; off < 64; off <<= 1) v += __shfl_xor(v, off);
      dbacc[i] = v;
    }
    if (lane < C::CPR) {
#pragma unroll
      for (int i = 0; i < C::CE; ++i) dbw[w][ccol + i] = dbacc[i];
    }
    __syncthreads();
    if (tid < 128 && n0 + tid < d.V)
      atomicAdd(&a.d_b64[n0 + tid], dbw[0][tid] + dbw[1][tid] + dbw[2][tid] + dbw[3][tid]);
  }
}

// h rows of every valid cell of the lattice ([B, Tpad, U1pad, H], untiled
// backward): h = tanh(enc[b,t] + pred[b,u]); rows of invalid cells are zero.
template <typename T>
__global__ __launch_bounds__(256) void hrow_kernel(JointArgs a, T* __restrict__ hout) {
  const Dims d = a.d;
  const int b = blockIdx.y;
  const int n_tu = d.U1pad / kTileU;
  const int t0 = (blockIdx.x / n_tu) * kTileT;
  const int u0 = (blockIdx.x % n_tu) * kTileU;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t0 >= Tl || u0 > Ul) return;
  const T* enc = static_cast<const T*>(a.enc);
  const T* pred = static_cast<const T*>(a.pred);
  const bool use_ep = (a.hdr[1] & kFlagEpBad) == 0;
  const int cpr = d.H / 8;
  for (int c = threadIdx.x; c < kTileCells * cpr; c += 256) {
    const int row = c / cpr, k0 = (c % cpr) * 8;
    const int t = t0 + (row >> 3), u = u0 + (row & 7);
    T* hp = hout + (((size_t)b * d.Tpad + t) * d.U1pad + u) * d.H + k0;
    Frag8<T> f;
    if (t < Tl && u <= Ul) {
      const size_t ie = ((size_t)b * d.T + t) * d.H + k0, ip = ((size_t)b * d.U1 + u) * d.H + k0;
      float x[8];
      if (use_ep) {
        const Frag8<float> e = load_frag(a.Eexp + ie), p = load_frag(a.Pexp + ip);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          x[i] = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e.get(i) * p.get(i));
      } else {
        const Frag8<T> e = load_frag(enc + ie), p = load_frag(pred + ip);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fast_tanh(e.get(i) + p.get(i));
      }
      pack_frag(f, x);
    } else {
      zero_frag(f);
    }
    store_frag(hp, f);
  }
}

__global__ void db_finalize_kernel(const double* __restrict__ src, float* __restrict__ dst, int V) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < V) dst[v] = (float)src[v];
}

}  // namespace

hipError_t launch_db_finalize(const double* db64, float* d_b, int V, hipStream_t st) {
  hipLaunchKernelGGL(db_finalize_kernel, dim3((V + 255) / 256), dim3(256), 0, st, db64, d_b, V);
  return hipGetLastError();
}

hipError_t launch_hrow(void* h, bool bf16, const JointArgs& a, hipStream_t st) {
  dim3 grid((a.d.Tpad / kTileT) * (a.d.U1pad / kTileU), a.d.B), block(256);
  if (bf16)
    hipLaunchKernelGGL(hrow_kernel<uint16_t>, grid, block, 0, st, a, static_cast<uint16_t*>(h));
  else
    hipLaunchKernelGGL(hrow_kernel<float>, grid, block, 0, st, a, static_cast<float*>(h));
  return hipGetLastError();
}

hipError_t launch_grad_inplace(void* z, bool bf16, const JointArgs& a, hipStream_t st) {
  dim3 grid((a.d.Tpad / kTileT) * (a.d.U1pad / kTileU), a.d.B), block(256);
  if (bf16)
    hipLaunchKernelGGL(grad_inplace_kernel<uint16_t>, grid, block, 0, st,
                       static_cast<uint16_t*>(z), a);
  else
    hipLaunchKernelGGL(grad_inplace_kernel<float>, grid, block, 0, st, static_cast<float*>(z),
                       a);
  return hipGetLastError();
}

hipError_t launch_dh(const DhArgs& a, bool bf16, hipStream_t st) {
  dim3 grid((a.CT / kTileT) * a.n_tu, (a.d.H + 127) / 128, a.d.B), block(256);
  if (bf16)
    hipLaunchKernelGGL(dh_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(dh_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dw(const DwArgs& a, bool bf16, hipStream_t st) {
  dim3 grid((a.d.V + 127) / 128, (a.d.H + 127) / 128, a.d.B * a.ksplit), block(256);
  if (bf16)
    hipLaunchKernelGGL(dw_kernel<uint16_t>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(dw_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace rnntj
