// Fused joint + vocabulary projection over one tile of lattice cells.
//
// "Flash RNN-T" page, Abstract: the joint network and the loss are computed
// by specialised kernels, optionally recomputing over tiles of the alignment
// lattice and of the vocabulary so that the [B,T,U+1,V] logits need not be
// kept.  Per cell (t,u) of utterance b:
//     h = tanh(enc[b,t] + pred[b,u])      (built once, kept in registers)
//     z = h @ W_out + b_out               (MFMA, one 128-column vocab tile
//                                          at a time)
// and one of three epilogues per vocabulary tile:
//   kLse    : online max / sum-exp (base 2) carried across vocabulary tiles;
//             at the end lse, LB = z[blank] - lse, LE = z[label] - lse.
//   kStoreZ : kLse plus the logits written to HBM (untiled mode).
//   kGrad   : logit gradient of the loss (tiled backward), from the per-cell
//             transition posteriors gB, gE and the stored lse:
//             dz[v] = gc * (occ * exp(z[v] - lse) - gB [v=blank] - gE [v=y_u]),
//             occ = gB + gE, written to a chunk buffer.
//
// Work decomposition (gfx950, wave64): a workgroup = 4 waves = one tile of
// 16 frames x 8 label positions of one utterance.  Wave w owns frames
// t0+4w..t0+4w+3 x label positions u0..u0+7 = 32 rows of a 32x32 MFMA block,
// row r <-> (t0 + 4w + r/8, u0 + r%8).  The wave keeps its 32 rows of h for
// the whole H in registers as MFMA A-fragments, and streams W_out^T through
// LDS in [128 vocab x BK] slices (double buffered); each slice feeds four
// 32x32 output blocks per wave.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr float kInf = __builtin_inff();

template <typename T>
struct StageCfg {
  static constexpr int BK = std::is_same<T, float>::value ? 32 : 64;  // k per slice
  static constexpr int CE = 16 / (int)sizeof(T);                       // elems per 16 B
  static constexpr int LDK = BK + CE;  // padded LDS row: 144 B, conflict-free b128 reads
  static constexpr int CHUNKS = kVocabTile * BK / CE / 256;            // 16 B loads/thread
};

template <typename T>
__device__ __forceinline__ void load_slice(const T* __restrict__ Wt, int H, int V, int vt,
                                           int kc, u32x4 (&regs)[StageCfg<T>::CHUNKS]) {
  using C = StageCfg<T>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < C::CHUNKS; ++q) {
    const int c = tid + 256 * q;
    const int row = c / (C::BK / C::CE);
    const int col = (c % (C::BK / C::CE)) * C::CE;
    const int n = vt + row, k = kc + col;
    if (n < V && k < H)
      regs[q] = *reinterpret_cast<const u32x4*>(Wt + (size_t)n * H + k);
    else
      regs[q] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <typename T>
__device__ __forceinline__ void store_slice(T* ws, const u32x4 (&regs)[StageCfg<T>::CHUNKS]) {
  using C = StageCfg<T>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < C::CHUNKS; ++q) {
    const int c = tid + 256 * q;
    const int row = c / (C::BK / C::CE);
    const int col = (c % (C::BK / C::CE)) * C::CE;
    *reinterpret_cast<u32x4*>(ws + row * C::LDK + col) = regs[q];
  }
}

__device__ __forceinline__ float sel4(const f32x16 (&acc)[4], int blk, int r) {
  float v = acc[0][r];
  v = blk == 1 ? acc[1][r] : v;
  v = blk == 2 ? acc[2][r] : v;
  v = blk == 3 ? acc[3][r] : v;
  return v;
}

}  // namespace

template <typename T, int KS, int MODE>
__global__ __launch_bounds__(256, 1) void joint_tile_kernel(JointArgs a) {
  using C = StageCfg<T>;
  constexpr int KC_MAX = (KS * 16 + C::BK - 1) / C::BK;
  __shared__ __align__(16) T Ws[2][kVocabTile * C::LDK];
  __shared__ float cap_blank[kTileCells];
  __shared__ float cap_label[kTileCells];
  __shared__ float row_c[kTileCells];  // kGrad: (lse - ln occ) * log2(e)
  __shared__ float row_b[kTileCells];  // kGrad: gc * gB
  __shared__ float row_e[kTileCells];  // kGrad: gc * gE

  const Dims d = a.d;
  const int b = blockIdx.y;
  const int tile = blockIdx.x;
  const int t0 = a.ct0 + (tile / a.n_tu) * kTileT;
  const int u0 = a.cu0 + (tile % a.n_tu) * kTileU;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  if (t0 >= Tl || u0 > Ul) return;  // whole tile outside the lattice (uniform)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kh = lane >> 5, lc = lane & 31;
  const int H = d.H, V = d.V;
  const int nks = H / 16;
  const T* __restrict__ enc = static_cast<const T*>(a.enc);
  const T* __restrict__ pred = static_cast<const T*>(a.pred);
  const T* __restrict__ Wt = static_cast<const T*>(a.Wt);
  const T* __restrict__ bias = static_cast<const T*>(a.bias);

  // ---- prologue: start the first W^T slice, build h in registers
  u32x4 regs[C::CHUNKS];
  load_slice<T>(Wt, H, V, 0, 0, regs);

  Frag8<T> hA[KS];
  {
    const int tt = lc >> 3, uu = lc & 7;
    const int t = t0 + 4 * w + tt, u = u0 + uu;
    const bool valid = (t < Tl) && (u <= Ul);
    const T* er = enc + ((size_t)b * d.T + (valid ? t : 0)) * H + 8 * kh;
    const T* pr = pred + ((size_t)b * d.U1 + (valid ? u : 0)) * H + 8 * kh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks < nks && valid) {
        Frag8<T> e = load_frag(er + ks * 16), p = load_frag(pr + ks * 16);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fast_tanh(e.get(i) + p.get(i));
        pack_frag(hA[ks], x);
      } else {
        zero_frag(hA[ks]);
      }
    }
  }
  store_slice<T>(Ws[0], regs);

  // labels of this lane's accumulator rows: u = u0 + 4*kh + j
  int lab[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = u0 + 4 * kh + j;
    lab[j] = (u < Ul) ? a.labels[(size_t)b * d.U + u] : -1;
  }

  float gc = 1.0f;
  float cst[16];  // kGrad: per-row exponent offsets
  if constexpr (MODE == kGrad) {
    if (tid < kTileCells) {
      const int rw = tid >> 5, rr = tid & 31;
      const int t = t0 + 4 * rw + (rr >> 3), u = u0 + (rr & 7);
      float c = kInf, gb = 0.f, ge = 0.f;
      if (t < Tl && u <= Ul) {
        const double g = a.gcost ? (double)a.gcost[b] : 1.0;
        double gB, gE;
        cell_posteriors(d, a.alpha, a.beta, a.LB, a.LE, a.logP[b], b, t, u, Tl, Ul, gB, gE);
        const double occ = gB + gE;
        const double lse = (double)a.lse[skew_idx(d, b, t, u)];
        c = occ > 0.0 ? (float)((lse - log(occ)) * 1.4426950408889634) : kInf;
        gb = (float)(g * gB);
        ge = (float)(g * gE);
      }
      row_c[tid] = c;
      row_b[tid] = gb;
      row_e[tid] = ge;
    }
    gc = a.gcost ? a.gcost[b] : 1.0f;
  }
  __syncthreads();
  if constexpr (MODE == kGrad) {
#pragma unroll
    for (int r = 0; r < 16; ++r) cst[r] = row_c[w * 32 + acc_row(r, kh)];
  }

  float mrun[16], srun[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mrun[r] = -kInf;
    srun[r] = 0.f;
  }

  const int nvt = (V + kVocabTile - 1) / kVocabTile;
  const int nkc = (H + C::BK - 1) / C::BK;
  const int nstage = nvt * nkc;
  int s = 0;
  for (int vti = 0; vti < nvt; ++vti) {
    const int vt = vti * kVocabTile;
    f32x16 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;

#pragma unroll
    for (int kc = 0; kc < KC_MAX; ++kc) {
      if (kc < nkc) {
        const int cur = s & 1;
        const bool has_next = (s + 1) < nstage;
        if (has_next) {
          const int ns = s + 1;
          load_slice<T>(Wt, H, V, (ns / nkc) * kVocabTile, (ns % nkc) * C::BK, regs);
        }
        const T* ws = Ws[cur];
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
          const int ks = kc * (C::BK / 16) + kk;
          if (ks < KS && ks < nks) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
              Frag8<T> bf = load_frag(ws + (blk * 32 + lc) * C::LDK + kk * 16 + 8 * kh);
              mma_step(acc[blk], hA[ks < KS ? ks : 0], bf);
            }
          }
        }
        if (has_next) store_slice<T>(Ws[cur ^ 1], regs);
        __syncthreads();
        ++s;
      }
    }

    // ---- epilogue for vocabulary columns vt .. vt+127
    float bcol[4];
    bool cvalid[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int col = vt + blk * 32 + lc;
      cvalid[blk] = col < V;
      bcol[blk] = cvalid[blk] ? ElemTraits<T>::to_f32(bias[col]) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[blk][r] += bcol[blk];
    }

    if constexpr (MODE == kLse || MODE == kStoreZ) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x[4];
        float mx = -kInf;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          x[blk] = cvalid[blk] ? acc[blk][r] * kLog2e : -kInf;
          mx = fmaxf(mx, x[blk]);
        }
        const float mn = fmaxf(mrun[r], mx);
        if (mn > -kInf) {
          float sum = srun[r] * exp2_fast(mrun[r] - mn);
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) sum += exp2_fast(x[blk] - mn);
          srun[r] = sum;
          mrun[r] = mn;
        }
      }
      // blank logit
      if (a.d.blank >= vt && a.d.blank < vt + kVocabTile) {
        const int bb = a.d.blank - vt;
        if (lc == (bb & 31)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) cap_blank[w * 32 + acc_row(r, kh)] = sel4(acc, bb >> 5, r);
        }
      }
      // label logits
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dl = lab[j] - vt;
        if (dl >= 0 && dl < kVocabTile && (dl & 31) == lc) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + j;
            cap_label[w * 32 + acc_row(r, kh)] = sel4(acc, dl >> 5, r);
          }
        }
      }
      if constexpr (MODE == kStoreZ) {
        T* zout = static_cast<T*>(a.zout);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + 4 * w + (r >> 2), u = u0 + 4 * kh + (r & 3);
          if (t < Tl && u <= Ul) {
            T* zrow = zout + (((size_t)b * d.Tpad + t) * d.U1pad + u) * V;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk)
              if (cvalid[blk]) zrow[vt + blk * 32 + lc] = ElemTraits<T>::from_f32(acc[blk][r]);
          }
        }
      }
    } else {  // kGrad
      T* gout = static_cast<T*>(a.gout);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rowi = w * 32 + acc_row(r, kh);
        const int t = t0 + 4 * w + (r >> 2), u = u0 + 4 * kh + (r & 3);
        const bool rvalid = (t < Tl) && (u <= Ul);
        const int yl = lab[r & 3];
        T* grow = gout + (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * V;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const int col = vt + blk * 32 + lc;
          if (cvalid[blk]) {
            float g = 0.f;
            if (rvalid) {
              g = gc * exp2_fast(acc[blk][r] * kLog2e - cst[r]);
              if (col == d.blank) g -= row_b[rowi];
              if (col == yl) g -= row_e[rowi];
            }
            grow[col] = ElemTraits<T>::from_f32(g);
          }
        }
      }
    }
  }

  if constexpr (MODE == kLse || MODE == kStoreZ) {
    // combine the per-lane (max, sum) of the 32 lanes that share each row
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float mo = __shfl_xor(mrun[r], off);
        const float so = __shfl_xor(srun[r], off);
        const float mn = fmaxf(mrun[r], mo);
        if (mn > -kInf) {
          srun[r] = srun[r] * exp2_fast(mrun[r] - mn) + so * exp2_fast(mo - mn);
          mrun[r] = mn;
        }
      }
    }
    __syncthreads();  // captures visible
    if (lc < 16) {
      const int r = lc;
      const int rowi = w * 32 + acc_row(r, kh);
      const int t = t0 + 4 * w + (r >> 2), u = u0 + 4 * kh + (r & 3);
      // select this lane's row value without dynamic register indexing
      float m = mrun[0], sm = srun[0];
#pragma unroll
      for (int q = 1; q < 16; ++q) {
        m = (r == q) ? mrun[q] : m;
        sm = (r == q) ? srun[q] : sm;
      }
      if (t < Tl && u <= Ul) {
        const float lse = (m + __builtin_amdgcn_logf(sm)) * kLn2;
        const size_t ix = skew_idx(d, b, t, u);
        a.lse[ix] = lse;
        a.LB[ix] = cap_blank[rowi] - lse;
        a.LE[ix] = (u < Ul) ? cap_label[rowi] - lse : 0.f;
      }
    }
  }
}

// ------------------------------------------------------------------ dispatch

template <typename T, int MODE>
static hipError_t launch_mode(const JointArgs& a, int n_tiles, hipStream_t st) {
  const int nks = a.d.H / 16;
  dim3 grid(n_tiles, a.d.B), block(256);
  if constexpr (std::is_same<T, float>::value) {
    if (nks <= 4) hipLaunchKernelGGL((joint_tile_kernel<T, 4, MODE>), grid, block, 0, st, a);
    else if (nks <= 8) hipLaunchKernelGGL((joint_tile_kernel<T, 8, MODE>), grid, block, 0, st, a);
    else if (nks <= 16) hipLaunchKernelGGL((joint_tile_kernel<T, 16, MODE>), grid, block, 0, st, a);
    else return hipErrorInvalidValue;
  } else {
    if (nks <= 8) hipLaunchKernelGGL((joint_tile_kernel<T, 8, MODE>), grid, block, 0, st, a);
    else if (nks <= 16) hipLaunchKernelGGL((joint_tile_kernel<T, 16, MODE>), grid, block, 0, st, a);
    else if (nks <= 32) hipLaunchKernelGGL((joint_tile_kernel<T, 32, MODE>), grid, block, 0, st, a);
    else if (nks <= 40) hipLaunchKernelGGL((joint_tile_kernel<T, 40, MODE>), grid, block, 0, st, a);
    else if (nks <= 48) hipLaunchKernelGGL((joint_tile_kernel<T, 48, MODE>), grid, block, 0, st, a);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_joint_tile(const JointArgs& a, int mode, bool bf16, int n_tiles,
                             hipStream_t st) {
  if (n_tiles <= 0 || a.d.B <= 0) return hipSuccess;
  if (bf16) {
    if (mode == kLse) return launch_mode<uint16_t, kLse>(a, n_tiles, st);
    if (mode == kStoreZ) return launch_mode<uint16_t, kStoreZ>(a, n_tiles, st);
    return launch_mode<uint16_t, kGrad>(a, n_tiles, st);
  }
  if (mode == kLse) return launch_mode<float, kLse>(a, n_tiles, st);
  if (mode == kStoreZ) return launch_mode<float, kStoreZ>(a, n_tiles, st);
  return launch_mode<float, kGrad>(a, n_tiles, st);
}

}  // namespace rnntj
