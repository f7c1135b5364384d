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

// ------------------------------------------------------------ dh GEMM
//
// d_enc / d_pred contributions of the 128 cells of one active 16 x 8 tile and
// 256 hidden columns:
//   dh[cell, n] = sum_v dz[cell, v] W_out[n, v]                    (MFMA)
//   dpre = (1 - h^2) dh,  d_enc[t] += sum_u dpre,  d_pred[u] += sum_t dpre
// The kernel is persistent over (tile, hidden block) items.  dz rows and W_out
// rows stream through LDS in K-slices of KB vocabulary entries (128-byte rows,
// three slices resident, direct global -> LDS copies); the slice stream runs
// on across items, so the next item's first slices load while this item's
// epilogue runs.  4 waves (2 x 2), each 64 cells x 128 hidden columns = 2 x 4
// blocks of 32 x 32.  Tile row r is cell (t0 + r/8, u0 + r%8).
template <typename T>
struct DhCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int CE = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int KB = 8 * CE;               // vocabulary entries per slice (128-byte rows)
  static constexpr int KSTEPS = KB / 16;          // 16-wide k-steps per slice: bf16 4, fp32 2
  static constexpr int NB = 256;                  // hidden columns per item
  static constexpr int ROWS = kTileCells + NB;    // slice rows: 128 dz rows, then 256 W_out rows
  static constexpr int SLICE = ROWS * 128;        // 48 KB
  static constexpr int NST = 3;                   // slices resident
  static constexpr int CPW = SLICE / 1024 / 4;    // 1 KB copies per wave per slice (12)
};

// slot of 16-byte chunk c (0..7) of 128-byte row r: 16-byte fragment reads of
// 16 consecutive rows at one chunk hit 16 distinct bank groups
__device__ __forceinline__ int slot128(int r, int c) { return c ^ ((r >> 1) & 7); }

template <typename T>
__global__ __launch_bounds__(256, 1) void dh_kernel(DhArgs a) {
  using C = DhCfg<T>;
  __shared__ __align__(16) char lds[C::NST * C::SLICE];
  const Dims d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, lc = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  const int H = d.H, V = d.V;
  const T* __restrict__ G = static_cast<const T*>(a.g);
  const T* __restrict__ W = static_cast<const T*>(a.W);
  const int nnb = (H + C::NB - 1) / C::NB;
  const int n_items = ld_const(a.tile_count) * nnb;
  const int nk = (V + C::KB - 1) / C::KB;
  const int bid = blockIdx.x, gsz = gridDim.x;
  const int my_items = bid < n_items ? (n_items - 1 - bid) / gsz + 1 : 0;
  const int total = my_items * nk;  // slices in this workgroup's stream
  if (total == 0) return;
  const uint32_t lbase = lds_addr(lds);
  const bool use_ep = (ld_const(a.hdr + 1) & kFlagEpBad) == 0;

  // An item is carried as its packed tile word and hidden block (two
  // uniform words); decode() expands it where needed (scalar loads).
  struct Item {
    int b, t0, u0, n0, Tl, Ul;
  };
  struct ItemRef {
    int tile, nb;
  };
  auto item_ref = [&](int i) {  // i-th item of this workgroup
    const int item = bid + i * gsz;
    ItemRef r;
    r.tile = ld_const(a.tiles + item / nnb);
    r.nb = item % nnb;
    return r;
  };
  auto decode = [&](ItemRef r) {
    Item it;
    int tt, tu;
    tile_unpack(r.tile, it.b, tt, tu);
    it.t0 = a.ct0 + tt * kTileT;
    it.u0 = a.cu0 + tu * kTileU;
    it.n0 = r.nb * C::NB;
    it.Tl = ld_const(a.Teff + it.b);
    it.Ul = ld_const(a.Ueff + it.b);
    return it;
  };

  // Direct copies of one slice: copy q of wave w fills slice rows
  // 8 (CPW w + q) .. +7; lane l takes row 8 (CPW w + q) + l/8 and LDS slot
  // l%8, holding 16-byte chunk slot128(row, l%8).  Rows below 128 are dz
  // rows of the tile (cells outside the lattice read the tile's first cell,
  // which is always inside; their results are never used), the rest W_out
  // rows n0 + r - 128 (clamped to H - 1).  The row + chunk source of every
  // copy is set once per item; a slice only adds its vocabulary offset.
  // Chunks past V (last slice, V not a multiple of KB) are clamped to the
  // row's last chunk; their fragments are zeroed before the MFMAs.
  // dz rows: offsets (elements) from the item's first cell row; W_out rows:
  // offsets from W_out.  Both fit 32 bits (a tile spans 16 frames of one
  // chunk; W_out is at most 768 rows).
  const T* gbase = G;
  uint32_t coff[C::CPW];
  auto set_sources = [&](ItemRef ref) {
    const Item it = decode(ref);
    gbase = G + (((size_t)it.b * a.CT + (it.t0 - a.ct0)) * a.CU + (it.u0 - a.cu0)) * V;
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) {
      const int ins = C::CPW * w + q;
      const int r = 8 * ins + (lane >> 3);
      const int c = slot128(r, lane & 7);
      if (ins < kTileCells / 8) {  // uniform: the first 16 copies hold dz rows
        int dt = r >> 3, du = r & 7;
        const bool ok = it.t0 + dt < it.Tl && it.u0 + du <= it.Ul;
        dt = ok ? dt : 0;
        du = ok ? du : 0;
        coff[q] = (uint32_t)((dt * a.CU + du) * V + c * C::CE);
      } else {
        const int n = min(it.n0 + r - kTileCells, H - 1);
        coff[q] = (uint32_t)(n * V + c * C::CE);
      }
    }
  };
  auto issue = [&](int s, int buf) {
    const int k0 = s * C::KB;
    const uint32_t st = lbase + buf * C::SLICE + C::CPW * w * 1024;
    const bool tail = k0 + C::KB > V;
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) {
      const T* base = (C::CPW * w + q < kTileCells / 8) ? gbase : W;
      uint32_t off = coff[q] + k0;
      if (tail) {  // chunks past V re-read the row's last chunk
        const int r = 8 * (C::CPW * w + q) + (lane >> 3);
        const int c = slot128(r, lane & 7);
        if (k0 + c * C::CE + C::CE > V) off = coff[q] - c * C::CE + (V - C::CE);
      }
      dma16(base + off, st + q * 1024);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Frag8<T> fa[2][2], fb[2][4];
  // fragments of k-step kk of stream slice g (buffer g % NST)
  auto rd = [&](int g, int kk, int fbuf) {
    const char* sl = lds + (g % C::NST) * C::SLICE;
    const int kbase = (g % nk) * C::KB + 16 * kk + 8 * kh;  // this lane's first k
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * wm + 32 * i + lc;
      const char* row = sl + r * 128;
      if constexpr (C::kBf16) {
        fa[fbuf][i].v = *reinterpret_cast<const u32x4*>(row + (slot128(r, 2 * kk + kh) << 4));
      } else {
        fa[fbuf][i].lo = *reinterpret_cast<const f32x4*>(row + (slot128(r, 4 * kk + 2 * kh) << 4));
        fa[fbuf][i].hi = *reinterpret_cast<const f32x4*>(row + (slot128(r, 4 * kk + 2 * kh + 1) << 4));
      }
      if (kbase >= V) zero_frag(fa[fbuf][i]);  // vocabulary tail
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = kTileCells + 128 * wn + 32 * j + lc;
      const char* row = sl + r * 128;
      if constexpr (C::kBf16) {
        fb[fbuf][j].v = *reinterpret_cast<const u32x4*>(row + (slot128(r, 2 * kk + kh) << 4));
      } else {
        fb[fbuf][j].lo = *reinterpret_cast<const f32x4*>(row + (slot128(r, 4 * kk + 2 * kh) << 4));
        fb[fbuf][j].hi = *reinterpret_cast<const f32x4*>(row + (slot128(r, 4 * kk + 2 * kh + 1) << 4));
      }
    }
  };
  auto mm = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_step(acc[i][j], fa[fbuf][i], fb[fbuf][j]);
  };

  // epilogue inputs, loaded during an item's last slice: for this lane's
  // columns j and frames (i, q4) / label positions q, e^{2 enc}, e^{2 pred}
  // (or enc, pred when those exponentials could overflow)
  float ex[2][4][4], px[4][4];  // [i][q4][j], [q][j]
  auto load_ep_from = [&](const Item& it, auto src_e, auto src_p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = min(it.n0 + 128 * wn + 32 * j + lc, H - 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int t = min(it.t0 + 8 * wm + 4 * i + q4, d.T - 1);
          ex[i][q4][j] = src_e(((size_t)it.b * d.T + t) * H + n);
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = min(it.u0 + 4 * kh + q, d.U1 - 1);
        px[q][j] = src_p(((size_t)it.b * d.U1 + u) * H + n);
      }
    }
  };
  auto load_ep = [&](const Item& it) {
    if (use_ep) {
      load_ep_from(it, [&](size_t i) { return a.Eexp[i]; }, [&](size_t i) { return a.Pexp[i]; });
    } else {
      const T* enc = static_cast<const T*>(a.enc);
      const T* pred = static_cast<const T*>(a.pred);
      load_ep_from(it, [&](size_t i) { return ElemTraits<T>::to_f32(enc[i]); },
                   [&](size_t i) { return ElemTraits<T>::to_f32(pred[i]); });
    }
  };
  // dpre = (1 - h^2) dh, reduced over label positions (d_enc) and frames
  // (d_pred) in registers, then added with float32 atomics
  auto epilogue = [&](const Item& it) {
    float psum[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) psum[j][q] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = it.n0 + 128 * wn + 32 * j + lc;
      const bool nvalid = n < H;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int t = it.t0 + 8 * wm + 4 * i + q4;
          const bool tv = nvalid && t < it.Tl;
          float esum = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = it.u0 + 4 * kh + q;
            const float hval = use_ep
                                   ? 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + ex[i][q4][j] * px[q][j])
                                   : fast_tanh(ex[i][q4][j] + px[q][j]);
            const float v = (tv && u <= it.Ul) ? (1.0f - hval * hval) * acc[i][j][4 * q4 + q] : 0.f;
            esum += v;
            psum[j][q] += v;
            acc[i][j][4 * q4 + q] = 0.f;
          }
          // the other 4 label positions of this frame live in lane l ^ 32
          esum += __shfl_xor(esum, 32);
          if (kh == 0 && tv) atomicAdd(&a.d_enc[((size_t)it.b * d.T + t) * H + n], esum);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = it.n0 + 128 * wn + 32 * j + lc;
      if (n < H) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = it.u0 + 4 * kh + q;
          if (u <= it.Ul) atomicAdd(&a.d_pred[((size_t)it.b * d.U1 + u) * H + n], psum[j][q]);
        }
      }
    }
  };

  // ---- the slice stream: slice g is slice g % nk of item g / nk.  Two
  // cursors walk it: the copy cursor (slices are issued two ahead) and the
  // compute cursor; each holds its item and loads the following one early
  // (scalar loads, waited for only at first use).
  ItemRef cur = item_ref(0);
  ItemRef cur_next = my_items > 1 ? item_ref(1) : cur;
  ItemRef iss_next = cur_next;
  int iss_i = 0, iss_s = 0, iss_g = 0;
  set_sources(cur);
  auto issue_next = [&]() {  // copy slice iss_g into buffer iss_g % NST
    issue(iss_s, iss_g % C::NST);
    ++iss_g;
    if (++iss_s == nk) {
      iss_s = 0;
      if (++iss_i < my_items) {
        set_sources(iss_next);
        if (iss_i + 1 < my_items) iss_next = item_ref(iss_i + 1);
      }
    }
  };
  issue_next();
  if (total > 1) {
    issue_next();
    wait_vm<C::CPW>();  // slice 0 landed, slice 1 may be in flight
  } else {
    wait_vm<0>();
  }
  __builtin_amdgcn_s_barrier();
  rd(0, 0, 0);
  // MFMAs of stream slice g, with the fragment reads one k-step ahead
  auto slice = [&](int g) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int fcur = kk & 1;
      if (kk + 1 < C::KSTEPS) {
        rd(g, kk + 1, fcur ^ 1);
      } else if (g + 1 < total) {
        // slice g+1 has landed (nothing newer is in flight) and every wave
        // is past slice g-1: refill that buffer with slice g+2
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (iss_g < total) issue_next();
        rd(g + 1, 0, fcur ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      mm(fcur);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int g = 0; g < total; ++g) {
    const int s = g % nk;
    // during an item's last slice its epilogue inputs load
    if (s == nk - 1) load_ep(decode(cur));
    slice(g);
    if (s == nk - 1) {
      epilogue(decode(cur));
      const int li = g / nk;
      cur = cur_next;
      if (li + 2 < my_items) cur_next = item_ref(li + 2);
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

hipError_t launch_dh(const DhArgs& a, bool bf16, int max_tiles, hipStream_t st) {
  const int nnb = (a.d.H + DhCfg<float>::NB - 1) / DhCfg<float>::NB;
  const long long items = (long long)max_tiles * nnb;
  if (items <= 0) return hipSuccess;
  const int ncu = device_cu_count();
  dim3 grid((unsigned)(items < ncu ? items : ncu)), block(256);
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
