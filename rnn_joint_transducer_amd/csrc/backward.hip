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
//   grad_inplace_kernel: untiled mode, the stored logits -> dz in place, one
//                        active tile per workgroup (constants of its rows
//                        from the float64 posteriors, then a 16-byte stream
//                        per lane).
//   dh_kernel          : MFMA GEMM dz[cells, V] x W_out^T -> [cells, H] per
//                        active 16x8 tile and 256 hidden columns, with the
//                        (1 - h^2) epilogue and the two lattice reductions
//                        done in registers before float32 atomics.
//   dw_kernel          : MFMA GEMM h^T[H, cells] x dz[cells, V] split over
//                        runs of the tile list (split-K); h and dz cell rows
//                        are read as MFMA operands with transposing LDS
//                        loads; the hidden-block-0 workgroups also sum dz
//                        columns into db_out (float64).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr float kInf = __builtin_inff();
// bits of the fourth word of a cell's logit-gradient constants
constexpr uint32_t kCellLabel = 0x3FFFFFFFu, kCellNeg = 0x40000000u, kCellOut = 0x80000000u;

// ------------------------------------------------------------ untiled dz

// Constants of the logit gradient of lattice row (t, u) of utterance b.
// With dz[v] = gc (occ p[v] - gB [v=blank] - gE [v=label]) and p = softmax(z):
//   x = (lse - ln(occ |gc|)) log2(e), so that gc occ p[v] = sgn(gc) 2^(z log2(e) - x)
//       (+inf when occ gc = 0: the term vanishes),
//   y = gc gB,  z = gc gE,
//   w (bits) = label + 1 in bits 0..29 (0: no label at this u), bit 30 set when
//       gc < 0, bit 31 set for a cell outside the lattice (dz = 0).
__device__ float4 cell_consts(const JointArgs& a, int b, int t, int u) {
  const Dims d = a.d;
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  float4 o = make_float4(kInf, 0.f, 0.f, __uint_as_float(kCellOut));
  if (t < Tl && u <= Ul) {
    const double g = a.gcost ? (double)a.gcost[b] : 1.0;
    double gB, gE;
    cell_posteriors(d, a.alpha, a.beta, a.LB, a.LE, a.logP[b], b, t, u, Tl, Ul, gB, gE, a.hdr[3]);
    const double m = (gB + gE) * fabs(g);
    const double lse = (double)a.lse[skew_idx(d, b, t, u)];
    o.x = m > 0.0 ? (float)((lse - log(m)) * 1.4426950408889634) : kInf;
    o.y = (float)(g * gB);
    o.z = (float)(g * gE);
    const uint32_t lab = u < Ul ? (uint32_t)a.labels[(size_t)b * d.U + u] + 1u : 0u;
    o.w = __uint_as_float(lab | (g < 0.0 ? kCellNeg : 0u));
  }
  return o;
}

// dz of logit v of a cell from the stored logit z and the cell's constants;
// v1 = v + 1 (compared with the stored label + 1)
__device__ __forceinline__ float dz_from_z(float z, int v, int v1, const float4& c, int blank) {
  const uint32_t w = __float_as_uint(c.w);
  const float e = exp2_fast(z * kLog2e - c.x);
  float g = __uint_as_float(__float_as_uint(e) ^ ((w << 1) & 0x80000000u));
  g -= (v == blank) ? c.y : 0.f;
  g -= ((int)(w & kCellLabel) == v1) ? c.z : 0.f;
  return (int)w < 0 ? 0.f : g;
}

// Untiled backward: the stored logits of active tile blockIdx.x become its
// logit gradients (in place, same type).  Wave w walks rows 32w .. 32w+31 of
// the tile (4 frames x 8 label positions, contiguous per frame); each lane
// takes 16-byte chunks of a row, eight loads in flight.  Rows outside the
// lattice are written as zeros.  A forward's logits serve one backward: the
// backward marks the state (kFlagConsumed, set by its last kernel), and a
// later backward from the same state reports kErrConsumed.
template <typename T>
__global__ __launch_bounds__(256) void grad_inplace_kernel(JointArgs a, T* __restrict__ z) {
  constexpr int CE = 16 / (int)sizeof(T);
  __shared__ float4 cs[kTileCells];
  const int tix = blockIdx.x, tid = threadIdx.x;
  if (ld_const(a.hdr + kHdrRefuse)) return;  // the state does not belong to this backward
  if (tix == 0 && tid == 0 && (a.hdr[1] & kFlagConsumed)) atomicOr(&a.hdr[0], kErrConsumed);
  if (tix >= a.tile_count[0]) return;
  int b, tt, tu;
  tile_unpack(a.tiles[tix], b, tt, tu);
  const Dims d = a.d;
  const int t0 = tt * kTileT, u0 = tu * kTileU;
  if (tid < kTileCells) cs[tid] = cell_consts(a, b, t0 + (tid >> 3), u0 + (tid & 7));
  __syncthreads();
  const int w = tid >> 6, lane = tid & 63, V = d.V;
  const int nch = (V + 64 * CE - 1) / (64 * CE);  // chunk columns per row per lane
  const int n = 32 * nch;                         // (row, chunk) pairs of this wave
  T* const zt = z + (((size_t)b * d.Tpad + t0) * d.U1pad + u0) * V;
  // bf16: the stored values are z - M, M per row and vocabulary step
  constexpr bool kShift = sizeof(T) == 2;
  const int nvs = kShift ? (V + a.zstep - 1) / a.zstep : 0;
  const float* zm = kShift ? a.zmax + (((size_t)b * d.Tpad + t0) * d.U1pad + u0) * nvs : nullptr;
  for (int i0 = 0; i0 < n; i0 += 8) {
    u32x4 x[8];
    float zoff[8];
    T* ptr[8];
    bool ok[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = i0 + k, rr = i / nch, v0 = ((i % nch) * 64 + lane) * CE;
      const int r = 32 * w + rr;
      ok[k] = i < n && v0 < V;
      const size_t row = (size_t)(r >> 3) * d.U1pad + (r & 7);
      ptr[k] = zt + row * V + v0;
      zoff[k] = 0.f;
      if (ok[k]) {
        x[k] = *reinterpret_cast<const u32x4*>(ptr[k]);
        if constexpr (kShift) zoff[k] = zm[row * nvs + v0 / a.zstep];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (!ok[k]) continue;
      const int i = i0 + k, v0 = ((i % nch) * 64 + lane) * CE;
      const float4 c = cs[32 * w + i / nch];
      float g[CE];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < CE; ++e) {
          const uint32_t bits = (x[k][e >> 1] >> (16 * (e & 1))) << 16;
          g[e] = dz_from_z(__uint_as_float(bits & 0xffff0000u) + zoff[k], v0 + e, v0 + e + 1, c,
                           d.blank);
        }
        u32x4 y;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          y[q] = pack_bf16x2(g[2 * q], g[2 * q + 1]);
        *reinterpret_cast<u32x4*>(ptr[k]) = y;
      } else {
#pragma unroll
        for (int e = 0; e < CE; ++e)
          g[e] = dz_from_z(__uint_as_float(x[k][e]), v0 + e, v0 + e + 1, c, d.blank);
        *reinterpret_cast<u32x4*>(ptr[k]) =
            u32x4{__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]), __float_as_uint(g[3])};
      }
    }
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
  // bf16: 64-byte slice rows and two workgroups per CU (two waves per SIMD);
  // fp32: 128-byte rows, one workgroup per CU
  static constexpr int RB = kBf16 ? 64 : 128;     // bytes per slice row
  static constexpr int CPR = RB / 16;             // chunks per row
  static constexpr int RPC = 1024 / RB;           // rows per 1 KB copy
  static constexpr int KB = RB / (int)sizeof(T);  // vocabulary entries per slice (32)
  static constexpr int KSTEPS = KB / 16;          // 16-wide k-steps per slice (2)
  static constexpr int NB = 256;                  // hidden columns per item
  static constexpr int ROWS = kTileCells + NB;    // slice rows: 128 dz rows, then 256 W_out rows
  static constexpr int SLICE = ROWS * RB;         // bf16 24 KB, fp32 48 KB
  static constexpr int NST = 3;                   // slices resident
  static constexpr int CPW = SLICE / 1024 / 4;    // 1 KB copies per wave per slice (6 / 12)
  static constexpr int OCC = kBf16 ? 2 : 1;       // workgroups per CU
  static constexpr int NMFMA = kBf16 ? 8 : 64;    // MFMA instructions per k-step and wave
  static constexpr int NVALU = kBf16 ? 2 : 1;     // other VALU per MFMA
  static_assert(KSTEPS % 2 == 0, "slice shape");
};

// slot of 16-byte chunk c of row r of a slice with RB-byte rows: the 16-byte
// fragment reads of 16 consecutive rows at one chunk hit distinct bank groups
template <int RB>
__device__ __forceinline__ int slot_of(int r, int c) {
  return c ^ ((r / (256 / RB)) & (RB / 16 - 1));
}

// Registers that a compiler-visible load filled are "used" here, right after
// an explicit vmcnt(0) and before the next direct copies are issued, so that
// the wait the compiler places before their first use falls where nothing
// else is in flight.
__device__ __forceinline__ void touch(float x) { asm volatile("" ::"v"(x)); }

// VTAIL: the vocabulary part is not a multiple of the slice width, so the
// fragments past its end are zeroed (a separate instantiation: otherwise the
// test would cost a select per fragment register at every k-step).
template <typename T, bool VTAIL>
__global__ __launch_bounds__(256, DhCfg<T>::OCC) void dh_kernel(DhArgs a) {
  using C = DhCfg<T>;
  __shared__ __align__(16) char lds[C::NST * C::SLICE];
  __shared__ __align__(16) float xch[2 * 64 * 16];  // d_pred partial sums of wave row 1
  const Dims d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, lc = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  const int H = d.H, V = d.V;
  // vocabulary part [V0, V0 + VW) of this launch: dz rows have stride LG, W_out
  // rows stride V
  const int V0 = a.v0, VW = a.vw, LG = a.ldg;
  const T* __restrict__ G = static_cast<const T*>(a.g);
  const T* __restrict__ W = static_cast<const T*>(a.W);
  const int nnb = (H + C::NB - 1) / C::NB;
  if (ld_const(a.hdr + kHdrRefuse)) return;  // the state does not belong to this backward
  const int n_tiles = ld_const(a.tile_count);
  // an item is (tile, hidden block, vocabulary part): with few tiles the
  // vocabulary is split so that the workgroups get equal shares (dh is
  // linear in dz, so the parts' d_enc / d_pred contributions simply add)
  const int ks = a.ksplit;
  const int n_items = n_tiles * nnb * ks;
  const int nk = (VW + C::KB - 1) / C::KB;  // slices of the vocabulary part
  const int nks = nk / ks;                  // slices of one item (ks divides nk)
  // Workgroups are dealt to the 8 XCDs round-robin (blockIdx % 8).  XCD x
  // takes the x-th of 8 contiguous runs of items, its workgroups striding
  // through the run together, so that the hidden blocks of one tile (which
  // read the same dz rows) and the tiles sharing W_out rows run at the same
  // time on one L2.
  const int wpx = gridDim.x >> 3, lx = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  const int per = (n_items + 7) >> 3;
  const int xbase = xcd * per;
  const int xcount = min(per, n_items - xbase);
  const int my_items = xcount > lx ? (xcount - 1 - lx) / wpx + 1 : 0;
  const int total = my_items * nks;  // slices in this workgroup's stream
  if (total == 0) return;
  const uint32_t lbase = lds_addr(lds);
  const bool use_ep = (ld_const(a.hdr + 1) & kFlagEpBad) == 0;

  // An item is carried as its packed tile word and hidden block (two
  // uniform words); decode() expands it where needed (scalar loads).
  struct Item {
    int b, t0, u0, n0, Tl, Ul, tix;
  };
  struct ItemRef {
    int tile, nb, tix, kp;
  };
  auto item_ref = [&](int i) {  // i-th item of this workgroup
    const int item = xbase + lx + i * wpx;
    ItemRef r;
    r.kp = item % ks;  // vocabulary part, then hidden block, then tile
    const int tn = item / ks;
    r.tix = tn / nnb;
    r.nb = tn % nnb;
    r.tile = ld_const(a.tiles + r.tix);
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
    it.tix = r.tix;
    return it;
  };

  // Direct copies of one slice: copy q of wave w fills slice rows
  // RPC (CPW w + q) .. +RPC-1; lane l takes row RPC (CPW w + q) + l/CPR and LDS
  // slot l%CPR, holding 16-byte chunk slot_of(row, l%CPR).  Rows below 128 are dz
  // rows of the tile (cells outside the lattice read the tile's first cell,
  // which is always inside; their results are never used), the rest W_out
  // rows n0 + r - 128 (clamped to H - 1), read from the blocked copy.  Chunks
  // past V (last slice, V not a multiple of KB) are clamped to the row's last
  // chunk; their fragments are zeroed before the MFMAs.  Element offsets fit
  // 32 bits (a tile spans 16 frames of one chunk; W_out is at most 768 rows).
  const int lr = lane / C::CPR, lcc = lane % C::CPR;
  const T* gbase = G;
  Item src_it = {};
  int src_k0 = 0;  // first vocabulary entry of the issuing item's part
  // General form (vocabulary tails, or tiles whose byte span exceeds 32
  // bits): element offset of copy q from the copy's base, formed at issue.
  auto copy_off = [&](int q, int k0) -> uint32_t {
    const int ins = C::CPW * w + q;  // uniform
    const int r = C::RPC * ins + lr;
    const int col = min(k0 + slot_of<C::RB>(r, lcc) * C::CE, VW - C::CE);
    if (ins < kTileCells / C::RPC) {  // dz rows of the tile
      int dt = r >> 3, du = r & 7;
      const bool ok = src_it.t0 + dt < src_it.Tl && src_it.u0 + du <= src_it.Ul;
      dt = ok ? dt : 0;
      du = ok ? du : 0;
      return (uint32_t)((dt * a.CU + du) * LG + col);
    }
    // W_out rows from the blocked copy: vocabulary entry g of row n is at
    // (g / 32, n, g % 32); a slice starts on a block (V0 and k0 are
    // multiples of 32), so its RPC consecutive rows form one contiguous 1 KB
    const int n = min(src_it.n0 + r - kTileCells, H - 1);
    const int g = V0 + col;
    return (uint32_t)(((g >> 5) * H + n) * 32 + (g & 31));
  };
  // Usual form: each copy is a wave-uniform base (dz rows: the slice's first
  // entry of the tile's first row; W_out rows: the slice's block) plus a
  // per-lane byte offset that stays fixed over the item's slices, set once
  // per item, so a slice's copies cost no vector arithmetic.  A tile's dz
  // rows span fewer than 16 frame rows of the chunk, which bounds the offsets.
  const bool soff = (uint64_t)kTileT * (uint64_t)a.CU * (uint64_t)LG * sizeof(T) < (1ull << 32);
  uint32_t coff[C::CPW];
  auto lane_off = [&](int q) -> uint32_t {  // bytes from the copy's base
    const int ins = C::CPW * w + q;  // uniform
    const int r = C::RPC * ins + lr;
    const uint32_t c = (uint32_t)(slot_of<C::RB>(r, lcc) * C::CE);
    if (ins < kTileCells / C::RPC) {
      int dt = r >> 3, du = r & 7;
      const bool ok = src_it.t0 + dt < src_it.Tl && src_it.u0 + du <= src_it.Ul;
      dt = ok ? dt : 0;
      du = ok ? du : 0;
      return ((uint32_t)(dt * a.CU + du) * (uint32_t)LG + c) * (uint32_t)sizeof(T);
    }
    const int n = min(src_it.n0 + r - kTileCells, H - 1);
    return ((uint32_t)n * 32u + c) * (uint32_t)sizeof(T);
  };
  auto set_sources = [&](ItemRef ref) {
    src_it = decode(ref);
    src_k0 = ref.kp * nks * C::KB;
    gbase = G + (((size_t)src_it.b * a.CT + (src_it.t0 - a.ct0)) * a.CU + (src_it.u0 - a.cu0)) * LG;
    if (soff) {
#pragma unroll
      for (int q = 0; q < C::CPW; ++q) coff[q] = lane_off(q);
    }
  };
  auto issue = [&](int s, int buf) {
    const int k0 = src_k0 + s * C::KB;
    const uint32_t st = lbase + buf * C::SLICE + C::CPW * w * 1024;
    const bool tail = k0 + C::KB > VW;
    if (soff && !tail) {
      const T* gb = gbase + k0;
      const T* wb = W + (size_t)((V0 + k0) >> 5) * H * 32;
#pragma unroll
      for (int q = 0; q < C::CPW; ++q)
        dma16s((C::CPW * w + q < kTileCells / C::RPC) ? gb : wb, coff[q], st + q * 1024);
    } else {
#pragma unroll
      for (int q = 0; q < C::CPW; ++q) {
        const T* base = (C::CPW * w + q < kTileCells / C::RPC) ? gbase : W;
        dma16(base + copy_off(q, k0), st + q * 1024);
      }
    }
  };
  constexpr int kCopies = C::CPW;  // per wave per slice

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Frag8<T> fa[2][2], fb[2][4];
  // fragments of k-step kk of stream slice g (buffer g % NST)
  const bool has_vtail = VTAIL && VW % C::KB != 0;
  auto rd = [&](int g, int kk, int fbuf) {
    const char* sl = lds + (g % C::NST) * C::SLICE;
    const int s = g % nks;  // slice of the item (ks == 1 whenever V has a tail)
    const bool vtail = has_vtail && s == nks - 1;  // uniform
    const int kbase = s * C::KB + 16 * kk + 8 * kh;  // this lane's first k
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * wm + 32 * i + lc;
      const char* row = sl + r * C::RB;
      if constexpr (C::kBf16) {
        fa[fbuf][i].v = *reinterpret_cast<const u32x4*>(row + (slot_of<C::RB>(r, 2 * kk + kh) << 4));
      } else {
        fa[fbuf][i].lo = *reinterpret_cast<const f32x4*>(row + (slot_of<C::RB>(r, 4 * kk + 2 * kh) << 4));
        fa[fbuf][i].hi = *reinterpret_cast<const f32x4*>(row + (slot_of<C::RB>(r, 4 * kk + 2 * kh + 1) << 4));
      }
      if constexpr (VTAIL)
        if (vtail && kbase >= VW) zero_frag(fa[fbuf][i]);  // vocabulary tail
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = kTileCells + 128 * wn + 32 * j + lc;
      const char* row = sl + r * C::RB;
      if constexpr (C::kBf16) {
        fb[fbuf][j].v = *reinterpret_cast<const u32x4*>(row + (slot_of<C::RB>(r, 2 * kk + kh) << 4));
      } else {
        fb[fbuf][j].lo = *reinterpret_cast<const f32x4*>(row + (slot_of<C::RB>(r, 4 * kk + 2 * kh) << 4));
        fb[fbuf][j].hi = *reinterpret_cast<const f32x4*>(row + (slot_of<C::RB>(r, 4 * kk + 2 * kh + 1) << 4));
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
  // (d_pred) in registers, then added with float32 atomics.
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
        float es[4];
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
          es[q4] = esum + __shfl_xor(esum, 32);
          if (C::kBf16 && kh == 0 && tv) {
            if (a.enc_part)
              a.enc_part[((size_t)it.tix * kTileT + (t - it.t0)) * H + n] = es[q4];
            else
              atomicAdd(&a.d_enc[((size_t)it.b * d.T + t) * H + n], es[q4]);
          }
        }
        // fp32: both lane halves hold every frame's sum, so each half adds
        // one of two frames and one full-wave atomic covers two frames (in
        // bf16 the extra registers this holds cost more than it saves)
        if constexpr (!C::kBf16) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int t = it.t0 + 8 * wm + 4 * i + 2 * m + kh;
            if (nvalid && t < it.Tl) {
              const float v = kh ? es[2 * m + 1] : es[2 * m];
              if (a.enc_part)
                a.enc_part[((size_t)it.tix * kTileT + (t - it.t0)) * H + n] = v;
              else
                atomicAdd(&a.d_enc[((size_t)it.b * d.T + t) * H + n], v);
            }
          }
        }
      }
    }
    // the two wave rows hold the d_pred sums of the tile's two frame halves
    // for the same (u, n): row 1 hands its sums over through LDS and row 0
    // adds both to memory, half the atomics.  The second barrier keeps the
    // next item's hand-over from overwriting sums row 0 has not read yet.
    f32x4* xw = reinterpret_cast<f32x4*>(xch + (wn * 64 + lane) * 16);
    if (wm == 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) xw[j] = f32x4{psum[j][0], psum[j][1], psum[j][2], psum[j][3]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wm == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 o = xw[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) psum[j][q] += o[q];
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wm == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = it.n0 + 128 * wn + 32 * j + lc;
        if (n < H) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int u = it.u0 + 4 * kh + q;
            if (u > it.Ul) continue;
            if (a.pred_part)
              a.pred_part[((size_t)it.tix * kTileU + (u - it.u0)) * H + n] = psum[j][q];
            else
              atomicAdd(&a.d_pred[((size_t)it.b * d.U1 + u) * H + n], psum[j][q]);
          }
        }
      }
    }
  };

  // ---- the slice stream: slice g is slice g % nk of item g / nk.  Two
  // cursors walk it: the copy cursor (slices are issued three ahead) and the
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
    if (++iss_s == nks) {
      iss_s = 0;
      if (++iss_i < my_items) {
        set_sources(iss_next);
        if (iss_i + 1 < my_items) iss_next = item_ref(iss_i + 1);
      }
    }
  };
  issue_next();
  if (total > 1) issue_next();
  if (total > 2) issue_next();
  // slice 0 landed; slices 1 and 2 may be in flight
  if (total > 2) wait_vm<2 * kCopies>();
  else if (total > 1) wait_vm<kCopies>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  rd(0, 0, 0);
  // MFMAs of stream slice g, with the fragment reads one k-step ahead; `last`
  // marks an item's last slice, whose epilogue loads (issued after the copies
  // of slice g+2) are waited for and touched at its end
  auto slice = [&](int g, bool last) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int fcur = kk & 1;  // KSTEPS is even: parity of the k-step in the stream
      __builtin_amdgcn_sched_barrier(0);
      mm(fcur);
      if (kk + 1 < C::KSTEPS) {
        rd(g, kk + 1, fcur ^ 1);
        interleave_mfma<C::NMFMA, 1, C::NVALU>();
      } else if (g + 1 < total) {
        // (the MFMAs above run on while this wave waits) slice g+1 has
        // landed (g+2 may still be in flight), this wave's reads of slice g
        // are done, and after the barrier every wave's are: refill that
        // buffer with slice g+3
        if (C::OCC == 1 && last) {
          wait_vm<0>();
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
              for (int j = 0; j < 4; ++j) touch(ex[i][q4][j]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) touch(px[q][j]);
        } else if (g + 2 < total) {
          wait_vm<kCopies>();
        } else {
          wait_vm<0>();
        }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        if (iss_g < total) issue_next();
        rd(g + 1, 0, fcur ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // items outside, their slices inside: the accumulators stay in the MFMA
  // registers through the slice loop and are only read by the epilogue
  for (int li = 0; li < my_items; ++li) {
    for (int s = 0; s < nks; ++s) {
      const bool last = s == nks - 1;
      // one workgroup per CU: the epilogue inputs load during an item's last
      // slice; two per CU: they load after it (the other workgroup's MFMAs
      // cover the wait, and the registers stay free during the slices)
      if (C::OCC == 1 && last) load_ep(decode(cur));
      slice(li * nks + s, last);
    }
    if constexpr (C::OCC > 1) load_ep(decode(cur));
    epilogue(decode(cur));
    cur = cur_next;
    if (li + 2 < my_items) cur_next = item_ref(li + 2);
  }
}


// ------------------------------------------------------------ dW GEMM
//
// d_W_out[m, n] += sum over cells h[cell, m] dz[cell, n] and d_b64[n] +=
// sum over cells dz[cell, n], over the active tiles of one chunk.  Items:
// 128 hidden rows x 256 vocabulary columns x one of `kparts` runs of the tile
// list (split-K); one workgroup per item.  Workgroups are dealt to the 8 XCDs
// round-robin; consecutive items (the column blocks of one run) are placed on
// one XCD so that the h and dz rows they share come from that XCD's L2.  Cell
// rows of h and dz stream through LDS in slices of KB cells (direct copies,
// three slices resident, issued three ahead) and are read as MFMA operands
// with transposing (bf16) or scalar (fp32) LDS reads, so neither operand is
// transposed in memory.  4 waves (2 x 2), each 64 hidden rows x 128
// vocabulary columns.
template <typename T>
struct DwCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int E = sizeof(T);
  static constexpr int CE = 16 / E;                    // elements per 16-byte granule
  static constexpr int BM = 128, BN = 256;
  static constexpr int KB = 32;                        // cells per slice
  static constexpr int KSTEPS = KB / 16;               // 2
  static constexpr int SPT = kTileCells / KB;          // slices per tile
  static constexpr int ROWA = BM * E, ROWB = BN * E;   // bytes per cell row
  static constexpr int GA = ROWA / 16, GB = ROWB / 16; // granules per row
  static constexpr int SA = KB * ROWA, SB = KB * ROWB; // bf16 8 + 16 KB, fp32 16 + 32 KB
  static constexpr int CA = SA / 1024, CB = SB / 1024; // 1 KB copies per part
  static constexpr int QPW = (CA + CB) / 4;            // row copies per wave per slice (6 / 12)
  static constexpr int SLICE = SA + SB;
  static constexpr int NST = 3;
  static constexpr int NMFMA = kBf16 ? 8 : 64;         // MFMA instructions per k-step and wave
  // bf16: two workgroups per CU (72 KB of LDS each, two waves per SIMD) so
  // that one workgroup's fragment reads and copies overlap the other's MFMAs
  static constexpr int OCC = kBf16 ? 2 : 1;
  static_assert(KSTEPS % 2 == 0 && (CA + CB) % 4 == 0, "slice shape");
};

// 16-byte granule swizzle of cell row r: the transposing reads of 4
// consecutive rows and the scalar reads of rows r, r+8 hit distinct banks
__device__ __forceinline__ int swz_dw(int r) { return (4 * (r & 3)) ^ (8 * ((r >> 3) & 1)); }

template <typename T>
__global__ __launch_bounds__(256, DwCfg<T>::OCC) void dw_kernel(DwArgs a) {
  using C = DwCfg<T>;
  __shared__ __align__(16) char lds[C::NST * C::SLICE];
  const Dims d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, lc = lane & 31;
  const int wm = w >> 1, wn = w & 1;
  const int H = d.H, V = d.V;
  // vocabulary part [V0, V0 + VW): dz columns (row stride LG), d_W_out columns
  const int V0 = a.v0, VW = a.vw, LG = a.ldg;
  const int nmb = (H + C::BM - 1) / C::BM, nnb = (VW + C::BN - 1) / C::BN;
  const int nmn = nmb * nnb;
  // item of this workgroup: XCD x = blockIdx % 8 takes items x * per .. +per-1
  const int per = gridDim.x >> 3;
  const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int kp = item / nmn, nb = (item % nmn) / nmb, mb = item % nmb;
  if (kp >= a.kparts) return;
  if (ld_const(a.hdr + kHdrRefuse)) return;  // the state does not belong to this backward
  const int count = ld_const(a.tile_count);
  const int tb = (int)((long long)count * kp / a.kparts);
  const int te = (int)((long long)count * (kp + 1) / a.kparts);
  const int total = (te - tb) * C::SPT;  // slices of this item
  // (with partial buffers an empty part still stores its zeros)
  if (total <= 0 && !a.w_part) return;
  const int m0 = mb * C::BM, n0 = nb * C::BN;
  const T* __restrict__ Hs = static_cast<const T*>(a.h);
  const T* __restrict__ Gs = static_cast<const T*>(a.g);
  const uint32_t lbase = lds_addr(lds);
  // column sums of dz for db_out: wave row 0 of the hidden-block-0 workgroups
  const bool do_db = mb == 0 && wm == 0;

  // Copies of one slice: copy q (0 .. CA-1: the h part, cell rows of BM
  // hidden values; CA .. CA+CB-1: the dz part, BN vocabulary values) is
  // issued by wave q % 4; lane l fills 16 bytes of the part at offset
  // 1024 q' + 16 l.  The element offset of each copy inside a tile is fixed
  // per item; a slice adds its tile base and (slice in tile) * KB/8 frames.
  constexpr int NQ = C::QPW;  // copies per wave per slice
  uint32_t coff[C::QPW];
#pragma unroll
  for (int k = 0; k < C::QPW; ++k) {
    const int q = w + 4 * k;
    uint32_t off;
    if (q < C::CA) {
      const int row = q * (1024 / C::ROWA) + lane / C::GA;
      const int lg = (lane % C::GA) ^ swz_dw(row);
      const int col = min(m0 + lg * C::CE, H - C::CE);
      off = (uint32_t)((((row >> 3) * a.CU) + (row & 7)) * H + col);
    } else {
      const int qb = q - C::CA;
      const int row = qb * (1024 / C::ROWB) + lane / C::GB;
      const int lg = (lane % C::GB) ^ swz_dw(row);
      const int col = min(n0 + lg * C::CE, VW - C::CE);
      off = (uint32_t)((((row >> 3) * a.CU) + (row & 7)) * LG + col);
    }
    coff[k] = off;
  }
  auto issue = [&](int g) {
    const int tix = tb + g / C::SPT, ss = g % C::SPT;
    int b, tt, tu;
    tile_unpack(ld_const(a.tiles + tix), b, tt, tu);
    // the slice's first cell row: frame tt*16 + ss*KB/8, label position tu*8
    const size_t crow = ((size_t)b * a.CT + tt * kTileT + ss * (C::KB / 8)) * a.CU + tu * kTileU;
    const T* hb = Hs + crow * H;
    const T* gb = Gs + crow * LG;
    const uint32_t st = lbase + (g % C::NST) * C::SLICE;
#pragma unroll
    for (int k = 0; k < C::QPW; ++k) {
      const int q = w + 4 * k;
      if (q < C::CA) dma16(hb + coff[k], st + q * 1024);
      else dma16(gb + coff[k], st + C::SA + (q - C::CA) * 1024);
    }
  };

  // Fragment of 8 consecutive cell rows (k) of one column: rows 16 kk + 8
  // (l/32) + e, column col0 + l%32, of a slice part with rowb-byte rows.
  // bf16: two transposing reads, of rows 16 kk + r and 16 kk + r + 4, where
  // lane l supplies r = 8 (l/32) + (l%16)/4 and 4 columns from
  // col0 + 16 ((l/16) & 1) + 4 (l%4).  The granule swizzle of those rows
  // does not depend on kk, so a lane's byte offset inside the part is fixed
  // (lane_off) and a k-step adds 16 kk rows.
  auto lane_off = [&](int rowb, int col0) -> uint32_t {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int r = 8 * (g16 >> 1) + (i16 >> 2);
    const int col = col0 + 16 * (g16 & 1) + 4 * (i16 & 3);
    return (uint32_t)(r * rowb + ((((col * 2) >> 4) ^ swz_dw(r)) << 4) + ((col * 2) & 15));
  };
  uint32_t offA[2], offB[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) offA[i] = lane_off(C::ROWA, 64 * wm + 32 * i);
#pragma unroll
  for (int j = 0; j < 4; ++j) offB[j] = C::SA + lane_off(C::ROWB, 128 * wn + 32 * j);
  auto frag_T = [&](const char* sl, uint32_t off, const char* part, int rowb, int kk, int col0) {
    Frag8<T> f;
    if constexpr (C::kBf16) {
      const char* p = sl + off + 16 * kk * rowb;
      const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
      const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * rowb));
      const u32x2_t x2 = __builtin_bit_cast(u32x2_t, x), y2 = __builtin_bit_cast(u32x2_t, y);
      f.v = u32x4{x2[0], x2[1], y2[0], y2[1]};
    } else {
      const int col = col0 + lc;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 16 * kk + 8 * kh + e;
        x[e] = *reinterpret_cast<const float*>(part + r * rowb + ((((col * 4) >> 4) ^ swz_dw(r)) << 4) +
                                               ((col * 4) & 15));
      }
      pack_frag(f, x);
    }
    return f;
  };
  // sum of a fragment's 8 values (the column's 8 cells of a k-step)
  auto fsum = [&](const Frag8<T>& f) {
    float sdb = 0.f;
    if constexpr (C::kBf16) {
      // two bf16 values per dot product with (1, 1); the builtin takes the
      // bf16 pairs as 2 x 16-bit integer vectors (bit patterns)
      typedef short s16x2 __attribute__((ext_vector_type(2)));
      const s16x2 one = __builtin_bit_cast(s16x2, 0x3f803f80u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = f.v[q];
        sdb = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, w), one, sdb, false);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) sdb += f.get(e);
    }
    return sdb;
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  double dbacc[4] = {0.0, 0.0, 0.0, 0.0};

  Frag8<T> fa[2][2], fb[2][4];
  auto rd = [&](int g, int kk, int fbuf) {
    const char* sl = lds + (g % C::NST) * C::SLICE;
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[fbuf][i] = frag_T(sl, offA[i], sl, C::ROWA, kk, 64 * wm + 32 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[fbuf][j] = frag_T(sl, offB[j], sl + C::SA, C::ROWB, kk, 128 * wn + 32 * j);
    if (do_db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dbacc[j] += (double)fsum(fb[fbuf][j]);
    }
  };
  auto mm = [&](int fbuf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_step(acc[i][j], fa[fbuf][i], fb[fbuf][j]);
  };

  // ---- slices 0, 1, 2 in flight; slice g+3 is issued into slice g's buffer
  // once every wave is done reading slice g
  if (total > 0) {
  issue(0);
  if (total > 1) issue(1);
  if (total > 2) issue(2);
  if (total > 2) wait_vm<2 * NQ>();
  else if (total > 1) wait_vm<NQ>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  rd(0, 0, 0);
  }
  for (int g = 0; g < total; ++g) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      const int fcur = kk & 1;  // KSTEPS is even: parity of the k-step in the stream
      __builtin_amdgcn_sched_barrier(0);
      mm(fcur);
      if (kk + 1 < C::KSTEPS) {
        rd(g, kk + 1, fcur ^ 1);
        interleave_mfma<C::NMFMA, C::kBf16 ? 3 : 1, C::kBf16 ? 4 : 1>();
      } else if (g + 1 < total) {
        // (the MFMAs above run on while this wave waits)
        if (g + 2 < total) wait_vm<NQ>();  // slice g+1 landed, g+2 may be in flight
        else wait_vm<0>();
        wait_lgkm0();  // this wave's reads of slice g are done
        __builtin_amdgcn_s_barrier();
        if (g + 3 < total) issue(g + 3);
        rd(g + 1, 0, fcur ^ 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- float32 atomics into d_W_out; float64 column sums into d_b64
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 128 * wn + 32 * j + lc;
      if (n < VW) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 64 * wm + 32 * i + acc_row(r, kh);
          if (m >= H) continue;
          if (a.w_part)
            a.w_part[((size_t)kp * H + m) * LG + n] = acc[i][j][r];
          else
            atomicAdd(&a.d_W[(size_t)m * V + V0 + n], acc[i][j][r]);
        }
      }
    }
  if (do_db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the other 8 cells of each k-step sit in lane l ^ 32
      const double v = dbacc[j] + __shfl_xor(dbacc[j], 32);
      const int n = n0 + 128 * wn + 32 * j + lc;
      if (kh == 0 && n < VW) {
        if (a.b_part)
          a.b_part[(size_t)kp * LG + n] = v;
        else
          atomicAdd(&a.d_b64[V0 + n], v);
      }
    }
  }
}

// First index of the sorted tile list [lo, hi) whose word is not below key
// (the words order by utterance, tile row, tile column; uniform scalar loads).
__device__ __forceinline__ int tile_lower_bound(const int32_t* tiles, int lo, int hi, uint32_t key) {
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((uint32_t)ld_const(tiles + mid) < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ bool tile_present(const int32_t* tiles, int lo, int hi, uint32_t key) {
  const int j = tile_lower_bound(tiles, lo, hi, key);
  return j < hi && (uint32_t)ld_const(tiles + j) == key;
}

// Deterministic d_enc / d_pred of one chunk, from the per-tile rows dh
// stored (enc_part / pred_part, indexed by list entry).  Workgroup (i, hidden
// block) belongs to list entry i = tile (b, tt, tu).  If i is the first entry
// of tile row (b, tt), it sums that row's entries' d_enc rows in list order
// and adds the sums to d_enc.  If no entry of an earlier tile row of
// utterance b has column tu, it sums the d_pred rows of column (b, tu) over
// the tile rows in order and adds them to d_pred.  Each output element of
// the chunk gets one addition, and every sum has a fixed order.
__global__ __launch_bounds__(256) void dh_reduce_kernel(DhArgs a) {
  if (ld_const(a.hdr + kHdrRefuse)) return;
  const int count = ld_const(a.tile_count);
  const int i = blockIdx.x;
  if (i >= count) return;
  const Dims d = a.d;
  const int H = d.H, n = blockIdx.y * 256 + threadIdx.x;
  const int32_t* tiles = a.tiles;
  const uint32_t key = (uint32_t)ld_const(tiles + i);
  int b, tt, tu;
  tile_unpack((int)key, b, tt, tu);
  const int Tl = ld_const(a.Teff + b), Ul = ld_const(a.Ueff + b);
  // d_enc: the run of tile row (b, tt) starts at i
  if (i == 0 || ((uint32_t)ld_const(tiles + i - 1) >> 7) != (key >> 7)) {
    int e = i + 1;
    while (e < count && ((uint32_t)ld_const(tiles + e) >> 7) == (key >> 7)) ++e;
    if (n < H) {
      for (int r = 0; r < kTileT; ++r) {
        const int t = a.ct0 + tt * kTileT + r;
        if (t >= Tl) break;
        float sum = 0.f;
        for (int j = i; j < e; ++j) sum += a.enc_part[((size_t)j * kTileT + r) * H + n];
        a.d_enc[((size_t)b * d.T + t) * H + n] += sum;
      }
    }
  }
  // d_pred: utterance b's entries are [ub, ue); column tu's first tile row
  // owns the column
  const int ub = tile_lower_bound(tiles, 0, count, (uint32_t)tile_pack(b, 0, 0));
  const int ue = tile_lower_bound(tiles, ub, count, (uint32_t)tile_pack(b + 1, 0, 0));
  int fb_, tt_first, tt_last, fu_;
  tile_unpack(ld_const(tiles + ub), fb_, tt_first, fu_);
  tile_unpack(ld_const(tiles + ue - 1), fb_, tt_last, fu_);
  for (int r = tt_first; r < tt; ++r)
    if (tile_present(tiles, ub, ue, (uint32_t)tile_pack(b, r, tu))) return;
  float sum[kTileU];
#pragma unroll
  for (int q = 0; q < kTileU; ++q) sum[q] = 0.f;
  for (int r = tt; r <= tt_last; ++r) {
    const int j = tile_lower_bound(tiles, ub, ue, (uint32_t)tile_pack(b, r, tu));
    if (j >= ue || (uint32_t)ld_const(tiles + j) != (uint32_t)tile_pack(b, r, tu)) continue;
    if (n < H) {
#pragma unroll
      for (int q = 0; q < kTileU; ++q) sum[q] += a.pred_part[((size_t)j * kTileU + q) * H + n];
    }
  }
  if (n < H) {
#pragma unroll
    for (int q = 0; q < kTileU; ++q) {
      const int u = a.cu0 + tu * kTileU + q;
      if (u <= Ul) a.d_pred[((size_t)b * d.U1 + u) * H + n] += sum[q];
    }
  }
}

// Deterministic d_W_out / d_b_out of one vocabulary part of one chunk: the
// split-K parts (stored [kparts, H, ldg] and [kparts, ldg]) added in order,
// one thread per element of the part's columns.
__global__ __launch_bounds__(256) void dw_reduce_kernel(DwArgs a) {
  if (ld_const(a.hdr + kHdrRefuse)) return;
  const int H = a.d.H, V = a.d.V, VW = a.vw, LG = a.ldg;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t HL = (size_t)H * LG;
  if (i < (size_t)H * VW) {
    const int m = (int)(i / VW), n = (int)(i % VW);
    float s = 0.f;
    for (int kp = 0; kp < a.kparts; ++kp) s += a.w_part[kp * HL + (size_t)m * LG + n];
    a.d_W[(size_t)m * V + a.v0 + n] += s;
  }
  if (i < (size_t)VW) {
    double s = 0.0;
    for (int kp = 0; kp < a.kparts; ++kp) s += a.b_part[(size_t)kp * LG + i];
    a.d_b64[a.v0 + i] += s;
  }
}

__global__ void db_finalize_kernel(const double* __restrict__ src, float* __restrict__ dst, int V,
                                   int32_t* mark) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < V) dst[v] = (float)src[v];
  // the stored logits are now dz (unless this backward refused the state)
  if (mark && v == 0 && mark[kHdrRefuse] == 0) atomicOr(&mark[1], kFlagConsumed);
}

}  // namespace

hipError_t launch_db_finalize(const double* db64, float* d_b, int V, int32_t* mark, hipStream_t st) {
  hipLaunchKernelGGL(db_finalize_kernel, dim3((V + 255) / 256), dim3(256), 0, st, db64, d_b, V,
                     mark);
  return hipGetLastError();
}


hipError_t launch_grad_inplace(void* z, bool bf16, const JointArgs& a, int max_tiles,
                               hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(grad_inplace_kernel<uint16_t>, dim3(max_tiles), dim3(256), 0, st, a,
                       static_cast<uint16_t*>(z));
  else
    hipLaunchKernelGGL(grad_inplace_kernel<float>, dim3(max_tiles), dim3(256), 0, st, a,
                       static_cast<float*>(z));
  return hipGetLastError();
}

hipError_t launch_dh_reduce(const DhArgs& a, int max_tiles, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(dh_reduce_kernel, dim3(max_tiles, (a.d.H + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const DwArgs& a, hipStream_t st) {
  const size_t n = (size_t)a.d.H * a.vw;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dh(const DhArgs& a, bool bf16, int max_tiles, hipStream_t st) {
  const int nnb = (a.d.H + DhCfg<float>::NB - 1) / DhCfg<float>::NB;
  const int kb = bf16 ? DhCfg<uint16_t>::KB : DhCfg<float>::KB;
  const int nk = (a.vw + kb - 1) / kb;
  // resident workgroups (a multiple of 8: one per XCD in turn)
  const int gmax = max(8, (device_cu_count() * (bf16 ? DhCfg<uint16_t>::OCC : DhCfg<float>::OCC)) & ~7);
  // split the vocabulary of each (tile, hidden block) until every resident
  // workgroup gets at least three items (judged from the list capacity),
  // keeping at least 32 slices per part (the per-item overhead)
  DhArgs b = a;
  b.ksplit = 1;
  if (a.vw % kb == 0 && !a.enc_part)  // per-tile partial rows: one vocabulary part
    while (b.ksplit < 4 && nk % (2 * b.ksplit) == 0 && nk / (2 * b.ksplit) >= 32 &&
           (long long)max_tiles * nnb * b.ksplit < 3LL * gmax)
      b.ksplit *= 2;
  const long long items = (long long)max_tiles * nnb * b.ksplit;
  if (items <= 0) return hipSuccess;
  const long long g8 = (items + 7) / 8 * 8;
  dim3 grid((unsigned)(g8 < gmax ? g8 : gmax)), block(256);
  const bool vtail = a.vw % kb != 0;
  if (bf16) {
    if (vtail) hipLaunchKernelGGL((dh_kernel<uint16_t, true>), grid, block, 0, st, b);
    else hipLaunchKernelGGL((dh_kernel<uint16_t, false>), grid, block, 0, st, b);
  } else {
    if (vtail) hipLaunchKernelGGL((dh_kernel<float, true>), grid, block, 0, st, b);
    else hipLaunchKernelGGL((dh_kernel<float, false>), grid, block, 0, st, b);
  }
  return hipGetLastError();
}

hipError_t launch_dw(const DwArgs& a, bool bf16, hipStream_t st) {
  const int nmb = (a.d.H + DwCfg<float>::BM - 1) / DwCfg<float>::BM;
  const int nnb = (a.vw + DwCfg<float>::BN - 1) / DwCfg<float>::BN;
  const long long items = (long long)nmb * nnb * a.kparts;
  if (items <= 0) return hipSuccess;
  dim3 grid((unsigned)((items + 7) / 8 * 8)), block(256);  // 8 XCDs, items grouped per XCD
  if (bf16) hipLaunchKernelGGL(dw_kernel<uint16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(dw_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace rnntj
