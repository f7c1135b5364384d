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
//   kLse    : running sum of exp(z) carried across vocabulary tiles (with a
//             running max unless every |z| is provably below 64); at the end
//             lse, LB = z[blank] - lse, LE = z[label] - lse.
//   kStoreZ : kLse plus the logits written to HBM (untiled mode), and the h
//             rows the weight gradient reads.
//   kGrad   : logit gradient of the loss (tiled backward), from the per-cell
//             transition posteriors gB, gE and the stored lse:
//             dz[v] = gc * (occ * exp(z[v] - lse) - gB [v=blank] - gE [v=y_u]),
//             occ = gB + gE, written to a chunk buffer, plus the h rows.
//
// Work decomposition (gfx950, wave64): the kernel is persistent -- one
// workgroup per compute unit walks the list of active tiles (tiles holding at
// least one lattice cell; the list is built on the device), so every compute
// unit gets the same number of tiles whatever the length mix.  A tile is
// 16 frames x 8 label positions of one utterance, processed by 4 waves.
// Wave w owns frames
// t0+4w..t0+4w+3 x label positions u0..u0+7 = 32 rows of a 32x32 MFMA block,
// row r <-> (t0 + 4w + r/8, u0 + r%8).  The wave keeps its 32 rows of h for
// the whole H in registers as MFMA A-fragments, and streams W_out^T through
// LDS in [128 vocab x BK hidden] slices (double buffered); each slice feeds
// four 32x32 output blocks per wave.  The slices are copied global -> LDS
// directly (no staging registers), which leaves the registers for h, the
// accumulators and B fragments read one k-step ahead of the MFMAs.
//
// h uses tanh(x) = 1 - 2 / (1 + e^{2 enc} e^{2 pred}) from the per-row
// exponentials the forward precomputes, unless some finite |enc| or |pred|
// exceeds 40 (then e^{2x} could overflow before the product), in which case
// it is evaluated directly.  Both give tanh to a few 1e-7.  The 16 + 8
// exponential rows of a tile are copied into LDS in one batch of direct
// loads (issued for the next tile while the current one runs), so building
// h costs LDS reads instead of a chain of dependent global loads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rnntj {

namespace {

constexpr float kInf = __builtin_inff();

// NBLK: 32-column output blocks per wave, i.e. a vocabulary step of
// VT = 32 NBLK columns (128 with one workgroup per compute unit; 64 with two,
// which halves the accumulators and the slices so that two workgroups fit)
template <typename T, int NBLK = 4>
struct StageCfg {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int BK = kBf16 ? 128 : 64;             // hidden elements per W^T slice
  static constexpr int CE = 16 / (int)sizeof(T);          // elements per 16-byte chunk
  static constexpr int ROWB = 256;                        // bytes per slice row (16 chunks)
  static constexpr int KK = BK / 16;                      // k-steps per slice
  static constexpr int VT = 32 * NBLK;                    // vocabulary columns per step
  static constexpr int SLICE = VT * ROWB;                 // 32 / 16 KB per slice
  static constexpr int CPW = VT / 16;                     // 1 KB copies per wave per slice
  static constexpr int OCC = NBLK == 2 ? 2 : 1;           // workgroups per compute unit
};

// One W^T slice [vt .. vt+VT) x [kc .. kc+BK) goes straight from global
// memory into LDS (global_load_lds, 16 bytes per lane, 1 KB per wave
// instruction, no staging registers; issued as `dma16`, which the compiler's
// wait insertion does not track, so that it never holds the current slice's
// reads back for the next slice's copy): wave w writes LDS chunks
// (CPW w + q)*64 + lane, q < CPW, i.e. slice row r = 4 (CPW w + q) + lane/16,
// chunk slot lane%16.  Slot s of row r holds hidden chunk s ^ (r & 15): rows are
// unpadded (the copy writes 1 KB contiguously) and the XOR keeps the
// fragment reads of 8 or 16 consecutive rows on distinct banks.  In an exact
// shape a copy's source is the slice origin Wt[vt][kc] (wave-uniform) plus
// the per-lane byte offset voff[q] of row r, chunk c, the same for every
// slice.  Otherwise the source row / column is clamped to valid memory;
// those columns are masked and those k-steps skipped by the caller.
template <typename T, int NBLK>
__device__ __forceinline__ void slice_offsets(int H, uint32_t (&voff)[StageCfg<T, NBLK>::CPW]) {
  using C = StageCfg<T, NBLK>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < C::CPW; ++q) {
    const int r = 4 * (C::CPW * w + q) + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    voff[q] = (uint32_t)((r * H + c * C::CE) * (int)sizeof(T));
  }
}
template <typename T, int NBLK, bool EXACT>
__device__ __forceinline__ void dma_slice(const T* __restrict__ Wt, int H, int V, int vt, int kc,
                                          const uint32_t (&voff)[StageCfg<T, NBLK>::CPW],
                                          char* lds_slice) {
  using C = StageCfg<T, NBLK>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t lds = lds_addr(lds_slice) + C::CPW * w * 1024;
  if constexpr (EXACT) {
    const T* base = Wt + (size_t)vt * H + kc;
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) dma16s(base, voff[q], lds + q * 1024);
  } else {
#pragma unroll
    for (int q = 0; q < C::CPW; ++q) {
      const int r = 4 * (C::CPW * w + q) + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      int n = vt + r, k = kc + c * C::CE;
      n = n < V ? n : V - 1;
      k = k < H ? k : H - C::CE;
      dma16(Wt + (size_t)n * H + k, lds + q * 1024);
    }
  }
}

// all of this wave's direct-to-LDS copies (and any other loads) have landed
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Butterfly reduce-scatter over the 32 lanes of a row group (lanes with the
// same lane / 32): v[r] is this lane's partial sum for accumulator row r; the
// result is the sum over the 32 lanes for row rs_row(lane).  Each of the four
// halving steps keeps half of the rows (by one lane bit) and adds the
// partner's copy of them; the last step adds the two 16-lane halves.
__device__ __forceinline__ int rs_row(int lane) {
  return ((lane & 1) << 3) | ((lane & 2) << 1) | ((lane & 4) >> 1) | ((lane & 8) >> 3);
}
__device__ __forceinline__ float rs_sum16(const float (&v)[16], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
  float a[8], c[4], e[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (b0 ? v[i + 8] : v[i]) + __shfl_xor(b0 ? v[i] : v[i + 8], 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = (b1 ? a[i + 4] : a[i]) + __shfl_xor(b1 ? a[i] : a[i + 4], 2);
#pragma unroll
  for (int i = 0; i < 2; ++i) e[i] = (b2 ? c[i + 2] : c[i]) + __shfl_xor(b2 ? c[i] : c[i + 2], 4);
  const float f = (b3 ? e[1] : e[0]) + __shfl_xor(b3 ? e[0] : e[1], 8);
  return f + __shfl_xor(f, 16);
}
// the same reduce-scatter with max in place of the sum
__device__ __forceinline__ float rs_max16(const float (&v)[16], int lane) {
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
  float a[8], c[4], e[2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a[i] = fmaxf(b0 ? v[i + 8] : v[i], __shfl_xor(b0 ? v[i] : v[i + 8], 1));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c[i] = fmaxf(b1 ? a[i + 4] : a[i], __shfl_xor(b1 ? a[i] : a[i + 4], 2));
#pragma unroll
  for (int i = 0; i < 2; ++i)
    e[i] = fmaxf(b2 ? c[i + 2] : c[i], __shfl_xor(b2 ? c[i] : c[i + 2], 4));
  const float f = fmaxf(b3 ? e[1] : e[0], __shfl_xor(b3 ? e[0] : e[1], 8));
  return fmaxf(f, __shfl_xor(f, 16));
}
// (m, s) <- (m, s) + (m2, s2) for sums s of 2^(x - m)
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn > -kInf) {
    s = s * exp2_fast(m - mn) + s2 * exp2_fast(m2 - mn);
    m = mn;
  }
}
// the same reduce-scatter over (max, sum) pairs
__device__ __forceinline__ void rs_lse16(const float (&m)[16], const float (&s)[16], int lane,
                                         float& mo, float& so) {
  float am[8], as[8], cm[4], cs[4], em[2], es[2];
  auto step = [&](bool hi, float km, float ks, float sm, float ss, int off, float& rm, float& rs) {
    (void)hi;
    const float pm = __shfl_xor(sm, off), ps = __shfl_xor(ss, off);
    rm = km;
    rs = ks;
    lse2_merge(rm, rs, pm, ps);
  };
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    step(b0, b0 ? m[i + 8] : m[i], b0 ? s[i + 8] : s[i], b0 ? m[i] : m[i + 8], b0 ? s[i] : s[i + 8],
         1, am[i], as[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    step(b1, b1 ? am[i + 4] : am[i], b1 ? as[i + 4] : as[i], b1 ? am[i] : am[i + 4],
         b1 ? as[i] : as[i + 4], 2, cm[i], cs[i]);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    step(b2, b2 ? cm[i + 2] : cm[i], b2 ? cs[i + 2] : cs[i], b2 ? cm[i] : cm[i + 2],
         b2 ? cs[i] : cs[i + 2], 4, em[i], es[i]);
  float fm, fs;
  step(b3, b3 ? em[1] : em[0], b3 ? es[1] : es[0], b3 ? em[0] : em[1], b3 ? es[0] : es[1], 8, fm, fs);
  step(false, fm, fs, fm, fs, 16, mo, so);
}

// acc[blk][r] without dynamic register indexing
template <int N>
__device__ __forceinline__ float sel_blk(const f32x16 (&acc)[N], int blk, int r) {
  float v = acc[0][r];
#pragma unroll
  for (int i = 1; i < N; ++i) v = blk == i ? acc[i][r] : v;
  return v;
}

// Transposed staging of one wave's 32 rows x 128 columns of bf16 output:
// Ts[col][row] (64 bytes per column), the 8-byte granules of a column
// permuted by swz(col) so that both the column writes from the accumulator
// layout and the transposing row reads are free of bank conflicts.
__device__ __forceinline__ int swz(int col) {
  return ((col >> 1) & 7) ^ (((col >> 1) & 1) << 2);
}
__device__ __forceinline__ int ts_idx(int col, int row) {
  return col * 32 + ((((row >> 2) ^ swz(col)) & 7) << 2) + (row & 3);
}

}  // namespace

// Pruned forward: the blank and label steps out of cell (t,u) of utterance b
// are kept only when both ends lie in the band s_t <= u <= s_t + S - 1
// (the final blank at (T'-1, U') always does); others get -inf.
__device__ __forceinline__ void band_mask(const JointArgs& a, int b, int t, int u, int Tl, int Ul,
                                          float& lb, float& le) {
  const int32_t* s = a.bounds + (size_t)b * a.d.T;
  const int S = a.band, s0 = s[t];
  const bool in = u >= s0 && u <= s0 + S - 1;
  bool nb;
  if (t + 1 < Tl) {
    const int s1 = s[t + 1];
    nb = u >= s1 && u <= s1 + S - 1;
  } else {
    nb = u == Ul;
  }
  if (!(in && nb)) lb = -kInf;
  if (!(in && u + 1 <= s0 + S - 1)) le = -kInf;
}

// Largest hidden size whose 24 exponential rows are staged in LDS (the
// budget left next to the W^T slices and the store staging); with two
// workgroups per compute unit the rows are read from global memory instead.
template <typename T, int KS, int NBLK>
struct EpCfg {
  static constexpr int kMaxH = sizeof(T) == 2 ? 640 : 768;
  static constexpr bool kStage = NBLK == 4 && KS * 16 <= kMaxH;
  // 16 e^{2 enc} rows then 8 e^{2 pred} rows (float32), plus one 1 KB copy
  // of slack for a partial last copy
  static constexpr int kBytes = kStage ? 96 * KS * 16 + 1024 : 16;
};

template <typename T, int KS, int MODE, bool EXACT, int NBLK>
__global__ __launch_bounds__(256, NBLK == 2 ? 2 : 1) void joint_tile_kernel(JointArgs a) {
  using C = StageCfg<T, NBLK>;
  using EP = EpCfg<T, KS, NBLK>;
  constexpr int VT = C::VT;
  constexpr bool kBf16 = C::kBf16;
  constexpr int KC_MAX = (KS * 16 + C::BK - 1) / C::BK;
  // k-steps of h held in registers at a time.  fp32 rows above 256 hidden
  // do not fit: there h is kept 16 k-steps (256 hidden) at a time and each
  // part is rebuilt from the staged exponential rows when a vocabulary step
  // reaches it (about 5 VALU per element against 256 MFMA flops)
  constexpr int KR = (!kBf16 && KS > 16) ? 16 : KS;
  constexpr int NCH = KS / KR;
  static_assert(KS % KR == 0 && KR % C::KK == 0, "h parts are whole slices");
  constexpr bool kStores = (MODE == kStoreZ || MODE == kGrad) && kBf16;
  // two separately named slice buffers: the compiler then knows that the
  // copy into one does not alias the fragment reads of the other
  __shared__ __align__(16) char Ws0[C::SLICE];
  __shared__ __align__(16) char Ws1[C::SLICE];
  __shared__ __align__(16) uint16_t Ts[kStores ? 4 : 1][kStores ? VT * 32 : 8];
  __shared__ float cap_blank[kTileCells];
  __shared__ float cap_label[kTileCells];
  __shared__ float row_c[kTileCells];  // kGrad: (lse - ln occ) * log2(e)
  __shared__ float row_b[kTileCells];  // kGrad: gc * gB
  __shared__ float row_e[kTileCells];  // kGrad: gc * gE
  __shared__ __align__(16) char Ep[EP::kBytes];
  // kStoreZ, bf16: each row's largest logit of the vocabulary step
  __shared__ __align__(16) float zm_row[(MODE == kStoreZ && kBf16) ? 4 : 1][32];

  const Dims d = a.d;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = lane >> 5, lc = lane & 31;
  const int H = d.H, V = d.V;
  const int nks = EXACT ? KS : H / 16;
  const T* __restrict__ enc = static_cast<const T*>(a.enc);
  const T* __restrict__ pred = static_cast<const T*>(a.pred);
  const T* __restrict__ Wt = static_cast<const T*>(a.Wt);
  const T* __restrict__ bias = static_cast<const T*>(a.bias);
  if (MODE == kGrad && ld_const(a.hdr + kHdrRefuse)) return;  // state refused by this backward
  const int hflags = a.hdr[1];
  const bool use_ep = (hflags & kFlagEpBad) == 0;
  // kGrad in a vocabulary part after the first: the tile's h rows were
  // stored by the first part; they are read back instead of rebuilt
  const bool h_from_mem = MODE == kGrad && a.gv0 > 0;
  const bool stage_ep = EP::kStage && use_ep && !h_from_mem;
  const bool bounded = __int_as_float(a.hdr[2]) < 64.0f;  // NaN bound -> false

  // vocabulary steps of this launch: [gv0, gv0 + gvw) (the whole vocabulary
  // outside the tiled backward's vocabulary parts)
  const int vt0 = (MODE == kGrad) ? a.gv0 / VT : 0;
  const int nvt_all = (MODE == kGrad) ? (a.gvw + VT - 1) / VT : (V + VT - 1) / VT;
  const int vsplit = (MODE == kGrad) ? a.vsplit : 1;
  const int nkc = EXACT ? KC_MAX : (H + C::BK - 1) / C::BK;
  const int n_items = a.tile_count[0] * vsplit;

  // item -> tile origin, utterance, vocabulary range (the tiled backward
  // splits a tile's vocabulary tiles over `vsplit` items)
  auto item_tile = [&](int item, int& b, int& t0, int& u0) {
    int tt, tu;
    tile_unpack(a.tiles[item / vsplit], b, tt, tu);
    t0 = a.ct0 + tt * kTileT;
    u0 = a.cu0 + tu * kTileU;
  };
  // the 16 e^{2 enc} rows t0.. and 8 e^{2 pred} rows u0.. of a tile -> Ep,
  // 1 KB direct copies spread over the waves (sources clamped to the tables)
  auto issue_ep = [&](int b, int t0, int u0) {
    if constexpr (EP::kStage) {
      const char* esrc = reinterpret_cast<const char*>(a.Eexp + ((size_t)b * d.T + t0) * H);
      const char* psrc = reinterpret_cast<const char*>(a.Pexp + ((size_t)b * d.U1 + u0) * H);
      const char* elim = reinterpret_cast<const char*>(a.Eexp + (size_t)d.B * d.T * H) - 16;
      const char* plim = reinterpret_cast<const char*>(a.Pexp + (size_t)d.B * d.U1 * H) - 16;
      const int ne = (64 * H + 1023) >> 10, np = (32 * H + 1023) >> 10;
      for (int q = w; q < ne + np; q += 4) {
        const bool isE = q < ne;
        const int j = isE ? q : q - ne;
        const char* src = (isE ? esrc : psrc) + j * 1024 + lane * 16;
        const char* lim = isE ? elim : plim;
        src = src < lim ? src : lim;
        dma16(src, lds_addr(Ep) + (isE ? 0 : 64 * H) + j * 1024);
      }
    }
  };
  // h = tanh(enc + pred) evaluated directly from the inputs (rows whose
  // e^{2x} could overflow)
  // (k-steps c KR .. c KR + KR - 1)
  auto build_h_direct = [&](Frag8<T>(&hA)[KR], int c, int b, int tv, int uv, bool valid) {
    const T* er = enc + ((size_t)b * d.T + tv) * H + 8 * kh;
    const T* pr = pred + ((size_t)b * d.U1 + uv) * H + 8 * kh;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int ks = c * KR + j;
      if ((EXACT || ks < nks) && valid) {
        const Frag8<T> e = load_frag(er + ks * 16), p = load_frag(pr + ks * 16);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = fast_tanh(e.get(i) + p.get(i));
        pack_frag(hA[j], x);
      } else {
        zero_frag(hA[j]);
      }
    }
  };
  uint32_t voff[C::CPW];
  slice_offsets<T, NBLK>(H, voff);
  // first vocabulary tile and slice count of an item
  auto item_range = [&](int it, int& vb, int& ns) {
    const int r = (MODE == kGrad) ? it % vsplit : 0;
    const int base = (nvt_all * r) / vsplit;
    vb = vt0 + base;
    ns = ((nvt_all * (r + 1)) / vsplit - base) * nkc;
  };
  // the slice being computed sits in Ws1 when `par` is set; the last slice
  // of an item starts the copy of the next item's first slice (`pre`)
  int par = 0;
  bool pre = false;
  if (stage_ep && (int)blockIdx.x < n_items) {
    int b, t0, u0;
    item_tile(blockIdx.x, b, t0, u0);
    issue_ep(b, t0, u0);
  }

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
  int b, t0, u0;
  item_tile(item, b, t0, u0);
  const int Tl = a.Teff[b], Ul = a.Ueff[b];
  // vocabulary tiles of this item
  const int vr = (MODE == kGrad) ? item % vsplit : 0;
  int vt_begin, nstage;
  item_range(item, vt_begin, nstage);
  const int vt_end = vt_begin + nstage / nkc;
  int next_vb = 0, next_ns = 0;
  if (item + (int)gridDim.x < n_items) item_range(item + gridDim.x, next_vb, next_ns);
  if (nstage <= 0) {  // uniform; no work, but keep the row prefetch going
    if (stage_ep && item + (int)gridDim.x < n_items) {
      wait_vmem();
      __syncthreads();
      int nb, nt0, nu0;
      item_tile(item + gridDim.x, nb, nt0, nu0);
      issue_ep(nb, nt0, nu0);
    }
    continue;
  }

  // ---- prologue: start the first W^T slice (unless the previous item
  // did), build h in registers
  if (!pre) dma_slice<T, NBLK, EXACT>(Wt, H, V, vt_begin * VT, 0, voff, par ? Ws1 : Ws0);
  if (stage_ep) {
    wait_vmem();  // this wave's exponential rows (and slice part) have landed
    __syncthreads();
  }
  // kGrad: the inputs of row tid's posteriors, loaded now and used after
  // the h build (which hides their latency)
  const int prw = tid >> 5, prr = tid & 31;
  const int pt = t0 + 4 * prw + (prr >> 3), pu = u0 + (prr & 7);
  const bool prow = MODE == kGrad && tid < kTileCells && pt < Tl && pu <= Ul;
  CellPostIn pin{0.0, 0.0, 0.0, 0.0, 0.f, 0.f};
  float plse = 0.f;
  double plogP = 0.0, pg = 1.0;
  if (prow) {
    pin = cell_post_load(d, a.alpha, a.beta, a.LB, a.LE, b, pt, pu, Tl, Ul, a.hdr[3]);
    plse = a.lse[skew_idx(d, b, pt, pu)];
    plogP = a.logP[b];
    pg = a.gcost ? (double)a.gcost[b] : 1.0;
  }

  // h of this lane's tile row (k-steps c KR .. c KR + KR - 1 of it)
  Frag8<T> hA[KR];
  if constexpr (NCH == 1)
  {
    const int tt = lc >> 3, uu = lc & 7;
    const int t = t0 + 4 * w + tt, u = u0 + uu;
    const bool valid = (t < Tl) && (u <= Ul);
    const int tv = valid ? t : 0, uv = valid ? u : 0;
    if (h_from_mem) {
      // the same fragments the first part built and stored (zero rows
      // outside the lattice)
      const T* hrow = static_cast<const T*>(a.hout) +
                      (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * H + 8 * kh;
#pragma unroll
      for (int ks = 0; ks < KR; ++ks) {
        if (EXACT || ks < nks) hA[ks] = load_frag(hrow + ks * 16);
        else zero_frag(hA[ks]);
      }
    } else if constexpr (EP::kStage) {
      // exponential rows from LDS
      if (use_ep) {
        const float* er = reinterpret_cast<const float*>(Ep) + (4 * w + tt) * H + 8 * kh;
        const float* pr = reinterpret_cast<const float*>(Ep + 64 * H) + uu * H + 8 * kh;
#pragma unroll
        for (int ks = 0; ks < KR; ++ks) {
          if ((EXACT || ks < nks) && valid) {
            const Frag8<float> e = load_frag(er + ks * 16), p = load_frag(pr + ks * 16);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
              x[i] = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e.get(i) * p.get(i));
            pack_frag(hA[ks], x);
          } else {
            zero_frag(hA[ks]);
          }
        }
      } else {
        build_h_direct(hA, 0, b, tv, uv, valid);
      }
    } else if (use_ep) {
      // exponential rows straight from global memory
      const float* er = a.Eexp + ((size_t)b * d.T + tv) * H + 8 * kh;
      const float* pr = a.Pexp + ((size_t)b * d.U1 + uv) * H + 8 * kh;
#pragma unroll
      for (int ks = 0; ks < KR; ++ks) {
        if ((EXACT || ks < nks) && valid) {
          const Frag8<float> e = load_frag(er + ks * 16), p = load_frag(pr + ks * 16);
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            x[i] = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e.get(i) * p.get(i));
          pack_frag(hA[ks], x);
        } else {
          zero_frag(hA[ks]);
        }
        // at most four k-steps of loads in flight: h itself fills most of
        // the registers of a two-workgroup-per-CU launch
        if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      build_h_direct(hA, 0, b, tv, uv, valid);
    }
  }
  // h rebuilt in parts (fp32, more than 256 hidden; the exponential rows
  // are always staged then): from the stored rows, the staged rows or the
  // inputs
  static_assert(NCH == 1 || EP::kStage, "parts of h are rebuilt from staged rows");
  auto build_part = [&](int c) {
    const int t = t0 + 4 * w + (lc >> 3), u = u0 + (lc & 7);
    const bool valid = (t < Tl) && (u <= Ul);
    if (h_from_mem) {
      const T* hrow = static_cast<const T*>(a.hout) +
                      (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * H + 8 * kh;
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        const int ks = c * KR + j;
        if (EXACT || ks < nks) hA[j] = load_frag(hrow + ks * 16);
        else zero_frag(hA[j]);
      }
    } else if (use_ep) {
      const float* er = reinterpret_cast<const float*>(Ep) + (t - t0) * H + 8 * kh;
      const float* pr = reinterpret_cast<const float*>(Ep + 64 * H) + (u - u0) * H + 8 * kh;
#pragma unroll
      for (int j = 0; j < KR; ++j) {
        const int ks = c * KR + j;
        if ((EXACT || ks < nks) && valid) {
          const Frag8<float> e = load_frag(er + ks * 16), p = load_frag(pr + ks * 16);
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            x[i] = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e.get(i) * p.get(i));
          pack_frag(hA[j], x);
        } else {
          zero_frag(hA[j]);
        }
      }
    } else {
      build_h_direct(hA, c, b, valid ? t : 0, valid ? u : 0, valid);
    }
  };
  // kStoreZ / kGrad: the weight-gradient GEMM reads these h rows back
  // ([B, CT, CU, H]); every row of the tile is written (zero outside the
  // lattice).  (Untiled forward: the h rows of the whole padded lattice,
  // kept for the backward.)
  const bool h_store = (MODE == kGrad || MODE == kStoreZ) && vr == 0 &&
                       (MODE == kGrad ? a.gv0 == 0 : a.hout != nullptr);
  // (parts of h: stored as each is built in the first vocabulary step)
  auto store_part = [&](int c) {
    const int t = t0 + 4 * w + (lc >> 3), u = u0 + (lc & 7);
    T* hrow = static_cast<T*>(a.hout) +
              (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * H + 8 * kh;
#pragma unroll
    for (int j = 0; j < KR; ++j) {
      const int ks = c * KR + j;
      if (EXACT || ks < nks) store_frag(hrow + ks * 16, hA[j]);
    }
  };
  // labels of this lane's accumulator rows: u = u0 + 4*kh + j
  int lab[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int u = u0 + 4 * kh + j;
    lab[j] = (u < Ul) ? a.labels[(size_t)b * d.U + u] : -1;
  }
  // kGrad: label of tile row lc (u = u0 + lc % 8), for the one-hot terms
  int lab_row = -1;
  if constexpr (MODE == kGrad) {
    const int u = u0 + (lc & 7);
    lab_row = (u < Ul) ? a.labels[(size_t)b * d.U + u] : -1;
  }

  float gc = 1.0f;
  float cst[16];  // kGrad, NBLK == 4: per-row exponent offsets (NBLK == 2 reads row_c)
  if constexpr (MODE == kGrad) {
    if (tid < kTileCells) {
      float c = kInf, gb = 0.f, ge = 0.f;
      if (prow) {
        double gB, gE;
        cell_post_eval(pin, plogP, pt, pu, Tl, Ul, gB, gE, a.hdr[3]);
        const double occ = gB + gE;
        c = occ > 0.0 ? (float)(((double)plse - log(occ)) * 1.4426950408889634) : kInf;
        gb = (float)(pg * gB);
        ge = (float)(pg * gE);
      }
      row_c[tid] = c;
      row_b[tid] = gb;
      row_e[tid] = ge;
    }
    gc = a.gcost ? a.gcost[b] : 1.0f;
  }
  wait_vmem();
  __syncthreads();
  // every wave has built its h: the next item's exponential rows may load
  // (h rebuilt in parts reads them until the item ends)
  if (NCH == 1 && stage_ep && item + (int)gridDim.x < n_items) {
    int nb, nt0, nu0;
    item_tile(item + gridDim.x, nb, nt0, nu0);
    issue_ep(nb, nt0, nu0);
  }
  if constexpr ((MODE == kGrad || MODE == kStoreZ) && NCH == 1) {
    // issued after the barrier, so the first slice's MFMAs cover their
    // completion instead of the barrier waiting for it
    if (h_store) {
      const int t = t0 + 4 * w + (lc >> 3), u = u0 + (lc & 7);
      T* hrow = static_cast<T*>(a.hout) +
                (((size_t)b * a.CT + (t - a.ct0)) * a.CU + (u - a.cu0)) * H + 8 * kh;
#pragma unroll
      for (int ks = 0; ks < KR; ++ks)
        if (EXACT || ks < nks) store_frag(hrow + ks * 16, hA[ks]);
    }
  }
  if constexpr (MODE == kGrad) {
#pragma unroll
    for (int r = 0; r < 16; ++r) cst[r] = NBLK == 4 ? row_c[w * 32 + acc_row(r, kh)] : 0.f;
  }

  // running max (base 2) and sum of each row: NBLK == 4 keeps this lane's
  // columns of its 16 rows and combines the lanes at the end; NBLK == 2 adds
  // every vocabulary step's reduce-scatter into one row per lane (rs_row)
  float mrun[16], srun[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mrun[r] = -kInf;
    srun[r] = 0.f;
  }
  float mrow = -kInf, srow = 0.f;

  // bias of a vocabulary step's columns, loaded one step ahead and kept
  // unconverted until the step starts: its wait then comes long after the
  // load and never covers a slice copy issued after it
  T bnx[NBLK];
  auto load_bias = [&](int vt) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const int col = vt + blk * 32 + lc;
      bnx[blk] = bias[(EXACT || col < V) ? col : V - 1];
    }
  };
  load_bias(vt_begin * VT);

  // B-fragment reads: row lc of each 32-row block; hidden chunk c of that
  // row is stored at slot c ^ (lc & 15).  bf16: a fragment is one 16-byte
  // chunk (2*kk + kh); fp32: two chunks (4*kk + 2*kh, +1), each at its own
  // swizzled slot
  const int xm = lc & 15;
  auto bfrag = [&](const char* slice, int blk, int kk) {
    const char* rb = slice + lc * C::ROWB + blk * 32 * C::ROWB;
    Frag8<T> f;
    if constexpr (kBf16) {
      f.v = *reinterpret_cast<const u32x4*>(rb + (((2 * kk + kh) ^ xm) << 4));
    } else {
      f.lo = *reinterpret_cast<const f32x4*>(rb + (((4 * kk + 2 * kh) ^ xm) << 4));
      f.hi = *reinterpret_cast<const f32x4*>(rb + (((4 * kk + 2 * kh + 1) ^ xm) << 4));
    }
    return f;
  };
  // fragments of the current k-step; after the first slice of the item
  // they were read by the previous slice (below)
  Frag8<T> bcur[NBLK];
  bool have_b = false;

  int s = 0;
  for (int vti = vt_begin; vti < vt_end; ++vti) {
    const int vt = vti * VT;
    // accumulators start at the bias of their column
    f32x16 acc[NBLK];
    bool cvalid[NBLK];
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      cvalid[blk] = EXACT || vt + blk * 32 + lc < V;
      const float bc = cvalid[blk] ? ElemTraits<T>::to_f32(bnx[blk]) : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[blk][r] = bc;
    }
    if (vti + 1 < vt_end) load_bias(vt + VT);
    // the bias is consumed before this step's first slice copy is issued
    __builtin_amdgcn_sched_barrier(0);

    // slices in parts of h (one part unless h is rebuilt in parts); the
    // slices of a part are unrolled, so every h fragment index is a constant
    constexpr int KCR = KR / C::KK;
    for (int c = 0; c < NCH; ++c) {
    if constexpr (NCH > 1) {
      if (!EXACT && c * KR >= nks) break;
      build_part(c);
      if constexpr (MODE == kGrad || MODE == kStoreZ)
        if (h_store && vti == vt_begin) store_part(c);
    }
#pragma unroll
    for (int kq = 0; kq < KCR; ++kq) {
      const int kc = c * KCR + kq;
      if (EXACT || kc < nkc) {
        const bool has_next = (s + 1) < nstage;
        const bool cross = !has_next && next_ns > 0;  // the next item's first slice
        const int ns = s + 1;
        const int nvt = has_next ? (vt_begin + ns / nkc) * VT : next_vb * VT;
        const int nkc0 = has_next ? (ns % nkc) * C::BK : 0;
        const char* src = par ? Ws1 : Ws0;
        char* nxt = par ? Ws0 : Ws1;
        // one stage: start the copy of the next slice into `nxt`, run the
        // MFMAs of this slice from `src` with the B fragments one k-step
        // ahead.  The slice barrier sits before the last k-step's MFMAs:
        // once every wave's reads of `src` are done and its part of `nxt`
        // has landed, the next slice's first fragments load while those
        // MFMAs run.
        if (has_next || cross) dma_slice<T, NBLK, EXACT>(Wt, H, V, nvt, nkc0, voff, nxt);
        if (!have_b) {
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) bcur[blk] = bfrag(src, blk, 0);
        }
        Frag8<T> bnxt[NBLK];
#pragma unroll
        for (int kk = 0; kk < C::KK; ++kk) {
          const int ks = kc * C::KK + kk;
          const bool live = ks < KS && (EXACT || ks < nks);
          if (kk + 1 < C::KK) {
            const bool nlive = ks + 1 < KS && (EXACT || ks + 1 < nks);
            if (nlive) {
#pragma unroll
              for (int blk = 0; blk < NBLK; ++blk) bnxt[blk] = bfrag(src, blk, kk + 1);
            }
          } else {
            wait_lgkm0();  // this wave's reads of `src` are done
            wait_vmem();   // and its part of `nxt` has landed
            __syncthreads();
            if (has_next) {
#pragma unroll
              for (int blk = 0; blk < NBLK; ++blk) bnxt[blk] = bfrag(nxt, blk, 0);
            }
          }
          // keep the reads for the next k-step issued ahead of this one's MFMAs
          __builtin_amdgcn_sched_barrier(0);
          if (live) {
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
              mma_step(acc[blk], hA[kq * C::KK + kk], bcur[blk]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) bcur[blk] = bnxt[blk];
        }
        have_b = has_next;
        ++s;
        par ^= 1;
      }
    }
    }  // parts of h

    // ---- epilogue for vocabulary columns vt .. vt+VT-1
    if constexpr ((MODE == kLse || MODE == kStoreZ) && NBLK == 2) {
      if (bounded) {
        float tsum[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            sum += cvalid[blk] ? exp2_fast(acc[blk][r] * kLog2e) : 0.f;
          tsum[r] = sum;
        }
        srow += rs_sum16(tsum, lane);
      } else {
        float tm[16], tsum[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x[NBLK];
          float mx = -kInf;
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) {
            x[blk] = cvalid[blk] ? acc[blk][r] * kLog2e : -kInf;
            mx = fmaxf(mx, x[blk]);
          }
          float sum = 0.f;
          if (mx > -kInf) {
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) sum += exp2_fast(x[blk] - mx);
          }
          tm[r] = mx;
          tsum[r] = sum;
        }
        float m2, s2;
        rs_lse16(tm, tsum, lane, m2, s2);
        lse2_merge(mrow, srow, m2, s2);
      }
    }
    if constexpr ((MODE == kLse || MODE == kStoreZ) && NBLK == 4) {
      if (bounded) {
        // every |z| < 64: sum e^z directly, no running max needed
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sum = srun[r];
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            sum += cvalid[blk] ? exp2_fast(acc[blk][r] * kLog2e) : 0.f;
          srun[r] = sum;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x[NBLK];
          float mx = -kInf;
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk) {
            x[blk] = cvalid[blk] ? acc[blk][r] * kLog2e : -kInf;
            mx = fmaxf(mx, x[blk]);
          }
          const float mn = fmaxf(mrun[r], mx);
          if (mn > -kInf) {
            float sum = srun[r] * exp2_fast(mrun[r] - mn);
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) sum += exp2_fast(x[blk] - mn);
            srun[r] = sum;
            mrun[r] = mn;
          }
        }
      }
    }
    if constexpr (MODE == kLse || MODE == kStoreZ) {
      // blank logit
      if (d.blank >= vt && d.blank < vt + VT) {
        const int bb = d.blank - vt;
        if (lc == (bb & 31)) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            cap_blank[w * 32 + acc_row(r, kh)] = sel_blk<NBLK>(acc, bb >> 5, r);
        }
      }
      // label logits
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dl = lab[j] - vt;
        if (dl >= 0 && dl < VT && (dl & 31) == lc) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * i + j;
            cap_label[w * 32 + acc_row(r, kh)] = sel_blk<NBLK>(acc, dl >> 5, r);
          }
        }
      }
    } else {  // kGrad: acc <- dz without the one-hot terms
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float c = NBLK == 4 ? cst[r] : row_c[w * 32 + acc_row(r, kh)];
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
          acc[blk][r] = gc * exp2_fast(acc[blk][r] * kLog2e - c);
      }
    }

    if constexpr (MODE == kStoreZ || MODE == kGrad) {
      const int RT = MODE == kGrad ? a.CT : d.Tpad, RU = MODE == kGrad ? a.CU : d.U1pad;
      const int rt0 = MODE == kGrad ? a.ct0 : 0, ru0 = MODE == kGrad ? a.cu0 : 0;
      T* out = static_cast<T*>(MODE == kGrad ? a.gout : a.zout);
      // rows of the output: the whole vocabulary (logits), or the launch's
      // vocabulary part (logit gradients)
      const size_t ldz = MODE == kGrad ? (size_t)a.gld : (size_t)V;
      const int zc0 = MODE == kGrad ? a.gv0 : 0;
      if constexpr (MODE == kStoreZ && kBf16) {
        // Stored as bf16(z - M), M = the row's largest logit of this step
        // (kept in float32 beside them).  A logit of size |z| would carry a
        // bf16 rounding error of up to |z| 2^-8 into exp(z - lse); relative
        // to M the error is at most |z - M| 2^-8, and since
        // exp(z - lse) <= exp(z - M), its effect on a softmax entry stays
        // below 2^-8 / e whatever the size of the logits.
        float tm[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float mx = -kInf;
#pragma unroll
          for (int blk = 0; blk < NBLK; ++blk)
            if (cvalid[blk]) mx = fmaxf(mx, acc[blk][r]);
          tm[r] = mx;
        }
        const float mr = rs_max16(tm, lane);  // accumulator row rs_row(lane) of this half
        if (lc < 16) {
          const int r = rs_row(lc);
          const int row = acc_row(r, kh);
          zm_row[w][row] = mr;
          const int t = t0 + 4 * w + (row >> 3), u = u0 + (row & 7);
          const int nvs = (V + VT - 1) / VT;
          a.zmax[(((size_t)b * d.Tpad + t) * d.U1pad + u) * nvs + vt / VT] = mr;
        }
        wait_lgkm0();  // this wave's rows are in LDS (read back by the same wave)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // rows acc_row(4i + j, kh) = 8i + 4kh + j
          const f32x4 m4 = *reinterpret_cast<const f32x4*>(&zm_row[w][8 * i + 4 * kh]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) acc[blk][4 * i + j] -= m4[j];
        }
      }
      if constexpr (kBf16) {
        // accumulator columns -> Ts[col][row] (8-byte writes of 4 rows) ...
        uint16_t* ts = Ts[w];
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
          const int col = blk * 32 + lc;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[blk][4 * i], acc[blk][4 * i + 1]);
            pk.y = pack_bf16x2(acc[blk][4 * i + 2], acc[blk][4 * i + 3]);
            *reinterpret_cast<uint2*>(&ts[ts_idx(col, 8 * i + 4 * kh)]) = pk;
          }
        }
        // Ts[w] is this wave's own: its writes are complete once the wave's
        // LDS counter drains, no workgroup barrier needed
        wait_lgkm0();
        if constexpr (MODE == kGrad) {
          // one-hot terms: lane lc of the first half fixes row lc
          if (kh == 0) {
            const int rowi = w * 32 + lc;
            if (d.blank >= vt && d.blank < vt + VT) {
              uint16_t* p = &ts[ts_idx(d.blank - vt, lc)];
              *p = f32_to_bf16_hw(bf16_to_f32(*p) - row_b[rowi]);
            }
            const int y = lab_row;
            if (y >= vt && y < vt + VT) {
              uint16_t* p = &ts[ts_idx(y - vt, lc)];
              *p = f32_to_bf16_hw(bf16_to_f32(*p) - row_e[rowi]);
            }
          }
          wait_lgkm0();
        }
        // ... then rows: each lane gets 8 consecutive columns of row l%32.
        // A transposing read hands a lane data addressed by the other lanes
        // of its 16-lane group, so every lane takes part in the reads; only
        // the stores are limited to lattice cells.
        const int row = lc;
        const int t = t0 + 4 * w + (row >> 3), u = u0 + (row & 7);
        const bool row_ok = t < Tl && u <= Ul;
        // logits: cells of the lattice only; logit gradients: every row of
        // the tile (zero outside the lattice), as the weight gradient reads
        // whole tiles
        const bool row_st = MODE == kGrad || row_ok;
        T* orow = out + (((size_t)b * RT + (row_st ? t - rt0 : 0)) * RU + (row_st ? u - ru0 : 0)) * ldz +
                  (vt - zc0);
        const int g = lane >> 4, i = lane & 15;
#pragma unroll
        for (int f = 0; f < VT / 16; ++f) {
          const int k0 = 16 * f + 8 * (g >> 1) + (i >> 2);
          const int cb = 16 * (g & 1) + 4 * (i & 3);
          const i16x4 lo =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&ts[ts_idx(k0, cb)]));
          const i16x4 hi =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&ts[ts_idx(k0 + 4, cb)]));
          const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo), hi2 = __builtin_bit_cast(u32x2_t, hi);
          u32x4 pk = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          const int colo = 16 * f + 8 * kh;
          if (!row_ok) pk = u32x4{0u, 0u, 0u, 0u};
          if (row_st && (EXACT || vt + colo < V)) *reinterpret_cast<u32x4*>(orow + colo) = pk;
        }
        // Ts is rewritten only after the next tile's slice barriers
      } else {
        // fp32: 32 lanes store 32 consecutive columns of a row (128 B)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rowi = w * 32 + acc_row(r, kh);
          const int t = t0 + 4 * w + (r >> 2), u = u0 + 4 * kh + (r & 3);
          const bool ok = t < Tl && u <= Ul;
          if (MODE == kGrad || ok) {
            T* orow = out + (((size_t)b * RT + (t - rt0)) * RU + (u - ru0)) * ldz;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) {
              const int col = vt + blk * 32 + lc;
              if (cvalid[blk]) {
                float g = acc[blk][r];
                if constexpr (MODE == kGrad) {
                  if (col == d.blank) g -= row_b[rowi];
                  if (col == lab[r & 3]) g -= row_e[rowi];
                  g = ok ? g : 0.f;
                }
                orow[col - zc0] = g;
              }
            }
          }
        }
      }
    }
  }
  pre = next_ns > 0;  // the last slice started the next item's first copy

  if constexpr ((MODE == kLse || MODE == kStoreZ) && NBLK == 2) {
    __syncthreads();  // captures visible
    if (lc < 16) {
      const int r = rs_row(lc);
      const int rowi = w * 32 + acc_row(r, kh);
      const int t = t0 + 4 * w + (r >> 2), u = u0 + 4 * kh + (r & 3);
      if (t < Tl && u <= Ul) {
        const float lse = ((bounded ? 0.f : mrow) + __builtin_amdgcn_logf(srow)) * kLn2;
        const size_t ix = skew_idx(d, b, t, u);
        float lb = cap_blank[rowi] - lse, le = (u < Ul) ? cap_label[rowi] - lse : 0.f;
        if (MODE == kLse && a.band > 0) band_mask(a, b, t, u, Tl, Ul, lb, le);
        a.lse[ix] = lse;
        a.LB[ix] = lb;
        a.LE[ix] = le;
      }
    }
  }
  if constexpr ((MODE == kLse || MODE == kStoreZ) && NBLK == 4) {
    // combine the per-lane partial sums of the 32 lanes that share each row
    if (bounded) {
#pragma unroll
      for (int off = 1; off < 32; off <<= 1)
#pragma unroll
        for (int r = 0; r < 16; ++r) srun[r] += __shfl_xor(srun[r], off);
#pragma unroll
      for (int r = 0; r < 16; ++r) mrun[r] = 0.f;
    } else {
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
        float lb = cap_blank[rowi] - lse, le = (u < Ul) ? cap_label[rowi] - lse : 0.f;
        if (MODE == kLse && a.band > 0) band_mask(a, b, t, u, Tl, Ul, lb, le);
        a.lse[ix] = lse;
        a.LB[ix] = lb;
        a.LE[ix] = le;
      }
    }
  }
  // the next item rewrites the captures, row constants and store staging
  __syncthreads();
  if constexpr (NCH > 1) {
    // every wave is done with this item's exponential rows
    if (stage_ep && item + (int)gridDim.x < n_items) {
      int nb, nt0, nu0;
      item_tile(item + gridDim.x, nb, nt0, nu0);
      issue_ep(nb, nt0, nu0);
    }
  }
  }  // item loop
}

// ------------------------------------------------------------------ dispatch

// compute units of the current device
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// bf16 with H <= 256: 64-column vocabulary steps and two workgroups per
// compute unit (the MFMA work of one overlaps the other's h build,
// exponentials, stores and slice barriers), which fits the registers of a
// two-wave-per-SIMD launch only while the h fragments of a wave take at most
// 64 of them; otherwise 128-column steps, one workgroup per compute unit
template <typename T, int KS>
constexpr int kJointBlocks = (sizeof(T) == 2 && KS <= 16) ? 2 : 4;

int joint_vocab_step(bool bf16, int H) {
  const int nks = (H + 15) / 16;
  return (bf16 && nks <= 16) ? 32 * 2 : 32 * 4;  // kJointBlocks<T, KS> 32-column blocks
}

template <typename T, int KS, int MODE>
static void launch_ks(const JointArgs& a, int n_items, hipStream_t st) {
  constexpr int NB = kJointBlocks<T, KS>;
  using C = StageCfg<T, NB>;
  const bool exact = a.d.H / 16 == KS && a.d.H % C::BK == 0 && a.d.V % C::VT == 0;
  const int slots = device_cu_count() * C::OCC;
  const dim3 grid(n_items < slots ? n_items : slots);
  if (exact)
    hipLaunchKernelGGL((joint_tile_kernel<T, KS, MODE, true, NB>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((joint_tile_kernel<T, KS, MODE, false, NB>), grid, dim3(256), 0, st, a);
}

template <typename T, int MODE>
static hipError_t launch_mode(const JointArgs& a, int n_items, hipStream_t st) {
  const int nks = a.d.H / 16;
  if constexpr (std::is_same<T, float>::value) {
    if (nks <= 4) launch_ks<T, 4, MODE>(a, n_items, st);
    else if (nks <= 8) launch_ks<T, 8, MODE>(a, n_items, st);
    else if (nks <= 16) launch_ks<T, 16, MODE>(a, n_items, st);
    else if (nks <= 32) launch_ks<T, 32, MODE>(a, n_items, st);
    else if (nks <= 48) launch_ks<T, 48, MODE>(a, n_items, st);
    else return hipErrorInvalidValue;
  } else {
    if (nks <= 8) launch_ks<T, 8, MODE>(a, n_items, st);
    else if (nks <= 16) launch_ks<T, 16, MODE>(a, n_items, st);
    else if (nks <= 32) launch_ks<T, 32, MODE>(a, n_items, st);
    else if (nks <= 40) launch_ks<T, 40, MODE>(a, n_items, st);
    else if (nks <= 48) launch_ks<T, 48, MODE>(a, n_items, st);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_joint_tile(const JointArgs& a, int mode, bool bf16, int n_items,
                             hipStream_t st) {
  if (n_items <= 0 || a.d.B <= 0) return hipSuccess;
  if (bf16) {
    if (mode == kLse) return launch_mode<uint16_t, kLse>(a, n_items, st);
    if (mode == kStoreZ) return launch_mode<uint16_t, kStoreZ>(a, n_items, st);
    return launch_mode<uint16_t, kGrad>(a, n_items, st);
  }
  if (mode == kLse) return launch_mode<float, kLse>(a, n_items, st);
  if (mode == kStoreZ) return launch_mode<float, kStoreZ>(a, n_items, st);
  return launch_mode<float, kGrad>(a, n_items, st);
}

}  // namespace rnntj
