// Kernel launch interfaces used by the C ABI (api.cpp).  Device code only
// sees plain pointers and the Dims struct.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace rnntj {

enum JointMode { kLse = 0, kStoreZ = 1, kGrad = 2 };

// Header of the forward -> backward state (int32 words): [0] data-error mask,
// [1] flags, [2] float bits of max_v (sum_k |W_out[k,v]| + |b_out[v]|), an
// upper bound on every |z| since |h| <= 1.
constexpr int kFlagEpBad = 1;     // some finite |enc| or |pred| > 40
constexpr int kFlagConsumed = 2;  // an untiled backward turned the stored logits into dz
// data-error bit: a backward found its logits already consumed by another
constexpr int kErrConsumed = 4;
// data-error bit: a backward's sizes, dtype, blank or mode do not match the
// forward that wrote the state; that backward then computes nothing
constexpr int kErrPlan = 8;
// Header words 4 and 5 hold the forward's plan tag and whether the state
// carries logits (untiled); word 6 is set by a backward that refuses the
// state (every later kernel of that backward returns at once).
constexpr int kHdrWords = 8;
constexpr int kHdrRefuse = 6;
// Header word 7: the pruning window S of a pruned forward (0: the full lattice).
constexpr int kHdrBand = 7;
// data-error bit: no band of pruning windows holds an alignment of the
// utterance (U' > T' (S - 1)); it is then treated as invalid
constexpr int kErrPruneInfeasible = 16;

// Active-tile lists.  A lattice chunk (frames ct0 .. ct0+CT-1, label
// positions cu0 .. cu0+CU-1) is covered by 16 x 8 cell tiles; a tile is
// active when it holds at least one cell t < T'_b, u <= U'_b.  The active
// tiles of chunk c are list[c * cap + i], i < count[c], utterance by
// utterance, each packed into the 32 bits of an int32 entry as
// b << 19 | tt << 7 | tu (tile row / column inside the chunk): 13 bits of
// utterance (B <= 8191), 12 of 16-frame tile row (T <= 65520), 7 of 8-label
// tile column (U + 1 <= 1024).
__host__ __device__ inline int tile_pack(int b, int tt, int tu) {
  return (int)(((uint32_t)b << 19) | ((uint32_t)tt << 7) | (uint32_t)tu);
}
__device__ inline void tile_unpack(int v, int& b, int& tt, int& tu) {
  const uint32_t x = (uint32_t)v;
  b = (int)(x >> 19);
  tt = (int)((x >> 7) & 0xfffu);
  tu = (int)(x & 127u);
}
// With a pruned forward's state (hdr[kHdrBand] = S > 0) only tiles holding a
// cell of the band s_t <= u <= s_t + S - 1 (bounds [B, T]) are listed.
hipError_t launch_tile_list(const int32_t* Teff, const int32_t* Ueff, const Dims& d, int CT, int CU,
                            int n_chunks_u, int n_chunks, int cap, int32_t* list, int32_t* count,
                            const int32_t* hdr, const int32_t* bounds, hipStream_t st);

struct JointArgs {
  const void* enc;
  const void* pred;
  const void* Wt;     // W_out transposed, [V, H], dtype
  const void* bias;   // [V], dtype
  const int32_t* labels;
  const int32_t* Teff;  // validated lengths (0 frames = invalid utterance)
  const int32_t* Ueff;
  int32_t* hdr;         // state header (data-error mask, flags, logit bound)
  const float* Eexp;    // e^{2 enc} [B, T, H]
  const float* Pexp;    // e^{2 pred} [B, U+1, H]
  Dims d;
  const int32_t* tiles;       // active tiles of this chunk
  const int32_t* tile_count;  // number of entries in `tiles`
  int vsplit;    // kGrad: vocabulary tiles split over this many workgroups
  int ct0, cu0;  // chunk origin (frame, label position)
  int CT, CU;    // chunk extents, multiples of kTileT / kTileU
  int n_tu;      // CU / kTileU
  // forward outputs (diagonal-skewed per-cell scalars)
  float* lse;
  float* LB;
  float* LE;
  void* zout;  // kStoreZ: logits [B, Tpad, U1pad, V]
  // kStoreZ, bf16: the logits are stored as bf16(z - M), M the row's largest
  // logit within each vocabulary step of `zstep` columns, and M (float32) in
  // zmax [B, Tpad, U1pad, ceil(V / zstep)]; read back as stored + M
  float* zmax;
  int zstep;
  // kLse of a pruned forward: window starts [B, T] and width band (0: none);
  // steps that leave the band get log-probability -inf
  const int32_t* bounds;
  int band;
  // backward inputs / output
  const double* alpha;
  const double* beta;
  const double* logP;
  const float* gcost;  // [B] or null
  // kGrad: the vocabulary part [gv0, gv0 + gvw) of this launch (gv0 a
  // multiple of the vocabulary step); gout rows have stride gld
  int gv0, gvw, gld;
  void* gout;          // kGrad: logit gradients [B, CT, CU, gld] of the part
  void* hout;          // kGrad: joint activations h [B, CT, CU, H]; kStoreZ: the h rows
                       // [B, Tpad, U1pad, H] of the active tiles, or null
};

// Vocabulary columns of one step of the forward joint kernel for this dtype
// and hidden size (the granularity of JointArgs::zmax).
int joint_vocab_step(bool bf16, int H);

// Persistent launch: `n_items` = (maximum number of active tiles) * vsplit
// bounds the work; the workgroups loop over the items the tile list holds.
hipError_t launch_joint_tile(const JointArgs& a, int mode, bool bf16, int n_items,
                             hipStream_t st);

// Length / label validation: writes Teff/Ueff (0 / 0 for an invalid
// utterance), ORs a bit mask into status[0] and stores the criterion
// (kCritSum / kCritMax) in status[3].
hipError_t launch_validate(const int32_t* T_lens, const int32_t* U_lens,
                           const int32_t* labels, const Dims& d, int32_t* Teff,
                           int32_t* Ueff, int32_t* status, int crit, int32_t tag,
                           int has_logits, int band, hipStream_t st);
// Backward's first check of the state header (see kErrPlan).
hipError_t launch_guard(int32_t* hdr, int32_t tag, int need_logits, hipStream_t st);

// One launch: Wt[V, H] = W_out transposed; Wb = W_out in blocks of 32
// vocabulary columns, [ceil(V / 32), H, 32], columns past V zero (each slice
// row that dh copies is then contiguous); Eexp = e^{2 enc}, Pexp = e^{2 pred}
// (float32), hdr[1] |= kFlagEpBad if some finite |enc| or |pred| exceeds 40;
// hdr[2] = max(hdr[2], bits of max_v sum_k |W[k,v]| + |b[v]|), hdr[2] zero on entry.
hipError_t launch_prep(const void* enc, const void* pred, const void* W, const void* bias,
                       bool bf16, const Dims& d, void* Wt, void* Wb, float* Eexp, float* Pexp,
                       int32_t* hdr, hipStream_t st);

// Pruning bounds of the pruned transducer loss (pruned.hip): the simple
// joiner's lattice in float64 and the window start of every frame.
struct PruneArgs {
  const void* enc;
  const void* pred;
  const void* W;     // W_out [H, V]
  const void* bias;  // b_out [V]
  bool bf16;
  const int32_t* labels;
  int32_t* Teff;     // zeroed for an utterance no band can hold
  int32_t* Ueff;
  int32_t* status;   // kErrPruneInfeasible
  Dims d;
  int S;
  // float64 workspace
  double* am;        // [B, T, V]
  double* lm;        // [B, U+1, V]
  double* ma;        // [B, T]
  double* ml;        // [B, U+1]
  double* amB;       // [B, T]
  double* amY;       // [B, T, U]
  double* lmB;       // [B, U+1]
  double* lmY;       // [B, U+1]
  double* LBs;       // diagonal-skewed [B, T+U, U+1]
  double* LEs;
  double* alpha;
  double* beta;
  double* logPs;     // [B]
  double* centres;   // [B, T]
  // outputs
  float* simple_costs;  // [B] or null
  int32_t* bounds;      // [B, T]
};
hipError_t launch_pruning_bounds(const PruneArgs& p, hipStream_t st);
// p[i] = v for i < n
hipError_t launch_fill(float* p, size_t n, float v, hipStream_t st);

// Largest U + 1: the lattice sweep blocks up to 16 label positions on each
// lane of one wave (and alpha / beta carry one trash slot per position past
// their cells); the token-and-duration and simple-joiner lattices put one
// thread on each label position of a 512-thread workgroup.
constexpr int kMaxU1 = 1024;
constexpr int kMaxU1Short = 512;

// Token-and-duration transducer (tdt.hip).  Up to kTdtMaxK durations, each
// in [0, kTdtMaxDur].
constexpr int kTdtMaxK = 8;
constexpr int kTdtMaxDur = 15;
struct TdtArgs {
  Dims d;
  bool bf16;
  const void* enc;
  const void* pred;
  const void* Wd;  // W_dur [H, K]
  const void* bd;  // b_dur [K]
  int K;
  int dur[kTdtMaxK];
  const int32_t* Teff;
  const int32_t* Ueff;
  const int32_t* hdr;
  const float* Eexp;
  const float* Pexp;
  const float* LB;   // token head (diagonal-skewed)
  const float* LE;
  float* LD;         // duration log-probabilities [cells, K]
  double* alpha;
  double* beta;
  double* logP;
  float* costs;
  const float* gcost;
  double* gB;        // backward: summed step posteriors per cell
  double* gE;
  float* dzd;        // backward: duration-logit gradients [cells, K]
  float* d_enc;
  float* d_pred;
  float* d_Wd;
  float* d_bd;
  // deterministic mode (both set): the duration-head backward stores each
  // frame block's d_W_dur / d_b_dur sums here ([blocks, H, K], [blocks, K];
  // blocks = B ceil(T / kTdtFrames)) instead of adding them with atomics,
  // and d_pred is formed by a pass with one writer per element
  float* part_w;
  float* part_b;
};
constexpr int kTdtFrames = 16;  // frames per block of the duration-head backward
hipError_t launch_tdt_dur_head(const TdtArgs& a, hipStream_t st);
hipError_t launch_tdt_lattice(const TdtArgs& a, hipStream_t st);
hipError_t launch_tdt_post(const TdtArgs& a, hipStream_t st);
hipError_t launch_tdt_dur_bwd(const TdtArgs& a, hipStream_t st);

// Fill n floats / int32s with zero (a kernel, never a memset node); the
// four-buffer form zeroes up to four (null pointers skipped) in one launch.
hipError_t launch_zero(void* p, size_t n_words, hipStream_t st);
hipError_t launch_zero4(void* p0, size_t n0, void* p1, size_t n1, void* p2, size_t n2, void* p3,
                        size_t n3, hipStream_t st);

// Alpha / beta recursion over the anti-diagonals; costs[b] = -logP.  With
// kCritMax: the max-plus alpha and, in beta, each cell's predecessor decision,
// which launch_backtrace turns into the best alignment's step marks (read by
// cell_posteriors).
hipError_t launch_lattice(const float* LB, const float* LE, const int32_t* Teff,
                          const int32_t* Ueff, const Dims& d, double* alpha, double* beta,
                          double* logP, float* costs, int crit, hipStream_t st);
hipError_t launch_backtrace(const int32_t* Teff, const int32_t* Ueff, const Dims& d, double* beta,
                            hipStream_t st);


// dh = dz @ W_out^T for the active tiles of one chunk; dpre = (1 - h^2) dh
// summed into d_enc over u and into d_pred over t.
// Compute units of the current device (persistent launches use one or two
// workgroups per unit).
int device_cu_count();

struct DhArgs {
  const void* g;      // [B, CT, CU, ldg] logit gradients of the chunk's vocabulary part
  const void* W;      // W_out in 32-column blocks [ceil(V / 32), H, 32] (launch_prep's Wb)
  const void* enc;
  const void* pred;
  const int32_t* Teff;
  const int32_t* Ueff;
  const int32_t* hdr;
  const float* Eexp;
  const float* Pexp;
  Dims d;
  const int32_t* tiles;       // active tiles of the chunk
  const int32_t* tile_count;
  const float* gcost;         // [B] or null
  int ct0, cu0, CT, CU;
  int ksplit;                 // vocabulary parts per (tile, hidden block); divides the slice count
  int v0, vw, ldg;            // vocabulary part [v0, v0 + vw) of g (row stride ldg) and W_out
  float* d_enc;
  float* d_pred;
  // deterministic reductions (both set, ksplit 1): each tile's d_enc rows
  // [tiles, 16, H] and d_pred rows [tiles, 8, H] are stored here instead of
  // being added with atomics; launch_dh_reduce then adds them, each sum in a
  // fixed order
  float* enc_part;
  float* pred_part;
};
// Persistent launch; max_tiles bounds the entries of the tile list.
hipError_t launch_dh(const DhArgs& a, bool bf16, int max_tiles, hipStream_t st);


// Untiled backward: the stored logits [B, Tpad, U1pad, V] of the active tiles
// become the logit gradients (same type), rows outside the lattice zero; a.hdr
// must point at the (writable) state header.  One workgroup per list entry.
hipError_t launch_grad_inplace(void* z, bool bf16, const JointArgs& a, int max_tiles,
                               hipStream_t st);

// d_W_out += h^T dz and d_b64 += column sums of dz (float64) over the active
// tiles of one chunk (split-K over the tile list).
struct DwArgs {
  const void* g;              // dz rows [B, CT, CU, ldg] of the vocabulary part
  const void* h;              // h rows [B, CT, CU, H]; rows of cells outside the lattice are 0
  const int32_t* tiles;       // active tiles of the chunk
  const int32_t* tile_count;
  Dims d;
  int ct0, cu0, CT, CU;
  int kparts;                 // split-K: parts of the tile list
  int v0, vw, ldg;            // vocabulary part [v0, v0 + vw): columns of g (row stride ldg)
  const int32_t* hdr;         // state header (refusal word)
  float* d_W;
  double* d_b64;
  // deterministic reductions (both set): split-K part kp stores its sums in
  // w_part [kparts, H, V] and b_part [kparts, V] instead of adding them with
  // atomics; launch_dw_reduce then adds the parts in order
  float* w_part;
  double* b_part;
};
hipError_t launch_dh_reduce(const DhArgs& a, int max_tiles, hipStream_t st);
hipError_t launch_dw_reduce(const DwArgs& a, hipStream_t st);
hipError_t launch_dw(const DwArgs& a, bool bf16, hipStream_t st);

// d_b[v] = (float) db64[v]; with `mark` (the state header of an untiled
// backward) also sets kFlagConsumed in mark[1].
hipError_t launch_db_finalize(const double* db64, float* d_b, int V, int32_t* mark,
                              hipStream_t st);

// Joint input projections (proj.hip), row-major operands, fp32 accumulation:
//   y[M,N] = x[M,K] W[K,N] + b[N] in the operand type;
//   dx[M,K] = dy[M,N] W^T (fp32, stored);
//   dW[K,N] += x^T dy and db[N] += column sums of dy (fp32 atomics: dW and
//   db must be zeroed first).
// K and N multiples of 16.
hipError_t launch_proj_fwd(const void* x, const void* W, const void* b, bool bf16, int M, int K,
                           int N, void* y, hipStream_t st);
hipError_t launch_proj_dx(const float* dy, const void* W, bool bf16, int M, int K, int N,
                          float* dx, hipStream_t st);
hipError_t launch_proj_dw(const void* x, const float* dy, bool bf16, int M, int K, int N,
                          float* dW, float* db, int cus, bool in_order, hipStream_t st);

}  // namespace rnntj
