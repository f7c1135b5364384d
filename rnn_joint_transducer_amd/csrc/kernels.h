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

// Active-tile lists.  A lattice chunk (frames ct0 .. ct0+CT-1, label
// positions cu0 .. cu0+CU-1) is covered by 16 x 8 cell tiles; a tile is
// active when it holds at least one cell t < T'_b, u <= U'_b.  The active
// tiles of chunk c are list[c * cap + i], i < count[c], utterance by
// utterance, each packed as b << 18 | tt << 6 | tu (tile row / column inside
// the chunk).
__host__ __device__ inline int tile_pack(int b, int tt, int tu) { return (b << 18) | (tt << 6) | tu; }
__device__ inline void tile_unpack(int v, int& b, int& tt, int& tu) {
  b = v >> 18;
  tt = (v >> 6) & 0xfff;
  tu = v & 63;
}
hipError_t launch_tile_list(const int32_t* Teff, const int32_t* Ueff, const Dims& d, int CT, int CU,
                            int n_chunks_u, int n_chunks, int cap, int32_t* list, int32_t* count,
                            hipStream_t st);

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
  // backward inputs / output
  const double* alpha;
  const double* beta;
  const double* logP;
  const float* gcost;  // [B] or null
  void* gout;          // kGrad: logit gradients [B, CT, CU, V]
  void* hout;          // kGrad: joint activations h [B, CT, CU, H]; kStoreZ: the h rows
                       // [B, Tpad, U1pad, H] of the active tiles, or null
};

// Persistent launch: `n_items` = (maximum number of active tiles) * vsplit
// bounds the work; the workgroups loop over the items the tile list holds.
hipError_t launch_joint_tile(const JointArgs& a, int mode, bool bf16, int n_items,
                             hipStream_t st);

// Length / label validation: writes Teff/Ueff (0 / 0 for an invalid
// utterance), ORs a bit mask into status[0] and stores the criterion
// (kCritSum / kCritMax) in status[3].
hipError_t launch_validate(const int32_t* T_lens, const int32_t* U_lens,
                           const int32_t* labels, const Dims& d, int32_t* Teff,
                           int32_t* Ueff, int32_t* status, int crit, hipStream_t st);

// One launch: Wt[V, H] = W_out transposed; Eexp = e^{2 enc}, Pexp = e^{2 pred}
// (float32), hdr[1] |= kFlagEpBad if some finite |enc| or |pred| exceeds 40;
// hdr[2] = max(hdr[2], bits of max_v sum_k |W[k,v]| + |b[v]|), hdr[2] zero on entry.
hipError_t launch_prep(const void* enc, const void* pred, const void* W, const void* bias,
                       bool bf16, const Dims& d, void* Wt, float* Eexp, float* Pexp,
                       int32_t* hdr, hipStream_t st);

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
  const void* g;      // [B, CT, CU, V] logit gradients of the chunk
  const void* W;      // [H, V]
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
  float* d_enc;
  float* d_pred;
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
  const void* g;              // dz rows [B, CT, CU, V]
  const void* h;              // h rows [B, CT, CU, H]; rows of cells outside the lattice are 0
  const int32_t* tiles;       // active tiles of the chunk
  const int32_t* tile_count;
  Dims d;
  int ct0, cu0, CT, CU;
  int kparts;                 // split-K: parts of the tile list
  float* d_W;
  double* d_b64;
};
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
                          float* dW, float* db, int cus, hipStream_t st);

}  // namespace rnntj
