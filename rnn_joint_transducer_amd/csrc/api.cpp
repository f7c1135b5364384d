// C ABI of the fused RNN-T joint + transducer loss (see include/rnnt_joint.h).
//
// Host side only: argument checks, carving of the caller's `saved` and
// `workspace` buffers, and the launch sequence.  Every step of the
// computation runs in the HIP kernels of this library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rnnt_joint.h"
#include "kernels.h"

using namespace rnntj;

namespace {

constexpr size_t kAlign = 256;
// Longest padded time axis of the pruned forward (its window starts of one
// utterance are kept in 64 KB of LDS as 16-bit values)
constexpr int kMaxPrunedT = 32000;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// process-wide switches (rnnt_joint_loss_set_flags), first read from the
// environment: RNNTJ_DEBUG=1, RNNTJ_DETERMINISTIC=1
int env_flags() {
  auto on = [](const char* n) {
    const char* v = getenv(n);
    return v && v[0] && !(v[0] == '0' && v[1] == 0);
  };
  return (on("RNNTJ_DEBUG") ? RNNTJ_FLAG_DEBUG : 0) |
         (on("RNNTJ_DETERMINISTIC") ? RNNTJ_FLAG_DETERMINISTIC : 0);
}
std::atomic<int> g_flags{env_flags()};
inline bool debug_on() { return (g_flags.load() & RNNTJ_FLAG_DEBUG) != 0; }
inline bool deterministic_on() { return (g_flags.load() & RNNTJ_FLAG_DETERMINISTIC) != 0; }

struct Plan {
  Dims d;
  bool bf16;
  bool untiled;
  int CT, CU;  // backward chunk extents
  int Vp;      // vocabulary columns per part of the tiled backward
  size_t elem;
  // saved layout (byte offsets)
  size_t o_h;  // untiled: h rows [B, Tpad, U1pad, H]
  size_t o_wb;  // W_out in 32-column blocks [ceil(V / 32), H, 32] (dh's copies)
  size_t o_status, o_teff, o_ueff, o_logp, o_wt, o_lse, o_lb, o_le, o_alpha, o_beta, o_E, o_P,
      o_tiles, o_tcount, o_z;
  size_t o_zm;  // untiled bf16: the per-(row, vocabulary step) logit offsets
  size_t o_bounds;  // pruning window starts [B, T] int32 (written by a pruned forward)
  // pruned forward workspace (float64 simple-joiner lattice; byte offsets)
  size_t o_pw_am, o_pw_lm, o_pw_ma, o_pw_ml, o_pw_amB, o_pw_amY, o_pw_lmB, o_pw_lmY, o_pw_LB,
      o_pw_LE, o_pw_alpha, o_pw_beta, o_pw_logP, o_pw_centres, ws_pruned;
  int zstep;    // vocabulary columns per forward step (the offsets' granularity)
  size_t saved_bytes;
  size_t ws_fwd, ws_bwd;
  size_t o_ws_db, o_ws_g, o_ws_h, o_ws_tiles, o_ws_tcount;  // backward workspace layout
  int cap_all;                // active-tile list capacity of the whole lattice
  int n_cu_chunks, n_chunks;  // backward chunk grid (tiled mode)
  int cap_chunk;              // active-tile list capacity of one chunk
  // deterministic mode: extra backward workspace and the fixed split-K count
  size_t o_ws_encp, o_ws_predp, o_ws_wpart, o_ws_bpart, ws_bwd_det;
  int kparts_det;
  size_t bwd_ws() const { return deterministic_on() ? ws_bwd_det : ws_bwd; }
  // tiled: bytes of a second chunk buffer pair (logit gradients, h rows),
  // placed after the rest of a backward workspace of `need` bytes; with it
  // consecutive chunks alternate buffers and a chunk's dW overlaps the next
  // chunk's logit gradients
  size_t ws_g = 0, ws_h = 0;
  size_t overlap_bytes(size_t need) const {
    return untiled ? need : align_up(need) + ws_g + ws_h;
  }
};

int make_plan(int B, int T, int U, int H, int V, int dtype, int tile_t, int tile_u, int tile_v,
              Plan* p) {
  if (B < 1 || T < 1 || U < 0 || H < 1 || V < 1) return RNNTJ_ERR_ARG;
  if (dtype != RNNTJ_F32 && dtype != RNNTJ_BF16) return RNNTJ_ERR_ARG;
  if (tile_t < 0 || tile_u < 0 || tile_v < 0) return RNNTJ_ERR_ARG;
  const bool bf16 = dtype == RNNTJ_BF16;
  if (H % 16 != 0 || H > 768) return RNNTJ_ERR_UNSUPPORTED;
  if (V % 8 != 0 || V < 8 || V > kMaxV) return RNNTJ_ERR_UNSUPPORTED;
  if (U + 1 > kMaxU1) return RNNTJ_ERR_UNSUPPORTED;
  if (B > 8191 || T > 65520) return RNNTJ_ERR_UNSUPPORTED;  // packed tile coordinates
  if (tile_t % kTileT != 0 || tile_u % kTileU != 0) return RNNTJ_ERR_UNSUPPORTED;
  // tile_v: vocabulary columns of one part of the tiled backward (and an
  // upper bound on the columns of one online log-sum-exp step, which steps
  // by at most kVocabTile); 0 = the whole vocabulary
  if (tile_v % kVocabTile != 0) return RNNTJ_ERR_UNSUPPORTED;
  Plan& q = *p;
  q.bf16 = bf16;
  q.elem = bf16 ? 2 : 4;
  q.d.B = B;
  q.d.T = T;
  q.d.U = U;
  q.d.H = H;
  q.d.V = V;
  q.d.blank = 0;
  q.d.U1 = U + 1;
  q.d.DG = T + U;
  q.d.Tpad = (T + kTileT - 1) / kTileT * kTileT;
  q.d.U1pad = (U + 1 + kTileU - 1) / kTileU * kTileU;
  q.untiled = (tile_t == 0 && tile_u == 0);
  q.CT = q.untiled ? q.d.Tpad : (tile_t ? (tile_t < q.d.Tpad ? tile_t : q.d.Tpad) : q.d.Tpad);
  q.CU = q.untiled ? q.d.U1pad : (tile_u ? (tile_u < q.d.U1pad ? tile_u : q.d.U1pad) : q.d.U1pad);
  // tiled backward: each chunk's vocabulary in parts of Vp columns, whose
  // logit gradients alone are held at once
  q.Vp = (q.untiled || tile_v == 0 || tile_v >= V) ? V : tile_v;
  const size_t cells = (size_t)B * q.d.DG * q.d.U1;
  size_t o = 0;
  q.o_status = o; o = align_up(o + 4 * kHdrWords);
  q.o_teff = o;   o = align_up(o + 4 * (size_t)B);
  q.o_ueff = o;   o = align_up(o + 4 * (size_t)B);
  q.o_logp = o;   o = align_up(o + 8 * (size_t)B);
  q.o_wt = o;     o = align_up(o + q.elem * (size_t)H * V);
  q.o_wb = o;     o = align_up(o + q.elem * (size_t)H * ((V + 31) / 32 * 32));
  q.o_lse = o;    o = align_up(o + 4 * cells);
  q.o_lb = o;     o = align_up(o + 4 * cells);
  q.o_le = o;     o = align_up(o + 4 * cells);
  // alpha / beta carry a trash area of kMaxU1 float64 past the cells (slots
  // of the lattice sweep that fall outside the lattice are stored there)
  q.o_alpha = o;  o = align_up(o + 8 * (cells + kMaxU1));
  q.o_beta = o;   o = align_up(o + 8 * (cells + kMaxU1));
  q.o_E = o;      o = align_up(o + 4 * (size_t)B * T * H);
  q.o_P = o;      o = align_up(o + 4 * (size_t)B * (U + 1) * H);
  q.cap_all = B * (q.d.Tpad / kTileT) * (q.d.U1pad / kTileU);
  q.o_tiles = o;  o = align_up(o + 4 * (size_t)q.cap_all);
  q.o_tcount = o; o = align_up(o + 16);
  q.o_z = o;
  if (q.untiled) o = align_up(o + q.elem * (size_t)B * q.d.Tpad * q.d.U1pad * V);
  // untiled: the forward keeps the h rows of the padded lattice for dW
  q.o_h = o;
  if (q.untiled) o = align_up(o + q.elem * (size_t)B * q.d.Tpad * q.d.U1pad * H);
  // untiled bf16: float32 offset of every row's stored logits per vocabulary step
  q.zstep = joint_vocab_step(bf16, H);
  q.o_zm = o;
  if (q.untiled && bf16)
    o = align_up(o + 4 * (size_t)B * q.d.Tpad * q.d.U1pad * ((V + q.zstep - 1) / q.zstep));
  q.o_bounds = o;
  o = align_up(o + 4 * (size_t)B * T);
  q.saved_bytes = o;
  q.ws_fwd = 0;
  {
    size_t w = 0;
    auto put = [&](size_t& off, size_t n) {
      off = w;
      w = align_up(w + 8 * n);
    };
    const size_t rt = (size_t)B * T, ru = (size_t)B * (U + 1);
    put(q.o_pw_am, rt * V);
    put(q.o_pw_lm, ru * V);
    put(q.o_pw_ma, rt);
    put(q.o_pw_ml, ru);
    put(q.o_pw_amB, rt);
    put(q.o_pw_amY, rt * (U > 0 ? U : 1));
    put(q.o_pw_lmB, ru);
    put(q.o_pw_lmY, ru);
    put(q.o_pw_LB, cells);
    put(q.o_pw_LE, cells);
    put(q.o_pw_alpha, cells);
    put(q.o_pw_beta, cells);
    put(q.o_pw_logP, B);
    put(q.o_pw_centres, rt);
    q.ws_pruned = w;
  }
  // backward workspace: float64 d_b_out accumulator [V], then (tiled) one
  // chunk's logit gradients of one vocabulary part [B, CT, CU, Vp] and its joint activations h
  // [B, CT, CU, H] (untiled: none, the forward keeps h)
  q.n_cu_chunks = (q.d.U1pad + q.CU - 1) / q.CU;
  q.n_chunks = ((q.d.Tpad + q.CT - 1) / q.CT) * q.n_cu_chunks;
  q.cap_chunk = B * (q.CT / kTileT) * (q.CU / kTileU);
  q.o_ws_db = 0;
  q.o_ws_g = align_up(8 * (size_t)V);
  q.ws_g = q.untiled ? 0 : align_up(q.elem * (size_t)B * q.CT * q.CU * q.Vp);
  q.ws_h = q.untiled ? 0 : align_up(q.elem * (size_t)B * q.CT * q.CU * H);
  q.o_ws_h = q.o_ws_g + q.ws_g;
  // (untiled: the h rows are part of the saved state instead)
  q.o_ws_tiles = q.o_ws_h + q.ws_h;
  q.o_ws_tcount = q.o_ws_tiles + (q.untiled ? 0 : align_up(4 * (size_t)q.n_chunks * q.cap_chunk));
  q.ws_bwd = q.o_ws_tcount + (q.untiled ? 0 : align_up(4 * (size_t)q.n_chunks));
  // deterministic reductions: per-tile d_enc / d_pred rows of one chunk and
  // the split-K parts of d_W_out / d_b_out
  {
    const int cap = q.untiled ? q.cap_all : q.cap_chunk;
    const int per = ((H + 127) / 128) * ((q.Vp + 255) / 256);
    int kp = 256 * (bf16 ? 2 : 1) / per;
    kp = kp < 1 ? 1 : (kp > cap ? cap : kp);
    q.kparts_det = kp;
    size_t w = align_up(q.ws_bwd);
    q.o_ws_encp = w;  w = align_up(w + 4 * (size_t)cap * kTileT * H);
    q.o_ws_predp = w; w = align_up(w + 4 * (size_t)cap * kTileU * H);
    q.o_ws_wpart = w; w = align_up(w + 4 * (size_t)kp * H * q.Vp);
    q.o_ws_bpart = w; w = align_up(w + 8 * (size_t)kp * q.Vp);
    q.ws_bwd_det = w;
  }
  return RNNTJ_OK;
}

template <typename P>
inline P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Tag of what a backward must share with the forward that filled `saved`:
// sizes, dtype and blank (FNV-1a over them, kept positive and nonzero).
int32_t plan_tag(const Plan& p, int blank) {
  const int v[7] = {p.d.B, p.d.T, p.d.U, p.d.H, p.d.V, p.bf16 ? 1 : 0, blank};
  uint32_t h = 2166136261u;
  for (int x : v)
    for (int k = 0; k < 4; ++k) {
      h ^= (uint32_t)(x >> (8 * k)) & 0xffu;
      h *= 16777619u;
    }
  h &= 0x7fffffffu;
  return (int32_t)(h ? h : 1);
}

// The duration head of a token-and-duration transducer call (host side).
struct TdtIn {
  const void* Wd;
  const void* bd;
  const int32_t* durations;  // host array of K distinct values in [0, kTdtMaxDur]
  int K;
};
int check_tdt(const TdtIn& t) {
  if (!t.Wd || !t.bd || !t.durations || t.K < 1 || t.K > kTdtMaxK) return RNNTJ_ERR_ARG;
  if (misaligned(t.Wd) || misaligned(t.bd)) return RNNTJ_ERR_ARG;
  bool moves = false;
  for (int j = 0; j < t.K; ++j) {
    const int dj = t.durations[j];
    if (dj < 0 || dj > kTdtMaxDur) return RNNTJ_ERR_UNSUPPORTED;
    for (int i = 0; i < j; ++i)
      if (t.durations[i] == dj) return RNNTJ_ERR_ARG;
    moves = moves || dj >= 1;
  }
  return moves ? RNNTJ_OK : RNNTJ_ERR_ARG;  // a blank needs a duration >= 1
}
// tag of a token-and-duration state: the plan's, mixed with the durations
int32_t tdt_tag(const Plan& p, int blank, const TdtIn& t) {
  uint32_t h = (uint32_t)plan_tag(p, blank) ^ 0x5bd1e995u;
  for (int j = 0; j < t.K; ++j) h = (h ^ (uint32_t)(t.durations[j] + 1)) * 16777619u;
  h = (h ^ (uint32_t)t.K) * 16777619u;
  h &= 0x7fffffffu;
  return (int32_t)(h ? h : 1);
}
size_t tdt_ld_bytes(const Plan& p, int K) {
  return align_up(4 * (size_t)p.d.B * p.d.DG * p.d.U1 * K);
}
// backward workspace of a token-and-duration call: the plain one, then the
// summed step posteriors (float64, two arrays) and the duration-logit
// gradients (float32 [cells, K]); in deterministic mode also the duration
// head's per-frame-block d_W_dur / d_b_dur sums
struct TdtWs {
  size_t gB, gE, dzd, part_w, part_b, total;
};
TdtWs tdt_ws(const Plan& p, int K) {
  const size_t cells = (size_t)p.d.B * p.d.DG * p.d.U1;
  const size_t blocks = (size_t)p.d.B * ((p.d.T + kTdtFrames - 1) / kTdtFrames);
  TdtWs w;
  w.gB = align_up(p.bwd_ws());
  w.gE = w.gB + align_up(8 * cells);
  w.dzd = w.gE + align_up(8 * cells);
  w.part_w = w.dzd + align_up(4 * cells * K);
  w.part_b = w.part_w;
  w.total = w.part_w;
  if (deterministic_on()) {
    w.part_b = w.part_w + align_up(4 * blocks * p.d.H * K);
    w.total = w.part_b + align_up(4 * blocks * K);
  }
  return w;
}

// ---- optional per-kernel event timing (rnnt_joint_loss_timing)
struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimedLaunch> g_timed;

// description of the last failed launch on this thread (rnnt_joint_loss_last_error)
thread_local char g_last_error[256] = "";

hipError_t note_error(const char* name, hipError_t e) {
  if (e != hipSuccess)
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", name, hipGetErrorName(e),
             hipGetErrorString(e));
  return e;
}

// Launch through `launch` (which returns the HIP status of its launches); a
// stale runtime error left by earlier, unrelated HIP calls is cleared first
// so that it is not attributed to this library.
template <class F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  (void)hipGetLastError();
  if (debug_on()) {
    // synchronous checking: every kernel completes (and reports) before
    // the call goes on
    hipError_t e = launch();
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
    return note_error(name, e);
  }
  if (!g_timing) return note_error(name, launch());
  TimedLaunch t{name, nullptr, nullptr};
  if (hipEventCreate(&t.start) != hipSuccess || hipEventCreate(&t.stop) != hipSuccess)
    return note_error(name, hipErrorOutOfMemory);
  hipEventRecord(t.start, st);
  const hipError_t e = launch();
  hipEventRecord(t.stop, st);
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timed.push_back(t);
  return note_error(name, e);
}

void drop_timed() {
  for (auto& t : g_timed) {
    hipEventDestroy(t.start);
    hipEventDestroy(t.stop);
  }
  g_timed.clear();
}

// ---- scratch of rnnt_joint_loss_bwd_noalloc: a static device array (each
// GPU the library runs on holds its own copy until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory; its
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever passed to kernels.
constexpr size_t kScratchBytes = RNNTJ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch on the device of `st` (NULL: the current
// device), which must be the calling thread's current device.
int scratch_for(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RNNTJ_ERR_HIP;
  if (st) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(st, &sd) != hipSuccess) return RNNTJ_ERR_HIP;
    if (sd != dev) return RNNTJ_ERR_ARG;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      note_error("scratch address", e != hipSuccess ? e : hipErrorInvalidSymbol);
      return RNNTJ_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RNNTJ_OK;
}

// ---- side stream of the tiled backward, one per device (default priority,
// not blocking on the null stream).  A chunk's dW GEMM runs on it, so that it
// overlaps that chunk's dh GEMM and the next chunk's logit gradients; events
// fork it from and join it to the caller's stream.  dw_done[k & 1] marks the
// end of the dW of vocabulary pass k.  The lock is held while a backward
// enqueues its chunks, so that two host threads never re-record these events
// at once.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t jg_done[2] = {}, dw_done[2] = {};
  std::mutex mu;
  bool tried = false;
};
SideStream g_side[kMaxDevices];

// The side stream of the current device (NULL if it cannot be created: the
// backward then runs its chunks on the caller's stream alone).
SideStream* side_stream() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& s = g_side[dev];
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!s.tried) {
    s.tried = true;
    bool ok = hipStreamCreateWithFlags(&s.s, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; i < 2 && ok; ++i)
      ok = hipEventCreateWithFlags(&s.jg_done[i], hipEventDisableTiming) == hipSuccess &&
           hipEventCreateWithFlags(&s.dw_done[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      (void)hipGetLastError();
      s.s = nullptr;
    }
  }
  return s.s ? &s : nullptr;
}

// Debug mode: wait for the call's kernels and report a nonzero data-error
// word of the state as RNNTJ_ERR_DATA (otherwise only
// rnnt_joint_loss_status reports it).
int debug_data_check(const int32_t* hdr, hipStream_t st) {
  if (!debug_on()) return RNNTJ_OK;
  int32_t v = 0;
  if (hipStreamSynchronize(st) != hipSuccess ||
      hipMemcpy(&v, hdr, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
    return RNNTJ_ERR_HIP;
  return v ? RNNTJ_ERR_DATA : RNNTJ_OK;
}

// The forward of both entry points: S = 0 the full lattice (criterion sum or
// max); S > 0 the pruned loss (full sum inside the band of S label positions
// per frame that the simple joiner's lattice selects; tiled mode only).
int fwd_impl(const void* enc, const void* pred, const void* W_out, const void* b_out, int dtype,
             const int32_t* labels, const int32_t* T_lens, const int32_t* U_lens, int B, int T,
             int U, int H, int V, int blank, int tile_t, int tile_u, int tile_v, int criterion,
             int S, float* costs, float* simple_costs, void* saved, void* workspace,
             size_t workspace_bytes, void* stream, const TdtIn* tdt = nullptr) {
  Plan p;
  int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (tdt) {
    if ((rc = check_tdt(*tdt))) return rc;
    if (criterion != RNNTJ_CRIT_SUM || S != 0) return RNNTJ_ERR_ARG;
    if (U + 1 > kMaxU1Short) return RNNTJ_ERR_UNSUPPORTED;
  }
  if (criterion != RNNTJ_CRIT_SUM && criterion != RNNTJ_CRIT_MAX) return RNNTJ_ERR_ARG;
  const bool pruned = S > 0;
  if (S < 0) return RNNTJ_ERR_ARG;
  if (pruned) {
    if (criterion != RNNTJ_CRIT_SUM || p.untiled || T > kMaxPrunedT || U + 1 > kMaxU1Short)
      return RNNTJ_ERR_UNSUPPORTED;
    if (workspace_bytes < p.ws_pruned || !workspace) return RNNTJ_ERR_WORKSPACE;
    if (misaligned(workspace) || misaligned(simple_costs)) return RNNTJ_ERR_ARG;
  }
  const int crit = criterion == RNNTJ_CRIT_MAX ? kCritMax : kCritSum;
  if (!enc || !pred || !W_out || !b_out || !T_lens || !U_lens || !costs || !saved)
    return RNNTJ_ERR_ARG;
  if (U > 0 && !labels) return RNNTJ_ERR_ARG;
  if (blank < 0 || blank >= V) return RNNTJ_ERR_ARG;
  if (misaligned(enc) || misaligned(pred) || misaligned(W_out) || misaligned(saved))
    return RNNTJ_ERR_ARG;
  if (workspace_bytes < p.ws_fwd) return RNNTJ_ERR_WORKSPACE;
  p.d.blank = blank;
  hipStream_t st = static_cast<hipStream_t>(stream);

  int32_t* status = at<int32_t>(saved, p.o_status);
  int32_t* Teff = at<int32_t>(saved, p.o_teff);
  int32_t* Ueff = at<int32_t>(saved, p.o_ueff);
  double* logP = at<double>(saved, p.o_logp);
  void* Wt = at<char>(saved, p.o_wt);
  float* lse = at<float>(saved, p.o_lse);
  float* LB = at<float>(saved, p.o_lb);
  float* LE = at<float>(saved, p.o_le);
  double* alpha = at<double>(saved, p.o_alpha);
  double* beta = at<double>(saved, p.o_beta);

  hipError_t e;
  if ((e = timed("zero", st, [&] { return launch_zero(status, kHdrWords, st); })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  const int32_t tag = tdt ? tdt_tag(p, blank, *tdt) : plan_tag(p, blank);
  if ((e = timed("validate", st, [&] {
         return launch_validate(T_lens, U_lens, labels, p.d, Teff, Ueff, status,
                                tdt ? kCritTdt : crit, tag, p.untiled ? 1 : 0, S, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  float* Eexp = at<float>(saved, p.o_E);
  float* Pexp = at<float>(saved, p.o_P);
  if ((e = timed("prep", st, [&] {
         return launch_prep(enc, pred, W_out, b_out, p.bf16, p.d, Wt, at<char>(saved, p.o_wb),
                            Eexp, Pexp, status, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;

  int32_t* bounds = at<int32_t>(saved, p.o_bounds);
  if (pruned) {
    // the simple joiner's lattice and the window of every frame; then every
    // step weight starts at -inf, so that cells of tiles outside the band
    // carry no alignment
    PruneArgs g = {};
    g.enc = enc;
    g.pred = pred;
    g.W = W_out;
    g.bias = b_out;
    g.bf16 = p.bf16;
    g.labels = labels;
    g.Teff = Teff;
    g.Ueff = Ueff;
    g.status = status;
    g.d = p.d;
    g.S = S;
    g.am = at<double>(workspace, p.o_pw_am);
    g.lm = at<double>(workspace, p.o_pw_lm);
    g.ma = at<double>(workspace, p.o_pw_ma);
    g.ml = at<double>(workspace, p.o_pw_ml);
    g.amB = at<double>(workspace, p.o_pw_amB);
    g.amY = at<double>(workspace, p.o_pw_amY);
    g.lmB = at<double>(workspace, p.o_pw_lmB);
    g.lmY = at<double>(workspace, p.o_pw_lmY);
    g.LBs = at<double>(workspace, p.o_pw_LB);
    g.LEs = at<double>(workspace, p.o_pw_LE);
    g.alpha = at<double>(workspace, p.o_pw_alpha);
    g.beta = at<double>(workspace, p.o_pw_beta);
    g.logPs = at<double>(workspace, p.o_pw_logP);
    g.centres = at<double>(workspace, p.o_pw_centres);
    g.simple_costs = simple_costs;
    g.bounds = bounds;
    if ((e = timed("pruning_bounds", st, [&] { return launch_pruning_bounds(g, st); })) !=
        hipSuccess)
      return RNNTJ_ERR_HIP;
    const size_t cells = (size_t)B * p.d.DG * p.d.U1;
    if ((e = timed("fill", st, [&] {
           hipError_t r = launch_fill(LB, cells, -__builtin_inff(), st);
           return r != hipSuccess ? r : launch_fill(LE, cells, -__builtin_inff(), st);
         })) != hipSuccess)
      return RNNTJ_ERR_HIP;
  }

  int32_t* tiles = at<int32_t>(saved, p.o_tiles);
  int32_t* tcount = at<int32_t>(saved, p.o_tcount);
  if ((e = timed("tile_list", st, [&] {
         return launch_tile_list(Teff, Ueff, p.d, p.d.Tpad, p.d.U1pad, 1, 1, p.cap_all, tiles,
                                 tcount, status, bounds, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;

  JointArgs a = {};
  a.enc = enc;
  a.pred = pred;
  a.Wt = Wt;
  a.bias = b_out;
  a.labels = labels;
  a.Teff = Teff;
  a.Ueff = Ueff;
  a.hdr = status;
  a.Eexp = Eexp;
  a.Pexp = Pexp;
  a.tiles = tiles;
  a.tile_count = tcount;
  a.vsplit = 1;
  a.d = p.d;
  a.ct0 = 0;
  a.cu0 = 0;
  a.CT = p.d.Tpad;
  a.CU = p.d.U1pad;
  a.n_tu = p.d.U1pad / kTileU;
  a.lse = lse;
  a.LB = LB;
  a.LE = LE;
  a.zout = p.untiled ? at<char>(saved, p.o_z) : nullptr;
  a.hout = p.untiled ? at<char>(saved, p.o_h) : nullptr;
  a.zmax = (p.untiled && p.bf16) ? at<float>(saved, p.o_zm) : nullptr;
  a.zstep = p.zstep;
  a.bounds = bounds;
  a.band = S;
  a.gv0 = 0;
  a.gvw = V;
  a.gld = V;
  if ((e = timed(p.untiled ? "joint_fwd_store" : "joint_fwd", st, [&] {
         return launch_joint_tile(a, p.untiled ? kStoreZ : kLse, p.bf16, p.cap_all, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if (tdt) {
    // the duration head's log-probabilities, then the lattice whose steps
    // jump by the durations
    TdtArgs g = {};
    g.d = p.d;
    g.bf16 = p.bf16;
    g.enc = enc;
    g.pred = pred;
    g.Wd = tdt->Wd;
    g.bd = tdt->bd;
    g.K = tdt->K;
    for (int j = 0; j < tdt->K; ++j) g.dur[j] = tdt->durations[j];
    g.Teff = Teff;
    g.Ueff = Ueff;
    g.hdr = status;
    g.Eexp = Eexp;
    g.Pexp = Pexp;
    g.LB = LB;
    g.LE = LE;
    g.LD = at<float>(saved, p.saved_bytes);
    g.alpha = alpha;
    g.beta = beta;
    g.logP = logP;
    g.costs = costs;
    if ((e = timed("tdt_dur_head", st, [&] { return launch_tdt_dur_head(g, st); })) !=
        hipSuccess)
      return RNNTJ_ERR_HIP;
    if ((e = timed("tdt_lattice", st, [&] { return launch_tdt_lattice(g, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    return debug_data_check(status, st);
  }
  if ((e = timed("lattice", st, [&] {
         return launch_lattice(LB, LE, Teff, Ueff, p.d, alpha, beta, logP, costs, crit, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if (crit == kCritMax &&
      (e = timed("backtrace", st, [&] { return launch_backtrace(Teff, Ueff, p.d, beta, st); })) !=
          hipSuccess)
    return RNNTJ_ERR_HIP;
  return debug_data_check(status, st);
}

// The backward of every entry point (tdt: a token-and-duration state, with
// the duration head's weights and gradients).
int bwd_impl(const void* enc, const void* pred, const void* W_out, const void* b_out, int dtype,
             const int32_t* labels, int B, int T, int U, int H, int V, int blank, int tile_t,
             int tile_u, int tile_v, const float* grad_costs, void* saved, float* d_enc,
             float* d_pred, float* d_W_out, float* d_b_out, void* workspace,
             size_t workspace_bytes, void* stream, const TdtIn* tdt = nullptr,
             float* d_Wd = nullptr, float* d_bd = nullptr, bool side_ok = true) {
  Plan p;
  int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  TdtWs tw = {};
  size_t ws_need = p.bwd_ws();
  if (tdt) {
    if ((rc = check_tdt(*tdt))) return rc;
    if (U + 1 > kMaxU1Short) return RNNTJ_ERR_UNSUPPORTED;
    if (!d_Wd || !d_bd || misaligned(d_Wd) || misaligned(d_bd)) return RNNTJ_ERR_ARG;
    tw = tdt_ws(p, tdt->K);
    ws_need = tw.total;
  }
  if (!enc || !pred || !W_out || !b_out || !saved || !d_enc || !d_pred || !d_W_out || !d_b_out)
    return RNNTJ_ERR_ARG;
  if (U > 0 && !labels) return RNNTJ_ERR_ARG;
  if (blank < 0 || blank >= V) return RNNTJ_ERR_ARG;
  if (misaligned(enc) || misaligned(pred) || misaligned(W_out) || misaligned(saved) ||
      misaligned(d_enc) || misaligned(d_pred) || misaligned(d_W_out) || misaligned(d_b_out) ||
      misaligned(grad_costs))
    return RNNTJ_ERR_ARG;
  if (workspace_bytes < ws_need || !workspace) return RNNTJ_ERR_WORKSPACE;
  if (misaligned(workspace)) return RNNTJ_ERR_ARG;
  p.d.blank = blank;
  hipStream_t st = static_cast<hipStream_t>(stream);

  int32_t* Teff = at<int32_t>(saved, p.o_teff);
  int32_t* Ueff = at<int32_t>(saved, p.o_ueff);
  double* logP = at<double>(saved, p.o_logp);
  void* Wt = at<char>(saved, p.o_wt);
  double* db64 = at<double>(workspace, p.o_ws_db);
  void* gchunk = at<char>(workspace, p.o_ws_g);
  void* hchunk = at<char>(workspace, p.o_ws_h);

  hipError_t e;
  if ((e = timed("zero", st, [&] {
         return launch_zero4(d_enc, (size_t)B * T * H, d_pred, (size_t)B * (U + 1) * H, d_W_out,
                             (size_t)H * V, db64, 2 * (size_t)V, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  // the state must come from a forward with these sizes, dtype and blank
  // (and, for the untiled backward, one that stored the logits)
  int32_t* hdr = at<int32_t>(saved, p.o_status);
  if ((e = timed("guard", st, [&] {
         return launch_guard(hdr, tdt ? tdt_tag(p, blank, *tdt) : plan_tag(p, blank),
                             p.untiled ? 1 : 0, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;

  JointArgs a = {};
  a.enc = enc;
  a.pred = pred;
  a.Wt = Wt;
  a.bias = b_out;
  a.labels = labels;
  a.Teff = Teff;
  a.Ueff = Ueff;
  a.hdr = hdr;
  a.Eexp = at<float>(saved, p.o_E);
  a.Pexp = at<float>(saved, p.o_P);
  a.d = p.d;
  a.lse = at<float>(saved, p.o_lse);
  a.LB = at<float>(saved, p.o_lb);
  a.LE = at<float>(saved, p.o_le);
  a.alpha = at<double>(saved, p.o_alpha);
  a.beta = at<double>(saved, p.o_beta);
  a.logP = logP;
  a.gcost = grad_costs;
  a.zmax = (p.untiled && p.bf16) ? at<float>(saved, p.o_zm) : nullptr;
  a.zstep = p.zstep;
  TdtArgs g = {};
  if (tdt) {
    // per-cell step posteriors (summed over the durations) and the duration
    // logits' gradients; the token head's kernels then read the posteriors
    // in place of alpha / beta
    g.d = p.d;
    g.d.blank = blank;
    g.bf16 = p.bf16;
    g.enc = enc;
    g.pred = pred;
    g.Wd = tdt->Wd;
    g.bd = tdt->bd;
    g.K = tdt->K;
    for (int j = 0; j < tdt->K; ++j) g.dur[j] = tdt->durations[j];
    g.Teff = Teff;
    g.Ueff = Ueff;
    g.hdr = hdr;
    g.Eexp = a.Eexp;
    g.Pexp = a.Pexp;
    g.LB = a.LB;
    g.LE = a.LE;
    g.LD = at<float>(saved, p.saved_bytes);
    g.alpha = at<double>(saved, p.o_alpha);
    g.beta = at<double>(saved, p.o_beta);
    g.logP = logP;
    g.gcost = grad_costs;
    g.gB = at<double>(workspace, tw.gB);
    g.gE = at<double>(workspace, tw.gE);
    g.dzd = at<float>(workspace, tw.dzd);
    if (deterministic_on()) {
      g.part_w = at<float>(workspace, tw.part_w);
      g.part_b = at<float>(workspace, tw.part_b);
    }
    g.d_enc = d_enc;
    g.d_pred = d_pred;
    g.d_Wd = d_Wd;
    g.d_bd = d_bd;
    if ((e = timed("zero", st, [&] {
           return launch_zero4(d_Wd, (size_t)H * tdt->K, d_bd, (size_t)tdt->K, nullptr, 0,
                               nullptr, 0, st);
         })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    if ((e = timed("tdt_post", st, [&] { return launch_tdt_post(g, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    a.alpha = g.gB;
    a.beta = g.gE;
  }

  DhArgs h = {};
  h.W = at<char>(saved, p.o_wb);  // written by the forward
  h.enc = enc;
  h.pred = pred;
  h.Teff = Teff;
  h.Ueff = Ueff;
  h.hdr = a.hdr;
  h.Eexp = a.Eexp;
  h.Pexp = a.Pexp;
  h.d = p.d;
  h.d_enc = d_enc;
  h.d_pred = d_pred;
  h.ksplit = 1;
  h.v0 = 0;
  h.vw = V;
  h.ldg = V;
  const bool det = deterministic_on();
  if (det) {
    h.enc_part = at<float>(workspace, p.o_ws_encp);
    h.pred_part = at<float>(workspace, p.o_ws_predp);
  }
  DwArgs w = {};
  w.v0 = 0;
  w.vw = V;
  w.ldg = V;
  if (det) {
    w.w_part = at<float>(workspace, p.o_ws_wpart);
    w.b_part = at<double>(workspace, p.o_ws_bpart);
  }
  w.h = hchunk;
  w.d = p.d;
  w.d_W = d_W_out;
  w.d_b64 = db64;
  w.hdr = hdr;
  h.gcost = grad_costs;
  // split-K runs of the dW GEMM: one round of resident workgroups (two per
  // compute unit for bf16, one for fp32), fewest float32 partial sums per
  // output element
  auto kparts_for = [&](int max_tiles) {
    const int per = ((H + 127) / 128) * ((p.Vp + 255) / 256);  // items of one part
    int k = device_cu_count() * (p.bf16 ? 2 : 1) / per;
    // each run at least 4 tiles: shorter runs spend more on their atomics
    // (an H x 256 block per item) than on their MFMAs
    const int kmax = max_tiles / 4 > 1 ? max_tiles / 4 : 1;
    k = k < 1 ? 1 : (k > kmax ? kmax : k);
    return det ? (k < p.kparts_det ? k : p.kparts_det) : k;
  };
  // deterministic mode: dh and dW store partial sums that two ordered
  // reduction kernels add after each GEMM, in place of float atomics
  auto reduce_dh = [&]() -> hipError_t {
    if (!det) return hipSuccess;
    return timed("dh_reduce", st, [&] {
      return launch_dh_reduce(h, p.untiled ? p.cap_all : p.cap_chunk, st);
    });
  };
  auto reduce_dw = [&](hipStream_t s) -> hipError_t {
    if (!det) return hipSuccess;
    return timed("dw_reduce", s, [&] { return launch_dw_reduce(w, s); });
  };
  auto finalize = [&](int32_t* mark) {
    if (tdt) {
      const hipError_t r = timed("tdt_dur_bwd", st, [&] { return launch_tdt_dur_bwd(g, st); });
      if (r != hipSuccess) return r;
    }
    return timed("db_finalize", st,
                 [&] { return launch_db_finalize(db64, d_b_out, V, mark, st); });
  };

  if (p.untiled) {
    // the stored logits become the logit gradients in place; dh and dW then
    // read them as plain GEMM operands
    void* z = at<char>(saved, p.o_z);
    a.tiles = at<int32_t>(saved, p.o_tiles);
    a.tile_count = at<int32_t>(saved, p.o_tcount);
    a.ct0 = 0; a.cu0 = 0; a.CT = p.d.Tpad; a.CU = p.d.U1pad;
    if ((e = timed("grad_inplace", st,
                   [&] { return launch_grad_inplace(z, p.bf16, a, p.cap_all, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    h.g = z;
    h.ct0 = 0; h.cu0 = 0; h.CT = p.d.Tpad; h.CU = p.d.U1pad;
    h.tiles = a.tiles;
    h.tile_count = a.tile_count;
    w.g = z;
    w.h = at<char>(saved, p.o_h);  // written by the forward
    w.ct0 = 0; w.cu0 = 0; w.CT = p.d.Tpad; w.CU = p.d.U1pad;
    w.tiles = a.tiles;
    w.tile_count = a.tile_count;
    w.kparts = kparts_for(p.cap_all);
    if ((e = timed("dh", st, [&] { return launch_dh(h, p.bf16, p.cap_all, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    if ((e = timed("dw", st, [&] { return launch_dw(w, p.bf16, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    if (reduce_dh() != hipSuccess || reduce_dw(st) != hipSuccess) return RNNTJ_ERR_HIP;
    if (finalize(a.hdr) != hipSuccess) return RNNTJ_ERR_HIP;
    return debug_data_check(hdr, st);
  }

  // tiled: one lattice chunk of CT frames x CU label positions at a time.
  // The logit-gradient kernel splits the vocabulary tiles of each cell tile
  // over several workgroups when a chunk alone has too few cell tiles to
  // give every compute unit (256 on gfx950) about four of them, as long as
  // each part keeps at least 8 vocabulary tiles: every part rebuilds the
  // tile's h rows and posteriors, which shorter parts do not amortise.
  const int chunk_tiles = p.cap_chunk;
  const int nvt = (p.Vp + kVocabTile - 1) / kVocabTile;
  int vsplit = 1;
  while (chunk_tiles * vsplit < 1024 && nvt / (2 * vsplit) >= 8) vsplit *= 2;
  int32_t* ctiles = at<int32_t>(workspace, p.o_ws_tiles);
  int32_t* ccount = at<int32_t>(workspace, p.o_ws_tcount);
  if ((e = timed("tile_list", st, [&] {
         return launch_tile_list(Teff, Ueff, p.d, p.CT, p.CU, p.n_cu_chunks, p.n_chunks,
                                 p.cap_chunk, ctiles, ccount, hdr, at<int32_t>(saved, p.o_bounds),
                                 st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  // Chunk schedule.  With room for a second buffer pair after the workspace
  // proper, vocabulary pass k (one chunk's vocabulary part) writes buffer
  // pair k & 1 (the h rows: pair c & 1 of its chunk c) and its dW runs on the
  // side stream: it overlaps the pass's dh and the next pass's logit
  // gradients, and pass k + 2 first waits for it, since it overwrites what
  // that dW reads.  Otherwise every kernel runs in order on the caller's
  // stream over one buffer pair.
  SideStream* ss = nullptr;
  std::unique_lock<std::mutex> side_lk;
  void* gbuf[2] = {gchunk, gchunk};
  void* hbuf[2] = {hchunk, hchunk};
  const int n_passes = p.n_chunks * ((V + p.Vp - 1) / p.Vp);
  if (side_ok && workspace_bytes >= p.overlap_bytes(ws_need) && n_passes > 1 &&
      (ss = side_stream()) != nullptr) {
    side_lk = std::unique_lock<std::mutex>(ss->mu);
    char* second = at<char>(workspace, align_up(ws_need));
    gbuf[1] = second;
    hbuf[1] = second + p.ws_g;
  }
  hipStream_t sw = ss ? ss->s : st;  // stream of the dW GEMMs
  int chunk = 0, pass = 0;
  // on an error after the fork, the caller's stream still waits for the dW
  // GEMMs already enqueued on the side stream
  int joined_to = -1;  // last pass whose dW end was recorded
  auto fail = [&](const char* what, hipError_t err) {
    if (what) note_error(what, err);
    if (ss && joined_to >= 0) (void)hipStreamWaitEvent(st, ss->dw_done[joined_to & 1], 0);
    return RNNTJ_ERR_HIP;
  };
  for (int ct0 = 0; ct0 < p.d.Tpad; ct0 += p.CT) {
    for (int cu0 = 0; cu0 < p.d.U1pad; cu0 += p.CU, ++chunk) {
      a.ct0 = ct0;
      a.cu0 = cu0;
      a.CT = p.CT;
      a.CU = p.CU;
      a.n_tu = p.CU / kTileU;
      a.vsplit = vsplit;
      a.hout = hbuf[chunk & 1];
      a.tiles = ctiles + (size_t)chunk * p.cap_chunk;
      a.tile_count = ccount + chunk;
      h.ct0 = ct0; h.cu0 = cu0; h.CT = p.CT; h.CU = p.CU;
      h.tiles = a.tiles;
      h.tile_count = a.tile_count;
      w.h = hbuf[chunk & 1];
      w.ct0 = ct0; w.cu0 = cu0; w.CT = p.CT; w.CU = p.CU;
      w.tiles = a.tiles;
      w.tile_count = a.tile_count;
      w.kparts = kparts_for(p.cap_chunk);
      // the chunk's vocabulary in parts of Vp columns: the logit gradients
      // of one part, that part's share of dh (linear in dz, so the parts'
      // d_enc / d_pred contributions add) and its columns of dW
      for (int v0 = 0; v0 < V; v0 += p.Vp, ++pass) {
        const int vw = V - v0 < p.Vp ? V - v0 : p.Vp;
        void* g = gbuf[pass & 1];
        a.gout = g;
        h.g = g;
        w.g = g;
        a.gv0 = v0; a.gvw = vw; a.gld = p.Vp;
        h.v0 = v0; h.vw = vw; h.ldg = p.Vp;
        w.v0 = v0; w.vw = vw; w.ldg = p.Vp;
        // buffer pair pass & 1 (and the h rows of chunk pair chunk & 1, last
        // read by a dW at or before pass - 2) are free once the dW of pass - 2 is done
        if (ss && pass >= 2 &&
            (e = hipStreamWaitEvent(st, ss->dw_done[pass & 1], 0)) != hipSuccess)
          return fail("stream wait", e);
        if ((e = timed("joint_grad", st, [&] {
               return launch_joint_tile(a, kGrad, p.bf16, p.cap_chunk * vsplit, st);
             })) != hipSuccess)
          return fail(nullptr, e);
        if (ss && ((e = hipEventRecord(ss->jg_done[pass & 1], st)) != hipSuccess ||
                   (e = hipStreamWaitEvent(sw, ss->jg_done[pass & 1], 0)) != hipSuccess))
          return fail("stream fork", e);
        if ((e = timed("dh", st, [&] { return launch_dh(h, p.bf16, p.cap_chunk, st); })) !=
            hipSuccess)
          return fail(nullptr, e);
        if (reduce_dh() != hipSuccess) return fail(nullptr, hipSuccess);
        if ((e = timed("dw", sw, [&] { return launch_dw(w, p.bf16, sw); })) != hipSuccess)
          return fail(nullptr, e);
        if (reduce_dw(sw) != hipSuccess) return fail(nullptr, hipSuccess);
        if (ss) {
          if ((e = hipEventRecord(ss->dw_done[pass & 1], sw)) != hipSuccess)
            return fail("stream event", e);
          joined_to = pass;
        }
      }
    }
  }
  // join: the caller's stream waits for the last dW (the side stream runs in order)
  if (ss && joined_to >= 0 &&
      (e = hipStreamWaitEvent(st, ss->dw_done[joined_to & 1], 0)) != hipSuccess)
    return note_error("stream join", e), RNNTJ_ERR_HIP;
  if (finalize(nullptr) != hipSuccess) return RNNTJ_ERR_HIP;
  return debug_data_check(hdr, st);
}

}  // namespace

extern "C" {

int rnnt_joint_loss_abi_version(void) { return RNNTJ_ABI_VERSION; }

int rnnt_joint_loss_get_flags(void) { return g_flags.load(); }

int rnnt_joint_loss_set_flags(int flags) {
  if (flags & ~(RNNTJ_FLAG_DEBUG | RNNTJ_FLAG_DETERMINISTIC)) return RNNTJ_ERR_ARG;
  g_flags.store(flags);
  return RNNTJ_OK;
}

const char* rnnt_joint_loss_strerror(int code) {
  switch (code) {
    case RNNTJ_OK: return "ok";
    case RNNTJ_ERR_ARG: return "invalid argument (null pointer, bad size, dtype or blank)";
    case RNNTJ_ERR_UNSUPPORTED: return "unsupported shape or tile size";
    case RNNTJ_ERR_WORKSPACE: return "workspace too small";
    case RNNTJ_ERR_HIP: return "HIP runtime error";
    case RNNTJ_ERR_DATA: return "invalid lengths or labels in the batch";
    default: return "unknown status code";
  }
}

int rnnt_joint_loss_saved_bytes(int B, int T, int U, int H, int V, int dtype, int tile_t,
                                int tile_u, int tile_v, size_t* out) {
  if (!out) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  *out = p.saved_bytes;
  return RNNTJ_OK;
}

int rnnt_joint_loss_workspace_bytes(int B, int T, int U, int H, int V, int dtype, int tile_t,
                                    int tile_u, int tile_v, int pass, size_t* out) {
  if (!out || pass < 0 || pass > 2) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  *out = pass == 0 ? p.ws_fwd : pass == 1 ? p.overlap_bytes(p.bwd_ws()) : p.bwd_ws();
  return RNNTJ_OK;
}

int rnnt_joint_loss_fwd(const void* enc, const void* pred, const void* W_out, const void* b_out,
                        int dtype, const int32_t* labels, const int32_t* T_lens,
                        const int32_t* U_lens, int B, int T, int U, int H, int V, int blank,
                        int tile_t, int tile_u, int tile_v, float* costs, void* saved,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return rnnt_joint_loss_fwd_ex(enc, pred, W_out, b_out, dtype, labels, T_lens, U_lens, B, T, U,
                                H, V, blank, tile_t, tile_u, tile_v, RNNTJ_CRIT_SUM, costs, saved,
                                workspace, workspace_bytes, stream);
}

int rnnt_joint_loss_fwd_ex(const void* enc, const void* pred, const void* W_out,
                           const void* b_out, int dtype, const int32_t* labels,
                           const int32_t* T_lens, const int32_t* U_lens, int B, int T, int U,
                           int H, int V, int blank, int tile_t, int tile_u, int tile_v,
                           int criterion, float* costs, void* saved, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return fwd_impl(enc, pred, W_out, b_out, dtype, labels, T_lens, U_lens, B, T, U, H, V, blank,
                  tile_t, tile_u, tile_v, criterion, 0, costs, nullptr, saved, workspace,
                  workspace_bytes, stream);
}

int rnnt_joint_loss_pruned_workspace_bytes(int B, int T, int U, int H, int V, int dtype,
                                           size_t* out) {
  if (!out) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, kTileT, kTileU, 0, &p);
  if (rc) return rc;
  if (T > kMaxPrunedT || U + 1 > kMaxU1Short) return RNNTJ_ERR_UNSUPPORTED;
  *out = p.ws_pruned;
  return RNNTJ_OK;
}

int rnnt_joint_loss_pruned_fwd(const void* enc, const void* pred, const void* W_out,
                               const void* b_out, int dtype, const int32_t* labels,
                               const int32_t* T_lens, const int32_t* U_lens, int B, int T, int U,
                               int H, int V, int blank, int tile_t, int tile_u, int tile_v, int S,
                               float* costs, float* simple_costs, void* saved, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (S < 1) return RNNTJ_ERR_ARG;
  return fwd_impl(enc, pred, W_out, b_out, dtype, labels, T_lens, U_lens, B, T, U, H, V, blank,
                  tile_t, tile_u, tile_v, RNNTJ_CRIT_SUM, S, costs, simple_costs, saved,
                  workspace, workspace_bytes, stream);
}

int rnnt_joint_loss_pruned_bounds(const void* saved, int B, int T, int U, int H, int V, int dtype,
                                  int tile_t, int tile_u, int tile_v, int32_t* bounds,
                                  void* stream) {
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (!saved || !bounds) return RNNTJ_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* src = static_cast<const char*>(saved) + p.o_bounds;
  return note_error("bounds copy", hipMemcpyAsync(bounds, src, 4 * (size_t)B * T,
                                                  hipMemcpyDeviceToDevice, st)) == hipSuccess
             ? RNNTJ_OK
             : RNNTJ_ERR_HIP;
}

int rnnt_joint_loss_bwd(const void* enc, const void* pred, const void* W_out, const void* b_out,
                        int dtype, const int32_t* labels, const int32_t* T_lens,
                        const int32_t* U_lens, int B, int T, int U, int H, int V, int blank,
                        int tile_t, int tile_u, int tile_v, const float* grad_costs,
                        void* saved, float* d_enc, float* d_pred, float* d_W_out,
                        float* d_b_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  (void)T_lens;
  (void)U_lens;
  return bwd_impl(enc, pred, W_out, b_out, dtype, labels, B, T, U, H, V, blank, tile_t, tile_u,
                  tile_v, grad_costs, saved, d_enc, d_pred, d_W_out, d_b_out, workspace,
                  workspace_bytes, stream);
}

int rnnt_joint_loss_tdt_saved_bytes(int B, int T, int U, int H, int V, int dtype, int tile_t,
                                    int tile_u, int tile_v, int K, size_t* out) {
  if (!out || K < 1 || K > kTdtMaxK) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (U + 1 > kMaxU1Short) return RNNTJ_ERR_UNSUPPORTED;
  *out = p.saved_bytes + tdt_ld_bytes(p, K);
  return RNNTJ_OK;
}

int rnnt_joint_loss_tdt_workspace_bytes(int B, int T, int U, int H, int V, int dtype, int tile_t,
                                        int tile_u, int tile_v, int K, int pass, size_t* out) {
  if (!out || K < 1 || K > kTdtMaxK || pass < 0 || pass > 2) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (U + 1 > kMaxU1Short) return RNNTJ_ERR_UNSUPPORTED;
  const size_t need = tdt_ws(p, K).total;
  *out = pass == 0 ? p.ws_fwd : pass == 1 ? p.overlap_bytes(need) : need;
  return RNNTJ_OK;
}

int rnnt_joint_loss_tdt_fwd(const void* enc, const void* pred, const void* W_out,
                            const void* b_out, const void* W_dur, const void* b_dur, int dtype,
                            const int32_t* labels, const int32_t* T_lens, const int32_t* U_lens,
                            int B, int T, int U, int H, int V, int blank,
                            const int32_t* durations, int K, int tile_t, int tile_u, int tile_v,
                            float* costs, void* saved, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const TdtIn t{W_dur, b_dur, durations, K};
  return fwd_impl(enc, pred, W_out, b_out, dtype, labels, T_lens, U_lens, B, T, U, H, V, blank,
                  tile_t, tile_u, tile_v, RNNTJ_CRIT_SUM, 0, costs, nullptr, saved, workspace,
                  workspace_bytes, stream, &t);
}

int rnnt_joint_loss_tdt_bwd(const void* enc, const void* pred, const void* W_out,
                            const void* b_out, const void* W_dur, const void* b_dur, int dtype,
                            const int32_t* labels, const int32_t* T_lens, const int32_t* U_lens,
                            int B, int T, int U, int H, int V, int blank,
                            const int32_t* durations, int K, int tile_t, int tile_u, int tile_v,
                            const float* grad_costs, void* saved, float* d_enc, float* d_pred,
                            float* d_W_out, float* d_b_out, float* d_W_dur, float* d_b_dur,
                            void* workspace, size_t workspace_bytes, void* stream) {
  (void)T_lens;
  (void)U_lens;
  const TdtIn t{W_dur, b_dur, durations, K};
  return bwd_impl(enc, pred, W_out, b_out, dtype, labels, B, T, U, H, V, blank, tile_t, tile_u,
                  tile_v, grad_costs, saved, d_enc, d_pred, d_W_out, d_b_out, workspace,
                  workspace_bytes, stream, &t, d_W_dur, d_b_dur);
}

int rnnt_joint_loss_bwd_noalloc(const void* enc, const void* pred, const void* W_out,
                                const void* b_out, int dtype, const int32_t* labels,
                                const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                                int U, int H, int V, int blank, int tile_t, int tile_u,
                                int tile_v, const float* grad_costs, void* saved, float* d_enc,
                                float* d_pred, float* d_W_out, float* d_b_out, void* stream) {
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (p.bwd_ws() > kScratchBytes) return RNNTJ_ERR_WORKSPACE;  // before anything is enqueued
  if (!enc || !pred || !W_out || !b_out || !saved || !d_enc || !d_pred || !d_W_out || !d_b_out)
    return RNNTJ_ERR_ARG;
  void* ws = nullptr;
  const int src = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (src) return src;
  (void)T_lens;
  (void)U_lens;
  // one stream: creating the side stream could allocate
  return bwd_impl(enc, pred, W_out, b_out, dtype, labels, B, T, U, H, V, blank, tile_t, tile_u,
                  tile_v, grad_costs, saved, d_enc, d_pred, d_W_out, d_b_out, ws, kScratchBytes,
                  stream, nullptr, nullptr, nullptr, false);
}

int rnnt_joint_loss_status(const void* saved, void* stream, int32_t* data_error) {
  if (!saved || !data_error) return RNNTJ_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return RNNTJ_ERR_HIP;
  int32_t v = 0;
  if (hipMemcpy(&v, saved, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return RNNTJ_ERR_HIP;
  *data_error = v;
  return RNNTJ_OK;
}

const char* rnnt_joint_loss_last_error(void) { return g_last_error; }

int rnnt_joint_proj_fwd(const void* x, const void* W, const void* b, int dtype, int M, int K,
                        int N, void* y, void* stream) {
  if (!x || !W || !y || M < 1 || K < 1 || N < 1) return RNNTJ_ERR_ARG;
  if (dtype != RNNTJ_F32 && dtype != RNNTJ_BF16) return RNNTJ_ERR_ARG;
  if (misaligned(x) || misaligned(W) || misaligned(y)) return RNNTJ_ERR_ARG;
  if (K % 16 != 0 || N % 16 != 0 || K > kMaxProj || N > kMaxProj) return RNNTJ_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return timed("proj_fwd", st, [&] {
           return launch_proj_fwd(x, W, b, dtype == RNNTJ_BF16, M, K, N, y, st);
         }) == hipSuccess
             ? RNNTJ_OK
             : RNNTJ_ERR_HIP;
}

int rnnt_joint_proj_bwd(const void* x, const void* W, int dtype, int M, int K, int N,
                        const float* dy, float* dx, float* dW, float* db, void* stream) {
  if (!x || !W || !dy || !dW || M < 1 || K < 1 || N < 1) return RNNTJ_ERR_ARG;
  if (dtype != RNNTJ_F32 && dtype != RNNTJ_BF16) return RNNTJ_ERR_ARG;
  if (misaligned(x) || misaligned(W) || misaligned(dy) || misaligned(dx) || misaligned(dW) ||
      misaligned(db))
    return RNNTJ_ERR_ARG;
  if (K % 16 != 0 || N % 16 != 0 || K > kMaxProj || N > kMaxProj) return RNNTJ_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == RNNTJ_BF16;
  if (timed("zero", st, [&] { return launch_zero4(dW, (size_t)K * N, db, db ? N : 0, nullptr, 0,
                                                  nullptr, 0, st); }) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if (dx && timed("proj_dx", st, [&] { return launch_proj_dx(dy, W, bf16, M, K, N, dx, st); }) !=
                hipSuccess)
    return RNNTJ_ERR_HIP;
  if (timed("proj_dw", st, [&] {
        return launch_proj_dw(x, dy, bf16, M, K, N, dW, db, device_cu_count(), deterministic_on(),
                              st);
      }) != hipSuccess)
    return RNNTJ_ERR_HIP;
  return RNNTJ_OK;
}

int rnnt_joint_loss_timing(int enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing = enable != 0;
  if (!g_timing) drop_timed();
  return RNNTJ_OK;
}

int rnnt_joint_loss_timing_report(char* buf, size_t len) {
  if (!buf || len == 0) return RNNTJ_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  std::map<std::string, std::pair<int, double>> agg;
  int rc = RNNTJ_OK;
  for (auto& t : g_timed) {
    float ms = 0.f;
    if (hipEventSynchronize(t.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess)
      rc = RNNTJ_ERR_HIP;
    auto& a = agg[t.name];
    a.first += 1;
    a.second += ms;
  }
  drop_timed();
  std::string out;
  char line[160];
  for (auto& kv : agg) {
    snprintf(line, sizeof(line), "%s %d %.6f\n", kv.first.c_str(), kv.second.first,
             kv.second.second);
    out += line;
  }
  const size_t n = out.size() < len - 1 ? out.size() : len - 1;
  memcpy(buf, out.data(), n);
  buf[n] = 0;
  return rc;
}

}  // extern "C"
