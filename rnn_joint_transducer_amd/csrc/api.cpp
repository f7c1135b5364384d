// C ABI of the fused RNN-T joint + transducer loss (see include/rnnt_joint.h).
//
// Host side only: argument checks, carving of the caller's `saved` and
// `workspace` buffers, and the launch sequence.  Every step of the
// computation runs in the HIP kernels of this library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rnnt_joint.h"
#include "kernels.h"

using namespace rnntj;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  Dims d;
  bool bf16;
  bool untiled;
  int CT, CU;  // backward chunk extents
  size_t elem;
  // saved layout (byte offsets)
  size_t o_h;  // untiled: h rows [B, Tpad, U1pad, H]
  size_t o_status, o_teff, o_ueff, o_logp, o_wt, o_lse, o_lb, o_le, o_alpha, o_beta, o_E, o_P,
      o_tiles, o_tcount, o_z;
  size_t saved_bytes;
  size_t ws_fwd, ws_bwd;
  size_t o_ws_db, o_ws_g, o_ws_h, o_ws_tiles, o_ws_tcount;  // backward workspace layout
  int cap_all;                // active-tile list capacity of the whole lattice
  int n_cu_chunks, n_chunks;  // backward chunk grid (tiled mode)
  int cap_chunk;              // active-tile list capacity of one chunk
};

int make_plan(int B, int T, int U, int H, int V, int dtype, int tile_t, int tile_u, int tile_v,
              Plan* p) {
  if (B < 1 || T < 1 || U < 0 || H < 1 || V < 1) return RNNTJ_ERR_ARG;
  if (dtype != RNNTJ_F32 && dtype != RNNTJ_BF16) return RNNTJ_ERR_ARG;
  if (tile_t < 0 || tile_u < 0 || tile_v < 0) return RNNTJ_ERR_ARG;
  const bool bf16 = dtype == RNNTJ_BF16;
  if (H % 16 != 0 || H > (bf16 ? 768 : 256)) return RNNTJ_ERR_UNSUPPORTED;
  if (V % 8 != 0 || V < 8 || V > kMaxV) return RNNTJ_ERR_UNSUPPORTED;
  if (U + 1 > 512) return RNNTJ_ERR_UNSUPPORTED;
  if (B > 8191 || T > 65520) return RNNTJ_ERR_UNSUPPORTED;  // packed tile coordinates
  if (tile_t % kTileT != 0 || tile_u % kTileU != 0) return RNNTJ_ERR_UNSUPPORTED;
  // tile_v bounds the vocabulary columns of one online log-sum-exp step; the
  // kernels step by kVocabTile, which is within any accepted tile_v
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
  const size_t cells = (size_t)B * q.d.DG * q.d.U1;
  size_t o = 0;
  q.o_status = o; o = align_up(o + 16);
  q.o_teff = o;   o = align_up(o + 4 * (size_t)B);
  q.o_ueff = o;   o = align_up(o + 4 * (size_t)B);
  q.o_logp = o;   o = align_up(o + 8 * (size_t)B);
  q.o_wt = o;     o = align_up(o + q.elem * (size_t)H * V);
  q.o_lse = o;    o = align_up(o + 4 * cells);
  q.o_lb = o;     o = align_up(o + 4 * cells);
  q.o_le = o;     o = align_up(o + 4 * cells);
  // alpha / beta carry a trash area of 512 float64 past the cells (slots of
  // the lattice sweep that fall outside the lattice are stored there)
  q.o_alpha = o;  o = align_up(o + 8 * (cells + 512));
  q.o_beta = o;   o = align_up(o + 8 * (cells + 512));
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
  q.saved_bytes = o;
  q.ws_fwd = 0;
  // backward workspace: float64 d_b_out accumulator [V], then (tiled) one
  // chunk of logit gradients [B, CT, CU, V] and its joint activations h
  // [B, CT, CU, H] (untiled: none, the forward keeps h)
  q.n_cu_chunks = (q.d.U1pad + q.CU - 1) / q.CU;
  q.n_chunks = ((q.d.Tpad + q.CT - 1) / q.CT) * q.n_cu_chunks;
  q.cap_chunk = B * (q.CT / kTileT) * (q.CU / kTileU);
  q.o_ws_db = 0;
  q.o_ws_g = align_up(8 * (size_t)V);
  q.o_ws_h = q.o_ws_g + (q.untiled ? 0 : align_up(q.elem * (size_t)B * q.CT * q.CU * V));
  // (untiled: the h rows are part of the saved state instead)
  q.o_ws_tiles = q.o_ws_h + (q.untiled ? 0 : align_up(q.elem * (size_t)B * q.CT * q.CU * H));
  q.o_ws_tcount = q.o_ws_tiles + (q.untiled ? 0 : align_up(4 * (size_t)q.n_chunks * q.cap_chunk));
  q.ws_bwd = q.o_ws_tcount + (q.untiled ? 0 : align_up(4 * (size_t)q.n_chunks));
  return RNNTJ_OK;
}

template <typename P>
inline P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

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

}  // namespace

extern "C" {

int rnnt_joint_loss_abi_version(void) { return RNNTJ_ABI_VERSION; }

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
  if (!out || (pass != 0 && pass != 1)) return RNNTJ_ERR_ARG;
  Plan p;
  const int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  *out = pass == 0 ? p.ws_fwd : p.ws_bwd;
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
  (void)workspace;
  Plan p;
  int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (criterion != RNNTJ_CRIT_SUM && criterion != RNNTJ_CRIT_MAX) return RNNTJ_ERR_ARG;
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
  if ((e = timed("zero", st, [&] { return launch_zero(status, 4, st); })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if ((e = timed("validate", st, [&] {
         return launch_validate(T_lens, U_lens, labels, p.d, Teff, Ueff, status, crit, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  float* Eexp = at<float>(saved, p.o_E);
  float* Pexp = at<float>(saved, p.o_P);
  if ((e = timed("prep", st, [&] {
         return launch_prep(enc, pred, W_out, b_out, p.bf16, p.d, Wt, Eexp, Pexp, status, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;

  int32_t* tiles = at<int32_t>(saved, p.o_tiles);
  int32_t* tcount = at<int32_t>(saved, p.o_tcount);
  if ((e = timed("tile_list", st, [&] {
         return launch_tile_list(Teff, Ueff, p.d, p.d.Tpad, p.d.U1pad, 1, 1, p.cap_all, tiles,
                                 tcount, st);
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
  if ((e = timed(p.untiled ? "joint_fwd_store" : "joint_fwd", st, [&] {
         return launch_joint_tile(a, p.untiled ? kStoreZ : kLse, p.bf16, p.cap_all, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if ((e = timed("lattice", st, [&] {
         return launch_lattice(LB, LE, Teff, Ueff, p.d, alpha, beta, logP, costs, crit, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  if (crit == kCritMax &&
      (e = timed("backtrace", st, [&] { return launch_backtrace(Teff, Ueff, p.d, beta, st); })) !=
          hipSuccess)
    return RNNTJ_ERR_HIP;
  return RNNTJ_OK;
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
  Plan p;
  int rc = make_plan(B, T, U, H, V, dtype, tile_t, tile_u, tile_v, &p);
  if (rc) return rc;
  if (!enc || !pred || !W_out || !b_out || !saved || !d_enc || !d_pred || !d_W_out || !d_b_out)
    return RNNTJ_ERR_ARG;
  if (U > 0 && !labels) return RNNTJ_ERR_ARG;
  if (blank < 0 || blank >= V) return RNNTJ_ERR_ARG;
  if (misaligned(enc) || misaligned(pred) || misaligned(W_out) || misaligned(saved))
    return RNNTJ_ERR_ARG;
  if (workspace_bytes < p.ws_bwd || !workspace) return RNNTJ_ERR_WORKSPACE;
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

  JointArgs a = {};
  a.enc = enc;
  a.pred = pred;
  a.Wt = Wt;
  a.bias = b_out;
  a.labels = labels;
  a.Teff = Teff;
  a.Ueff = Ueff;
  a.hdr = at<int32_t>(saved, p.o_status);
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

  DhArgs h = {};
  h.W = W_out;
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
  DwArgs w = {};
  w.h = hchunk;
  w.d = p.d;
  w.d_W = d_W_out;
  w.d_b64 = db64;
  h.gcost = grad_costs;
  // split-K runs of the dW GEMM: one round of resident workgroups (two per
  // compute unit for bf16, one for fp32), fewest float32 partial sums per
  // output element
  auto kparts_for = [&](int max_tiles) {
    const int per = ((H + 127) / 128) * ((V + 255) / 256);
    int k = device_cu_count() * (p.bf16 ? 2 : 1) / per;
    return k < 1 ? 1 : (k > max_tiles ? max_tiles : k);
  };
  auto finalize = [&](int32_t* mark) {
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
    if ((e = timed("dh", st, [&] { return launch_dh(h, p.bf16, p.cap_all, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    w.g = z;
    w.h = at<char>(saved, p.o_h);  // written by the forward
    w.ct0 = 0; w.cu0 = 0; w.CT = p.d.Tpad; w.CU = p.d.U1pad;
    w.tiles = a.tiles;
    w.tile_count = a.tile_count;
    w.kparts = kparts_for(p.cap_all);
    if ((e = timed("dw", st, [&] { return launch_dw(w, p.bf16, st); })) != hipSuccess)
      return RNNTJ_ERR_HIP;
    return finalize(a.hdr) == hipSuccess ? RNNTJ_OK : RNNTJ_ERR_HIP;
  }

  // tiled: one lattice chunk of CT frames x CU label positions at a time.
  // The logit-gradient kernel splits the vocabulary tiles of each cell tile
  // over several workgroups when a chunk alone has too few cell tiles to
  // give every compute unit (256 on gfx950) about four of them, as long as
  // each part keeps at least 8 vocabulary tiles: every part rebuilds the
  // tile's h rows and posteriors, which shorter parts do not amortise.
  const int chunk_tiles = p.cap_chunk;
  const int nvt = (V + kVocabTile - 1) / kVocabTile;
  int vsplit = 1;
  while (chunk_tiles * vsplit < 1024 && nvt / (2 * vsplit) >= 8) vsplit *= 2;
  int32_t* ctiles = at<int32_t>(workspace, p.o_ws_tiles);
  int32_t* ccount = at<int32_t>(workspace, p.o_ws_tcount);
  if ((e = timed("tile_list", st, [&] {
         return launch_tile_list(Teff, Ueff, p.d, p.CT, p.CU, p.n_cu_chunks, p.n_chunks,
                                 p.cap_chunk, ctiles, ccount, st);
       })) != hipSuccess)
    return RNNTJ_ERR_HIP;
  int chunk = 0;
  for (int ct0 = 0; ct0 < p.d.Tpad; ct0 += p.CT) {
    for (int cu0 = 0; cu0 < p.d.U1pad; cu0 += p.CU, ++chunk) {
      a.ct0 = ct0;
      a.cu0 = cu0;
      a.CT = p.CT;
      a.CU = p.CU;
      a.n_tu = p.CU / kTileU;
      a.vsplit = vsplit;
      a.gout = gchunk;
      a.hout = hchunk;
      a.tiles = ctiles + (size_t)chunk * p.cap_chunk;
      a.tile_count = ccount + chunk;
      if ((e = timed("joint_grad", st, [&] {
             return launch_joint_tile(a, kGrad, p.bf16, p.cap_chunk * vsplit, st);
           })) != hipSuccess)
        return RNNTJ_ERR_HIP;
      h.g = gchunk;
      h.ct0 = ct0; h.cu0 = cu0; h.CT = p.CT; h.CU = p.CU;
      h.tiles = a.tiles;
      h.tile_count = a.tile_count;
      if ((e = timed("dh", st, [&] { return launch_dh(h, p.bf16, p.cap_chunk, st); })) !=
          hipSuccess)
        return RNNTJ_ERR_HIP;
      w.g = gchunk;
      w.ct0 = ct0; w.cu0 = cu0; w.CT = p.CT; w.CU = p.CU;
      w.tiles = a.tiles;
      w.tile_count = a.tile_count;
      w.kparts = kparts_for(p.cap_chunk);
      if ((e = timed("dw", st, [&] { return launch_dw(w, p.bf16, st); })) != hipSuccess)
        return RNNTJ_ERR_HIP;
    }
  }
  return finalize(nullptr) == hipSuccess ? RNNTJ_OK : RNNTJ_ERR_HIP;
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
  if (misaligned(x) || misaligned(W) || misaligned(dy) || misaligned(dx) || misaligned(dW))
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
        return launch_proj_dw(x, dy, bf16, M, K, N, dW, db, device_cu_count(), st);
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
