/*
 * rnnt_joint.h -- C ABI of the fused RNN-T joint network + transducer loss
 * (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed ("Flash RNN-T: Memory-Efficient Joint Network and
 * Transducer Loss Computation", Abstract: the joint and the loss are evaluated
 * over the full alignment space and the full vocabulary, untiled or with tiled
 * recomputation; "Daily Papers" page, Transformer-Transducer abstract: one
 * label distribution per (frame, label history) from a feed-forward
 * combination of the two encodings; "Daily Papers" page, abstract on sequence
 * transduction with recurrent networks: the loss sums over every alignment):
 *
 *   for every utterance b and lattice cell (t, u), t < T'_b, u <= U'_b:
 *     h      = tanh(enc[b,t,:] + pred[b,u,:])                  [H]
 *     z      = h @ W_out + b_out                               [V]
 *     LB     = log_softmax(z)[blank],  LE = log_softmax(z)[labels[b,u]]  (u < U')
 *   alpha/beta recursions over the lattice (blank: t -> t+1, label: u -> u+1,
 *   final blank at (T'-1, U')),  costs[b] = -log P(labels_b | enc_b, pred_b);
 *   backward: gradients of sum_b grad_costs[b] * costs[b] with respect to
 *   enc, pred, W_out and b_out.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller: contiguous,
 *     row-major, 16-byte aligned.  The library never allocates, frees or keeps
 *     device memory between calls and is reentrant; its only global state is
 *     the optional kernel-timing record (rnnt_joint_loss_timing, below).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronising, except
 *     rnnt_joint_loss_status, which synchronises `stream`.
 *   - Shapes: enc [B,T,H], pred [B,U+1,H] (row 0 = state before any label,
 *     row u = state after u labels), W_out [H,V], b_out [V], labels int32
 *     [B,U] (labels[b,u] is the (u+1)-th label), T_lens / U_lens int32 [B].
 *     enc, pred, W_out and b_out all have type `dtype`; costs and every
 *     gradient are float32 whatever `dtype` is.
 *   - Modes: tile_t == 0 and tile_u == 0 selects the UNTILED mode: the forward
 *     stores the logits (dtype) in `saved` and the backward turns them into
 *     the logit gradients in place, so one forward feeds one backward.
 *     Otherwise the TILED mode stores only per-cell scalars and recomputes the
 *     joint and logits in the backward, one lattice chunk of tile_t frames x
 *     tile_u label positions (all utterances) at a time; 0 on one axis means
 *     the whole axis.  tile_t must be a multiple of 16 and tile_u of 8.
 *     tile_v bounds the vocabulary columns of one step of the online max /
 *     log-sum-exp (which never materialises more than one step of logits per
 *     cell): 0 or any multiple of 128.  The kernels step by 128 columns (64
 *     for bf16 with H <= 256), which is within every accepted bound, so tile_v
 *     changes neither memory nor results (the order of the floating-point sums
 *     is the same).
 *   - Limits (else RNNTJ_ERR_UNSUPPORTED): H a multiple of 16 with
 *     16 <= H <= 768 for bf16 and H <= 256 for fp32; V a multiple of 8,
 *     8 <= V <= 262144; U + 1 <= 512; B <= 8191; T <= 65520.
 *   - Host-side argument errors (null pointers, bad shapes, blank outside
 *     [0,V), unsupported tiles, workspace too small) return a nonzero code
 *     before anything is enqueued; outputs are untouched.
 *   - Data errors are detected on the device: T'_b outside [1,T], U'_b outside
 *     [0,U], or labels[b,u] (u < U'_b) outside [0,V) or equal to blank.  The
 *     utterance then gets costs[b] = NaN and zero gradients, and a status
 *     word in `saved` is set; rnnt_joint_loss_status reports it.
 *   - NaN / Inf in the float inputs propagate to the outputs; they are not
 *     reported as errors.
 */
#ifndef RNNT_JOINT_H_
#define RNNT_JOINT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RNNTJ_ABI_VERSION 1

enum rnntj_dtype { RNNTJ_F32 = 0, RNNTJ_BF16 = 1 };

/* Training criterion ("Daily Papers" page, abstract comparing the full-sum
 * RNN-T criterion with the maximum approximation):
 *   RNNTJ_CRIT_SUM  cost = -log of the probability summed over all alignments;
 *   RNNTJ_CRIT_MAX  cost = -log of the probability of the best alignment
 *                   (ties between a cell's two predecessors go to the blank
 *                   step (t-1,u) -> (t,u)); gradients flow through that
 *                   alignment only (its transitions' posteriors are 1, all
 *                   others 0). */
enum rnntj_criterion { RNNTJ_CRIT_SUM = 0, RNNTJ_CRIT_MAX = 1 };

enum rnntj_status {
  RNNTJ_OK = 0,
  RNNTJ_ERR_ARG = 1,          /* null pointer, non-positive size, blank out of range */
  RNNTJ_ERR_UNSUPPORTED = 2,  /* shape or tile outside the limits above */
  RNNTJ_ERR_WORKSPACE = 3,    /* workspace_bytes smaller than required */
  RNNTJ_ERR_HIP = 4,          /* a HIP launch or copy failed */
  RNNTJ_ERR_DATA = 5          /* (status only) invalid lengths or labels seen on the device */
};

/* Version of this ABI (RNNTJ_ABI_VERSION of the built library). */
int rnnt_joint_loss_abi_version(void);

/* Human-readable text for a status code; never NULL, static storage. */
const char* rnnt_joint_loss_strerror(int code);

/* Text naming the kernel launch and HIP error behind the calling thread's
 * most recent RNNTJ_ERR_HIP ("" if none); never NULL, thread-local storage. */
const char* rnnt_joint_loss_last_error(void);

/*
 * Bytes of the forward -> backward state `saved` for these sizes and tiles.
 * saved holds the per-utterance validated lengths, log P and status, a
 * transposed copy of W_out, e^{2 enc} and e^{2 pred} (float32), and per cell
 * (diagonal-skewed [B, T+U, U+1]): lse, LB, LE (float32) and alpha, beta
 * (float64), and the list of active 16 x 8 cell tiles (int32, one word per
 * tile of the padded lattice).  In the untiled mode it also holds the logits
 * [B, ceil16(T), ceil8(U+1), V] in dtype and the joint activations h
 * [B, ceil16(T), ceil8(U+1), H] of the active tiles in dtype.
 * Writes *out; returns a status code.
 */
int rnnt_joint_loss_saved_bytes(int B, int T, int U, int H, int V, int dtype,
                                int tile_t, int tile_u, int tile_v, size_t* out);

/*
 * Bytes of scratch `workspace` needed by the forward (pass = 0) or the
 * backward (pass = 1).  The forward needs none.  The backward needs a float64
 * accumulator for d_b_out [V] and, in the tiled mode, the joint activations
 * h of one lattice chunk [B, tile_t, tile_u, H] in dtype (untiled: none,
 * they are in `saved`), that chunk's logit gradients [B, tile_t, tile_u, V]
 * in dtype plus the active-tile list of every chunk (int32, one word per
 * 16 x 8 tile).  Writes *out; returns a status code.
 */
int rnnt_joint_loss_workspace_bytes(int B, int T, int U, int H, int V, int dtype,
                                    int tile_t, int tile_u, int tile_v, int pass,
                                    size_t* out);

/*
 * Forward: costs[b] = -log P(labels_b) for every utterance, and the state the
 * backward needs, written into `saved` (rnnt_joint_loss_saved_bytes bytes,
 * caller-owned, contents overwritten).  enc/pred/W_out/b_out are read only.
 * Launch order on `stream`: length/label validation, W_out transpose, fused
 * joint + projection + online log-sum-exp (+ logit and h-row store when
 * untiled),
 * alpha/beta lattice recursion.  Returns a status code (host-side checks and
 * launch errors only).
 */
int rnnt_joint_loss_fwd(const void* enc, const void* pred, const void* W_out,
                        const void* b_out, int dtype, const int32_t* labels,
                        const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                        int U, int H, int V, int blank, int tile_t, int tile_u,
                        int tile_v, float* costs, void* saved, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Forward with a choice of criterion (rnntj_criterion; rnnt_joint_loss_fwd is
 * this with RNNTJ_CRIT_SUM).  The criterion is recorded in `saved`, and the
 * backward from that state follows it: with RNNTJ_CRIT_MAX the alpha pass is
 * the max-plus recursion and the best alignment is read back into `saved`.
 * Buffer sizes are the same for both criteria.  An unknown criterion returns
 * RNNTJ_ERR_ARG before anything is enqueued.
 */
int rnnt_joint_loss_fwd_ex(const void* enc, const void* pred, const void* W_out,
                           const void* b_out, int dtype, const int32_t* labels,
                           const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                           int U, int H, int V, int blank, int tile_t, int tile_u,
                           int tile_v, int criterion, float* costs, void* saved,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward: overwrites d_enc [B,T,H], d_pred [B,U+1,H], d_W_out [H,V] and
 * d_b_out [V] (float32) with the gradients of sum_b grad_costs[b] * costs[b]
 * (grad_costs float32 [B] on the device, or NULL for all ones).  Takes the
 * same inputs, sizes and tiles as the forward that filled `saved`; the whole
 * batch is handled in one call.  Tiled mode: `saved` is only read, so one
 * forward may feed several backward calls.  Untiled mode: the stored logits
 * become the logit gradients in place and `saved` is marked consumed; a
 * second backward from it gives invalid gradients and sets data-error bit 4
 * (rnnt_joint_loss_status).  Entries of d_enc / d_pred past each utterance's
 * lengths are zero.  Returns a status code (host-side checks and launch
 * errors only).
 */
int rnnt_joint_loss_bwd(const void* enc, const void* pred, const void* W_out,
                        const void* b_out, int dtype, const int32_t* labels,
                        const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                        int U, int H, int V, int blank, int tile_t, int tile_u,
                        int tile_v, const float* grad_costs, void* saved,
                        float* d_enc, float* d_pred, float* d_W_out, float* d_b_out,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronises `stream`, then copies the data-error word of `saved` to
 * *data_error: 0 = every utterance valid, else a bit mask (1 = a length out of
 * range, 2 = a label out of range or equal to blank, 4 = an untiled backward
 * ran on a state whose logits an earlier backward had already consumed).
 * Returns a status code.
 */
int rnnt_joint_loss_status(const void* saved, void* stream, int32_t* data_error);

/*
 * Joint input projections ("Daily Papers" page, Transformer-Transducer
 * abstract: the two encodings are combined by a feed-forward layer; read as
 * one affine map per encoding ahead of the joint's add):
 *     enc_p = enc @ W_enc + b_enc,   pred_p = pred @ W_pred + b_pred,
 * each computed by rnnt_joint_proj_fwd and fed to rnnt_joint_loss_fwd/bwd as
 * `enc` / `pred`; the d_enc / d_pred that the loss backward returns are the
 * `dy` of rnnt_joint_proj_bwd.
 *
 * rnnt_joint_proj_fwd: y[M,N] = x[M,K] @ W[K,N] + b[N].  x, W, b, y device
 * pointers of `dtype` (row-major, contiguous; b may be NULL for no bias);
 * products accumulate in fp32 and y is rounded once to dtype.  y must not
 * overlap x, W or b.  For enc: M = B*T, K = E (input width),
 * N = H; for pred: M = B*(U+1), K = P, N = H.
 *
 * rnnt_joint_proj_bwd: from dy[M,N] (float32) writes dx[M,K] = dy @ W^T,
 * dW[K,N] = x^T @ dy and db[N] = sum of the rows of dy, all float32 and
 * overwritten (dx and db may be NULL to skip them).  x and W as in the
 * forward; the outputs must not overlap each other or the inputs.
 *
 * Both: x, W, y / dy, dx, dW 16-byte aligned; K and N multiples of 16 and at
 * most 65536, M >= 1 (else RNNTJ_ERR_UNSUPPORTED / RNNTJ_ERR_ARG, returned
 * before anything is enqueued).  Kernels run on `stream` (hipStream_t, NULL =
 * default stream) and allocate nothing; results are ready when the stream
 * reaches them.  Returns a status code.
 */
int rnnt_joint_proj_fwd(const void* x, const void* W, const void* b, int dtype, int M, int K,
                        int N, void* y, void* stream);
int rnnt_joint_proj_bwd(const void* x, const void* W, int dtype, int M, int K, int N,
                        const float* dy, float* dx, float* dW, float* db, void* stream);

/*
 * Kernel timing (measurement aid; no counterpart on the pages).
 * rnnt_joint_loss_timing(1) makes every later call bracket each kernel it
 * enqueues with a pair of HIP events recorded on that call's `stream`;
 * rnnt_joint_loss_timing(0) stops it and drops pending events.  Process-wide
 * and not thread-safe; off by default.  Events are host-side HIP resources,
 * not device memory.
 * rnnt_joint_loss_timing_report waits for the recorded events, writes one
 * line "<kernel> <launches> <total_ms>\n" per kernel name into buf (NUL
 * terminated, truncated to len), frees the events and clears the record.
 */
int rnnt_joint_loss_timing(int enable);
int rnnt_joint_loss_timing_report(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* RNNT_JOINT_H_ */
