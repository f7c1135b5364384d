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
 *     the optional kernel-timing record (rnnt_joint_loss_timing, below) and
 *     the static scratch array of rnnt_joint_loss_bwd_noalloc (one per GPU).
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
 *     the logit gradients in place, so one forward feeds one backward.  In
 *     bf16 each row's logits are stored relative to the row's largest logit
 *     within each vocabulary step of the forward kernel (64 or 128 columns),
 *     with those offsets kept in float32: the rounding error of a stored
 *     logit then moves its softmax entry by at most 2^-8 / e, whatever the
 *     size of the logits.
 *     Otherwise the TILED mode stores only per-cell scalars and recomputes the
 *     joint and logits in the backward, one lattice chunk of tile_t frames x
 *     tile_u label positions (all utterances) at a time; 0 on one axis means
 *     the whole axis.  tile_t must be a multiple of 16 and tile_u of 8.
 *     tile_v (0 or a multiple of 128; 0 = the whole vocabulary) splits each
 *     chunk of the tiled backward into vocabulary parts of tile_v columns:
 *     the logit gradients of one part alone are held in the workspace (its
 *     size falls with tile_v), and every part recomputes the joint for its
 *     columns.  It is also an upper bound on the columns of one step of the
 *     online max / log-sum-exp, which the kernels keep at 128 (64 for bf16
 *     with H <= 256).  The untiled mode stores whole rows of logits and
 *     ignores tile_v.
 *   - Limits (else RNNTJ_ERR_UNSUPPORTED): H a multiple of 16 with
 *     16 <= H <= 768; V a multiple of 8,
 *     8 <= V <= 262144; U + 1 <= 1024 (512 for the pruned and the
 *     token-and-duration entry points); B <= 8191; T <= 65520.
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

/*
 * Process-wide switches (robustness aids; no counterpart on the pages).
 * Initialised when the library loads from the environment: RNNTJ_DEBUG=1 sets
 * RNNTJ_FLAG_DEBUG, RNNTJ_DETERMINISTIC=1 sets RNNTJ_FLAG_DETERMINISTIC.
 *   RNNTJ_FLAG_DEBUG: every call waits for each of its kernels and returns
 *     RNNTJ_ERR_HIP naming the first one that fails (rnnt_joint_loss_last_error),
 *     and the forward and backward return RNNTJ_ERR_DATA when the state's
 *     data-error word is nonzero at their end (results are written as usual).
 *   RNNTJ_FLAG_DETERMINISTIC: the backward reduces d_enc, d_pred, d_W_out and
 *     d_b_out through partial-sum buffers added in a fixed order instead of
 *     float atomics, so repeated calls give bitwise identical gradients.  The
 *     backward workspace is larger in this mode (rnnt_joint_loss_workspace_bytes
 *     reports the size for the current flags).  The token-and-duration head's
 *     own reductions and the projection gradients keep their atomics.
 * Changing the flags while calls are in flight on other threads is not
 * supported.  set returns RNNTJ_ERR_ARG for unknown bits.
 */
#define RNNTJ_FLAG_DEBUG 1
#define RNNTJ_FLAG_DETERMINISTIC 2
int rnnt_joint_loss_get_flags(void);
int rnnt_joint_loss_set_flags(int flags);

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
 * [B, ceil16(T), ceil8(U+1), H] of the active tiles in dtype, and for bf16
 * the float32 offsets of the stored logits (one per row and vocabulary step
 * of 64 columns when H <= 256, else 128).  A 32-byte header records the
 * status, the criterion and what a backward must match (sizes, dtype, blank,
 * whether the logits are stored).
 * Writes *out; returns a status code.
 */
int rnnt_joint_loss_saved_bytes(int B, int T, int U, int H, int V, int dtype,
                                int tile_t, int tile_u, int tile_v, size_t* out);

/*
 * Bytes of scratch `workspace` needed by the forward (pass = 0) or the
 * backward (pass = 1: the size for the fastest schedule; pass = 2: the
 * least the backward accepts).  The forward needs none.  The backward needs
 * a float64 accumulator for d_b_out [V] and, in the tiled mode, the joint
 * activations h of one lattice chunk [B, tile_t, tile_u, H] in dtype
 * (untiled: none, they are in `saved`), that chunk's logit gradients of one
 * vocabulary part [B, tile_t, tile_u, min(tile_v, V)] (tile_v = 0: V) in
 * dtype plus the active-tile list of every chunk (int32, one word per
 * 16 x 8 tile); in the deterministic mode (rnnt_joint_loss_set_flags) also
 * its partial-sum buffers.  That is pass 2.  Pass 1 adds, in the tiled mode,
 * a second pair of chunk buffers: given that much, the tiled backward
 * alternates the pairs between consecutive chunks and runs each chunk's dW
 * GEMM on a library-owned side stream of the same device (created once,
 * default priority), so that it overlaps that chunk's dh GEMM and the next
 * chunk's logit gradients; events join the side stream back to `stream`
 * before the call returns, so the results are ordered on `stream` as
 * always.  Given less than pass 1 (and at least pass 2), every kernel runs
 * on `stream` in order.  The results are the same either way.  Writes *out;
 * returns a status code.
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
 * (rnnt_joint_loss_status).  The backward checks on the device, before it
 * reads anything but the header of `saved`, that the state comes from a
 * forward with the same B, T, U, H, V, dtype and blank (and, for the untiled
 * backward, one that stored the logits; a tiled backward accepts an untiled
 * forward's state): otherwise it computes nothing, leaves the gradients zero
 * and sets data-error bit 8.  Entries of d_enc / d_pred past each utterance's
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
 * Backward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as rnnt_joint_loss_bwd without `workspace` / `workspace_bytes`: the
 * backward's scratch is instead a static device array of
 * RNNTJ_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends.  Sizes whose backward workspace
 * (rnnt_joint_loss_workspace_bytes, pass 2) exceeds it return
 * RNNTJ_ERR_WORKSPACE before anything is enqueued: this covers the untiled
 * mode at every accepted size and the tiled mode while one chunk's logit
 * gradients and activations fit.  `stream` must belong to the calling
 * thread's current device (else RNNTJ_ERR_ARG).  No hipMalloc / hipFree or
 * allocating library call is made, and every kernel runs on `stream` (no
 * side stream).  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents (the backward clears what it
 * needs zeroed itself): calls that overlap on one GPU race, so serialise
 * them (for example, issue them on one stream).
 */
#define RNNTJ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int rnnt_joint_loss_bwd_noalloc(const void* enc, const void* pred, const void* W_out,
                                const void* b_out, int dtype, const int32_t* labels,
                                const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                                int U, int H, int V, int blank, int tile_t, int tile_u,
                                int tile_v, const float* grad_costs, void* saved,
                                float* d_enc, float* d_pred, float* d_W_out, float* d_b_out,
                                void* stream);

/*
 * Pruned transducer loss ("Pruned RNN-T for fast, memory-efficient ASR
 * training", Abstract: pruning bounds from a simple joiner linear in the two
 * embeddings, then the full joiner evaluated inside them).
 *
 * rnnt_joint_loss_pruned_fwd: as rnnt_joint_loss_fwd (full sum, TILED mode
 * only: tile_t or tile_u > 0), except that
 *   1. the simple joiner zs(t,u) = (enc[t] + pred[u]) @ W_out + b_out (the
 *      joiner without its tanh, same weights) is evaluated over the whole
 *      lattice in float64 without a [T, U+1, V] tensor; its cost goes to
 *      simple_costs[b] (float32 [B], or NULL to skip);
 *   2. each frame t gets a window of S label positions starting at s_t: the
 *      window centred on the frame's occupancy-weighted mean label position
 *      under the simple joiner's alignment posterior (rounded half up,
 *      clamped to [0, max(0, U'+1-S)]), then made to hold an alignment (first
 *      window at 0, starts non-decreasing and at most S-1 apart, last window
 *      at max(0, U'+1-S));
 *   3. costs[b] is minus the log of the full joiner's probability summed over
 *      the alignments that stay inside the windows.  With S >= U'+1 that is
 *      the full-sum cost.
 * The window starts are kept in `saved`; rnnt_joint_loss_bwd (tiled, same
 * arguments) then returns the gradients of sum_b grad_costs[b] costs[b] with
 * the windows held fixed, evaluating the full joiner only on cell tiles
 * that meet the band.  An utterance with U' > T' (S - 1) fits in no band: its
 * cost is NaN, its gradients zero, and data-error bit 16 is set.  S >= 1,
 * T <= 32000 (else RNNTJ_ERR_ARG / RNNTJ_ERR_UNSUPPORTED); the untiled mode
 * and the maximum approximation are not offered (RNNTJ_ERR_UNSUPPORTED).
 * `workspace` (device, 16-byte aligned) holds the float64 simple-joiner
 * lattice: rnnt_joint_loss_pruned_workspace_bytes bytes (about
 * 8 B (T + U + 1) V + 40 B (T+U)(U+1) per utterance).  `saved` is sized by
 * rnnt_joint_loss_saved_bytes with the same tiles.
 */
int rnnt_joint_loss_pruned_workspace_bytes(int B, int T, int U, int H, int V, int dtype,
                                           size_t* out);
/* Copies the window starts s_t of a pruned forward's `saved` (int32 [B, T],
 * entries past T'_b repeat the last window) to the device buffer `bounds`,
 * enqueued on `stream`.  Sizes and tiles as given to that forward. */
int rnnt_joint_loss_pruned_bounds(const void* saved, int B, int T, int U, int H, int V,
                                  int dtype, int tile_t, int tile_u, int tile_v,
                                  int32_t* bounds, void* stream);
int rnnt_joint_loss_pruned_fwd(const void* enc, const void* pred, const void* W_out,
                               const void* b_out, int dtype, const int32_t* labels,
                               const int32_t* T_lens, const int32_t* U_lens, int B, int T,
                               int U, int H, int V, int blank, int tile_t, int tile_u,
                               int tile_v, int S, float* costs, float* simple_costs,
                               void* saved, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Token-and-duration transducer ("Daily Papers" page, Token-and-Duration
 * Transducer abstract: the joint has two outputs, normalised independently,
 * over tokens and over durations -- the number of frames a token covers).
 *
 * A duration head W_dur [H, K], b_dur [K] (dtype) reads the same joint
 * hidden h = tanh(enc[t] + pred[u]) as the token head; durations[K] (HOST
 * int32 array, K <= 8 distinct values in [0, 15], at least one >= 1) lists
 * the frames each duration class covers.  P(v, d_k | t, u) =
 * softmax(h W_out + b_out)[v] * softmax(h W_dur + b_dur)[k].  Steps out of
 * cell (t,u): a blank of duration d_k >= 1 to (t + d_k, u) (a blank of
 * duration 0 would not move and is no step), label labels[b,u] (u < U') of
 * duration d_k to (t + d_k, u + 1); an alignment starts at (0,0), visits
 * cells t < T', u <= U' only and ends with a blank from (t, U') landing
 * exactly on t + d_k = T'.  costs[b] = -log of the sum over alignments.  An
 * utterance no alignment reaches (for example durations {1} with U' >= T')
 * gets cost +inf and zero gradients.
 *
 * Buffers: `saved` of rnnt_joint_loss_tdt_saved_bytes bytes (the plain state
 * plus the duration log-probabilities, float32 [cells, K]); the backward's
 * workspace of rnnt_joint_loss_tdt_workspace_bytes (pass 1, or at least
 * pass 2, as for rnnt_joint_loss_workspace_bytes) bytes (the plain
 * one plus the summed step posteriors, float64, and the duration-logit
 * gradients, float32; in deterministic mode also each 16-frame block's
 * d_W_dur / d_b_dur sums, so query it with the mode already set); the
 * forward needs none (pass 0).  Untiled and tiled
 * modes as in rnnt_joint_loss_fwd / _bwd; full sum over alignments.  The
 * backward overwrites d_enc, d_pred, d_W_out, d_b_out, d_W_dur [H, K] and
 * d_b_dur [K] (float32) and checks, like rnnt_joint_loss_bwd, that `saved`
 * comes from a forward with the same sizes, dtype, blank and durations
 * (else data-error bit 8, nothing computed).
 */
int rnnt_joint_loss_tdt_saved_bytes(int B, int T, int U, int H, int V, int dtype, int tile_t,
                                    int tile_u, int tile_v, int K, size_t* out);
int rnnt_joint_loss_tdt_workspace_bytes(int B, int T, int U, int H, int V, int dtype,
                                        int tile_t, int tile_u, int tile_v, int K, int pass,
                                        size_t* out);
int rnnt_joint_loss_tdt_fwd(const void* enc, const void* pred, const void* W_out,
                            const void* b_out, const void* W_dur, const void* b_dur, int dtype,
                            const int32_t* labels, const int32_t* T_lens, const int32_t* U_lens,
                            int B, int T, int U, int H, int V, int blank,
                            const int32_t* durations, int K, int tile_t, int tile_u, int tile_v,
                            float* costs, void* saved, void* workspace, size_t workspace_bytes,
                            void* stream);
int rnnt_joint_loss_tdt_bwd(const void* enc, const void* pred, const void* W_out,
                            const void* b_out, const void* W_dur, const void* b_dur, int dtype,
                            const int32_t* labels, const int32_t* T_lens, const int32_t* U_lens,
                            int B, int T, int U, int H, int V, int blank,
                            const int32_t* durations, int K, int tile_t, int tile_u, int tile_v,
                            const float* grad_costs, void* saved, float* d_enc, float* d_pred,
                            float* d_W_out, float* d_b_out, float* d_W_dur, float* d_b_dur,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Synchronises `stream`, then copies the data-error word of `saved` to
 * *data_error: 0 = every utterance valid, else a bit mask (1 = a length out of
 * range, 2 = a label out of range or equal to blank, 4 = an untiled backward
 * ran on a state whose logits an earlier backward had already consumed, 8 = a
 * backward was given a state whose sizes, dtype, blank or mode do not match
 * its own arguments and computed nothing, 16 = no pruning band of the pruned
 * forward holds an alignment of some utterance).
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
 * forward; the outputs must not overlap each other or the inputs.  In
 * deterministic mode the row splits of dW and db run one after another, so
 * each element's partial sums are added in a fixed order (bitwise
 * repeatable; fewer workgroups at a time).
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
