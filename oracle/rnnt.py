"""Float64 oracle: RNN-T joint network + transducer loss (full sum over
alignments, or its maximum approximation), fwd + bwd.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

Notation (per utterance b): T' = T_lens[b] >= 1 frames, U' = U_lens[b] >= 0
labels y_0..y_{U'-1} = labels[b, :U'].  A lattice cell is (t, u) with
0 <= t < T' and 0 <= u <= U'.  pred row u is the prediction state after u
labels, so the emission at (t, u) scores y_u.

Joint ("Daily Papers" page, Transformer-Transducer abstract: a feed-forward
combination of the two encodings gives one label distribution per
(frame, label history); "Flash RNN-T" page, Abstract: joint + loss):

    h(t,u) = tanh(enc[t] + pred[u]),   z(t,u) = h(t,u) @ W_out + b_out
    lse(t,u) = log sum_v exp z(t,u)[v]
    LB(t,u) = z(t,u)[blank] - lse(t,u),   LE(t,u) = z(t,u)[y_u] - lse(t,u)

Lattice ("Daily Papers" page, abstract on sequence transduction with
recurrent networks; abstract on full-sum vs maximum approximation -- the full
sum is used): an alignment is a monotone path from (0,0) that takes a blank
step (t,u)->(t+1,u) with log-weight LB(t,u) or a label step (t,u)->(t,u+1)
with log-weight LE(t,u), and ends with the blank emitted at (T'-1, U').

    alpha(0,0) = 0
    alpha(t,u) = logaddexp(alpha(t-1,u) + LB(t-1,u), alpha(t,u-1) + LE(t,u-1))
    logP       = alpha(T'-1,U') + LB(T'-1,U'),   cost = -logP
    beta(T'-1,U') = LB(T'-1,U')
    beta(t,u)  = logaddexp(beta(t+1,u) + LB(t,u), beta(t,u+1) + LE(t,u))

Transition posteriors and gradient of sum_b gc_b * cost_b:

    gB(t,u) = exp(alpha(t,u) + LB(t,u) + beta(t+1,u) - logP)   (t < T'-1)
    gB(T'-1,U') = exp(alpha(T'-1,U') + LB(T'-1,U') - logP)      (= 1)
    gB(T'-1,u<U') = 0
    gE(t,u) = exp(alpha(t,u) + LE(t,u) + beta(t,u+1) - logP)    (u < U')
    gE(t,U') = 0
    dL/dz(t,u)[v] = gc * ((gB+gE) * softmax(z)[v] - gB*[v=blank] - gE*[v=y_u])
    dW_out += h^T dz,  db_out += dz,  dh = dz @ W_out^T,  dpre = (1 - h^2) * dh
    dEnc[t] += dpre(t,u) over u,  dPred[u] += dpre(t,u) over t

Maximum approximation ("Daily Papers" page, abstract comparing the full-sum
criterion with the maximum approximation; read here as the single best
alignment): the sum over alignments becomes a maximum,

    alpha*(t,u) = max(alpha*(t-1,u) + LB(t-1,u), alpha*(t,u-1) + LE(t,u-1))
    logP* = alpha*(T'-1,U') + LB(T'-1,U'),   cost = -logP*

the best alignment is read back from the predecessor decisions (on equal
scores the blank predecessor (t-1,u) is taken), and the posteriors become
that alignment's transition indicators: gB(t,u) = 1 where it takes the blank
step out of (t,u) (including the final blank), gE(t,u) = 1 where it takes the
label step.  The gradient is the formula above with these 0/1 posteriors
(the cost is -sum of the path's log-probabilities; the path is constant where
the maximum is unique).

Cells outside (t < T', u <= U') do not exist: the gradients of enc rows t >= T',
pred rows u > U' are exactly zero and labels past U' are never read.

Loops run over t (one lattice row at a time, vectorised over u) and over the
anti-diagonals t+u of the lattice; nothing larger than one row of logits
[U'+1, V] is held at a time.
"""
from __future__ import annotations

import itertools
import math
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

NEG_INF = -np.inf


def _logsumexp_rows(z: np.ndarray) -> np.ndarray:
    m = np.max(z, axis=1)
    return m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))


def _row(enc_b, pred_b, W, b_out, t, Up1):
    """h and z for lattice row t (all u <= U'): shapes [U'+1, H], [U'+1, V]."""
    h = np.tanh(enc_b[t][None, :] + pred_b[:Up1])
    z = h @ W + b_out[None, :]
    return h, z


def cell_scores(enc_b, pred_b, W, b_out, y, T_len, U_len, blank):
    """lse, LB [T', U'+1] and LE [T', U'] (float64) for one utterance."""
    enc_b = np.asarray(enc_b, np.float64)
    pred_b = np.asarray(pred_b, np.float64)
    W = np.asarray(W, np.float64)
    b_out = np.asarray(b_out, np.float64)
    Up1 = U_len + 1
    lse = np.empty((T_len, Up1))
    LB = np.empty((T_len, Up1))
    LE = np.empty((T_len, U_len))
    us = np.arange(U_len)
    for t in range(T_len):
        _, z = _row(enc_b, pred_b, W, b_out, t, Up1)
        lse[t] = _logsumexp_rows(z)
        LB[t] = z[:, blank] - lse[t]
        LE[t] = z[us, y[:U_len]] - lse[t, :U_len]
    return lse, LB, LE


def alpha_lattice(LB, LE):
    """Forward variables alpha [T', U'+1] and logP, one anti-diagonal at a time."""
    T_len, Up1 = LB.shape
    alpha = np.full((T_len, Up1), NEG_INF)
    alpha[0, 0] = 0.0
    for d in range(1, T_len + Up1 - 1):
        u = np.arange(max(0, d - T_len + 1), min(d, Up1 - 1) + 1)
        t = d - u
        from_t = np.full(u.shape, NEG_INF)
        ok = t >= 1
        from_t[ok] = alpha[t[ok] - 1, u[ok]] + LB[t[ok] - 1, u[ok]]
        from_u = np.full(u.shape, NEG_INF)
        ok = u >= 1
        from_u[ok] = alpha[t[ok], u[ok] - 1] + LE[t[ok], u[ok] - 1]
        alpha[t, u] = np.logaddexp(from_t, from_u)
    logP = alpha[T_len - 1, Up1 - 1] + LB[T_len - 1, Up1 - 1]
    return alpha, logP


def beta_lattice(LB, LE):
    """Backward variables beta [T', U'+1]; beta(0,0) equals logP."""
    T_len, Up1 = LB.shape
    beta = np.full((T_len, Up1), NEG_INF)
    beta[T_len - 1, Up1 - 1] = LB[T_len - 1, Up1 - 1]
    for d in range(T_len + Up1 - 3, -1, -1):
        u = np.arange(max(0, d - T_len + 1), min(d, Up1 - 1) + 1)
        t = d - u
        from_t = np.full(u.shape, NEG_INF)
        ok = t + 1 < T_len
        from_t[ok] = beta[t[ok] + 1, u[ok]] + LB[t[ok], u[ok]]
        from_u = np.full(u.shape, NEG_INF)
        ok = u + 1 < Up1
        from_u[ok] = beta[t[ok], u[ok] + 1] + LE[t[ok], u[ok]]
        beta[t, u] = np.logaddexp(from_t, from_u)
    return beta


def viterbi_lattice(LB, LE):
    """Maximum approximation: alpha* [T', U'+1], logP* and the best
    alignment's transition indicators gB, gE [T', U'+1] (0/1)."""
    T_len, Up1 = LB.shape
    alpha = np.full((T_len, Up1), NEG_INF)
    from_blank = np.zeros((T_len, Up1), dtype=bool)  # predecessor is (t-1, u)
    alpha[0, 0] = 0.0
    for d in range(1, T_len + Up1 - 1):
        u = np.arange(max(0, d - T_len + 1), min(d, Up1 - 1) + 1)
        t = d - u
        from_t = np.full(u.shape, NEG_INF)
        ok = t >= 1
        from_t[ok] = alpha[t[ok] - 1, u[ok]] + LB[t[ok] - 1, u[ok]]
        from_u = np.full(u.shape, NEG_INF)
        ok = u >= 1
        from_u[ok] = alpha[t[ok], u[ok] - 1] + LE[t[ok], u[ok] - 1]
        pick_t = from_t >= from_u
        alpha[t, u] = np.where(pick_t, from_t, from_u)
        from_blank[t, u] = pick_t
    logP = alpha[T_len - 1, Up1 - 1] + LB[T_len - 1, Up1 - 1]
    gB = np.zeros((T_len, Up1))
    gE = np.zeros((T_len, Up1))
    t, u = T_len - 1, Up1 - 1
    gB[t, u] = 1.0  # the final blank
    while (t, u) != (0, 0):
        if from_blank[t, u]:
            t -= 1
            gB[t, u] = 1.0
        else:
            u -= 1
            gE[t, u] = 1.0
    return alpha, logP, gB, gE


def posteriors(alpha, beta, LB, LE, logP):
    """Blank and label transition posteriors gB, gE [T', U'+1]."""
    T_len, Up1 = LB.shape
    gB = np.zeros((T_len, Up1))
    gE = np.zeros((T_len, Up1))
    if T_len > 1:
        gB[:-1, :] = np.exp(alpha[:-1, :] + LB[:-1, :] + beta[1:, :] - logP)
    gB[T_len - 1, Up1 - 1] = np.exp(alpha[T_len - 1, Up1 - 1] + LB[T_len - 1, Up1 - 1] - logP)
    if Up1 > 1:
        gE[:, :-1] = np.exp(alpha[:, :-1] + LE + beta[:, 1:] - logP)
    return gB, gE


def utterance_loss_and_grads(enc_b, pred_b, W, b_out, y, T_len, U_len, blank,
                             grad_cost=1.0, want_cell_grads=False, criterion="sum"):
    """Cost and gradients of grad_cost * cost for one utterance.

    criterion "sum" (full sum over alignments) or "max" (maximum
    approximation).  Returns a dict: cost, logP, dEnc [T', H], dPred [U'+1, H],
    dW [H, V], db [V], lse, LB, LE, alpha, beta (None for "max"), gB, gE and,
    if want_cell_grads, the per-cell logit gradients dz [T', U'+1, V] (small
    shapes only)."""
    enc_b = np.asarray(enc_b, np.float64)
    pred_b = np.asarray(pred_b, np.float64)
    W = np.asarray(W, np.float64)
    b_out = np.asarray(b_out, np.float64)
    y = np.asarray(y)
    H, V = W.shape
    Up1 = U_len + 1
    lse, LB, LE = cell_scores(enc_b, pred_b, W, b_out, y, T_len, U_len, blank)
    if criterion == "max":
        alpha, logP, gB, gE = viterbi_lattice(LB, LE)
        beta = None
    else:
        assert criterion == "sum", criterion
        alpha, logP = alpha_lattice(LB, LE)
        beta = beta_lattice(LB, LE)
        gB, gE = posteriors(alpha, beta, LB, LE, logP)
    dEnc = np.zeros((T_len, H))
    dPred = np.zeros((Up1, H))
    dW = np.zeros((H, V))
    db = np.zeros(V)
    cell_grads = np.zeros((T_len, Up1, V)) if want_cell_grads else None
    us = np.arange(U_len)
    for t in range(T_len):
        h, z = _row(enc_b, pred_b, W, b_out, t, Up1)
        p = np.exp(z - lse[t][:, None])
        dz = (gB[t] + gE[t])[:, None] * p
        dz[:, blank] -= gB[t]
        dz[us, y[:U_len]] -= gE[t, :U_len]
        dz *= grad_cost
        if want_cell_grads:
            cell_grads[t] = dz
        dW += h.T @ dz
        db += dz.sum(axis=0)
        dpre = (1.0 - h * h) * (dz @ W.T)
        dEnc[t] = dpre.sum(axis=0)
        dPred += dpre
    return dict(cost=-logP, logP=logP, dEnc=dEnc, dPred=dPred, dW=dW, db=db,
                lse=lse, LB=LB, LE=LE, alpha=alpha, beta=beta, gB=gB, gE=gE,
                cell_grads=cell_grads)


def _utt_job(args):
    (enc_b, pred_b, W, b_out, y, T_len, U_len, blank, gc, threads, criterion) = args
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads):
            return utterance_loss_and_grads(enc_b, pred_b, W, b_out, y, T_len,
                                            U_len, blank, gc, criterion=criterion)
    except ImportError:  # pragma: no cover
        return utterance_loss_and_grads(enc_b, pred_b, W, b_out, y, T_len, U_len,
                                        blank, gc, criterion=criterion)


def loss_and_grads(enc, pred, W, b_out, labels, T_lens, U_lens, blank,
                   grad_costs=None, workers=1, keep_cells=False, criterion="sum"):
    """Batched costs [B] and gradients (dEnc [B,T,H], dPred [B,U+1,H],
    dW [H,V], db [V]), float64.  ``workers`` > 1 runs utterances in a
    process pool.  With keep_cells the per-utterance dicts are returned too."""
    enc = np.asarray(enc, np.float64)
    pred = np.asarray(pred, np.float64)
    W = np.asarray(W, np.float64)
    b_out = np.asarray(b_out, np.float64)
    B, T, H = enc.shape
    V = W.shape[1]
    gcs = np.ones(B) if grad_costs is None else np.asarray(grad_costs, np.float64)
    jobs = []
    threads = max(1, (os.cpu_count() or 1) // max(1, workers))
    for b in range(B):
        jobs.append((enc[b], pred[b], W, b_out, np.asarray(labels[b]),
                     int(T_lens[b]), int(U_lens[b]), blank, gcs[b], threads, criterion))
    if workers > 1 and B > 1:
        # spawn, never fork: the caller may have initialised a GPU runtime
        ctx = multiprocessing.get_context("spawn")
        with ProcessPoolExecutor(max_workers=min(workers, B), mp_context=ctx) as ex:
            outs = list(ex.map(_utt_job, jobs))
    else:
        outs = [utterance_loss_and_grads(*j[:9], criterion=criterion) for j in jobs]
    costs = np.array([o["cost"] for o in outs])
    dEnc = np.zeros((B, T, H))
    dPred = np.zeros((B, pred.shape[1], H))
    dW = np.zeros((H, V))
    db = np.zeros(V)
    for b, o in enumerate(outs):
        dEnc[b, :o["dEnc"].shape[0]] = o["dEnc"]
        dPred[b, :o["dPred"].shape[0]] = o["dPred"]
        dW += o["dW"]
        db += o["db"]
    res = dict(costs=costs, dEnc=dEnc, dPred=dPred, dW=dW, db=db)
    if keep_cells:
        res["utts"] = outs
    return res


def loss_only(enc, pred, W, b_out, labels, T_lens, U_lens, blank, criterion="sum"):
    """Costs [B] only (forward scores + alpha recursion)."""
    out = []
    for b in range(len(T_lens)):
        _, LB, LE = cell_scores(enc[b], pred[b], W, b_out, np.asarray(labels[b]),
                                int(T_lens[b]), int(U_lens[b]), blank)
        if criterion == "max":
            _, logP, _, _ = viterbi_lattice(LB, LE)
        else:
            _, logP = alpha_lattice(LB, LE)
        out.append(-logP)
    return np.array(out)


def brute_force_utterance(LB, LE, criterion="sum"):
    """Enumerate every alignment of one utterance (small T', U' only).

    "sum": logP = log of the summed path probabilities and the posteriors
    gB, gE obtained by adding up the probability of every path that takes each
    transition.  "max": logP = the largest path log-probability and gB, gE the
    transitions of that path (the first one enumerated on a tie)."""
    T_len, Up1 = LB.shape
    U_len = Up1 - 1
    n_moves = T_len - 1 + U_len          # moves before the final blank
    logws = []
    paths = []
    for label_slots in itertools.combinations(range(n_moves), U_len):
        slots = set(label_slots)
        t = u = 0
        lw = 0.0
        steps = []
        for k in range(n_moves):
            if k in slots:
                lw += LE[t, u]
                steps.append(("E", t, u))
                u += 1
            else:
                lw += LB[t, u]
                steps.append(("B", t, u))
                t += 1
        assert (t, u) == (T_len - 1, U_len)
        lw += LB[t, u]
        steps.append(("B", t, u))
        logws.append(lw)
        paths.append(steps)
    logws = np.array(logws)
    m = logws.max()
    gB = np.zeros((T_len, Up1))
    gE = np.zeros((T_len, Up1))
    if criterion == "max":
        for kind, t, u in paths[int(np.argmax(logws))]:
            (gB if kind == "B" else gE)[t, u] = 1.0
        return m, gB, gE, len(paths)
    logP = m + math.log(np.sum(np.exp(logws - m)))
    for lw, steps in zip(logws, paths):
        w = math.exp(lw - logP)
        for kind, t, u in steps:
            if kind == "B":
                gB[t, u] += w
            else:
                gE[t, u] += w
    return logP, gB, gE, len(paths)


def closed_form_zero_weights(T_len, U_len, y, b_out, blank):
    """Cost when W_out = 0: every cell has the same distribution
    p = softmax(b_out); every alignment has the same probability
    p_blank^T' * prod_u p_{y_u}, and there are C(T'+U'-1, U') of them."""
    b_out = np.asarray(b_out, np.float64)
    logp = b_out - (b_out.max() + math.log(np.sum(np.exp(b_out - b_out.max()))))
    n_paths = math.comb(T_len + U_len - 1, U_len)
    return -(T_len * logp[blank] + sum(logp[int(k)] for k in y[:U_len])
             + math.log(n_paths))


def closed_form_zero_weights_max(T_len, U_len, y, b_out, blank):
    """Maximum-approximation cost when W_out = 0: all alignments have the same
    probability, so the best one is any of them."""
    b_out = np.asarray(b_out, np.float64)
    logp = b_out - (b_out.max() + math.log(np.sum(np.exp(b_out - b_out.max()))))
    return -(T_len * logp[blank] + sum(logp[int(k)] for k in y[:U_len]))
