"""Float64 oracle: token-and-duration transducer loss ("Daily Papers" page,
Token-and-Duration Transducer abstract), fwd + bwd.

TEST INFRASTRUCTURE ONLY (tests and the benchmark's CPU baseline).

The abstract: the joint network has two outputs, normalised independently,
giving a distribution over tokens and one over durations, the number of
input frames the emitted token covers; at inference the duration lets the
model skip frames.  Readings taken here (one per point the abstract leaves
open):

* Durations: an explicit set D = (d_0, ..., d_{K-1}) of distinct non-negative
  integers, with at least one d >= 1.
* Heads: both read the joint hidden h(t,u) = tanh(enc[t] + pred[u]) of this
  path: token logits z = h W_out + b_out (blank included), duration logits
  zd = h W_dur + b_dur; P(v, d | t, u) = softmax(z)[v] softmax(zd)[d].
  LB = log P_tok(blank), LE = log P_tok(y_u), LD[k] = log P_dur(d_k).
* Steps out of cell (t,u) (t < T', u <= U'):
      blank with duration d >= 1:   (t,u) -> (t+d, u),    log-weight LB + LD[k]
      label y_u with duration d:    (t,u) -> (t+d, u+1),  log-weight LE + LD[k]  (u < U')
  A blank of duration 0 would not move: no alignment uses it.  An alignment
  starts at (0,0), visits cells only, and ends with a blank from (t, U') that
  lands exactly on t + d = T'.  (With D = {0, 1} and the label step taking
  only d = 0 and the blank only d = 1 this is the RNN-T lattice.)
* cost = -log of the sum over alignments of the product of their steps'
  probabilities; gradients of sum_b gc_b cost_b.

Recursions (cells in order of t, then u: every predecessor has a smaller t,
or the same t and u-1 through a label of duration 0):
    alpha(0,0) = 0
    alpha(t,u) = logsumexp over k of
                 alpha(t-d_k, u)   + LB(t-d_k, u)   + LD(t-d_k, u, k)    (d_k >= 1)
                 alpha(t-d_k, u-1) + LE(t-d_k, u-1) + LD(t-d_k, u-1, k)  (u >= 1)
    logP = logsumexp over k with d_k >= 1 of
           alpha(T'-d_k, U') + LB(T'-d_k, U') + LD(T'-d_k, U', k)
    beta(t,u) = logsumexp over k of
                LB + LD[k] + (0 if (t+d_k, u) = (T', U') else beta(t+d_k, u))   (d_k >= 1)
                LE + LD[k] + beta(t+d_k, u+1)                                   (u < U')
    (beta of a position that is not a cell is -inf)
Step posteriors and gradients (p = softmax(z), q = softmax(zd)):
    gB(t,u,k), gE(t,u,k) = exp(alpha(t,u) + step log-weight + beta(target) - logP)
    dz  = gc ((sum_k gB + gE) p - (sum_k gB) [v = blank] - (sum_k gE) [v = y_u])
    dzd = gc ((sum_k gB + gE) q - (gB + gE)(k))
    dW_out += h^T dz, db_out += dz, dW_dur += h^T dzd, db_dur += dzd,
    dpre = (1 - h^2) (dz W_out^T + dzd W_dur^T),
    dEnc[t] += sum_u dpre,  dPred[u] += sum_t dpre.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _lse(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=axis, keepdims=True))).squeeze(axis)


def _logsumexp(terms):
    terms = [x for x in terms if x != NEG_INF]
    if not terms:
        return NEG_INF
    m = max(terms)
    return m + np.log(sum(np.exp(x - m) for x in terms))


def cell_scores(enc_b, pred_b, W, b_out, Wd, bd, y, T_len, U_len, blank):
    """LB [T', U'+1], LE [T', U'], LD [T', U'+1, K] (float64)."""
    enc_b = np.asarray(enc_b, np.float64)
    pred_b = np.asarray(pred_b, np.float64)
    Up1 = U_len + 1
    K = Wd.shape[1]
    LB = np.empty((T_len, Up1))
    LE = np.empty((T_len, U_len))
    LD = np.empty((T_len, Up1, K))
    us = np.arange(U_len)
    for t in range(T_len):
        h = np.tanh(enc_b[t][None, :] + pred_b[:Up1])
        z = h @ W + b_out[None, :]
        zd = h @ Wd + bd[None, :]
        lse = _lse(z, 1)
        LB[t] = z[:, blank] - lse
        LE[t] = z[us, np.asarray(y)[:U_len]] - lse[:U_len]
        LD[t] = zd - _lse(zd, 1)[:, None]
    return LB, LE, LD


def alpha_lattice(LB, LE, LD, durations):
    T_len, Up1 = LB.shape
    alpha = np.full((T_len, Up1), NEG_INF)
    alpha[0, 0] = 0.0
    for t in range(T_len):
        for u in range(Up1):
            if t == 0 and u == 0:
                continue
            terms = []
            for k, d in enumerate(durations):
                s = t - d
                if s < 0:
                    continue
                if d >= 1:
                    terms.append(alpha[s, u] + LB[s, u] + LD[s, u, k])
                if u >= 1:
                    terms.append(alpha[s, u - 1] + LE[s, u - 1] + LD[s, u - 1, k])
            alpha[t, u] = _logsumexp(terms)
    U_len = Up1 - 1
    logP = _logsumexp([alpha[T_len - d, U_len] + LB[T_len - d, U_len] + LD[T_len - d, U_len, k]
                       for k, d in enumerate(durations) if 1 <= d <= T_len])
    return alpha, logP


def _next(beta, t, u, T_len, U_len):
    """beta of the position (t, u) a step lands on: 0 at (T', U'), the cell's
    beta inside the lattice, -inf elsewhere."""
    if t == T_len and u == U_len:
        return 0.0
    if t < T_len and u <= U_len:
        return beta[t, u]
    return NEG_INF


def beta_lattice(LB, LE, LD, durations):
    T_len, Up1 = LB.shape
    U_len = Up1 - 1
    beta = np.full((T_len, Up1), NEG_INF)
    for t in range(T_len - 1, -1, -1):
        for u in range(U_len, -1, -1):
            terms = []
            for k, d in enumerate(durations):
                if d >= 1:
                    terms.append(LB[t, u] + LD[t, u, k] + _next(beta, t + d, u, T_len, U_len))
                if u < U_len:
                    nx = _next(beta, t + d, u + 1, T_len, U_len) if t + d < T_len else NEG_INF
                    terms.append(LE[t, u] + LD[t, u, k] + nx)
            beta[t, u] = _logsumexp(terms)
    return beta


def posteriors(alpha, beta, LB, LE, LD, durations, logP):
    """Step posteriors gB, gE [T', U'+1, K]."""
    T_len, Up1 = LB.shape
    U_len = Up1 - 1
    K = len(durations)
    gB = np.zeros((T_len, Up1, K))
    gE = np.zeros((T_len, Up1, K))
    for t in range(T_len):
        for u in range(Up1):
            if alpha[t, u] == NEG_INF:
                continue
            for k, d in enumerate(durations):
                if d >= 1:
                    nx = _next(beta, t + d, u, T_len, U_len)
                    if nx != NEG_INF:
                        gB[t, u, k] = np.exp(alpha[t, u] + LB[t, u] + LD[t, u, k] + nx - logP)
                if u < U_len and t + d < T_len:
                    nx = beta[t + d, u + 1]
                    if nx != NEG_INF:
                        gE[t, u, k] = np.exp(alpha[t, u] + LE[t, u] + LD[t, u, k] + nx - logP)
    return gB, gE


def utterance(enc_b, pred_b, W, b_out, Wd, bd, y, T_len, U_len, blank, durations,
              grad_cost=1.0, want_grads=True):
    """TDT loss of one utterance: dict with cost, logP, alpha, beta, LB, LE,
    LD, gB, gE and (want_grads) dEnc [T', H], dPred [U'+1, H], dW, db, dWd,
    dbd.  An utterance no alignment reaches has cost +inf and zero
    gradients."""
    enc_b = np.asarray(enc_b, np.float64)
    pred_b = np.asarray(pred_b, np.float64)
    W = np.asarray(W, np.float64)
    b_out = np.asarray(b_out, np.float64)
    Wd = np.asarray(Wd, np.float64)
    bd = np.asarray(bd, np.float64)
    y = np.asarray(y)
    durations = [int(d) for d in durations]
    H, V = W.shape
    K = Wd.shape[1]
    Up1 = U_len + 1
    LB, LE, LD = cell_scores(enc_b, pred_b, W, b_out, Wd, bd, y, T_len, U_len, blank)
    alpha, logP = alpha_lattice(LB, LE, LD, durations)
    beta = beta_lattice(LB, LE, LD, durations)
    out = dict(cost=-logP, logP=logP, alpha=alpha, beta=beta, LB=LB, LE=LE, LD=LD)
    if logP == NEG_INF:
        out.update(gB=np.zeros((T_len, Up1, K)), gE=np.zeros((T_len, Up1, K)),
                   dEnc=np.zeros((T_len, H)), dPred=np.zeros((Up1, H)), dW=np.zeros((H, V)),
                   db=np.zeros(V), dWd=np.zeros((H, K)), dbd=np.zeros(K))
        return out
    gB, gE = posteriors(alpha, beta, LB, LE, LD, durations, logP)
    out.update(gB=gB, gE=gE)
    if not want_grads:
        return out
    dEnc = np.zeros((T_len, H))
    dPred = np.zeros((Up1, H))
    dW = np.zeros((H, V))
    db = np.zeros(V)
    dWd = np.zeros((H, K))
    dbd = np.zeros(K)
    us = np.arange(U_len)
    sB = gB.sum(axis=2)
    sE = gE.sum(axis=2)
    for t in range(T_len):
        h = np.tanh(enc_b[t][None, :] + pred_b[:Up1])
        z = h @ W + b_out[None, :]
        zd = h @ Wd + bd[None, :]
        p = np.exp(z - _lse(z, 1)[:, None])
        q = np.exp(zd - _lse(zd, 1)[:, None])
        occ = sB[t] + sE[t]
        dz = occ[:, None] * p
        dz[:, blank] -= sB[t]
        dz[us, y[:U_len]] -= sE[t, :U_len]
        dz *= grad_cost
        dzd = grad_cost * (occ[:, None] * q - (gB[t] + gE[t]))
        dW += h.T @ dz
        db += dz.sum(axis=0)
        dWd += h.T @ dzd
        dbd += dzd.sum(axis=0)
        dpre = (1.0 - h * h) * (dz @ W.T + dzd @ Wd.T)
        dEnc[t] = dpre.sum(axis=0)
        dPred += dpre
    out.update(dEnc=dEnc, dPred=dPred, dW=dW, db=db, dWd=dWd, dbd=dbd)
    return out


def loss_and_grads(enc, pred, W, b_out, Wd, bd, labels, T_lens, U_lens, blank, durations,
                   grad_costs=None, want_grads=True):
    """Batched TDT loss: costs [B] and (want_grads) dEnc [B,T,H],
    dPred [B,U+1,H], dW, db, dWd, dbd."""
    enc = np.asarray(enc, np.float64)
    pred = np.asarray(pred, np.float64)
    B, T, H = enc.shape
    V = np.asarray(W).shape[1]
    K = np.asarray(Wd).shape[1]
    gcs = np.ones(B) if grad_costs is None else np.asarray(grad_costs, np.float64)
    res = dict(costs=np.empty(B))
    if want_grads:
        res.update(dEnc=np.zeros((B, T, H)), dPred=np.zeros((B, pred.shape[1], H)),
                   dW=np.zeros((H, V)), db=np.zeros(V), dWd=np.zeros((H, K)), dbd=np.zeros(K))
    for b in range(B):
        Tl, Ul = int(T_lens[b]), int(U_lens[b])
        o = utterance(enc[b, :Tl], pred[b, :Ul + 1], W, b_out, Wd, bd, labels[b], Tl, Ul, blank,
                      durations, gcs[b], want_grads=want_grads)
        res["costs"][b] = o["cost"]
        if want_grads:
            res["dEnc"][b, :Tl] = o["dEnc"]
            res["dPred"][b, :Ul + 1] = o["dPred"]
            for k in ("dW", "db", "dWd", "dbd"):
                res[k] += o[k]
    return res
