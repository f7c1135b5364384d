"""Float64 oracle: pruned RNN-T loss ("Pruned RNN-T for fast, memory-efficient
ASR training", Abstract), fwd + bwd.

TEST INFRASTRUCTURE ONLY (tests and the benchmark's CPU baseline).

The abstract gives two steps: pruning bounds for the transducer recursion
from a simple joiner that is linear in the encoder and decoder embeddings,
then the full non-linear joiner evaluated inside those bounds.  It leaves the
details open; the readings taken here (one per point) are:

1. Simple joiner: the full joiner of this path without its non-linearity and
   with the same weights,
       zs(t,u) = (enc[t] + pred[u]) @ W_out + b_out,
   so that zs(t,u) = am[t] + lm[u] with am = enc @ W_out and
   lm = pred @ W_out + b_out: its normaliser over the vocabulary needs no
   [T, U+1, V] tensor.  Its log-probabilities LBs, LEs (blank, label) give a
   full lattice, whose alpha / beta (as in oracle.rnnt) yield the simple cost
   -logPs and the occupancy of each cell,
       occ(t,u) = exp(alpha_s(t,u) + beta_s(t,u) - logPs),
   the probability that an alignment passes through (t,u).
2. Bounds: a window of S consecutive label positions per frame,
   band_t = {u : s_t <= u <= min(s_t + S - 1, U')}.  Each frame's window is
   centred on the occupancy-weighted mean label position
       c_t = sum_u u occ(t,u) / sum_u occ(t,u),
       s0_t = clamp(floor(c_t - (S - 1)/2 + 1/2), 0, smax),  smax = max(0, U'+1-S),
   and then made to hold at least one alignment: the first window starts at
   0 (alignments start at (0,0)), consecutive windows start in
   non-decreasing order and at most S-1 apart (an alignment leaves frame t
   by a blank from a position it also occupies at t+1), and the last one
   starts at smax (alignments end at (T'-1, U')):
       forward   s_0 = 0,     s_t = min(max(s0_t, s_{t-1}), s_{t-1} + S - 1)
       backward  s_{T'-1} = smax,  s_t = max(s_t, s_{t+1} - (S - 1))
   If the backward pass moves s_0 above 0 (U' > T' (S - 1)), no alignment fits
   in any such band: the utterance is infeasible.  (A window by largest
   contained occupancy is the other plain choice; it is not taken because
   wherever the occupancy of a frame sits inside fewer than S positions many
   windows hold the same mass up to rounding, so the choice would be decided
   by rounding noise.)
3. Pruned loss: the full joiner's log-probabilities LB, LE (oracle.rnnt),
   summed over the alignments whose every cell lies in the band only:
       LB(t,u) is kept iff (t,u) and (t+1,u) are in the band (the final blank
       at (T'-1, U') is always in it), LE(t,u) iff (t,u) and (t,u+1) are;
       every other step gets -inf;
   cost = -log sum over those alignments; the gradients are those of that
   sum with the bounds held fixed (they are piecewise constant in the
   inputs).  A band of S >= U'+1 positions is the whole lattice: the pruned
   loss is then the full-sum loss.
"""
from __future__ import annotations

import math

import numpy as np

from . import rnnt

NEG_INF = -np.inf


def simple_cell_scores(enc_b, pred_b, W, b_out, y, T_len, U_len, blank):
    """Simple joiner (reading 1): lse_s, LBs [T', U'+1], LEs [T', U'],
    computed per lattice row from zs = (enc[t] + pred[u]) @ W + b."""
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
        z = (enc_b[t][None, :] + pred_b[:Up1]) @ W + b_out[None, :]
        m = np.max(z, axis=1)
        lse[t] = m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))
        LB[t] = z[:, blank] - lse[t]
        LE[t] = z[us, np.asarray(y)[:U_len]] - lse[t, :U_len]
    return lse, LB, LE


def occupancy(LB, LE):
    """alpha, beta, logP of a full lattice and occ(t,u) = exp(alpha + beta - logP)."""
    alpha, logP = rnnt.alpha_lattice(LB, LE)
    beta = rnnt.beta_lattice(LB, LE)
    return alpha, beta, logP, np.exp(alpha + beta - logP)


def window_centres(occ):
    """c_t = sum_u u occ(t,u) / sum_u occ(t,u) for every frame."""
    u = np.arange(occ.shape[1], dtype=np.float64)
    return (occ * u[None, :]).sum(axis=1) / occ.sum(axis=1)


def pruning_bounds(centres, U_len, S):
    """Window starts s_t (int64 [T']) from the centres (reading 2), and
    whether a band of them holds an alignment."""
    T_len = len(centres)
    smax = max(0, U_len + 1 - S)
    s0 = np.clip(np.floor(centres - (S - 1) / 2.0 + 0.5), 0, smax).astype(np.int64)
    s = np.empty(T_len, dtype=np.int64)
    s[0] = 0
    for t in range(1, T_len):
        s[t] = min(max(s0[t], s[t - 1]), s[t - 1] + S - 1)
    s[T_len - 1] = smax
    for t in range(T_len - 2, -1, -1):
        s[t] = max(s[t], s[t + 1] - (S - 1))
    return s, bool(s[0] == 0)


def band_mask(s, U_len, S):
    """in_band [T', U'+1] (bool) of the windows s."""
    u = np.arange(U_len + 1)[None, :]
    return (u >= s[:, None]) & (u <= s[:, None] + S - 1)


def band_weights(LB, LE, inb):
    """LB, LE with every step that leaves the band set to -inf (reading 3)."""
    T_len, Up1 = LB.shape
    LBp = np.full_like(LB, NEG_INF)
    LEp = np.full_like(LE, NEG_INF)
    keep_b = inb.copy()
    keep_b[:-1] &= inb[1:]               # blank (t,u) -> (t+1,u) stays in the band
    keep_b[T_len - 1, :] = False         # no blank out of the last frame ...
    keep_b[T_len - 1, Up1 - 1] = inb[T_len - 1, Up1 - 1]  # ... but the final one
    LBp[keep_b] = LB[keep_b]
    if Up1 > 1:
        keep_e = inb[:, :-1] & inb[:, 1:]  # label (t,u) -> (t,u+1)
        LEp[keep_e] = LE[keep_e]
    return LBp, LEp


def utterance(enc_b, pred_b, W, b_out, y, T_len, U_len, blank, S, grad_cost=1.0,
              want_grads=True):
    """Pruned loss of one utterance.  Returns a dict: simple_cost, bounds s
    [T'], feasible, centres, occ, cost (NaN if infeasible), logP, and with
    want_grads dEnc [T', H], dPred [U'+1, H], dW [H, V], db [V] (zero if
    infeasible), plus LB, LE (full joiner), LBp, LEp, gB, gE."""
    assert S >= 1
    enc_b = np.asarray(enc_b, np.float64)
    pred_b = np.asarray(pred_b, np.float64)
    W = np.asarray(W, np.float64)
    b_out = np.asarray(b_out, np.float64)
    y = np.asarray(y)
    H, V = W.shape
    Up1 = U_len + 1
    # 1. simple joiner over the full lattice
    _, LBs, LEs = simple_cell_scores(enc_b, pred_b, W, b_out, y, T_len, U_len, blank)
    _, _, logPs, occ = occupancy(LBs, LEs)
    centres = window_centres(occ)
    # 2. bounds
    s, feasible = pruning_bounds(centres, U_len, S)
    out = dict(simple_cost=-logPs, bounds=s, feasible=feasible, centres=centres, occ=occ)
    if not feasible:
        out.update(cost=math.nan, logP=math.nan, dEnc=np.zeros((T_len, H)),
                   dPred=np.zeros((Up1, H)), dW=np.zeros((H, V)), db=np.zeros(V))
        return out
    # 3. the full joiner inside the band
    lse, LB, LE = rnnt.cell_scores(enc_b, pred_b, W, b_out, y, T_len, U_len, blank)
    inb = band_mask(s, U_len, S)
    LBp, LEp = band_weights(LB, LE, inb)
    alpha, logP = rnnt.alpha_lattice(LBp, LEp)
    beta = rnnt.beta_lattice(LBp, LEp)
    gB, gE = rnnt.posteriors(alpha, beta, LBp, LEp, logP)
    out.update(cost=-logP, logP=logP, LB=LB, LE=LE, LBp=LBp, LEp=LEp, gB=gB, gE=gE)
    if not want_grads:
        return out
    dEnc = np.zeros((T_len, H))
    dPred = np.zeros((Up1, H))
    dW = np.zeros((H, V))
    db = np.zeros(V)
    us = np.arange(U_len)
    for t in range(T_len):
        h = np.tanh(enc_b[t][None, :] + pred_b[:Up1])
        z = h @ W + b_out[None, :]
        p = np.exp(z - lse[t][:, None])
        dz = (gB[t] + gE[t])[:, None] * p
        dz[:, blank] -= gB[t]
        dz[us, y[:U_len]] -= gE[t, :U_len]
        dz *= grad_cost
        dW += h.T @ dz
        db += dz.sum(axis=0)
        dpre = (1.0 - h * h) * (dz @ W.T)
        dEnc[t] = dpre.sum(axis=0)
        dPred += dpre
    out.update(dEnc=dEnc, dPred=dPred, dW=dW, db=db)
    return out


def loss_and_grads(enc, pred, W, b_out, labels, T_lens, U_lens, blank, S, grad_costs=None,
                   want_grads=True):
    """Batched pruned loss: costs [B] (NaN for an infeasible utterance),
    simple_costs [B], bounds [B, T] (entries past T' repeat the last window),
    feasible [B], and with want_grads dEnc [B,T,H], dPred [B,U+1,H], dW, db."""
    enc = np.asarray(enc, np.float64)
    pred = np.asarray(pred, np.float64)
    B, T, H = enc.shape
    V = np.asarray(W).shape[1]
    gcs = np.ones(B) if grad_costs is None else np.asarray(grad_costs, np.float64)
    costs = np.empty(B)
    simple = np.empty(B)
    bounds = np.zeros((B, T), dtype=np.int64)
    feasible = np.zeros(B, dtype=bool)
    dEnc = np.zeros((B, T, H))
    dPred = np.zeros((B, pred.shape[1], H))
    dW = np.zeros((H, V))
    db = np.zeros(V)
    for b in range(B):
        Tl, Ul = int(T_lens[b]), int(U_lens[b])
        o = utterance(enc[b], pred[b], W, b_out, labels[b], Tl, Ul, blank, S, gcs[b],
                      want_grads=want_grads)
        costs[b] = o["cost"]
        simple[b] = o["simple_cost"]
        bounds[b, :Tl] = o["bounds"]
        bounds[b, Tl:] = o["bounds"][-1]
        feasible[b] = o["feasible"]
        if want_grads:
            dEnc[b, :Tl] = o["dEnc"]
            dPred[b, :Ul + 1] = o["dPred"]
            dW += o["dW"]
            db += o["db"]
    res = dict(costs=costs, simple_costs=simple, bounds=bounds, feasible=feasible)
    if want_grads:
        res.update(dEnc=dEnc, dPred=dPred, dW=dW, db=db)
    return res
