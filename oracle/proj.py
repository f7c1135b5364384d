"""Float64 oracle: joint input projections in front of the RNN-T joint.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).

"Daily Papers" page, Transformer-Transducer abstract: the audio and label
encodings are combined by a feed-forward layer into one label distribution
per (frame, label history).  Read here (plainest reading) as one affine map
per encoding into the joint's hidden size ahead of the add:

    enc_p[b,t]  = enc[b,t]  @ W_enc  + b_enc      enc  [B,T,E],   W_enc  [E,H]
    pred_p[b,u] = pred[b,u] @ W_pred + b_pred     pred [B,U+1,P], W_pred [P,H]
    h(t,u) = tanh(enc_p[t] + pred_p[u])           (then as in rnnt.py)

and the gradients of sum_b gc_b * cost_b chain through them from the joint's
dEnc_p, dPred_p:

    d enc = dEnc_p @ W_enc^T,   dW_enc = sum_{b,t} enc[b,t]^T dEnc_p[b,t],
    db_enc = sum_{b,t} dEnc_p[b,t]        (the same for pred)

Rows past an utterance's lengths are projected too; their joint gradients
are zero, so they contribute nothing to any gradient.
"""
from __future__ import annotations

import numpy as np

from . import rnnt


def linear(x, W, b):
    """x [..., K] @ W [K, N] + b [N], float64."""
    return np.asarray(x, np.float64) @ np.asarray(W, np.float64) + np.asarray(b, np.float64)


def linear_grads(x, W, dy):
    """Gradients of a linear map y = x @ W + b from dy [..., N]:
    (dx [..., K], dW [K, N], db [N]), float64."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    dy = np.asarray(dy, np.float64)
    K, N = W.shape
    x2 = x.reshape(-1, K)
    dy2 = dy.reshape(-1, N)
    return dy @ W.T, x2.T @ dy2, dy2.sum(axis=0)


def projected_loss_and_grads(enc, pred, W_enc, b_enc, W_pred, b_pred, W, b_out, labels, T_lens,
                             U_lens, blank, grad_costs=None, workers=1, criterion="sum"):
    """Costs [B] and the gradients of every input: enc, pred, W_enc, b_enc,
    W_pred, b_pred, W_out, b_out (float64).  The projected encodings are
    returned too (enc_p, pred_p)."""
    enc_p = linear(enc, W_enc, b_enc)
    pred_p = linear(pred, W_pred, b_pred)
    r = rnnt.loss_and_grads(enc_p, pred_p, W, b_out, labels, T_lens, U_lens, blank,
                            grad_costs=grad_costs, workers=workers, criterion=criterion)
    d_enc, dW_enc, db_enc = linear_grads(enc, W_enc, r["dEnc"])
    d_pred, dW_pred, db_pred = linear_grads(pred, W_pred, r["dPred"])
    return dict(costs=r["costs"], enc_p=enc_p, pred_p=pred_p, dEncP=r["dEnc"], dPredP=r["dPred"],
                dEnc=d_enc, dPred=d_pred, dW_enc=dW_enc, db_enc=db_enc, dW_pred=dW_pred,
                db_pred=db_pred, dW=r["dW"], db=r["db"])
