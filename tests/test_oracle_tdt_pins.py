"""Pins of the token-and-duration transducer oracle (oracle/tdt.py) against
facts that do not come from the oracle itself: enumeration of every
alignment of small lattices, a closed form with one duration and zero
weights, alpha/beta agreement, the label-count and frame-count invariants of
the step posteriors, central finite differences and batch padding."""
import math

import numpy as np
import pytest

from oracle import tdt

from synth import make_inputs


def _case(seed, T, U, K, H=10, V=7, sigma=0.8):
    inp = make_inputs(1, T, U, H, V, sigma=sigma, seed=seed)
    rng = np.random.default_rng(seed + 900)
    b = rng.normal(0.0, 0.5, V)
    Wd = rng.normal(0.0, sigma, (H, K))
    bd = rng.normal(0.0, 0.5, K)
    return inp.enc_f64[0], inp.pred_f64[0], inp.W_f64, b, Wd, bd, inp.labels[0]


def _enumerate(LB, LE, LD, durations):
    """Every alignment by depth-first search over (token, duration) steps:
    returns logP and the step posteriors gB, gE [T', U'+1, K]."""
    T_len, Up1 = LB.shape
    U_len = Up1 - 1
    paths = []

    def walk(t, u, steps, lp):
        for k, d in enumerate(durations):
            if d >= 1:
                if t + d == T_len and u == U_len:
                    paths.append((lp + LB[t, u] + LD[t, u, k], steps + [("b", t, u, k)]))
                elif t + d < T_len:
                    walk(t + d, u, steps + [("b", t, u, k)], lp + LB[t, u] + LD[t, u, k])
            if u < U_len and t + d < T_len:
                walk(t + d, u + 1, steps + [("e", t, u, k)], lp + LE[t, u] + LD[t, u, k])

    walk(0, 0, [], 0.0)
    logs = np.array([p[0] for p in paths])
    logP = np.logaddexp.reduce(logs) if len(logs) else -np.inf
    K = len(durations)
    gB = np.zeros((T_len, Up1, K))
    gE = np.zeros((T_len, Up1, K))
    for lp, steps in paths:
        w = math.exp(lp - logP)
        for kind, t, u, k in steps:
            (gB if kind == "b" else gE)[t, u, k] += w
    return logP, gB, gE, len(paths)


@pytest.mark.parametrize("seed,T,U,durations", [
    (1, 5, 2, (0, 1, 2)), (2, 6, 3, (0, 1, 2, 3)), (3, 4, 3, (1, 2)), (4, 7, 2, (0, 2, 3)),
    (5, 3, 4, (0, 1)), (6, 6, 0, (0, 1, 2, 4)), (7, 1, 2, (0, 1))])
def test_against_alignment_enumeration(seed, T, U, durations):
    """Every alignment enumerated: the cost and every step posterior."""
    enc, pred, W, b, Wd, bd, y = _case(seed, T, U, len(durations), sigma=1.1)
    o = tdt.utterance(enc, pred, W, b, Wd, bd, y, T, U, 0, durations)
    LB, LE, LD = tdt.cell_scores(enc, pred, W, b, Wd, bd, y, T, U, 0)
    logP, gB, gE, n = _enumerate(LB, LE, LD, durations)
    assert n > 0
    assert o["logP"] == pytest.approx(logP, rel=1e-12)
    np.testing.assert_allclose(o["gB"], gB, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(o["gE"], gE, rtol=1e-10, atol=1e-14)
    # alpha / beta agreement
    assert o["beta"][0, 0] == pytest.approx(o["logP"], rel=1e-12)


def test_heads_are_normalised_independently():
    """The token and duration log-probabilities of every cell are the two
    log-softmaxes of the joint's two outputs: exp sums to 1 over each set,
    whatever the other head holds."""
    enc, pred, W, b, Wd, bd, y = _case(8, 6, 3, 4)
    LB, LE, LD = tdt.cell_scores(enc, pred, W, b, Wd, bd, y, 6, 3, 0)
    np.testing.assert_allclose(np.exp(LD).sum(axis=2), 1.0, rtol=1e-13)
    LB2, LE2, LD2 = tdt.cell_scores(enc, pred, W, b, 5 * Wd, bd - 3, y, 6, 3, 0)
    np.testing.assert_array_equal(LB2, LB)
    np.testing.assert_array_equal(LE2, LE)
    # the duration head is the softmax of tanh(enc + pred) W_dur + b_dur
    h = np.tanh(enc[2] + pred[1])
    zd = h @ Wd + bd
    np.testing.assert_allclose(LD[2, 1], zd - np.log(np.sum(np.exp(zd))), rtol=1e-13)


@pytest.mark.parametrize("T,U", [(9, 4), (12, 0), (7, 6), (5, 5)])
def test_single_duration_closed_form(T, U):
    """D = {1}: every step covers one frame, so an alignment emits one token
    per frame, its U' labels in U' of the first T'-1 frames and a blank in
    every other frame; with W_out = 0 and b_out = 0 every token has
    probability 1/V, so cost = T' log V - log C(T'-1, U') (+inf if U' > T'-1)."""
    V = 7
    enc, pred, W, b, Wd, bd, y = _case(11, T, U, 1, V=V)
    o = tdt.utterance(enc, pred, 0 * W, 0 * b, Wd, bd, y, T, U, 0, (1,))
    if U > T - 1:
        assert o["cost"] == math.inf
        assert np.all(o["dEnc"] == 0)
        return
    want = T * math.log(V) - math.log(math.comb(T - 1, U))
    assert o["cost"] == pytest.approx(want, rel=1e-13)


@pytest.mark.parametrize("seed,T,U,durations", [(21, 30, 8, (0, 1, 2, 3, 4)),
                                                (22, 25, 12, (0, 1, 3)), (23, 20, 5, (1, 2, 4))])
def test_posterior_invariants(seed, T, U, durations):
    """Each label is emitted exactly once, so sum_{t,k} gE(t,u,k) = 1 for
    every u < U'; the steps of an alignment cover the T' frames exactly, so
    sum_{t,u,k} d_k (gB + gE) = T'; exactly one blank ends the alignment."""
    enc, pred, W, b, Wd, bd, y = _case(seed, T, U, len(durations), sigma=0.6)
    o = tdt.utterance(enc, pred, W, b, Wd, bd, y, T, U, 0, durations, want_grads=False)
    gB, gE = o["gB"], o["gE"]
    np.testing.assert_allclose(gE.sum(axis=(0, 2))[:U], 1.0, rtol=1e-10)
    d = np.asarray(durations, np.float64)
    assert float(((gB + gE) * d).sum()) == pytest.approx(T, rel=1e-10)
    final = sum(gB[T - dk, U, k] for k, dk in enumerate(durations) if 1 <= dk <= T)
    assert final == pytest.approx(1.0, rel=1e-10)


def test_finite_differences():
    """Central differences of the cost in every entry of enc, pred, W_out,
    b_out, W_dur and b_dur."""
    T, U, H, V, durations = 6, 3, 5, 6, (0, 1, 2)
    enc, pred, W, b, Wd, bd, y = _case(31, T, U, len(durations), H=H, V=V, sigma=0.7)
    gc = 1.3
    o = tdt.utterance(enc, pred, W, b, Wd, bd, y, T, U, 0, durations, grad_cost=gc)
    eps = 1e-6
    params = dict(enc=enc, pred=pred, W=W, b=b, Wd=Wd, bd=bd)
    grads = dict(enc=o["dEnc"], pred=o["dPred"], W=o["dW"], b=o["db"], Wd=o["dWd"], bd=o["dbd"])
    for name, arr in params.items():
        flat = arr.reshape(-1)
        g = grads[name].reshape(-1)
        n = (U + 1) * H if name == "pred" else g.size
        for i in range(n):
            vals = []
            for sgn in (1, -1):
                x = flat.copy()
                x[i] += sgn * eps
                p = dict(params)
                p[name] = x.reshape(arr.shape)
                vals.append(tdt.utterance(p["enc"], p["pred"], p["W"], p["b"], p["Wd"], p["bd"],
                                          y, T, U, 0, durations, want_grads=False)["cost"])
            fd = gc * (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - g[i]) <= 1e-6 * max(1.0, abs(g[i])), (name, i, fd, g[i])


def test_batch_padding_invariance():
    """Padded batch = each utterance alone; padding content changes nothing."""
    inp = make_inputs(3, 12, 5, 8, 9, sigma=0.7, seed=41, t_range=(2, 12), u_range=(0, 5))
    rng = np.random.default_rng(42)
    durations = (0, 1, 2, 3)
    Wd = rng.normal(0, 0.7, (8, 4))
    bd = rng.normal(0, 0.5, 4)
    gcs = [1.0, -0.5, 2.0]
    res = tdt.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, Wd, bd,
                             inp.labels, inp.T_lens, inp.U_lens, 0, durations, grad_costs=gcs)
    for k in range(3):
        Tl, Ul = int(inp.T_lens[k]), int(inp.U_lens[k])
        o = tdt.utterance(inp.enc_f64[k, :Tl], inp.pred_f64[k, :Ul + 1], inp.W_f64, inp.b_f64,
                          Wd, bd, inp.labels[k, :Ul], Tl, Ul, 0, durations, grad_cost=gcs[k])
        assert res["costs"][k] == pytest.approx(o["cost"], rel=1e-14)
        np.testing.assert_allclose(res["dEnc"][k, :Tl], o["dEnc"], rtol=1e-13, atol=1e-15)
        assert np.all(res["dEnc"][k, Tl:] == 0) and np.all(res["dPred"][k, Ul + 1:] == 0)
    enc2 = inp.enc_f64.copy()
    for k in range(3):
        enc2[k, inp.T_lens[k]:] = 50.0
    res2 = tdt.loss_and_grads(enc2, inp.pred_f64, inp.W_f64, inp.b_f64, Wd, bd, inp.labels,
                              inp.T_lens, inp.U_lens, 0, durations, grad_costs=gcs)
    np.testing.assert_array_equal(res2["costs"], res["costs"])
    np.testing.assert_array_equal(res2["dWd"], res["dWd"])
