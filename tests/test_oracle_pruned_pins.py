"""Pins of the pruned RNN-T oracle (oracle/pruned.py) against facts that do not
come from the oracle itself: enumeration of every alignment of small
lattices, closed forms with zero weights, the linear limit of the joiner,
the whole-lattice band, central finite differences and batch padding."""
import itertools
import math

import numpy as np
import pytest

from oracle import pruned, rnnt

from synth import make_inputs


def _alignments(T_len, U_len):
    """Every alignment as its list of steps ((t, u), kind), kind 'b' or 'e',
    the final blank at (T'-1, U') included."""
    n = T_len - 1 + U_len
    for lab in itertools.combinations(range(n), U_len):
        lab = set(lab)
        t = u = 0
        steps = []
        for k in range(n):
            if k in lab:
                steps.append(((t, u), "e"))
                u += 1
            else:
                steps.append(((t, u), "b"))
                t += 1
        steps.append(((t, u), "b"))
        yield steps


def _brute(LB, LE, allowed_cell=None):
    """log of the summed probability over alignments whose every cell is
    allowed, the posteriors of each step and the occupancy of each cell."""
    T_len, Up1 = LB.shape
    logs, paths = [], []
    for steps in _alignments(T_len, Up1 - 1):
        if allowed_cell is not None and not all(allowed_cell[c] for c, _ in steps):
            continue
        lp = sum(LB[c] if k == "b" else LE[c] for c, k in steps)
        logs.append(lp)
        paths.append(steps)
    logs = np.array(logs)
    logP = np.logaddexp.reduce(logs) if len(logs) else -np.inf
    gB = np.zeros((T_len, Up1))
    gE = np.zeros((T_len, Up1))
    occ = np.zeros((T_len, Up1))
    for lp, steps in zip(logs, paths):
        w = math.exp(lp - logP)
        for c, k in steps:
            (gB if k == "b" else gE)[c] += w
            occ[c] += w
    return logP, gB, gE, occ


def _case(seed, T, U, H=12, V=7, sigma=0.8):
    """One utterance at full lengths with a nonzero output bias."""
    inp = make_inputs(1, T, U, H, V, sigma=sigma, seed=seed)
    b = np.random.default_rng(seed + 500).normal(0.0, 0.5, V)
    return inp.enc_f64[0], inp.pred_f64[0], inp.W_f64, b, inp.labels[0], T, U


@pytest.mark.parametrize("seed,T,U,S", [(1, 5, 3, 10), (2, 7, 4, 5), (3, 1, 2, 3), (4, 6, 0, 2)])
def test_whole_band_is_the_full_sum(seed, T, U, S):
    """S >= U'+1: every window starts at 0, the band is the whole lattice and
    the pruned loss is the full-sum loss, gradients included."""
    enc, pred, W, b, y, Tl, Ul = _case(seed, T, U)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, S)
    ref = rnnt.utterance_loss_and_grads(enc, pred, W, b, y, Tl, Ul, 0)
    assert o["feasible"] and np.all(o["bounds"] == 0)
    assert o["cost"] == pytest.approx(ref["cost"], rel=1e-13)
    for k in ("dEnc", "dPred", "dW", "db"):
        np.testing.assert_allclose(o[k], ref[k], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed,T,U,S", [(11, 6, 5, 2), (12, 7, 5, 3), (13, 5, 4, 2), (14, 8, 3, 2),
                                        (15, 4, 5, 3), (16, 6, 6, 4)])
def test_against_alignment_enumeration(seed, T, U, S):
    """Small lattices, every alignment enumerated: the simple joiner's cost and
    cell occupancies (all alignments, simple joiner log-probabilities), and the
    pruned cost and step posteriors (alignments inside the band only, full
    joiner log-probabilities)."""
    enc, pred, W, b, y, Tl, Ul = _case(seed, T, U, sigma=1.2)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, S)
    _, LBs, LEs = pruned.simple_cell_scores(enc, pred, W, b, y, Tl, Ul, 0)
    logPs, _, _, occ = _brute(LBs, LEs)
    assert o["simple_cost"] == pytest.approx(-logPs, rel=1e-12)
    np.testing.assert_allclose(o["occ"], occ, rtol=1e-10, atol=1e-14)
    assert o["feasible"]
    inb = pruned.band_mask(o["bounds"], Ul, S)
    _, LB, LE = rnnt.cell_scores(enc, pred, W, b, y, Tl, Ul, 0)
    logP, gB, gE, _ = _brute(LB, LE, allowed_cell=inb)
    assert np.isfinite(logP)
    assert o["cost"] == pytest.approx(-logP, rel=1e-12)
    np.testing.assert_allclose(o["gB"], gB, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(o["gE"], gE, rtol=1e-10, atol=1e-14)
    # a band narrower than the lattice drops alignments: the pruned
    # probability is below the full sum's
    if S < Ul + 1:
        full = rnnt.utterance_loss_and_grads(enc, pred, W, b, y, Tl, Ul, 0)["cost"]
        assert o["cost"] > full


def test_zero_weights_occupancy_closed_form():
    """W_out = 0: every alignment has the same probability, so a cell's
    occupancy is the share of lattice paths through it,
    C(t+u, u) C(T'-1-t + U'-u, U'-u) / C(T'-1+U', U'), and the window
    centres and bounds follow from integers alone."""
    T, U, S = 9, 6, 3
    enc, pred, W, b, y, Tl, Ul = _case(21, T, U)
    W = np.zeros_like(W)
    b = np.zeros_like(b)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, S)
    tot = math.comb(T - 1 + U, U)
    occ = np.array([[math.comb(t + u, u) * math.comb(T - 1 - t + U - u, U - u) / tot
                     for u in range(U + 1)] for t in range(T)])
    np.testing.assert_allclose(o["occ"], occ, rtol=1e-12)
    c = (occ * np.arange(U + 1)).sum(1) / occ.sum(1)
    np.testing.assert_allclose(o["centres"], c, rtol=1e-12)
    # by symmetry of the path counts the centres rise from 0 to U'
    assert c[0] < c[-1] and np.all(np.diff(c) > 0)
    # simple and full joiner coincide when W_out = 0 (tanh is irrelevant)
    full = rnnt.utterance_loss_and_grads(enc, pred, W, b, y, Tl, Ul, 0)["cost"]
    assert o["simple_cost"] == pytest.approx(full, rel=1e-13)
    # the full-sum cost with b_out = 0: (T'+U') log V - log C(T'+U'-1, U')
    assert full == pytest.approx((T + U) * math.log(7) - math.log(tot), rel=1e-13)


def test_simple_joiner_is_the_linear_limit():
    """For tiny encodings tanh(x) = x - x^3/3 + ..., so the simple joiner's
    cost approaches the full joiner's at rate |x|^3; a simple joiner that drops
    or misplaces either embedding, or transposes W_out, misses by orders of
    magnitude more."""
    inp = make_inputs(1, 10, 4, 16, 9, sigma=1e-3, seed=5)
    W = inp.W_f64 * 3000.0  # logits of size ~0.1
    enc, pred, y = inp.enc_f64[0], inp.pred_f64[0], inp.labels[0]
    b = np.random.default_rng(6).normal(0.0, 0.5, 9)
    lse_s, LBs, LEs = pruned.simple_cell_scores(enc, pred, W, b, y, 10, 4, 0)
    lse, LB, LE = rnnt.cell_scores(enc, pred, W, b, y, 10, 4, 0)
    # |x| ~ 2e-3 -> |x^3/3| ~ 3e-9 per hidden unit, times sum_k |W_kv| ~ 1e3
    assert np.max(np.abs(LBs - LB)) < 1e-5
    assert np.max(np.abs(LEs - LE)) < 1e-5
    # the same comparison with the prediction embedding or the bias dropped
    # fails by far
    _, LBw, _ = pruned.simple_cell_scores(enc, 0 * pred, W, b, y, 10, 4, 0)
    assert np.max(np.abs(LBw - LB)) > 1e-3
    _, LBw, _ = pruned.simple_cell_scores(enc, pred, W, 0 * b, y, 10, 4, 0)
    assert np.max(np.abs(LBw - LB)) > 1e-3


@pytest.mark.parametrize("seed,T,U,S", [(31, 40, 12, 2), (32, 60, 20, 3), (33, 25, 25, 4),
                                        (34, 30, 9, 5), (35, 12, 30, 4)])
def test_bounds_hold_an_alignment(seed, T, U, S):
    """The windows start at 0, never move back, move forward by at most S-1
    per frame and end at max(0, U'+1-S); inside those rules each frame's
    window is the one centred on its occupancy centre, and the band's cost
    is finite."""
    enc, pred, W, b, y, Tl, Ul = _case(seed, T, U, sigma=0.7)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, S, want_grads=False)
    s = o["bounds"]
    smax = max(0, Ul + 1 - S)
    feasible = Ul <= Tl * (S - 1)
    assert o["feasible"] == feasible
    if not feasible:
        assert math.isnan(o["cost"])
        return
    assert s[0] == 0 and s[-1] == smax
    assert np.all(np.diff(s) >= 0) and np.all(np.diff(s) <= S - 1)
    assert np.all((s >= 0) & (s <= smax))
    s0 = np.clip(np.floor(o["centres"] - (S - 1) / 2 + 0.5), 0, smax)
    # where the rules do not bind, the window is the centred one
    free = np.ones(Tl, dtype=bool)
    free[0] = free[-1] = False
    for t in range(1, Tl - 1):
        free[t] = (s[t] - s[t - 1] < S - 1) and (s[t + 1] - s[t] < S - 1) and s[t] > s[t - 1]
    assert np.all(s[free] == s0[free])
    assert np.isfinite(o["cost"])


def test_infeasible_band_is_reported():
    """U' > T'(S-1): no band of windows of S positions connects (0,0) to
    (T'-1, U'), so the utterance is infeasible (cost NaN, zero gradients)."""
    enc, pred, W, b, y, Tl, Ul = _case(41, 2, 5)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, 2)
    assert not o["feasible"] and math.isnan(o["cost"])
    assert np.all(o["dEnc"] == 0) and np.all(o["dW"] == 0)
    # one more position per window makes it feasible (U' = 5 <= 2 * 3)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, 4)
    assert o["feasible"] and np.isfinite(o["cost"])


def test_finite_differences():
    """Central differences of the pruned cost in every entry of enc, pred,
    W_out and b_out, with the bounds (piecewise constant) unchanged by the
    perturbation."""
    T, U, S, H, V = 7, 4, 2, 6, 5
    enc, pred, W, b, y, Tl, Ul = _case(51, T, U, H=H, V=V, sigma=0.6)
    o = pruned.utterance(enc, pred, W, b, y, Tl, Ul, 0, S, grad_cost=1.7)
    assert np.any(o["bounds"] > 0)
    eps = 1e-6
    for name, arr, grad in (("enc", enc, o["dEnc"]), ("pred", pred, o["dPred"]),
                            ("W", W, o["dW"]), ("b", b, o["db"])):
        flat = arr.reshape(-1)
        g = grad.reshape(-1)
        n = min(flat.size, g.size) if name != "pred" else (Ul + 1) * H
        for i in range(n):
            vals = []
            for sgn in (1, -1):
                x = flat.copy()
                x[i] += sgn * eps
                args = dict(enc=enc, pred=pred, W=W, b=b)
                args[name] = x.reshape(arr.shape)
                r = pruned.utterance(args["enc"], args["pred"], args["W"], args["b"], y, Tl, Ul,
                                     0, S, want_grads=False)
                assert np.array_equal(r["bounds"], o["bounds"])
                vals.append(r["cost"])
            fd = 1.7 * (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - g[i]) <= 1e-6 * max(1.0, abs(g[i])), (name, i, fd, g[i])


def test_batch_padding_invariance():
    """The padded batch gives each utterance's results computed alone; padded
    encodings and labels past the lengths change nothing."""
    inp = make_inputs(3, 14, 6, 8, 11, sigma=0.7, seed=61, t_range=(3, 14), u_range=(0, 6))
    S = 3
    res = pruned.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                                inp.T_lens, inp.U_lens, 0, S, grad_costs=[1.0, -0.5, 2.0])
    for k, gc in enumerate([1.0, -0.5, 2.0]):
        Tl, Ul = int(inp.T_lens[k]), int(inp.U_lens[k])
        o = pruned.utterance(inp.enc_f64[k, :Tl], inp.pred_f64[k, :Ul + 1], inp.W_f64, inp.b_f64,
                             inp.labels[k, :Ul], Tl, Ul, 0, S, grad_cost=gc)
        assert res["costs"][k] == pytest.approx(o["cost"], rel=1e-14)
        np.testing.assert_array_equal(res["bounds"][k, :Tl], o["bounds"])
        np.testing.assert_allclose(res["dEnc"][k, :Tl], o["dEnc"], rtol=1e-13, atol=1e-15)
        assert np.all(res["dEnc"][k, Tl:] == 0) and np.all(res["dPred"][k, Ul + 1:] == 0)
    enc2 = inp.enc_f64.copy()
    lab2 = inp.labels.copy()
    for k in range(3):
        enc2[k, inp.T_lens[k]:] = 99.0
        lab2[k, inp.U_lens[k]:] = 1
    res2 = pruned.loss_and_grads(enc2, inp.pred_f64, inp.W_f64, inp.b_f64, lab2, inp.T_lens,
                                 inp.U_lens, 0, S, grad_costs=[1.0, -0.5, 2.0])
    np.testing.assert_array_equal(res2["costs"], res["costs"])
    np.testing.assert_array_equal(res2["dW"], res["dW"])
