"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test is chosen so that a plausible mistake (a dropped term, a wrong sign
or index, a transposed operand, a wrong boundary) fails at least one of them:

* brute-force enumeration of every alignment (logP and both posteriors),
* a hand-worked example stored under tests/golden/,
* closed forms: W_out = 0 at full workload shapes, one frame (T' = 1) with a
  saturated joint, no labels (U' = 0), a saturated joint with H = V,
* invariants: alpha/beta agreement, posterior sums, zero row sums of the
  logit gradient, occupancy totals, bias-gradient identities,
* central finite differences of every gradient,
* padding, vocabulary-permutation, enc/pred shift and odd-symmetry
  invariances, and linearity in the per-utterance gradient weights.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import rnnt
from synth import make_config, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _utt(inp, b, **kw):
    return rnnt.utterance_loss_and_grads(
        inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64, inp.labels[b],
        int(inp.T_lens[b]), int(inp.U_lens[b]), inp.blank, **kw)


# ---------------------------------------------------------------- brute force

def test_brute_force_tiny_config():
    """The tiny workload itself: C(24,5) = 42,504 alignments per utterance."""
    inp = make_config("tiny")
    for b in range(inp.B):
        o = _utt(inp, b)
        logP, gB, gE, n = rnnt.brute_force_utterance(o["LB"], o["LE"])
        assert n == math.comb(20 + 5 - 1, 5) == 42504
        assert abs(o["logP"] - logP) <= 1e-10 * abs(logP)
        np.testing.assert_allclose(o["gB"], gB, atol=1e-11)
        np.testing.assert_allclose(o["gE"], gE, atol=1e-11)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_random_small(seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 7))
    U = int(rng.integers(0, 6))
    inp = make_inputs(1, T, U, 5, 7, sigma=0.8, seed=seed)
    o = _utt(inp, 0)
    logP, gB, gE, _ = rnnt.brute_force_utterance(o["LB"], o["LE"])
    assert abs(o["logP"] - logP) <= 1e-11 * max(1.0, abs(logP))
    np.testing.assert_allclose(o["gB"], gB, atol=1e-12)
    np.testing.assert_allclose(o["gE"], gE, atol=1e-12)


# ---------------------------------------------------------------- hand-worked

def test_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_t2_u1.json")))
    enc = np.array(g["enc"])
    pred = np.array(g["pred"])
    res = oracle.loss_and_grads(enc, pred, np.array(g["W_out"]), np.array(g["b_out"]),
                                np.array(g["labels"]), g["T_lens"], g["U_lens"], g["blank"],
                                keep_cells=True)
    assert abs(res["costs"][0] - g["cost"]) < 1e-13
    u = res["utts"][0]
    np.testing.assert_allclose(u["gB"], g["gamma_blank"], atol=1e-14)
    np.testing.assert_allclose(u["gE"], g["gamma_label"], atol=1e-14)
    np.testing.assert_allclose(res["db"], g["d_b_out"], atol=1e-14)
    # W_out = 0 makes dh = 0, hence no encoder / prediction gradient
    assert np.all(res["dEnc"] == 0) and np.all(res["dPred"] == 0)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("name", ["tiny", "short"])
def test_zero_weights_closed_form_full_shapes(name):
    inp = make_config(name)
    W0 = np.zeros_like(inp.W_f64)
    res = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, W0, inp.b_f64, inp.labels,
                                inp.T_lens, inp.U_lens, inp.blank)
    V = inp.V
    for b in range(inp.B):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        # with b_out = 0 the closed form is (T'+U') log V - log C(T'+U'-1, U')
        want = (Tl + Ul) * math.log(V) - math.log(math.comb(Tl + Ul - 1, Ul))
        assert abs(res["costs"][b] - want) <= 1e-12 * want
        assert abs(rnnt.closed_form_zero_weights(Tl, Ul, inp.labels[b], inp.b_f64, 0) - want) < 1e-9
    # bias gradient: sum_b [(T'+U')/V - T' [k=blank] - count_k(y_b)]
    want_db = np.zeros(V)
    for b in range(inp.B):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        want_db += (Tl + Ul) / V
        want_db[0] -= Tl
        np.add.at(want_db, inp.labels[b, :Ul], -1.0)
    np.testing.assert_allclose(res["db"], want_db, atol=1e-9)
    assert np.all(res["dEnc"] == 0) and np.all(res["dPred"] == 0)


def test_zero_weights_closed_form_worked_values():
    """Full-length costs at each workload's maximal (T, U) with W_out = 0."""
    want = {"tiny": 75.99, "short": 1437.47, "medium": 3891.86,
            "medium_lv": 4723.64, "long": 14164.83}
    for name, v in want.items():
        inp = make_config(name)
        c = rnnt.closed_form_zero_weights(inp.T, inp.U, inp.labels[0], np.zeros(inp.V), 0)
        assert abs(c - v) < 0.006, (name, c)


def test_zero_weights_nonuniform_bias_medium_utterance():
    """One medium-workload utterance at full H, V with a random bias."""
    inp = make_config("medium")
    rng = np.random.default_rng(7)
    bias = rng.normal(0, 1.0, size=inp.V)
    b = 3
    Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
    W0 = np.zeros_like(inp.W_f64)
    c = rnnt.loss_only(inp.enc_f64[b:b + 1], inp.pred_f64[b:b + 1], W0, bias,
                       inp.labels[b:b + 1], [Tl], [Ul], 0)[0]
    want = rnnt.closed_form_zero_weights(Tl, Ul, inp.labels[b], bias, 0)
    # independent restatement: every path has T' blanks and the U' labels
    lp = bias - np.log(np.sum(np.exp(bias)))
    want2 = -(Tl * lp[0] + lp[inp.labels[b, :Ul]].sum()
              + math.lgamma(Tl + Ul) - math.lgamma(Ul + 1) - math.lgamma(Tl))
    assert abs(c - want) <= 1e-11 * abs(want)
    assert abs(c - want2) <= 1e-10 * abs(want)


def _saturated_dist(W, b_out, sign):
    """Distribution when tanh saturates to +/-1 on every hidden unit:
    z = sign * (column sums of W_out) + b_out."""
    z = sign * W.sum(axis=0) + b_out
    return z - (z.max() + np.log(np.sum(np.exp(z - z.max()))))


def test_single_frame_saturated_pred_rows():
    """T' = 1: the only alignment emits every label at frame 0 then a blank.
    pred row u is saturated to +1 (u even) or -1 (u odd), so the distribution
    at cell (0,u) is known in closed form and the cost pins the pairing of pred
    row u with label y_u and the final blank at pred row U'."""
    H, V, U = 6, 9, 5
    rng = np.random.default_rng(3)
    W = rng.normal(0, 0.7, size=(H, V))
    bo = rng.normal(0, 0.3, size=V)
    enc = np.zeros((1, 1, H))
    pred = np.zeros((1, U + 1, H))
    for u in range(U + 1):
        pred[0, u] = 40.0 if u % 2 == 0 else -40.0
    y = np.array([[3, 1, 8, 2, 5]])
    res = oracle.loss_and_grads(enc, pred, W, bo, y, [1], [U], 0)
    want = 0.0
    for u in range(U):
        want -= _saturated_dist(W, bo, 1.0 if u % 2 == 0 else -1.0)[y[0, u]]
    want -= _saturated_dist(W, bo, 1.0 if U % 2 == 0 else -1.0)[0]
    assert abs(res["costs"][0] - want) < 1e-12
    # saturated tanh has zero derivative: no gradient reaches enc or pred
    assert np.abs(res["dEnc"]).max() < 1e-30 and np.abs(res["dPred"]).max() < 1e-30


def test_no_labels_closed_form():
    """U' = 0: a single path of T' blanks through column u = 0."""
    inp = make_inputs(2, 7, 3, 8, 11, sigma=0.6, seed=5)
    inp.U_lens[:] = 0
    for b in range(2):
        Tl = int(inp.T_lens[b])
        o = _utt(inp, b)
        z = np.tanh(inp.enc_f64[b, :Tl] + inp.pred_f64[b, 0][None]) @ inp.W_f64 + inp.b_f64
        lsm = z - np.log(np.exp(z).sum(axis=1, keepdims=True))
        assert abs(o["cost"] + lsm[:, 0].sum()) < 1e-12


def test_saturated_joint_square_orientation():
    """H = V and every joint input saturated at +1: z = column sums of W_out +
    b_out in every cell, so the cost is the constant-distribution closed form
    with that bias; using W_out transposed would give row sums instead."""
    H = V = 6
    rng = np.random.default_rng(11)
    W = rng.normal(0, 0.8, size=(H, V))
    bo = np.zeros(V)
    T, U = 4, 3
    enc = np.full((1, T, H), 30.0)
    pred = np.full((1, U + 1, H), 30.0)
    y = np.array([[2, 5, 1]])
    res = oracle.loss_and_grads(enc, pred, W, bo, y, [T], [U], 0)
    want = rnnt.closed_form_zero_weights(T, U, y[0], W.sum(axis=0) + bo, 0)
    wrong = rnnt.closed_form_zero_weights(T, U, y[0], W.sum(axis=1) + bo, 0)
    assert abs(res["costs"][0] - want) < 1e-11
    assert abs(want - wrong) > 1e-3


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("name", ["tiny", "short"])
def test_alpha_beta_agree_and_posterior_sums(name):
    inp = make_config(name)
    for b in range(min(inp.B, 3)):
        o = _utt(inp, b, want_cell_grads=(name == "tiny"))
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        assert abs(o["beta"][0, 0] - o["logP"]) <= 1e-12 * abs(o["logP"])
        # every path leaves every frame by exactly one blank
        np.testing.assert_allclose(o["gB"].sum(axis=1), np.ones(Tl), atol=1e-10)
        # every label is emitted exactly once
        np.testing.assert_allclose(o["gE"][:, :Ul].sum(axis=0), np.ones(Ul), atol=1e-10)
        occ = o["gB"] + o["gE"]
        assert abs(occ.sum() - (Tl + Ul)) < 1e-9
        # occupancy equals exp(alpha + beta - logP)
        np.testing.assert_allclose(occ, np.exp(o["alpha"] + o["beta"] - o["logP"]), atol=1e-10)
        if o["cell_grads"] is not None:
            np.testing.assert_allclose(o["cell_grads"].sum(axis=2), 0.0, atol=1e-12)
        assert abs(o["db"].sum()) < 1e-9
        # db[blank] = sum_cells occ * p_blank - T'
        pblank = np.exp(o["LB"])
        assert abs(o["db"][0] - ((occ * pblank).sum() - Tl)) < 1e-9


# ---------------------------------------------------------------- finite differences

def test_finite_differences_tiny():
    inp = make_inputs(2, 5, 3, 6, 7, sigma=0.5, seed=9, t_range=(3, 5), u_range=(1, 3))
    gc = np.array([1.0, 0.7])

    def total(enc, pred, W, bo):
        c = rnnt.loss_only(enc, pred, W, bo, inp.labels, inp.T_lens, inp.U_lens, 0)
        return float(np.dot(gc, c))

    res = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64,
                                inp.labels, inp.T_lens, inp.U_lens, 0, grad_costs=gc)
    base = [inp.enc_f64.copy(), inp.pred_f64.copy(), inp.W_f64.copy(), inp.b_f64.copy()]
    grads = [res["dEnc"], res["dPred"], res["dW"], res["db"]]
    eps = 1e-6
    for k in range(4):
        it = np.nditer(base[k], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [a.copy() for a in base]
            args_m = [a.copy() for a in base]
            args_p[k][idx] += eps
            args_m[k][idx] -= eps
            fd = (total(*args_p) - total(*args_m)) / (2 * eps)
            assert abs(fd - grads[k][idx]) <= 1e-7 + 1e-6 * abs(fd), (k, idx, fd, grads[k][idx])


# ---------------------------------------------------------------- invariances

def test_padding_invariance():
    """A padded batch gives the same results as each utterance alone; padded
    enc/pred rows and labels past U' (random here) change nothing."""
    inp = make_inputs(3, 9, 6, 8, 10, sigma=0.5, seed=21, t_range=(2, 9), u_range=(0, 6))
    full = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64,
                                 inp.labels, inp.T_lens, inp.U_lens, 0)
    dW = np.zeros_like(inp.W_f64)
    for b in range(3):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        one = oracle.loss_and_grads(inp.enc_f64[b:b + 1, :Tl], inp.pred_f64[b:b + 1, :Ul + 1],
                                    inp.W_f64, inp.b_f64, inp.labels[b:b + 1, :Ul], [Tl], [Ul], 0)
        assert abs(one["costs"][0] - full["costs"][b]) < 1e-12
        np.testing.assert_allclose(full["dEnc"][b, :Tl], one["dEnc"][0], atol=1e-14)
        np.testing.assert_allclose(full["dPred"][b, :Ul + 1], one["dPred"][0], atol=1e-14)
        assert np.all(full["dEnc"][b, Tl:] == 0) and np.all(full["dPred"][b, Ul + 1:] == 0)
        dW += one["dW"]
    np.testing.assert_allclose(full["dW"], dW, atol=1e-13)
    enc2 = inp.enc_f64.copy()
    lab2 = inp.labels.copy()
    for b in range(3):
        enc2[b, int(inp.T_lens[b]):] = 1e3
        lab2[b, int(inp.U_lens[b]):] = 7
    again = oracle.loss_and_grads(enc2, inp.pred_f64, inp.W_f64, inp.b_f64, lab2,
                                  inp.T_lens, inp.U_lens, 0)
    np.testing.assert_array_equal(again["costs"], full["costs"])


def test_vocabulary_permutation():
    inp = make_inputs(2, 6, 4, 5, 9, sigma=0.5, seed=4, t_range=(3, 6), u_range=(1, 4))
    rng = np.random.default_rng(1)
    bo = rng.normal(0, 0.5, size=9)
    perm = rng.permutation(9)              # new column j holds old column perm[j]
    inv = np.argsort(perm)
    a = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, bo, inp.labels,
                              inp.T_lens, inp.U_lens, 0)
    b = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64[:, perm], bo[perm],
                              inv[inp.labels], inp.T_lens, inp.U_lens, int(inv[0]))
    np.testing.assert_allclose(a["costs"], b["costs"], rtol=1e-13)
    np.testing.assert_allclose(a["dW"][:, perm], b["dW"], atol=1e-13)
    np.testing.assert_allclose(a["db"][perm], b["db"], atol=1e-13)
    np.testing.assert_allclose(a["dEnc"], b["dEnc"], atol=1e-13)


def test_shift_and_odd_symmetry():
    """The joint sees enc[t] + pred[u] only (a shift moved from pred to enc
    changes nothing) and tanh is odd (negating enc, pred and W_out together
    changes nothing)."""
    inp = make_inputs(2, 6, 4, 5, 8, sigma=0.5, seed=8, t_range=(4, 6), u_range=(2, 4))
    c = np.random.default_rng(2).normal(0, 0.3, size=5)
    a = rnnt.loss_only(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                       inp.T_lens, inp.U_lens, 0)
    s = rnnt.loss_only(inp.enc_f64 + c, inp.pred_f64 - c, inp.W_f64, inp.b_f64,
                       inp.labels, inp.T_lens, inp.U_lens, 0)
    n = rnnt.loss_only(-inp.enc_f64, -inp.pred_f64, -inp.W_f64, inp.b_f64, inp.labels,
                       inp.T_lens, inp.U_lens, 0)
    np.testing.assert_allclose(a, s, rtol=1e-13)
    np.testing.assert_allclose(a, n, rtol=1e-13)


def test_grad_cost_linearity():
    inp = make_inputs(3, 5, 3, 4, 6, sigma=0.5, seed=12, t_range=(2, 5), u_range=(0, 3))
    gc = np.array([2.0, 0.0, -1.5])
    a = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                              inp.T_lens, inp.U_lens, 0)
    w = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                              inp.T_lens, inp.U_lens, 0, grad_costs=gc)
    np.testing.assert_allclose(w["costs"], a["costs"])
    for b in range(3):
        np.testing.assert_allclose(w["dEnc"][b], gc[b] * a["dEnc"][b], atol=1e-14)
    assert np.all(w["dEnc"][1] == 0)


def test_pool_matches_serial():
    inp = make_inputs(3, 6, 4, 5, 8, sigma=0.5, seed=13, t_range=(3, 6), u_range=(1, 4))
    a = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                              inp.T_lens, inp.U_lens, 0, workers=1)
    b = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                              inp.T_lens, inp.U_lens, 0, workers=3)
    for k in ("costs", "dEnc", "dPred", "dW", "db"):
        np.testing.assert_allclose(a[k], b[k], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- maximum approximation
#
# The maximum approximation ("Daily Papers" page, abstract comparing the
# full-sum criterion with it) keeps only the best alignment.  Its pins do not
# use the oracle's recursion: brute-force maximum over every alignment, the
# bounds that relate it to the full sum, a lattice whose alignments all tie
# exactly (pins the tie rule and the read-back of the path), the closed form
# for W_out = 0, and finite differences.

def _max_margin(LB, LE):
    """Gap between the best and second-best alignment scores (brute force)."""
    T_len, Up1 = LB.shape
    n_moves = T_len - 1 + Up1 - 1
    scores = []
    import itertools
    for slots in itertools.combinations(range(n_moves), Up1 - 1):
        s = set(slots)
        t = u = 0
        lw = 0.0
        for k in range(n_moves):
            if k in s:
                lw += LE[t, u]
                u += 1
            else:
                lw += LB[t, u]
                t += 1
        scores.append(lw + LB[t, u])
    scores = np.sort(np.array(scores))
    return scores[-1] - scores[-2] if len(scores) > 1 else np.inf


def test_max_brute_force_tiny_config():
    inp = make_config("tiny")
    for b in range(inp.B):
        o = _utt(inp, b, criterion="max")
        logP, gB, gE, n = rnnt.brute_force_utterance(o["LB"], o["LE"], criterion="max")
        assert n == 42504
        assert _max_margin(o["LB"], o["LE"]) > 1e-9  # the best alignment is unique
        assert abs(o["logP"] - logP) <= 1e-12 * abs(logP)
        np.testing.assert_array_equal(o["gB"], gB)
        np.testing.assert_array_equal(o["gE"], gE)


@pytest.mark.parametrize("seed", range(6))
def test_max_brute_force_random_small(seed):
    rng = np.random.default_rng(200 + seed)
    T = int(rng.integers(1, 7))
    U = int(rng.integers(0, 6))
    inp = make_inputs(1, T, U, 5, 7, sigma=0.8, seed=50 + seed)
    o = _utt(inp, 0, criterion="max")
    logP, gB, gE, _ = rnnt.brute_force_utterance(o["LB"], o["LE"], criterion="max")
    assert _max_margin(o["LB"], o["LE"]) > 1e-9
    assert abs(o["logP"] - logP) <= 1e-12 * max(1.0, abs(logP))
    np.testing.assert_array_equal(o["gB"], gB)
    np.testing.assert_array_equal(o["gE"], gE)


@pytest.mark.parametrize("name", ["tiny", "short"])
def test_max_bounds_and_path_counts(name):
    """cost_sum <= cost_max <= cost_sum + log(#alignments); the best alignment
    takes T' blanks and U' labels, one outgoing step per visited cell."""
    inp = make_config(name)
    for b in range(min(inp.B, 3)):
        T_len, U_len = int(inp.T_lens[b]), int(inp.U_lens[b])
        s = _utt(inp, b)
        m = _utt(inp, b, criterion="max")
        n_paths = math.comb(T_len + U_len - 1, U_len)
        assert s["cost"] <= m["cost"] + 1e-9
        assert m["cost"] <= s["cost"] + math.log(n_paths) + 1e-9
        assert m["gB"].sum() == T_len and m["gE"].sum() == U_len
        assert np.all(m["gB"] + m["gE"] <= 1.0)
        # the steps chain from (0,0) to the final blank at (T'-1, U')
        t = u = 0
        for _ in range(T_len + U_len):
            if m["gB"][t, u]:
                if (t, u) == (T_len - 1, U_len):
                    break
                t += 1
            else:
                assert m["gE"][t, u]
                u += 1
        assert (t, u) == (T_len - 1, U_len)


def test_max_exact_ties_take_blank_predecessor():
    """LB = -1, LE = -2 everywhere: every alignment scores exactly
    -(T' + 2 U'), and taking the blank predecessor on each tie reads back the
    alignment that emits all labels in frame 0."""
    T_len, U_len = 5, 3
    LB = np.full((T_len, U_len + 1), -1.0)
    LE = np.full((T_len, U_len), -2.0)
    _, logP, gB, gE = rnnt.viterbi_lattice(LB, LE)
    assert logP == -(T_len + 2 * U_len)
    want_gB = np.zeros((T_len, U_len + 1))
    want_gB[:, U_len] = 1.0
    want_gE = np.zeros((T_len, U_len + 1))
    want_gE[0, :U_len] = 1.0
    np.testing.assert_array_equal(gB, want_gB)
    np.testing.assert_array_equal(gE, want_gE)


@pytest.mark.parametrize("name", ["tiny", "short"])
def test_max_zero_weights_closed_form(name):
    inp = make_config(name)
    inp.W_f64 = np.zeros_like(inp.W_f64)
    c = rnnt.loss_only(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                       inp.T_lens, inp.U_lens, inp.blank, criterion="max")
    for b in range(inp.B):
        want = oracle.closed_form_zero_weights_max(int(inp.T_lens[b]), int(inp.U_lens[b]),
                                                   inp.labels[b], inp.b_f64, inp.blank)
        assert abs(c[b] - want) <= 1e-10 * abs(want)


def test_max_finite_differences_tiny():
    inp = make_inputs(2, 5, 3, 6, 7, sigma=0.5, seed=9, t_range=(3, 5), u_range=(1, 3))
    gc = np.array([1.0, -0.6])

    def total(enc, pred, W, bo):
        c = rnnt.loss_only(enc, pred, W, bo, inp.labels, inp.T_lens, inp.U_lens, 0,
                           criterion="max")
        return float(np.dot(gc, c))

    res = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64,
                                inp.labels, inp.T_lens, inp.U_lens, 0, grad_costs=gc,
                                criterion="max")
    base = [inp.enc_f64.copy(), inp.pred_f64.copy(), inp.W_f64.copy(), inp.b_f64.copy()]
    grads = [res["dEnc"], res["dPred"], res["dW"], res["db"]]
    eps = 1e-6
    for k in range(4):
        it = np.nditer(base[k], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args_p = [a.copy() for a in base]
            args_m = [a.copy() for a in base]
            args_p[k][idx] += eps
            args_m[k][idx] -= eps
            fd = (total(*args_p) - total(*args_m)) / (2 * eps)
            assert abs(fd - grads[k][idx]) <= 1e-7 + 1e-6 * abs(fd), (k, idx, fd, grads[k][idx])
