"""Pins of the joint-input-projection oracle (oracle/proj.py) against facts
that do not come from it:

* identity projections reduce it exactly to the plain joint,
* central finite differences of the cost in every projection parameter and
  in both encodings (a transposed or misplaced operand fails them),
* the adjoint identities <dy, d(x W)> = <dx_grad, dx> and <dy, x dW> =
  <dW_grad, dW> of the linear-map gradients,
* invariance under a permutation of the hidden units applied to W_enc,
  b_enc, W_pred, b_pred and the rows of W_out, with the gradients permuted
  alike,
* W_out = 0: the cost no longer depends on the projections (closed form) and
  every projection gradient is exactly zero.
"""
import numpy as np
import pytest

import oracle
from oracle import proj, rnnt


def _case(seed=7, B=2, T=4, U=2, E=5, P=3, H=6, V=7, sigma=0.6):
    rng = np.random.default_rng(seed)
    enc = rng.normal(0, sigma, (B, T, E))
    pred = rng.normal(0, sigma, (B, U + 1, P))
    W_enc = rng.normal(0, sigma, (E, H))
    b_enc = rng.normal(0, sigma, H)
    W_pred = rng.normal(0, sigma, (P, H))
    b_pred = rng.normal(0, sigma, H)
    W = rng.normal(0, sigma, (H, V))
    b_out = rng.normal(0, sigma, V)
    labels = rng.integers(1, V, (B, U))
    T_lens = np.array([T, T - 1][:B])
    U_lens = np.array([U, U - 1][:B])
    return dict(enc=enc, pred=pred, W_enc=W_enc, b_enc=b_enc, W_pred=W_pred, b_pred=b_pred, W=W,
                b_out=b_out, labels=labels, T_lens=T_lens, U_lens=U_lens, blank=0)


def _run(c, gcs=None):
    return proj.projected_loss_and_grads(c["enc"], c["pred"], c["W_enc"], c["b_enc"], c["W_pred"],
                                         c["b_pred"], c["W"], c["b_out"], c["labels"], c["T_lens"],
                                         c["U_lens"], c["blank"], grad_costs=gcs)


def test_identity_projection_is_the_plain_joint():
    c = _case(E=6, P=6, H=6)
    c["W_enc"] = np.eye(6)
    c["W_pred"] = np.eye(6)
    c["b_enc"] = np.zeros(6)
    c["b_pred"] = np.zeros(6)
    r = _run(c)
    ref = rnnt.loss_and_grads(c["enc"], c["pred"], c["W"], c["b_out"], c["labels"], c["T_lens"],
                              c["U_lens"], 0)
    np.testing.assert_array_equal(r["costs"], ref["costs"])
    np.testing.assert_array_equal(r["dEnc"], ref["dEnc"])
    np.testing.assert_array_equal(r["dPred"], ref["dPred"])
    np.testing.assert_array_equal(r["dW"], ref["dW"])


@pytest.mark.parametrize("name", ["W_enc", "b_enc", "W_pred", "b_pred", "enc", "pred"])
def test_finite_differences(name):
    c = _case()
    gcs = np.array([1.0, -0.7])
    r = _run(c, gcs)
    grad = {"W_enc": r["dW_enc"], "b_enc": r["db_enc"], "W_pred": r["dW_pred"],
            "b_pred": r["db_pred"], "enc": r["dEnc"], "pred": r["dPred"]}[name]
    rng = np.random.default_rng(3)
    eps = 1e-6
    for _ in range(6):
        idx = tuple(rng.integers(0, n) for n in c[name].shape)
        cp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        cm = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        cp[name][idx] += eps
        cm[name][idx] -= eps
        fd = (np.dot(gcs, _run(cp)["costs"]) - np.dot(gcs, _run(cm)["costs"])) / (2 * eps)
        assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_linear_grads_adjoint_identities():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(3, 5, 4))
    W = rng.normal(size=(4, 6))
    dy = rng.normal(size=(3, 5, 6))
    gx, gW, gb = proj.linear_grads(x, W, dy)
    dx = rng.normal(size=x.shape)
    dW = rng.normal(size=W.shape)
    db = rng.normal(size=6)
    assert np.isclose(np.sum(dy * (dx @ W)), np.sum(gx * dx), rtol=1e-12)
    assert np.isclose(np.sum(dy * (x @ dW)), np.sum(gW * dW), rtol=1e-12)
    assert np.isclose(np.sum(dy * db), np.sum(gb * db), rtol=1e-12)


def test_hidden_unit_permutation():
    c = _case(seed=19)
    r = _run(c)
    perm = np.random.default_rng(5).permutation(c["W"].shape[0])
    cq = dict(c)
    cq["W_enc"] = c["W_enc"][:, perm]
    cq["b_enc"] = c["b_enc"][perm]
    cq["W_pred"] = c["W_pred"][:, perm]
    cq["b_pred"] = c["b_pred"][perm]
    cq["W"] = c["W"][perm, :]
    q = _run(cq)
    np.testing.assert_allclose(q["costs"], r["costs"], rtol=1e-12)
    np.testing.assert_allclose(q["dW_enc"], r["dW_enc"][:, perm], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(q["db_pred"], r["db_pred"][perm], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(q["dW"], r["dW"][perm, :], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(q["dEnc"], r["dEnc"], rtol=1e-9, atol=1e-12)


def test_zero_output_weights_cut_the_projections_off():
    c = _case(seed=23)
    c["W"] = np.zeros_like(c["W"])
    r = _run(c)
    want = [oracle.closed_form_zero_weights(int(c["T_lens"][b]), int(c["U_lens"][b]),
                                            c["labels"][b], c["b_out"], 0)
            for b in range(len(c["T_lens"]))]
    np.testing.assert_allclose(r["costs"], want, rtol=1e-12)
    for k in ("dW_enc", "db_enc", "dW_pred", "db_pred", "dEnc", "dPred"):
        assert np.all(r[k] == 0.0), k
