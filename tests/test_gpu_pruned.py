"""GPU parity of the pruned transducer loss ("Pruned RNN-T for fast,
memory-efficient ASR training", Abstract) against oracle/pruned.py.

Compared: the window starts (exactly: they are integers decided by rounding
a float64 centre; a frame whose oracle centre lies within 1e-7 of a rounding
boundary would allow either, and then its utterance's costs and gradients
are not compared -- none of these inputs has one), the simple joiner's costs
(float64 on both sides: 1e-6), the pruned costs and every gradient (the
dtype's bar), utterances that no band can hold (NaN cost, zero gradients,
data-error bit 16)."""
import math
import os

import numpy as np
import pytest

from oracle import rnnt
from synth import make_config, make_inputs

from gpu_common import check_costs, check_grad, pruned_oracle, to_device

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)
SIMPLE_REL = 1e-6


def _run(inp, S, tiles, grad_costs=None, bwd=True):
    import torch
    import rnn_joint_transducer_amd as rj
    d = to_device(inp)
    dc = rj.RNNTJ_BF16 if inp.dtype == "bf16" else rj.RNNTJ_F32
    costs, simple, saved = rj.rnnt_joint_loss_pruned_fwd(**d, S=S, blank=inp.blank,
                                                         tile_t=tiles[0], tile_u=tiles[1],
                                                         tile_v=tiles[2])
    bounds = rj.rnnt_joint_loss_pruned_bounds(saved, inp.B, inp.T, inp.U, inp.H, inp.V, dc,
                                              *tiles)
    out = dict(costs=costs, simple=simple, bounds=bounds)
    if bwd:
        gc = None if grad_costs is None else torch.tensor(grad_costs, dtype=torch.float32,
                                                          device="cuda")
        g = rj.rnnt_joint_loss_bwd(**d, saved=saved, blank=inp.blank, tile_t=tiles[0],
                                   tile_u=tiles[1], tile_v=tiles[2], grad_costs=gc)
        out.update(dEnc=g[0], dPred=g[1], dW=g[2], db=g[3])
    out["status"] = rj.rnnt_joint_loss_status(saved)
    return {k: (v.cpu().numpy().astype(np.float64) if k != "bounds" and hasattr(v, "cpu")
                else (v.cpu().numpy() if hasattr(v, "cpu") else v)) for k, v in out.items()}


def _ambiguous(o, S):
    """Does some frame's centre lie within 1e-7 of a rounding boundary?"""
    x = o["centres"] - (S - 1) / 2.0 + 0.5
    return bool(np.any(np.abs(x - np.round(x)) < 1e-7))


def _check_utts(inp, S, g, refs, utts, grads=True):
    """Bounds, simple and pruned costs of `utts`, and (grads) their d_enc /
    d_pred rows; returns the utterances whose results were compared."""
    compared = []
    for b, o in zip(utts, refs):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        assert g["simple"][b] == pytest.approx(o["simple_cost"], rel=SIMPLE_REL), b
        same = np.array_equal(g["bounds"][b, :Tl], o["bounds"])
        amb = _ambiguous(o, S)
        assert same or amb, (b, g["bounds"][b, :Tl], o["bounds"])
        if not same:
            print(f"  utterance {b}: a centre at a rounding boundary; not compared", flush=True)
            continue
        if not o["feasible"]:
            assert math.isnan(g["costs"][b])
            assert np.all(g["dEnc"][b] == 0) and np.all(g["dPred"][b] == 0) if grads else True
            continue
        check_costs(g["costs"], [o["cost"]], inp.dtype, idx=[b])
        if grads:
            check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
            check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)
            assert np.all(g["dEnc"][b, Tl:] == 0) and np.all(g["dPred"][b, Ul + 1:] == 0)
        compared.append(b)
    return compared


def _full(inp, S, tiles, gcs=None):
    """Every output of the batch against the oracle."""
    g = _run(inp, S, tiles, grad_costs=gcs)
    refs = pruned_oracle(inp, S, range(inp.B), WORKERS, grad_costs=gcs)
    cmp = _check_utts(inp, S, g, refs, range(inp.B))
    assert len(cmp) + sum(not o["feasible"] for o in refs) == inp.B
    dW = sum(o["dW"] for o in refs)
    db = sum(o["db"] for o in refs)
    check_grad("d_W_out", g["dW"], dW, inp.dtype)
    check_grad("d_b_out", g["db"], db, inp.dtype)
    return g, refs


@pytest.mark.parametrize("S", [2, 3])
@pytest.mark.parametrize("tiles", [(16, 8, 0), (0, 8, 128)])
def test_pruned_tiny(S, tiles):
    inp = make_config("tiny")
    print(f"[pruned tiny S={S} tiles={tiles}]", flush=True)
    g, refs = _full(inp, S, tiles, gcs=[1.0, -0.5])
    assert g["status"] == 0
    assert np.any(g["bounds"] > 0)  # the band is narrower than the lattice


def test_pruned_whole_band_is_the_full_sum():
    """S = U'+1 on every utterance: the band is the whole lattice and the
    pruned path returns the full-sum costs and gradients."""
    inp = make_config("tiny")
    g = _run(inp, inp.U + 1, (16, 8, 0))
    assert g["status"] == 0 and np.all(g["bounds"] == 0)
    ref = rnnt.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                              inp.T_lens, inp.U_lens, 0)
    check_costs(g["costs"], ref["costs"], "fp32")
    for k, r in (("dEnc", "dEnc"), ("dPred", "dPred"), ("dW", "dW"), ("db", "db")):
        check_grad(k, g[k], ref[r], "fp32")


@pytest.mark.parametrize("tiles", [(64, 64, 128), (16, 0, 0)])
def test_pruned_short(tiles):
    inp = make_config("short")
    print(f"[pruned short S=4 tiles={tiles}]", flush=True)
    g, _ = _full(inp, 4, tiles)
    assert g["status"] == 0


@pytest.mark.parametrize("dtype,sigma", [("fp32", 0.4), ("bf16", 0.4), ("bf16", 1.5)])
def test_pruned_ragged_and_infeasible(dtype, sigma):
    """Ragged shapes (T not a multiple of 16, U+1 not of 8, V not of 128), a
    one-frame utterance, one without labels, signed cost weights, large
    logits, and an utterance that no band of S = 3 can hold (U' = 5 > 2 T')."""
    inp = make_inputs(6, 37, 11, 48, 40, dtype=dtype, sigma=sigma, seed=17, t_range=(1, 37),
                      u_range=(0, 11))
    inp.T_lens[:] = [37, 1, 20, 2, 33, 25]
    inp.U_lens[:] = [11, 2, 0, 5, 7, 9]
    gcs = [1.0, 0.5, 2.0, 1.0, -1.0, 0.25]
    print(f"[pruned ragged {dtype} sigma={sigma}]", flush=True)
    g, refs = _full(inp, 3, (16, 8, 0), gcs=gcs)
    assert not refs[3]["feasible"] and all(o["feasible"] for k, o in enumerate(refs) if k != 3)
    assert g["status"] == 16


def test_pruned_fp32_wide_hidden():
    """fp32 at H = 640 (h rebuilt in 256-wide parts by the joint kernel),
    S = 4: every output against the oracle."""
    inp = make_inputs(3, 30, 9, 640, 200, dtype="fp32", sigma=0.05, seed=29, t_range=(12, 30),
                      u_range=(2, 9))
    print("[pruned fp32 H=640 S=4 tiles=(16, 8, 0)]", flush=True)
    g, _ = _full(inp, 4, (16, 8, 0), gcs=[1.0, -0.5, 2.0])
    assert g["status"] == 0


@pytest.mark.parametrize("tiles", [(64, 64, 0), (16, 0, 0)])
def test_pruned_deterministic_mode(tiles):
    """Deterministic mode over a banded tile list (rows of the chunk hold
    different tile columns): bitwise identical outputs run after run, and
    still the oracle's."""
    from rnn_joint_transducer_amd import _lib
    inp = make_inputs(4, 70, 23, 48, 40, dtype="fp32", sigma=0.4, seed=31, t_range=(40, 70),
                      u_range=(10, 23))
    gcs = [1.0, -0.5, 2.0, 0.25]
    old = _lib.get_flags()
    try:
        _lib.set_flags(_lib.FLAG_DETERMINISTIC)
        print(f"[pruned deterministic S=3 tiles={tiles}]", flush=True)
        runs = [_run(inp, 3, tiles, grad_costs=gcs) for _ in range(2)]
    finally:
        _lib.set_flags(old)
    for k in ("costs", "simple", "bounds", "dEnc", "dPred", "dW", "db"):
        assert np.array_equal(runs[0][k], runs[1][k], equal_nan=True), k
    refs = pruned_oracle(inp, 3, range(inp.B), WORKERS, grad_costs=gcs)
    cmp = _check_utts(inp, 3, runs[0], refs, range(inp.B))
    assert len(cmp) == inp.B
    check_grad("d_W_out", runs[0]["dW"], sum(o["dW"] for o in refs), inp.dtype)
    check_grad("d_b_out", runs[0]["db"], sum(o["db"] for o in refs), inp.dtype)


def test_pruned_medium():
    """The medium workload (bf16, H = 640, V = 1024) with S = 5: every
    utterance's bounds, simple and pruned cost; the gradients of one
    utterance; d_W_out and d_b_out of a two-utterance sub-batch."""
    import dataclasses
    inp = make_config("medium")
    S, tiles = 5, (128, 0, 256)
    print(f"[pruned medium S={S} tiles={tiles}]", flush=True)
    g = _run(inp, S, tiles)
    assert g["status"] == 0
    refs = pruned_oracle(inp, S, range(inp.B), WORKERS, want_grads=False)
    _check_utts(inp, S, g, refs, range(inp.B), grads=False)
    b = 7
    o = pruned_oracle(inp, S, [b], 1)[0]
    Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
    check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
    check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)
    utts = [3, 11]
    sub = dataclasses.replace(
        inp, B=2, enc=inp.enc[utts], pred=inp.pred[utts], labels=inp.labels[utts],
        T_lens=inp.T_lens[utts], U_lens=inp.U_lens[utts], enc_f64=inp.enc_f64[utts],
        pred_f64=inp.pred_f64[utts])
    gs = _run(sub, S, tiles)
    rs = pruned_oracle(sub, S, range(2), 2)
    check_grad("d_W_out(sub)", gs["dW"], rs[0]["dW"] + rs[1]["dW"], inp.dtype)
    check_grad("d_b_out(sub)", gs["db"], rs[0]["db"] + rs[1]["db"], inp.dtype)
