"""GPU parity of the token-and-duration transducer loss ("Daily Papers" page,
Token-and-Duration Transducer abstract) against oracle/tdt.py: every cost
and every gradient (enc, pred, W_out, b_out, W_dur, b_dur), untiled and
tiled, fp32 and bf16, several duration sets, an utterance no alignment
reaches, and the medium workload (all costs, one utterance's gradients, the
weight gradients of a sub-batch)."""
import math
import os

import numpy as np
import pytest

from synth import make_config, make_duration_head, make_inputs

from gpu_common import check_costs, check_grad, tdt_oracle, to_device

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _head_to_device(inp, head):
    import torch
    if inp.dtype == "fp32":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).cuda()
    return conv(head.W_dur), conv(head.b_dur)


def _run(inp, head, tiles, gcs=None, bwd=True):
    import torch
    import rnn_joint_transducer_amd as rj
    d = to_device(inp)
    Wd, bd = _head_to_device(inp, head)
    costs, saved = rj.rnnt_joint_loss_tdt_fwd(**d, W_dur=Wd, b_dur=bd, durations=head.durations,
                                              blank=inp.blank, tile_t=tiles[0], tile_u=tiles[1],
                                              tile_v=tiles[2])
    out = dict(costs=costs)
    if bwd:
        gc = None if gcs is None else torch.tensor(gcs, dtype=torch.float32, device="cuda")
        g = rj.rnnt_joint_loss_tdt_bwd(**d, W_dur=Wd, b_dur=bd, durations=head.durations,
                                       saved=saved, blank=inp.blank, tile_t=tiles[0],
                                       tile_u=tiles[1], tile_v=tiles[2], grad_costs=gc)
        out.update(zip(("dEnc", "dPred", "dW", "db", "dWd", "dbd"), g))
    out["status"] = rj.rnnt_joint_loss_status(saved)
    return {k: (v.cpu().double().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()}


def _compare(inp, g, refs, utts=None, weights=True):
    utts = list(range(inp.B)) if utts is None else utts
    live = []
    for b, o in zip(utts, refs):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        if math.isinf(o["cost"]):  # no alignment reaches the end
            assert g["costs"][b] == math.inf, (b, g["costs"][b])
            if "dEnc" in g:
                assert np.all(g["dEnc"][b] == 0) and np.all(g["dPred"][b] == 0)
            continue
        check_costs(g["costs"], [o["cost"]], inp.dtype, idx=[b])
        if "dEnc" in o and "dEnc" in g:
            check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
            check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)
            assert np.all(g["dEnc"][b, Tl:] == 0) and np.all(g["dPred"][b, Ul + 1:] == 0)
        live.append(b)
    if weights:
        for k, name in (("dW", "d_W_out"), ("db", "d_b_out"), ("dWd", "d_W_dur"),
                        ("dbd", "d_b_dur")):
            check_grad(name, g[k], sum(o[k] for o in refs), inp.dtype)
    return live


@pytest.mark.parametrize("durations", [(0, 1, 2), (1, 2, 4), (0, 1, 2, 3, 4, 5, 6, 7)])
@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_tdt_tiny(durations, tiles):
    inp = make_config("tiny")
    head = make_duration_head(inp, durations, seed=1, sigma=0.3)
    print(f"[tdt tiny durations={durations} tiles={tiles}]", flush=True)
    gcs = [1.0, -0.5]
    g = _run(inp, head, tiles, gcs=gcs)
    assert g["status"] == 0
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, grad_costs=gcs)
    assert len(_compare(inp, g, refs)) == inp.B


@pytest.mark.parametrize("durations", [(1,), (0, 2), (1, 2, 3, 5), (0, 1, 2, 3, 4, 5),
                                       (1, 2, 3, 4, 5, 6, 7), (0, 1, 3, 4, 6, 7, 8, 9)])
def test_tdt_every_duration_count(durations):
    """The token-and-duration kernels are instantiated per duration count:
    every count from the ones the other tests leave out (1, 2, 4, 6, 7) and
    8 with gaps in the set, with and without the zero duration, against the
    oracle (every cost and gradient, tiled)."""
    inp = make_inputs(3, 23, 6, 32, 24, dtype="fp32", sigma=0.3, seed=41, t_range=(9, 23),
                      u_range=(1, 6))
    head = make_duration_head(inp, durations, seed=5, sigma=0.3)
    gcs = [1.0, -0.5, 2.0]
    print(f"[tdt durations={durations}]", flush=True)
    g = _run(inp, head, (16, 8, 0), gcs=gcs)
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, grad_costs=gcs)
    live = _compare(inp, g, refs)
    # (durations {0, 2} reach only even frame counts: an odd T' has no
    # alignment, cost +inf on both sides)
    assert len(live) >= 1


@pytest.mark.parametrize("tiles", [(0, 0, 0), (64, 64, 128)])
def test_tdt_short(tiles):
    inp = make_config("short")
    head = make_duration_head(inp, (0, 1, 2, 3, 4), seed=2, sigma=0.2)
    print(f"[tdt short tiles={tiles}]", flush=True)
    g = _run(inp, head, tiles)
    assert g["status"] == 0
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS)
    assert len(_compare(inp, g, refs)) == inp.B


@pytest.mark.parametrize("dtype,sigma", [("fp32", 0.4), ("bf16", 0.4), ("bf16", 1.5)])
def test_tdt_ragged_and_unreachable(dtype, sigma):
    """Ragged shapes, a one-frame utterance, one without labels, signed cost
    weights, large logits; durations (1, 2, 4) make every label cover at
    least one frame, so the utterance with U' = T' has no alignment (cost
    +inf, zero gradients)."""
    inp = make_inputs(5, 37, 11, 48, 40, dtype=dtype, sigma=sigma, seed=19, t_range=(1, 37),
                      u_range=(0, 11))
    inp.T_lens[:] = [37, 1, 20, 9, 30]
    inp.U_lens[:] = [11, 0, 3, 9, 7]
    head = make_duration_head(inp, (1, 2, 4), seed=3, sigma=sigma)
    gcs = [1.0, 0.5, -1.0, 1.0, 2.0]
    print(f"[tdt ragged {dtype} sigma={sigma}]", flush=True)
    g = _run(inp, head, (16, 8, 0), gcs=gcs)
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, grad_costs=gcs)
    assert math.isinf(refs[3]["cost"])
    live = _compare(inp, g, refs)
    assert 3 not in live and len(live) == inp.B - 1


@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_tdt_fp32_wide_hidden(tiles):
    """fp32 at H = 640 (h rebuilt in 256-wide parts by the joint kernel):
    every cost and gradient, durations 0..4."""
    inp = make_inputs(3, 30, 9, 640, 200, dtype="fp32", sigma=0.05, seed=23, t_range=(12, 30),
                      u_range=(2, 9))
    head = make_duration_head(inp, (0, 1, 2, 3, 4), seed=4, sigma=0.1)
    gcs = [1.0, -0.5, 2.0]
    print(f"[tdt fp32 H=640 tiles={tiles}]", flush=True)
    g = _run(inp, head, tiles, gcs=gcs)
    assert g["status"] == 0
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, grad_costs=gcs)
    assert len(_compare(inp, g, refs)) == inp.B


@pytest.mark.parametrize("tiles", [(16, 8, 0), (0, 0, 0)])
def test_tdt_deterministic_mode(tiles):
    """Deterministic mode with the duration head: three runs bitwise equal in
    every output (the duration head's d_pred by its own pass, d_W_dur /
    d_b_dur from per-block sums added in order), and the oracle's values."""
    from rnn_joint_transducer_amd import _lib
    inp = make_inputs(4, 40, 9, 64, 40, dtype="fp32", sigma=0.3, seed=43, t_range=(20, 40),
                      u_range=(2, 9))
    head = make_duration_head(inp, (0, 1, 2, 3), seed=6, sigma=0.3)
    gcs = [1.0, -0.5, 2.0, 0.25]
    old = _lib.get_flags()
    try:
        _lib.set_flags(_lib.FLAG_DETERMINISTIC)
        print(f"[tdt deterministic tiles={tiles}]", flush=True)
        runs = [_run(inp, head, tiles, gcs=gcs) for _ in range(3)]
    finally:
        _lib.set_flags(old)
    for g in runs[1:]:
        for k in ("costs", "dEnc", "dPred", "dW", "db", "dWd", "dbd"):
            assert np.array_equal(g[k], runs[0][k]), k
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, grad_costs=gcs)
    assert len(_compare(inp, runs[0], refs)) == inp.B


def test_tdt_medium():
    """Medium workload (bf16, H = 640, V = 1024), durations 0..4: every cost,
    one utterance's gradients, the weight gradients of a two-utterance
    sub-batch at the full sizes."""
    import dataclasses
    inp = make_config("medium")
    head = make_duration_head(inp, (0, 1, 2, 3, 4), seed=4)
    tiles = (128, 0, 256)
    print(f"[tdt medium tiles={tiles}]", flush=True)
    g = _run(inp, head, tiles)
    assert g["status"] == 0
    refs = tdt_oracle(inp, head, range(inp.B), WORKERS, want_grads=False)
    _compare(inp, g, refs, weights=False)
    b = 7
    o = tdt_oracle(inp, head, [b], 1)[0]
    Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
    check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
    check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)
    utts = [3, 11]
    sub = dataclasses.replace(
        inp, B=2, enc=inp.enc[utts], pred=inp.pred[utts], labels=inp.labels[utts],
        T_lens=inp.T_lens[utts], U_lens=inp.U_lens[utts], enc_f64=inp.enc_f64[utts],
        pred_f64=inp.pred_f64[utts])
    gs = _run(sub, head, tiles)
    rs = tdt_oracle(sub, head, range(2), 2)
    _compare(sub, gs, rs)
