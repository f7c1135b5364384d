"""GPU parity of the joint input projections (rnnt_joint_proj_fwd / _bwd
through the C ABI) against the float64 oracle (oracle/proj.py): the whole
chain projections -> fused joint + loss -> projection gradients on small
batches and on a two-utterance sub-batch of the medium workload at its full
sizes, and the three GEMMs alone at the full medium shapes with a seeded
synthetic upstream gradient."""
import os

import numpy as np
import pytest

from oracle import proj
from synth import make_config, make_inputs, make_proj_inputs

from gpu_common import BF16_REL, FP32_GRAD_ABS, check_costs, check_grad

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _dev(a, dtype):
    import torch
    if dtype == "fp32" or a.dtype != np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.float().cpu().double().numpy()


def _check_act(name, gpu, ref, dtype):
    """Projected activations (not gradients): fp32 within 1e-5 of max(1,|ref|),
    bf16 (one rounding of the fp32 result) within the bf16 bound."""
    err = float(np.max(np.abs(gpu - ref)))
    scale = max(1.0, float(np.max(np.abs(ref))))
    tol = 1e-5 if dtype == "fp32" else BF16_REL
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol} * {scale:.3g}"


def _run_chain(inp, pj, tiles, grad_costs=None):
    """Projections, fused joint + loss and projection gradients on the GPU."""
    import torch
    import rnn_joint_transducer_amd as rj
    dt = inp.dtype
    enc_in, pred_in = _dev(pj.enc_in, dt), _dev(pj.pred_in, dt)
    W_enc, b_enc = _dev(pj.W_enc, dt), _dev(pj.b_enc, dt)
    W_pred, b_pred = _dev(pj.W_pred, dt), _dev(pj.b_pred, dt)
    W_out, b_out = _dev(inp.W, dt), _dev(inp.b, dt)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    labels, T_lens, U_lens = i32(inp.labels), i32(inp.T_lens), i32(inp.U_lens)
    enc_p = rj.rnnt_joint_proj_fwd(enc_in, W_enc, b_enc)
    pred_p = rj.rnnt_joint_proj_fwd(pred_in, W_pred, b_pred)
    tt, tu, tv = tiles
    costs, saved = rj.rnnt_joint_loss_fwd(enc_p, pred_p, W_out, b_out, labels, T_lens, U_lens,
                                          blank=inp.blank, tile_t=tt, tile_u=tu, tile_v=tv)
    gc = None if grad_costs is None else torch.tensor(grad_costs, dtype=torch.float32).cuda()
    dEncP, dPredP, dW, db = rj.rnnt_joint_loss_bwd(enc_p, pred_p, W_out, b_out, labels, T_lens,
                                                    U_lens, saved=saved, blank=inp.blank,
                                                    tile_t=tt, tile_u=tu, tile_v=tv, grad_costs=gc)
    d_enc, dW_enc, db_enc = rj.rnnt_joint_proj_bwd(enc_in, W_enc, dEncP)
    d_pred, dW_pred, db_pred = rj.rnnt_joint_proj_bwd(pred_in, W_pred, dPredP)
    status = rj.rnnt_joint_loss_status(saved)
    out = dict(costs=costs, enc_p=enc_p, pred_p=pred_p, dEnc=d_enc, dPred=d_pred, dW_enc=dW_enc,
               db_enc=db_enc, dW_pred=dW_pred, db_pred=db_pred, dW=dW, db=db)
    return {k: _np(v) for k, v in out.items()}, status


def _oracle(inp, pj, grad_costs=None, idx=None):
    sl = slice(None) if idx is None else idx
    return proj.projected_loss_and_grads(
        pj.enc_in_f64[sl], pj.pred_in_f64[sl], pj.W_enc_f64, pj.b_enc_f64, pj.W_pred_f64,
        pj.b_pred_f64, inp.W_f64, inp.b_f64, inp.labels[sl], inp.T_lens[sl], inp.U_lens[sl],
        inp.blank, grad_costs=grad_costs, workers=WORKERS)


def _compare(inp, g, ref):
    dt = inp.dtype
    check_costs(g["costs"], ref["costs"], dt)
    _check_act("enc_p", g["enc_p"], ref["enc_p"], dt)
    _check_act("pred_p", g["pred_p"], ref["pred_p"], dt)
    for k in ("dEnc", "dPred", "dW_enc", "db_enc", "dW_pred", "db_pred", "dW", "db"):
        check_grad(k, g[k], ref[k], dt)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_projected_chain_small(dtype, tiles):
    """E = 48 and P = 32 into H = 64 (partial k-steps and tiles), ragged
    lengths, an utterance without labels, mixed-sign cost weights."""
    inp = make_inputs(3, 21, 6, 64, 72, dtype=dtype, sigma=0.3, seed=61, t_range=(4, 21),
                      u_range=(0, 6))
    pj = make_proj_inputs(inp, 48, 32, seed=62, sigma=0.3)
    gcs = [1.0, -0.5, 0.75]
    print(f"[proj chain {dtype} tiles={tiles}]", flush=True)
    g, status = _run_chain(inp, pj, tiles, gcs)
    assert status == 0
    _compare(inp, g, _oracle(inp, pj, gcs))
    # gradients of encoder rows past each utterance's frames are exactly zero
    for b in range(inp.B):
        assert np.all(g["dEnc"][b, inp.T_lens[b]:] == 0)


def test_projected_chain_medium_subbatch():
    """Two utterances of the medium workload at its full sizes (bf16, H = E =
    P = 640, V = 1024, tiled 64 x 64 x 256)."""
    full = make_config("medium")
    idx = [3, 11]
    inp = make_inputs(2, full.T, full.U, full.H, full.V, dtype=full.dtype, sigma=0.05, seed=0)
    inp.T_lens = full.T_lens[idx].copy()
    inp.U_lens = full.U_lens[idx].copy()
    inp.labels = full.labels[idx].copy()
    pj = make_proj_inputs(inp, 640, 640, seed=71)
    print("[proj chain medium sub-batch]", flush=True)
    g, status = _run_chain(inp, pj, (64, 64, 256))
    assert status == 0
    _compare(inp, g, _oracle(inp, pj))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("M,K,N", [(16 * 500, 640, 640), (16 * 101, 640, 640), (1234, 48, 80)])
def test_projection_gemms_full_size(dtype, M, K, N):
    """The three products at the medium workload's projection shapes (enc:
    16*500 rows, pred: 16*101 rows) and a ragged one, against float64
    matmuls; the upstream gradient is seeded synthetic data."""
    import rnn_joint_transducer_amd as rj
    from synth import _cast
    rng = np.random.default_rng(M + K + N)
    x_s, x64 = _cast(rng.normal(0, 0.5, (M, K)), dtype)
    W_s, W64 = _cast(rng.normal(0, 1 / np.sqrt(K), (K, N)), dtype)
    b_s, b64 = _cast(rng.normal(0, 0.1, N), dtype)
    dy = rng.normal(0, 1.0, (M, N)).astype(np.float32)
    print(f"[proj gemm {dtype} M={M} K={K} N={N}]", flush=True)
    y = _np(rj.rnnt_joint_proj_fwd(_dev(x_s, dtype), _dev(W_s, dtype), _dev(b_s, dtype)))
    dx, dW, db = rj.rnnt_joint_proj_bwd(_dev(x_s, dtype), _dev(W_s, dtype), _dev(dy, "fp32"))
    _check_act("y", y, proj.linear(x64, W64, b64), dtype)
    rdx, rdW, rdb = proj.linear_grads(x64, W64, dy.astype(np.float64))
    # operands are exact in float64 and accumulate in fp32 on the GPU, so the
    # fp32 gradient bound applies to both dtypes
    for name, gv, rv in (("dx", _np(dx), rdx), ("dW", _np(dW), rdW), ("db", _np(db), rdb)):
        err = float(np.max(np.abs(gv - rv)))
        assert err <= FP32_GRAD_ABS * max(1.0, float(np.max(np.abs(rv))) / 100), (name, err)


def test_projection_autograd_matches_explicit_calls():
    """rnnt_joint_proj + rnnt_joint_loss under torch.autograd give the
    gradients of the explicit call sequence."""
    import torch
    import rnn_joint_transducer_amd as rj
    inp = make_inputs(2, 13, 4, 64, 40, dtype="fp32", sigma=0.3, seed=81, t_range=(6, 13),
                      u_range=(1, 4))
    pj = make_proj_inputs(inp, 32, 48, seed=82, sigma=0.3)
    g, _ = _run_chain(inp, pj, (16, 8, 0))
    t = {k: _dev(getattr(pj, k), "fp32").requires_grad_() for k in
         ("enc_in", "pred_in", "W_enc", "b_enc", "W_pred", "b_pred")}
    W_out, b_out = _dev(inp.W, "fp32").requires_grad_(), _dev(inp.b, "fp32").requires_grad_()
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    enc_p = rj.rnnt_joint_proj(t["enc_in"], t["W_enc"], t["b_enc"])
    pred_p = rj.rnnt_joint_proj(t["pred_in"], t["W_pred"], t["b_pred"])
    costs = rj.rnnt_joint_loss(enc_p, pred_p, W_out, b_out, i32(inp.labels), i32(inp.T_lens),
                               i32(inp.U_lens), blank=0, tile_t=16, tile_u=8)
    costs.sum().backward()
    for k, name in (("enc_in", "dEnc"), ("W_enc", "dW_enc"), ("b_enc", "db_enc"),
                    ("pred_in", "dPred"), ("W_pred", "dW_pred"), ("b_pred", "db_pred")):
        np.testing.assert_allclose(_np(t[k].grad), g[name], rtol=1e-6, atol=1e-7, err_msg=k)
    np.testing.assert_allclose(_np(W_out.grad), g["dW"], rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_projection_without_bias_and_skipped_outputs(dtype):
    """b = NULL is a projection without bias; dx and db may be skipped."""
    import rnn_joint_transducer_amd as rj
    from synth import _cast
    rng = np.random.default_rng(91)
    M, K, N = 300, 32, 48
    x_s, x64 = _cast(rng.normal(0, 0.5, (M, K)), dtype)
    W_s, W64 = _cast(rng.normal(0, 0.2, (K, N)), dtype)
    dy = rng.normal(0, 1.0, (M, N)).astype(np.float32)
    y = _np(rj.rnnt_joint_proj_fwd(_dev(x_s, dtype), _dev(W_s, dtype), None))
    _check_act("y", y, proj.linear(x64, W64, np.zeros(N)), dtype)
    dx, dW, db = rj.rnnt_joint_proj_bwd(_dev(x_s, dtype), _dev(W_s, dtype), _dev(dy, "fp32"),
                                        need_dx=False, need_db=False)
    assert dx is None and db is None
    _, rdW, _ = proj.linear_grads(x64, W64, dy.astype(np.float64))
    assert float(np.max(np.abs(_np(dW) - rdW))) <= FP32_GRAD_ABS


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_projection_gradients_deterministic_mode(dtype):
    """Deterministic mode: the row splits of the projection gradients run
    one after another, so three runs are bitwise equal, and still match
    float64 to the same bound."""
    import rnn_joint_transducer_amd as rj
    from rnn_joint_transducer_amd import _lib
    from synth import _cast
    rng = np.random.default_rng(93)
    M, K, N = 16 * 101, 640, 640
    x_s, x64 = _cast(rng.normal(0, 0.5, (M, K)), dtype)
    W_s, W64 = _cast(rng.normal(0, 1 / np.sqrt(K), (K, N)), dtype)
    dy = rng.normal(0, 1.0, (M, N)).astype(np.float32)
    old = _lib.get_flags()
    try:
        _lib.set_flags(_lib.FLAG_DETERMINISTIC)
        print(f"[proj deterministic {dtype}]", flush=True)
        runs = [[_np(t) for t in rj.rnnt_joint_proj_bwd(_dev(x_s, dtype), _dev(W_s, dtype),
                                                        _dev(dy, "fp32"))] for _ in range(3)]
    finally:
        _lib.set_flags(old)
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert np.array_equal(a, b)
    rdx, rdW, rdb = proj.linear_grads(x64, W64, dy.astype(np.float64))
    for name, gv, rv in zip(("dx", "dW", "db"), runs[0], (rdx, rdW, rdb)):
        err = float(np.max(np.abs(gv - rv)))
        assert err <= FP32_GRAD_ABS * max(1.0, float(np.max(np.abs(rv))) / 100), (name, err)
