"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Small workloads are compared element by element on every output; the large
workloads (at their full sizes and in the tiling the benchmark uses) are
compared on sampled utterances the oracle computes one by one, on a
two-utterance sub-batch for the weight gradients, and on closed forms that
hold at any size.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import rnnt
from synth import make_config, make_inputs

from gpu_common import BF16_REL, check_costs, check_grad, oracle_costs, run_gpu, to_device

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _oracle_full(inp, grad_costs=None, criterion="sum"):
    return oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                                 inp.T_lens, inp.U_lens, inp.blank, grad_costs=grad_costs,
                                 workers=min(WORKERS, inp.B), criterion=criterion)


def _compare_all(inp, g, ref):
    check_costs(g["costs"], ref["costs"], inp.dtype)
    check_grad("d_enc", g["dEnc"], ref["dEnc"], inp.dtype)
    check_grad("d_pred", g["dPred"], ref["dPred"], inp.dtype)
    check_grad("d_W_out", g["dW"], ref["dW"], inp.dtype)
    check_grad("d_b_out", g["db"], ref["db"], inp.dtype)


# ------------------------------------------------------------------ small, every output

@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0), (0, 8, 128)])
def test_tiny(tiles):
    inp = make_config("tiny")
    print(f"[tiny tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles)
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp))


@pytest.mark.parametrize("tiles", [(0, 0, 0), (64, 64, 128), (16, 8, 0)])
def test_short(tiles):
    inp = make_config("short")
    print(f"[short tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles)
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_ragged_edges(dtype):
    """T not a multiple of 16, U+1 not a multiple of 8, V not a multiple of
    128, a one-frame utterance, an utterance without labels, H = 48."""
    inp = make_inputs(5, 37, 11, 48, 40, dtype=dtype, sigma=0.4, seed=3, t_range=(1, 37),
                      u_range=(0, 11))
    inp.T_lens[:] = [37, 1, 20, 5, 33]
    inp.U_lens[:] = [11, 4, 0, 11, 7]
    ref = _oracle_full(inp, grad_costs=[1.0, 0.5, 2.0, -1.0, 0.0])
    for tiles in [(0, 0, 0), (16, 8, 0), (32, 16, 0)]:
        print(f"[ragged {dtype} tiles={tiles}]", flush=True)
        g = run_gpu(inp, *tiles, grad_costs=[1.0, 0.5, 2.0, -1.0, 0.0])
        _compare_all(inp, g, ref)
        # gradients past each utterance's lengths are exactly zero
        for b in range(inp.B):
            assert np.all(g["dEnc"][b, inp.T_lens[b]:] == 0)
            assert np.all(g["dPred"][b, inp.U_lens[b] + 1:] == 0)


@pytest.mark.parametrize("dtype,H,V,sigma", [
    ("bf16", 128, 256, 0.05),  # exact shape, every |z| provably below 64
    ("bf16", 128, 256, 1.5),   # exact shape, bound above 64: running maxima
    ("bf16", 64, 200, 2.0),    # partial vocabulary step, running maxima
    ("fp32", 64, 200, 2.0),
])
def test_small_hidden_and_logit_bound(dtype, H, V, sigma):
    """Hidden sizes up to 256 in bf16 (the 64-column vocabulary step with
    two workgroups per compute unit), with the max-free log-sum-exp and, when
    sum_k |W_kv| + |b_v| reaches 64, the one with running maxima.  The large
    weights give logits |z| ~ 30: untiled bf16 stores them relative to each
    row's largest logit of the vocabulary step, which keeps the storage error
    of every softmax entry below 2^-8 / e whatever |z| is (stored as plain
    bf16 they would carry |z| 2^-8 ~ 0.1 into exp(z - lse))."""
    inp = make_inputs(3, 29, 9, H, V, dtype=dtype, sigma=sigma, seed=53, t_range=(5, 29),
                      u_range=(0, 9))
    ref = _oracle_full(inp, grad_costs=[1.0, -0.5, 0.25])
    for tiles in [(0, 0, 0), (16, 8, 0), (0, 8, 128)]:
        print(f"[small hidden {dtype} H={H} V={V} sigma={sigma} tiles={tiles}]", flush=True)
        g = run_gpu(inp, *tiles, grad_costs=[1.0, -0.5, 0.25])
        assert g["status"] == 0
        _compare_all(inp, g, ref)


@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_bf16_wide_hidden_partial_tiles(tiles):
    """H = 640 (the widest hidden size whose h rows are staged in LDS) with
    label counts that leave the last 8-wide label tile of every utterance
    partly outside the lattice: the logit / gradient store path of partly
    valid tiles, element by element."""
    inp = make_inputs(3, 40, 13, 640, 256, dtype="bf16", sigma=0.05, seed=11, t_range=(17, 40),
                      u_range=(3, 13))
    inp.U_lens[:] = [13, 9, 4]
    print(f"[bf16 H=640 tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles)
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp))


@pytest.mark.parametrize("H,V,big", [
    (272, 200, False),  # two 256-wide parts of h, one live k-step in the second
    (512, 256, False),  # two whole parts, exact shape
    (640, 200, False),  # three parts, the last half used
    (768, 256, False),  # three whole parts, exact shape (the largest hidden size)
    (640, 200, True),   # one |enc| > 40: h evaluated from the inputs, part by part
])
def test_fp32_wide_hidden(H, V, big):
    """fp32 above 256 hidden: h is held in registers 256 hidden at a time and
    each part is rebuilt when a vocabulary step reaches it.  Untiled, tiled,
    and tiled in vocabulary parts (the later parts read the first part's
    stored h rows back); every output against the oracle."""
    inp = make_inputs(3, 40, 13, H, V, dtype="fp32", sigma=0.05, seed=13, t_range=(17, 40),
                      u_range=(3, 13))
    inp.U_lens[:] = [13, 9, 4]
    if big:
        inp.enc[1, 2, 5] = 45.0
        inp.enc_f64[1, 2, 5] = 45.0
    gcs = [1.0, -0.5, 2.0]
    ref = _oracle_full(inp, grad_costs=gcs)
    for tiles in [(0, 0, 0), (16, 8, 0), (16, 8, 128)]:
        print(f"[fp32 wide hidden H={H} V={V} big={big} tiles={tiles}]", flush=True)
        g = run_gpu(inp, *tiles, grad_costs=gcs)
        assert g["status"] == 0
        _compare_all(inp, g, ref)


def test_data_errors_flagged():
    inp = make_inputs(4, 12, 5, 32, 24, sigma=0.4, seed=5, t_range=(4, 12), u_range=(1, 5))
    good = make_inputs(4, 12, 5, 32, 24, sigma=0.4, seed=5, t_range=(4, 12), u_range=(1, 5))
    inp.labels[1, 0] = 0          # a label equal to blank
    inp.T_lens[2] = 13            # T' > T
    g = run_gpu(inp)
    assert g["status"] == 3
    assert math.isnan(g["costs"][1]) and math.isnan(g["costs"][2])
    assert np.all(g["dEnc"][1] == 0) and np.all(g["dEnc"][2] == 0)
    assert np.all(g["dPred"][1] == 0) and np.all(g["dPred"][2] == 0)
    # the valid utterances are untouched by their invalid neighbours
    sub = [0, 3]
    ref = oracle.loss_and_grads(good.enc_f64[sub], good.pred_f64[sub], good.W_f64, good.b_f64,
                                good.labels[sub], good.T_lens[sub], good.U_lens[sub], 0)
    check_costs(g["costs"], ref["costs"], "fp32", idx=sub)
    check_grad("d_enc", g["dEnc"][sub], ref["dEnc"], "fp32")
    check_grad("d_W_out", g["dW"], ref["dW"], "fp32")


@pytest.mark.parametrize("criterion", ["sum", "max"])
@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_nan_input_stays_in_its_utterance(criterion, tiles):
    """A NaN in one utterance's encodings makes that utterance's cost NaN and
    leaves every other cost and encoder / prediction gradient as the oracle
    computes it without that utterance: the lattice carries NaN through its
    log-add-exp (or max) steps but never into another utterance, and no
    finite cell of the NaN utterance turns a neighbour's result into a
    sentinel or -inf."""
    inp = make_inputs(4, 24, 6, 32, 40, sigma=0.4, seed=23, t_range=(10, 24), u_range=(2, 6))
    inp.enc[1, 3, 5] = np.nan
    print(f"[nan input {criterion} tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles, criterion=criterion)
    assert g["status"] == 0
    assert math.isnan(g["costs"][1])
    sub = [0, 2, 3]
    ref = oracle.loss_and_grads(inp.enc_f64[sub], inp.pred_f64[sub], inp.W_f64, inp.b_f64,
                                inp.labels[sub], inp.T_lens[sub], inp.U_lens[sub], 0,
                                criterion=criterion)
    check_costs(g["costs"], ref["costs"], "fp32", idx=sub)
    check_grad("d_enc", g["dEnc"][sub], ref["dEnc"], "fp32")
    check_grad("d_pred", g["dPred"][sub], ref["dPred"], "fp32")


@pytest.mark.parametrize("criterion", ["sum", "max"])
@pytest.mark.parametrize("U1", [64, 65, 129, 192, 193, 256, 320, 321, 385, 448, 449, 512, 513,
                                577, 640, 705, 768, 833, 896, 961, 1024])
def test_lattice_label_blocking(U1, criterion):
    """Every label-position blocking of the lattice sweep (1 to 16 positions
    per lane, each with its own chunk length), at and just past each block
    boundary, with label counts up to the padded maximum: every output
    against the oracle."""
    U = U1 - 1
    inp = make_inputs(2, 12, U, 32, 64, sigma=0.3, seed=U1, t_range=(5, 12),
                      u_range=(max(0, U - 70), U))
    inp.U_lens[0] = U
    print(f"[lattice blocking U+1={U1} {criterion} U'={list(inp.U_lens)}]", flush=True)
    g = run_gpu(inp, criterion=criterion)
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, criterion=criterion))


def test_tile_invariance_short():
    inp = make_config("short")
    base = run_gpu(inp, 0, 0, 0)
    for tiles in [(32, 16, 0), (0, 24, 0), (208, 56, 128)]:
        g = run_gpu(inp, *tiles)
        np.testing.assert_allclose(g["costs"], base["costs"], rtol=2e-6)
        for k in ("dEnc", "dPred", "dW", "db"):
            # float32 atomics sum in a different order per tiling
            np.testing.assert_allclose(g[k], base[k], atol=2e-5, rtol=1e-4)


def test_autograd_wrapper():
    import torch
    import rnn_joint_transducer_amd as rj
    inp = make_config("tiny")
    dev = to_device(inp)
    for k in ("enc", "pred", "W_out", "b_out"):
        dev[k].requires_grad_(True)
    costs = rj.rnnt_joint_loss(**dev, tile_t=16, tile_u=8)
    (costs * torch.tensor([1.0, 3.0], device=costs.device)).sum().backward()
    ref = _oracle_full(inp, grad_costs=[1.0, 3.0])
    check_grad("d_enc", dev["enc"].grad.double().cpu().numpy(), ref["dEnc"], "fp32")
    check_grad("d_W_out", dev["W_out"].grad.double().cpu().numpy(), ref["dW"], "fp32")


def _grad_leaves(tiles, grad_costs):
    import torch
    import rnn_joint_transducer_amd as rj
    inp = make_config("tiny")
    dev = to_device(inp)
    for k in ("enc", "pred", "W_out", "b_out"):
        dev[k].requires_grad_(True)
    costs = rj.rnnt_joint_loss(**dev, tile_t=tiles[0], tile_u=tiles[1], tile_v=tiles[2])
    loss = (costs * torch.tensor(grad_costs, device=costs.device)).sum()
    return inp, dev, loss


def test_saved_state_reused_tiled():
    """Tiled mode: the backward only reads the forward's saved state, so a
    second backward from the same forward (retain_graph) gives the same
    gradients; a negative cost gradient exercises the sign handling."""
    inp, dev, loss = _grad_leaves((16, 8, 0), [2.0, -0.5])
    keys = ("enc", "pred", "W_out", "b_out")
    loss.backward(retain_graph=True)
    first = [dev[k].grad.clone() for k in keys]
    for k in keys:
        dev[k].grad = None
    loss.backward()
    ref = _oracle_full(inp, grad_costs=[2.0, -0.5])
    check_grad("d_enc", first[0].double().cpu().numpy(), ref["dEnc"], "fp32")
    check_grad("d_W_out", first[2].double().cpu().numpy(), ref["dW"], "fp32")
    check_grad("d_b_out", first[3].double().cpu().numpy(), ref["db"], "fp32")
    for k, a in zip(keys, first):
        # float32 atomics may add in another order
        np.testing.assert_allclose(dev[k].grad.cpu().numpy(), a.cpu().numpy(), atol=1e-6, rtol=1e-5)


def test_untiled_state_consumed_once():
    """Untiled mode: the backward turns the stored logits into gradients in
    place.  Its gradients are right (negative cost gradient included); the
    autograd wrapper refuses a second backward, and a second call through the
    C ABI is reported by the status word (bit 4)."""
    import rnn_joint_transducer_amd as rj
    inp, dev, loss = _grad_leaves((0, 0, 0), [2.0, -0.5])
    loss.backward(retain_graph=True)
    ref = _oracle_full(inp, grad_costs=[2.0, -0.5])
    check_grad("d_enc", dev["enc"].grad.double().cpu().numpy(), ref["dEnc"], "fp32")
    check_grad("d_pred", dev["pred"].grad.double().cpu().numpy(), ref["dPred"], "fp32")
    check_grad("d_W_out", dev["W_out"].grad.double().cpu().numpy(), ref["dW"], "fp32")
    check_grad("d_b_out", dev["b_out"].grad.double().cpu().numpy(), ref["db"], "fp32")
    with pytest.raises(RuntimeError, match="once per forward"):
        loss.backward()
    d = to_device(inp)
    costs, saved = rj.rnnt_joint_loss_fwd(**d)
    rj.rnnt_joint_loss_bwd(**d, saved=saved)
    assert rj.rnnt_joint_loss_status(saved) == 0
    rj.rnnt_joint_loss_bwd(**d, saved=saved)
    assert rj.rnnt_joint_loss_status(saved) == 4
    # a new forward into the same buffer starts clean
    rj.rnnt_joint_loss_fwd(**d, costs=costs, saved=saved)
    g = rj.rnnt_joint_loss_bwd(**d, saved=saved)
    assert rj.rnnt_joint_loss_status(saved) == 0
    check_grad("d_W_out", g[2].double().cpu().numpy(), _oracle_full(inp)["dW"], "fp32")


# ------------------------------------------------------------------ full-size workloads

_COST_CACHE = {}


def _sampled(inp, tiles, cost_utts, grad_utts, key=None):
    """Costs of `cost_utts` and the encoder / prediction gradients of
    `grad_utts` against the oracle; with `key`, the oracle costs of a
    workload are computed once for all the tilings that check them."""
    g = run_gpu(inp, *tiles)
    assert g["status"] == 0
    ck = (key, tuple(cost_utts))
    if key is None or ck not in _COST_CACHE:
        _COST_CACHE[ck] = oracle_costs(inp, cost_utts, WORKERS)
    refc = _COST_CACHE[ck]
    worst = check_costs(g["costs"], refc, inp.dtype, idx=cost_utts)
    print(f"  costs of {len(cost_utts)} utterances: worst rel err {worst:.2e}", flush=True)
    for b in grad_utts:
        o = rnnt.utterance_loss_and_grads(inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64,
                                          inp.labels[b], int(inp.T_lens[b]),
                                          int(inp.U_lens[b]), 0)
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
        check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)
    return g


def _sub_batch_weights(inp, tiles, utts):
    """Weight gradients of a two-utterance sub-batch at the full H, V, T, U."""
    from synth import Inputs
    import dataclasses
    sub = dataclasses.replace(
        inp, B=len(utts), enc=inp.enc[utts], pred=inp.pred[utts], labels=inp.labels[utts],
        T_lens=inp.T_lens[utts], U_lens=inp.U_lens[utts], enc_f64=inp.enc_f64[utts],
        pred_f64=inp.pred_f64[utts])
    g = run_gpu(sub, *tiles)
    ref = _oracle_full(sub)
    check_costs(g["costs"], ref["costs"], inp.dtype)
    check_grad("d_W_out(sub)", g["dW"], ref["dW"], inp.dtype)
    check_grad("d_b_out(sub)", g["db"], ref["db"], inp.dtype)


@pytest.mark.parametrize("tiles", [(64, 0, 0), (128, 0, 0), (64, 64, 0), (0, 0, 0),
                                   (128, 0, 256)])
def test_medium(tiles):
    """Every cost of the batch, the gradients of one utterance, and the weight
    gradients of a two-utterance sub-batch at the full sizes; (64, 0, 0) is
    the tiling the benchmark times."""
    inp = make_config("medium")
    print(f"[medium tiles={tiles}]", flush=True)
    _sampled(inp, tiles, cost_utts=list(range(inp.B)), grad_utts=[7], key="medium")
    _sub_batch_weights(inp, tiles, [3, 11])


@pytest.mark.parametrize("tiles", [(0, 64, 256), (0, 128, 256), (64, 64, 256), (32, 0, 256)])
def test_medium_large_vocab(tiles):
    """(0, 64, 256) -- chunks of all frames x 64 label positions, vocabulary
    parts of 256 columns -- is the tiling the benchmark times."""
    inp = make_config("medium_lv")
    print(f"[medium_lv tiles={tiles}]", flush=True)
    _sampled(inp, tiles, cost_utts=list(range(inp.B)), grad_utts=[9], key="medium_lv")
    _sub_batch_weights(inp, tiles, [5, 13])


# The long workload in the tiling the benchmark times (64 x 64 chunks, the
# whole vocabulary per chunk), split into three tests so that each one's
# oracle work stays around a minute on the host cores; the costs are also
# checked with the vocabulary split into 256-column parts.
LONG_TILES = (64, 64, 0)


@pytest.mark.parametrize("tiles", [LONG_TILES, (64, 64, 256)])
def test_long_tiled_costs(tiles):
    """Every utterance's cost."""
    inp = make_config("long")
    print(f"[long costs tiles={tiles}]", flush=True)
    _sampled(inp, tiles, cost_utts=list(range(inp.B)), grad_utts=[], key="long")


def test_long_tiled_largest_utterance_grads():
    """d_enc and d_pred of the utterance with the most lattice cells (its
    lattice reaches into the last frame and label chunks), from the whole
    batch's backward."""
    inp = make_config("long")
    b = int(np.argmax(inp.T_lens.astype(np.int64) * (inp.U_lens + 1)))
    print(f"[long grads utt {b}: T'={inp.T_lens[b]} U'={inp.U_lens[b]} tiles={LONG_TILES}]",
          flush=True)
    _sampled(inp, LONG_TILES, cost_utts=[b], grad_utts=[b])


def test_long_tiled_sub_batch_weights():
    """d_W_out and d_b_out of a two-utterance sub-batch at the full H, V, T, U."""
    inp = make_config("long")
    cells = inp.T_lens.astype(np.int64) * (inp.U_lens + 1)
    utts = [int(i) for i in np.argsort(cells)[:2]]
    print(f"[long sub-batch {utts} tiles={LONG_TILES}]", flush=True)
    _sub_batch_weights(inp, LONG_TILES, utts)


@pytest.mark.parametrize("name", ["medium", "long"])
def test_zero_weights_closed_form_full_size(name):
    """W_out = 0 at full size: cost = (T'+U') log V - log C(T'+U'-1, U'),
    d_enc = d_pred = 0, d_b_out from label counts."""
    inp = make_config(name)
    inp.W = np.zeros_like(inp.W)
    g = run_gpu(inp, *((64, 64, 128) if name == "long" else (0, 0, 0)))
    V = inp.V
    want = np.array([(Tl + Ul) * math.log(V) - math.log(math.comb(Tl + Ul - 1, Ul))
                     for Tl, Ul in zip(inp.T_lens.tolist(), inp.U_lens.tolist())])
    np.testing.assert_allclose(g["costs"], want, rtol=1e-5)
    assert np.all(g["dEnc"] == 0) and np.all(g["dPred"] == 0)
    want_db = np.zeros(V)
    for b in range(inp.B):
        Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
        want_db += (Tl + Ul) / V
        want_db[0] -= Tl
        np.add.at(want_db, inp.labels[b, :Ul], -1.0)
    np.testing.assert_allclose(g["db"], want_db, atol=2e-2 * np.abs(want_db).max())
    assert abs(g["db"].sum()) <= 1e-3 * np.abs(want_db).max()


# ------------------------------------------------------------------ maximum approximation
#
# The best-alignment criterion against the oracle's maximum-approximation
# mode.  The inputs are continuous random draws, so the best alignment is
# unique and both sides read back the same one.

@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_max_tiny(tiles):
    inp = make_config("tiny")
    print(f"[max tiny tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles, grad_costs=[1.0, -0.5], criterion="max")
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, grad_costs=[1.0, -0.5], criterion="max"))


@pytest.mark.parametrize("tiles", [(0, 0, 0), (64, 64, 128)])
def test_max_short(tiles):
    inp = make_config("short")
    print(f"[max short tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles, criterion="max")
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, criterion="max"))


def test_max_ragged_bf16():
    inp = make_inputs(5, 37, 11, 64, 96, sigma=0.2, seed=31, dtype="bf16",
                      t_range=(1, 37), u_range=(0, 11))
    print("[max ragged bf16]", flush=True)
    g = run_gpu(inp, 16, 8, 0, criterion="max")
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, criterion="max"))


def test_max_long_paths_chunked():
    """Best-alignment read-back over more frames than its packed decision bits
    hold at once: with U'+1 = 401 rows the bits cover 640 frames, so T' = 1500
    is read in three chunks of t; U' = 300 in two, U' = 137 in one, U' = 0 is
    a single row.  Every output is compared.  With unit upstream gradients
    these 1500-frame paths give |d_pred| up to ~380 and |d_b_out| ~4300, where
    an fp32 value cannot hold a 1e-4 absolute error (half an ulp at 4300 is
    2.4e-4); upstream gradients of at most 0.3 keep every entry below ~1300,
    while a single wrong step on a path would still move d_enc by ~1e-2."""
    inp = make_inputs(4, 1500, 400, 64, 32, sigma=0.1, seed=47, dtype="fp32")
    inp.T_lens = np.array([1500, 1500, 1201, 300], dtype=np.int32)
    inp.U_lens = np.array([400, 300, 137, 0], dtype=np.int32)
    gcs = [0.25, -0.2, 0.25, 0.3]
    print("[max long paths chunked]", flush=True)
    g = run_gpu(inp, 0, 0, 0, grad_costs=gcs, criterion="max")
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, grad_costs=gcs, criterion="max"))


@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_max_exact_ties_follow_blank_first(tiles):
    """W_out = 0 and b_out = 0: every alignment has exactly the same score, so
    the best one is decided by the tie rule alone (the blank predecessor wins).
    d_enc and d_pred vanish, but d_W_out = sum over the path of h (x) dz does
    depend on which cells the path visits."""
    inp = make_config("short")
    inp.W = np.zeros_like(inp.W)
    inp.W_f64 = np.zeros_like(inp.W_f64)
    print(f"[max exact ties tiles={tiles}]", flush=True)
    g = run_gpu(inp, *tiles, criterion="max")
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp, criterion="max"))


def test_max_medium_sampled():
    inp = make_config("medium")
    print("[max medium sampled]", flush=True)
    g = run_gpu(inp, 64, 64, 0, criterion="max")
    assert g["status"] == 0
    utts = [4, 12]
    refc = rnnt.loss_only(inp.enc_f64[utts], inp.pred_f64[utts], inp.W_f64, inp.b_f64,
                          inp.labels[utts], inp.T_lens[utts], inp.U_lens[utts], 0,
                          criterion="max")
    check_costs(g["costs"], refc, inp.dtype, idx=utts)
    b = 12
    o = rnnt.utterance_loss_and_grads(inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64,
                                      inp.labels[b], int(inp.T_lens[b]), int(inp.U_lens[b]),
                                      0, criterion="max")
    Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
    check_grad(f"d_enc[{b}]", g["dEnc"][b, :Tl], o["dEnc"], inp.dtype)
    check_grad(f"d_pred[{b}]", g["dPred"][b, :Ul + 1], o["dPred"], inp.dtype)


def test_max_zero_weights_closed_form_medium():
    """W_out = 0: every alignment has the same probability, so the best one's
    cost is -(T' log p_blank + sum_u log p_{y_u}) whatever the tie order."""
    inp = make_config("medium")
    inp.W = np.zeros_like(inp.W)
    g = run_gpu(inp, 64, 64, 0, bwd=False, criterion="max")
    assert g["status"] == 0
    want = [oracle.closed_form_zero_weights_max(int(inp.T_lens[b]), int(inp.U_lens[b]),
                                                inp.labels[b], inp.b_f64, inp.blank)
            for b in range(inp.B)]
    check_costs(g["costs"], want, inp.dtype)


# ------------------------------------------------------------------ maximum sizes

@pytest.mark.parametrize("case", ["U_max", "V_max", "H_max_bf16", "B_max", "T_max",
                                  "wide_rows"])
def test_maximum_sizes(case):
    """Each size limit the library accepts, with the other sizes small enough
    for the oracle: U + 1 = 1024 (both criteria), V = 262144, H = 768 in bf16,
    B = 8191, T = 65520.  Every output is compared.  "wide_rows" pairs
    U + 1 = 1024 with V = 131072 (fp32): the logit rows of one 16-frame tile
    then span 8 GiB, beyond the 32-bit per-lane offsets of dh's usual copy
    form, so dh takes its general address form (untiled, and tiled with every
    label position in one chunk).  The largest-B and
    longest-T cases weight their costs by 1e-3 and 1e-4: unweighted, d_b_out
    sums to ~1.1e4 over 8191 utterances (half an fp32 ulp there is 4.9e-4)
    and d_W_out to ~40 over 65520 frames, beyond what an fp32 value can hold
    to the 1e-4 absolute bound.  Weighted, the gradients are small enough
    that the absolute bound alone would also accept zeros, so those cases
    also compare every gradient relative to its largest oracle entry: fp32
    sums of up to 65520 terms keep that within 1e-4."""
    gcs = None
    runs = [((0, 0, 0), "sum"), ((16, 8, 0), "sum")]
    if case == "U_max":
        inp = make_inputs(2, 24, 1023, 64, 40, sigma=0.2, seed=101)
        inp.U_lens = np.array([1023, 600], dtype=np.int32)
        runs += [((0, 0, 0), "max"), ((64, 64, 128), "max")]
    elif case == "V_max":
        inp = make_inputs(2, 5, 2, 32, 262144, sigma=0.2, seed=102)
    elif case == "H_max_bf16":
        inp = make_inputs(2, 20, 6, 768, 96, dtype="bf16", sigma=0.05, seed=103)
    elif case == "wide_rows":
        inp = make_inputs(1, 2, 1023, 16, 131072, sigma=0.2, seed=106)
        runs = [((0, 0, 0), "sum"), ((16, 0, 0), "sum")]
    elif case == "B_max":
        inp = make_inputs(8191, 2, 1, 16, 16, sigma=0.3, seed=104, t_range=(1, 2), u_range=(0, 1))
        gcs = [1e-3] * inp.B
    else:
        inp = make_inputs(1, 65520, 0, 16, 8, sigma=0.3, seed=105)
        gcs = [1e-4]
    refs = {}
    for tiles, crit in runs:
        print(f"[maximum size {case} tiles={tiles} criterion={crit}]", flush=True)
        g = run_gpu(inp, *tiles, grad_costs=gcs, criterion=crit)
        assert g["status"] == 0
        if crit not in refs:
            refs[crit] = _oracle_full(inp, grad_costs=gcs, criterion=crit)
        _compare_all(inp, g, refs[crit])
        if gcs is not None:
            for k in ("dEnc", "dPred", "dW", "db"):
                scale = float(np.max(np.abs(refs[crit][k])))
                rel = float(np.max(np.abs(g[k] - refs[crit][k]))) / scale
                print(f"  {k}: max|ref| {scale:.3e}, rel err {rel:.2e}", flush=True)
                assert scale > 0 and rel <= 1e-4, (k, scale, rel)


# ------------------------------------------------------------------ state / backward mismatch

def test_backward_checks_the_state_it_is_given():
    """A backward checks that `saved` comes from a forward with its sizes,
    dtype and blank, and (untiled) one that stored the logits.  On a mismatch
    it computes nothing: gradients zero, data-error bit 8.  The buffers here
    are sized for the larger (untiled) layout, so nothing could be read out of
    bounds even without the check.  An untiled forward's state carries all a
    tiled backward needs, which is accepted and exact."""
    import torch
    import rnn_joint_transducer_amd as rj
    inp = make_config("tiny")
    d = to_device(inp)
    B, T, U, H, V = inp.B, inp.T, inp.U, inp.H, inp.V
    nbytes = rj.rnnt_joint_loss_saved_bytes(B, T, U, H, V, rj.RNNTJ_F32, 0, 0, 0)
    ref = _oracle_full(inp)
    # untiled backward from a tiled forward's state
    saved = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rj.rnnt_joint_loss_fwd(**d, tile_t=16, tile_u=8, saved=saved)
    g = rj.rnnt_joint_loss_bwd(**d, saved=saved)
    assert rj.rnnt_joint_loss_status(saved) == 8
    assert all(float(x.abs().max()) == 0.0 for x in g)
    # a backward with another blank than its forward
    saved = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rj.rnnt_joint_loss_fwd(**d, tile_t=16, tile_u=8, saved=saved)
    g = rj.rnnt_joint_loss_bwd(**d, saved=saved, blank=1, tile_t=16, tile_u=8)
    assert rj.rnnt_joint_loss_status(saved) == 8
    assert all(float(x.abs().max()) == 0.0 for x in g)
    # a tiled backward from the untiled forward's state: accepted and exact
    costs, saved = rj.rnnt_joint_loss_fwd(**d)
    g = rj.rnnt_joint_loss_bwd(**d, saved=saved, tile_t=16, tile_u=8)
    assert rj.rnnt_joint_loss_status(saved) == 0
    for name, x, k in zip(("d_enc", "d_pred", "d_W_out", "d_b_out"), g,
                          ("dEnc", "dPred", "dW", "db")):
        check_grad(name, x.double().cpu().numpy(), ref[k], "fp32")
    # the binding refuses a state buffer smaller than the backward's layout
    _, small = rj.rnnt_joint_loss_fwd(**d, tile_t=16, tile_u=8)
    with pytest.raises(ValueError, match="saved"):
        rj.rnnt_joint_loss_bwd(**d, saved=small)


# ------------------------------------------------------------------ vocabulary parts

@pytest.mark.parametrize("tile_v", [128, 256, 384])
def test_vocabulary_parts_short(tile_v):
    """The tiled backward in vocabulary parts of tile_v columns (V = 512: four,
    two, or a part of 384 and one of 128): every output against the oracle."""
    inp = make_config("short")
    print(f"[vocabulary parts short tiles=(64, 64, {tile_v})]", flush=True)
    g = run_gpu(inp, 64, 64, tile_v)
    assert g["status"] == 0
    _compare_all(inp, g, _oracle_full(inp))


@pytest.mark.parametrize("dtype,H", [("fp32", 48), ("bf16", 64), ("bf16", 640)])
def test_vocabulary_parts_ragged(dtype, H):
    """V = 200 in parts of 128 (a last part of 72 columns, not a multiple of
    any kernel's vocabulary step), ragged lengths and signed cost weights;
    H = 64 bf16 uses the 64-column joint step, H = 640 the 128-column one."""
    inp = make_inputs(4, 37, 11, H, 200, dtype=dtype, sigma=0.3, seed=71, t_range=(1, 37),
                      u_range=(0, 11))
    gcs = [1.0, -0.5, 2.0, 0.25]
    ref = _oracle_full(inp, grad_costs=gcs)
    for tiles in [(16, 8, 128), (32, 0, 128)]:
        print(f"[vocabulary parts ragged {dtype} H={H} tiles={tiles}]", flush=True)
        g = run_gpu(inp, *tiles, grad_costs=gcs)
        assert g["status"] == 0
        _compare_all(inp, g, ref)
