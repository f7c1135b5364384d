"""The tiled backward's two chunk schedules on the GPU: with the workspace of
pass 1 it alternates two chunk buffer pairs and runs each chunk's dW GEMM on a
side stream; with the least workspace (pass 2) every kernel runs in order on
the caller's stream.  Both must give the oracle's gradients, and in the
deterministic mode the same bits."""
import numpy as np
import pytest

from synth import make_config, make_inputs

from gpu_common import check_costs, check_grad, to_device

pytestmark = pytest.mark.gpu


def _run(inp, tiles, least, grad_costs):
    import torch
    import rnn_joint_transducer_amd as rj
    d = to_device(inp)
    costs, saved = rj.rnnt_joint_loss_fwd(**d, blank=inp.blank, tile_t=tiles[0],
                                          tile_u=tiles[1], tile_v=tiles[2])
    B, T, U = inp.B, inp.enc.shape[1], inp.labels.shape[1]
    H, V = inp.W.shape
    dc = rj.RNNTJ_F32 if inp.dtype == "fp32" else rj.RNNTJ_BF16
    nb = rj.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, *tiles, 2 if least else 1)
    ws = torch.empty(nb, dtype=torch.uint8, device=costs.device)
    gc = torch.tensor(grad_costs, dtype=torch.float32, device=costs.device)
    g = rj.rnnt_joint_loss_bwd(**d, saved=saved, blank=inp.blank, tile_t=tiles[0],
                               tile_u=tiles[1], tile_v=tiles[2], grad_costs=gc, workspace=ws)
    assert rj.rnnt_joint_loss_status(saved) == 0
    out = dict(costs=costs, dEnc=g[0], dPred=g[1], dW=g[2], db=g[3])
    return {k: v.cpu().double().numpy() for k, v in out.items()}


CASES = [
    ("short", (64, 64, 0)),     # 4 chunks, whole vocabulary
    ("short", (64, 64, 128)),   # 4 chunks x 4 vocabulary parts
    ("short", (16, 16, 256)),   # 52 chunks x 2 parts
    ("bf16", (16, 8, 0)),       # ragged bf16, many small chunks
    ("bf16", (32, 16, 128)),    # ragged bf16, vocabulary parts of 128 and 72
]


def _inputs(name):
    if name == "short":
        return make_config("short")
    return make_inputs(4, 60, 17, 128, 200, dtype="bf16", sigma=0.3, seed=29,
                       t_range=(20, 60), u_range=(5, 17))


@pytest.mark.parametrize("name,tiles", CASES)
def test_overlapped_and_serial_schedules_match_the_oracle(name, tiles):
    import oracle
    inp = _inputs(name)
    gcs = list(np.linspace(-1.0, 1.0, inp.B))
    print(f"[schedule {name} tiles={tiles}]", flush=True)
    ref = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                                inp.T_lens, inp.U_lens, inp.blank, grad_costs=gcs,
                                workers=min(8, inp.B))
    for least in (False, True):
        g = _run(inp, tiles, least, gcs)
        check_costs(g["costs"], ref["costs"], inp.dtype)
        for k, n in (("dEnc", "d_enc"), ("dPred", "d_pred"), ("dW", "d_W_out"),
                     ("db", "d_b_out")):
            check_grad(n, g[k], ref[k], inp.dtype)


@pytest.mark.parametrize("name,tiles", [("short", (64, 64, 128)), ("bf16", (16, 8, 0))])
def test_schedules_agree_bitwise_in_deterministic_mode(name, tiles):
    from rnn_joint_transducer_amd import _lib
    inp = _inputs(name)
    gcs = list(np.linspace(-1.0, 1.0, inp.B))
    old = _lib.get_flags()
    try:
        _lib.set_flags(_lib.FLAG_DETERMINISTIC)
        print(f"[schedule deterministic {name} tiles={tiles}]", flush=True)
        a = _run(inp, tiles, False, gcs)
        b = _run(inp, tiles, True, gcs)
        c = _run(inp, tiles, False, gcs)
    finally:
        _lib.set_flags(old)
    for k in ("costs", "dEnc", "dPred", "dW", "db"):
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k


def test_two_threads_on_two_streams():
    """Two host threads run tiled forward + backward calls at once, each on a
    stream of its own; the library's side stream and its events are shared
    per device.  Each thread's gradients must match those of the same call run
    alone, to the parity bar of its dtype."""
    import threading

    import torch
    inps = [make_config("short"),
            make_inputs(4, 60, 17, 128, 200, dtype="bf16", sigma=0.3, seed=29,
                        t_range=(20, 60), u_range=(5, 17))]
    tiles = [(16, 16, 256), (16, 8, 0)]
    alone = [_run(inp, t, False, [1.0] * inp.B) for inp, t in zip(inps, tiles)]
    results = [None, None]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [_run(inps[i], tiles[i], False, [1.0] * inps[i].B) for _ in range(3)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below, in the test's own thread
            errors.append(repr(e))

    print("[schedule two threads]", flush=True)
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for i, inp in enumerate(inps):
        for g in results[i]:
            check_costs(g["costs"], alone[i]["costs"], inp.dtype)
            for k in ("dEnc", "dPred", "dW", "db"):
                check_grad(k, g[k], alone[i][k], inp.dtype)
