"""The library's robustness switches on the GPU: the deterministic mode gives
bitwise identical gradients run after run (and still the oracle's), and the
debug mode turns a data error into RNNTJ_ERR_DATA."""
import numpy as np
import pytest

from synth import make_config, make_inputs

from gpu_common import check_costs, check_grad, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture
def flags():
    from rnn_joint_transducer_amd import _lib
    old = _lib.get_flags()
    yield _lib
    _lib.set_flags(old)


@pytest.mark.parametrize("name,tiles", [("short", (64, 64, 0)), ("short", (0, 0, 0)),
                                        ("short", (64, 64, 128)), ("bf16", (16, 8, 0))])
def test_deterministic_mode_is_bitwise_reproducible(flags, name, tiles):
    import oracle
    if name == "short":
        inp = make_config("short")
    else:
        inp = make_inputs(4, 60, 17, 128, 200, dtype="bf16", sigma=0.3, seed=29,
                          t_range=(20, 60), u_range=(5, 17))
    gcs = list(np.linspace(-1.0, 1.0, inp.B))
    flags.set_flags(flags.FLAG_DETERMINISTIC)
    print(f"[deterministic {name} tiles={tiles}]", flush=True)
    runs = [run_gpu(inp, *tiles, grad_costs=gcs) for _ in range(3)]
    for g in runs[1:]:
        for k in ("costs", "dEnc", "dPred", "dW", "db"):
            assert np.array_equal(g[k], runs[0][k]), k
    ref = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                                inp.T_lens, inp.U_lens, inp.blank, grad_costs=gcs,
                                workers=min(8, inp.B))
    g = runs[0]
    check_costs(g["costs"], ref["costs"], inp.dtype)
    for k, n in (("dEnc", "d_enc"), ("dPred", "d_pred"), ("dW", "d_W_out"), ("db", "d_b_out")):
        check_grad(n, g[k], ref[k], inp.dtype)


def test_debug_mode_reports_data_errors(flags):
    import rnn_joint_transducer_amd as rj
    from gpu_common import to_device
    inp = make_inputs(3, 12, 4, 32, 24, sigma=0.3, seed=9, t_range=(4, 12), u_range=(1, 4))
    flags.set_flags(flags.FLAG_DEBUG)
    g = run_gpu(inp, 16, 8, 0)  # valid input: no error
    assert g["status"] == 0
    inp.labels[1, 0] = 0  # a label equal to blank
    d = to_device(inp)
    with pytest.raises(rj.RNNTJointError) as e:
        rj.rnnt_joint_loss_fwd(**d, tile_t=16, tile_u=8)
    assert e.value.code == 5
    flags.set_flags(0)
    costs, saved = rj.rnnt_joint_loss_fwd(**d, tile_t=16, tile_u=8)  # reported by status only
    assert rj.rnnt_joint_loss_status(saved) == 2
