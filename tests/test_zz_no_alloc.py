"""The no-allocation backward (rnnt_joint_loss_bwd_noalloc, static per-GPU
scratch instead of a workspace) against rnnt_joint_loss_bwd, both called
through the C ABI: two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), in the untiled and tiled modes."""
import ctypes

import numpy as np
import pytest

from synth import make_config, make_inputs

from gpu_common import check_grad, to_device

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(inp, tiles, gcs=None):
    """(workspace backward, no-allocation backward) outputs from two copies of
    one forward's state (an untiled backward consumes its state)."""
    import torch
    import rnn_joint_transducer_amd as rj
    from rnn_joint_transducer_amd import _lib
    lib = _lib.load()
    d = to_device(inp)
    B, T, U, H, V = inp.B, inp.T, inp.U, inp.H, inp.V
    dc = rj.RNNTJ_BF16 if inp.dtype == "bf16" else rj.RNNTJ_F32
    _, saved = rj.rnnt_joint_loss_fwd(**d, blank=inp.blank, tile_t=tiles[0], tile_u=tiles[1],
                                      tile_v=tiles[2])
    saved2 = saved.clone()
    gc = None if gcs is None else torch.tensor(gcs, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for k, st in enumerate((saved, saved2)):
        o = (torch.full((B, T, H), 7.0, device="cuda"), torch.full((B, U + 1, H), 7.0, device="cuda"),
             torch.full((H, V), 7.0, device="cuda"), torch.full((V,), 7.0, device="cuda"))
        args = [_p(d["enc"]), _p(d["pred"]), _p(d["W_out"]), _p(d["b_out"]), dc, _p(d["labels"]),
                _p(d["T_lens"]), _p(d["U_lens"]), B, T, U, H, V, inp.blank, *tiles, _p(gc),
                _p(st), *(_p(x) for x in o)]
        if k == 0:
            wsb = rj.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, *tiles, 1)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
            rc = lib.rnnt_joint_loss_bwd(*args, _p(ws), ws.numel(), stream)
        else:
            rc = lib.rnnt_joint_loss_bwd_noalloc(*args, stream)
        assert rc == 0, rc
        assert rj.rnnt_joint_loss_status(st) == 0
        outs.append([x.double().cpu().numpy() for x in o])
    return outs


@pytest.mark.parametrize("tiles", [(0, 0, 0), (16, 8, 0)])
def test_noalloc_backward_matches_workspace_backward(tiles):
    names = ("d_enc", "d_pred", "d_W_out", "d_b_out")
    big = make_config("short")
    print(f"[noalloc short fp32 tiles={tiles}]", flush=True)
    ref, got = _both(big, tiles, gcs=list(np.linspace(-1.0, 1.0, big.B)))
    for n, a, b in zip(names, got, ref):
        check_grad(n, a, b, "fp32")
    small = make_inputs(3, 40, 9, 128, 96, dtype="bf16", sigma=0.3, seed=7, t_range=(1, 40),
                        u_range=(0, 9))
    print(f"[noalloc small bf16 tiles={tiles}]", flush=True)
    ref, got = _both(small, tiles)
    for n, a, b in zip(names, got, ref):
        check_grad(n, a, b, "bf16")
        # entries past the smaller problem's lengths carry nothing over from the first call
    for x in got[:2]:
        assert np.isfinite(x).all()
