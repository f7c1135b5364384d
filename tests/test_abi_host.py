"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, sizes its buffers, and rejects bad arguments before enqueuing any
work (so these run without a GPU)."""
import ctypes

import pytest

from rnn_joint_transducer_amd import _lib

lib = pytest.importorskip("rnn_joint_transducer_amd._lib").load()


def test_exports_every_declared_symbol():
    names = _lib.declared_functions()
    assert set(names) == {"rnnt_joint_loss_abi_version", "rnnt_joint_loss_strerror",
                          "rnnt_joint_loss_saved_bytes", "rnnt_joint_loss_workspace_bytes",
                          "rnnt_joint_loss_fwd", "rnnt_joint_loss_fwd_ex", "rnnt_joint_loss_bwd",
                          "rnnt_joint_loss_last_error",
                          "rnnt_joint_loss_status", "rnnt_joint_loss_timing",
                          "rnnt_joint_loss_timing_report", "rnnt_joint_proj_fwd",
                          "rnnt_joint_proj_bwd"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert lib.rnnt_joint_loss_abi_version() == 1
    for code in range(6):
        assert lib.rnnt_joint_loss_strerror(code)
    assert b"unknown" in lib.rnnt_joint_loss_strerror(99)
    assert lib.rnnt_joint_loss_last_error() == b""


def _saved(B, T, U, H, V, dt, tt=0, tu=0, tv=0):
    out = ctypes.c_size_t(0)
    rc = lib.rnnt_joint_loss_saved_bytes(B, T, U, H, V, dt, tt, tu, tv, ctypes.byref(out))
    return rc, out.value


def _ws(B, T, U, H, V, dt, tt=0, tu=0, tv=0, p=1):
    out = ctypes.c_size_t(0)
    rc = lib.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dt, tt, tu, tv, p, ctypes.byref(out))
    return rc, out.value


def test_buffer_sizes():
    # medium workload, bf16: per cell lse/LB/LE (12 B) + alpha/beta (16 B) over
    # the skewed [B, T+U, U+1] layout, W^T, and e^{2 enc}, e^{2 pred} (float32);
    # untiled adds the logits and the h rows of the padded lattice.
    rc, tiled = _saved(16, 500, 100, 640, 1024, 1, 64, 64, 0)
    assert rc == 0
    cells = 16 * 600 * 101
    tiles = 16 * 32 * 13  # 16 x 8 tiles of the padded lattice, one int32 each
    fixed = cells * 28 + 640 * 1024 * 2 + 4 * 16 * (500 + 101) * 640 + 4 * tiles
    assert fixed <= tiled <= fixed + 64 * 1024
    rc, untiled = _saved(16, 500, 100, 640, 1024, 1)
    assert rc == 0
    assert untiled - tiled >= 16 * 512 * 104 * (1024 + 640) * 2
    chunk = 16 * 64 * 64
    # 8 x 2 chunks, each with a list of 16 * 4 * 8 tiles, and 16 tile counts
    lists = 16 * (16 * 4 * 8) * 4 + 256
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64) == (0, 8 * 1024 + chunk * (1024 + 640) * 2 + lists)
    # untiled: only the bias-gradient accumulator (the h rows are in the saved
    # state, and the logit gradients replace the stored logits in place)
    assert _ws(16, 500, 100, 640, 1024, 1) == (0, 8 * 1024)
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64, 0, 0) == (0, 0)


@pytest.mark.parametrize("args,code", [
    ((0, 10, 2, 64, 32, 0), 1),        # B < 1
    ((2, 0, 2, 64, 32, 0), 1),         # T < 1
    ((2, 10, -1, 64, 32, 0), 1),       # U < 0
    ((2, 10, 2, 64, 32, 7), 1),        # dtype
    ((2, 10, 2, 60, 32, 0), 2),        # H not a multiple of 16
    ((2, 10, 2, 512, 32, 0), 2),       # fp32 H > 256
    ((2, 10, 2, 64, 30, 0), 2),        # V not a multiple of 8
    ((2, 10, 600, 64, 32, 0), 2),      # U + 1 > 512
    ((8192, 10, 2, 64, 32, 0), 2),     # B > 8191
    ((2, 65521, 2, 64, 32, 0), 2),     # T > 65520
    ((2, 10, 2, 64, 262152, 0), 2),    # V > 262144
])
def test_shape_errors(args, code):
    assert _saved(*args)[0] == code


def test_tile_errors():
    assert _saved(2, 10, 2, 64, 32, 0, 10, 8)[0] == 2   # tile_t not a multiple of 16
    assert _saved(2, 10, 2, 64, 32, 0, 16, 4)[0] == 2   # tile_u not a multiple of 8
    assert _saved(2, 10, 2, 64, 32, 0, 16, 8, 64)[0] == 2
    assert _saved(2, 10, 2, 64, 32, 0, 16, 8, 128)[0] == 0
    assert _saved(2, 10, 2, 64, 32, 0, 16, 8, 256)[0] == 0
    assert _saved(2, 10, 2, 64, 32, 0, 16, 8, 320)[0] == 2
    assert _saved(2, 10, 2, 64, 32, 0, -16, 8)[0] == 1


def _fwd(**kw):
    p = dict(enc=1, pred=1, W=1, b=1, dtype=0, labels=1, T=1, U_lens=1, B=2, Tm=10, Um=2,
             H=64, V=32, blank=0, tt=0, tu=0, tv=0, costs=1, saved=1, ws=None, wsb=0)
    p.update(kw)
    ptr = lambda v: None if v is None else ctypes.c_void_p(16 * v)  # 16-aligned fake pointers
    return lib.rnnt_joint_loss_fwd(ptr(p["enc"]), ptr(p["pred"]), ptr(p["W"]), ptr(p["b"]),
                                   p["dtype"], ptr(p["labels"]), ptr(p["T"]), ptr(p["U_lens"]),
                                   p["B"], p["Tm"], p["Um"], p["H"], p["V"], p["blank"], p["tt"],
                                   p["tu"], p["tv"], ptr(p["costs"]), ptr(p["saved"]),
                                   ptr(p["ws"]), p["wsb"], None)


def test_fwd_rejects_before_launch():
    # each of these returns before any HIP call (the fake pointers are never used)
    assert _fwd(enc=None) == 1
    assert _fwd(costs=None) == 1
    assert _fwd(saved=None) == 1
    assert _fwd(labels=None) == 1
    assert _fwd(blank=32) == 1
    assert _fwd(blank=-1) == 1
    assert _fwd(H=60) == 2
    assert _fwd(tt=8) == 2
    assert lib.rnnt_joint_loss_fwd(ctypes.c_void_p(17), *([ctypes.c_void_p(16)] * 3), 0,
                                   *([ctypes.c_void_p(16)] * 3), 2, 10, 2, 64, 32, 0, 0, 0, 0,
                                   ctypes.c_void_p(16), ctypes.c_void_p(16), None, 0, None) == 1


def test_bwd_rejects_before_launch():
    v = lambda: ctypes.c_void_p(16)
    base = [v(), v(), v(), v(), 0, v(), v(), v(), 2, 10, 2, 64, 32, 0]
    # tiled mode needs a workspace
    rc = lib.rnnt_joint_loss_bwd(*base, 16, 8, 0, None, v(), v(), v(), v(), v(), None, 0, None)
    assert rc == 3
    rc = lib.rnnt_joint_loss_bwd(*base, 0, 0, 0, None, v(), v(), v(), v(), v(), None, 0, None)
    assert rc == 3
    rc = lib.rnnt_joint_loss_bwd(*base, 0, 0, 0, None, None, v(), v(), v(), v(), v(), 4096, None)
    assert rc == 1
    rc = lib.rnnt_joint_loss_bwd(*base, 0, 0, 0, None, v(), v(), None, v(), v(), v(), 4096, None)
    assert rc == 1


def test_status_rejects_null():
    assert lib.rnnt_joint_loss_status(None, None, None) == 1


def test_timing_report_empty():
    assert lib.rnnt_joint_loss_timing(1) == 0
    assert _lib.timing_report() == {}
    assert lib.rnnt_joint_loss_timing(0) == 0
    assert lib.rnnt_joint_loss_timing_report(None, 0) == 1


def test_fwd_ex_rejects_unknown_criterion():
    """rnnt_joint_loss_fwd_ex checks the criterion on the host (nothing is
    enqueued, so fake aligned pointers suffice)."""
    v = lambda: ctypes.c_void_p(16 * 4096)
    args = [v(), v(), v(), v(), 0, v(), v(), v(), 2, 10, 2, 64, 32, 0, 0, 0, 0]
    for crit in (-1, 2, 7):
        rc = lib.rnnt_joint_loss_fwd_ex(*args, crit, v(), v(), None, 0, None)
        assert rc == 1, (crit, rc)


def test_proj_rejects_before_launch():
    """The projection entry points check pointers, dtype, sizes and alignment
    on the host (nothing is enqueued, so fake aligned pointers suffice)."""
    v = lambda k=1: ctypes.c_void_p(16 * 4096 * k)
    fwd = lambda *a: lib.rnnt_joint_proj_fwd(*a)
    assert fwd(v(), v(), v(), 0, 10, 64, 64, None, None) == 1          # y missing
    assert fwd(v(), v(), v(), 2, 10, 64, 64, v(), None) == 1           # dtype
    assert fwd(v(), v(), v(), 0, 0, 64, 64, v(), None) == 1            # M < 1
    assert fwd(v(), v(), v(), 0, 10, 60, 64, v(), None) == 2           # K not a multiple of 16
    assert fwd(v(), v(), v(), 1, 10, 64, 72, v(), None) == 2           # N not a multiple of 16
    assert fwd(v(), v(), v(), 0, 10, 65552, 64, v(), None) == 2        # K > 65536
    assert fwd(ctypes.c_void_p(16 * 4096 + 8), v(), v(), 0, 10, 64, 64, v(), None) == 1  # align
    bwd = lambda *a: lib.rnnt_joint_proj_bwd(*a)
    assert bwd(v(), v(), 0, 10, 64, 64, None, v(), v(), v(), None) == 1   # dy missing
    assert bwd(v(), v(), 0, 10, 64, 64, v(), v(), None, v(), None) == 1   # dW missing
    assert bwd(v(), v(), 0, 10, 48, 40, v(), v(), v(), v(), None) == 2    # N not a multiple of 16
