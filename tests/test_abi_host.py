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
                          "rnnt_joint_loss_bwd_noalloc", "rnnt_joint_loss_pruned_fwd",
                          "rnnt_joint_loss_pruned_workspace_bytes", "rnnt_joint_loss_pruned_bounds",
                          "rnnt_joint_loss_tdt_saved_bytes", "rnnt_joint_loss_tdt_workspace_bytes",
                          "rnnt_joint_loss_tdt_fwd", "rnnt_joint_loss_tdt_bwd",
                          "rnnt_joint_loss_get_flags", "rnnt_joint_loss_set_flags",
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
    # the skewed [B, T+U, U+1] layout, W^T and W_out in 32-column blocks, and
    # e^{2 enc}, e^{2 pred} (float32);
    # untiled adds the logits and the h rows of the padded lattice.
    rc, tiled = _saved(16, 500, 100, 640, 1024, 1, 64, 64, 0)
    assert rc == 0
    cells = 16 * 600 * 101
    tiles = 16 * 32 * 13  # 16 x 8 tiles of the padded lattice, one int32 each
    fixed = cells * 28 + 2 * 640 * 1024 * 2 + 4 * 16 * (500 + 101) * 640 + 4 * tiles
    assert fixed <= tiled <= fixed + 64 * 1024
    rc, untiled = _saved(16, 500, 100, 640, 1024, 1)
    assert rc == 0
    assert untiled - tiled >= 16 * 512 * 104 * (1024 + 640) * 2
    chunk = 16 * 64 * 64
    # 8 x 2 chunks, each with a list of 16 * 4 * 8 tiles, and 16 tile counts
    lists = 16 * (16 * 4 * 8) * 4 + 256
    least = 8 * 1024 + chunk * (1024 + 640) * 2 + lists
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64, p=2) == (0, least)
    # pass 1: a second chunk buffer pair, for the overlapped chunk schedule
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64) == (0, least + chunk * (1024 + 640) * 2)
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64, p=3)[0] == 1
    # untiled: only the bias-gradient accumulator (the h rows are in the saved
    # state, and the logit gradients replace the stored logits in place)
    assert _ws(16, 500, 100, 640, 1024, 1) == (0, 8 * 1024)
    assert _ws(16, 500, 100, 640, 1024, 1, p=2) == (0, 8 * 1024)
    assert _ws(16, 500, 100, 640, 1024, 1, 64, 64, 0, 0) == (0, 0)


@pytest.mark.parametrize("args,code", [
    ((0, 10, 2, 64, 32, 0), 1),        # B < 1
    ((2, 0, 2, 64, 32, 0), 1),         # T < 1
    ((2, 10, -1, 64, 32, 0), 1),       # U < 0
    ((2, 10, 2, 64, 32, 7), 1),        # dtype
    ((2, 10, 2, 60, 32, 0), 2),        # H not a multiple of 16
    ((2, 10, 2, 784, 32, 0), 2),       # fp32 H > 768
    ((2, 10, 2, 784, 32, 1), 2),       # bf16 H > 768
    ((2, 10, 2, 64, 30, 0), 2),        # V not a multiple of 8
    ((2, 10, 1024, 64, 32, 0), 2),     # U + 1 > 1024
    ((8192, 10, 2, 64, 32, 0), 2),     # B > 8191
    ((2, 65521, 2, 64, 32, 0), 2),     # T > 65520
    ((2, 10, 2, 64, 262152, 0), 2),    # V > 262144
])
def test_shape_errors(args, code):
    assert _saved(*args)[0] == code


def test_label_limit():
    """U + 1 up to 1024 for the fused path; the token-and-duration and pruned
    entry points keep U + 1 <= 512."""
    assert _saved(2, 10, 1023, 64, 32, 0)[0] == 0
    assert _saved(2, 10, 600, 64, 32, 0, 16, 8)[0] == 0
    out = ctypes.c_size_t(0)
    assert lib.rnnt_joint_loss_pruned_workspace_bytes(2, 20, 511, 64, 32, 0, ctypes.byref(out)) == 0
    assert lib.rnnt_joint_loss_pruned_workspace_bytes(2, 20, 512, 64, 32, 0, ctypes.byref(out)) == 2
    assert lib.rnnt_joint_loss_tdt_saved_bytes(2, 20, 511, 64, 32, 0, 16, 8, 0, 5,
                                               ctypes.byref(out)) == 0
    assert lib.rnnt_joint_loss_tdt_saved_bytes(2, 20, 512, 64, 32, 0, 16, 8, 0, 5,
                                               ctypes.byref(out)) == 2
    assert lib.rnnt_joint_loss_tdt_workspace_bytes(2, 20, 512, 64, 32, 0, 16, 8, 0, 5, 0,
                                                   ctypes.byref(out)) == 2


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


def test_noalloc_backward_rejects_sizes_beyond_its_scratch():
    """The no-allocation backward refuses, before anything is enqueued, sizes
    whose backward workspace exceeds its static scratch (64 MiB): the long
    workload in 64 x 64 chunks over the whole vocabulary needs ~0.3 GB of
    logit gradients per chunk.  In vocabulary parts of 256 columns it needs
    ~59 MB, which passes the size check (and then fails the null pointers)."""
    ws = _ws(8, 1500, 300, 640, 4096, 1, 64, 64, 0)[1]
    assert ws > (64 << 20)
    rc = lib.rnnt_joint_loss_bwd_noalloc(None, None, None, None, 1, None, None, None, 8, 1500,
                                         300, 640, 4096, 0, 64, 64, 0, None, None, None, None,
                                         None, None, None)
    assert rc == 3
    # the least workspace (pass 2) is what the scratch must hold: the
    # no-allocation backward runs every kernel on one stream
    assert _ws(8, 1500, 300, 640, 4096, 1, 64, 64, 256, p=2)[1] <= (64 << 20)
    rc = lib.rnnt_joint_loss_bwd_noalloc(None, None, None, None, 1, None, None, None, 8, 1500,
                                         300, 640, 4096, 0, 64, 64, 256, None, None, None, None,
                                         None, None, None)
    assert rc == 1
    # bad sizes are reported as for the other entry points
    rc = lib.rnnt_joint_loss_bwd_noalloc(None, None, None, None, 1, None, None, None, 0, 10,
                                         3, 64, 64, 0, 0, 0, 0, None, None, None, None,
                                         None, None, None)
    assert rc == 1


def test_pruned_forward_host_checks():
    """The pruned forward refuses, before anything is enqueued: the untiled
    mode, a window below one position, too long a time axis, and a
    workspace smaller than rnnt_joint_loss_pruned_workspace_bytes."""
    out = ctypes.c_size_t(0)
    assert lib.rnnt_joint_loss_pruned_workspace_bytes(2, 20, 5, 64, 32, 0, ctypes.byref(out)) == 0
    ws = out.value
    # float64 simple-joiner rows (am, lm), per-cell lattice arrays and row scalars
    assert ws >= 8 * 2 * (20 + 6) * 32 + 4 * 8 * 2 * 25 * 6
    assert lib.rnnt_joint_loss_pruned_workspace_bytes(1, 32001, 5, 64, 32, 0,
                                                      ctypes.byref(out)) == 2
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    args = lambda tt, tu, S, wsb: (p, p, p, p, 0, p, p, p, 2, 20, 5, 64, 32, 0, tt, tu, 0, S, p,
                                   None, p, p, wsb, None)
    assert lib.rnnt_joint_loss_pruned_fwd(*args(0, 0, 3, ws)) == 2   # untiled
    assert lib.rnnt_joint_loss_pruned_fwd(*args(16, 8, 0, ws)) == 1  # S < 1
    assert lib.rnnt_joint_loss_pruned_fwd(*args(16, 8, 3, ws - 8)) == 3


def test_tdt_host_checks():
    """Token-and-duration calls: buffer sizes grow by the duration
    log-probabilities (saved) and the posteriors and duration gradients
    (backward workspace); bad duration sets are refused before anything is
    enqueued."""
    base = _saved(2, 20, 5, 64, 32, 0, 16, 8)[1]
    out = ctypes.c_size_t(0)
    assert lib.rnnt_joint_loss_tdt_saved_bytes(2, 20, 5, 64, 32, 0, 16, 8, 0, 5,
                                               ctypes.byref(out)) == 0
    cells = 2 * 25 * 6
    assert out.value >= base + 4 * cells * 5
    wsb = _ws(2, 20, 5, 64, 32, 0, 16, 8)[1]
    assert lib.rnnt_joint_loss_tdt_workspace_bytes(2, 20, 5, 64, 32, 0, 16, 8, 0, 5, 1,
                                                   ctypes.byref(out)) == 0
    assert out.value >= wsb + 16 * cells + 4 * cells * 5
    assert lib.rnnt_joint_loss_tdt_saved_bytes(2, 20, 5, 64, 32, 0, 16, 8, 0, 9,
                                               ctypes.byref(out)) == 1
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its host checks
    for durs, code in (((0,), 1), ((1, 1), 1), ((0, 16), 2), ((-1, 1), 2)):
        arr = (ctypes.c_int32 * len(durs))(*durs)
        rc = lib.rnnt_joint_loss_tdt_fwd(p, p, p, p, p, p, 0, p, p, p, 2, 20, 5, 64, 32, 0, arr,
                                         len(durs), 16, 8, 0, p, p, None, 0, None)
        assert rc == code, (durs, rc)


def test_flags_roundtrip_and_environment():
    """The debug / deterministic switches: set and read back, unknown bits
    refused, the environment read when the library loads, and the backward
    workspace growing by the partial-sum buffers in deterministic mode."""
    import os
    import subprocess
    import sys
    old = _lib.get_flags()
    try:
        _lib.set_flags(0)
        assert _lib.get_flags() == 0
        plain = _ws(8, 200, 50, 256, 512, 0, 64, 64, 128)[1]
        out = ctypes.c_size_t(0)
        assert lib.rnnt_joint_loss_tdt_workspace_bytes(8, 200, 50, 256, 512, 0, 64, 64, 128, 5, 1,
                                                       ctypes.byref(out)) == 0
        tdt_plain = out.value
        _lib.set_flags(_lib.FLAG_DETERMINISTIC)
        assert _lib.get_flags() == _lib.FLAG_DETERMINISTIC
        det = _ws(8, 200, 50, 256, 512, 0, 64, 64, 128)[1]
        # per-tile d_enc / d_pred rows of a 64 x 64 chunk (8 x 4 x 8 tiles) and
        # at least one split-K part of d_W_out
        assert det >= plain + 4 * 256 * 24 * 256 + 4 * 256 * 512
        # token-and-duration: also each 16-frame block's d_W_dur / d_b_dur sums
        # (8 utterances x 13 blocks)
        assert lib.rnnt_joint_loss_tdt_workspace_bytes(8, 200, 50, 256, 512, 0, 64, 64, 128, 5, 1,
                                                       ctypes.byref(out)) == 0
        assert out.value >= tdt_plain + (det - plain) + 4 * 8 * 13 * 256 * 5
        assert lib.rnnt_joint_loss_set_flags(4) == 1
        assert _lib.get_flags() == _lib.FLAG_DETERMINISTIC
    finally:
        _lib.set_flags(old)
    code = ("import sys; sys.path.insert(0, %r); from rnn_joint_transducer_amd import _lib; "
            "print(_lib.get_flags())" % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    env = dict(os.environ, RNNTJ_DEBUG="1", RNNTJ_DETERMINISTIC="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "3"
    env = dict(os.environ, RNNTJ_DEBUG="0")
    env.pop("RNNTJ_DETERMINISTIC", None)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.stdout.strip().splitlines()[-1] == "0"


def test_workspace_falls_with_tile_v():
    """The tiled backward holds one vocabulary part of a chunk's logit
    gradients: its workspace shrinks by B*tile_t*tile_u*(V - tile_v)
    elements as tile_v narrows; the untiled mode ignores tile_v."""
    B, T, U, H, V = 8, 1500, 300, 640, 4096
    full = _ws(B, T, U, H, V, 1, 64, 64, 0)[1]
    for tv in (128, 256, 1024):
        part = _ws(B, T, U, H, V, 1, 64, 64, tv)[1]
        assert full - part >= 2 * B * 64 * 64 * (V - tv) - 4096
    assert _ws(B, T, U, H, V, 1, 64, 64, 8192)[1] == full
    assert _ws(2, 20, 5, 64, 32, 0, 0, 0, 128)[1] == _ws(2, 20, 5, 64, 32, 0, 0, 0, 0)[1]
