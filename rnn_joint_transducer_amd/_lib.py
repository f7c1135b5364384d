"""ctypes loader for librnntjoint.so (no torch import here).

The library is built in-tree by ``python -m rnn_joint_transducer_amd.build``
(or ``__graft_entry__.build()``).  Loading fails loudly if it is missing:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librnntjoint.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "rnnt_joint.h")

RNNTJ_F32 = 0
RNNTJ_BF16 = 1
STATUS = {0: "RNNTJ_OK", 1: "RNNTJ_ERR_ARG", 2: "RNNTJ_ERR_UNSUPPORTED",
          3: "RNNTJ_ERR_WORKSPACE", 4: "RNNTJ_ERR_HIP", 5: "RNNTJ_ERR_DATA"}

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
_SIG = {
    "rnnt_joint_loss_abi_version": (_c_int, []),
    "rnnt_joint_loss_get_flags": (_c_int, []),
    "rnnt_joint_loss_set_flags": (_c_int, [_c_int]),
    "rnnt_joint_loss_strerror": (ctypes.c_char_p, [_c_int]),
    "rnnt_joint_loss_last_error": (ctypes.c_char_p, []),
    "rnnt_joint_loss_saved_bytes": (_c_int, [_c_int] * 9 + [ctypes.POINTER(_c_size)]),
    "rnnt_joint_loss_workspace_bytes": (_c_int, [_c_int] * 10 + [ctypes.POINTER(_c_size)]),
    "rnnt_joint_loss_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 9
                            + [_vp, _vp, _vp, _c_size, _vp]),
    "rnnt_joint_loss_fwd_ex": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 10
                               + [_vp, _vp, _vp, _c_size, _vp]),
    "rnnt_joint_loss_bwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 9
                            + [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "rnnt_joint_loss_bwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]
                                    + [_c_int] * 9 + [_vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "rnnt_joint_loss_pruned_workspace_bytes": (_c_int, [_c_int] * 6 + [ctypes.POINTER(_c_size)]),
    "rnnt_joint_loss_pruned_fwd": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp]
                                   + [_c_int] * 10 + [_vp, _vp, _vp, _vp, _c_size, _vp]),
    "rnnt_joint_loss_pruned_bounds": (_c_int, [_vp] + [_c_int] * 9 + [_vp, _vp]),
    "rnnt_joint_loss_tdt_saved_bytes": (_c_int, [_c_int] * 10 + [ctypes.POINTER(_c_size)]),
    "rnnt_joint_loss_tdt_workspace_bytes": (_c_int, [_c_int] * 11 + [ctypes.POINTER(_c_size)]),
    "rnnt_joint_loss_tdt_fwd": (_c_int, [_vp] * 6 + [_c_int, _vp, _vp, _vp] + [_c_int] * 6
                                + [_vp] + [_c_int] * 4 + [_vp, _vp, _vp, _c_size, _vp]),
    "rnnt_joint_loss_tdt_bwd": (_c_int, [_vp] * 6 + [_c_int, _vp, _vp, _vp] + [_c_int] * 6
                                + [_vp] + [_c_int] * 4 + [_vp] * 8 + [_vp, _c_size, _vp]),
    "rnnt_joint_loss_status": (_c_int, [_vp, _vp, ctypes.POINTER(ctypes.c_int32)]),
    "rnnt_joint_loss_timing": (_c_int, [_c_int]),
    "rnnt_joint_loss_timing_report": (_c_int, [ctypes.c_char_p, _c_size]),
    "rnnt_joint_proj_fwd": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "rnnt_joint_proj_bwd": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                     _vp]),
}

_lib = None


class RNNTJointError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = STATUS.get(code, str(code))
        try:
            msg += ": " + load().rnnt_joint_loss_strerror(code).decode()
            if code == 4:
                msg += " [" + load().rnnt_joint_loss_last_error().decode() + "]"
        except Exception:  # pragma: no cover
            pass
        super().__init__(f"{where} failed with {msg}")


def load(path: str = LIB_PATH):
    """Load the built library (cached).  Raises OSError if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run `python -m rnn_joint_transducer_amd.build` "
                      "(the HIP extension is required: there is no CPU fallback)")
    # PyTorch ships its own HIP runtime under the same soname.  Load it first so
    # that this library binds to that one: two HIP runtimes in one process do
    # not share the device (the one loaded second sees none).
    try:
        import torch  # noqa: F401
    except ImportError:  # a plain C/ctypes user: /opt/rocm's runtime is used
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIG.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def declared_functions(header: str = HEADER):
    """Names of the functions include/rnnt_joint.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rnnt_joint_(?:loss|proj)_\w+)\s*\(", text)))


def check(code: int, where: str):
    if code != 0:
        raise RNNTJointError(code, where)


def timing(enable: bool):
    """Turn the library's per-kernel HIP-event timing on or off."""
    check(load().rnnt_joint_loss_timing(1 if enable else 0), "rnnt_joint_loss_timing")


def timing_report() -> dict:
    """{kernel: (launches, total_ms)} for the launches recorded since timing
    was enabled (waits for them); clears the record."""
    buf = ctypes.create_string_buffer(1 << 16)
    check(load().rnnt_joint_loss_timing_report(buf, len(buf)), "rnnt_joint_loss_timing_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split()
        out[name] = (int(n), float(ms))
    return out


FLAG_DEBUG = 1
FLAG_DETERMINISTIC = 2


def get_flags() -> int:
    """The library's process-wide switches (FLAG_DEBUG | FLAG_DETERMINISTIC)."""
    return load().rnnt_joint_loss_get_flags()


def set_flags(flags: int) -> None:
    check(load().rnnt_joint_loss_set_flags(flags), "rnnt_joint_loss_set_flags")
