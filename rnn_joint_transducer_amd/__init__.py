"""Fused RNN-T joint network + transducer loss for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/rnnt_joint.h`` (argument
marshalling only; every step runs in the HIP kernels of librnntjoint.so).
PyTorch provides device memory and the current stream.

    costs, saved = rnnt_joint_loss_fwd(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    d_enc, d_pred, d_W, d_b = rnnt_joint_loss_bwd(enc, ..., saved=saved)
    costs = rnnt_joint_loss(enc, pred, W_out, b_out, labels, T_lens, U_lens)  # autograd

Tiling (``tile_t``, ``tile_u``, ``tile_v``) follows the C ABI: tile_t = tile_u
= 0 is the untiled mode (logits stored by the forward); otherwise the backward
recomputes the joint per lattice chunk of tile_t x tile_u cells.
"""
from __future__ import annotations

import ctypes

from ._lib import (RNNTJ_BF16, RNNTJ_F32, RNNTJointError, check, declared_functions,  # noqa: F401
                   load)

__all__ = ["rnnt_joint_loss_fwd", "rnnt_joint_loss_bwd", "rnnt_joint_loss_bwd_noalloc",
           "rnnt_joint_loss_status", "rnnt_joint_loss_pruned_fwd",
           "rnnt_joint_loss_pruned_workspace_bytes", "rnnt_joint_loss_pruned_bounds",
           "rnnt_joint_loss_tdt_fwd", "rnnt_joint_loss_tdt_bwd",
           "rnnt_joint_loss_saved_bytes", "rnnt_joint_loss_workspace_bytes",
           "rnnt_joint_loss", "RNNTJointError", "load"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return RNNTJ_F32
    if t.dtype == torch.bfloat16:
        return RNNTJ_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def rnnt_joint_loss_saved_bytes(B, T, U, H, V, dtype_code, tile_t=0, tile_u=0, tile_v=0) -> int:
    out = ctypes.c_size_t(0)
    check(load().rnnt_joint_loss_saved_bytes(B, T, U, H, V, dtype_code, tile_t, tile_u, tile_v,
                                             ctypes.byref(out)), "rnnt_joint_loss_saved_bytes")
    return out.value


def rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dtype_code, tile_t=0, tile_u=0, tile_v=0,
                                    pass_=1) -> int:
    out = ctypes.c_size_t(0)
    check(load().rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dtype_code, tile_t, tile_u,
                                                 tile_v, pass_, ctypes.byref(out)),
          "rnnt_joint_loss_workspace_bytes")
    return out.value


def _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens):
    import torch
    B, T, H = enc.shape
    U = pred.shape[1] - 1
    V = W_out.shape[1]
    dt = enc.dtype
    for name, t, shape in (("pred", pred, (B, U + 1, H)), ("W_out", W_out, (H, V)),
                           ("b_out", b_out, (V,))):
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"{name}: expected shape {shape} dtype {dt}, got "
                             f"{tuple(t.shape)} {t.dtype}")
    for name, t, shape in (("labels", labels, (B, U)), ("T_lens", T_lens, (B,)),
                           ("U_lens", U_lens, (B,))):
        if tuple(t.shape) != shape or t.dtype != torch.int32:
            raise ValueError(f"{name}: expected int32 shape {shape}, got {tuple(t.shape)} {t.dtype}")
    dev = enc.device
    for t in (enc, pred, W_out, b_out, labels, T_lens, U_lens):
        if t.device != dev or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the same GPU")
    if dev.type != "cuda":
        raise ValueError("tensors must live on the GPU (no CPU path)")
    return B, T, U, H, V


CRITERIA = {"sum": 0, "max": 1}  # rnntj_criterion


def rnnt_joint_loss_fwd(enc, pred, W_out, b_out, labels, T_lens, U_lens, blank=0, tile_t=0,
                        tile_u=0, tile_v=0, costs=None, saved=None, criterion="sum"):
    """Costs [B] (float32) and the uint8 `saved` state for the backward.
    criterion: "sum" (full sum over alignments) or "max" (best alignment);
    the backward follows the criterion recorded in `saved`."""
    if criterion not in CRITERIA:
        raise ValueError(f"criterion must be one of {sorted(CRITERIA)}, not {criterion!r}")
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    dc = _dtype_code(enc)
    nbytes = rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v)
    if saved is None:
        saved = torch.empty(nbytes, dtype=torch.uint8, device=enc.device)
    elif saved.numel() < nbytes:
        raise ValueError(f"saved buffer too small ({saved.numel()} < {nbytes})")
    if costs is None:
        costs = torch.empty(B, dtype=torch.float32, device=enc.device)
    rc = load().rnnt_joint_loss_fwd_ex(_ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out), dc,
                                       _ptr(labels), _ptr(T_lens), _ptr(U_lens), B, T, U, H, V,
                                       blank, tile_t, tile_u, tile_v, CRITERIA[criterion],
                                       _ptr(costs), _ptr(saved), None, 0, _stream(enc.device))
    check(rc, "rnnt_joint_loss_fwd_ex")
    return costs, saved


def rnnt_joint_loss_pruned_workspace_bytes(B, T, U, H, V, dtype_code) -> int:
    out = ctypes.c_size_t(0)
    check(load().rnnt_joint_loss_pruned_workspace_bytes(B, T, U, H, V, dtype_code,
                                                        ctypes.byref(out)),
          "rnnt_joint_loss_pruned_workspace_bytes")
    return out.value


def rnnt_joint_loss_pruned_fwd(enc, pred, W_out, b_out, labels, T_lens, U_lens, S, blank=0,
                               tile_t=64, tile_u=0, tile_v=0, costs=None, simple_costs=None,
                               saved=None, workspace=None):
    """Pruned transducer loss (tiled mode): costs [B], simple_costs [B] (the
    simple joiner's cost) and `saved`, from which rnnt_joint_loss_bwd with the
    same tiles returns the gradients with the windows held fixed."""
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    dc = _dtype_code(enc)
    dev = enc.device
    nbytes = rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v)
    if saved is None:
        saved = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    elif saved.numel() < nbytes:
        raise ValueError(f"saved buffer too small ({saved.numel()} < {nbytes})")
    ws = rnnt_joint_loss_pruned_workspace_bytes(B, T, U, H, V, dc)
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    elif workspace.numel() < ws:
        raise ValueError(f"workspace too small ({workspace.numel()} < {ws})")
    if costs is None:
        costs = torch.empty(B, dtype=torch.float32, device=dev)
    if simple_costs is None:
        simple_costs = torch.empty(B, dtype=torch.float32, device=dev)
    rc = load().rnnt_joint_loss_pruned_fwd(_ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out), dc,
                                           _ptr(labels), _ptr(T_lens), _ptr(U_lens), B, T, U, H,
                                           V, blank, tile_t, tile_u, tile_v, S, _ptr(costs),
                                           _ptr(simple_costs), _ptr(saved), _ptr(workspace),
                                           workspace.numel(), _stream(dev))
    check(rc, "rnnt_joint_loss_pruned_fwd")
    return costs, simple_costs, saved


def rnnt_joint_loss_pruned_bounds(saved, B, T, U, H, V, dtype_code, tile_t=64, tile_u=0,
                                  tile_v=0):
    """Window starts int32 [B, T] of a pruned forward's state."""
    import torch
    out = torch.empty(B, T, dtype=torch.int32, device=saved.device)
    check(load().rnnt_joint_loss_pruned_bounds(_ptr(saved), B, T, U, H, V, dtype_code, tile_t,
                                               tile_u, tile_v, _ptr(out), _stream(saved.device)),
          "rnnt_joint_loss_pruned_bounds")
    return out


def _durations(durations):
    arr = (ctypes.c_int32 * len(durations))(*[int(d) for d in durations])
    return arr, len(durations)


def rnnt_joint_loss_tdt_fwd(enc, pred, W_out, b_out, W_dur, b_dur, labels, T_lens, U_lens,
                            durations, blank=0, tile_t=0, tile_u=0, tile_v=0, costs=None,
                            saved=None):
    """Token-and-duration transducer loss: costs [B] (float32) and `saved`.
    W_dur [H, K], b_dur [K] in the dtype of enc; durations: K ints (host)."""
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    K = len(durations)
    if (tuple(W_dur.shape) != (H, K) or tuple(b_dur.shape) != (K,) or W_dur.dtype != enc.dtype
            or b_dur.dtype != enc.dtype or not W_dur.is_contiguous() or not b_dur.is_contiguous()
            or W_dur.device != enc.device or b_dur.device != enc.device):
        raise ValueError(f"W_dur / b_dur: expected contiguous [{H}, {K}] / [{K}] {enc.dtype}")
    dc = _dtype_code(enc)
    dev = enc.device
    out = ctypes.c_size_t(0)
    check(load().rnnt_joint_loss_tdt_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v, K,
                                                 ctypes.byref(out)), "rnnt_joint_loss_tdt_saved_bytes")
    if saved is None:
        saved = torch.empty(out.value, dtype=torch.uint8, device=dev)
    elif saved.numel() < out.value:
        raise ValueError(f"saved buffer too small ({saved.numel()} < {out.value})")
    if costs is None:
        costs = torch.empty(B, dtype=torch.float32, device=dev)
    dur, K = _durations(durations)
    rc = load().rnnt_joint_loss_tdt_fwd(_ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out),
                                        _ptr(W_dur), _ptr(b_dur), dc, _ptr(labels), _ptr(T_lens),
                                        _ptr(U_lens), B, T, U, H, V, blank, dur, K, tile_t, tile_u,
                                        tile_v, _ptr(costs), _ptr(saved), None, 0, _stream(dev))
    check(rc, "rnnt_joint_loss_tdt_fwd")
    return costs, saved


def rnnt_joint_loss_tdt_bwd(enc, pred, W_out, b_out, W_dur, b_dur, labels, T_lens, U_lens,
                            durations, saved, blank=0, tile_t=0, tile_u=0, tile_v=0,
                            grad_costs=None, workspace=None):
    """(d_enc, d_pred, d_W_out, d_b_out, d_W_dur, d_b_dur), float32."""
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    K = len(durations)
    dc = _dtype_code(enc)
    dev = enc.device
    need = ctypes.c_size_t(0)
    check(load().rnnt_joint_loss_tdt_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v, K,
                                                 ctypes.byref(need)), "rnnt_joint_loss_tdt_saved_bytes")
    if saved.dtype != torch.uint8 or saved.device != dev or saved.numel() < need.value:
        raise ValueError(f"saved: expected a uint8 buffer of at least {need.value} bytes on {dev}")
    ws = ctypes.c_size_t(0)
    least = ctypes.c_size_t(0)
    for pass_, out_ in ((1, ws), (2, least)):
        check(load().rnnt_joint_loss_tdt_workspace_bytes(B, T, U, H, V, dc, tile_t, tile_u,
                                                         tile_v, K, pass_, ctypes.byref(out_)),
              "rnnt_joint_loss_tdt_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(ws.value, dtype=torch.uint8, device=dev)
    elif workspace.numel() < least.value:
        raise ValueError(f"workspace too small ({workspace.numel()} < {least.value})")
    if grad_costs is not None:
        if grad_costs.dtype != torch.float32 or tuple(grad_costs.shape) != (B,):
            raise ValueError("grad_costs must be float32 [B]")
        grad_costs = grad_costs.contiguous()
    out = (torch.empty(B, T, H, dtype=torch.float32, device=dev),
           torch.empty(B, U + 1, H, dtype=torch.float32, device=dev),
           torch.empty(H, V, dtype=torch.float32, device=dev),
           torch.empty(V, dtype=torch.float32, device=dev),
           torch.empty(H, K, dtype=torch.float32, device=dev),
           torch.empty(K, dtype=torch.float32, device=dev))
    dur, K = _durations(durations)
    rc = load().rnnt_joint_loss_tdt_bwd(_ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out),
                                        _ptr(W_dur), _ptr(b_dur), dc, _ptr(labels), _ptr(T_lens),
                                        _ptr(U_lens), B, T, U, H, V, blank, dur, K, tile_t, tile_u,
                                        tile_v, _ptr(grad_costs), _ptr(saved),
                                        *(_ptr(x) for x in out), _ptr(workspace),
                                        workspace.numel(), _stream(dev))
    check(rc, "rnnt_joint_loss_tdt_bwd")
    return out


def rnnt_joint_loss_bwd(enc, pred, W_out, b_out, labels, T_lens, U_lens, saved, blank=0,
                        tile_t=0, tile_u=0, tile_v=0, grad_costs=None, workspace=None,
                        out=None):
    """(d_enc, d_pred, d_W_out, d_b_out), all float32."""
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    dc = _dtype_code(enc)
    dev = enc.device
    need = rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v)
    if saved.dtype != torch.uint8 or saved.device != dev or saved.numel() < need:
        raise ValueError(f"saved: expected a uint8 buffer of at least {need} bytes on {dev} "
                         f"(the forward's state for these sizes and tiles), got "
                         f"{saved.numel()} {saved.dtype} on {saved.device}")
    if workspace is None:
        # the size for the overlapped chunk schedule (pass 1)
        ws = rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v, 1)
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev)
    else:
        least = rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v, 2)
        if workspace.numel() < least:
            raise ValueError(f"workspace too small ({workspace.numel()} < {least})")
    if out is None:
        out = (torch.empty(B, T, H, dtype=torch.float32, device=dev),
               torch.empty(B, U + 1, H, dtype=torch.float32, device=dev),
               torch.empty(H, V, dtype=torch.float32, device=dev),
               torch.empty(V, dtype=torch.float32, device=dev))
    if grad_costs is not None:
        if grad_costs.dtype != torch.float32 or tuple(grad_costs.shape) != (B,):
            raise ValueError("grad_costs must be float32 [B]")
        grad_costs = grad_costs.contiguous()
    d_enc, d_pred, d_W, d_b = out
    rc = load().rnnt_joint_loss_bwd(_ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out), dc,
                                    _ptr(labels), _ptr(T_lens), _ptr(U_lens), B, T, U, H, V,
                                    blank, tile_t, tile_u, tile_v, _ptr(grad_costs),
                                    _ptr(saved), _ptr(d_enc), _ptr(d_pred), _ptr(d_W),
                                    _ptr(d_b), _ptr(workspace), workspace.numel(),
                                    _stream(dev))
    check(rc, "rnnt_joint_loss_bwd")
    return out


def rnnt_joint_loss_bwd_noalloc(enc, pred, W_out, b_out, labels, T_lens, U_lens, saved, blank=0,
                                tile_t=0, tile_u=0, tile_v=0, grad_costs=None, out=None):
    """As rnnt_joint_loss_bwd, with the library's static per-GPU scratch in
    place of a workspace (for callers that cannot allocate device memory;
    `out` must then be given).  Calls that overlap on one GPU race."""
    import torch
    B, T, U, H, V = _check_inputs(enc, pred, W_out, b_out, labels, T_lens, U_lens)
    dc = _dtype_code(enc)
    dev = enc.device
    need = rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tile_t, tile_u, tile_v)
    if saved.dtype != torch.uint8 or saved.device != dev or saved.numel() < need:
        raise ValueError(f"saved: expected a uint8 buffer of at least {need} bytes on {dev}")
    if out is None:
        out = (torch.empty(B, T, H, dtype=torch.float32, device=dev),
               torch.empty(B, U + 1, H, dtype=torch.float32, device=dev),
               torch.empty(H, V, dtype=torch.float32, device=dev),
               torch.empty(V, dtype=torch.float32, device=dev))
    if grad_costs is not None and (grad_costs.dtype != torch.float32
                                   or tuple(grad_costs.shape) != (B,)
                                   or not grad_costs.is_contiguous()):
        raise ValueError("grad_costs must be a contiguous float32 [B] tensor")
    d_enc, d_pred, d_W, d_b = out
    rc = load().rnnt_joint_loss_bwd_noalloc(
        _ptr(enc), _ptr(pred), _ptr(W_out), _ptr(b_out), dc, _ptr(labels), _ptr(T_lens),
        _ptr(U_lens), B, T, U, H, V, blank, tile_t, tile_u, tile_v, _ptr(grad_costs),
        _ptr(saved), _ptr(d_enc), _ptr(d_pred), _ptr(d_W), _ptr(d_b), _stream(dev))
    check(rc, "rnnt_joint_loss_bwd_noalloc")
    return out


def rnnt_joint_loss_status(saved) -> int:
    """Synchronises the current stream and returns the data-error bit mask."""
    v = ctypes.c_int32(0)
    check(load().rnnt_joint_loss_status(_ptr(saved), _stream(saved.device), ctypes.byref(v)),
          "rnnt_joint_loss_status")
    return v.value


def _make_function():
    import torch

    class _RNNTJointLoss(torch.autograd.Function):
        @staticmethod
        def forward(ctx, enc, pred, W_out, b_out, labels, T_lens, U_lens, blank, tile_t, tile_u,
                    tile_v, criterion):
            costs, saved = rnnt_joint_loss_fwd(enc, pred, W_out, b_out, labels, T_lens, U_lens,
                                               blank, tile_t, tile_u, tile_v, criterion=criterion)
            ctx.save_for_backward(enc, pred, W_out, b_out, labels, T_lens, U_lens, saved)
            ctx.cfg = (blank, tile_t, tile_u, tile_v)
            ctx.consumed = False
            return costs

        @staticmethod
        def backward(ctx, grad_costs):
            enc, pred, W_out, b_out, labels, T_lens, U_lens, saved = ctx.saved_tensors
            blank, tile_t, tile_u, tile_v = ctx.cfg
            if tile_t == 0 and tile_u == 0:
                if ctx.consumed:
                    raise RuntimeError(
                        "rnnt_joint_loss: the untiled backward turns the forward's stored logits "
                        "into gradients in place, so it runs once per forward; use a tiled mode "
                        "(tile_t or tile_u > 0) to differentiate the same graph again")
                ctx.consumed = True
            d_enc, d_pred, d_W, d_b = rnnt_joint_loss_bwd(
                enc, pred, W_out, b_out, labels, T_lens, U_lens, saved, blank, tile_t, tile_u,
                tile_v, grad_costs=grad_costs.float().contiguous())
            return (d_enc.to(enc.dtype), d_pred.to(pred.dtype), d_W.to(W_out.dtype),
                    d_b.to(b_out.dtype), None, None, None, None, None, None, None, None)

    return _RNNTJointLoss


_FN = None


def rnnt_joint_loss(enc, pred, W_out, b_out, labels, T_lens, U_lens, blank=0, tile_t=0,
                    tile_u=0, tile_v=0, criterion="sum"):
    """Per-utterance costs [B] with autograd support.  In the untiled mode the
    backward consumes the forward's stored logits (one backward per forward);
    in a tiled mode the saved state is only read, so a graph kept with
    retain_graph=True may be differentiated again."""
    global _FN
    if _FN is None:
        _FN = _make_function()
    return _FN.apply(enc, pred, W_out, b_out, labels, T_lens, U_lens, blank, tile_t, tile_u,
                     tile_v, criterion)


# ---------------------------------------------------------------- joint input projections

def _check_linear(x, W, b=None):
    """Shapes (M, K, N) of y = x @ W + b; b may be None."""
    import torch
    if not (x.is_cuda and W.is_cuda) or x.dtype != W.dtype or (b is not None and b.dtype != x.dtype):
        raise TypeError("x, W (and b) must be device tensors of one dtype")
    if W.dim() != 2 or x.shape[-1] != W.shape[0] or (b is not None and b.shape != (W.shape[1],)):
        raise ValueError(f"shapes x {tuple(x.shape)}, W {tuple(W.shape)} do not form x @ W + b")
    for t in (x, W) + (() if b is None else (b,)):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    M = x.numel() // x.shape[-1] if x.numel() else 0
    return M, W.shape[0], W.shape[1]


def rnnt_joint_proj_fwd(x, W, b=None):
    """Joint input projection y = x @ W + b (x [..., K], W [K, N], b [N] or
    None, one dtype; fp32 accumulation, y rounded once to that dtype)."""
    import torch
    M, K, N = _check_linear(x, W, b)
    y = torch.empty(*x.shape[:-1], N, dtype=x.dtype, device=x.device)
    check(load().rnnt_joint_proj_fwd(_ptr(x), _ptr(W), _ptr(b), _dtype_code(x), M, K, N, _ptr(y),
                                     _stream(x.device)), "rnnt_joint_proj_fwd")
    return y


def rnnt_joint_proj_bwd(x, W, dy, need_dx=True, need_db=True):
    """Gradients of y = x @ W + b from dy [..., N] (float32): (dx or None,
    dW, db or None), all float32."""
    import torch
    M, K, N = _check_linear(x, W)
    if dy.dtype != torch.float32 or not dy.is_contiguous() or dy.shape != (*x.shape[:-1], N):
        raise ValueError("dy must be a contiguous float32 tensor shaped like y")
    dev = x.device
    dx = torch.empty(x.shape, dtype=torch.float32, device=dev) if need_dx else None
    dW = torch.empty(K, N, dtype=torch.float32, device=dev)
    db = torch.empty(N, dtype=torch.float32, device=dev) if need_db else None
    check(load().rnnt_joint_proj_bwd(_ptr(x), _ptr(W), _dtype_code(x), M, K, N, _ptr(dy), _ptr(dx),
                                     _ptr(dW), _ptr(db), _stream(dev)), "rnnt_joint_proj_bwd")
    return dx, dW, db


def _make_proj_function():
    import torch

    class _JointProj(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, W, b):
            ctx.save_for_backward(x, W)
            return rnnt_joint_proj_fwd(x, W, b)

        @staticmethod
        def backward(ctx, dy):
            x, W = ctx.saved_tensors
            dx, dW, db = rnnt_joint_proj_bwd(x, W, dy.float().contiguous(),
                                             need_dx=ctx.needs_input_grad[0])
            return (None if dx is None else dx.to(x.dtype)), dW.to(W.dtype), db.to(W.dtype)

    return _JointProj


_PROJ = None


def rnnt_joint_proj(x, W, b):
    """y = x @ W + b with autograd support (feed y to rnnt_joint_loss as enc
    or pred)."""
    global _PROJ
    if _PROJ is None:
        _PROJ = _make_proj_function()
    return _PROJ.apply(x, W, b)


__all__ += ["rnnt_joint_proj_fwd", "rnnt_joint_proj_bwd", "rnnt_joint_proj"]
