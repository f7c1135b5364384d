"""Helpers shared by the GPU tests: move synth inputs to the GPU, run the HIP
path through the C ABI binding, and compare with the float64 oracle."""
from __future__ import annotations

import numpy as np

# Parity bar: fp32 |dloss|/loss <= 1e-5 and grad abs err <= 1e-4;
# bf16 2e-2 relative (loss per utterance, gradients as max-abs error over the
# tensor's max-abs value).
FP32_LOSS_REL = 1e-5
FP32_GRAD_ABS = 1e-4
BF16_REL = 2e-2


def to_device(inp, device="cuda"):
    import torch
    if inp.dtype == "fp32":
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return dict(enc=conv(inp.enc), pred=conv(inp.pred), W_out=conv(inp.W), b_out=conv(inp.b),
                labels=i32(inp.labels), T_lens=i32(inp.T_lens), U_lens=i32(inp.U_lens))


def run_gpu(inp, tile_t=0, tile_u=0, tile_v=0, grad_costs=None, dev=None, bwd=True,
            criterion="sum"):
    import torch
    import rnn_joint_transducer_amd as rj
    dev = dev or to_device(inp)
    costs, saved = rj.rnnt_joint_loss_fwd(**dev, blank=inp.blank, tile_t=tile_t,
                                          tile_u=tile_u, tile_v=tile_v, criterion=criterion)
    out = dict(costs=costs)
    if bwd:
        gc = None if grad_costs is None else torch.tensor(grad_costs, dtype=torch.float32,
                                                          device=costs.device)
        d_enc, d_pred, d_W, d_b = rj.rnnt_joint_loss_bwd(**dev, saved=saved, blank=inp.blank,
                                                         tile_t=tile_t, tile_u=tile_u,
                                                         tile_v=tile_v, grad_costs=gc)
        out.update(dEnc=d_enc, dPred=d_pred, dW=d_W, db=d_b)
    out["status"] = rj.rnnt_joint_loss_status(saved)
    return {k: (v.cpu().double().numpy() if hasattr(v, "cpu") else v) for k, v in out.items()}


def check_costs(gpu, ref, dtype, idx=None):
    idx = range(len(ref)) if idx is None else idx
    tol = FP32_LOSS_REL if dtype == "fp32" else BF16_REL
    worst = 0.0
    for k, b in enumerate(idx):
        r = abs(gpu[b] - ref[k]) / abs(ref[k])
        worst = max(worst, r)
        assert r <= tol, f"utt {b}: gpu {gpu[b]} oracle {ref[k]} rel {r:.3e} > {tol}"
    return worst


def check_grad(name, gpu, ref, dtype):
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    if dtype == "fp32":
        assert err <= FP32_GRAD_ABS, f"{name}: max abs err {err:.3e} > {FP32_GRAD_ABS}"
        return err
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel = err / scale if scale > 0 else err
    assert rel <= BF16_REL, f"{name}: rel err {rel:.3e} > {BF16_REL} (abs {err:.3e})"
    return rel


def _loss_only_job(args):
    """One utterance's cost from the oracle (process-pool worker)."""
    enc_b, pred_b, W, b_out, y, Tl, Ul, blank, threads, criterion = args
    from oracle import rnnt
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads):
        return float(rnnt.loss_only(enc_b[None], pred_b[None], W, b_out, y[None],
                                    np.array([Tl]), np.array([Ul]), blank,
                                    criterion=criterion)[0])


def oracle_costs(inp, utts, workers, criterion="sum"):
    """Oracle costs of the given utterances, one process per utterance (spawned:
    the calling process may hold a GPU runtime)."""
    import multiprocessing
    import os
    from concurrent.futures import ProcessPoolExecutor
    utts = list(utts)
    workers = max(1, min(workers, len(utts)))
    threads = max(1, (os.cpu_count() or 1) // workers)
    jobs = [(inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64, inp.labels[b],
             int(inp.T_lens[b]), int(inp.U_lens[b]), inp.blank, threads, criterion)
            for b in utts]
    if workers == 1:
        return [_loss_only_job(j) for j in jobs]
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        return list(ex.map(_loss_only_job, jobs))


def _pruned_job(args):
    """One utterance of the pruned-loss oracle (process-pool worker)."""
    enc_b, pred_b, W, b_out, y, Tl, Ul, blank, S, gc, want, threads = args
    from oracle import pruned
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads):
        o = pruned.utterance(enc_b[:Tl], pred_b[:Ul + 1], W, b_out, y, Tl, Ul, blank, S,
                             grad_cost=gc, want_grads=want)
    keep = ("cost", "simple_cost", "bounds", "centres", "feasible", "dEnc", "dPred", "dW", "db")
    return {k: o[k] for k in keep if k in o}


def pruned_oracle(inp, S, utts, workers, grad_costs=None, want_grads=True):
    """Per-utterance pruned-loss oracle results (dicts), one process each."""
    import multiprocessing
    import os
    from concurrent.futures import ProcessPoolExecutor
    utts = list(utts)
    gcs = np.ones(inp.B) if grad_costs is None else np.asarray(grad_costs, np.float64)
    workers = max(1, min(workers, len(utts)))
    threads = max(1, (os.cpu_count() or 1) // workers)
    jobs = [(inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64, inp.labels[b],
             int(inp.T_lens[b]), int(inp.U_lens[b]), inp.blank, S, float(gcs[b]), want_grads,
             threads) for b in utts]
    if workers == 1:
        return [_pruned_job(j) for j in jobs]
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        return list(ex.map(_pruned_job, jobs))


def _tdt_job(args):
    """One utterance of the token-and-duration oracle (process-pool worker)."""
    enc_b, pred_b, W, b_out, Wd, bd, y, Tl, Ul, blank, durs, gc, want, threads = args
    from oracle import tdt
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=threads):
        o = tdt.utterance(enc_b[:Tl], pred_b[:Ul + 1], W, b_out, Wd, bd, y, Tl, Ul, blank, durs,
                          grad_cost=gc, want_grads=want)
    keep = ("cost", "dEnc", "dPred", "dW", "db", "dWd", "dbd")
    return {k: o[k] for k in keep if k in o}


def tdt_oracle(inp, head, utts, workers, grad_costs=None, want_grads=True):
    """Per-utterance token-and-duration oracle results, one process each."""
    import multiprocessing
    import os
    from concurrent.futures import ProcessPoolExecutor
    utts = list(utts)
    gcs = np.ones(inp.B) if grad_costs is None else np.asarray(grad_costs, np.float64)
    workers = max(1, min(workers, len(utts)))
    threads = max(1, (os.cpu_count() or 1) // workers)
    jobs = [(inp.enc_f64[b], inp.pred_f64[b], inp.W_f64, inp.b_f64, head.W_dur_f64,
             head.b_dur_f64, inp.labels[b], int(inp.T_lens[b]), int(inp.U_lens[b]), inp.blank,
             head.durations, float(gcs[b]), want_grads, threads) for b in utts]
    if workers == 1:
        return [_tdt_job(j) for j in jobs]
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        return list(ex.map(_tdt_job, jobs))
