"""Benchmark of the fused RNN-T joint + transducer loss (forward + backward).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]
                    [--tile-t T --tile-u U --tile-v V] [--no-cpu-baseline]
    python bench.py --sweep --workload medium --steps 3 --warmup 1

One step = one forward + one backward over a whole synthetic batch (every
kernel of the path: validation, W_out transpose, fused joint + projection +
online log-sum-exp, lattice recursions, logit gradients, the dh and dW GEMMs
and the lattice reductions), with the inputs already resident in HBM and all
output / state buffers allocated once before timing.  The line printed is

    value = B*T*U lattice cells of the workload per second (padded maxima,
            the metric's definition), whole job, one GPU.

`roofline` describes the kernel with the largest share of step time: its
algorithmic flops (2*H*V per valid lattice cell for each MFMA pass) or bytes
per launch over its mean launch duration, measured with HIP events that the
library records on the launch stream around each of its kernels.
`cpu_baseline` times the float64 oracle on a bounded sample of the same
workload on the host cores and scales it to the same unit.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "lattice cells/sec (B·T·U) fused joint+loss fwd+bwd"
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0
PEAK_F64 = 78.6  # TFLOP/s, float64 MFMA (dense) = float64 vector: 256 CUs x 4 SIMDs x 16 lanes x 2 x 2.4 GHz
MFMA_KERNELS = ("joint_fwd", "joint_fwd_store", "joint_grad", "dh", "dw")
PROJ_KERNELS = ("proj_fwd", "proj_dx", "proj_dw")
# Tiled defaults: medium takes the lowest-memory tiling within 95 % of the
# best tiled throughput of a full tile sweep (`--sweep`, overlapped chunk
# schedule: 64 frames x all label positions); medium_lv keeps its
# configured vocabulary parts of 256 columns and takes the same choice among
# the tilings with those parts (chunks of all frames x 64 label positions);
# long keeps its configured 64 x 64 chunks (over the whole vocabulary: the
# long configuration fixes no tile_v).
DEFAULT_TILES = {"tiny": (0, 0, 0), "short": (0, 0, 0), "medium": (64, 0, 0),
                 "medium_lv": (0, 64, 256), "long": (64, 64, 0)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long",
                    choices=["tiny", "short", "medium", "medium_lv", "long"])
    ap.add_argument("--criterion", default="sum", choices=["sum", "max"],
                    help="full sum over alignments, or the best alignment only")
    ap.add_argument("--proj", default=None, metavar="E,P",
                    help="put joint input projections (enc: E -> H, pred: P -> H) in front of the "
                         "joint, their gradients after it, inside the timed step")
    ap.add_argument("--pruned", type=int, default=0, metavar="S",
                    help="time the pruned transducer loss with windows of S label positions "
                         "(tiled mode) instead of the full lattice")
    ap.add_argument("--tdt", default=None, metavar="D0,D1,...",
                    help="time the token-and-duration transducer loss with these durations "
                         "(duration head from synth.make_duration_head, seed 1)")
    ap.add_argument("--tile-t", type=int, default=None)
    ap.add_argument("--tile-u", type=int, default=None)
    ap.add_argument("--tile-v", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-workspace", action="store_true",
                    help="give the backward its least workspace (one chunk buffer pair: every "
                         "kernel in order on one stream) instead of the size for the "
                         "overlapped chunk schedule")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--sweep", action="store_true",
                    help="time the tile grid (tile_t, tile_u in 16, 32, 64, 128, 0; tile_v in "
                         "128, 256, 512, 0) instead of one configuration and print the "
                         "throughput-memory frontier")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run 5 plain device-to-device copies of BYTES bytes (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def kernel_source_digest():
    """sha256 over the HIP/C++ sources of the library (sorted by name)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "rnn_joint_transducer_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(workload, kernel, mode, criterion="sum"):
    """HBM bytes per launch recorded in profiles/traffic.json by rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the copy calibration), or None
    when no entry exists or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        entries = json.load(open(path))["entries"]
    except (OSError, ValueError, KeyError):
        return None
    digest = kernel_source_digest()
    for e in entries:
        if (e.get("workload") == workload and e.get("kernel") == kernel
                and e.get("mode") == mode and e.get("criterion", "sum") == criterion
                and e.get("source_sha256") == digest):
            return e.get("bytes_per_launch")
    return None


def calibrate_copy(nbytes):
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 5}))


def cpu_baseline(inp, target_s, criterion="sum", pj=None, pruned_S=0, head=None):
    """Float64 oracle (fwd+bwd, one utterance at a time, NumPy BLAS on all host
    threads) on a bounded sample of the workload: whole utterances in order
    until about target_s seconds are spent (whole passes over the batch
    repeated while a pass takes less), or the first utterance cut to its
    first t_s frames when even one utterance would take longer (t_s from a
    4-frame pilot).  Scaled to B*T*U cells/s of the whole workload by the
    ratio of valid lattice cells."""
    import numpy as np
    from oracle import rnnt
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    nproc = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cpu_model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass

    def run(b, t_s):
        t0 = time.perf_counter()
        if head is not None:
            from oracle import tdt
            tdt.utterance(inp.enc_f64[b, :t_s], inp.pred_f64[b], inp.W_f64, inp.b_f64,
                          head.W_dur_f64, head.b_dur_f64, inp.labels[b], t_s, int(inp.U_lens[b]),
                          inp.blank, head.durations)
        elif pruned_S:
            from oracle import pruned
            pruned.utterance(inp.enc_f64[b, :t_s], inp.pred_f64[b], inp.W_f64, inp.b_f64,
                             inp.labels[b], t_s, int(inp.U_lens[b]), inp.blank, pruned_S)
        elif pj is None:
            rnnt.utterance_loss_and_grads(inp.enc_f64[b, :t_s], inp.pred_f64[b], inp.W_f64,
                                          inp.b_f64, inp.labels[b], t_s, int(inp.U_lens[b]),
                                          inp.blank, criterion=criterion)
        else:
            from oracle import proj
            ep = proj.linear(pj.enc_in_f64[b, :t_s], pj.W_enc_f64, pj.b_enc_f64)
            pp = proj.linear(pj.pred_in_f64[b], pj.W_pred_f64, pj.b_pred_f64)
            o = rnnt.utterance_loss_and_grads(ep, pp, inp.W_f64, inp.b_f64, inp.labels[b], t_s,
                                              int(inp.U_lens[b]), inp.blank, criterion=criterion)
            proj.linear_grads(pj.enc_in_f64[b, :t_s], pj.W_enc_f64, o["dEnc"])
            proj.linear_grads(pj.pred_in_f64[b, :o["dPred"].shape[0]], pj.W_pred_f64, o["dPred"])
        return time.perf_counter() - t0

    Tl0, Ul0 = int(inp.T_lens[0]), int(inp.U_lens[0])
    pilot_t = min(Tl0, 4)
    pt = run(0, pilot_t)
    if pt * Tl0 / pilot_t > target_s:
        t_s = int(min(Tl0, max(pilot_t, round(pilot_t * target_s / max(pt, 1e-6)))))
        el = run(0, t_s)
        sample_cells = t_s * (Ul0 + 1)
        desc = f"utterance 0 (T'={Tl0}, U'={Ul0}) cut to its first {t_s} frames"
    else:
        el, sample_cells, nb, full, extra = 0.0, 0, 0, 0, 0
        while el < target_s:
            done = 0
            for b in range(inp.B):
                el += run(b, int(inp.T_lens[b]))
                sample_cells += int(inp.T_lens[b]) * (int(inp.U_lens[b]) + 1)
                nb = max(nb, b + 1)
                done += 1
                if el >= target_s:
                    break
            if done == inp.B:
                full += 1
            else:
                extra = done
        if full == 0:
            desc = f"utterances 0..{nb - 1} of {inp.B} in full"
        else:
            desc = f"{full} full pass{'es' if full > 1 else ''} over all {inp.B} utterances" + (
                f" and utterances 0..{extra - 1} once more" if extra else "")
    total_valid = int(np.sum(inp.T_lens.astype(np.int64) * (inp.U_lens.astype(np.int64) + 1)))
    full_time = el * total_valid / sample_cells
    value = inp.B * inp.T * inp.U / full_time
    return {"value": value, "unit": "cells/s", "cores": int(threads), "kind": "oracle",
            "nproc": int(nproc or 1), "cpu_model": cpu_model,
            "numpy": np.__version__,
            "sample": f"{desc}: {sample_cells} valid cells in {el:.2f} s, float64 NumPy "
                      f"fwd+bwd{'' if pj is None else ' with the input projections'}"
                      f"{'' if not pruned_S else f' (pruned loss, S={pruned_S})'}"
                      f"{'' if head is None else f' (token-and-duration loss, durations {head.durations})'}, scaled by "
                      f"valid cells ({total_valid}) to the B*T*U metric"}


def tile_sweep(args, rj, torch, tensors, inp, dev, dc):
    """Throughput and memory over the tile grid: tile_t, tile_u in {16, 32, 64,
    128, 0} (0: the whole axis; both 0: the untiled mode) and tile_v in {128,
    256, 512, 0}.  Memory is the peak allocated above the inputs in one
    fwd+bwd (saved state, workspace, costs and gradients).  Prints one JSON
    line: every configuration, the throughput-memory frontier (no other
    configuration is both faster and smaller), and per mode the
    lowest-memory configuration within 95 % of that mode's best throughput."""
    B, T, U, H, V = inp.B, inp.T, inp.U, inp.H, inp.V
    costs = torch.empty(B, dtype=torch.float32, device=dev)
    grads = (torch.empty(B, T, H, device=dev), torch.empty(B, U + 1, H, device=dev),
             torch.empty(H, V, device=dev), torch.empty(V, device=dev))
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated(dev) - sum(
        t.numel() * t.element_size() for t in (costs, *grads))
    rows = []
    for tt in (16, 32, 64, 128, 0):
        for tu in (16, 32, 64, 128, 0):
            for tv in (128, 256, 512, 0):
                torch.cuda.synchronize()
                torch.cuda.reset_peak_memory_stats(dev)
                saved = torch.empty(rj.rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tt, tu, tv),
                                    dtype=torch.uint8, device=dev)
                ws = torch.empty(rj.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, tt, tu,
                                                                     tv, ws_pass(args)),
                                 dtype=torch.uint8, device=dev)

                def step():
                    rj.rnnt_joint_loss_fwd(**tensors, tile_t=tt, tile_u=tu, tile_v=tv,
                                           costs=costs, saved=saved)
                    rj.rnnt_joint_loss_bwd(**tensors, saved=saved, tile_t=tt, tile_u=tu,
                                           tile_v=tv, workspace=ws, out=grads)

                for _ in range(max(1, args.warmup)):
                    step()
                torch.cuda.synchronize()
                gb = (torch.cuda.max_memory_allocated(dev) - base) / 1e9
                status = rj.rnnt_joint_loss_status(saved)
                ev0 = torch.cuda.Event(enable_timing=True)
                ev1 = torch.cuda.Event(enable_timing=True)
                ev0.record()
                for _ in range(args.steps):
                    step()
                ev1.record()
                torch.cuda.synchronize()
                ms = ev0.elapsed_time(ev1) / args.steps
                mode = "untiled" if (tt == 0 and tu == 0) else "tiled"
                rows.append({"mode": mode, "tile_t": tt, "tile_u": tu, "tile_v": tv,
                             "ms_per_step": round(ms, 4),
                             "cells_per_s": B * T * U / (ms / 1e3), "gb_above_inputs": round(gb, 4),
                             "status": status})
                print(f"# sweep {mode:7s} tile_t={tt:3d} tile_u={tu:3d} tile_v={tv:3d}: "
                      f"{ms:9.3f} ms/step, {gb:7.3f} GB above inputs, status {status}",
                      file=sys.stderr, flush=True)
                del saved, ws

    def dominated(r):
        return any(o["ms_per_step"] <= r["ms_per_step"] and o["gb_above_inputs"] <= r["gb_above_inputs"]
                   and (o["ms_per_step"] < r["ms_per_step"] or o["gb_above_inputs"] < r["gb_above_inputs"])
                   for o in rows)

    frontier = sorted((r for r in rows if not dominated(r)), key=lambda r: r["gb_above_inputs"])
    pick = {}
    for mode in ("untiled", "tiled"):
        rs = [r for r in rows if r["mode"] == mode and r["status"] == 0]
        best = min(r["ms_per_step"] for r in rs)
        pick[mode] = min((r for r in rs if best / r["ms_per_step"] >= 0.95),
                         key=lambda r: (r["gb_above_inputs"], r["ms_per_step"]))
    print(json.dumps({"metric": METRIC, "workload": args.workload, "steps": args.steps,
                      "warmup": max(1, args.warmup), "data": "synthetic", "sweep": rows,
                      "frontier": frontier, "lowest_memory_within_95pct": pick}), flush=True)


def ws_pass(args):
    """Backward workspace query: 1 = the overlapped chunk schedule, 2 = the least."""
    return 2 if args.min_workspace else 1


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over utterances across GPUs by design, but multi-GPU runs are "
              "not part of it", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import rnn_joint_transducer_amd as rj
    from rnn_joint_transducer_amd import _lib
    from synth import make_config, make_proj_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_config(args.workload)
    tt, tu, tv = DEFAULT_TILES[args.workload]
    tt = tt if args.tile_t is None else args.tile_t
    tu = tu if args.tile_u is None else args.tile_u
    tv = tv if args.tile_v is None else args.tile_v
    bf16 = inp.dtype == "bf16"
    dt = "bf16" if bf16 else "f32"

    def conv(a):
        if bf16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    tensors = dict(enc=conv(inp.enc), pred=conv(inp.pred), W_out=conv(inp.W), b_out=conv(inp.b),
                   labels=i32(inp.labels), T_lens=i32(inp.T_lens), U_lens=i32(inp.U_lens))
    B, T, U, H, V = inp.B, inp.T, inp.U, inp.H, inp.V
    pj = None
    if args.proj:
        E, P = (int(x) for x in args.proj.split(","))
        pj = make_proj_inputs(inp, E, P, seed=1)
        ptens = dict(enc_in=conv(pj.enc_in), pred_in=conv(pj.pred_in), W_enc=conv(pj.W_enc),
                     b_enc=conv(pj.b_enc), W_pred=conv(pj.W_pred), b_pred=conv(pj.b_pred))
    dc = rj.RNNTJ_BF16 if bf16 else rj.RNNTJ_F32
    if args.sweep:
        tile_sweep(args, rj, torch, tensors, inp, dev, dc)
        return
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base_mem = torch.cuda.memory_allocated(dev)
    saved = torch.empty(rj.rnnt_joint_loss_saved_bytes(B, T, U, H, V, dc, tt, tu, tv),
                        dtype=torch.uint8, device=dev)
    wsb = rj.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, tt, tu, tv, ws_pass(args))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    costs = torch.empty(B, dtype=torch.float32, device=dev)
    grads = (torch.empty(B, T, H, device=dev), torch.empty(B, U + 1, H, device=dev),
             torch.empty(H, V, device=dev), torch.empty(V, device=dev))

    head = None
    if args.tdt:
        from synth import make_duration_head
        head = make_duration_head(inp, tuple(int(x) for x in args.tdt.split(",")), seed=1)
        Wd, bd = conv(head.W_dur), conv(head.b_dur)
        K = len(head.durations)
        import ctypes
        sz = ctypes.c_size_t(0)
        _lib.check(_lib.load().rnnt_joint_loss_tdt_saved_bytes(B, T, U, H, V, dc, tt, tu, tv, K,
                                                               ctypes.byref(sz)), "tdt_saved")
        saved = torch.empty(sz.value, dtype=torch.uint8, device=dev)
        _lib.check(_lib.load().rnnt_joint_loss_tdt_workspace_bytes(B, T, U, H, V, dc, tt, tu, tv,
                                                                   K, ws_pass(args),
                                                                   ctypes.byref(sz)),
                   "tdt_ws")
        ws = torch.empty(sz.value, dtype=torch.uint8, device=dev)
    if args.pruned:
        if tt == 0 and tu == 0:
            sys.exit("bench.py: the pruned loss runs in the tiled mode (give --tile-t/--tile-u)")
        pws = torch.empty(rj.rnnt_joint_loss_pruned_workspace_bytes(B, T, U, H, V, dc),
                          dtype=torch.uint8, device=dev)
        simple = torch.empty(B, dtype=torch.float32, device=dev)

    def step(wsx=None):
        wsx = ws if wsx is None else wsx
        if pj is not None:
            tensors["enc"] = rj.rnnt_joint_proj_fwd(ptens["enc_in"], ptens["W_enc"], ptens["b_enc"])
            tensors["pred"] = rj.rnnt_joint_proj_fwd(ptens["pred_in"], ptens["W_pred"],
                                                     ptens["b_pred"])
        if head is not None:
            rj.rnnt_joint_loss_tdt_fwd(**tensors, W_dur=Wd, b_dur=bd, durations=head.durations,
                                       tile_t=tt, tile_u=tu, tile_v=tv, costs=costs, saved=saved)
            rj.rnnt_joint_loss_tdt_bwd(**tensors, W_dur=Wd, b_dur=bd, durations=head.durations,
                                       saved=saved, tile_t=tt, tile_u=tu, tile_v=tv, workspace=wsx)
            return
        if args.pruned:
            rj.rnnt_joint_loss_pruned_fwd(**tensors, S=args.pruned, tile_t=tt, tile_u=tu,
                                          tile_v=tv, costs=costs, simple_costs=simple,
                                          saved=saved, workspace=pws)
        else:
            rj.rnnt_joint_loss_fwd(**tensors, tile_t=tt, tile_u=tu, tile_v=tv, costs=costs,
                                   saved=saved, criterion=args.criterion)
        rj.rnnt_joint_loss_bwd(**tensors, saved=saved, tile_t=tt, tile_u=tu, tile_v=tv,
                               workspace=wsx, out=grads)
        if pj is not None:
            rj.rnnt_joint_proj_bwd(ptens["enc_in"], ptens["W_enc"], grads[0])
            rj.rnnt_joint_proj_bwd(ptens["pred_in"], ptens["W_pred"], grads[1])

    mode_tiled = not (tt == 0 and tu == 0)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    peak_gb = torch.cuda.max_memory_allocated(dev) / 1e9
    extra_gb = (torch.cuda.max_memory_allocated(dev) - base_mem) / 1e9
    status = rj.rnnt_joint_loss_status(saved)

    # one event between consecutive steps: the mean over the K steps gives
    # ms_per_step and value, the per-step spans give the median and p10 / p90
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    spans = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    pct = lambda q: float(np.percentile(spans, q))
    value = B * T * U / (ms / 1e3)
    print(f"# {args.workload}: {ms:.3f} ms/step (wall {wall / args.steps * 1e3:.3f}; median "
          f"{pct(50):.3f}, p10 {pct(10):.3f}, p90 {pct(90):.3f}), {value:.4g} cells/s, "
          f"peak {peak_gb:.2f} GB, status {status}", file=sys.stderr, flush=True)

    # per-kernel durations from HIP events recorded by the library on its stream
    _lib.timing(True)
    kin = max(1, min(args.steps, 10))
    for _ in range(kin):
        step()
    torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.timing(False)
    # In the overlapped chunk schedule the launches above share the compute
    # units with the side stream's dW, so their durations include shared
    # time.  Two more steps with the least workspace (every kernel in order
    # on one stream) give each kernel's duration alone.
    rep_alone = None
    if mode_tiled and not args.min_workspace:
        if head is not None:
            import ctypes
            sz = ctypes.c_size_t(0)
            _lib.check(_lib.load().rnnt_joint_loss_tdt_workspace_bytes(
                B, T, U, H, V, dc, tt, tu, tv, len(head.durations), 2, ctypes.byref(sz)), "tdt_ws")
            least = sz.value
        else:
            least = rj.rnnt_joint_loss_workspace_bytes(B, T, U, H, V, dc, tt, tu, tv, 2)
        ws_least = ws[:least]
        step(ws_least)
        torch.cuda.synchronize()
        _lib.timing(True)
        for _ in range(2):
            step(ws_least)
        torch.cuda.synchronize()
        rep_alone = _lib.timing_report()
        _lib.timing(False)
    valid = int(np.sum(inp.T_lens.astype(np.int64) * (inp.U_lens.astype(np.int64) + 1)))
    band_cells = None
    if args.pruned:
        # cells of the band: the joint's algorithmic work in the pruned loss
        bd = rj.rnnt_joint_loss_pruned_bounds(saved, B, T, U, H, V, dc, tt, tu, tv).cpu().numpy()
        band_cells = 0
        for b in range(B):
            Tl, Ul = int(inp.T_lens[b]), int(inp.U_lens[b])
            s0 = bd[b, :Tl].astype(np.int64)
            band_cells += int(np.sum(np.minimum(s0 + args.pruned - 1, Ul) - s0 + 1))
    work_cells = band_cells if band_cells is not None else valid
    kernels = {}
    for name, (n, tot) in rep.items():
        per_launch_ms = tot / n
        k = {"launches_per_step": n / kin, "ms_per_step": tot / kin, "ms_per_launch": per_launch_ms}
        if name in MFMA_KERNELS:
            flops_step = 2.0 * H * V * work_cells
            k["tflops"] = flops_step / (tot / kin / 1e3) / 1e12
        elif name in PROJ_KERNELS and pj is not None:
            # each of the three products: 2 * rows * in_width * H per projection
            flops_step = 2.0 * H * (B * T * pj.E + B * (U + 1) * pj.P)
            k["tflops"] = flops_step / (tot / kin / 1e3) / 1e12
        kernels[name] = k
        print(f"#   {name:16s} {n / kin:5.1f} launches/step {tot / kin:9.4f} ms/step", file=sys.stderr)
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    launches = kd["launches_per_step"]
    if dom in MFMA_KERNELS:
        per_launch = 2.0 * H * V * work_cells / launches
        achieved = per_launch / (kd["ms_per_launch"] / 1e3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[dt],
                "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS[dt], "traffic": None,
                "algorithmic_per_launch": per_launch}
    elif dom == "pruning_bounds":
        # float64 products on the MFMA units: am = enc W_out and lm = pred W_out
        # over the valid rows (2 H V flops per row), and the normaliser
        # product EA EL^T of every utterance (2 V flops per valid cell); the
        # group also holds the simple lattice and the window bounds
        rows = int(np.sum(inp.T_lens.astype(np.int64) + inp.U_lens.astype(np.int64) + 1))
        per_launch = (2.0 * H * V * rows + 2.0 * V * valid) / launches
        achieved = per_launch / (kd["ms_per_launch"] / 1e3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_F64,
                "unit": "TFLOP/s", "frac": achieved / PEAK_F64, "traffic": None,
                "algorithmic_per_launch": per_launch}
    else:
        # lattice: 32 B per valid cell (alpha and beta chains each read LB, LE and
        # write one float64); token-and-duration lattice: the same plus the K
        # float32 duration log-probabilities read by each chain; grad_inplace:
        # read + write the logits
        elem = 2 if bf16 else 4
        if dom == "lattice":
            per_cell = 32.0
        elif dom == "tdt_lattice":
            per_cell = 32.0 + 8.0 * len(args.tdt.split(","))
        elif dom == "grad_inplace":
            per_cell = 2.0 * elem * V
        else:
            per_cell = 0.0
        per_launch = per_cell * valid / launches
        achieved = per_launch / (kd["ms_per_launch"] / 1e3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_per_launch": per_launch}

    mode = "untiled" if (tt == 0 and tu == 0) else "tiled"
    roof["traffic"] = measured_traffic(args.workload, dom, mode, args.criterion)
    alone = None
    if rep_alone is not None:
        alone = {"schedule": "least workspace: every kernel in order on one stream, 2 steps"}
        for name, (n, tot) in rep_alone.items():
            if name in MFMA_KERNELS:
                per_launch = 2.0 * H * V * work_cells / (n / 2.0)
                tf = per_launch / (tot / n / 1e3) / 1e12
                alone[name] = {"ms_per_launch": round(tot / n, 6), "tflops": round(tf, 2),
                               "frac": round(tf / PEAK_TFLOPS[dt], 4)}
    # the whole step against the matrix peak: the joint projection's
    # algorithmic flops (forward 2HV, dh 2HV, dW 2HV per cell) and those the
    # kernels execute (the tiled backward recomputes the forward's 2HV), over
    # the step time (kernels on the side stream overlap the others, so the
    # per-kernel rates above do not add up to this)
    n_mm = sum(1 for k in ("joint_fwd", "joint_fwd_store", "joint_grad", "dh", "dw")
               if k in kernels)
    useful = 6.0 * H * V * work_cells
    executed = 2.0 * H * V * work_cells * n_mm
    step_mfma = {"useful_tflops": useful / (ms / 1e3) / 1e12,
                 "executed_tflops": executed / (ms / 1e3) / 1e12, "peak": PEAK_TFLOPS[dt]}
    step_mfma["useful_frac"] = step_mfma["useful_tflops"] / PEAK_TFLOPS[dt]
    step_mfma["executed_frac"] = step_mfma["executed_tflops"] / PEAK_TFLOPS[dt]
    # the lattice pass against HBM peak (32 B per valid cell: the alpha and beta
    # chains each read LB, LE and write one float64) and per anti-diagonal step
    lat = None
    if "lattice" in kernels:
        kl = kernels["lattice"]
        diags = int(np.max(inp.T_lens.astype(np.int64) + inp.U_lens))
        gbs = 32.0 * valid / kl["launches_per_step"] / (kl["ms_per_launch"] / 1e3) / 1e9
        lat = {"ms_per_launch": kl["ms_per_launch"], "gb_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
               "bytes_per_valid_cell": 32, "diagonals": diags,
               "us_per_diagonal": kl["ms_per_launch"] * 1e3 / diags}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds, args.criterion, pj, args.pruned, head)

    line = {
        "metric": METRIC, "value": value, "unit": "cells/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "ms_median": pct(50), "ms_p10": pct(10), "ms_p90": pct(90),
        "config": {"workload": args.workload, "B": B, "T": T, "U": U, "H": H, "V": V,
                   "mode": mode, "criterion": args.criterion,
                   "proj": None if pj is None else {"E": pj.E, "P": pj.P},
                   "pruned_S": args.pruned or None, "band_cells": band_cells,
                   "tdt_durations": None if head is None else list(head.durations),
                   "tile_t": tt, "tile_u": tu, "tile_v": tv,
                   "workspace": "least" if args.min_workspace else "overlapped",
                   "valid_cells": valid, "valid_cells_per_s": valid / (ms / 1e3),
                   "peak_gb": round(peak_gb, 3), "peak_gb_above_inputs": round(extra_gb, 3)},
        "roofline": roof,
        "kernels_alone": alone,
        "step_mfma": step_mfma,
        "lattice": lat,
        "kernels": {k: {kk: round(vv, 6) for kk, vv in v.items()} for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
