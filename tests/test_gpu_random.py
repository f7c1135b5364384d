"""GPU parity on seeded random shapes.

Each case draws, from its own seed, the batch size, the padded and actual
lengths (single frames and utterances without labels included), hidden and
vocabulary sizes, the blank index (first, last or inside the vocabulary), a
nonzero output bias, the weight scale (every fourth case, odd seeds: bf16,
large logits in the untiled mode), the tiling (untiled, or tiled with or without a
vocabulary bound), the dtype, the criterion and signed cost weights.  Every
output is compared with the float64 oracle, element by element.  Each case
prints its parameters before it runs.
"""
import os

import numpy as np
import pytest

import oracle
from synth import _cast, make_inputs

from gpu_common import check_costs, check_grad, run_gpu

pytestmark = pytest.mark.gpu

WORKERS = min(16, os.cpu_count() or 1)


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = "fp32" if seed % 2 == 0 else "bf16"
    criterion = "max" if seed % 4 == 3 else "sum"
    B = int(rng.integers(1, 6))
    T = int(rng.integers(1, 71))
    U = int(rng.integers(0, 21))
    H = 16 * int(rng.integers(1, (256 if dtype == "fp32" else 384) // 16 + 1))
    V = 8 * int(rng.integers(1, 65))
    blank = [0, V - 1, int(rng.integers(0, V))][seed % 3]
    # every fourth case draws large weights (logits of size ~10-40)
    sigma = 1.5 if seed % 4 == 1 else 0.3
    inp = make_inputs(B, T, U, H, V, dtype=dtype, sigma=sigma, seed=2000 + seed, blank=blank,
                      t_range=(1, T), u_range=(0, U))
    # labels anywhere in the vocabulary except the blank
    lab = rng.integers(0, V - 1, size=(B, U))
    inp.labels = (lab + (lab >= blank)).astype(np.int32)
    inp.b, inp.b_f64 = _cast(rng.normal(0.0, 0.3, V), dtype)
    if rng.random() < 0.4 or sigma > 1.0:
        tiles = (0, 0, 0)
    else:
        tiles = (16 * int(rng.integers(0, 4)), 8 * int(rng.integers(0, 3)),
                 [0, 128, 256][int(rng.integers(0, 3))])
        if tiles[0] == 0 and tiles[1] == 0:
            tiles = (16, tiles[1], tiles[2])
    gcs = rng.uniform(-1.0, 1.0, B)
    return inp, tiles, criterion, gcs


@pytest.mark.parametrize("seed", range(32))
def test_random_shapes(seed):
    inp, tiles, criterion, gcs = _case(seed)
    print(f"[random seed={seed} {inp.dtype} {criterion} B={inp.B} T={inp.T} U={inp.U} "
          f"H={inp.H} V={inp.V} blank={inp.blank} tiles={tiles} T'={list(inp.T_lens)} "
          f"U'={list(inp.U_lens)}]", flush=True)
    g = run_gpu(inp, *tiles, grad_costs=gcs, criterion=criterion)
    assert g["status"] == 0
    ref = oracle.loss_and_grads(inp.enc_f64, inp.pred_f64, inp.W_f64, inp.b_f64, inp.labels,
                                inp.T_lens, inp.U_lens, inp.blank, grad_costs=gcs,
                                workers=min(WORKERS, inp.B), criterion=criterion)
    check_costs(g["costs"], ref["costs"], inp.dtype)
    check_grad("d_enc", g["dEnc"], ref["dEnc"], inp.dtype)
    check_grad("d_pred", g["dPred"], ref["dPred"], inp.dtype)
    check_grad("d_W_out", g["dW"], ref["dW"], inp.dtype)
    check_grad("d_b_out", g["db"], ref["db"], inp.dtype)
