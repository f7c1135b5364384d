"""Seeded synthetic inputs for the fused RNN-T joint + transducer loss.

This module only draws and casts numbers; it holds none of the method's
arithmetic.  Both the float64 oracle (through the tests) and the HIP path
(through the tests and the benchmark) read the arrays it returns, so the two
sides always see bit-identical values.

Recipe (one fixed draw order per call, ``numpy.random.default_rng(seed)``):

1. ``enc``   [B, T, H]    ~ N(0, sigma)   (sigma is the standard deviation)
2. ``pred``  [B, U+1, H]  ~ N(0, sigma)
3. ``W_out`` [H, V]       ~ N(0, sigma)
4. ``T_lens`` [B]  integers uniform in [t_lo, t_hi] (inclusive), unless full
5. ``U_lens`` [B]  integers uniform in [u_lo, u_hi] (inclusive), unless full
6. ``labels`` [B, U] integers in [1, V): uniform, or Zipf(s) by inverse CDF
   with p(k) proportional to k**-s on k = 1..V-1.
``b_out`` is zero.  Values are drawn in float64 and then cast to the storage
dtype (float32, or bfloat16 with round-to-nearest-even); ``*_f64`` hold the
exact cast values upcast to float64.  Rows past an utterance's lengths hold
ordinary random values and labels past U' are random too: they are padding
that must not influence any result.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["CONFIGS", "Inputs", "make_inputs", "make_config", "to_bf16_bits",
           "bf16_bits_to_f64", "make_duration_head"]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN stays NaN (quiet)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    out = ((u + rounding) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """One batch.  ``enc``/``pred``/``W``/``b`` are storage arrays (float32 or
    uint16 bf16 bits); the ``*_f64`` twins hold the same values in float64."""
    name: str
    dtype: str            # "fp32" or "bf16"
    B: int
    T: int
    U: int
    H: int
    V: int
    blank: int
    enc: np.ndarray
    pred: np.ndarray
    W: np.ndarray
    b: np.ndarray
    labels: np.ndarray    # int32 [B, U]
    T_lens: np.ndarray    # int32 [B]
    U_lens: np.ndarray    # int32 [B]
    enc_f64: np.ndarray
    pred_f64: np.ndarray
    W_f64: np.ndarray
    b_f64: np.ndarray
    mode: str = "T"
    tile_t: int = 0
    tile_u: int = 0
    tile_v: int = 0

    @property
    def cells_btu(self) -> int:
        return self.B * self.T * self.U

    @property
    def valid_cells(self) -> int:
        return int(np.sum(self.T_lens.astype(np.int64) * (self.U_lens.astype(np.int64) + 1)))


def _cast(x64: np.ndarray, dtype: str):
    if dtype == "fp32":
        s = x64.astype(np.float32)
        return s, s.astype(np.float64)
    if dtype == "bf16":
        bits = to_bf16_bits(x64)
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(f"unknown dtype {dtype!r}")


def _zipf_labels(rng, shape, V, s):
    k = np.arange(1, V, dtype=np.float64)
    p = k ** (-s)
    cdf = np.cumsum(p / p.sum())
    cdf[-1] = 1.0
    r = rng.random(size=shape)
    idx = np.searchsorted(cdf, r, side="right")
    return (np.minimum(idx, V - 2) + 1).astype(np.int32)


def make_inputs(B, T, U, H, V, *, dtype="fp32", sigma=0.05, seed=0, blank=0,
                t_range: Optional[tuple] = None, u_range: Optional[tuple] = None,
                labels_dist="uniform", zipf_s=1.1, name="custom",
                mode="T", tile_t=0, tile_u=0, tile_v=0) -> Inputs:
    """Draw one batch by the recipe in the module docstring.

    ``t_range``/``u_range`` = None means full lengths (T' = T, U' = U).
    Labels avoid ``blank`` only for blank = 0 (they are drawn from [1, V))."""
    rng = np.random.default_rng(seed)
    enc = rng.normal(0.0, sigma, size=(B, T, H))
    pred = rng.normal(0.0, sigma, size=(B, U + 1, H))
    W = rng.normal(0.0, sigma, size=(H, V))
    if t_range is None:
        T_lens = np.full(B, T, dtype=np.int32)
    else:
        T_lens = rng.integers(t_range[0], t_range[1] + 1, size=B).astype(np.int32)
    if u_range is None:
        U_lens = np.full(B, U, dtype=np.int32)
    else:
        U_lens = rng.integers(u_range[0], u_range[1] + 1, size=B).astype(np.int32)
    if labels_dist == "uniform":
        labels = rng.integers(1, V, size=(B, U)).astype(np.int32)
    elif labels_dist == "zipf":
        labels = _zipf_labels(rng, (B, U), V, zipf_s)
    else:
        raise ValueError(labels_dist)
    b = np.zeros(V)
    enc_s, enc_f = _cast(enc, dtype)
    pred_s, pred_f = _cast(pred, dtype)
    W_s, W_f = _cast(W, dtype)
    b_s, b_f = _cast(b, dtype)
    return Inputs(name=name, dtype=dtype, B=B, T=T, U=U, H=H, V=V, blank=blank,
                  enc=enc_s, pred=pred_s, W=W_s, b=b_s, labels=labels,
                  T_lens=T_lens, U_lens=U_lens, enc_f64=enc_f, pred_f64=pred_f,
                  W_f64=W_f, b_f64=b_f, mode=mode, tile_t=tile_t, tile_u=tile_u,
                  tile_v=tile_v)


# The five workloads: shapes, value and length distributions and the loss mode
# each runs in.  "medium" is run both untiled and tiled by the tests.
CONFIGS = {
    "tiny": dict(B=2, T=20, U=5, H=64, V=32, dtype="fp32", sigma=0.1,
                 t_range=None, u_range=None, mode="U"),
    "short": dict(B=8, T=200, U=50, H=256, V=512, dtype="fp32", sigma=0.05,
                  t_range=(150, 200), u_range=(30, 50), mode="U"),
    "medium": dict(B=16, T=500, U=100, H=640, V=1024, dtype="bf16", sigma=0.05,
                   t_range=(400, 500), u_range=(70, 100), mode="T",
                   tile_t=64, tile_u=64, tile_v=256),
    "medium_lv": dict(B=16, T=500, U=100, H=640, V=4096, dtype="bf16", sigma=0.05,
                      t_range=(400, 500), u_range=(70, 100), labels_dist="zipf",
                      mode="T", tile_t=64, tile_u=64, tile_v=256),
    "long": dict(B=8, T=1500, U=300, H=640, V=4096, dtype="bf16", sigma=0.05,
                 t_range=(1200, 1500), u_range=(200, 300), mode="T",
                 tile_t=64, tile_u=64, tile_v=256),
}


def make_config(name: str, seed: int = 0, **overrides) -> Inputs:
    kw = dict(CONFIGS[name])
    kw.update(overrides)
    return make_inputs(seed=seed, name=name, **kw)


@dataclasses.dataclass
class ProjInputs:
    """Joint input projections for one batch: raw encodings enc_in [B,T,E],
    pred_in [B,U+1,P] and the affine maps W_enc [E,H], b_enc [H], W_pred [P,H],
    b_pred [H], as storage arrays (float32 or uint16 bf16 bits) with float64
    twins holding the same values."""
    E: int
    P: int
    enc_in: np.ndarray
    pred_in: np.ndarray
    W_enc: np.ndarray
    b_enc: np.ndarray
    W_pred: np.ndarray
    b_pred: np.ndarray
    enc_in_f64: np.ndarray
    pred_in_f64: np.ndarray
    W_enc_f64: np.ndarray
    b_enc_f64: np.ndarray
    W_pred_f64: np.ndarray
    b_pred_f64: np.ndarray


def make_proj_inputs(inp: Inputs, E: int, P: int, *, seed: int = 0, sigma: float = 0.05,
                     w_scale: Optional[float] = None) -> ProjInputs:
    """Projection inputs matching batch ``inp`` (its B, T, U, H and dtype):
    enc_in, pred_in ~ N(0, sigma); W_enc, W_pred ~ N(0, w_scale) with w_scale
    = 1/sqrt(fan-in) by default (so the projected encodings keep about the
    spread of the inputs); biases ~ N(0, sigma).  Drawn in that order from
    numpy.random.default_rng(seed) in float64, then cast like the batch."""
    rng = np.random.default_rng(seed)
    B, T, U, H = inp.B, inp.T, inp.U, inp.H
    enc_in = rng.normal(0.0, sigma, size=(B, T, E))
    pred_in = rng.normal(0.0, sigma, size=(B, U + 1, P))
    W_enc = rng.normal(0.0, w_scale or 1.0 / np.sqrt(E), size=(E, H))
    b_enc = rng.normal(0.0, sigma, size=H)
    W_pred = rng.normal(0.0, w_scale or 1.0 / np.sqrt(P), size=(P, H))
    b_pred = rng.normal(0.0, sigma, size=H)
    parts = [_cast(x, inp.dtype) for x in (enc_in, pred_in, W_enc, b_enc, W_pred, b_pred)]
    s = [p[0] for p in parts]
    f = [p[1] for p in parts]
    return ProjInputs(E, P, *s, *f)


@dataclasses.dataclass
class DurationHead:
    """Duration head of a token-and-duration transducer for one batch:
    durations (frames per duration class), W_dur [H, K], b_dur [K] as storage
    arrays with float64 twins."""
    durations: tuple
    W_dur: np.ndarray
    b_dur: np.ndarray
    W_dur_f64: np.ndarray
    b_dur_f64: np.ndarray


def make_duration_head(inp: Inputs, durations=(0, 1, 2, 3, 4), *, seed: int = 0,
                       sigma: float = 0.05, b_sigma: float = 0.5) -> DurationHead:
    """W_dur ~ N(0, sigma) then b_dur ~ N(0, b_sigma), drawn in that order from
    numpy.random.default_rng(seed) in float64 and cast like the batch."""
    rng = np.random.default_rng(seed)
    K = len(durations)
    W = rng.normal(0.0, sigma, size=(inp.H, K))
    b = rng.normal(0.0, b_sigma, size=K)
    (Ws, Wf), (bs, bf) = _cast(W, inp.dtype), _cast(b, inp.dtype)
    return DurationHead(tuple(int(d) for d in durations), Ws, bs, Wf, bf)
