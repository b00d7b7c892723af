"""Helpers for the GPU parity tests: tolerances written out once.

Tolerances (each justified by the arithmetic; the pages ask for a tolerance
"justified by the dtype", "Online softmax" (roadmapper), Why the values are
preserved):
  - fp32 softmax: elementwise relative error <= 1e-5 where the reference is a
    normal fp32 number (>= 2^-126); below that, absolute error <= 2^-126
    (flush to zero accepted).  A reference within its own relative tolerance
    of 2^-126 (below 2^-126 * (1 + rel)) may be computed on either side of
    it, so it falls under the absolute rule (<= 2^-126 * (1 + rel)): the
    kernel's exponential gives 0 for an exponent below -126 and the rounded
    exponent of such an element can cross -126.  Outputs finite and in
    [0, 1].
  - bf16 softmax: elementwise relative <= 4e-3 (bf16 keeps 8 significant
    bits, so rounding to nearest is at most 2^-8 = 3.91e-3 relative, plus the
    fp32 computation), same floor.
  - attention / decode: max abs error <= 1e-2 against the fp64 oracle; where
    |ref| >= 4 a bf16 output alone can be off by half an ulp (>= 2^-6), so
    those entries are held to half a bf16 ulp of ref plus 2e-3.
"""
import os
import sys

import numpy as np
import torch

FLOOR = 2.0 ** -126


def say(msg: str):
    """Progress line, flushed, so the last GPU step is known if a run dies."""
    sys.stdout.write(f"[gpu-step] {msg}\n")
    sys.stdout.flush()


def check_softmax(y: np.ndarray, ref: np.ndarray, rel: float, what: str = ""):
    y = np.asarray(y, np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert np.all(y >= 0.0) and np.all(y <= 1.0), f"{what}: output outside [0, 1]"
    big = ref >= FLOOR * (1.0 + rel)
    err = np.abs(y - ref)
    if np.any(big):
        r = np.max(err[big] / ref[big])
        assert r <= rel, f"{what}: max relative error {r:.3e} > {rel:.1e}"
    if np.any(~big):
        a = np.max(err[~big])
        assert a <= FLOOR * (1.0 + rel), f"{what}: absolute error {a:.3e} below the normal range"
    return float(np.max(err[big] / ref[big])) if np.any(big) else 0.0


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def check_attention(o: np.ndarray, ref: np.ndarray, what: str = "", atol: float = 1e-2):
    o = np.asarray(o, np.float64)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref)
    big = np.abs(ref) >= 4.0
    small_err = float(np.max(err[~big])) if np.any(~big) else 0.0
    assert small_err <= atol, f"{what}: max abs error {small_err:.3e} > {atol}"
    if np.any(big):
        lim = half_ulp_bf16(ref[big]) + 2e-3
        assert np.all(err[big] <= lim), f"{what}: large-|ref| entries beyond half a bf16 ulp + 2e-3"
    return small_err


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def box_cores() -> int:
    return os.cpu_count() or 1
