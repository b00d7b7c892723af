"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and lays them out: it holds none of the
method's arithmetic, and it is the one piece of code that both the oracle's
tests and the HIP path consume (they receive the same host arrays).

Recipe: standard normal fp32 values from ``numpy.random.default_rng`` keyed by
(seed, chunk index) so that any slice can be drawn on its own and the result
never depends on the thread count; logits are multiplied by the scale in fp32;
bf16 tensors are the fp32 values rounded to nearest-even by torch on the CPU.
Inputs past 2^31 elements are drawn on the device instead (device_normal),
and the oracle gets slices of them copied back.
The workshop of "The Online Softmax" (curionode, "Workshop") draws its logits
the same way: normal values times a chosen scale, in blocks of a chosen size.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

# The five workloads: one row softmax case the oracle finishes in seconds, a
# large bandwidth-bound row softmax, non-causal and causal attention forward,
# and split-KV decode.
WORKLOADS = {
    "softmax_small": dict(rows=4096, cols=1024, dtype="f32", scales=(1.0, 1000.0), block=8),
    "softmax_large": dict(rows=65536, cols=8192, dtypes=("f32", "bf16"), scales=(1.0, 30.0, 1000.0)),
    "attn_noncausal": dict(B=4, H=16, S=2048, D=64, causal=False),
    "attn_causal": dict(B=2, H=32, S=8192, D=128, causal=True),
    "decode_splitkv": dict(B=16, H=32, Lmax=32768, D=128, num_splits=64),
    # too few query blocks to fill the GPU (32 workgroups): split-K attention
    "attn_lowocc": dict(B=1, H=8, Sq=1024, Sk=65536, D=128, causal=False, num_splits=8),
    # rows longer than 16384: the streaming (two reads, one write) row softmax
    "softmax_long": dict(rows=1024, cols=262144, dtype="f32", scale=30.0),
}

_CHUNK_ROWS = 1024
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _normal_rows(rows: int, cols: int, seed, tag: int) -> np.ndarray:
    """[rows, cols] fp32 N(0,1); rows drawn in fixed chunks, each from its own
    generator keyed by (seed, tag, chunk)."""
    out = np.empty((rows, cols), np.float32)
    seed = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]

    def fill(c):
        r0 = c * _CHUNK_ROWS
        r1 = min(rows, r0 + _CHUNK_ROWS)
        rng = np.random.default_rng(seed + [tag, c])
        out[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32)

    n = -(-rows // _CHUNK_ROWS)
    if n <= 1:
        for c in range(n):
            fill(c)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(n)))
    return out


def _to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype}")


def logits(rows: int, cols: int, scale: float = 1.0, seed: int = 0, dtype: str = "f32") -> torch.Tensor:
    """Row-softmax input: N(0,1) * scale, [rows, cols], as a CPU tensor."""
    x = _normal_rows(rows, cols, seed, 0)
    if scale != 1.0:
        x *= np.float32(scale)
    return _to_torch(x, dtype)


def device_normal(shape, seed: int, device, scale: float = 1.0, dtype: str = "f32") -> torch.Tensor:
    """N(0,1) * scale of the given shape, drawn on `device` by torch's own
    generator seeded with `seed` (fp32, multiplied by the scale in fp32, bf16
    rounded to nearest-even from that).  For inputs past 2^31 elements, which
    would take minutes to draw on the host; the oracle receives slices of the
    same tensor copied back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype}")


def vector64(scale: float = 1.0, seed: int = 0) -> np.ndarray:
    """The workshop's single vector: 64 logits N(0,1) * scale, fp64."""
    rng = np.random.default_rng([int(seed), 7])
    return rng.standard_normal(64) * scale


def qkv(B: int, H: int, Sq: int, Sk: int, D: int, seed: int = 0, dtype: str = "bf16"):
    """Attention inputs Q [B,H,Sq,D], K and V [B,H,Sk,D], N(0,1), CPU tensors."""
    q = _normal_rows(B * H * Sq, D, seed, 1).reshape(B, H, Sq, D)
    k = _normal_rows(B * H * Sk, D, seed, 2).reshape(B, H, Sk, D)
    v = _normal_rows(B * H * Sk, D, seed, 3).reshape(B, H, Sk, D)
    return _to_torch(q, dtype), _to_torch(k, dtype), _to_torch(v, dtype)


def kv_lengths(B: int, Lmax: int, seed: int = 0, low: int = 1) -> np.ndarray:
    """Per-sequence KV lengths, uniform integers in [low, Lmax], int32."""
    rng = np.random.default_rng([int(seed), 4])
    return rng.integers(low, Lmax + 1, size=B).astype(np.int32)


def decode_inputs(B: int, H: int, Lmax: int, D: int, seed: int = 0, kv_len=None, dtype: str = "bf16"):
    """Split-KV decode inputs: q [B,H,1,D]; K, V [B,H,Lmax,D] with N(0,1)
    values in the first kv_len[b] positions of every (b, h) and zeros in the
    padding (which no kernel reads); kv_len [B] int32.  CPU tensors."""
    if kv_len is None:
        kv_len = kv_lengths(B, Lmax, seed)
    kv_len = np.asarray(kv_len, np.int32)
    q = _normal_rows(B * H, D, seed, 5).reshape(B, H, 1, D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    K = torch.zeros((B, H, Lmax, D), dtype=tdt)
    V = torch.zeros((B, H, Lmax, D), dtype=tdt)

    def fill(bh):
        b, h = divmod(bh, H)
        L = int(kv_len[b])
        if L == 0:
            return
        rk = np.random.default_rng([int(seed), 6, b, h]).standard_normal((L, D), dtype=np.float32)
        rv = np.random.default_rng([int(seed), 8, b, h]).standard_normal((L, D), dtype=np.float32)
        K[b, h, :L] = _to_torch(rk, dtype)
        V[b, h, :L] = _to_torch(rv, dtype)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(B * H)))
    return _to_torch(q, dtype), K, V, torch.from_numpy(kv_len.copy())


def decode_kv_pair(b: int, h: int, L: int, D: int, seed: int = 0):
    """The valid keys and values of one (b, h) of decode_inputs(..., seed),
    [L, D] fp32 each after rounding to bf16: the same draws, without
    building the whole cache."""
    rk = np.random.default_rng([int(seed), 6, b, h]).standard_normal((L, D), dtype=np.float32)
    rv = np.random.default_rng([int(seed), 8, b, h]).standard_normal((L, D), dtype=np.float32)
    widen = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy()  # noqa: E731
    return widen(rk), widen(rv)


def decode_q(B: int, H: int, D: int, seed: int = 0) -> np.ndarray:
    """The queries of decode_inputs(..., seed), [B, H, D] fp32 after rounding
    to bf16."""
    q = _normal_rows(B * H, D, seed, 5).reshape(B, H, D)
    return torch.from_numpy(q).to(torch.bfloat16).float().numpy()


def partials(N: int, S: int, D: int, seed: int = 0, empty_frac: float = 0.0, m_spread: float = 10.0):
    """Random partial states for the merge: m [N,S] (natural units, spread
    over +-m_spread), l [N,S] > 0, O [N,S,D] (unnormalised), fp32; a fraction
    of them set to the empty state (-inf, 0, 0)."""
    rng = np.random.default_rng([int(seed), 9])
    m = (rng.standard_normal((N, S)) * m_spread).astype(np.float32)
    l = rng.uniform(0.5, 64.0, size=(N, S)).astype(np.float32)
    O = (rng.standard_normal((N, S, D)).astype(np.float32) * l[:, :, None]).astype(np.float32)
    if empty_frac > 0:
        e = rng.random((N, S)) < empty_frac
        m[e] = -np.inf
        l[e] = 0.0
        O[e] = 0.0
    return torch.from_numpy(m), torch.from_numpy(l), torch.from_numpy(O)
