"""Plain fp64 CPU oracle for the online softmax, attention and split-KV decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The product path (the
HIP library and its binding) never imports, links or calls it, and the two
share no code: the oracle is C (``oracle.c``) compiled with gcc, no HIP header,
no constant or helper in common.

Each function computes the plain definition in double precision from the
exact values the GPU receives (fp32 arrays; bf16 widened exactly to fp32 by
the caller).  Sources are cited by page title and section in ``oracle.c``:
"Online softmax" (roadmapper), "The Online Softmax" (curionode, Vol. XVI
plate 3) and "Online Softmax" (metalworking).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

# Plain IEEE double: no fast-math (it would delete the -inf handling), no
# contraction of a*b+c into fma, so the oracle rounds the way its C reads.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (always, when ``force``)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", *CFLAGS, "-I", _HERE, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            D = ctypes.c_double
            lib.oracle_softmax_rows.argtypes = [P, I64, I64, P, P, P]
            lib.oracle_softmax_f64.argtypes = [P, I64, P, P, P]
            lib.oracle_naive_normaliser.argtypes = [P, I64, P, P, P]
            lib.oracle_online_trace.argtypes = [P, I64, I64, ctypes.c_int, P, P, P, P, P, P]
            lib.oracle_online_trace.restype = I64
            lib.oracle_online_attention_row.argtypes = [P, P, I64, I64, I64, ctypes.c_int, P, P, P]
            lib.oracle_attention_rows.argtypes = [P, P, P, I64, I64, I64, I64, I64, D, ctypes.c_int, P, I64, P, P]
            lib.oracle_partial.argtypes = [P, P, I64, I64, P, P, P]
            lib.oracle_combine.argtypes = [D, D, P, D, D, P, I64, P, P, P]
            lib.oracle_merge_direct.argtypes = [P, P, P, I64, I64, I64, P, P, P]
            lib.oracle_abi_version.restype = ctypes.c_int
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _swap_library(path):
    """Point the binding at another build of ``oracle.c`` (tests use this to
    show that mistakes planted in the oracle's source fail its pins); returns
    the previous handle, to be restored with ``_restore_library``."""
    global _lib
    prev = _load()
    with _lock:
        _lib = None
    global _LIB_PATH
    saved = _LIB_PATH
    _LIB_PATH = path
    try:
        _load()
    finally:
        _LIB_PATH = saved
    return prev


def _restore_library(prev):
    global _lib
    with _lock:
        _lib = prev


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def softmax_rows(x: np.ndarray):
    """Two-pass safe softmax of each row of fp32 logits -> (y, m, l) in fp64."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float64)
    m = np.empty(rows, np.float64)
    l = np.empty(rows, np.float64)
    _load().oracle_softmax_rows(_p(x), rows, cols, _p(y), _p(m), _p(l))
    return y, m, l


def softmax_f64(x: np.ndarray):
    """Two-pass safe softmax of one fp64 vector -> (y, m, l)."""
    x = _c(x, np.float64)
    y = np.empty_like(x)
    m = np.empty(1)
    l = np.empty(1)
    _load().oracle_softmax_f64(_p(x), x.size, _p(y), _p(m), _p(l))
    return y, float(m[0]), float(l[0])


def naive_normaliser(x: np.ndarray):
    """(sum exp(x), that sum times exp(-max), finite flag) in fp64."""
    x = _c(x, np.float64)
    s = np.empty(1)
    r = np.empty(1)
    f = np.zeros(1, np.int32)
    _load().oracle_naive_normaliser(_p(x), x.size, _p(s), _p(r), _p(f))
    return float(s[0]), float(r[0]), bool(f[0])


VARIANTS = {
    "natural": 0,
    "base2": 1,
    "l0_one": 2,
    "conditional": 3,
    "bug_no_carry": 10,
    "bug_mixed_bases": 11,
    "bug_no_guard": 12,
    "bug_rescale_l_only": 20,
    "bug_rescale_acc_only": 21,
}


def online_trace(x: np.ndarray, block: int, variant: str = "natural"):
    """Run the online normaliser recurrence block by block; return its trace."""
    x = _c(x, np.float64)
    nb = -(-x.size // block) if x.size else 0
    mt = np.empty(max(nb, 1))
    lt = np.empty(max(nb, 1))
    ct = np.empty(max(nb, 1))
    nres = np.zeros(1, np.int64)
    mf = np.empty(1)
    lf = np.empty(1)
    k = _load().oracle_online_trace(_p(x), x.size, block, VARIANTS[variant], _p(mt), _p(lt), _p(ct),
                                    _p(nres), _p(mf), _p(lf))
    return {
        "updates": int(k),
        "rescales": int(nres[0]),
        "m": float(mf[0]),
        "l": float(lf[0]),
        "m_trace": mt[:k].copy(),
        "l_trace": lt[:k].copy(),
        "c_trace": ct[:k].copy(),
    }


def online_attention_row(s: np.ndarray, V: np.ndarray, block: int, variant: str = "natural"):
    """Recurrence with the output accumulator for one query row -> (o, m, l)."""
    s = _c(s, np.float64)
    V = _c(V, np.float64)
    n = s.size
    D = V.shape[1]
    o = np.empty(D)
    m = np.empty(1)
    l = np.empty(1)
    _load().oracle_online_attention_row(_p(s), _p(V), n, D, block, VARIANTS[variant], _p(o), _p(m), _p(l))
    return o, float(m[0]), float(l[0])


def attention(Q, K, V, scale: float, causal: bool = False, rows=None):
    """Attention from the definition.  Q [B,H,Sq,D], K/V [B,H,Sk,D] (fp32
    values).  ``rows``: optional flat (b*H+h)*Sq+i indices.  Returns
    (O [nrows, D] or [B,H,Sq,D], lse) in fp64."""
    Q = _c(Q, np.float32)
    K = _c(K, np.float32)
    V = _c(V, np.float32)
    B, H, Sq, D = Q.shape
    Sk = K.shape[2]
    if rows is None:
        nrows = B * H * Sq
        rp = None
    else:
        rows = _c(rows, np.int64)
        nrows = rows.size
        rp = _p(rows)
    O = np.empty((nrows, D), np.float64)
    lse = np.empty(nrows, np.float64)
    _load().oracle_attention_rows(_p(Q), _p(K), _p(V), B, H, Sq, Sk, D, float(scale), int(bool(causal)), rp, nrows,
                                  _p(O), _p(lse))
    if rows is None:
        return O.reshape(B, H, Sq, D), lse.reshape(B, H, Sq)
    return O, lse


def decode(q, K, V, kv_len, scale: float, pairs=None, widen=None):
    """Decode attention from the definition: one query per (b, h) over the
    first kv_len[b] keys.  q [B,H,D]; K/V [B,H,Lmax,D] (any array type whose
    slices ``widen`` turns into fp32 numpy; default numpy conversion).
    ``pairs``: optional list of (b, h).  Returns (O [n, D], lse [n])."""
    B, H = q.shape[0], q.shape[1]
    if pairs is None:
        pairs = [(b, h) for b in range(B) for h in range(H)]
    widen = widen or (lambda a: np.asarray(a, np.float32))
    D = q.shape[-1]
    O = np.empty((len(pairs), D))
    lse = np.empty(len(pairs))
    for n, (b, h) in enumerate(pairs):
        L = int(kv_len[b])
        qq = widen(q[b, h]).reshape(1, 1, 1, D)
        kk = widen(K[b, h, :L]).reshape(1, 1, L, D)
        vv = widen(V[b, h, :L]).reshape(1, 1, L, D)
        o, s = attention(qq, kk, vv, scale, False)
        O[n] = o.reshape(D)
        lse[n] = s.reshape(())
    return O, lse


def partial(s, V):
    """(m, l, unnormalised O) of one set of scores s[n] with values V[n, D]."""
    s = _c(s, np.float64)
    V = _c(V, np.float64).reshape(s.size, -1) if s.size else _c(V, np.float64)
    D = V.shape[-1]
    O = np.empty(D)
    m = np.empty(1)
    l = np.empty(1)
    _load().oracle_partial(_p(s), _p(V), s.size, D, _p(m), _p(l), _p(O))
    return float(m[0]), float(l[0]), O


def combine(a, b):
    """Pairwise combine of two partial states (m, l, O)."""
    m1, l1, O1 = a
    m2, l2, O2 = b
    O1 = _c(O1, np.float64)
    O2 = _c(O2, np.float64)
    O = np.empty_like(O1)
    m = np.empty(1)
    l = np.empty(1)
    _load().oracle_combine(float(m1), float(l1), _p(O1), float(m2), float(l2), _p(O2), O1.size, _p(m), _p(l),
                           _p(O))
    return float(m[0]), float(l[0]), O


def merge_direct(m, l, O):
    """Merged (m, l, unnormalised O) of partials m,l [N,S], O [N,S,D]."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    O = _c(O, np.float64)
    N, S, D = O.shape
    mo = np.empty(N)
    lo = np.empty(N)
    Oo = np.empty((N, D))
    _load().oracle_merge_direct(_p(m), _p(l), _p(O), N, S, D, _p(mo), _p(lo), _p(Oo))
    return mo, lo, Oo


def abi_version() -> int:
    return int(_load().oracle_abi_version())


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops run on."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Run the oracle's OpenMP loops on n threads; returns the previous count."""
    return int(_load().oracle_set_num_threads(int(n)))
