"""GPU parity over randomly drawn shapes and options, against the oracle.

The cases are drawn once, at import, from a fixed seed (so every run checks
the same cases and a failure names its case): shapes that fall on and off
the kernels' tile and block sizes, both head dimensions, both output dtypes,
causal and not, KV splits, softmax block sizes and scales, decode lengths
from 0 to Lmax, more and fewer than 64 sequences.  Each case is held to the
tolerances of the other parity tests (tests/gpu_util.py): fp32 softmax 1e-5
relative, bf16 4e-3; attention and decode 1e-2 absolute (bf16 output), or
2^-8 max|v| with an fp32 output; log-sum-exp 4e-3; maxima exact and
normalisers to 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as tea
from tiled_exact_attention_amd import inputs
from gpu_util import check_attention, check_softmax, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 4e-3
_rng = np.random.default_rng(20261202)


def _attn_cases(n):
    out = []
    for i in range(n):
        D = int(_rng.choice([64, 128]))
        causal = bool(_rng.random() < 0.4)
        Sq = max(1, int(np.exp(_rng.uniform(0.0, np.log(700.0)))))
        Sk = Sq if causal else max(1, int(np.exp(_rng.uniform(0.0, np.log(1500.0)))))
        out.append(dict(B=int(_rng.integers(1, 4)), H=int(_rng.integers(1, 6)), Sq=Sq, Sk=Sk, D=D, causal=causal,
                        scale=float(np.exp(_rng.uniform(np.log(0.02), np.log(4.0))) / math.sqrt(D)),
                        f32=bool(_rng.random() < 0.3), splits=int(_rng.integers(1, 10)), seed=1000 + i))
    return out


def _softmax_cases(n):
    out = []
    for i in range(n):
        cols = int(np.exp(_rng.uniform(0.0, np.log(40000.0))))
        out.append(dict(rows=int(_rng.integers(1, 300)), cols=max(cols, 1),
                        dtype=str(_rng.choice(["f32", "bf16"])), block=int(_rng.choice([0, 1, 2, 4, 8, 16, 32, 64])),
                        scale=float(_rng.choice([1.0, 30.0, 1000.0])), seed=2000 + i))
    return out


def _decode_cases(n):
    out = []
    for i in range(n):
        B = int(_rng.choice([1, 3, 17, 70]))
        Lmax = int(_rng.integers(1, 5000))
        lengths = _rng.integers(0, Lmax + 1, size=B).astype(np.int32)
        if B > 1:
            lengths[int(_rng.integers(0, B))] = Lmax  # the longest possible
        if B > 2:
            lengths[int(_rng.integers(0, B))] = 0  # a sequence with no keys
        out.append(dict(B=B, H=int(_rng.integers(1, 4)), Lmax=Lmax, lengths=lengths, D=int(_rng.choice([64, 128])),
                        splits=int(_rng.choice([1, 2, 7, 64, 100, 1024])), f32=bool(_rng.random() < 0.3),
                        seed=3000 + i))
    return out


ATTN = _attn_cases(120)
SOFTMAX = _softmax_cases(80)
DECODE = _decode_cases(40)


def _cid(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k not in ("lengths",))


def _check_attn_out(o, O, v, f32, what):
    if f32:
        err = np.max(np.abs(to_np(o) - O)) if O.size else 0.0
        bound = 2.0 ** -8 * float(np.abs(v).max() if v.size else 0.0) + 1e-5
        assert err <= bound, f"{what}: fp32-output max abs err {err:.2e} > {bound:.2e}"
    else:
        check_attention(to_np(o), O, what)


@pytest.mark.parametrize("c", ATTN, ids=[_cid(c) for c in ATTN])
def test_attention_random(c):
    say(f"attention random {_cid(c)}")
    B, H, Sq, Sk, D = c["B"], c["H"], c["Sq"], c["Sk"], c["D"]
    q, k, v = inputs.qkv(B, H, Sq, Sk, D, seed=c["seed"])
    od = torch.float32 if c["f32"] else torch.bfloat16
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = tea.attn_fwd(qd, kd, vd, scale=c["scale"], causal=c["causal"], out_dtype=od, return_lse=True)
    os_, lses = tea.attn_fwd_splitk(qd, kd, vd, c["splits"], scale=c["scale"], causal=c["causal"], out_dtype=od,
                                    return_lse=True)
    torch.cuda.synchronize()
    O, L = oracle.attention(q.float().numpy(), k.float().numpy(), v.float().numpy(), c["scale"], c["causal"])
    vf = v.float().numpy()
    _check_attn_out(o, O, vf, c["f32"], "attn_fwd")
    _check_attn_out(os_, O, vf, c["f32"], f"attn_fwd_splitk({c['splits']})")
    for name, ll in (("attn_fwd", lse), ("attn_fwd_splitk", lses)):
        err = np.max(np.abs(to_np(ll) - L))
        assert err <= LSE_TOL, f"{name}: LSE error {err:.2e}"


@pytest.mark.parametrize("c", SOFTMAX, ids=[_cid(c) for c in SOFTMAX])
def test_softmax_random(c):
    say(f"row_softmax random {_cid(c)}")
    x = inputs.logits(c["rows"], c["cols"], c["scale"], c["seed"], c["dtype"])
    y, m, l = tea.row_softmax(x.to(DEV), block=c["block"], stats=True)
    torch.cuda.synchronize()
    ref, mref, lref = oracle.softmax_rows(x.float().numpy())
    check_softmax(to_np(y), ref, 1e-5 if c["dtype"] == "f32" else 4e-3, _cid(c))
    assert np.array_equal(to_np(m).astype(np.float64), mref), "row maxima differ"
    assert np.max(np.abs(to_np(l) - lref) / lref) <= 1e-5, "normalisers differ"


@pytest.mark.parametrize("c", DECODE, ids=[_cid(c) for c in DECODE])
def test_decode_random(c):
    say(f"decode random {_cid(c)} lengths {c['lengths'].tolist()[:8]}...")
    B, H, Lmax, D, S = c["B"], c["H"], c["Lmax"], c["D"], c["splits"]
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=c["seed"], kv_len=c["lengths"])
    scale = 1.0 / math.sqrt(D)
    od = torch.float32 if c["f32"] else torch.bfloat16
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    outs = [("splitkv", tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=S, scale=scale, out_dtype=od))]
    if S <= 64:
        outs.append(("fused", tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=S, scale=scale, out_dtype=od)))
    torch.cuda.synchronize()
    ref = np.zeros((B, H, D))
    for b in range(B):
        L = int(c["lengths"][b])
        if L:
            o, _ = oracle.attention(q[b:b + 1].float().numpy(), K[b:b + 1, :, :L].float().numpy(),
                                    V[b:b + 1, :, :L].float().numpy(), scale, False)
            ref[b] = o.reshape(H, D)
    for name, o in outs:
        for b in range(B):
            L = int(c["lengths"][b])
            if L == 0:
                assert bool(torch.all(o[b] == 0)), f"{name}: sequence {b} has no keys but a nonzero output"
                continue
            _check_attn_out(o[b], ref[b], V[b, :, :L].float().numpy(), c["f32"], f"{name} sequence {b} (L={L})")
