"""GPU parity of attn_fwd against the fp64 oracle (attention from its
definition).

The log-sum-exp output is m + ln(l), and l sums the same bf16-rounded weights
that multiply V.  bf16 keeps 8 significant bits, so rounding a weight to
nearest moves it by at most 2^-8 relative, l by as much and ln(l) by at most
-ln(1 - 2^-8) < 3.92e-3: the tolerance is 4e-3.

Workloads: non-causal B4 H16 S2048 D64 and causal B2 H32 S8192 D128, bf16
N(0,1), scale 1/sqrt(D), at full size, every row; small shapes in
full, spanning several tiles with ragged tails; closed forms that hold
exactly (one key, causal row 0) or in general (constant V); fp32 output,
log-sum-exp, determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as tea
from tiled_exact_attention_amd import inputs
from gpu_util import check_attention, half_ulp_bf16, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 4e-3


def _np32(t):
    return t.float().numpy()


def _run(q, k, v, causal, out_dtype=torch.bfloat16, scale=None):
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    o, lse = tea.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal, out_dtype=out_dtype,
                          return_lse=True)
    torch.cuda.synchronize()
    return o, lse, scale


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 2, 17, 64, 127, 128, 129, 300, 1000])
def test_small_full_parity(D, causal, S):
    say(f"attn_fwd small S={S} D={D} causal={causal}")
    q, k, v = inputs.qkv(2, 3, S, S, D, seed=S * 7 + D)
    o, lse, scale = _run(q, k, v, causal)
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), scale, causal)
    check_attention(to_np(o), O, f"S={S} D={D} causal={causal}")
    assert np.max(np.abs(to_np(lse) - L)) <= LSE_TOL


@pytest.mark.parametrize("Sq,Sk", [(1, 1000), (100, 1), (129, 65), (64, 1000), (333, 2049)])
def test_noncausal_rectangular(Sq, Sk):
    say(f"attn_fwd Sq={Sq} Sk={Sk}")
    q, k, v = inputs.qkv(1, 4, Sq, Sk, 128, seed=Sq + Sk)
    o, lse, scale = _run(q, k, v, False)
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), scale, False)
    check_attention(to_np(o), O, f"Sq={Sq} Sk={Sk}")
    assert np.max(np.abs(to_np(lse) - L)) <= LSE_TOL


def test_fp32_output():
    """With an fp32 output the error left is P's rounding to bf16 before the
    P V product (2^-8 relative per weight), so at most 2^-8 * max|v| per
    entry; every entry is checked against that bound."""
    say("attn_fwd fp32 output")
    q, k, v = inputs.qkv(1, 2, 500, 500, 128, seed=3)
    o, _, scale = _run(q, k, v, True, out_dtype=torch.float32)
    O, _ = oracle.attention(_np32(q), _np32(k), _np32(v), scale, True)
    err = np.abs(to_np(o) - O)
    bound = 2.0 ** -8 * np.abs(_np32(v)).max() + 1e-5
    assert np.max(err) <= bound, f"fp32-output max abs err {np.max(err):.2e} > {bound:.2e}"
    print(f"fp32-output max abs err {np.max(err):.2e} (bound {bound:.2e})")


def test_closed_forms():
    say("attn_fwd closed forms")
    q, k, v = inputs.qkv(2, 2, 200, 200, 64, seed=4)
    # one key: O = v0 exactly
    o, lse, _ = _run(q, k[:, :, :1].contiguous(), v[:, :, :1].contiguous(), False)
    assert torch.equal(o.cpu(), v[:, :, :1].expand(-1, -1, 200, -1))
    # causal row 0 sees key 0 only
    o, _, _ = _run(q, k, v, True)
    assert torch.equal(o.cpu()[:, :, 0], v[:, :, 0])
    # constant V: constant O (bf16 1.5 is exact): l sums the same rounded
    # weights as the numerator, so only the fp32 sums' order differs
    vc = torch.full_like(v, 1.5)
    o, _, _ = _run(q, k, vc, True, out_dtype=torch.float32)
    assert float((o - 1.5).abs().max()) <= 1e-5
    q2, k2, _ = inputs.qkv(2, 2, 200, 200, 128, seed=5)
    o, _, _ = _run(q2, k2, torch.full_like(q2, 1.5), True, out_dtype=torch.float32)
    assert float((o - 1.5).abs().max()) <= 1e-5
    # large scale: logits far apart, no overflow or NaN
    o, lse, _ = _run(q, k, v, False, scale=30.0)
    O, _ = oracle.attention(_np32(q), _np32(k), _np32(v), 30.0, False)
    check_attention(to_np(o), O, "scale 30")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(D, causal):
    """Identical keys give every visible key the same score, so every weight
    is exactly 1 (2^0) and O is the mean of V over the visible keys (row i's
    first i + 1 keys when causal), up to the fp32 sums of at most S values."""
    say(f"attn_fwd identical keys D={D} causal={causal}")
    S = 333
    q, k, v = inputs.qkv(1, 2, S, S, D, seed=D + int(causal))
    k = k[:, :, :1].expand(-1, -1, S, -1).contiguous()
    o, _, _ = _run(q, k, v, causal, out_dtype=torch.float32)
    vf = _np32(v).astype(np.float64)
    if causal:
        ref = np.cumsum(vf, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    else:
        ref = np.broadcast_to(vf.mean(axis=2, keepdims=True), vf.shape)
    bound = 2.0 * S * 2.0 ** -24 * np.abs(vf).max() + 1e-6
    err = np.abs(to_np(o) - ref)
    assert np.max(err) <= bound, f"max err {np.max(err):.2e} > {bound:.2e}"


def _ramp_inputs(B, H, Sq, Sk, D, slope, seed):
    """Scores that drift along the keys: q has a unit first component and
    key j's first component is slope * j, so the score of key j rises (or,
    for slope < 0, falls) by about slope * j / sqrt(D) on top of N(0, 0.25)
    noise.  The running maximum then moves in every tile, by amounts below
    and above the kernel's lag threshold."""
    q, k, v = inputs.qkv(B, H, Sq, Sk, D, seed=seed)
    q = (q.float() * 0.5).bfloat16()
    k = (k.float() * 0.5).bfloat16()
    q[..., 0] = 1.0
    k[..., 0] = (slope * torch.arange(Sk, dtype=torch.float32)).bfloat16()
    return q.contiguous(), k.contiguous(), v


def _p_rounding_bound(q, k, v, scale, causal, O, L):
    """Bound on what rounding the weights to bf16 does to O, with
    p~_j = p_j (1 + d_j), |d_j| <= 2^-8 (bf16 keeps 8 significant bits).
    l sums the same p~, so the output is the convex combination
    sum_j w~_j v_j with w~_j = w_j (1 + d_j) / (1 + sum_i w_i d_i), and
    |O~ - O| <= 2^-7 / (1 - 2^-8) * sum_j w_j |v_j - O|, per row and dim.
    The scores carry errors of their own: an fp32 dot product of D bf16
    products is within D 2^-24 g_j of the exact one (g_j = scale sum_i
    |q_i k_ji|), and the exponent s c - mu (c = scale log2 e, mu the row's
    reference, at most the row's largest |s| c plus the lag) is rounded once
    more, within 2^-24 (|s_j| + max_i |s_i| + 6) / ln 2 in base-two units,
    i.e. 2^-24 (g_j + max_i g_i + 6) in the weight's logarithm; the
    exponential adds a few ulps (2^-21).  An error e_j in weight j's
    logarithm moves O, to first order, by sum_j w_j e_j (v_j - O), so at
    most sum_j w_j |e_j| (|v_j| + |O|); that term is added with 1% for the
    second order.
    The weights w_j = exp(s_j - L) come from the oracle's L (fp64)."""
    qf, kf, vf = (np.asarray(t, np.float64) for t in (q, k, v))
    out = np.empty_like(O)
    Sq, Sk = qf.shape[2], kf.shape[2]
    for r0 in range(0, Sq, 128):
        r1 = min(Sq, r0 + 128)
        s = np.einsum("bhqd,bhkd->bhqk", qf[:, :, r0:r1], kf) * scale
        if causal:
            s = np.where(np.arange(Sk)[None, :] <= np.arange(r0, r1)[:, None], s, -np.inf)
        w = np.exp(s - L[:, :, r0:r1, None])
        g = np.einsum("bhqd,bhkd->bhqk", np.abs(qf[:, :, r0:r1]), np.abs(kf)) * scale
        e = 2.0 ** -24 * ((qf.shape[-1] + 1) * g + g.max(axis=-1, keepdims=True) + 6.0) + 2.0 ** -21
        we = w * e
        s_term = 1.01 * (np.einsum("bhqk,bhkd->bhqd", we, np.abs(vf)) + we.sum(-1)[..., None] * np.abs(O[:, :, r0:r1]))
        dev = np.abs(vf[:, :, None, :, :] - O[:, :, r0:r1, None, :])  # [b, h, q, k, d]
        out[:, :, r0:r1] = np.einsum("bhqk,bhqkd->bhqd", w, dev) * (2.0 ** -7 / (1.0 - 2.0 ** -8)) + s_term
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("rise", [-8.0, 0.5, 4.0, 12.0, 60.0])
def test_drifting_maximum(D, causal, rise):
    """rise: growth of the score per 64-key tile, in base-two units.  Below
    the kernel's lag (8) its reference trails the running maximum and moves
    only every few tiles; above it the reference moves every tile; falling
    scores keep the first tile's maximum.  The result must not depend on
    which.  With steep rises the weights sit on a few keys, so the 1e-2 of
    diffuse attention is replaced by the bound the arithmetic gives: the
    bf16 rounding of the weights (see _p_rounding_bound) plus, for a bf16
    output, half a bf16 ulp of the result, plus the fp32 summation error."""
    S = 700
    slope = rise / 64.0 * math.sqrt(D) / math.log2(math.e)
    say(f"attn_fwd drifting maximum rise={rise}/tile D={D} causal={causal}")
    q, k, v = _ramp_inputs(1, 2, S, S, D, slope, seed=int(abs(rise) * 10) + D)
    o, lse, scale = _run(q, k, v, causal)
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), scale, causal)
    # the log-sum-exp also carries the error of the scores themselves: an fp32
    # dot product of D terms is within D 2^-24 sum_i |q_i k_i| of the exact
    # one, and the log-sum-exp moves by at most the largest score error
    qa, ka = np.abs(_np32(q)).astype(np.float64), np.abs(_np32(k)).astype(np.float64)
    gross = np.einsum("bhqd,bhkd->bhqk", qa, ka)
    if causal:
        gross = np.where(np.tril(np.ones((S, S), bool)), gross, 0.0)
    s_err = D * 2.0 ** -24 * scale * gross.max(axis=-1)
    assert np.all(np.abs(to_np(lse) - L) <= LSE_TOL + s_err)
    # fp32 sums of at most S products p v and p, each <= 2^8 |v|max relative
    # to the reference: S 2^-24 relative error each, on O and on l
    acc = 2.0 * S * 2.0 ** -24 * float(np.abs(_np32(v)).max())
    pb = _p_rounding_bound(_np32(q), _np32(k), _np32(v), scale, causal, O, L) + acc
    err = np.abs(to_np(o).astype(np.float64) - O)
    lim = half_ulp_bf16(np.abs(O) + pb) + pb  # the ulp of the computed value, which may sit one binade up
    assert np.all(err <= lim), f"bf16 output: worst err/bound {np.max(err / lim):.3f}"
    # and the attention bar itself: max abs error <= 1e-2 (entries with
    # |ref| >= 4 held to half a bf16 ulp + 2e-3), for both output dtypes
    check_attention(to_np(o), O, f"drift rise={rise} D={D} causal={causal} bf16 out")
    o32, _, _ = _run(q, k, v, causal, out_dtype=torch.float32)
    err32 = np.abs(to_np(o32).astype(np.float64) - O)
    assert np.all(err32 <= pb), f"fp32 output: worst err/bound {np.max(err32 / pb):.3f}"
    check_attention(to_np(o32), O, f"drift rise={rise} D={D} causal={causal} fp32 out")
    print(f"rise {rise}: max abs err bf16 {err.max():.2e}, fp32 {err32.max():.2e}; "
          f"worst err/bound {np.max(err / lim):.3f} / {np.max(err32 / pb):.3f}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H", [8, 16, 24, 6])
def test_causal_grid_orders(D, H):
    """Causal grids whose (batch, head) count is a multiple of 8 are dealt to
    the 8 XCDs and walked longest block first within pairs of heads (one
    head at a time when an XCD's share of heads is odd: H = 8, 24); other
    grids (H = 6) take the plain reversed order.  Every output row, and the
    log-sum-exp, must match the oracle whichever order ran."""
    S = 700  # 2 query blocks at D = 64, 3 at D = 128
    say(f"attn_fwd causal grid order H={H} D={D}")
    q, k, v = inputs.qkv(1, H, S, S, D, seed=H * 3 + D)
    o, lse, scale = _run(q, k, v, True)
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), scale, True)
    check_attention(to_np(o), O, f"causal order H={H} D={D}")
    assert np.max(np.abs(to_np(lse) - L)) <= LSE_TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 3, 8, 64])
def test_splitk_parity(D, causal, splits):
    """attn_fwd_splitk: each query block's KV tiles split `splits` ways, the
    partials merged by the combine.  Against the oracle, and against attn_fwd
    up to rounding (fp32 outputs).  With 64 splits most tile ranges of the
    early causal blocks are empty, so their partials are the empty state."""
    S = 700
    say(f"attn_fwd_splitk S={S} D={D} causal={causal} splits={splits}")
    q, k, v = inputs.qkv(1, 3, S, S, D, seed=splits * 13 + D + int(causal))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1.0 / math.sqrt(D)
    o, lse = tea.attn_fwd_splitk(qd, kd, vd, splits, scale=scale, causal=causal, return_lse=True)
    o32 = tea.attn_fwd_splitk(qd, kd, vd, splits, scale=scale, causal=causal, out_dtype=torch.float32)
    r32 = tea.attn_fwd(qd, kd, vd, scale=scale, causal=causal, out_dtype=torch.float32)
    torch.cuda.synchronize()
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), scale, causal)
    check_attention(to_np(o), O, f"splitk D={D} causal={causal} splits={splits}")
    assert np.max(np.abs(to_np(lse) - L)) <= LSE_TOL
    # the same weights, rounded to bf16 against a different reference per
    # range: within the fp32-output bound of either against the oracle
    bound = 2.0 ** -8 * np.abs(_np32(v)).max() + 1e-5
    assert float((o32 - r32).abs().max()) <= bound


def test_splitk_rectangular_and_full_size_sample():
    """Non-causal Sq != Sk with a ragged last tile, and the low-occupancy
    shape of the bench (B1 H8 Sq1024 Sk65536 D128, 8 splits) on sampled
    rows."""
    say("attn_fwd_splitk rectangular 129 x 2049")
    q, k, v = inputs.qkv(2, 2, 129, 2049, 128, seed=77)
    o = tea.attn_fwd_splitk(q.to(DEV), k.to(DEV), v.to(DEV), 5)
    torch.cuda.synchronize()
    O, _ = oracle.attention(_np32(q), _np32(k), _np32(v), 1 / math.sqrt(128), False)
    check_attention(to_np(o), O, "splitk 129x2049")
    w = inputs.WORKLOADS["attn_lowocc"]
    B, H, Sq, Sk, D, ns = w["B"], w["H"], w["Sq"], w["Sk"], w["D"], w["num_splits"]
    say(f"attn_fwd_splitk B{B} H{H} Sq{Sq} Sk{Sk} D{D} splits {ns}")
    q, k, v = inputs.qkv(B, H, Sq, Sk, D, seed=601)
    o, lse = tea.attn_fwd_splitk(q.to(DEV), k.to(DEV), v.to(DEV), ns, return_lse=True)
    torch.cuda.synchronize()
    flat = np.array([bh * Sq + i for bh in range(B * H) for i in (0, 1, 31, 32, 500, Sq - 1)])
    O, L = oracle.attention(_np32(q), _np32(k), _np32(v), 1 / math.sqrt(D), False, rows=flat)
    check_attention(to_np(o).reshape(-1, D)[flat], O, "splitk low occupancy")
    assert np.max(np.abs(to_np(lse).reshape(-1)[flat] - L)) <= LSE_TOL


def test_empty_keys_give_zero():
    say("attn_fwd Sk=0")
    q = torch.randn(1, 2, 10, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    o, lse = tea.attn_fwd(q, k, k, causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -math.inf)


def test_deterministic():
    say("attn_fwd determinism")
    q, k, v = (t.to(DEV) for t in inputs.qkv(2, 4, 1000, 1000, 128, seed=5))
    a = tea.attn_fwd(q, k, v, causal=True)
    b = tea.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("cfg", ["attn_noncausal", "attn_causal"])
def test_full_size(cfg):
    """Both attention workloads at full size, in the launch configuration the
    benchmark times, every output row and its log-sum-exp against the
    oracle, element by element: non-causal B4 H16 S2048 D64 (131,072 rows)
    and causal B2 H32 S8192 D128 (524,288 rows, compared in chunks of
    65,536 rows; about 13 s of oracle work on a 16-thread host)."""
    w = inputs.WORKLOADS[cfg]
    B, H, S, D, causal = w["B"], w["H"], w["S"], w["D"], w["causal"]
    seed = 301 if cfg == "attn_noncausal" else 401
    say(f"attn_fwd full size {cfg} B{B} H{H} S{S} D{D} causal={causal}")
    q, k, v = inputs.qkv(B, H, S, S, D, seed=seed)
    o, lse, scale = _run(q, k, v, causal)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    got = to_np(o).reshape(-1, D)
    gl = to_np(lse).reshape(-1)
    del o, lse
    qn, kn, vn = _np32(q), _np32(k), _np32(v)
    n = B * H * S
    err = lerr = 0.0
    step = 65536
    for r0 in range(0, n, step):
        rows = np.arange(r0, min(n, r0 + step), dtype=np.int64)
        O, L = oracle.attention(qn, kn, vn, scale, causal, rows=rows)
        err = max(err, check_attention(got[rows], O, f"{cfg} rows {r0}.."))
        lerr = max(lerr, float(np.max(np.abs(gl[rows] - L))))
        assert lerr <= LSE_TOL
        if (r0 // step) % 2 == 1:
            say(f"attn_fwd full size {cfg}: {r0 + step} of {n} rows compared")
    print(f"{cfg}: max abs err {err:.3e}, LSE {lerr:.3e}, over all {n} rows")


@pytest.mark.parametrize("D,H", [(128, 256), (64, 512)])
def test_beyond_2_31_elements(D, H):
    """K and V of more than 2^31 elements each (B1, Sk 65549: 2.15e9
    elements), so the heads near the end sit past byte offset 2^32 and are
    reached through 64-bit offsets.  16 queries per head (a partial query
    block) against every key of its head, plain and with 8 KV splits; the
    first, middle and last heads against the oracle in full."""
    B, Sq, Sk = 1, 16, 65549
    assert H * Sk * D > 2 ** 31
    say(f"attn_fwd past 2^31 elements: B{B} H{H} Sq{Sq} Sk{Sk} D{D}")
    q = inputs.device_normal((B, H, Sq, D), 611, DEV, dtype="bf16")
    k = inputs.device_normal((B, H, Sk, D), 612, DEV, dtype="bf16")
    v = inputs.device_normal((B, H, Sk, D), 613, DEV, dtype="bf16")
    scale = 1.0 / math.sqrt(D)
    o, lse = tea.attn_fwd(q, k, v, scale=scale, return_lse=True)
    o8, lse8 = tea.attn_fwd_splitk(q, k, v, 8, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    for h in (0, 1, H // 2, H - 2, H - 1):
        sl = slice(h, h + 1)
        O, L = oracle.attention(_np32(q[:, sl].cpu()), _np32(k[:, sl].cpu()), _np32(v[:, sl].cpu()), scale, False)
        for name, oo, ll in (("plain", o, lse), ("8 splits", o8, lse8)):
            check_attention(to_np(oo[:, sl]), O, f"{name} D={D} head {h}")
            assert np.max(np.abs(to_np(ll[:, sl]) - L)) <= LSE_TOL, f"{name} D={D} head {h}: LSE"
    del q, k, v
