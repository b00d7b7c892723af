"""GPU parity of attn_decode_splitkv and merge_partials against the fp64
oracle.

Decode: B16 H32, one query, KV length uniform in [1, 32768], D128, 64 splits
at full size on every (b, h) pair, and by properties at any size; lengths
at chunk and tile edges (including L < 64, where chunks are empty, and
L = 0); other split counts.  Merge: random partials against the merged state
written out directly; the empty state as identity; all-empty rows; any S and
D; agreement of different tree shapes up to rounding.  The single-launch
decode against the oracle and against the two-launch form.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_exact_attention_amd as tea
from tiled_exact_attention_amd import inputs
from gpu_util import check_attention, say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _decode_ref(q, K, V, kv, scale, pairs):
    O, lse = oracle.decode(q[:, :, 0], K, V, kv, scale, pairs=pairs, widen=lambda t: t.float().numpy())
    return O


@pytest.mark.parametrize("lengths", [[1, 2, 63, 64], [65, 511, 512, 513], [1000, 4096, 32767, 32768], [0, 5, 0, 70]])
@pytest.mark.parametrize("splits", [1, 2, 64, 1024])
def test_decode_edge_lengths(lengths, splits):
    say(f"decode lengths={lengths} splits={splits}")
    B, H, D = len(lengths), 3, 128
    Lmax = max(max(lengths), 1)
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=sum(lengths) + splits, kv_len=np.array(lengths))
    scale = 1.0 / math.sqrt(D)
    o = tea.attn_decode_splitkv(q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV), num_splits=splits, scale=scale)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    ref = _decode_ref(q, K, V, kv.numpy(), scale, pairs)
    check_attention(to_np(o).reshape(-1, D), ref, f"lengths={lengths} splits={splits}")
    for n, (b, h) in enumerate(pairs):
        if lengths[b] == 0:
            assert torch.all(o[b, h] == 0)


@pytest.mark.parametrize("B", [63, 64, 65, 70])
def test_decode_many_sequences(B):
    """Sequences are taken longest first when there are at most 64 of them
    and in grid order beyond; either way every (b, h) must get its own
    sequence's result.  Lengths include ties and zeros."""
    say(f"decode many sequences B={B}")
    H, D, Lmax = 2, 128, 700
    rng = np.random.default_rng(B)
    lengths = rng.integers(0, Lmax + 1, size=B)
    lengths[::7] = 333  # ties
    lengths[3] = 0
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=B, kv_len=lengths)
    scale = 1.0 / math.sqrt(D)
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    o = tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=8, scale=scale)
    of = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=8, scale=scale)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    ref = _decode_ref(q, K, V, kv.numpy(), scale, pairs)
    check_attention(to_np(o).reshape(-1, D), ref, f"two launches B={B}")
    check_attention(to_np(of).reshape(-1, D), ref, f"one launch B={B}")
    assert torch.all(o[3] == 0) and torch.all(of[3] == 0)


def test_decode_d64_and_fp32_out():
    say("decode D=64 fp32 out")
    B, H, D, Lmax = 3, 4, 64, 3000
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=9, kv_len=np.array([3000, 17, 1234]))
    o = tea.attn_decode_splitkv(q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV), num_splits=64, scale=0.125,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    ref = _decode_ref(q, K, V, kv.numpy(), 0.125, pairs)
    check_attention(to_np(o).reshape(-1, D), ref, "D64 fp32", atol=2e-3)


def _decode_ref_all(q, K, V, kv, scale):
    """The oracle's decode for every (b, h), one call per sequence so the
    oracle's threads run across its heads: O [B*H, D] in (b, h) order."""
    B, H, D = q.shape[0], q.shape[1], q.shape[-1]
    out = np.zeros((B * H, D))
    for b in range(B):
        L = int(kv[b])
        if L == 0:
            continue
        o, _ = oracle.attention(q[b:b + 1].float().numpy(), K[b:b + 1, :, :L].float().numpy(),
                                V[b:b + 1, :, :L].float().numpy(), scale, False)
        out[b * H:(b + 1) * H] = o.reshape(H, D)
    return out


def test_decode_full_size():
    """The decode workload at full size (B16 H32, KV lengths uniform in
    [1, 32768], D128, 64 splits) in the launch configuration the benchmark
    times: every one of the 512 (b, h) outputs against the oracle, element by
    element; two runs bit-identical (no atomics)."""
    w = inputs.WORKLOADS["decode_splitkv"]
    B, H, Lmax, D, S = w["B"], w["H"], w["Lmax"], w["D"], w["num_splits"]
    say(f"decode full size B{B} H{H} Lmax{Lmax} D{D} splits{S}")
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=501)
    scale = 1.0 / math.sqrt(D)
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    o = tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=S, scale=scale)
    o2 = tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=S, scale=scale)
    of = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)  # deterministic: no atomics
    assert bool(torch.isfinite(o).all())
    say(f"decode full size: oracle over all {B * H} (b, h) pairs")
    ref = _decode_ref_all(q, K, V, kv.numpy(), scale)
    err = check_attention(to_np(o).reshape(-1, D), ref, "decode full size")
    errf = check_attention(to_np(of).reshape(-1, D), ref, "decode full size, one launch")
    print(f"decode: max abs err {err:.3e} (one launch {errf:.3e}) over all {B * H} (b, h) pairs; "
          f"kv_len={kv.tolist()}")


def test_decode_beyond_2_31_elements():
    """K and V of 2.15e9 elements each (B4 H64 Lmax 65600 D128, lengths
    40000, 1, 65599 and 65600): the last sequences' heads sit past element
    2^31 and are reached through 64-bit offsets.  The padding past each
    length holds random values (no kernel may read it).  Two-launch (64
    splits) and one-launch forms; the first, middle and last heads of every
    sequence against the oracle in full."""
    B, H, Lmax, D, S = 4, 64, 65600, 128, 64
    assert B * H * Lmax * D > 2 ** 31
    say(f"decode past 2^31 elements: B{B} H{H} Lmax{Lmax} D{D} splits{S}")
    kv = torch.tensor([40000, 1, 65599, 65600], dtype=torch.int32)
    q = inputs.device_normal((B, H, 1, D), 631, DEV, dtype="bf16")
    K = inputs.device_normal((B, H, Lmax, D), 632, DEV, dtype="bf16")
    V = inputs.device_normal((B, H, Lmax, D), 633, DEV, dtype="bf16")
    scale = 1.0 / math.sqrt(D)
    kvd = kv.to(DEV)
    o = tea.attn_decode_splitkv(q, K, V, kvd, num_splits=S, scale=scale)
    of = tea.attn_decode_fused(q, K, V, kvd, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    for b in range(B):
        L = int(kv[b])
        for h in (0, H // 2, H - 1):
            ref, _ = oracle.attention(q[b:b + 1, h:h + 1].float().cpu().numpy(),
                                      K[b:b + 1, h:h + 1, :L].float().cpu().numpy(),
                                      V[b:b + 1, h:h + 1, :L].float().cpu().numpy(), scale, False)
            ref = ref.reshape(1, D)
            check_attention(to_np(o[b, h]).reshape(1, D), ref, f"two launches b={b} h={h} L={L}")
            check_attention(to_np(of[b, h]).reshape(1, D), ref, f"one launch b={b} h={h} L={L}")
    del K, V


# ---- attn_decode_fused: the single-launch form ------------------------------

@pytest.mark.parametrize("lengths", [[1, 2, 63, 64], [65, 511, 512, 513], [1000, 4096, 32767, 32768], [0, 5, 0, 70]])
@pytest.mark.parametrize("splits", [1, 3, 16, 64])
def test_decode_fused_edge_lengths(lengths, splits):
    say(f"decode fused lengths={lengths} splits={splits}")
    B, H, D = len(lengths), 3, 128
    Lmax = max(max(lengths), 1)
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=sum(lengths) + splits + 7, kv_len=np.array(lengths))
    scale = 1.0 / math.sqrt(D)
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    o = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=splits, scale=scale)
    o32 = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=splits, scale=scale, out_dtype=torch.float32)
    o2 = tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=splits, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(B) for h in range(H)]
    ref = _decode_ref(q, K, V, kv.numpy(), scale, pairs)
    check_attention(to_np(o).reshape(-1, D), ref, f"fused lengths={lengths} splits={splits}")
    # the two forms share chunk bounds, tree and combine; only the order of
    # the fp32 sums inside a chunk differs
    assert float((o32 - o2).abs().max()) <= 1e-5
    for b in range(B):
        if lengths[b] == 0:
            assert torch.all(o[b] == 0)


def test_decode_fused_d64_full_size_sampled():
    say("decode fused D=64 fp32 out; full-size workload sampled")
    q, K, V, kv = inputs.decode_inputs(3, 4, 3000, 64, seed=19, kv_len=np.array([3000, 17, 1234]))
    o = tea.attn_decode_fused(q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV), num_splits=64, scale=0.125,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    pairs = [(b, h) for b in range(3) for h in range(4)]
    check_attention(to_np(o).reshape(-1, 64), _decode_ref(q, K, V, kv.numpy(), 0.125, pairs), "fused D64", atol=2e-3)
    w = inputs.WORKLOADS["decode_splitkv"]
    B, H, Lmax, D, S = w["B"], w["H"], w["Lmax"], w["D"], w["num_splits"]
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=501)
    scale = 1.0 / math.sqrt(D)
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    o = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=S, scale=scale)
    o2 = tea.attn_decode_fused(qd, Kd, Vd, kvd, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    pairs = [(0, 0), (B - 1, H - 1), (int(np.argmax(kv.numpy())), 5), (int(np.argmin(kv.numpy())), 9)]
    got = np.stack([to_np(o[b, h]) for b, h in pairs])
    check_attention(got, _decode_ref(q, K, V, kv.numpy(), scale, pairs), "fused full size")


# ---- merge_partials ----------------------------------------------------------

def _merge_ref(m, l, O):
    mo, lo, Oo = oracle.merge_direct(m.numpy(), l.numpy(), O.numpy())
    with np.errstate(invalid="ignore", divide="ignore"):
        on = np.where(lo[:, None] > 0, Oo / np.where(lo > 0, lo, 1.0)[:, None], 0.0)
    return mo, lo, Oo, on


@pytest.mark.parametrize("S", [1, 2, 3, 63, 64, 65, 200, 1024])
@pytest.mark.parametrize("D", [1, 7, 8, 64, 128])
def test_merge_parity(S, D):
    say(f"merge S={S} D={D}")
    N = 50
    m, l, O = inputs.partials(N, S, D, seed=S * 131 + D, empty_frac=0.1)
    o, mo, lo = tea.merge_partials(m.to(DEV), l.to(DEV), O.to(DEV), stats=True)
    torch.cuda.synchronize()
    mref, lref, _, oref = _merge_ref(m, l, O)
    assert np.array_equal(to_np(mo).astype(np.float64), mref)
    ok = lref > 0
    assert np.all(np.abs(to_np(lo)[ok] - lref[ok]) <= 2e-5 * lref[ok])
    assert np.all(to_np(lo)[~ok] == 0) and np.all(to_np(o)[~ok] == 0)
    # fp32 weights exp(m_s - M) carry ~|m_s - M| * 2^-24 relative error; the
    # partials here spread m over +-40, so 3e-5 of the row's magnitude
    scale = np.maximum(np.abs(oref).max(axis=1, keepdims=True), 1.0)
    assert np.max(np.abs(to_np(o) - oref) / scale) <= 3e-5


def test_merge_unnormalised_bf16_and_identity():
    say("merge unnormalised / bf16 / identity")
    N, S, D = 40, 64, 128
    m, l, O = inputs.partials(N, S, D, seed=77)
    mref, lref, Oref, oref = _merge_ref(m, l, O)
    u = tea.merge_partials(m.to(DEV), l.to(DEV), O.to(DEV), normalize=False)
    b = tea.merge_partials(m.to(DEV), l.to(DEV), O.to(DEV), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.max(np.abs(to_np(u) - Oref) / np.abs(Oref).max(axis=1, keepdims=True)) <= 3e-5
    check_attention(to_np(b), oref, "merge bf16")
    # appending empty partials changes nothing, bitwise
    e_m = torch.full((N, S), -math.inf)
    e_l = torch.zeros((N, S))
    e_O = torch.zeros((N, S, D))
    m2 = torch.cat([m, e_m], 1)
    l2 = torch.cat([l, e_l], 1)
    O2 = torch.cat([O, e_O], 1)
    a1 = tea.merge_partials(m.to(DEV), l.to(DEV), O.to(DEV))
    a2 = tea.merge_partials(m2.to(DEV), l2.to(DEV), O2.to(DEV))
    torch.cuda.synchronize()
    # With 128 partials each lane first folds two ((identity, p), p'), which
    # is the first tree level of the 64-partial merge; the upper 32 lanes
    # hold only empty states, and combining with the empty state is exact.
    assert torch.equal(a1, a2)
    # all-empty rows
    z, zm, zl = tea.merge_partials(e_m.to(DEV), e_l.to(DEV), e_O.to(DEV), stats=True)
    torch.cuda.synchronize()
    assert torch.all(z == 0) and torch.all(zm == -math.inf) and torch.all(zl == 0)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 13, 16, 31, 32])
@pytest.mark.parametrize("D", [7, 64, 128, 200])
def test_merge_few_partials_match_padded(S, D):
    """Up to 32 partials per row are merged by a kernel with one wave per
    row; padded with empty states to 64 partials the same rows go through
    the butterfly kernel.  Both build the balanced tree over the partial
    index (the padding's combines are exact no-ops), so the outputs, m and
    l agree bit for bit, normalised and not, bf16 and fp32."""
    say(f"merge few partials S={S} D={D}")
    N = 300
    m, l, O = inputs.partials(N, S, D, seed=S * 1000 + D, empty_frac=0.1)
    pad = 64 - S
    m2 = torch.cat([m, torch.full((N, pad), -math.inf)], 1)
    l2 = torch.cat([l, torch.zeros((N, pad))], 1)
    O2 = torch.cat([O, torch.zeros((N, pad, D))], 1)
    dm, dl, dO = m.to(DEV), l.to(DEV), O.to(DEV)
    pm2, pl2, pO2 = m2.to(DEV), l2.to(DEV), O2.to(DEV)
    for kw in (dict(), dict(normalize=False), dict(out_dtype=torch.bfloat16)):
        a, am, al = tea.merge_partials(dm, dl, dO, stats=True, **kw)
        b, bm, bl = tea.merge_partials(pm2, pl2, pO2, stats=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a, b), f"S={S} D={D} {kw}"
        assert torch.equal(am, bm) and torch.equal(al, bl)
    mref, lref, Oref, oref = _merge_ref(m, l, O)
    check_attention(to_np(tea.merge_partials(dm, dl, dO)), oref, f"merge S={S} D={D}")


def test_merge_tree_shapes_agree():
    """Merging 64 partials at once, or as two merged halves merged again,
    agrees up to rounding (the combine is associative)."""
    say("merge tree shapes")
    N, S, D = 30, 64, 64
    m, l, O = (t.to(DEV) for t in inputs.partials(N, S, D, seed=78))
    whole = tea.merge_partials(m, l, O)
    halves = [tea.merge_partials(m[:, i:i + 32].contiguous(), l[:, i:i + 32].contiguous(),
                                 O[:, i:i + 32].contiguous(), normalize=False, stats=True) for i in (0, 32)]
    mm = torch.stack([h[1] for h in halves], 1)
    ll = torch.stack([h[2] for h in halves], 1)
    OO = torch.stack([h[0] for h in halves], 1)
    again = tea.merge_partials(mm.contiguous(), ll.contiguous(), OO.contiguous())
    torch.cuda.synchronize()
    assert float((whole - again).abs().max()) <= 3e-5 * float(whole.abs().max())
