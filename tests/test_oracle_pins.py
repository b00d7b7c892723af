"""Pins for the fp64 CPU oracle, against what the pages and mathematics fix.

Sources (page title, section):
  [OS-R] "Online softmax" (roadmapper): The recurrence; Why the values are
         preserved; Initialise honestly; Things that break.
  [OS-C] "The Online Softmax" (curionode, Vol. XVI plate 3): intro; Workshop;
         One pass, exactly; Terms.
  [OS-M] "Online Softmax" (metalworking): The problem; Recognition guide.

Each check is independent of the oracle's own code: printed values of the
worked example (tests/golden), closed forms, invariants, 50-digit decimal
brute force, and torch's fp64 CPU routines.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workshop_64.json")
FP64_REL = 4e-15  # a few ulp of fp64 (the printed error 4.4e-16 is 4 ulp at 2**-53 ~ 1.1e-16)


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _vec(seed, scale=1.0):
    return np.random.default_rng([seed, 7]).standard_normal(64) * scale


def _rel(a, b):
    return abs(a - b) / abs(b)


def _block_rescales(x, B):
    """Independent count of blocks whose maximum strictly exceeds the maximum
    of everything before them (the first block excluded)."""
    bm = [x[i:i + B].max() for i in range(0, len(x), B)]
    run = np.maximum.accumulate(bm)
    return int(sum(1 for k in range(1, len(bm)) if bm[k] > run[k - 1]))


# ---- worked example: [OS-C] One pass, exactly --------------------------------

def test_workshop_updates_match_printed_count():
    g = _golden()
    x = _vec(0)
    assert oracle.online_trace(x, g["block"])["updates"] == g["updates"]
    assert oracle.online_trace(x, 1)["updates"] == 64
    for B in (3, 7, 64, 100):
        assert oracle.online_trace(x, B)["updates"] == -(-64 // B)


def test_rescales_exactly_when_maximum_rises():
    counts = []
    for seed in range(300):
        x = _vec(seed)
        c1 = oracle.online_trace(x, 1)["rescales"]
        records = int(sum(1 for i in range(1, 64) if x[i] > x[:i].max()))
        assert c1 == records
        for B in (2, 3, 8, 64):
            t = oracle.online_trace(x, B)
            assert t["rescales"] == _block_rescales(x, B)
            assert t["rescales"] <= c1
            # the correction is exactly 1 on blocks that do not raise the max
            bm = [x[i:i + B].max() for i in range(0, 64, B)]
            run = np.maximum.accumulate(bm)
            for k in range(1, len(bm)):
                if bm[k] <= run[k - 1]:
                    assert t["c_trace"][k] == 1.0
                else:
                    assert 0.0 < t["c_trace"][k] < 1.0
        counts.append((oracle.online_trace(x, 8)["rescales"], c1))
    # the printed example (2 rescales with blocks of 8 and with blocks of 1)
    # is a case the rule produces for some draws
    g = _golden()
    assert (g["rescales_printed"], g["block_one_rescales_printed"]) in counts


def test_online_normaliser_matches_two_pass_to_rounding():
    g = _golden()
    errs = []
    for seed in range(2000):
        x = _vec(seed)
        t = oracle.online_trace(x, g["block"])
        _, m, l = oracle.softmax_f64(x)
        assert t["m"] == m
        errs.append(_rel(t["l"], l))
    assert max(errs) <= FP64_REL
    # the printed error is of the same order as the typical one
    assert np.median(errs) <= 10 * g["relative_error_printed"]


def test_large_scale_naive_overflows_online_stays_exact():
    g = _golden()
    exact_zero = 0
    for seed in range(500):
        x = _vec(seed, g["scale_large"])
        s, _, finite = oracle.naive_normaliser(x)
        assert finite is g["naive_finite_at_large_scale"] and math.isinf(s)
        t = oracle.online_trace(x, g["block"])
        _, m, l = oracle.softmax_f64(x)
        assert math.isfinite(t["l"]) and t["l"] >= 1.0
        err = _rel(t["l"], l)
        assert err <= FP64_REL
        exact_zero += err == 0.0
    assert exact_zero >= 450  # the printed "0" is the typical case


def test_naive_normaliser_at_unit_scale():
    x = _vec(3)
    s, rel, finite = oracle.naive_normaliser(x)
    assert finite
    assert _rel(s, math.fsum(math.exp(v) for v in x)) < 1e-14
    _, m, l = oracle.softmax_f64(x)
    assert _rel(rel, l) < 1e-13


@pytest.mark.parametrize("scale", [1.0, 30.0, 1000.0])
def test_block_size_invariance(scale):
    for seed in range(100):
        x = _vec(seed, scale)
        _, m, l = oracle.softmax_f64(x)
        for B in (1, 2, 3, 7, 8, 64):
            t = oracle.online_trace(x, B)
            assert t["m"] == m
            assert _rel(t["l"], l) <= FP64_REL


def test_equivalent_forms():
    """[OS-R] Initialise honestly (l0 = 1 also works); [OS-M] Recognition
    guide (conditional and unconditional correction); [OS-R] Things that break
    (base two works when every exponential is base two)."""
    for seed in range(200):
        x = _vec(seed, 5.0)
        ref = oracle.online_trace(x, 8)
        for v in ("l0_one", "conditional"):
            t = oracle.online_trace(x, 8, v)
            assert t["l"] == ref["l"] and t["m"] == ref["m"]
            assert np.array_equal(t["l_trace"], ref["l_trace"])
        b2 = oracle.online_trace(x, 8, "base2")
        assert _rel(b2["l"], ref["l"]) <= FP64_REL


def test_correction_factor_bounds():
    """[OS-M] The problem: the correction is at most 1; [OS-R] Initialise
    honestly: it is 0 on the first non-empty block."""
    for seed in range(200):
        t = oracle.online_trace(_vec(seed, 3.0), 8)
        c = t["c_trace"]
        assert c[0] == 0.0
        assert np.all((c >= 0.0) & (c <= 1.0))


# ---- failure modes: [OS-R] Initialise honestly, Things that break ------------

def _rising(n, D, seed):
    """Scores with a maximum that keeps rising across blocks."""
    rng = np.random.default_rng(seed)
    s = np.sort(rng.standard_normal(n)) * 3.0
    V = rng.standard_normal((n, D))
    return s, V


def _definition_row(s, V):
    y, _, _ = oracle.softmax_f64(s)
    return y @ V


def test_online_attention_row_matches_definition():
    for seed in range(50):
        rng = np.random.default_rng(seed)
        n = int(rng.integers(1, 200))
        s = rng.standard_normal(n) * 4
        V = rng.standard_normal((n, 16))
        ref = _definition_row(s, V)
        for B in (1, 5, 16, 1000):
            o, _, _ = oracle.online_attention_row(s, V, B)
            assert np.max(np.abs(o - ref)) <= 1e-13


def test_bug_rescale_l_not_acc_passes_short_fails_long():
    s, V = _rising(256, 8, 1)
    ref = _definition_row(s, V)
    o1, _, _ = oracle.online_attention_row(s[:16], V[:16], 16, "bug_rescale_l_only")
    assert np.max(np.abs(o1 - _definition_row(s[:16], V[:16]))) <= 1e-13  # one tile: fine
    o, _, _ = oracle.online_attention_row(s, V, 16, "bug_rescale_l_only")
    assert np.max(np.abs(o - ref)) > 1e-2  # many tiles: drifts


def test_bug_rescale_acc_not_l_fails():
    s, V = _rising(256, 8, 2)
    o, _, _ = oracle.online_attention_row(s, V, 16, "bug_rescale_acc_only")
    assert np.max(np.abs(o - _definition_row(s, V))) > 1e-2


def test_bug_mixed_bases_fails():
    s, V = _rising(256, 8, 3)
    o, _, _ = oracle.online_attention_row(s, V, 16, "bug_mixed_bases")
    assert np.max(np.abs(o - _definition_row(s, V))) > 1e-2
    x = np.sort(_vec(4, 3.0))
    t = oracle.online_trace(x, 8, "bug_mixed_bases")
    _, _, l = oracle.softmax_f64(x)
    assert _rel(t["l"], l) > 1e-3


def test_bug_max_not_carried_fails():
    # the largest logit in the first block: later blocks have smaller maxima
    x = _vec(5, 1000.0)
    x[0] = abs(x).max() + 1.0
    t = oracle.online_trace(x, 8, "bug_no_carry")
    _, m, l = oracle.softmax_f64(x)
    assert not (t["m"] == m and math.isfinite(t["l"]) and _rel(t["l"], l) < 1e-6)


def test_bug_no_guard_empty_first_block_is_nan():
    x = np.concatenate([np.full(8, -np.inf), _vec(6)])
    bad = oracle.online_trace(x, 8, "bug_no_guard")
    assert math.isnan(bad["l"])
    good = oracle.online_trace(x, 8)
    _, m, l = oracle.softmax_f64(x)
    assert good["m"] == m and _rel(good["l"], l) <= FP64_REL
    s = np.concatenate([np.full(8, -np.inf), np.random.default_rng(0).standard_normal(24)])
    V = np.random.default_rng(1).standard_normal((32, 4))
    o, _, _ = oracle.online_attention_row(s, V, 8, "bug_no_guard")
    assert np.all(np.isnan(o))
    o, _, _ = oracle.online_attention_row(s, V, 8)
    assert np.max(np.abs(o - _definition_row(s, V))) <= 1e-13


def test_empty_set_is_merge_identity():
    y, m, l = oracle.softmax_f64(np.full(5, -np.inf))
    assert m == -math.inf and l == 0.0 and np.all(y == 0.0)
    Q = np.zeros((1, 1, 1, 4), np.float32)
    K = np.zeros((1, 1, 0, 4), np.float32)
    O, lse = oracle.attention(Q, K, K, 1.0)
    assert np.all(O == 0.0) and lse[0, 0, 0] == -math.inf


# ---- rows sum to one; closed forms --------------------------------------------

@pytest.mark.parametrize("scale", [1.0, 30.0, 1000.0])
def test_rows_sum_to_one(scale):
    x = (np.random.default_rng(11).standard_normal((64, 1000)) * scale).astype(np.float32)
    y, m, l = oracle.softmax_rows(x)
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) <= 1e-13
    assert np.array_equal(m, x.max(axis=1).astype(np.float64))
    assert np.all(y >= 0.0) and np.all(y <= 1.0)


def test_closed_forms_softmax():
    for n in (1, 2, 7, 1000):
        y, _, l = oracle.softmax_rows(np.full((1, n), 3.25, np.float32))
        assert np.all(y == 1.0 / n) and l[0] == n
    for a, b in [(0.0, 1.0), (2.5, -1.25), (100.0, 90.0)]:
        y, _, _ = oracle.softmax_rows(np.array([[a, b]], np.float32))
        assert abs(y[0, 0] - 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
    x = np.random.default_rng(2).standard_normal((4, 33)).astype(np.float32)
    y0, _, _ = oracle.softmax_rows(x)
    y1, _, _ = oracle.softmax_rows(x + np.float32(8.0))  # exact shift in fp32 here
    assert np.max(np.abs(y0 - y1) / y0) <= 1e-5  # the shifted fp32 inputs round


def test_closed_forms_attention():
    rng = np.random.default_rng(3)
    V = rng.standard_normal((1, 2, 5, 8)).astype(np.float32)
    Q = rng.standard_normal((1, 2, 5, 8)).astype(np.float32)
    K = rng.standard_normal((1, 2, 5, 8)).astype(np.float32)
    # one key: O = v0 exactly
    O, _ = oracle.attention(Q, K[:, :, :1], V[:, :, :1], 0.3)
    assert np.array_equal(O, np.broadcast_to(V[:, :, :1].astype(np.float64), O.shape))
    # causal row 0 sees only key 0
    O, lse = oracle.attention(Q, K, V, 0.3, causal=True)
    assert np.array_equal(O[:, :, 0], V[:, :, 0].astype(np.float64))
    # identical keys: uniform weights, O = mean(V)
    Kc = np.broadcast_to(K[:, :, :1], K.shape).copy()
    O, lse = oracle.attention(Q, Kc, V, 0.3)
    assert np.max(np.abs(O - V.astype(np.float64).mean(axis=2, keepdims=True))) <= 1e-14
    # constant V: constant O
    Vc = np.full_like(V, 1.5)
    O, _ = oracle.attention(Q, K, Vc, 0.3, causal=True)
    assert np.max(np.abs(O - 1.5)) <= 1e-14


# ---- 50-digit decimal brute force (no maximum subtracted) --------------------

getcontext().prec = 50


def _dec_softmax(x):
    ex = [Decimal(float(v)).exp() for v in x]
    s = sum(ex)
    return [e / s for e in ex], s


@pytest.mark.parametrize("scale", [1.0, 30.0, 1000.0])
def test_decimal_brute_force_softmax(scale):
    x = (np.random.default_rng(21).standard_normal((3, 9)) * scale).astype(np.float32)
    y, m, l = oracle.softmax_rows(x)
    for r in range(3):
        yd, sd = _dec_softmax(x[r])
        for j in range(9):
            ref = float(yd[j])
            if ref > 1e-300:
                assert abs(y[r, j] - ref) <= 1e-14 * ref
            else:
                assert y[r, j] <= 1e-300
        # l is the normaliser relative to the maximum
        lref = float(sd / Decimal(float(m[r])).exp())
        assert _rel(l[r], lref) <= 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_decimal_brute_force_attention(causal):
    rng = np.random.default_rng(22)
    B, H, S, D = 1, 2, 5, 4
    Q = rng.standard_normal((B, H, S, D)).astype(np.float32)
    K = rng.standard_normal((B, H, S, D)).astype(np.float32)
    V = rng.standard_normal((B, H, S, D)).astype(np.float32)
    scale = 0.37
    O, lse = oracle.attention(Q, K, V, scale, causal)
    for h in range(H):
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            sc = [Decimal(scale) * sum(Decimal(float(Q[0, h, i, d])) * Decimal(float(K[0, h, j, d]))
                                       for d in range(D)) for j in keys]
            ex = [s.exp() for s in sc]
            tot = sum(ex)
            for d in range(D):
                ref = float(sum(e * Decimal(float(V[0, h, j, d])) for e, j in zip(ex, keys)) / tot)
                assert abs(O[0, h, i, d] - ref) <= 1e-14 * max(1.0, abs(ref))
            assert abs(lse[0, h, i] - float(tot.ln())) <= 1e-14 * max(1.0, abs(float(tot.ln())))


# ---- library cross-check (torch fp64 on the CPU) ------------------------------

def test_torch_crosscheck_softmax():
    x = (np.random.default_rng(31).standard_normal((16, 777)) * 30).astype(np.float32)
    y, m, l = oracle.softmax_rows(x)
    t = torch.softmax(torch.from_numpy(x).double(), dim=1).numpy()
    assert np.max(np.abs(y - t)) <= 1e-12
    lse = torch.logsumexp(torch.from_numpy(x).double(), dim=1).numpy()
    assert np.max(np.abs(m + np.log(l) - lse)) <= 1e-12


@pytest.mark.parametrize("causal,Sq,Sk", [(False, 7, 13), (False, 33, 5), (True, 19, 19)])
def test_torch_crosscheck_attention(causal, Sq, Sk):
    rng = np.random.default_rng(32)
    B, H, D = 2, 3, 16
    Q = rng.standard_normal((B, H, Sq, D)).astype(np.float32)
    K = rng.standard_normal((B, H, Sk, D)).astype(np.float32)
    V = rng.standard_normal((B, H, Sk, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    O, lse = oracle.attention(Q, K, V, scale, causal)
    q, k, v = (torch.from_numpy(a).double() for a in (Q, K, V))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale).numpy()
    assert np.max(np.abs(O - ref)) <= 1e-12
    s = (q @ k.transpose(-1, -2)) * scale
    if causal:
        s = s.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(1), float("-inf"))
    assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-12


# ---- merge algebra: [OS-C] One pass, exactly; [OS-M] Recognition guide --------

@settings(max_examples=60, deadline=None)
@given(n=st.integers(0, 120), D=st.integers(1, 9), seed=st.integers(0, 10**6),
       ncuts=st.integers(0, 12), data=st.data())
def test_merge_any_partition_order_tree(n, D, seed, ncuts, data):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal(n) * 6
    V = rng.standard_normal((n, D))
    cuts = sorted(data.draw(st.lists(st.integers(0, n), min_size=ncuts, max_size=ncuts)))
    bounds = [0] + cuts + [n]
    parts = [oracle.partial(s[a:b], V[a:b].reshape(b - a, D)) for a, b in zip(bounds[:-1], bounds[1:])]
    # direct definition of the whole set
    m_ref, l_ref, O_ref = oracle.partial(s, V.reshape(n, D))
    # left fold in a random order
    order = data.draw(st.permutations(range(len(parts))))
    acc = (-math.inf, 0.0, np.zeros(D))
    for i in order:
        acc = oracle.combine(acc, parts[i])
    # a random tree
    pool = list(parts)
    while len(pool) > 1:
        i = data.draw(st.integers(0, len(pool) - 2))
        pool[i:i + 2] = [oracle.combine(pool[i], pool[i + 1])]
    for m, l, O in (acc, pool[0]):
        assert m == m_ref
        if l_ref == 0.0:
            assert l == 0.0 and np.all(O == 0.0)
        else:
            assert _rel(l, l_ref) <= 1e-14
            assert np.max(np.abs(O / l - O_ref / l_ref)) <= 1e-14
    # the direct merge formula agrees too
    mm, ll, OO = oracle.merge_direct(np.array([[p[0] for p in parts]]), np.array([[p[1] for p in parts]]),
                                     np.array([[p[2] for p in parts]]))
    assert mm[0] == m_ref
    if l_ref > 0:
        assert _rel(ll[0], l_ref) <= 1e-14
        assert np.max(np.abs(OO[0] / ll[0] - O_ref / l_ref)) <= 1e-14
    else:
        assert ll[0] == 0.0 and np.all(OO[0] == 0.0)


def test_merge_identity_is_bitwise():
    rng = np.random.default_rng(41)
    for _ in range(100):
        p = (float(rng.standard_normal() * 50), float(rng.uniform(0.1, 9)), rng.standard_normal(5))
        e = (-math.inf, 0.0, np.zeros(5))
        for a, b in ((p, e), (e, p)):
            m, l, O = oracle.combine(a, b)
            assert m == p[0] and l == p[1] and np.array_equal(O, p[2])
    m, l, O = oracle.combine((-math.inf, 0.0, np.zeros(3)), (-math.inf, 0.0, np.zeros(3)))
    assert m == -math.inf and l == 0.0 and np.all(O == 0.0)


def test_split_kv_chunks_reach_full_decode():
    """Keys cut into num_splits balanced contiguous chunks
    [floor(c L / S), floor((c+1) L / S)), partials merged, equal the decode
    result from the definition; L < S leaves chunks empty."""
    rng = np.random.default_rng(42)
    D = 8
    for L, S in [(1, 64), (5, 64), (63, 64), (64, 64), (65, 64), (1000, 64), (777, 7), (3, 1)]:
        q = rng.standard_normal(D).astype(np.float32)
        K = rng.standard_normal((L, D)).astype(np.float32)
        V = rng.standard_normal((L, D)).astype(np.float32)
        scale = 0.25
        O, lse = oracle.attention(q.reshape(1, 1, 1, D), K.reshape(1, 1, L, D), V.reshape(1, 1, L, D), scale)
        s = scale * (K.astype(np.float64) @ q.astype(np.float64))
        parts = []
        for c in range(S):
            a, b = (c * L) // S, ((c + 1) * L) // S
            parts.append(oracle.partial(s[a:b], V[a:b].astype(np.float64).reshape(b - a, D)))
        while len(parts) > 1:  # balanced pairwise tree
            nxt = [oracle.combine(parts[i], parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        m, l, Ou = parts[0]
        assert np.max(np.abs(Ou / l - O.reshape(D))) <= 1e-13
        assert abs(m + math.log(l) - lse.reshape(())) <= 1e-13


def test_decode_wrapper_matches_attention():
    rng = np.random.default_rng(43)
    B, H, Lmax, D = 3, 2, 40, 8
    q = rng.standard_normal((B, H, 1, D)).astype(np.float32)
    K = rng.standard_normal((B, H, Lmax, D)).astype(np.float32)
    V = rng.standard_normal((B, H, Lmax, D)).astype(np.float32)
    kv = np.array([1, 40, 17], np.int32)
    O, lse = oracle.decode(q, K, V, kv, 0.5)
    for n, (b, h) in enumerate([(b, h) for b in range(B) for h in range(H)]):
        L = kv[b]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b, h]).double()[None], torch.from_numpy(K[b, h, :L]).double()[None],
            torch.from_numpy(V[b, h, :L]).double()[None], scale=0.5).numpy().reshape(D)
        assert np.max(np.abs(O[n] - ref)) <= 1e-12


@pytest.mark.parametrize("S", [1, 2, 7, 64, 1024])
def test_merge_direct_output_matches_attention_of_whole_set(S):
    """The merged state written out directly (oracle_merge_direct) for N rows
    of S partials each equals attention over the whole set, for the output as
    well as the normaliser ([OS-C] One pass, exactly: partial results merge
    into the result of the whole set, in any order or tree).

    Each row's keys are cut into S contiguous chunks at random points
    (repeated cut points give empty chunks; with S = 1024 and 300 keys most
    chunks are empty), each chunk's partial (m, l, unnormalised O) is taken
    with oracle_partial, and the partials of a row are shuffled before the
    merge.  The whole-set result comes from oracle_attention, which decimal
    brute force and torch's scaled_dot_product_attention pin above:
    O / l matches it to 1e-13, m is the largest score and m + ln l the
    log-sum-exp.  A row whose partials are all empty merges to (-inf, 0, 0)."""
    rng = np.random.default_rng(50 + S)
    N, L, D = 6, 300, 12
    scale = 0.7
    q = rng.standard_normal((1, N, 1, D)).astype(np.float32)
    K = (rng.standard_normal((1, N, L, D)) * 1.5).astype(np.float32)
    V = rng.standard_normal((1, N, L, D)).astype(np.float32)
    O_ref, lse_ref = oracle.attention(q, K, V, scale, False)
    m = np.empty((N + 1, S))
    l = np.empty((N + 1, S))
    Op = np.empty((N + 1, S, D))
    smax = np.empty(N)
    for n in range(N):
        s = scale * (K[0, n].astype(np.float64) @ q[0, n, 0].astype(np.float64))
        smax[n] = s.max()
        cuts = np.sort(rng.integers(0, L + 1, S - 1))
        bounds = [0, *cuts.tolist(), L]
        order = rng.permutation(S)
        for slot, c in enumerate(order):
            a, b = bounds[c], bounds[c + 1]
            m[n, slot], l[n, slot], Op[n, slot] = oracle.partial(s[a:b], V[0, n, a:b].astype(np.float64).reshape(b - a, D))
    m[N], l[N], Op[N] = -math.inf, 0.0, 0.0  # a row with no key at all
    mm, ll, OO = oracle.merge_direct(m, l, Op)
    for n in range(N):
        assert abs(mm[n] - smax[n]) <= 1e-15 * abs(smax[n])
        assert np.max(np.abs(OO[n] / ll[n] - O_ref[0, n, 0])) <= 1e-13
        assert abs(mm[n] + math.log(ll[n]) - lse_ref[0, n, 0]) <= 1e-13
    assert mm[N] == -math.inf and ll[N] == 0.0 and np.all(OO[N] == 0.0)
