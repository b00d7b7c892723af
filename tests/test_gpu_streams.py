"""Every entry point runs on the stream it is given: results on a side stream
equal those on the default stream bit for bit, and the calls (which allocate
nothing and never synchronise) can be captured in a HIP graph and replayed."""
import numpy as np
import pytest
import torch

import tiled_exact_attention_amd as tea
from tiled_exact_attention_amd import inputs
from gpu_util import say, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    t = t.contiguous()
    if t.dtype == torch.float32:
        return to_np(t.view(torch.int32))
    return to_np(t.view(torch.int16))


def _calls():
    """The entry points on small inputs: name -> (function writing into
    preallocated outputs, list of output tensors)."""
    torch.manual_seed(0)
    x = inputs.logits(64, 3000, 30.0, 11, "f32").to(DEV)
    y = torch.empty_like(x)
    y2 = torch.empty_like(x)
    q, k, v = (t.to(DEV) for t in inputs.qkv(2, 3, 333, 333, 128, seed=12))
    o = torch.empty_like(q)
    ns = 5
    wsk = torch.empty(tea.attn_fwd_splitk_workspace_bytes(2, 3, 333, 128, ns), dtype=torch.uint8, device=DEV)
    osk = torch.empty_like(q)
    qd, K, V, kv = inputs.decode_inputs(3, 4, 2000, 128, seed=13)
    qd, K, V, kv = qd.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    wsd = torch.empty(tea.attn_decode_workspace_bytes(3, 4, 128, 16), dtype=torch.uint8, device=DEV)
    od = torch.empty((3, 4, 128), dtype=torch.bfloat16, device=DEV)
    of = torch.empty((3, 4, 128), dtype=torch.bfloat16, device=DEV)
    on = torch.empty((3, 4, 128), dtype=torch.bfloat16, device=DEV)
    # merge_partials with 8 partials per row (one wave per row) and 64 (butterfly)
    pm8, pl8, pO8 = (t.to(DEV) for t in inputs.partials(500, 8, 128, seed=14, empty_frac=0.1))
    pm64, pl64, pO64 = (t.to(DEV) for t in inputs.partials(100, 64, 96, seed=15, empty_frac=0.1))
    om8 = torch.empty((500, 128), dtype=torch.float32, device=DEV)
    om64 = torch.empty((100, 96), dtype=torch.bfloat16, device=DEV)
    return {
        "row_softmax": (lambda: tea.row_softmax(x, out=y, block=8), [y]),
        "row_softmax_variant": (lambda: tea.row_softmax_variant(x, tea.TEA_RESCALE_IF_RISE, out=y2), [y2]),
        "attn_fwd": (lambda: tea.attn_fwd(q, k, v, causal=True, out=o), [o]),
        "attn_fwd_splitk": (lambda: tea.attn_fwd_splitk(q, k, v, ns, workspace=wsk, out=osk), [osk]),
        "attn_decode_splitkv": (lambda: tea.attn_decode_splitkv(qd, K, V, kv, num_splits=16, workspace=wsd, out=od),
                                [od]),
        "attn_decode_fused": (lambda: tea.attn_decode_fused(qd, K, V, kv, num_splits=16, out=of), [of]),
        # partials in the library's static scratch: nothing allocated, so it
        # can be captured once its scratch address is known (first call)
        "attn_decode_splitkv_noalloc": (lambda: tea.attn_decode_splitkv_noalloc(qd, K, V, kv, on, num_splits=16),
                                        [on]),
        "merge_partials_8": (lambda: tea.merge_partials(pm8, pl8, pO8, out=om8), [om8]),
        "merge_partials_64": (lambda: tea.merge_partials(pm64, pl64, pO64, out_dtype=torch.bfloat16, out=om64), [om64]),
    }


def test_side_stream_matches_default_stream():
    calls = _calls()
    ref = {}
    for name, (fn, outs) in calls.items():
        say(f"default stream: {name}")
        fn()
        torch.cuda.synchronize()
        ref[name] = [_bits(t) for t in outs]
    s = torch.cuda.Stream()  # default priority
    for name, (fn, outs) in calls.items():
        say(f"side stream: {name}")
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            fn()
        s.synchronize()
        for r, t in zip(ref[name], outs):
            assert np.array_equal(r, _bits(t)), f"{name}: side-stream result differs"


def test_graph_capture_and_replay():
    calls = _calls()
    say("graph capture of every entry point")
    eager = {}
    for name, (fn, outs) in calls.items():
        fn()
        torch.cuda.synchronize()
        eager[name] = [_bits(t) for t in outs]
    # warm up on a side stream, as torch asks before a capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn, _ in calls.values():
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn, _ in calls.values():
            fn()
    torch.cuda.synchronize()
    scratch = torch.empty(1 << 20, device=DEV)
    for rep in range(3):
        say(f"graph replay {rep}")
        for _, outs in calls.values():
            for t in outs:
                t.fill_(float("nan"))
        scratch.normal_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, (_, outs) in calls.items():
            for r, t in zip(eager[name], outs):
                assert np.array_equal(r, _bits(t)), f"{name}: replay {rep} differs from the eager result"
