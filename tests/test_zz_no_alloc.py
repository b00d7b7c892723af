"""attn_decode_splitkv_noalloc, the decode for callers that cannot allocate,
against attn_decode_splitkv (the same kernels with a caller workspace) through
the C ABI: bit-identical outputs on two calls in a row, the second with a
smaller input (so the scratch still holds the first call's partials), and the
first also against the fp64 oracle within the attention bar."""
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


def _pair(B, H, Lmax, D, S, seed, out_dtype, kv_len=None):
    q, K, V, kv = inputs.decode_inputs(B, H, Lmax, D, seed=seed, kv_len=kv_len)
    qd, Kd, Vd, kvd = q.to(DEV), K.to(DEV), V.to(DEV), kv.to(DEV)
    scale = 1.0 / math.sqrt(D)
    ref = tea.attn_decode_splitkv(qd, Kd, Vd, kvd, num_splits=S, scale=scale, out_dtype=out_dtype)
    out = torch.full((B, H, D), float("nan"), dtype=out_dtype, device=DEV)
    got = tea.attn_decode_splitkv_noalloc(qd, Kd, Vd, kvd, out, num_splits=S, scale=scale)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    return q, K, V, kv, scale, ref, got


def test_noalloc_matches_workspace_decode_twice():
    # first call: B16 H32 D128, 64 splits (17 MB of partials, most of the
    # scratch), KV lengths uniform in [1, 4096]
    say("decode noalloc call 1: B16 H32 Lmax4096 D128 splits64")
    q, K, V, kv, scale, ref, got = _pair(16, 32, 4096, 128, 64, seed=71, out_dtype=torch.bfloat16)
    assert torch.equal(got, ref), "noalloc decode differs from the workspace decode"
    O = np.zeros((16 * 32, 128))
    for b in range(16):
        L = int(kv[b])
        o, _ = oracle.attention(q[b:b + 1].float().numpy(), K[b:b + 1, :, :L].float().numpy(),
                                V[b:b + 1, :, :L].float().numpy(), scale, False)
        O[b * 32:(b + 1) * 32] = o.reshape(32, 128)
    check_attention(to_np(got).reshape(-1, 128), O, "noalloc call 1")
    # second call, smaller: B3 H4 D64, 16 splits, lengths 0, 17 and 700 (an
    # empty sequence, chunks empty below 16 keys), fp32 output
    say("decode noalloc call 2: B3 H4 Lmax700 D64 splits16 fp32 out")
    _, _, _, _, _, ref2, got2 = _pair(3, 4, 700, 64, 16, seed=72, out_dtype=torch.float32,
                                      kv_len=np.array([0, 17, 700]))
    assert torch.equal(got2, ref2), "second call differs from the workspace decode"
    assert torch.all(got2[0] == 0)


def test_noalloc_rejects_requests_beyond_its_scratch():
    say("decode noalloc beyond the scratch")
    B, H, D = 64, 32, 128
    assert tea.attn_decode_workspace_bytes(B, H, D, 64) > tea.DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros(B, H, 1, D, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(B, H, 8, D, dtype=torch.bfloat16, device=DEV)
    kv = torch.full((B,), 8, dtype=torch.int32, device=DEV)
    out = torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tea.TeaError) as e:
        tea.attn_decode_splitkv_noalloc(q, k, k, kv, out, num_splits=64)
    assert e.value.status == tea.TEA_ENOSPACE
