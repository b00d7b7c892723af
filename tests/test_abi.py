"""C ABI checks that need no GPU: libtea.so loads, exports every entry point
include/tea.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import tiled_exact_attention_amd as tea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tea.h")

NULL = None
FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x10002)   # misaligned


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return tea.load_library()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("row_softmax", "attn_fwd", "attn_decode_splitkv", "merge_partials"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    for name in tea.EXPORTS:
        assert name in _declared()


def test_status_strings_and_version(lib):
    assert lib.tea_abi_version() == 1
    for s in (tea.TEA_OK, tea.TEA_EINVAL, tea.TEA_EUNSUPPORTED, tea.TEA_EHIP):
        assert lib.tea_status_string(s)
    assert lib.tea_status_string(99) == b"unknown status"


def test_row_softmax_validation(lib):
    f = lib.row_softmax
    assert f(NULL, NULL, 4, 8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_EINVAL      # null x, y
    assert f(FAKE, FAKE, -1, 8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_EINVAL      # negative rows
    assert f(FAKE, FAKE, 4, -8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_EINVAL      # negative cols
    assert f(FAKE, FAKE, 4, 8, 7, 8, NULL, NULL, NULL) == tea.TEA_EINVAL                 # bad dtype
    assert f(FAKE, FAKE, 4, 8, tea.TEA_F32, -2, NULL, NULL, NULL) == tea.TEA_EINVAL      # bad block
    assert f(FAKE, FAKE, 4, 8, tea.TEA_F32, 3, NULL, NULL, NULL) == tea.TEA_EUNSUPPORTED  # non power of two
    assert f(ODD, FAKE, 4, 8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_EINVAL        # misaligned f32
    y_overlap = ctypes.c_void_p(0x10000 + 16)
    assert f(FAKE, y_overlap, 4, 8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_EINVAL  # partial overlap
    assert f(NULL, NULL, 0, 8, tea.TEA_F32, 8, NULL, NULL, NULL) == tea.TEA_OK           # no rows: no-op


def test_row_softmax_variant_validation(lib):
    f = lib.row_softmax_variant
    for bad in (-1, 3, 7):
        assert f(FAKE, FAKE, 4, 8, tea.TEA_F32, 8, bad, NULL, NULL, NULL) == tea.TEA_EINVAL  # unknown policy
    for rs in (tea.TEA_RESCALE_ALWAYS, tea.TEA_RESCALE_IF_RISE, tea.TEA_RESCALE_L0_ONE):
        assert f(NULL, NULL, 4, 8, tea.TEA_F32, 8, rs, NULL, NULL, NULL) == tea.TEA_EINVAL      # null x, y
        assert f(FAKE, FAKE, 4, 8, tea.TEA_F32, 3, rs, NULL, NULL, NULL) == tea.TEA_EUNSUPPORTED  # block 3
        assert f(ODD, FAKE, 4, 8, tea.TEA_F32, 8, rs, NULL, NULL, NULL) == tea.TEA_EINVAL       # misaligned
        assert f(NULL, NULL, 0, 8, tea.TEA_F32, 8, rs, NULL, NULL, NULL) == tea.TEA_OK          # no rows


def test_attn_fwd_validation(lib):
    f = lib.attn_fwd
    A = [FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)]
    ok = dict(B=1, H=1, Sq=8, Sk=8, D=64, scale=0.125, causal=0, od=tea.TEA_BF16)

    def call(ptrs=A, **kw):
        a = {**ok, **kw}
        return f(*ptrs, a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["scale"], a["causal"], a["od"], NULL, NULL)

    assert call(D=96) == tea.TEA_EUNSUPPORTED
    assert call(D=0) == tea.TEA_EINVAL
    assert call(causal=1, Sk=9) == tea.TEA_EUNSUPPORTED
    assert call(causal=2) == tea.TEA_EINVAL
    assert call(scale=0.0) == tea.TEA_EINVAL
    assert call(scale=float("nan")) == tea.TEA_EINVAL
    assert call(scale=-1.0) == tea.TEA_EINVAL
    assert call(od=5) == tea.TEA_EINVAL
    assert call(B=-1) == tea.TEA_EINVAL
    assert call(ptrs=[NULL, *A[1:]]) == tea.TEA_EINVAL
    assert call(ptrs=[ODD, *A[1:]]) == tea.TEA_EINVAL
    assert call(ptrs=[A[0], A[1], A[2], A[0]]) == tea.TEA_EINVAL  # o overlaps q
    assert call(B=0) == tea.TEA_OK


def test_attn_fwd_splitk_validation(lib):
    f = lib.attn_fwd_splitk
    A = [FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)]
    W = ctypes.c_void_p(0x1000000)
    need = lib.attn_fwd_splitk_workspace_bytes(1, 1, 8, 64, 4)
    assert need >= 8 * 4 * (64 + 2) * 4
    assert lib.attn_fwd_splitk_workspace_bytes(1, 1, 8, 64, 65) == 0

    def call(ptrs=A, B=1, H=1, Sq=8, Sk=8, D=64, scale=0.125, causal=0, S=4, od=tea.TEA_BF16, ws=W, wsb=need):
        return f(*ptrs, B, H, Sq, Sk, D, scale, causal, S, od, NULL, ws, wsb, NULL)

    assert call(S=0) == tea.TEA_EINVAL
    assert call(S=65) == tea.TEA_EINVAL
    assert call(wsb=need - 1) == tea.TEA_EINVAL
    assert call(ws=NULL) == tea.TEA_EINVAL
    assert call(ws=ctypes.c_void_p(0x40000 + 64)) == tea.TEA_EINVAL  # workspace overlaps o
    assert call(D=96) == tea.TEA_EUNSUPPORTED
    assert call(causal=1, Sk=9) == tea.TEA_EUNSUPPORTED
    assert call(scale=-1.0) == tea.TEA_EINVAL
    assert call(B=0) == tea.TEA_OK


def test_decode_validation(lib):
    f = lib.attn_decode_splitkv
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 64) >= 16 * 32 * 64 * (128 + 2) * 4
    assert lib.attn_decode_workspace_bytes(1, 1, 128, 0) == 0
    need = lib.attn_decode_workspace_bytes(2, 2, 128, 64)
    P = [FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
         ctypes.c_void_p(0x50000)]
    W = ctypes.c_void_p(0x100000)

    def call(B=2, H=2, Lmax=100, D=128, S=64, scale=0.1, od=tea.TEA_BF16, ws=W, wsb=need, ptrs=P):
        return f(*ptrs, B, H, Lmax, D, S, scale, od, ws, wsb, NULL)

    assert call(S=0) == tea.TEA_EINVAL
    assert call(S=1025) == tea.TEA_EINVAL
    assert call(D=80) == tea.TEA_EUNSUPPORTED
    assert call(wsb=need - 1) == tea.TEA_EINVAL
    assert call(ws=NULL) == tea.TEA_EINVAL
    assert call(Lmax=0) == tea.TEA_EINVAL
    assert call(scale=0.0) == tea.TEA_EINVAL
    assert call(ptrs=[P[0], P[1], P[2], NULL, P[4]]) == tea.TEA_EINVAL
    assert call(B=0) == tea.TEA_OK


def test_decode_fused_validation(lib):
    f = lib.attn_decode_fused
    P = [FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
         ctypes.c_void_p(0x50000)]

    def call(B=2, H=2, Lmax=100, D=128, S=64, scale=0.1, od=tea.TEA_BF16, ptrs=P):
        return f(*ptrs, B, H, Lmax, D, S, scale, od, NULL)

    assert call(S=0) == tea.TEA_EINVAL
    assert call(S=65) == tea.TEA_EINVAL  # 64 leaves at most
    assert call(D=96) == tea.TEA_EUNSUPPORTED
    assert call(Lmax=0) == tea.TEA_EINVAL
    assert call(scale=float("inf")) == tea.TEA_EINVAL
    assert call(od=7) == tea.TEA_EINVAL
    assert call(ptrs=[P[0], P[1], P[2], P[3], NULL]) == tea.TEA_EINVAL
    assert call(ptrs=[ODD, *P[1:]]) == tea.TEA_EINVAL
    assert call(H=0) == tea.TEA_OK


def test_merge_validation(lib):
    f = lib.merge_partials
    m, l, O, o = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000, 0x90000))
    assert f(m, l, O, 4, 0, 8, NULL, NULL, o, tea.TEA_F32, 1, NULL) == tea.TEA_EINVAL   # S = 0
    assert f(m, l, O, 4, 8, 0, NULL, NULL, o, tea.TEA_F32, 1, NULL) == tea.TEA_EINVAL   # D = 0
    assert f(m, l, O, -1, 8, 8, NULL, NULL, o, tea.TEA_F32, 1, NULL) == tea.TEA_EINVAL  # N < 0
    assert f(m, l, O, 4, 8, 8, NULL, NULL, o, tea.TEA_BF16, 0, NULL) == tea.TEA_EINVAL  # unnormalised bf16
    assert f(m, l, O, 4, 8, 8, NULL, NULL, o, tea.TEA_F32, 2, NULL) == tea.TEA_EINVAL
    assert f(NULL, l, O, 4, 8, 8, NULL, NULL, o, tea.TEA_F32, 1, NULL) == tea.TEA_EINVAL
    assert f(m, l, O, 4, 8, 8, NULL, NULL, O, tea.TEA_F32, 1, NULL) == tea.TEA_EINVAL   # output overlaps input
    assert f(m, l, O, 0, 8, 8, NULL, NULL, o, tea.TEA_F32, 1, NULL) == tea.TEA_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tea, "_lib", None)
    monkeypatch.setattr(tea, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        tea.load_library()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "tiled_exact_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src and "liboracle" not in src, fn
                assert "oracle.h" not in src, fn


def test_binding_rejects_mismatched_tensors():
    """The C ABI cannot see a tensor's size, so the binding checks shapes
    and dtypes against the sizes it passes; these CPU tensors fail there,
    before anything reaches the library or a device."""
    import torch

    bf = torch.bfloat16
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="out"):
        tea.row_softmax(x, out=torch.zeros(4, 7))
    with pytest.raises(ValueError, match="out"):
        tea.row_softmax_variant(x, 0, out=torch.zeros(4, 8, dtype=bf))
    q = torch.zeros(1, 2, 16, 64, dtype=bf)
    with pytest.raises(ValueError, match="k must be"):
        tea.attn_fwd(q, torch.zeros(1, 2, 16, 128, dtype=bf), torch.zeros(1, 2, 16, 128, dtype=bf))
    with pytest.raises(ValueError, match="v must be"):
        tea.attn_fwd(q, torch.zeros(1, 2, 32, 64, dtype=bf), torch.zeros(1, 2, 16, 64, dtype=bf))
    with pytest.raises(ValueError, match="out"):
        tea.attn_fwd(q, q, q, out=torch.zeros(1, 2, 15, 64, dtype=bf))
    with pytest.raises(ValueError, match="k must be"):
        tea.attn_fwd_splitk(q, torch.zeros(2, 2, 16, 64, dtype=bf), q, 2)
    qd = torch.zeros(3, 2, 1, 64, dtype=bf)
    kd = torch.zeros(3, 2, 100, 64, dtype=bf)
    kv = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match="kv_len"):
        tea.attn_decode_splitkv(qd, kd, kd, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError, match="v must be"):
        tea.attn_decode_fused(qd, kd, torch.zeros(3, 2, 99, 64, dtype=bf), kv)
    with pytest.raises(ValueError, match="out"):
        tea.attn_decode_fused(qd, kd, kd, kv, out=torch.zeros(3, 2, 32, dtype=bf))
    m = torch.zeros(5, 4)
    O = torch.zeros(5, 4, 8)
    with pytest.raises(ValueError, match="l must be"):
        tea.merge_partials(m, torch.zeros(5, 3), O)
    with pytest.raises(ValueError, match="O must be"):
        tea.merge_partials(m, m, O.double())
    with pytest.raises(ValueError, match="out"):
        tea.merge_partials(m, m, O, out=torch.zeros(5, 4))


def test_output_overlap_is_rejected(lib):
    """Every written region (outputs, statistics, workspaces) must overlap no
    input and no other output; each such call is rejected before any HIP
    call (the fake addresses are never dereferenced)."""
    at = lambda a: ctypes.c_void_p(a)  # noqa: E731
    # row_softmax: x, y [4, 8] f32 (128 B each); m_out, l_out [4] f32
    x, y = at(0x10000), at(0x20000)
    for rs in (lib.row_softmax, lambda *a: lib.row_softmax_variant(*a[:6], tea.TEA_RESCALE_ALWAYS, *a[6:])):
        assert rs(x, y, 4, 8, tea.TEA_F32, 8, at(0x10000 + 64), NULL, NULL) == tea.TEA_EINVAL  # m_out in x
        assert rs(x, y, 4, 8, tea.TEA_F32, 8, NULL, at(0x20000 + 124), NULL) == tea.TEA_EINVAL  # l_out in y
        assert rs(x, y, 4, 8, tea.TEA_F32, 8, at(0x30000), at(0x30000 + 8), NULL) == tea.TEA_EINVAL  # m/l overlap
        assert rs(x, x, 4, 8, tea.TEA_F32, 8, at(0x10000), NULL, NULL) == tea.TEA_EINVAL  # in place, m_out in x
    # attn_fwd: q, k, v [1, 1, 8, 64] bf16 (1 KiB each); lse [8] f32
    A = [at(0x10000), at(0x20000), at(0x30000), at(0x40000)]
    for lse in (at(0x10000 + 16), at(0x20000), at(0x30000 + 1008)):  # lse inside q, k, v
        assert lib.attn_fwd(*A, 1, 1, 8, 8, 64, 0.125, 0, tea.TEA_BF16, lse, NULL) == tea.TEA_EINVAL
        assert lib.attn_fwd_splitk(*A, 1, 1, 8, 8, 64, 0.125, 0, 2, tea.TEA_BF16, lse, at(0x1000000),
                                   lib.attn_fwd_splitk_workspace_bytes(1, 1, 8, 64, 2), NULL) == tea.TEA_EINVAL
    # decode: q [2, 2, 1, 128] bf16 (1 KiB), k, v [2, 2, 100, 128] bf16 (100 KiB
    # each), kv_len [2] int32 (8 B), o [2, 2, 128] bf16 (1 KiB)
    q, k, v, kv, o = at(0x10000), at(0x100000), at(0x200000), at(0x300000), at(0x400000)
    need = lib.attn_decode_workspace_bytes(2, 2, 128, 64)
    W = at(0x1000000)

    def dec(q=q, k=k, v=v, kv=kv, o=o, ws=W):
        return lib.attn_decode_splitkv(q, k, v, kv, o, 2, 2, 100, 128, 64, 0.1, tea.TEA_BF16, ws, need, NULL)

    def fused(q=q, k=k, v=v, kv=kv, o=o):
        return lib.attn_decode_fused(q, k, v, kv, o, 2, 2, 100, 128, 64, 0.1, tea.TEA_BF16, NULL)

    for f in (dec, fused):
        assert f(o=at(0x10000 + 512)) == tea.TEA_EINVAL     # o inside q
        assert f(o=at(0x100000 + 4096)) == tea.TEA_EINVAL   # o inside k
        assert f(o=at(0x200000 + 100 * 1024 - 16)) == tea.TEA_EINVAL  # o over the tail of v
        assert f(o=at(0x300000 - 16)) == tea.TEA_EINVAL     # o runs into kv_len
    assert dec(ws=at(0x100000)) == tea.TEA_EINVAL           # workspace over k
    assert dec(ws=at(0x200000 + 1024)) == tea.TEA_EINVAL    # workspace inside v
    assert dec(ws=at(0x300000 - 256)) == tea.TEA_EINVAL     # workspace over kv_len
    assert dec(ws=at(0x10000 - 256)) == tea.TEA_EINVAL      # workspace over q
    # merge_partials: m, l [4, 8] f32 (128 B), O [4, 8, 8] f32 (1 KiB), O_out [4, 8] f32
    m, l, O, oo = at(0x10000), at(0x20000), at(0x30000), at(0x40000)

    def merge(m_out=NULL, l_out=NULL):
        return lib.merge_partials(m, l, O, 4, 8, 8, m_out, l_out, oo, tea.TEA_F32, 1, NULL)

    assert merge(m_out=at(0x10000 + 64)) == tea.TEA_EINVAL  # m_out inside m
    assert merge(l_out=at(0x20000)) == tea.TEA_EINVAL       # l_out over l
    assert merge(m_out=at(0x30000 + 512)) == tea.TEA_EINVAL  # m_out inside O
    assert merge(l_out=at(0x40000 + 112)) == tea.TEA_EINVAL  # l_out inside O_out
    assert merge(at(0x50000), at(0x50000 + 4)) == tea.TEA_EINVAL  # m_out and l_out overlap


def test_decode_noalloc_validation(lib):
    """The allocation-free decode checks its arguments like
    attn_decode_splitkv, and refuses (TEA_ENOSPACE, before any HIP call) a
    request whose partials exceed the scratch it holds."""
    f = lib.attn_decode_splitkv_noalloc
    P = [FAKE, ctypes.c_void_p(0x20000), ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000),
         ctypes.c_void_p(0x50000)]

    def call(B=2, H=2, Lmax=100, D=128, S=64, scale=0.1, od=tea.TEA_BF16, ptrs=P):
        return f(*ptrs, B, H, Lmax, D, S, scale, od, NULL)

    assert lib.tea_status_string(tea.TEA_ENOSPACE)
    cap = tea.DECODE_NOALLOC_MAX_BYTES
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 64) <= cap  # the decode workload fits
    assert lib.attn_decode_workspace_bytes(64, 32, 128, 64) > cap
    assert call(B=64, H=32) == tea.TEA_ENOSPACE
    assert call(B=16, H=32, S=1024) == tea.TEA_ENOSPACE
    assert call(S=0) == tea.TEA_EINVAL
    assert call(S=1025) == tea.TEA_EINVAL
    assert call(D=80) == tea.TEA_EUNSUPPORTED
    assert call(Lmax=0) == tea.TEA_EINVAL
    assert call(scale=float("nan")) == tea.TEA_EINVAL
    assert call(od=3) == tea.TEA_EINVAL
    assert call(ptrs=[P[0], P[1], P[2], NULL, P[4]]) == tea.TEA_EINVAL
    assert call(ptrs=[ODD, *P[1:]]) == tea.TEA_EINVAL
    assert call(ptrs=[*P[:4], ctypes.c_void_p(0x30000 + 64)]) == tea.TEA_EINVAL  # o overlaps v
    assert call(B=0) == tea.TEA_OK
