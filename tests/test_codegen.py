"""Checks on the gfx950 assembly hipcc produces for the kernels (CPU only).

- Every kernel keeps its working set in registers: no VGPR spills and no
  private (scratch) segment.  A spill in the attention loop costs more than
  any of the scheduling choices it is tuned by, and one in the streaming
  kernels adds memory traffic the byte counts do not allow for.
- The attention kernels take the row sum of P on the matrix core
  (v_mfma_f32_16x16x32_bf16 against a 0/1 selector) for both head
  dimensions: no v_dot2c (which waits for a busy matrix core), and per KV
  tile one selector MFMA per 16-key chunk of P.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_exact_attention_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
SOURCES = ["attn_fwd.hip", "softmax.hip", "decode.hip", "merge.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _asm(src_path, out_path):
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-fno-fast-math", "-ffp-contract=fast", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, src_path, "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out_path).read()


def _kernels(asm: str) -> dict:
    """kernel symbol -> (its code, its metadata fields)"""
    code = {}
    for m in re.finditer(r"^(_Z\S+):[^\n]*$(.*?)^\.Lfunc_end", asm, re.M | re.S):
        code[m.group(1)] = m.group(2)
    meta = {}
    for blk in re.split(r"\n\s*-\s+\.", asm.split("amdhsa.kernels:")[-1])[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if name:
            meta[name.group(1)] = {k: int(v) for k, v in re.findall(r"\.(\w+):\s+(\d+)\s*$", blk, re.M)}
    return {k: (code.get(k, ""), meta[k]) for k in meta}


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    return {src: _kernels(_asm(os.path.join(CSRC, src), str(d / (src + ".s")))) for src in SOURCES}


def test_every_source_has_kernels(kernels):
    for src, ks in kernels.items():
        assert ks, f"no kernels found in the assembly of {src}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_spills(kernels, src):
    for name, (_, meta) in kernels[src].items():
        assert meta.get("vgpr_spill_count", 0) == 0, f"{name}: {meta['vgpr_spill_count']} VGPRs spilled"
        assert meta.get("private_segment_fixed_size", 0) == 0, f"{name}: uses a scratch segment"


def test_attention_row_sum_on_matrix_core(kernels):
    ks = {n: c for n, (c, _) in kernels["attn_fwd.hip"].items() if "attn_fwd_kernel" in n}
    assert len(ks) == 4, sorted(ks)  # D 64 and 128, bf16 and fp32 output
    for name, code in ks.items():
        assert "v_dot2" not in code, f"{name}: vector dot2 in the attention kernel"
        sel = len(re.findall(r"v_mfma_f32_16x16x32_bf16", code))
        # four 16-key chunks per 64-key tile, the loop unrolled two tiles deep;
        # at D = 64 the lag check and its second pass each take the sum
        assert sel in (8, 16), f"{name}: {sel} selector MFMAs"
