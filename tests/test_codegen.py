"""Properties of the generated gfx950 code that the kernels rely on (CPU only:
hipcc cross-compiles the sources here and the AMD assembly is inspected).

* No packed fp32 arithmetic (v_pk_fma_f32 / v_pk_mul_f32 / v_pk_add_f32) in
  any kernel: every source is built with the packed-fp32 feature disabled.
* The bf16 MFMA kernels (forward, and the backward's dQ and dK/dV) keep
  everything in registers (no scratch) at two waves per SIMD: a scratch
  access inside a main loop would make the compiler wait for all outstanding
  vector-memory operations, including the untracked LDS-DMA prefetch of the
  next tile.
* m0 is written only by the LDS-DMA helpers (the compiler must not rely on m0
  anywhere in those kernels, since the helpers' inline assembly clobbers it).
"""
import glob
import os
import re
import shutil
import subprocess

import pytest

from ring_attention_step_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _device_asm(src, tmp_path, extra=()):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.COMMON, *extra, "-S", "--cuda-device-only", src, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.mark.parametrize("src", sorted(glob.glob(os.path.join(B.CSRC, "*.hip"))), ids=os.path.basename)
def test_no_packed_fp32_instructions(src, tmp_path):
    asm = _device_asm(src, tmp_path)
    bad = re.findall(r"\bv_pk_(?:fma|mul|add)_f32\b", asm)
    assert not bad, f"{os.path.basename(src)} contains packed fp32 instructions: {sorted(set(bad))}"


def _kernels(asm, pattern=r"block_mfma_kernel"):
    """Split device assembly into {symbol: body} for each kernel matching pattern."""
    out = {}
    for m in re.finditer(r"^(_Z\S*(?:" + pattern + r")\S*):", asm, flags=re.M):
        start = m.end()
        end = asm.find(".Lfunc_end", start)
        out[m.group(1)] = asm[start:end]
    return out


@pytest.mark.parametrize("src,pattern,count", [("block_attn_mfma.hip", "block_mfma_kernel", 4),
                                               ("block_attn_bwd_mfma.hip", "dq_kernel|dkdv_kernel", 4)])
def test_mfma_kernel_registers_scratch_and_m0(tmp_path, src, pattern, count):
    src = os.path.join(B.CSRC, src)
    asm = _device_asm(src, tmp_path)
    kernels = _kernels(asm, pattern)
    assert len(kernels) == count, f"expected {count} instantiations (head_dim 64 and 128; forward: whole-tile and ragged blocks)"
    for name, body in kernels.items():
        for line in body.splitlines():
            code = line.split(";")[0]
            if re.search(r"\bm0\b", code):
                assert re.match(r"\s*s_mov_b32 m0, (?:s\d+|vcc_lo|vcc_hi)\s*$", code), f"{name}: unexpected m0 use: {code.strip()}"
    # resource metadata: scratch (private segment) size and VGPR count per kernel
    for name in kernels:
        at = asm.find(f".name:           {name}")
        assert at >= 0, f"no metadata for {name}"
        nxt = [i for i in (asm.find("- .args:", at), asm.find("amdhsa.target", at)) if i > 0]
        meta = asm[at:min(nxt) if nxt else len(asm)]
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", meta)
        vgpr = re.search(r"\.vgpr_count:\s+(\d+)", meta)
        assert priv and int(priv.group(1)) == 0, f"{name} uses scratch"
        assert vgpr and int(vgpr.group(1)) <= 256, f"{name} needs more than 256 VGPRs (1 wave/SIMD)"
