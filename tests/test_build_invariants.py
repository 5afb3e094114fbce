"""Invariants of the generated gfx950 code, checked from the compiler's assembly on the
CPU (hipcc cross-compiles; no GPU needed):

* M0 is written only by the direct-load sequences (s_mov_b32 m0 ... global_load_lds):
  the inline assembly that issues them clobbers M0, which is safe only while no
  compiler-generated code in these kernels relies on M0;
* no packed-fp32 VALU instructions (v_pk_fma/mul/add_f32) are generated;
* the hot kernels keep everything in registers (no scratch spills).
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_exact_tiled_amd import build as B

HOT = ("attn_fwd_direct_kernel", "attn_fwd_fp8_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel",
       "lse_merge_kernel", "permute_kernel", "permute_rows_kernel", "quant_amax_kernel",
       "quant_convert_kernel", "quant_convert_t_kernel", "bwd_delta_kernel")


def _asm(src):
    out = f"/tmp/_inv_{os.getpid()}_{src}.s"
    cmd = [B.hipcc(), *B.flags_for(src), "-I", os.path.join(B.ROOT, "include"), "-S", "--cuda-device-only",
           os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    text = open(out).read()
    os.remove(out)
    return text


@pytest.fixture(scope="module")
def asm():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    return {src: _asm(src) for src in B.SOURCES if src != "api.hip"}


def test_m0_only_in_dma_sequences(asm):
    for src, text in asm.items():
        lines = [l.strip() for l in text.splitlines()]
        for i, l in enumerate(lines):
            if re.search(r"\bm0\b", l) and not l.startswith(";"):
                # the DMA sequence's scalar operand: any SGPR, vcc_lo/vcc_hi included
                assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$", l), (src, l)
                nxt = [x for x in lines[i + 1:i + 4] if x and not x.startswith(";")]
                assert nxt[0].startswith("s_nop") and nxt[1].startswith("global_load_lds_dwordx4"), \
                    (src, l, nxt)


def test_no_packed_fp32(asm):
    for src, text in asm.items():
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", text), src


def _kernel_metadata(text):
    """(name, private segment bytes, VGPR spills, SGPR spills) of every kernel, from the
    code object metadata the compiler writes after the code."""
    meta = text[text.find("amdhsa.kernels:"):]
    out = []
    for block in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        vsp = re.search(r"\.vgpr_spill_count:\s+(\d+)", block)
        ssp = re.search(r"\.sgpr_spill_count:\s+(\d+)", block)
        if name and priv and vsp:
            out.append((name.group(1), int(priv.group(1)), int(vsp.group(1)),
                        int(ssp.group(1)) if ssp else 0))
    return out


def test_hot_kernels_do_not_spill(asm):
    seen = set()
    for src, text in asm.items():
        for name, priv, vspill, _ in _kernel_metadata(text):
            if not any(k in name for k in HOT):
                continue
            seen.update(k for k in HOT if k in name)
            assert vspill == 0 and priv == 0, (src, name, vspill, priv)
            assert "scratch_store" not in text, src
    assert seen == set(HOT), set(HOT) - seen
