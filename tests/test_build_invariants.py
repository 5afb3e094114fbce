"""Invariants of the generated gfx950 code, checked from the compiler's assembly on the
CPU (hipcc cross-compiles; no GPU needed):

* M0 is written only by the direct-load sequences (s_mov_b32 m0 ... global_load_lds):
  the inline assembly that issues them clobbers M0, which is safe only while no
  compiler-generated code in these kernels relies on M0;
* no packed-fp32 VALU instructions (v_pk_fma/mul/add_f32) are generated;
* the hot kernels keep everything in registers (no scratch spills);
* the MFMAs written out in inline assembly (the dK/dV kernel), which the compiler's
  hazard recognizer does not see, keep the ISA's distances: no VALU, memory or other
  MFMA instruction reads their result registers (other than the same accumulator chain)
  before NumPasses + 4 wait states (the CDNA3/CDNA4 table asks NumPasses + 3 for an XDL
  write read by VALU or memory instructions; one more for margin), and no non-MFMA
  instruction overwrites a register they read as SrcC before NumPasses + 3.  Wait
  states are counted along every control-flow path: s_nop n counts n + 1, an
  intervening XDL instruction counts its NumPasses (one wave's XDL instructions run one
  after another, each occupying the unit for all its passes), anything else 1.
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_exact_tiled_amd import build as B

HOT = ("attn_fwd_direct_kernel", "attn_fwd_fp8_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel",
       "lse_merge_kernel", "permute_kernel", "permute_rows_kernel", "quant_amax_kernel",
       "quant_convert_kernel", "bwd_delta_kernel")


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


# ---------------------------------------------------------------- MFMA hazard distances

_REG = re.compile(r"^([va])(?:\[(\d+):(\d+)\]|(\d+))$")
_PASSES = {"v_mfma_f32_32x32x16_bf16": 8}  # 32 cycles on gfx950 = 8 passes of 4 cycles
_STORES = ("global_store", "buffer_store", "flat_store", "scratch_store", "ds_write", "ds_store")


def _regs(tok):
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = _REG.match(tok)
    if not m:
        return set()
    if m.group(4) is not None:
        return {(m.group(1), int(m.group(4)))}
    return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}


def _program(fn_text):
    """Instructions of one function (op, operands, from inline asm?) and label positions."""
    ins, labels, in_asm = [], {}, False
    for raw in fn_text.splitlines():
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        t = t.split(";")[0].strip()
        if not t or (t.startswith(".") and not t.endswith(":")):
            continue
        if t.endswith(":"):
            labels[t[:-1]] = len(ins)
            continue
        parts = t.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        ins.append({"op": parts[0], "ops": ops, "asm": in_asm, "text": t})
    return ins, labels


def _is_xdl(op):
    return op.startswith("v_mfma")


def _cost(x):
    if x["op"] == "s_nop":
        return int(x["ops"][0], 0) + 1 if x["ops"] else 1
    if _is_xdl(x["op"]):
        return _PASSES.get(x["op"], 4)  # unlisted XDL ops: the smallest shape's passes
    return 1


def _reads_writes(x):
    rs = [_regs(o) for o in x["ops"]]
    if not rs:
        return set(), set()
    if x["op"].startswith(_STORES):
        return set().union(*rs), set()
    return (set().union(*rs[1:]) if len(rs) > 1 else set()), rs[0]


def mfma_hazards(fn_text):
    """(kind, wait states found, MFMA, offending instruction) for every inline-asm MFMA
    whose result is read, or whose SrcC registers are overwritten, too early on some
    control-flow path."""
    ins, labels = _program(fn_text)

    def succ(j):
        op = ins[j]["op"]
        if op == "s_endpgm":
            return []
        if op == "s_branch":
            return [labels[ins[j]["ops"][0]]]
        if op.startswith("s_cbranch"):
            return [labels[ins[j]["ops"][0]], j + 1]
        return [j + 1] if j + 1 < len(ins) else []

    def walk(i, need, hit):
        best, stack, found = {}, [(s, 0) for s in succ(i)], []
        while stack:
            j, d = stack.pop()
            if d >= need or best.get(j, 1 << 30) <= d:
                continue
            best[j] = d
            kind = hit(ins[j])
            if kind == "bad":
                found.append((d, ins[j]["text"]))
                continue
            if kind == "stop":
                continue
            stack.extend((s, d + _cost(ins[j])) for s in succ(j))
        return found

    bad = []
    for i, x in enumerate(ins):
        if not (x["asm"] and _is_xdl(x["op"])):
            continue
        passes = _PASSES.get(x["op"])
        assert passes, f"no pass count known for {x['op']}"
        dst = _regs(x["ops"][0])
        srcc = _regs(x["ops"][3]) - dst if len(x["ops"]) > 3 else set()

        def raw_hit(y):
            r, w = _reads_writes(y)
            if r & dst:
                chained = (_is_xdl(y["op"]) and len(y["ops"]) > 3 and _regs(y["ops"][0]) == dst
                           and _regs(y["ops"][3]) == dst
                           and not (_regs(y["ops"][1]) | _regs(y["ops"][2])) & dst)
                return "stop" if chained else "bad"
            return "stop" if dst <= w else "go"

        def war_hit(y):
            _, w = _reads_writes(y)
            return "bad" if (w & srcc and not _is_xdl(y["op"])) else "go"

        bad += [("RAW", d, x["text"], t) for d, t in walk(i, passes + 4, raw_hit)]
        if srcc:
            bad += [("WAR", d, x["text"], t) for d, t in walk(i, passes + 3, war_hit)]
    return bad


def _functions(text):
    return {m.group(1): m.group(2)
            for m in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.S | re.M)}


_MF = "v_mfma_f32_32x32x16_bf16"


@pytest.mark.parametrize("body,expect", [
    # a VALU read right after the MFMA
    (f";;#ASMSTART\n{_MF} v[0:15], v[16:19], a[0:3], 0\n;;#ASMEND\nv_add_f32 v20, v1, v2\n"
     "s_endpgm\n", ["RAW"]),
    # one independent MFMA in between (8) is short of 12
    (f";;#ASMSTART\n{_MF} v[0:15], v[16:19], a[0:3], 0\n;;#ASMEND\n"
     f"{_MF} v[32:47], v[16:19], a[0:3], 0\nv_add_f32 v20, v1, v2\ns_endpgm\n", ["RAW"]),
    # two MFMAs in between (16): fine; so is s_nop 7 + s_nop 3 (12)
    (f";;#ASMSTART\n{_MF} v[0:15], v[16:19], a[0:3], 0\n;;#ASMEND\n"
     f"{_MF} v[32:47], v[16:19], a[0:3], 0\n{_MF} v[48:63], v[16:19], a[0:3], 0\n"
     "v_add_f32 v20, v1, v2\ns_endpgm\n", []),
    (f";;#ASMSTART\n{_MF} a[0:15], v[16:19], v[20:23], a[0:15]\n;;#ASMEND\n"
     "s_nop 7\ns_nop 3\nv_accvgpr_read_b32 v0, a3\ns_endpgm\n", []),
    # the same accumulator chain right after: allowed; a store of the result: not
    (f";;#ASMSTART\n{_MF} a[0:15], v[16:19], v[20:23], a[0:15]\n;;#ASMEND\n"
     f";;#ASMSTART\n{_MF} a[0:15], v[24:27], v[20:23], a[0:15]\n;;#ASMEND\n"
     "s_nop 7\nglobal_store_dwordx4 v1, a[0:3], s[0:1]\ns_endpgm\n", ["RAW"]),
    # a branch that skips the padding reaches the read too early
    (f";;#ASMSTART\n{_MF} v[0:15], v[16:19], a[0:3], 0\n;;#ASMEND\ns_cbranch_scc1 .LBB0_2\n"
     "s_nop 7\ns_nop 7\n.LBB0_2:\nv_mov_b32 v30, v5\ns_endpgm\n", ["RAW"]),
    # SrcC registers overwritten by an LDS read two instructions later
    (f";;#ASMSTART\n{_MF} v[32:47], v[16:19], a[0:3], v[0:15]\n;;#ASMEND\n"
     "ds_read_b128 v[0:3], v40\ns_endpgm\n", ["RAW", "WAR"]),
])
def test_hazard_checker_flags_short_distances(body, expect):
    """The checker itself: it flags reads (and SrcC overwrites) closer than the rule and
    accepts the distances the rule allows, on every control-flow path."""
    kinds = sorted({k for k, *_ in mfma_hazards(body)})
    assert kinds == sorted(expect), mfma_hazards(body)


def test_inline_mfma_distances(asm):
    """Every written-out MFMA of the dK/dV kernels (every D = 128 instantiation; D = 64
    has none) keeps the ISA's distances to its readers and to writers of its SrcC
    registers."""
    fns = {n: b for n, b in _functions(asm["attn_bwd.hip"]).items() if "bwd_dkdv_kernel" in n}
    assert len(fns) >= 8, list(fns)
    for name, body in fns.items():
        n_asm = sum(1 for x in _program(body)[0] if x["asm"] and _is_xdl(x["op"]))
        if "kernelILi64E" in name:  # D = 64 uses the compiler's MFMAs and wait states
            assert n_asm == 0, (name, n_asm)
            continue
        assert n_asm >= 32, (name, n_asm)  # the check is not vacuous
        bad = mfma_hazards(body)
        assert not bad, (name, bad[:5])
