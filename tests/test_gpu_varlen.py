"""GPU parity of ra_attn_fwd_varlen (packed documents) against the CPU oracle.

Small cases compare every element against ``oracle.varlen_attention``; the packed 32K
workload compares every row of two documents (the shortest and the longest) for sampled
heads, which the oracle computes as full attention of that document's slice.
"""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import check_grad, check_lse, check_o, require_gpu, say, to_dev, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


CASES = [
    # D, causal, B, Hq, Hkv, T, cu_seqlens
    (128, True, 1, 4, 2, 700, [0, 100, 100, 357, 358, 600, 700]),   # empty and 1-token docs
    (128, False, 1, 4, 2, 700, [0, 100, 100, 357, 358, 600, 700]),
    (128, True, 2, 2, 2, 600, [0, 600]),                           # one document
    (128, True, 1, 7, 1, 1000, [0, 129, 255, 256, 513, 900]),      # tokens 900.. in none
    (64, True, 1, 4, 4, 520, [0, 37, 64, 65, 200, 300, 301, 520]),
    (64, False, 2, 2, 1, 300, [0, 1, 2, 3, 150, 300]),
    (128, True, 1, 2, 2, 2048, list(range(0, 2049, 64))),          # 32 docs of 64
    (128, False, 1, 2, 2, 1300, [0, 700, 1300]),                   # docs across blocks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"D{c[0]}-c{int(c[1])}-B{c[2]}-H{c[3]}/{c[4]}-T{c[5]}-n{len(c[6]) - 1}")
def test_varlen_parity(case):
    D, causal, B, Hq, Hkv, T, cu = case
    say(f"varlen D={D} causal={causal} B={B} Hq={Hq} Hkv={Hkv} T={T} cu={cu}")
    q, k, v = si.draw_qkv(2000 + T + len(cu), (B, Hq, T, D), (B, Hkv, T, D), "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    out = torch.full(qd.shape, float("nan"), dtype=qd.dtype, device="cuda")
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ra.attn_fwd_varlen(qd, kd, vd, cud, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    q64, k64, v64 = (si.as_f64(x, "bf16") for x in (q, k, v))
    o_ref, l_ref = oracle.varlen_attention(q64, k64, v64, cu, causal=causal)
    check_o(to_np64(out), o_ref, "bf16")
    check_lse(to_np64(lse), l_ref, "bf16")


def test_varlen_single_document_matches_attn_fwd():
    """One document spanning every token is plain attention: both entry points agree."""
    say("varlen single document vs attn_fwd")
    q, k, v = si.draw_qkv(77, (1, 4, 900, 128), (1, 2, 900, 128), "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    cud = torch.tensor([0, 900], dtype=torch.int32, device="cuda")
    o1, l1 = ra.attn_fwd_varlen(qd, kd, vd, cud, causal=True)
    o2, l2 = ra.attn_fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_packed_32k_workload_sampled():
    w = si.WORKLOADS["qwen7b_packed_32k"]
    cu = si.draw_doc_offsets(w.seed, w.q_shape[2])
    say(f"varlen workload {w.name} docs={len(cu) - 1}")
    q, k, v = si.draw_qkv(w.seed, w.q_shape, w.kv_shape, w.dtype)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    out, lse = ra.attn_fwd_varlen(qd, kd, vd, cud, causal=w.causal)
    torch.cuda.synchronize()
    lens = np.diff(cu)
    group = w.q_shape[1] // w.kv_shape[1]
    for d in (int(np.argmin(lens)), int(np.argmax(lens))):
        a, b = cu[d], cu[d + 1]
        for h in (0, w.q_shape[1] - 1):
            g = h // group
            q64 = si.as_f64(q[:, h:h + 1, a:b], "bf16")
            k64 = si.as_f64(k[:, g:g + 1, a:b], "bf16")
            v64 = si.as_f64(v[:, g:g + 1, a:b], "bf16")
            o_ref, l_ref = oracle.full_attention(q64, k64, v64, causal=w.causal)
            check_o(to_np64(out[:, h:h + 1, a:b]), o_ref, "bf16", f"doc {d} head {h} o")
            check_lse(to_np64(lse[:, h:h + 1, a:b]), l_ref, "bf16", f"doc {d} head {h} lse")


# Gradients: the tolerance derived for ra_attn_bwd (check_grad), applied to every element.
BWD_CASES = [
    # D, causal, B, Hq, Hkv, T, cu_seqlens
    (128, True, 1, 4, 2, 700, [0, 100, 100, 357, 358, 600, 700]),
    (128, False, 1, 4, 2, 700, [0, 100, 100, 357, 358, 600, 700]),
    (128, True, 1, 2, 1, 1000, [0, 129, 255, 256, 513, 900]),       # tokens 900.. in none
    (64, True, 2, 2, 2, 520, [0, 37, 64, 65, 200, 300, 301, 520]),
    (64, False, 1, 4, 2, 300, [0, 1, 2, 3, 150, 300]),
    (128, True, 1, 2, 2, 1024, list(range(0, 1025, 64))),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"D{c[0]}-c{int(c[1])}-B{c[2]}-H{c[3]}/{c[4]}-T{c[5]}-n{len(c[6]) - 1}")
def test_varlen_bwd_parity(case):
    D, causal, B, Hq, Hkv, T, cu = case
    say(f"varlen bwd D={D} causal={causal} B={B} Hq={Hq} Hkv={Hkv} T={T} cu={cu}")
    q, k, v, do = si.draw_qkv(3000 + T + len(cu), (B, Hq, T, D), (B, Hkv, T, D), "bf16",
                              with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    cud = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o, lse = ra.attn_fwd_varlen(qd, kd, vd, cud, causal=causal)
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(kd, float("nan"))
    dv = torch.full_like(vd, float("nan"))
    ra.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cud, causal=causal, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.varlen_attention_bwd(*(si.as_f64(x, "bf16") for x in (q, k, v, do)), cu,
                                      causal=causal)
    for got, r, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(to_np64(got), r, name)


def test_varlen_bwd_single_document_matches_attn_bwd():
    say("varlen bwd single document vs attn_bwd")
    q, k, v, do = si.draw_qkv(78, (1, 4, 640, 128), (1, 2, 640, 128), "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    cud = torch.tensor([0, 640], dtype=torch.int32, device="cuda")
    o, lse = ra.attn_fwd(qd, kd, vd, causal=True)
    g1 = ra.attn_bwd_varlen(qd, kd, vd, o, dod, lse, cud, causal=True)
    g2 = ra.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
