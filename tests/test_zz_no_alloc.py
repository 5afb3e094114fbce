"""ra_attn_bwd_noalloc (the backward whose workspace is the library's fixed per-GPU scratch)
against ra_attn_bwd through the C ABI: two calls in a row, the second with a smaller
input.  dq is bitwise ra_attn_bwd's (same kernels), and so are dk, dv with one query
head per key/value head; with grouped heads ra_attn_bwd sums per-head partials kept in
its workspace, which the fixed scratch does not hold, so noalloc sums the group inside
each workgroup instead: there dk, dv agree to the bf16 gradient bound, and both entry
points are within the oracle's gradient bound.  A problem needing more than the scratch
holds is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import check_grad, require_gpu, say, to_dev, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _case(B, Hq, Hkv, S, D, causal, seed):
    q, k, v, do = si.draw_qkv(seed, (B, Hq, S, D), (B, Hkv, S, D), "bf16", with_dout=True)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = ra.attn_fwd(qd, kd, vd, causal=causal)
    return (q, k, v, do), (qd, kd, vd, o, dod, lse)


def _noalloc_via_abi(qd, kd, vd, o, dod, lse, dq, dk, dv, causal):
    L = ra.lib()
    p = ra._params(causal, 1, 0, 0, 0, None)
    return int(L.ra_attn_bwd_noalloc(ra.desc(qd), ra.desc(kd), ra.desc(vd), ra.desc(o),
                                     ra.desc(dod), ra.desc(lse), ctypes.byref(p), ra.desc(dq),
                                     ra.desc(dk), ra.desc(dv),
                                     torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("first,second", [
    ((1, 8, 2, 1500, 128, True), (1, 4, 4, 333, 64, False)),
    ((2, 7, 1, 900, 128, True), (1, 2, 2, 1, 128, True)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (B, Hq, Hkv, S, D, causal) in enumerate((first, second)):
        say(f"bwd noalloc call {i}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D} causal={causal}")
        host, (qd, kd, vd, o, dod, lse) = _case(B, Hq, Hkv, S, D, causal, 40 + i)
        ref = ra.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal)
        got = [torch.full_like(t, float("nan")) for t in (qd, kd, vd)]
        rc = _noalloc_via_abi(qd, kd, vd, o, dod, lse, *got, causal)
        assert rc == 0, ra.status_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16))
        for g, r, name in zip(got[1:], ref[1:], ("dk", "dv")):
            if Hq == Hkv:
                assert torch.equal(g.view(torch.int16), r.view(torch.int16)), name
            else:  # the same sum over the group in another fp32 order
                check_grad(to_np64(g), to_np64(r), f"noalloc {name} vs ra_attn_bwd")
        want = oracle.attention_bwd(*(si.as_f64(x, "bf16") for x in host), causal=causal)
        for g, r, w, name in zip(got, ref, want, ("dq", "dk", "dv")):
            check_grad(to_np64(g), w, f"noalloc {name}")
            check_grad(to_np64(r), w, f"ra_attn_bwd {name}")


def test_noalloc_refuses_problem_beyond_scratch():
    """B * Hq * Sq fp32 deltas beyond the fixed scratch: RA_ERR_SCRATCH, nothing launched
    (the check runs on the host before any device work)."""
    cap = ra.noalloc_scratch_bytes()
    rows = cap // 4 + 256
    Hq = 64
    S = (rows + Hq - 1) // Hq
    say(f"bwd noalloc refusal S={S}")
    q = torch.empty(1, Hq, S, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, 1, 16, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, Hq, S, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    rc = _noalloc_via_abi(q, k, k, q, q, lse, dq, dk, dv, True)
    assert ra.STATUS[rc] == "RA_ERR_SCRATCH"
