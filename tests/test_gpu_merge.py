"""GPU parity of ra_lse_merge fed with the oracle's own chunk partials."""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import check_lse, check_o, require_gpu, say, to_np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _oracle_parts(seed, B, H, Sq, Skv, D, P, causal, q_off):
    q, k, v = si.draw_qkv(seed, (B, H, Sq, D), (B, H, Skv, D), "f32")
    q64, k64, v64 = (si.as_f64(x, "f32") for x in (q, k, v))
    parts = [oracle.chunk_partial(q64, k64, v64, c, P, causal=causal, q_offset=q_off)
             for c in range(P)]
    full = oracle.full_attention(q64, k64, v64, causal=causal, q_offset=q_off)
    return parts, full


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
def test_merge_fp32_partials(out_dtype, D):
    say(f"merge fp32 parts D={D} out={out_dtype}")
    # causal share at an offset: the last chunks hold no visible key (empty partials),
    # and the first rows see only part of the chunks
    parts, (o_full, l_full) = _oracle_parts(3, 2, 3, 96, 256, D, 8, True, 40)
    o_parts = [torch.from_numpy(p[0].astype(np.float32)).cuda() for p in parts]
    l_parts = [torch.from_numpy(p[1].astype(np.float32)).cuda() for p in parts]
    o, lse = ra.lse_merge(o_parts, l_parts, out_dtype=out_dtype)
    torch.cuda.synchronize()
    dt = "f32" if out_dtype == torch.float32 else "bf16"
    # the oracle merge of the same (fp32-rounded) partials, and the full definition
    o_ref, l_ref = oracle.lse_merge([x.cpu().numpy() for x in o_parts],
                                    [x.cpu().numpy() for x in l_parts])
    check_o(to_np64(o), o_ref, dt, "o vs oracle merge")
    check_lse(to_np64(lse), l_ref, "f32", "lse vs oracle merge")
    check_o(to_np64(o), o_full, "bf16" if dt == "bf16" else "f32", "o vs full attention",
            tol=dict(o_max=2e-2 if dt == "bf16" else 2e-5, o_mean=2e-3 if dt == "bf16" else 2e-5))


def test_merge_bf16_partials_and_all_empty_rows():
    say("merge bf16 parts with all-empty rows")
    rng = np.random.default_rng(9)
    n, shape = 5, (1, 2, 40, 128)
    o_np = [rng.standard_normal(shape).astype(np.float32) for _ in range(n)]
    l_np = [(3 * rng.standard_normal(shape[:3])).astype(np.float32) for _ in range(n)]
    for i in range(n):          # rows 0..9 empty in every part, row 10.. empty in some
        l_np[i][:, :, :10] = -np.inf
        o_np[i][:, :, :10] = 0.0
    l_np[1][:, :, 10:20] = -np.inf
    o_bf = [torch.from_numpy(x).bfloat16().cuda() for x in o_np]
    l_t = [torch.from_numpy(x).cuda() for x in l_np]
    o, lse = ra.lse_merge(o_bf, l_t, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge([x.float().cpu().numpy() for x in o_bf], l_np)
    check_o(to_np64(o), o_ref, "f32", "o")
    check_lse(to_np64(lse), l_ref, "f32", "lse")
    assert torch.all(o[:, :, :10] == 0) and torch.all(torch.isneginf(lse[:, :, :10]))


def test_merge_in_place():
    say("merge in place")
    rng = np.random.default_rng(10)
    shape = (1, 2, 33, 64)
    o_np = [rng.standard_normal(shape).astype(np.float32) for _ in range(3)]
    l_np = [rng.standard_normal(shape[:3]).astype(np.float32) for _ in range(3)]
    o_t = [torch.from_numpy(x).cuda() for x in o_np]
    l_t = [torch.from_numpy(x).cuda() for x in l_np]
    ra.lse_merge(o_t, l_t, out=o_t[0], lse=l_t[0])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.lse_merge(o_np, l_np)
    check_o(to_np64(o_t[0]), o_ref, "f32", "o in place")
    check_lse(to_np64(l_t[0]), l_ref, "f32", "lse in place")


def test_merge_identity_single_part():
    o = torch.randn(1, 1, 7, 128, device="cuda")
    l = torch.randn(1, 1, 7, device="cuda")
    mo, ml = ra.lse_merge([o], [l])
    torch.cuda.synchronize()
    assert torch.allclose(mo, o, atol=1e-6) and torch.allclose(ml, l, atol=1e-6)
