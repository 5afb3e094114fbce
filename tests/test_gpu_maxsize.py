"""GPU parity at the largest per-tensor sizes: one head whose operand spans 4 GiB, so that
element offsets pass 2^31 and byte offsets pass 2^32 (the API takes any extent up to
2^31 - 1 per axis and 64-bit strides).

The oracle cannot read 4 GiB operands in fp64, so each case is built so that the exact
result follows from a small oracle call:

* many queries (2^24 + 300 rows): query rows are independent, so sampled rows are
  checked one by one against the oracle.  The rows repeat with a period of 4099, which
  does not divide 2^24: a row read or written at an offset wrapped by 2^31 elements
  would be another row's data.
* many keys (2^24 + 256 rows): every key and value row is zero except the last 256.
  The zero rows all score 0 and carry v = 0, so their partial result is exactly
  (o = 0, lse = ln n) for n zero rows; the oracle computes the last 256 rows and its
  merge combines the two parts.  The last rows' scores (about 22.6 above the zero rows)
  make them dominate, so reading wrapped (zero) rows instead would give o close to 0.
* backward over many queries: dO is zero except on a few rows.  A row with dO = 0 has
  dP = 0 and D = 0, hence dS = 0: it adds nothing to dK, dV and its dQ is exactly 0.
  The oracle's backward over the active rows alone is therefore the exact answer, and
  the rows a wrapped write would hit must stay exactly 0.

Inputs are seeded (``seeded_inputs``), rounded to bf16, and the oracle reads the same
rounded values.
"""
import math

import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import check_grad, check_lse, check_o, require_gpu, say, to_dev, to_np64

pytestmark = pytest.mark.gpu

D = 128
WRAP = 1 << 24              # rows of D bf16 elements in 2^31 elements
BIG = WRAP + 300            # (BIG - 1) * D > 2^31
PERIOD = 4099               # repeat period of the query rows (not a divisor of 2^24)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _periodic_rows(seed: int, n_rows: int):
    """(host bf16 bits [PERIOD, D], device tensor [1, 1, n_rows, D]) with row i equal to
    host row i % PERIOD."""
    blk = si.draw(np.random.default_rng(seed), (PERIOD, D), "bf16")
    dev = to_dev(blk, "bf16")
    reps = -(-n_rows // PERIOD)
    big = dev.repeat(reps, 1)[:n_rows].view(1, 1, n_rows, D)
    del dev
    return blk, big


def _sample(n: int, seed: int):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 150, 299, PERIOD - 1, PERIOD, WRAP - 1, WRAP, WRAP + 1, WRAP + 150,
             n - 2, n - 1}
    return sorted(i for i in fixed | set(rng.integers(0, n, size=8).tolist()) if 0 <= i < n)


def _rows(t: torch.Tensor, rows):
    idx = torch.tensor(rows, dtype=torch.long, device=t.device)
    return t[0, 0].index_select(0, idx)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_queries_past_2_31(causal):
    n, skv = BIG, 256
    say(f"maxsize fwd queries causal={causal} Sq={n} Skv={skv} D={D}")
    qblk, q = _periodic_rows(3001, n)
    rng = np.random.default_rng(3002)
    k, v = si.draw(rng, (1, 1, skv, D), "bf16"), si.draw(rng, (1, 1, skv, D), "bf16")
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    out = torch.empty_like(q)
    lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
    ra.attn_fwd(q, kd, vd, causal=causal, out=out, lse=lse)
    torch.cuda.synchronize()
    rows = _sample(n, 3003)
    o_got = to_np64(_rows(out, rows))
    l_got = to_np64(_rows(lse.unsqueeze(-1), rows))[:, 0]
    del q, out, lse
    k64, v64 = si.as_f64(k, "bf16"), si.as_f64(v, "bf16")
    o_ref = np.empty((len(rows), D))
    l_ref = np.empty(len(rows))
    for j, i in enumerate(rows):
        qi = si.as_f64(qblk[i % PERIOD].reshape(1, 1, 1, D), "bf16")
        o1, l1 = oracle.full_attention(qi, k64, v64, causal=causal, q_offset=i)
        o_ref[j], l_ref[j] = o1[0, 0, 0], l1[0, 0, 0]
    check_o(o_got, o_ref, "bf16")
    check_lse(l_got, l_ref, "bf16")


def _dominant(rng, rows: int, col0: float):
    """N(0,1) bf16 rows with column 0 set to col0 (exact in bf16)."""
    x = rng.standard_normal((1, 1, rows, D), dtype=np.float32)
    x[..., 0] = col0
    return si.bf16_bits(x)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_keys_past_2_31(causal):
    sq, nk, tail = 256, WRAP + 256, 256
    n0 = nk - tail                      # zero rows
    say(f"maxsize fwd keys causal={causal} Sq={sq} Skv={nk} D={D}")
    rng = np.random.default_rng(3004)
    q = _dominant(rng, sq, 16.0)
    k_tail = _dominant(rng, tail, 16.0)
    v_tail = si.draw(rng, (1, 1, tail, D), "bf16")
    kd = torch.zeros((1, 1, nk, D), dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    kd[:, :, n0:] = to_dev(k_tail, "bf16")
    vd[:, :, n0:] = to_dev(v_tail, "bf16")
    q_off = n0 if causal else 0         # causal: the queries are the last block's rows
    qd = to_dev(q, "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((1, 1, sq), dtype=torch.float32, device="cuda")
    ra.attn_fwd(qd, kd, vd, causal=causal, q_offset=q_off, out=out, lse=lse)
    torch.cuda.synchronize()
    del kd, vd
    q64 = si.as_f64(q, "bf16")
    # zero rows: n0 equal scores (0) over v = 0, all visible to every query row
    o_a = np.zeros((1, 1, sq, D))
    l_a = np.full((1, 1, sq), math.log(n0))
    o_b, l_b = oracle.full_attention(q64, si.as_f64(k_tail, "bf16"), si.as_f64(v_tail, "bf16"),
                                     causal=causal, q_offset=q_off, kv_offset=n0)
    o_ref, l_ref = oracle.lse_merge([o_a, o_b], [l_a, l_b])
    # the tail carries the softmax mass, so wrapped (zero) reads would move o far past
    # the tolerance
    assert np.exp(l_b - l_ref).min() > 0.99 and np.abs(o_ref).mean() > 0.05
    check_o(to_np64(out), o_ref, "bf16")
    check_lse(to_np64(lse), l_ref, "bf16")


def test_bwd_queries_past_2_31():
    n, skv = BIG, 256
    say(f"maxsize bwd queries Sq={n} Skv={skv} D={D}")
    qblk, q = _periodic_rows(3005, n)
    rng = np.random.default_rng(3006)
    k, v = si.draw(rng, (1, 1, skv, D), "bf16"), si.draw(rng, (1, 1, skv, D), "bf16")
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    active = sorted({PERIOD + 7, 1000} | set(range(n - 300, n)))
    do_act = si.draw(rng, (len(active), D), "bf16")
    dout = torch.zeros_like(q)
    idx = torch.tensor(active, dtype=torch.long, device="cuda")
    dout[0, 0].index_copy_(0, idx, to_dev(do_act, "bf16"))
    o, lse = ra.attn_fwd(q, kd, vd)
    dq, dk, dv = ra.attn_bwd(q, kd, vd, o, dout, lse)
    torch.cuda.synchronize()
    o_got = to_np64(_rows(o, active))
    dq_got = to_np64(_rows(dq, active))
    idle = [0, 1, 150, 299, PERIOD - 1, WRAP - 1, WRAP - 300]   # where wrapped writes land
    dq_idle = _rows(dq, idle).float().cpu().numpy()
    dk_got, dv_got = to_np64(dk), to_np64(dv)
    del q, o, lse, dout, dq
    q_act = si.as_f64(qblk[np.array(active) % PERIOD].reshape(1, 1, -1, D), "bf16")
    k64, v64 = si.as_f64(k, "bf16"), si.as_f64(v, "bf16")
    do64 = si.as_f64(do_act.reshape(1, 1, -1, D), "bf16")
    o_ref, _ = oracle.full_attention(q_act, k64, v64)
    dq_ref, dk_ref, dv_ref = oracle.attention_bwd(q_act, k64, v64, do64)
    check_o(o_got, o_ref[0, 0], "bf16")
    check_grad(dq_got, dq_ref[0, 0], "dq")
    check_grad(dk_got, dk_ref, "dk")
    check_grad(dv_got, dv_ref, "dv")
    assert not dq_idle.any(), "dq of a row with dO = 0 must be exactly 0"
