"""GPU ra_ulysses_permute is bit-exact against the oracle, all ranks, both directions."""
import numpy as np
import pytest
import torch

import long_context_exact_tiled_amd as ra
import oracle
import seeded_inputs as si
from _gpu import require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().view(torch.int32).numpy().view(np.uint32)


@pytest.mark.parametrize("P,Sl,H,D,dtype", [
    (4, 8192, 28, 128, "bf16"),   # the Qwen2.5-7B-shaped query source
    (4, 8192, 4, 128, "bf16"),    # its key/value source
    (2, 37, 6, 64, "bf16"),
    (8, 5, 8, 128, "f32"),
    (1, 19, 3, 64, "f32"),
    (3, 11, 6, 96, "bf16"),       # 192-byte rows: the flat kernel
    (2, 70, 4, 32, "bf16"),       # 64-byte rows: the flat kernel
])
def test_permute_all_ranks_both_directions(P, Sl, H, D, dtype):
    say(f"permute P={P} Sl={Sl} H={H} D={D} {dtype}")
    rng = np.random.Generator(np.random.PCG64(77))
    src = si.draw(rng, (P, Sl, H, D), dtype)
    src_bits = src if dtype == "bf16" else src.view(np.uint32)
    sd = to_dev(src, dtype)
    back = torch.zeros_like(sd)
    for r in range(P):
        dst = ra.ulysses_permute(sd, P, r, 0)
        ref = oracle.seq_to_head(src_bits, P, r)
        assert np.array_equal(_bits(dst), ref), f"seq->head rank {r}"
        ra.ulysses_permute(dst, P, r, 1, out=back)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back), src_bits), "head->seq round trip"
    # every rank at once, then back
    allr = ra.ulysses_permute(sd, P, -1, 0)
    assert np.array_equal(_bits(allr), oracle.seq_to_head(src_bits, P, -1))
    back2 = torch.zeros_like(sd)
    ra.ulysses_permute(allr, P, -1, 1, out=back2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(back2), src_bits)


def test_head_to_seq_writes_only_its_slice():
    say("permute head->seq slice only")
    P, Sl, H, D = 4, 64, 8, 128
    dst = torch.full((P, Sl, H, D), 7.0, dtype=torch.bfloat16, device="cuda")
    shard = torch.randn(H // P, P * Sl, D, device="cuda").bfloat16()
    ra.ulysses_permute(shard, P, 2, 1, out=dst)
    torch.cuda.synchronize()
    ref = oracle.head_to_seq(_bits(shard), P, 2,
                             np.full((P, Sl, H, D), _bits(torch.tensor(7.0).bfloat16())[()],
                                     dtype=np.uint16))
    assert np.array_equal(_bits(dst), ref)


@pytest.mark.parametrize("rank", [0, 3, -1])
def test_permute_multi_qkv_one_launch(rank):
    """q, k and v of the 32K GQA layer (28 and 4 heads, 4 shards of 8192 tokens) moved by
    one ra_ulysses_permute_n call: each bit-exact, then back (dir 1) in one call."""
    say(f"permute multi q/k/v rank={rank}")
    qs, ks, vs = si.draw_ulysses_sources(1004)
    P = 4
    srcs = [to_dev(x, "bf16") for x in (qs, ks, vs)]
    outs = ra.ulysses_permute_multi(srcs, P, rank, 0)
    torch.cuda.synchronize()
    for got, src in zip(outs, (qs, ks, vs)):
        assert np.array_equal(_bits(got), oracle.seq_to_head(src, P, rank))
    backs = [torch.zeros_like(s) for s in srcs]
    if rank >= 0:  # dir 1 writes only the rank's head slice: compare that against the oracle
        ra.ulysses_permute_multi(outs, P, rank, 1, outs=backs)
        torch.cuda.synchronize()
        for got, src, o in zip(backs, (qs, ks, vs), outs):
            zero = np.zeros(src.shape, dtype=np.uint16)
            assert np.array_equal(_bits(got), oracle.head_to_seq(_bits(o), P, rank, zero))
    else:
        ra.ulysses_permute_multi(outs, P, -1, 1, outs=backs)
        torch.cuda.synchronize()
        for got, src in zip(backs, (qs, ks, vs)):
            assert np.array_equal(_bits(got), src)


def test_permute_multi_mixed_rows_and_dtypes():
    """Pairs with different row sizes or dtypes (pair by pair) and a pair with no tokens."""
    say("permute multi mixed")
    rng = np.random.Generator(np.random.PCG64(78))
    a = si.draw(rng, (2, 37, 6, 64), "bf16")     # 128-byte rows
    b = si.draw(rng, (2, 37, 4, 96), "bf16")     # 192-byte rows
    c = si.draw(rng, (2, 37, 2, 32), "f32")      # 128-byte rows, fp32
    e = np.zeros((2, 0, 4, 64), dtype=np.uint16)
    srcs = [to_dev(a, "bf16"), to_dev(b, "bf16"), to_dev(c, "f32"), to_dev(e, "bf16")]
    outs = ra.ulysses_permute_multi(srcs, 2, 1, 0)
    torch.cuda.synchronize()
    for got, src in zip(outs[:3], (a, b, c.view(np.uint32))):
        assert np.array_equal(_bits(got), oracle.seq_to_head(src, 2, 1))
    assert outs[3].numel() == 0
    # bf16 and fp32 pairs with 128-byte rows share one launch
    outs = ra.ulysses_permute_multi([srcs[0], srcs[2]], 2, 0, 0)
    torch.cuda.synchronize()
    for got, src in zip(outs, (a, c.view(np.uint32))):
        assert np.array_equal(_bits(got), oracle.seq_to_head(src, 2, 0))
