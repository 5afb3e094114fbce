"""Pins of the oracle's Ulysses layout step (bit-exact moves)."""
import numpy as np
import pytest

import oracle


def _src(P, Sl, H, D, seed=0):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 16, size=(P, Sl, H, D), dtype=np.uint16)


def _loop_seq_to_head(src, P, rank):
    _, Sl, H, D = src.shape
    Hl = H // P
    dst = np.zeros((Hl, P * Sl, D), dtype=src.dtype)
    for hh in range(Hl):
        for s in range(P):
            for t in range(Sl):
                for d in range(D):
                    dst[hh, s * Sl + t, d] = src[s, t, rank * Hl + hh, d]
    return dst


@pytest.mark.parametrize("P,Sl,H,D", [(4, 3, 8, 2), (2, 5, 2, 3), (1, 4, 3, 2)])
def test_explicit_loop(P, Sl, H, D):
    src = _src(P, Sl, H, D, seed=P * 7 + H)
    for r in range(P):
        assert np.array_equal(oracle.seq_to_head(src, P, r), _loop_seq_to_head(src, P, r))


@pytest.mark.parametrize("P,Sl,H,D", [(4, 6, 28, 4), (4, 6, 4, 4), (8, 2, 8, 3)])
def test_round_trip_bitwise(P, Sl, H, D):
    src = _src(P, Sl, H, D, seed=1)
    out = np.zeros_like(src)
    for r in range(P):
        oracle.head_to_seq(oracle.seq_to_head(src, P, r), P, r, out)
    assert np.array_equal(out, src)
    out2 = np.zeros_like(src)
    oracle.head_to_seq(oracle.seq_to_head(src, P, -1), P, -1, out2)
    assert np.array_equal(out2, src)


def test_every_element_moved_once():
    P, Sl, H, D = 4, 5, 8, 3
    src = np.arange(P * Sl * H * D, dtype=np.int64).reshape(P, Sl, H, D)
    allr = oracle.seq_to_head(src, P, -1)
    assert allr.shape == (P, H // P, P * Sl, D)
    assert np.array_equal(np.sort(allr.ravel()), np.arange(src.size))


def test_head_shard_contents():
    """Rank r's shard holds heads r*H/P.. over the whole sequence in token order."""
    P, Sl, H, D = 4, 3, 8, 1
    tok = np.arange(P * Sl).reshape(P, Sl)
    src = np.zeros((P, Sl, H, D), dtype=np.int64)
    for h in range(H):
        src[:, :, h, 0] = tok * 100 + h
    for r in range(P):
        dst = oracle.seq_to_head(src, P, r)
        for hh in range(H // P):
            assert np.array_equal(dst[hh, :, 0], np.arange(P * Sl) * 100 + r * (H // P) + hh)
