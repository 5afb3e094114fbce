"""Helpers shared by the GPU parity tests: device transfer and the tolerance checks."""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si

# Tolerances stated for this method: fp32 -> 1e-5 max abs on o and lse; bf16 inputs with
# fp32 accumulation -> o max abs 2e-2 and mean abs 2e-3, lse max abs 1e-3.
TOL = {
    "f32": dict(o_max=1e-5, o_mean=1e-5, lse_max=1e-5),
    "bf16": dict(o_max=2e-2, o_mean=2e-3, lse_max=1e-3),
}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    """Name the case before a GPU step, flushed (a fault may end the process)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_o(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "o", tol=None):
    tol = tol or TOL[dtype]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    print(f"[parity] {what}: max|err|={mx:.3e} mean|err|={mean:.3e} max|ref|="
          f"{float(np.abs(ref).max(initial=0.0)):.3e}", flush=True)
    assert mx <= tol["o_max"], f"{what}: max abs err {mx} > {tol['o_max']}"
    assert mean <= tol["o_mean"], f"{what}: mean abs err {mean} > {tol['o_mean']}"


def check_lse(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "lse"):
    tol = TOL[dtype]["lse_max"]
    assert got.shape == ref.shape
    assert not np.isnan(got).any(), f"{what}: NaN"
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    mx = float(np.abs(got[fin] - ref[fin]).max(initial=0.0))
    print(f"[parity] {what}: max|err|={mx:.3e}", flush=True)
    assert mx <= tol, f"{what}: max abs err {mx} > {tol}"


def sample_rows(B, H, S, per_head=6, seed=0):
    """(b, h, i) rows: tile edges, both ends of the sequence and a few random rows."""
    rng = np.random.default_rng(seed)
    fixed = sorted({i for i in (0, 1, 31, 32, 63, 64, 127, 128, S // 2, S - 129, S - 65, S - 2,
                                S - 1) if 0 <= i < S})
    out = []
    for b in range(B):
        for h in range(H):
            rows = set(fixed) | set(rng.integers(0, S, size=per_head).tolist())
            out += [(b, h, i) for i in sorted(rows)]
    return out


def gather_rows(t: np.ndarray, idx):
    return np.stack([t[b, h, i] for (b, h, i) in idx])


def gather_lse(t: np.ndarray, idx):
    return np.array([t[b, h, i] for (b, h, i) in idx])


# Gradient tolerance (derived in test_gpu_bwd.py's header): element-wise
# 2e-2 + 2^-8 |ref|, mean abs 2e-3, L2 within max(1e-2 |ref|, 2e-3 sqrt(n)): the relative
# L2 bound, with the mean bound's floor only where the reference itself is below it
# (gradients that vanish exactly, such as dK of a row that sees a single key).
GRAD_TOL = dict(o_max=2e-2, o_mean=2e-3)


def check_grad(got, ref, what):
    assert np.isfinite(got).all(), f"{what}: non-finite"
    err = np.abs(got - ref)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    print(f"[parity] {what}: max|err|={mx:.3e} mean|err|={mean:.3e} relL2={rel:.3e} "
          f"max|ref|={float(np.abs(ref).max(initial=0.0)):.3e}", flush=True)
    excess = float((err - (GRAD_TOL["o_max"] + 2.0 ** -8 * np.abs(ref))).max(initial=-1.0))
    assert excess <= 0.0, f"{what}: element error over 2e-2 + 2^-8|ref| by {excess}"
    assert mean <= GRAD_TOL["o_mean"], f"{what}: mean abs err {mean}"
    l2_bound = max(1e-2 * float(np.linalg.norm(ref)), GRAD_TOL["o_mean"] * np.sqrt(err.size))
    assert float(np.linalg.norm(got - ref)) <= l2_bound, f"{what}: relative L2 {rel}"
