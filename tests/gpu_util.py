"""Helpers for the GPU parity tests: host<->device moves and the tolerances."""
import numpy as np
import torch

import oracle

# attention-output tolerances (bf16: |d| <= 2e-2 + 1e-2 |ref|; fp32: |d| <= 1e-5 |ref| + 1e-6)
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-6, 1e-5)}


def dev(arr: np.ndarray) -> torch.Tensor:
    """Host array from synth (uint16 bf16 bits, float32 or int32) -> GPU tensor."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst |d|={err.max():.3e} "
                           f"at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def assert_lse_close(got: np.ndarray, ref: np.ndarray, what: str, tol: float = 1e-3):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    err = np.abs(got[fin] - ref[fin])
    assert (err <= tol * (1 + np.abs(ref[fin]))).all(), f"{what}: lse worst |d|={err.max():.3e}"


def causal_scores_equal(gpu_scores: np.ndarray, ref_rows, ts, what: str):
    """Exact equality of the visible part of each sampled score row."""
    for t, r in zip(ts, ref_rows):
        g = gpu_scores[t, :len(r)]
        ref32 = r.astype(np.float32)
        assert np.array_equal(g, ref32), f"{what}: row {t} differs at {np.flatnonzero(g != ref32)[:8]}"


def as_f64(x):
    return oracle.as_f64(x)
