"""Shared helpers of the GPU parity tests: uploads, tolerance checks, progress lines."""
import sys

import numpy as np

BF16_ULP = 2.0 ** -8   # relative spacing of bf16 numbers near 1 (half of it is the RNE bound)
F32_EPS = 2.0 ** -23


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str = "f32", device: str = "cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device=device, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_within(got: np.ndarray, ref: np.ndarray, tol, what: str) -> float:
    """Element-wise |got - ref| <= tol (tol scalar or array). Returns the worst ratio."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    ratio = err / np.maximum(tol, 1e-300)
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: |got-ref| exceeds tolerance at {i}: got {got[i]!r} ref "
                             f"{ref[i]!r} tol {np.broadcast_to(tol, ratio.shape)[i]!r}; "
                             f"worst ratio {worst:.3g}")
    say(f"  {what}: max err {float(err.max()) if err.size else 0:.3e}, worst err/tol {worst:.3f}")
    return worst


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    return float(np.abs(np.asarray(got, np.float64) - ref).max() / np.abs(ref).max())


def gemm_tol(a: np.ndarray, w: np.ndarray, ref: np.ndarray, out_bf16: bool) -> np.ndarray:
    """Bound for y = a w^T computed with fp32 accumulation over K terms and (optionally) one
    bf16 rounding of the result: K * 2^-23 * (|a| |w|^T) + rounding of |ref|."""
    K = a.shape[-1]
    mag = np.abs(a.reshape(-1, K)) @ np.abs(w).T.astype(np.float64)
    tol = 2.0 * K * F32_EPS * mag.reshape(ref.shape) + 1e-30
    if out_bf16:
        tol = tol + BF16_ULP * np.abs(ref)
    return tol
