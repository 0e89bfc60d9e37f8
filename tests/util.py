"""Shared helpers of the test-suite (tolerance of the fused product)."""
import numpy as np

# Per-element bound on y: |y_gpu - y_ref| <= REL * |y_ref| + ABS_RMS * rms(y_ref),
# rms over all M x N outputs of one call.
REL = 8e-3
ABS_RMS = 1e-3


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    err = np.abs(y_gpu - y_ref)
    bound = REL * np.abs(y_ref) + ABS_RMS * rms
    bad = np.nonzero(err > bound)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite outputs"
    assert bad[0].size == 0, (
        f"{what}: {bad[0].size} of {y_ref.size} outputs out of tolerance; worst "
        f"err/bound={float(np.max(err / np.maximum(bound, 1e-300))):.3g}; first at "
        f"{tuple(int(b[0]) for b in bad)} gpu={y_gpu[tuple(b[0] for b in bad)]} "
        f"ref={y_ref[tuple(b[0] for b in bad)]} rms={rms:.4g}")
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
