"""Helpers for the GPU parity tests: numpy <-> device tensors and the
tolerances the comparisons use.

bf16 arrays travel as uint16 bit patterns, so the device sees exactly the
bytes the oracle reads.
"""
import numpy as np
import pytest
import torch

import swa_inputs as si

# Attention outputs: bf16 inputs -> max-abs 2e-2 and mean-abs 2e-3 against the
# fp64 oracle; fp32 inputs -> max-abs 1e-5.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5


def have_gpu():
    return torch.cuda.is_available()


def require_gpu():
    if not have_gpu():
        pytest.skip("no GPU")


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 is read as bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy; bf16 comes back as uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return si.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = ""):
    """Compare a device result (bf16 bits or fp32) with the fp64 oracle."""
    g = as_f64(got)
    assert g.shape == want.shape, (what, g.shape, want.shape)
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    err = np.abs(g - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    if dtype == "bf16":
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, \
            "%s: max-abs %.3g (tol %.3g), mean-abs %.3g (tol %.3g)" % (what, mx, BF16_MAX_ABS, mean, BF16_MEAN_ABS)
    else:
        assert mx <= F32_MAX_ABS, "%s: max-abs %.3g (tol %.3g)" % (what, mx, F32_MAX_ABS)
    return mx, mean


def log(msg: str):
    """Name the case before each GPU step, flushed, so a crash is attributable."""
    print(msg, flush=True)
