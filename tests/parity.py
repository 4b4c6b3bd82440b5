"""Tolerance checks shared by the GPU parity tests.

The bar: float32 path max |err| <= 1e-5 (O and L); bf16 inputs: O and the
gradients max |err| <= 2e-2 and ||err||_F / ||ref||_F <= 1e-2; L |err| <= 1e-3.
"""

import numpy as np
import pytest
import torch

FP32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_RFRO = 1e-2
LSE_ATOL = 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().float().cpu().numpy()
    return np.asarray(t, dtype=np.float64)


def check_fp32(got, ref, what, atol=FP32_ATOL):
    got, ref = to64(got), to64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    err = np.abs(got[fin] - ref[fin]).max(initial=0.0)
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol:g}"
    return err


def check_bf16(got, ref, what):
    got, ref = to64(got), to64(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    diff = got - ref
    err = np.abs(diff).max(initial=0.0)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    assert err <= BF16_ATOL and rel <= BF16_RFRO, \
        f"{what}: max abs err {err:.3e} (bar {BF16_ATOL}), rel Frobenius {rel:.3e} (bar {BF16_RFRO})"
    return err, rel


def check_lse(got, ref, what, atol=LSE_ATOL):
    return check_fp32(got, ref, what, atol=atol)
