"""Shared test helpers: device upload/download and the error bound.

The per-element bound for every GEMM result is |gpu - ref| <= 1e-3 * S + 1e-5
with S = sum_k |a_ik * b_kj| (ref and S from the oracle, in float64).  Where
the device output is bf16, the rounding of the output itself is part of its
specified type: half a bf16 quantum of the reference value is added.
"""
import numpy as np


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def bf16_from_dev(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_half_quantum(ref: np.ndarray) -> np.ndarray:
    a = np.abs(ref)
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


def err_ratio(got, ref, scale, bf16_out=False) -> float:
    """max over elements of |got - ref| / tol; <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    tol = 1e-3 * np.asarray(scale, dtype=np.float64) + 1e-5
    if bf16_out:
        tol = tol + bf16_half_quantum(ref)
    r = np.abs(got - ref) / tol
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(r.max()) if r.size else 0.0
