"""Comparison helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_rounded_slot(gpu_bits, ora_bits, ora_exact, kvtype: str, rel_tol: float):
    """Cache slot written by the GPU against the oracle's.

    The stored value is a rounding of a float computation, so the bits are
    unique except where the exact value sits within the arithmetic error of a
    rounding boundary. Elements whose bits differ must be the neighbouring
    representable value and the oracle's exact value must lie within the
    arithmetic error of the midpoint between the two. The error of a float32
    dot product scales with the magnitude of the whole vector, not of one
    element, so the bound is `rel_tol` times the RMS of the slot. Returns the
    number of such ties.
    """
    gpu_bits = np.asarray(gpu_bits)
    ora_bits = np.asarray(ora_bits)
    if kvtype == "f32":
        assert rel_l2(gpu_bits, ora_exact) <= rel_tol
        return 0
    scale = float(np.sqrt(np.mean(np.asarray(ora_exact, dtype=np.float64) ** 2)))
    diff = gpu_bits.astype(np.uint16) != ora_bits.astype(np.uint16)
    if not diff.any():
        return 0
    g = bf16_value(gpu_bits[diff])
    o = bf16_value(ora_bits[diff])
    e = np.asarray(ora_exact, dtype=np.float64)[diff]
    gi = gpu_bits[diff].astype(np.int64)
    oi = ora_bits[diff].astype(np.int64)
    assert np.all(np.abs(gi - oi) == 1), "GPU value is not a neighbour of the oracle's rounding"
    mid = 0.5 * (g + o)
    assert np.all(np.abs(e - mid) <= rel_tol * scale), "differing rounding away from a tie"
    return int(diff.sum())
