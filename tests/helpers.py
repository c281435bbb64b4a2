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

    The stored value is a rounding of a float computation, so its bits are
    unique except where the exact value lies within the arithmetic error of a
    rounding boundary. With delta = rel_tol times the RMS of the slot (the
    error of a float32 dot product scales with the whole vector), every
    element whose bits differ from the oracle's rounding must lie, as a
    value, between the roundings of (exact - delta) and (exact + delta):
    it is the correct rounding of a value within delta of the exact one.
    Returns the number of such elements.
    """
    import oracle
    ora_exact = np.asarray(ora_exact, dtype=np.float64)
    if kvtype == "f32":
        assert rel_l2(gpu_bits, ora_exact) <= rel_tol
        return 0
    gpu_bits = np.asarray(gpu_bits).astype(np.uint16)
    ora_bits = np.asarray(ora_bits).astype(np.uint16)
    diff = gpu_bits != ora_bits
    if not diff.any():
        return 0
    delta = rel_tol * float(np.sqrt(np.mean(ora_exact ** 2)))
    e = ora_exact[diff]
    g = bf16_value(gpu_bits[diff])
    lo = bf16_value(oracle.round_to_cache(e - delta, "bf16"))
    hi = bf16_value(oracle.round_to_cache(e + delta, "bf16"))
    assert np.all((lo <= g) & (g <= hi)), "a cache value is not a rounding of a value near the exact one"
    assert diff.mean() < 0.05, f"{diff.sum()} of {diff.size} cache values differ"
    return int(diff.sum())
