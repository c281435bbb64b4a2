"""The oracle's row-sliced projection path, pinned (CPU only).

Without a decoded copy of the weights in memory (the case for every
full-size workload), ``Oracle.proj`` decodes a stored matrix a slice of
``ROWS_PER_SLICE`` rows at a time and takes each output row's dot product
from its slice. Here that path is checked against a projection built from a
decode of every stored weight written out independently of the oracle's
decoders (bf16: the 16 bits shifted into the upper half of a binary32;
4-bit: each nibble sign-extended from its two's-complement pattern and
multiplied by its block's fp16 scale), and against the oracle's
keep-decoded path, for f32, bf16 and 4-bit matrices whose row counts leave
a ragged last slice. Planted mistakes in the slicing (rows shifted by one,
4-bit scales taken from the next slice, the ragged tail dropped) must each
fail the check.
"""
import struct

import numpy as np
import pytest

import oracle
import oracle.ref as ref
import synth

SHAPES = [(300, 256), (128, 64), (129, 96), (1, 32)]


def _decode_independent(st) -> np.ndarray:
    """Every stored weight as a Python float, element by element."""
    rows, cols = st.shape
    out = np.empty((rows, cols), dtype=np.float64)
    if st.kind == "f32":
        for r in range(rows):
            for c in range(cols):
                out[r, c] = float(st.data[r, c])
    elif st.kind == "bf16":
        for r in range(rows):
            for c in range(cols):
                out[r, c] = struct.unpack("<f", struct.pack("<I", int(st.data[r, c]) << 16))[0]
    else:
        for r in range(rows):
            for c in range(cols):
                byte = int(st.data[r, c // 2])
                nib = (byte >> 4) if c % 2 else (byte & 0xF)
                code = nib - 16 if nib >= 8 else nib
                out[r, c] = code * float(st.scales[r, c // 32])
    return out


def _stack(kind, rows, cols):
    """A one-matrix 'layer' and an oracle that must take the sliced path."""
    st = synth.rand_matrix((41, rows, cols), rows, cols, kind)
    cfg = synth.tiny(wtype=kind, ntype="f32", kvtype="f32")
    sliced = oracle.Oracle(cfg, [{"w": st}], keep_dequant=False)
    kept = oracle.Oracle(cfg, [{"w": st}], keep_dequant=True)
    assert not sliced.keep and kept.keep
    return st, sliced, kept


def _check(kind, rows, cols):
    st, sliced, kept = _stack(kind, rows, cols)
    u = synth.rand_f32((41, 7, cols), (cols,)).astype(np.float64)
    W = _decode_independent(st)
    want = np.array([sum(W[r, c] * u[c] for c in range(cols)) for r in range(rows)])
    got = sliced.proj(0, "w", u)
    scale = max(1e-300, float(np.max(np.abs(want))))
    assert np.max(np.abs(got - want)) <= 1e-12 * scale, "sliced projection differs from the scalar decode"
    assert np.max(np.abs(got - kept.proj(0, "w", u))) <= 1e-13 * scale, "sliced and kept paths differ"


@pytest.mark.parametrize("kind", ["f32", "bf16", "q4"])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_sliced_projection_matches_scalar_decode(kind, rows, cols):
    _check(kind, rows, cols)


def test_sliced_path_covers_a_ragged_last_slice():
    assert 300 % oracle.Oracle.ROWS_PER_SLICE != 0 and 129 % oracle.Oracle.ROWS_PER_SLICE != 0


_orig_dequant_rows = ref.dequant_rows


def _rows_shifted(st, r0, r1, dtype=np.float64):
    rows = st.shape[0]
    idx = np.minimum(np.arange(r0, r1) + 1, rows - 1)
    return _orig_dequant_rows(st, 0, rows, dtype)[idx]


def _scales_next_slice(st, r0, r1, dtype=np.float64):
    if st.kind != "q4":
        return _orig_dequant_rows(st, r0, r1, dtype)
    rolled = np.roll(st.scales, -oracle.Oracle.ROWS_PER_SLICE, axis=0)
    return ref.q4_dequant(st.data[r0:r1], rolled[r0:r1], dtype)


def _tail_dropped(st, r0, r1, dtype=np.float64):
    out = _orig_dequant_rows(st, r0, r1, dtype)
    if r1 - r0 < oracle.Oracle.ROWS_PER_SLICE:
        out = np.zeros_like(out)
    return out


@pytest.mark.parametrize("name,repl,kind", [("rows shifted by one", _rows_shifted, "bf16"),
                                            ("4-bit scales from the next slice", _scales_next_slice, "q4"),
                                            ("ragged last slice dropped", _tail_dropped, "f32")])
def test_planted_slicing_mistake_fails(name, repl, kind, monkeypatch):
    monkeypatch.setattr(ref, "dequant_rows", repl)
    with pytest.raises(AssertionError):
        _check(kind, 300, 256)
