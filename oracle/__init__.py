"""CPU oracle for one batch-1 decoder-layer step (test infrastructure).

This package is test infrastructure. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the GPU path never does, and the
two share no code. It computes the plain definition of each step of the
decode layer in NumPy, in float64 by default (float32 on request), one token
at a time, with no blocking, fusion or reordering.

The step order is the decode layer as "RDNA4 Decode Kernel Fusion: Pipeline
Barriers, Not Launches, Are the Win" lists it (section "Decode is where the
bubble has nowhere to go"): input RMSNorm and its weight multiply, QKV
projection, RoPE on Q and K, attention against the KV cache, output
projection, post-attention RMSNorm and multiply, gate and up projections,
SwiGLU, down projection. The same page (section "Fusion removes the barrier
by removing the write") states that fusing these steps leaves the arithmetic
unchanged, so the oracle computes them unfused. The pages give no formula for
any step; each function below states the standard definition it uses and the
reading taken where the pages are silent.

Parity pins: every function here is pinned by tests under ``tests/``
(invariants, closed forms, hand-computed cases, library routines on the CPU,
and a dense causal forward). The composition over a stack of layers and the
greedy argmax are pinned only through their parts.
"""
from .ref import (  # noqa: F401
    Oracle,
    attend,
    bf16_bits_to_f64,
    dequant,
    q4_dequant,
    quantize_i8,
    rmsnorm,
    rope,
    rope_inv_freq,
    round_to_cache,
    silu,
    swiglu,
    gemv,
)
