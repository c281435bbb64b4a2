"""Workload shapes for the batch-1 decode stack.

Each entry describes one synthetic decode workload: the layer shape, the
storage type of the projection weights, norm weights and KV cache, the RoPE
base, the context the cache holds before decoding starts, the number of
decode steps, and the seed. The five named workloads follow the decode
layer described in "RDNA4 Decode Kernel Fusion: Pipeline Barriers, Not
Launches, Are the Win" (section "Decode is where the bubble has nowhere to
go": norm, QKV projection, RoPE, attention, output projection, norm,
gate/up, SwiGLU, down) at the sizes of the models the pages name
(a 9B-class model, Llama-2-7B, Llama-3.2-1B).

This module holds shapes only; no arithmetic of the method lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace, asdict


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    wtype: str          # projection weights: "f32" | "bf16" | "q4"
    ntype: str          # norm weights: "f32" | "bf16"
    kvtype: str         # KV cache: "f32" | "bf16"
    htype: str          # LM head: "f32" | "bf16"
    rope_theta: float
    rms_eps: float
    ctx: int            # positions already in the cache when decoding starts
    steps: int          # decode steps
    seed: int
    vocab: int = 32000
    real_prefill: bool = False   # fill the cache by decoding `ctx` tokens

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def max_ctx(self) -> int:
        return self.ctx + self.steps

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


_ELEM = {"f32": 4.0, "bf16": 2.0, "q4": 0.5 + 2.0 / 32.0, "i8": 1.0}


def elem_bytes(t: str) -> float:
    """Bytes per stored element (q4: one nibble plus a 2-byte scale per 32)."""
    return _ELEM[t]


def layer_weight_bytes(c: DecodeConfig) -> dict:
    """Bytes each fused kernel streams from its weights, per layer."""
    w = elem_bytes(c.wtype)
    n = elem_bytes(c.ntype)
    H, F = c.hidden, c.ffn
    return {
        "qkv": c.n_qkv * H * w + H * n,
        "o": H * c.q_dim * w,
        "ffn": 2 * F * H * w + H * n,
        "down": H * F * w,
    }


def kv_bytes(c: DecodeConfig, length: int) -> dict:
    """KV bytes one layer reads (over `length` positions) and writes (an
    int8 cache row also carries its 4-byte scale)."""
    row = c.head_dim * elem_bytes(c.kvtype) + (4 if c.kvtype == "i8" else 0)
    return {"read": 2 * c.n_kv_heads * row * length,
            "write": 2 * c.n_kv_heads * row}


def head_bytes(c: DecodeConfig) -> float:
    """Algorithmic HBM bytes of the LM head step: the head's weights
    ``[vocab, H]`` and the final norm weight (logits and x excluded)."""
    return c.vocab * c.hidden * elem_bytes(c.htype) + c.hidden * elem_bytes(c.ntype)


def token_bytes(c: DecodeConfig, steps: int = None) -> float:
    """Algorithmic HBM bytes of one decode token of the layer stack.

    Weights and norms of every layer, plus the KV read averaged over the
    first `steps` decode positions (default: the whole decode window; the
    cache holds ctx+1 .. ctx+steps entries while they run), plus the KV
    write. Activations (tens of KB) and the LM head are not counted.
    """
    n = c.steps if steps is None else steps
    wb = sum(layer_weight_bytes(c).values())
    avg_len = c.ctx + (n + 1) / 2.0
    kv = kv_bytes(c, 1)
    per_layer = wb + kv["read"] * avg_len + kv["write"]
    return per_layer * c.n_layers


C1 = DecodeConfig("C1_single_layer_f32", 1, 256, 4, 4, 64, 1024, "f32", "f32",
                  "f32", "f32", 10000.0, 1e-6, 16, 8, 0, real_prefill=True)
C2 = DecodeConfig("C2_llama32_1b_bf16", 16, 2048, 32, 8, 64, 8192, "bf16", "bf16",
                  "bf16", "bf16", 500000.0, 1e-6, 512, 128, 1)
C3 = DecodeConfig("C3_llama2_7b_bf16", 32, 4096, 32, 32, 128, 11008, "bf16", "bf16",
                  "bf16", "bf16", 10000.0, 1e-6, 2048, 128, 2)
C4 = DecodeConfig("C4_9b_bf16", 40, 4096, 32, 8, 128, 12288, "bf16", "bf16",
                  "bf16", "bf16", 10000.0, 1e-6, 4096, 256, 3)
C5 = DecodeConfig("C5_9b_q4", 40, 4096, 32, 8, 128, 12288, "q4", "bf16",
                  "bf16", "bf16", 10000.0, 1e-6, 8192, 256, 4)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def tiny(**kw) -> DecodeConfig:
    """A small config for brute-force checks; fields may be overridden."""
    base = DecodeConfig("tiny", 1, 8, 2, 1, 4, 16, "f32", "f32", "f32", "f32",
                        10000.0, 1e-6, 0, 6, 11, vocab=64, real_prefill=True)
    return base.with_(**kw)
