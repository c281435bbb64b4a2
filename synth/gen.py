"""Seeded synthetic inputs for the decode stack, shared by both implementations.

Every tensor is drawn from NumPy's PCG64 generator keyed by
``SeedSequence([seed, layer, tensor_id, chunk, stream])``. Tensors are drawn
in fixed row chunks so that the values do not depend on the thread count and a
single tensor can be regenerated on its own.

Distributions (the decode workloads' stated recipe):

* projection and LM-head weights: N(0, 0.02^2), drawn as fp32 and stored as
  fp32, bf16 (round to nearest even) or 4-bit blocks;
* 4-bit blocks: 32 signed int4 codes per block along the input dimension,
  one fp16 scale per block drawn as |N(0, 0.02^2)| / 7. Workload codes are
  uniform over the symmetric range [-7, 7] (zero-mean, like the codes of
  quantized trained weights); test matrices may draw them uniformly over the
  whole range [-8, 7] to cover every code. Nibble layout: element 2i is the
  low nibble of byte i, element 2i+1 the high nibble;
* norm weights: 1 + N(0, 0.01^2);
* token embedding table: N(0, 1), fp32;
* synthetic cache prefill: N(0, (0.02 * sqrt(H))^2), the spread of a
  projection of a unit-RMS vector, stored in the cache type;
* tokens: uniform on [0, vocab).

Only storage encodings live here (fp32 -> bf16 and int4 packing of *inputs*);
no step of the decode-layer arithmetic does.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import DecodeConfig

# tensor ids inside a layer
ATTN_NORM, WQKV, WO, FFN_NORM, WGATE, WUP, WDOWN, KPRE, VPRE = range(9)
# tensor ids of the per-model tensors (stored under layer index GLOBAL)
GLOBAL = 10_000
FINAL_NORM, HEAD, EMBED, TOKENS = range(4)

CHUNK_ELEMS = 1 << 20


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_POOL: Optional[ThreadPoolExecutor] = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=_workers())
    return _POOL


def _rng(key, chunk: int, stream: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(k) for k in key] + [chunk, stream])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode fp32 values as bf16 bit patterns, round to nearest even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass
class Stored:
    """A tensor in its storage encoding.

    kind "f32": ``data`` is float32; kind "bf16": ``data`` is uint16 bf16 bit
    patterns; kind "q4": ``data`` is uint8 nibbles ``[rows, cols/2]`` and
    ``scales`` float16 ``[rows, cols/32]``; kind "i8" (cache rows): ``data``
    is int8 codes ``[..., d]`` and ``scales`` float32 ``[...]``, one per row.
    """
    kind: str
    data: np.ndarray
    scales: Optional[np.ndarray] = None

    @property
    def shape(self):
        if self.kind == "q4":
            return (self.data.shape[0], self.data.shape[1] * 2)
        return self.data.shape

    @property
    def nbytes(self) -> int:
        return self.data.nbytes + (0 if self.scales is None else self.scales.nbytes)


def _normal_rows(key, rows: int, cols: int, std: float, mean: float, kind: str) -> Stored:
    """rows x cols of N(mean, std^2) stored as `kind` ("f32" or "bf16")."""
    rpc = max(1, CHUNK_ELEMS // cols)
    nchunk = (rows + rpc - 1) // rpc
    out = np.empty((rows, cols), dtype=np.float32 if kind == "f32" else np.uint16)

    def work(ci: int) -> None:
        r0 = ci * rpc
        r1 = min(rows, r0 + rpc)
        buf = _rng(key, ci).standard_normal((r1 - r0, cols), dtype=np.float32)
        if std != 1.0:
            buf *= np.float32(std)
        if mean != 0.0:
            buf += np.float32(mean)
        out[r0:r1] = buf if kind == "f32" else f32_to_bf16_bits(buf)

    list(_pool().map(work, range(nchunk)))
    return Stored(kind, out)


def _q4_rows(key, rows: int, cols: int, std: float, codes: str = "symmetric") -> Stored:
    """rows x cols of 4-bit block-quantized weights (see module docstring).
    codes="symmetric": uniform over [-7, 7]; codes="uniform": uniform over [-8, 7]."""
    assert cols % 32 == 0 and codes in ("symmetric", "uniform")
    lo = -8 if codes == "uniform" else -7
    rpc = max(1, CHUNK_ELEMS // cols)
    nchunk = (rows + rpc - 1) // rpc
    nib = np.empty((rows, cols // 2), dtype=np.uint8)
    sc = np.empty((rows, cols // 32), dtype=np.float16)

    def work(ci: int) -> None:
        r0 = ci * rpc
        r1 = min(rows, r0 + rpc)
        c = _rng(key, ci, 0).integers(lo, 8, size=(r1 - r0, cols), dtype=np.int8)
        u = c.view(np.uint8) & np.uint8(0x0F)
        nib[r0:r1] = u[:, 0::2] | (u[:, 1::2] << np.uint8(4))
        z = _rng(key, ci, 1).standard_normal((r1 - r0, cols // 32), dtype=np.float32)
        sc[r0:r1] = (np.abs(z) * np.float32(std) / np.float32(7.0)).astype(np.float16)

    list(_pool().map(work, range(nchunk)))
    return Stored("q4", nib, sc)


def _matrix(cfg: DecodeConfig, key, rows: int, cols: int, kind: str) -> Stored:
    if kind == "q4":
        return _q4_rows(key, rows, cols, 0.02)
    return _normal_rows(key, rows, cols, 0.02, 0.0, kind)


def _norm(key, n: int, kind: str) -> Stored:
    s = _normal_rows(key, 1, n, 0.01, 1.0, kind)
    return Stored(s.kind, s.data.reshape(n))


def layer_weights(cfg: DecodeConfig, layer: int) -> dict:
    """One layer's weights in storage encoding.

    ``wqkv`` is ``[(n_q + 2 n_kv) * d, H]`` with rows ordered: the q heads,
    then the k heads, then the v heads, each head's ``d`` rows contiguous.
    ``wo`` is ``[H, n_q * d]``, ``wgate``/``wup`` are ``[F, H]`` and
    ``wdown`` is ``[H, F]``.
    """
    s, H, F = cfg.seed, cfg.hidden, cfg.ffn
    k = lambda tid: (s, layer, tid)
    return {
        "attn_norm": _norm(k(ATTN_NORM), H, cfg.ntype),
        "wqkv": _matrix(cfg, k(WQKV), cfg.n_qkv, H, cfg.wtype),
        "wo": _matrix(cfg, k(WO), H, cfg.q_dim, cfg.wtype),
        "ffn_norm": _norm(k(FFN_NORM), H, cfg.ntype),
        "wgate": _matrix(cfg, k(WGATE), F, H, cfg.wtype),
        "wup": _matrix(cfg, k(WUP), F, H, cfg.wtype),
        "wdown": _matrix(cfg, k(WDOWN), H, F, cfg.wtype),
    }


def prefill(cfg: DecodeConfig, layer: int) -> tuple:
    """Synthetic cache contents for positions 0..ctx-1 of one layer.

    Returns (K, V), each ``[n_kv, ctx, d]`` in the cache storage encoding.
    """
    std = 0.02 * float(np.sqrt(cfg.hidden))
    rows = cfg.n_kv_heads * cfg.ctx
    if cfg.kvtype == "i8":
        return tuple(_i8_rows((cfg.seed, layer, tid), cfg.n_kv_heads, cfg.ctx, cfg.head_dim, std)
                     for tid in (KPRE, VPRE))
    out = []
    for tid in (KPRE, VPRE):
        st = _normal_rows((cfg.seed, layer, tid), rows, cfg.head_dim, std, 0.0, cfg.kvtype)
        out.append(Stored(st.kind, st.data.reshape(cfg.n_kv_heads, cfg.ctx, cfg.head_dim)))
    return tuple(out)


def embedding(cfg: DecodeConfig) -> Stored:
    """The fp32 token embedding table ``[vocab, H]``."""
    return _normal_rows((cfg.seed, GLOBAL, EMBED), cfg.vocab, cfg.hidden, 1.0, 0.0, "f32")


def model_globals(cfg: DecodeConfig) -> dict:
    """Final norm weight ``[H]``, LM head ``[vocab, H]`` and fp32 embedding ``[vocab, H]``."""
    s, H = cfg.seed, cfg.hidden
    return {
        "final_norm": _norm((s, GLOBAL, FINAL_NORM), H, cfg.ntype),
        "head": _normal_rows((s, GLOBAL, HEAD), cfg.vocab, H, 0.02, 0.0, cfg.htype),
        "embed": embedding(cfg),
    }


def tokens(cfg: DecodeConfig, n: Optional[int] = None) -> np.ndarray:
    """Teacher-forced token list: ``ctx`` prefill tokens when the cache is
    filled by decoding, then one token per decode step."""
    if n is None:
        n = (cfg.ctx if cfg.real_prefill else 0) + cfg.steps
    return _rng((cfg.seed, GLOBAL, TOKENS), 0).integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)



def rand_f32(key, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """A seeded fp32 array of N(mean, std^2) values (test inputs)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    st = _normal_rows(tuple(key), 1, max(n, 1), std, mean, "f32")
    return st.data.reshape(-1)[:n].reshape(shape)


def rand_matrix(key, rows: int, cols: int, kind: str, std: float = 0.02, q4_codes: str = "uniform") -> Stored:
    """A seeded weight matrix in storage encoding `kind` (test inputs); 4-bit
    test matrices draw their codes uniformly over [-8, 7] unless q4_codes is
    "symmetric" (the workloads' [-7, 7])."""
    if kind == "q4":
        return _q4_rows(tuple(key), rows, cols, std, q4_codes)
    return _normal_rows(tuple(key), rows, cols, std, 0.0, kind)


def rand_norm(key, n: int, kind: str) -> Stored:
    """A seeded norm-weight vector 1 + N(0, 0.01^2) (test inputs)."""
    return _norm(tuple(key), n, kind)


def _i8_rows(key, n_kv: int, length: int, d: int, std: float) -> Stored:
    """int8 cache rows: codes uniform in [-127, 127] and one positive scale
    per row, drawn so that the values have about the given std (a uniform
    code has std 73.3)."""
    rng = _rng(tuple(key), 0, 1)
    codes = rng.integers(-127, 128, size=(n_kv, length, d), dtype=np.int16).astype(np.int8)
    scales = (np.float32(std / 73.3) * rng.uniform(0.75, 1.25, size=(n_kv, length))).astype(np.float32)
    return Stored("i8", codes, scales)


def rand_cache(key, n_kv: int, length: int, d: int, kind: str, std: float) -> Stored:
    """Seeded cache contents ``[n_kv, length, d]`` in storage encoding (test inputs)."""
    if kind == "i8":
        return _i8_rows(key, n_kv, length, d, std)
    st = _normal_rows(tuple(key), n_kv * length, d, std, 0.0, kind)
    return Stored(st.kind, st.data.reshape(n_kv, length, d))
