"""Plain CPU definition of one batch-1 decoder-layer step (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module. It shares no code with the GPU path.

Page citations name the page title and section:

* [P1] "RDNA4 Decode Kernel Fusion: Pipeline Barriers, Not Launches, Are the Win"
* [P2] "Vulkan Command Buffer Reuse vs CUDA Graphs: RDNA4 Decode Overhead"
* [P3] "backend-specific kernel fusion" (gearjunkie.de)
* [P4] "Kernel fusion and block bridging" (jitllm docs)

Readings taken where the pages are silent (each is listed in the design notes
of the repository):

* pre-norm residual layer: x += O(attn(norm(x))), then x += down(ffn(norm(x)));
* RMSNorm: r = 1 / sqrt(mean(x^2) + eps), u = (x * r) * g, weight applied as
  stored (not 1 + g);
* RoPE: half-split pairs (i, i + d/2), angle p * theta^(-2i/d) formed in
  float64, rotation by +angle;
* attention scale 1/sqrt(d); query head h reads KV head floor(h / (n_q/n_kv));
  the token is appended at position p first and attends to positions 0..p;
* the cache stores rotated k and plain v rounded to the cache type; for a
  bf16 cache the value is first rounded to fp32 (the GPU path's working
  precision) and then to bf16, both round-to-nearest-even;
* int8 cache (the pages name "a leaner KV cache" as a bytes-per-token lever
  and give no scheme): one binary32 scale per cached row (one kv head at one
  position, k and v separately) and symmetric codes in [-127, 127], every
  decision taken in binary32 (quantize_i8);
* SwiGLU: h = silu(gate) * up with silu(z) = z / (1 + exp(-z));
* 4-bit weights: w = scale * code, code a two's-complement nibble, element 2i
  the low nibble of byte i, one fp16 scale per 32 consecutive inputs;
* LM head: final RMSNorm, logits = W_head . x, argmax with the lowest index
  winning ties.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- storage decode

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to float64, exactly: a bf16 value is the upper half
    of an IEEE binary32 with the lower 16 mantissa bits zero."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64, copy=False)


# two's-complement value of each 4-bit pattern 0..15
_Q4_SIGNED = np.array([0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1], dtype=np.float64)
# for every byte value b: (value of the low nibble, value of the high nibble)
_Q4_PAIRS = np.stack([_Q4_SIGNED[np.arange(256) & 0x0F], _Q4_SIGNED[np.arange(256) >> 4]], axis=1)


def q4_dequant(nib: np.ndarray, scales: np.ndarray, dtype=np.float64) -> np.ndarray:
    """4-bit block weights to real values: w[r, c] = scale[r, c // 32] * code[r, c].

    ``nib`` is ``[rows, cols/2]`` bytes; element 2i is the low nibble of byte
    i and element 2i+1 the high nibble; each nibble is a two's-complement
    integer in [-8, 7]. ``scales`` is fp16 ``[rows, cols/32]``. The product of
    an 11-bit significand and a 4-bit integer is exact in float32 and float64.
    """
    rows, half = nib.shape
    cols = half * 2
    codes = _Q4_PAIRS[nib].reshape(rows, cols)   # [rows, half, 2] -> element order 2i, 2i+1
    s = scales.astype(np.float64)
    w = codes.reshape(rows, cols // 32, 32) * s[:, :, None]
    return w.reshape(rows, cols).astype(dtype, copy=False)


def dequant_rows(st, r0: int, r1: int, dtype=np.float64) -> np.ndarray:
    """Rows r0..r1-1 of a stored matrix as real values of `dtype`."""
    if st.kind == "q4":
        return q4_dequant(st.data[r0:r1], st.scales[r0:r1], dtype)
    if st.kind == "f32":
        return np.asarray(st.data[r0:r1], dtype=np.float32).astype(dtype)
    return bf16_bits_to_f64(st.data[r0:r1]).astype(dtype, copy=False)


def dequant(st, dtype=np.float64) -> np.ndarray:
    """A stored tensor (kind f32 / bf16 / q4) as real values of `dtype`."""
    if st.kind == "f32":
        return np.asarray(st.data, dtype=np.float32).astype(dtype)
    if st.kind == "bf16":
        return bf16_bits_to_f64(st.data).astype(dtype, copy=False)
    if st.kind == "q4":
        return q4_dequant(st.data, st.scales, dtype)
    raise ValueError(st.kind)


# ---------------------------------------------------------------- layer steps

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm and its weight multiply ([P1] "Fusion removes the barrier by
    removing the write": normalize the hidden state, then multiply by a
    learned weight vector). m = mean(x^2); r = 1/sqrt(m + eps); u = (x r) g."""
    m = np.mean(x * x)
    r = 1.0 / np.sqrt(m + x.dtype.type(eps))
    return (x * r) * g


def gemv(w: np.ndarray, u: np.ndarray) -> np.ndarray:
    """A projection at batch 1: y = W u, W stored [out, in] ([P1] "Decode is
    where the bubble has nowhere to go": QKV, output, gate/up and down
    projections). No bias."""
    return w @ u


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d) for i in 0..d/2-1, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope(h: np.ndarray, p: int, theta: float) -> np.ndarray:
    """RoPE on a set of heads ``h[n_heads, d]`` at position p ([P1] "Decode
    is where the bubble has nowhere to go": RoPE on Q and K).

    Pairs are (i, i + d/2). With phi = p * omega_i (float64),
    h_i <- h_i cos(phi) - h_{i+d/2} sin(phi) and
    h_{i+d/2} <- h_i sin(phi) + h_{i+d/2} cos(phi).
    """
    d = h.shape[-1]
    phi = np.float64(p) * rope_inv_freq(d, theta)
    c = np.cos(phi).astype(h.dtype)
    s = np.sin(phi).astype(h.dtype)
    a = h[..., : d // 2]
    b = h[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def round_to_cache(v: np.ndarray, kvtype: str) -> np.ndarray:
    """The value the KV cache stores for `v` (append step; [P4] "Fusion":
    k's rotation into its KV page and v's copy into its page).

    fp32 cache: round to binary32 (nearest even). bf16 cache: round to
    binary32, then keep the upper 16 bits rounded to nearest even, returned
    as uint16 bit patterns.
    """
    f = np.asarray(v).astype(np.float32)
    if kvtype == "f32":
        return f
    if kvtype != "bf16":
        raise ValueError(kvtype)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    out = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return out.astype(np.uint16)


def quantize_i8(v: np.ndarray) -> tuple:
    """The int8 cache entry of rows ``v[..., d]`` (each row one kv head's k
    or v at one position; [P2] "Vulkan Command Buffer Reuse vs CUDA Graphs:
    RDNA4 Decode Overhead", section "What I am building next": a leaner KV
    cache as a bytes-per-token lever, scheme not given).

    x = v rounded to binary32; m = max |x| over the row; scale = m / 127 and
    inv = 127 / m, each a binary32 division rounded to nearest; code = the
    binary32 product x * inv rounded to the nearest integer (ties to even),
    clamped to [-127, 127]. A row of zeros has scale 0 and codes 0. Returns
    (codes int8 ``[..., d]``, scales float32 ``[...]``); the cached value is
    code * scale.
    """
    x = np.asarray(v).astype(np.float32)
    m = np.abs(x).max(axis=-1)
    zero = m == 0
    msafe = np.where(zero, np.float32(1), m).astype(np.float32)
    scale = np.where(zero, np.float32(0), msafe / np.float32(127)).astype(np.float32)
    inv = np.where(zero, np.float32(0), np.float32(127) / msafe).astype(np.float32)
    prod = (x * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return codes, scale


def cache_values(c: np.ndarray, kvtype: str, dtype, scales=None) -> np.ndarray:
    """Cache storage (fp32 values, bf16 bit patterns, or int8 codes with
    their per-row scales) as real values."""
    if kvtype == "f32":
        return c.astype(dtype)
    if kvtype == "i8":
        return (c.astype(np.float64) * np.asarray(scales, dtype=np.float64)[..., None]).astype(dtype)
    return bf16_bits_to_f64(c).astype(dtype)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, group: int) -> np.ndarray:
    """Decode attention of one token against the cache ([P1] "Decode is where
    the bubble has nowhere to go": attention against the KV cache).

    ``q[n_q, d]``, ``K``/``V`` ``[n_kv, T, d]`` real values, T >= 1 positions.
    For head h, j = h // group, s_t = (q_h . K_j[t]) / sqrt(d),
    w_t = exp(s_t - max s), a_h = sum_t w_t V_j[t] / sum_t w_t.
    """
    n_q, d = q.shape
    scale = q.dtype.type(1.0) / np.sqrt(q.dtype.type(d))
    out = np.empty_like(q)
    for h in range(n_q):
        j = h // group
        s = (K[j] @ q[h]) * scale
        w = np.exp(s - s.max())
        out[h] = (w @ V[j]) / w.sum()
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SwiGLU activation of the gated FFN ([P1] "Fusion removes the barrier
    by removing the write": gate projection, up projection and SwiGLU):
    h = silu(gate) * up."""
    return silu(gate) * up


# ---------------------------------------------------------------- the stack

class Oracle:
    """The decode stack on the CPU, one token at a time.

    ``layers`` is a list of per-layer weight dicts in storage encoding
    (keys attn_norm, wqkv, wo, ffn_norm, wgate, wup, wdown); ``glob`` holds
    final_norm, head and embed. The cache is kept in its storage encoding
    (fp32 values or bf16 bit patterns) as ``K[l][j, t, :]`` and ``V[l][j, t, :]``.
    Weights are decoded to `dtype` when used (or once, with
    ``keep_dequant=True``).
    """

    def __init__(self, cfg, layers, glob=None, dtype=np.float64, keep_dequant=None):
        self.cfg = cfg
        self.layers = layers
        self.glob = glob
        self.dtype = np.dtype(dtype).type
        n_elem = sum(int(np.prod(v.shape)) for lw in layers for v in lw.values())
        self.keep = (n_elem * 8 <= (64 << 20)) if keep_dequant is None else keep_dequant
        self._deq = {}
        cdt = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[cfg.kvtype]
        shape = (cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
        # the cache in its storage encoding (an int8 cache also keeps one
        # scale per row), and the same entries decoded to real values
        # (written together; attention reads the decoded copy)
        self.K = [np.zeros(shape, dtype=cdt) for _ in layers]
        self.V = [np.zeros(shape, dtype=cdt) for _ in layers]
        self.Ks = [np.zeros(shape[:2], dtype=np.float32) for _ in layers]
        self.Vs = [np.zeros(shape[:2], dtype=np.float32) for _ in layers]
        self.Kd = [np.zeros(shape, dtype=self.dtype) for _ in layers]
        self.Vd = [np.zeros(shape, dtype=self.dtype) for _ in layers]

    # -- weights
    ROWS_PER_SLICE = 128

    def proj(self, l: int, name: str, u: np.ndarray) -> np.ndarray:
        """W u for layer l's matrix `name`. Without a decoded copy kept in
        memory, the rows are decoded slice by slice (bounding memory); each
        output is still one dot product over the whole row."""
        if self.keep or (l, name) in self._deq:
            return gemv(self.w(l, name), u)
        st = self.layers[l][name]
        rows = st.shape[0]
        out = np.empty(rows, dtype=self.dtype)
        for r0 in range(0, rows, self.ROWS_PER_SLICE):
            r1 = min(rows, r0 + self.ROWS_PER_SLICE)
            out[r0:r1] = gemv(dequant_rows(st, r0, r1, self.dtype), u)
        return out

    def w(self, l: int, name: str) -> np.ndarray:
        key = (l, name)
        if key in self._deq:
            return self._deq[key]
        v = dequant(self.layers[l][name], self.dtype)
        if self.keep:
            self._deq[key] = v
        return v

    def gw(self, name: str) -> np.ndarray:
        key = ("g", name)
        if key in self._deq:
            return self._deq[key]
        v = dequant(self.glob[name], self.dtype)
        if self.keep or name != "head":
            self._deq[key] = v
        return v

    def load_prefill(self, l: int, K, V) -> None:
        """Copy cache contents (storage encoding, ``[n_kv, n, d]``) into
        positions 0..n-1 of layer l."""
        n = K.data.shape[1]
        self.K[l][:, :n] = K.data
        self.V[l][:, :n] = V.data
        if self.cfg.kvtype == "i8":
            self.Ks[l][:, :n] = K.scales
            self.Vs[l][:, :n] = V.scales
        self.Kd[l][:, :n] = cache_values(self.K[l][:, :n], self.cfg.kvtype, self.dtype, self.Ks[l][:, :n])
        self.Vd[l][:, :n] = cache_values(self.V[l][:, :n], self.cfg.kvtype, self.dtype, self.Vs[l][:, :n])

    # -- the layer's steps, in the order of [P1]
    def qkv_rope_append(self, l: int, x: np.ndarray, p: int) -> np.ndarray:
        """Input RMSNorm, QKV projection, RoPE on q and k, append k and v at p.
        Returns q as ``[n_q, d]``."""
        c = self.cfg
        u = rmsnorm(x, self.w(l, "attn_norm"), c.rms_eps)
        y = self.proj(l, "wqkv", u)
        d = c.head_dim
        q = y[: c.q_dim].reshape(c.n_q_heads, d)
        k = y[c.q_dim: c.q_dim + c.kv_dim].reshape(c.n_kv_heads, d)
        v = y[c.q_dim + c.kv_dim:].reshape(c.n_kv_heads, d)
        q = rope(q, p, c.rope_theta)
        k = rope(k, p, c.rope_theta)
        self.append(l, k, v, p)
        return q

    def append(self, l: int, k: np.ndarray, v: np.ndarray, p: int) -> None:
        """Store the rotated k and plain v ``[n_kv, d]`` at position p of
        layer l, in the cache's encoding."""
        c = self.cfg
        if c.kvtype == "i8":
            self.K[l][:, p, :], self.Ks[l][:, p] = quantize_i8(k)
            self.V[l][:, p, :], self.Vs[l][:, p] = quantize_i8(v)
        else:
            self.K[l][:, p, :] = round_to_cache(k, c.kvtype)
            self.V[l][:, p, :] = round_to_cache(v, c.kvtype)
        self.Kd[l][:, p, :] = cache_values(self.K[l][:, p, :], c.kvtype, self.dtype, self.Ks[l][:, p])
        self.Vd[l][:, p, :] = cache_values(self.V[l][:, p, :], c.kvtype, self.dtype, self.Vs[l][:, p])

    def attention(self, l: int, q: np.ndarray, p: int) -> np.ndarray:
        """Attention of q over cache positions 0..p of layer l; returns the
        head outputs concatenated in head order, ``[n_q * d]``."""
        return attend(q, self.Kd[l][:, : p + 1], self.Vd[l][:, : p + 1], self.cfg.group).reshape(-1)

    def ffn(self, l: int, x: np.ndarray) -> np.ndarray:
        """Post-attention RMSNorm, gate and up projections, SwiGLU: h ``[F]``."""
        u = rmsnorm(x, self.w(l, "ffn_norm"), self.cfg.rms_eps)
        return swiglu(self.proj(l, "wgate", u), self.proj(l, "wup", u))

    def layer(self, l: int, x: np.ndarray, p: int) -> np.ndarray:
        """One decoder layer for the token at position p: returns the new x."""
        q = self.qkv_rope_append(l, x, p)
        a = self.attention(l, q, p)
        x = x + self.proj(l, "wo", a)
        h = self.ffn(l, x)
        return x + self.proj(l, "wdown", h)

    def embed(self, token: int) -> np.ndarray:
        """x = E[token]: one row of the fp32 embedding table."""
        st = self.glob["embed"]
        return np.asarray(st.data[int(token)], dtype=np.float32).astype(self.dtype)

    def step(self, token: int, p: int, layers=None) -> list:
        """Decode one token at position p. Returns [x_in, x after layer 0,
        x after layer 1, ...]."""
        x = self.embed(token)
        out = [x]
        for l in (range(len(self.layers)) if layers is None else layers):
            x = self.layer(l, x, p)
            out.append(x)
        return out

    def logits(self, x: np.ndarray) -> np.ndarray:
        xf = rmsnorm(x, self.gw("final_norm"), self.cfg.rms_eps)
        return gemv(self.gw("head"), xf)

    def greedy(self, x: np.ndarray) -> tuple:
        """argmax of the logits (lowest index on ties) and the top-2 margin."""
        z = self.logits(x)
        i = int(np.argmax(z))
        top2 = np.partition(z, -2)[-2:]
        return i, float(top2[1] - top2[0])

    # -- construction from the seeded recipe
    @classmethod
    def from_config(cls, cfg, n_layers=None, dtype=np.float64, with_globals=True,
                    keep_dequant=None):
        import synth
        L = cfg.n_layers if n_layers is None else n_layers
        layers = [synth.layer_weights(cfg, l) for l in range(L)]
        glob = synth.model_globals(cfg) if with_globals else None
        o = cls(cfg, layers, glob, dtype=dtype, keep_dequant=keep_dequant)
        if not cfg.real_prefill and cfg.ctx > 0:
            for l in range(L):
                o.load_prefill(l, *synth.prefill(cfg, l))
        return o

    def prefill_by_decoding(self, toks) -> None:
        """Fill positions 0..len(toks)-1 by decoding the tokens in order."""
        for p, t in enumerate(toks):
            self.step(int(t), p)
