"""The oracle pinned from two more directions (CPU only).

1. Brute force: one decoder layer written out as scalar Python loops over
   lists (math.sqrt, math.cos, math.sin, math.exp only; no NumPy or torch
   arithmetic), on tiny shapes with GQA 2:1, for several decode steps, must
   agree with the oracle in float64 (fp32 cache). The two share nothing but
   the stored weights.

2. Planted mistakes: each plausible mistake in the oracle's arithmetic (a
   flipped rotation, the wrong RoPE pairing, epsilon outside the root, no
   attention scale, the wrong kv head for a query head, an off-by-one in the
   attended positions, sigmoid for silu, a missing residual, swapped nibbles,
   truncation for round-to-nearest-even) is planted into a patched copy of the
   oracle's functions, and at least one of the pins in test_oracle_pins.py
   must then fail.
"""
import math
import struct

import numpy as np
import pytest

import oracle
import oracle.ref as ref
import synth
import test_oracle_pins as pins


# ----------------------------------------------------------------- brute force

def _loops_layer(cfg, W, x, p, Kc, Vc):
    """One decode layer of the pre-norm transformer, scalar loops; Kc and Vc
    are lists [n_kv][positions][d] extended in place with this position,
    each entry rounded to binary32 as an fp32 cache stores it (through the C
    library's float conversion in `struct`)."""
    H, d, nq, nkv, F = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.ffn
    eps, theta = cfg.rms_eps, cfg.rope_theta

    def rms(v, g):
        ms = sum(e * e for e in v) / len(v)
        r = 1.0 / math.sqrt(ms + eps)
        return [v[i] * r * g[i] for i in range(len(v))]

    def matvec(M, v):
        return [sum(M[r][c] * v[c] for c in range(len(v))) for r in range(len(M))]

    def rot(h):
        out = list(h)
        half = d // 2
        for i in range(half):
            ang = p * theta ** (-2.0 * i / d)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = h[i] * c - h[i + half] * s
            out[i + half] = h[i] * s + h[i + half] * c
        return out

    u = rms(x, W["attn_norm"])
    y = matvec(W["wqkv"], u)
    q = [rot(y[h * d:(h + 1) * d]) for h in range(nq)]
    k = [rot(y[(nq + j) * d:(nq + j + 1) * d]) for j in range(nkv)]
    v = [y[(nq + nkv + j) * d:(nq + nkv + j + 1) * d] for j in range(nkv)]
    f32 = lambda e: struct.unpack("<f", struct.pack("<f", e))[0]
    for j in range(nkv):
        Kc[j].append([f32(e) for e in k[j]])
        Vc[j].append([f32(e) for e in v[j]])
    att = []
    g = nq // nkv
    for h in range(nq):
        j = h // g
        s = [sum(q[h][e] * Kc[j][t][e] for e in range(d)) / math.sqrt(d) for t in range(p + 1)]
        m = max(s)
        w = [math.exp(z - m) for z in s]
        tot = sum(w)
        att += [sum(w[t] * Vc[j][t][e] for t in range(p + 1)) / tot for e in range(d)]
    o = matvec(W["wo"], att)
    x = [x[i] + o[i] for i in range(H)]
    u2 = rms(x, W["ffn_norm"])
    gt = matvec(W["wgate"], u2)
    up = matvec(W["wup"], u2)
    hh = [gt[f] / (1.0 + math.exp(-gt[f])) * up[f] for f in range(F)]
    dn = matvec(W["wdown"], hh)
    return [x[i] + dn[i] for i in range(H)]


@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_oracle_matches_scalar_loops(theta):
    cfg = synth.tiny(hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn=16, wtype="f32", ntype="f32",
                     kvtype="f32", rope_theta=theta, ctx=0, steps=5, seed=31)
    lw = synth.layer_weights(cfg, 0)
    o = oracle.Oracle(cfg, [lw])
    W = {}
    for name, st in lw.items():          # fp32 storage: the stored numbers themselves
        a = np.asarray(st.data, dtype=np.float64)
        W[name] = a.tolist()
    Kc = [[] for _ in range(cfg.n_kv_heads)]
    Vc = [[] for _ in range(cfg.n_kv_heads)]
    for p in range(cfg.steps):
        x = synth.rand_f32((31, 9, p), (cfg.hidden,)).astype(np.float64)
        want = _loops_layer(cfg, W, x.tolist(), p, Kc, Vc)
        got = o.layer(0, x, p)
        assert np.max(np.abs(got - np.array(want))) <= 1e-12 * max(1.0, np.max(np.abs(want))), f"pos {p}"


# -------------------------------------------------------------- planted mistakes

def _pins_that_should_fail():
    """The pins that together must catch every planted mistake."""
    return [
        pins.test_rmsnorm_unit_rms_before_weight,
        pins.test_rmsnorm_matches_torch,
        pins.test_rope_hand_cases,
        pins.test_rope_matches_rotate_half_formulation,
        pins.test_bf16_rounding_fixture,
        pins.test_q4_fixture_and_exactness,
        pins.test_attention_matches_torch_sdpa_gqa,
        pins.test_silu_fixture_and_swiglu_zero,
        pins.test_integer_exact_append,
        lambda: pins.test_decode_equals_dense_causal_forward("f32", 4, 2, "f32"),
        pins.test_i8_cache_row_fixture,
        pins.test_i8_cache_rows_round_to_nearest_step,
        lambda: pins.test_decode_equals_dense_causal_forward("bf16", 8, 2, "i8"),
        lambda: pins.test_greedy_sequence_equals_dense_forward_greedy("bf16", "bf16"),
    ]


def _rope_negative(h, p, theta):
    return _orig["rope"](h, -p, theta)


def _rope_adjacent(h, p, theta):
    h = np.asarray(h, dtype=np.float64)
    d = h.shape[-1]
    ang = p * np.power(float(theta), -np.arange(0, d, 2, dtype=np.float64) / d)
    c, s = np.cos(ang), np.sin(ang)
    out = h.copy()
    out[..., 0::2] = h[..., 0::2] * c - h[..., 1::2] * s
    out[..., 1::2] = h[..., 0::2] * s + h[..., 1::2] * c
    return out


def _rms_eps_outside(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x)) + eps) * np.asarray(g, dtype=np.float64)


def _attend_unscaled(q, K, V, group):
    return _orig["attend"](q * math.sqrt(q.shape[-1]), K, V, group)


def _attend_wrong_group(q, K, V, group):
    nq = q.shape[0]
    nkv = K.shape[0]
    out = np.empty((nq, V.shape[-1]))
    for h in range(nq):
        j = h % nkv
        out[h] = _orig["attend"](q[h:h + 1], K[j:j + 1], V[j:j + 1], 1)[0]
    return out


def _silu_sigmoid(z):
    z = np.asarray(z)
    return 1.0 / (1.0 + np.exp(-z))


def _q4_swapped(nib, scales, dtype=np.float64):
    nib = np.asarray(nib, dtype=np.uint8)
    swapped = ((nib & 0x0F) << 4) | (nib >> 4)
    return _orig["q4_dequant"](swapped.astype(np.uint8), scales, dtype)


def _round_truncate(v, kvtype):
    if kvtype != "bf16":
        return _orig["round_to_cache"](v, kvtype)
    f = np.asarray(v, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _i8_step_128(v):
    x = np.asarray(v).astype(np.float32)
    m = np.abs(x).max(axis=-1)
    scale = (m / np.float32(128)).astype(np.float32)
    inv = np.where(m == 0, np.float32(0), np.float32(128) / np.where(m == 0, np.float32(1), m)).astype(np.float32)
    return np.clip(np.rint(x * inv[..., None]), -127, 127).astype(np.int8), scale


def _i8_truncate(v):
    codes, scale = _orig["quantize_i8"](v)
    x = np.asarray(v).astype(np.float32)
    inv = np.where(scale == 0, np.float32(0), np.float32(1) / np.where(scale == 0, np.float32(1), scale))
    return np.clip(np.trunc(x * inv[..., None]), -127, 127).astype(np.int8), scale


def _i8_one_scale_per_head(v):
    # one scale for the whole [n_kv, d] block instead of one per row
    x = np.asarray(v)
    codes, scale = _orig["quantize_i8"](x.reshape(1, -1))
    return codes.reshape(x.shape), np.full(x.shape[:-1], scale[0], np.float32)


_orig = {}


def _mutations():
    return {
        "rope rotates the wrong way": [("rope", _rope_negative)],
        "rope pairs adjacent dims": [("rope", _rope_adjacent)],
        "rmsnorm eps outside the root": [("rmsnorm", _rms_eps_outside)],
        "attention without 1/sqrt(d)": [("attend", _attend_unscaled)],
        "query head h reads kv head h % n_kv": [("attend", _attend_wrong_group)],
        "sigmoid for silu": [("silu", _silu_sigmoid)],
        "nibbles swapped": [("q4_dequant", _q4_swapped)],
        "bf16 truncation": [("round_to_cache", _round_truncate)],
        "int8 step of 1/128": [("quantize_i8", _i8_step_128)],
        "int8 codes truncated": [("quantize_i8", _i8_truncate)],
        "int8 scale per block, not per row": [("quantize_i8", _i8_one_scale_per_head)],
    }


def test_pins_pass_without_a_planted_mistake():
    """The control: every pin used below passes on the oracle as written, so
    a failure under a planted mistake is that mistake's doing."""
    for pin in _pins_that_should_fail():
        pin()


@pytest.mark.parametrize("name", list(_mutations()))
def test_planted_mistake_fails_a_pin(name, monkeypatch):
    for fn in ("rope", "rmsnorm", "attend", "silu", "q4_dequant", "round_to_cache", "quantize_i8"):
        _orig[fn] = getattr(ref, fn)
    for fn, repl in _mutations()[name]:
        monkeypatch.setattr(ref, fn, repl)
        if hasattr(oracle, fn):
            monkeypatch.setattr(oracle, fn, repl)
    failed = []
    for pin in _pins_that_should_fail():
        try:
            pin()
        except AssertionError:
            failed.append(pin)
    assert failed, f"no pin caught: {name}"


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_planted_off_by_one_and_missing_residual_fail_a_pin(monkeypatch):
    """Mistakes in the layer's composition: attending to positions 0..p-1
    only, and dropping the residual add of the output projection."""
    def attention_short(self, l, q, p):
        n = max(p, 1)
        return ref.attend(q, self.Kd[l][:, :n], self.Vd[l][:, :n], self.cfg.group).reshape(-1)

    def layer_no_residual(self, l, x, p):
        q = self.qkv_rope_append(l, x, p)
        a = self.attention(l, q, p)
        x = self.proj(l, "wo", a)
        h = self.ffn(l, x)
        return x + self.proj(l, "wdown", h)

    for attr, repl in (("attention", attention_short), ("layer", layer_no_residual)):
        with monkeypatch.context() as m:
            m.setattr(ref.Oracle, attr, repl)
            failed = 0
            for pin in (lambda: pins.test_decode_equals_dense_causal_forward("f32", 4, 2, "f32"),
                        pins.test_integer_exact_append):
                try:
                    pin()
                except AssertionError:
                    failed += 1
            assert failed, f"no pin caught the planted {attr} mistake"


def test_planted_head_mistakes_fail_the_greedy_pin(monkeypatch):
    """Mistakes in the per-token tail: logits from x without the final
    RMSNorm, and the argmax taken over the logits shifted by one index."""
    def logits_no_norm(self, x):
        return ref.gemv(self.gw("head"), x)

    def greedy_shifted(self, x):
        z = self.logits(x)
        i = int(np.argmax(z[1:]))
        top2 = np.partition(z, -2)[-2:]
        return i, float(top2[1] - top2[0])

    for attr, repl in (("logits", logits_no_norm), ("greedy", greedy_shifted)):
        with monkeypatch.context() as m:
            m.setattr(ref.Oracle, attr, repl)
            with pytest.raises(AssertionError):
                pins.test_greedy_sequence_equals_dense_forward_greedy("bf16", "bf16")
