"""Pins for the CPU oracle: closed forms, invariants, hand-derived fixtures,
library routines on the CPU, brute force and a dense causal forward.

None of these compares the oracle with itself: each check comes from the
mathematics of the step (or an independent library formulation) so that a
dropped term, a sign or index error, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.ref import cache_values

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_unit_rms_before_weight():
    x = synth.rand_f32((1, 1, 1), (4096,)).astype(np.float64)
    u = oracle.rmsnorm(x, np.ones_like(x), 1e-6)
    m = np.mean(x * x)
    rms = math.sqrt(float(np.mean(u * u)))
    assert abs(rms - math.sqrt(m / (m + 1e-6))) < 1e-12
    assert abs(rms - 1.0) < 1e-6


def test_rmsnorm_constant_vector_closed_form():
    # x = c * 1  ->  u = c / sqrt(c^2 + eps) * g ; c small so eps matters
    c, eps = 1e-3, 1e-6
    g = 1.0 + synth.rand_f32((1, 1, 2), (64,), std=0.01).astype(np.float64)
    u = oracle.rmsnorm(np.full(64, c), g, eps)
    np.testing.assert_allclose(u, c / math.sqrt(c * c + eps) * g, rtol=1e-14)


def test_rmsnorm_matches_torch():
    x = synth.rand_f32((1, 1, 3), (2048,)).astype(np.float64)
    g = 1.0 + synth.rand_f32((1, 1, 4), (2048,), std=0.01).astype(np.float64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (2048,), weight=torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(oracle.rmsnorm(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=0)


# ------------------------------------------------------------------ RoPE

def test_rope_hand_cases():
    for case in _gold("rope_hand.json")["cases"]:
        x = np.array(case["x"], dtype=np.float64)[None]
        y = oracle.rope(x, case["p"], case["theta"])[0]
        np.testing.assert_allclose(y, case["y"], rtol=0, atol=2e-16, err_msg=case["why"])


def test_rope_identity_at_zero_and_pair_norms():
    h = synth.rand_f32((1, 1, 5), (4, 128)).astype(np.float64)
    assert np.array_equal(oracle.rope(h, 0, 10000.0), h)
    for p in (1, 17, 4095, 8447):
        y = oracle.rope(h, p, 10000.0)
        n0 = h[:, :64] ** 2 + h[:, 64:] ** 2
        n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_rope_relative_position_property():
    a = synth.rand_f32((1, 1, 6), (1, 64)).astype(np.float64)
    b = synth.rand_f32((1, 1, 7), (1, 64)).astype(np.float64)
    ref = float(oracle.rope(a, 30, 500000.0)[0] @ oracle.rope(b, 10, 500000.0)[0])
    for p, s in ((20, 0), (120, 100), (1030, 1010)):
        v = float(oracle.rope(a, p, 500000.0)[0] @ oracle.rope(b, s, 500000.0)[0])
        assert abs(v - ref) < 1e-11 * max(1.0, abs(ref))


def test_rope_matches_rotate_half_formulation():
    # the same rotation written as x*cos + rotate_half(x)*sin, rotate_half(x) = [-x2, x1]
    d, theta, p = 128, 10000.0, 777
    x = torch.from_numpy(synth.rand_f32((1, 1, 8), (3, d)).astype(np.float64))
    inv = 1.0 / (theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.cat([p * inv, p * inv])
    rot = torch.cat([-x[:, d // 2:], x[:, : d // 2]], dim=-1)
    ref = x * torch.cos(ang) + rot * torch.sin(ang)
    np.testing.assert_allclose(oracle.rope(x.numpy(), p, theta), ref.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ storage

def test_bf16_rounding_fixture():
    for case in _gold("bf16_rne.json")["cases"]:
        f = np.array([int(case["f32"], 16)], dtype=np.uint32).view(np.float32)
        with np.errstate(over="ignore"):
            got = int(oracle.round_to_cache(f.astype(np.float64), "bf16")[0])
        assert got == int(case["bf16"], 16), case["why"]


def test_bf16_rounding_is_nearest_even_brute_force():
    v = synth.rand_f32((1, 1, 9), (20000,), std=3.0).astype(np.float64)
    bits = oracle.round_to_cache(v, "bf16")
    f32 = v.astype(np.float32).astype(np.float64)
    got = cache_values(bits, "bf16", np.float64)
    # neighbours: truncation of the fp32 value and the next bf16 away from zero
    trunc = (f32.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    lo = cache_values(trunc, "bf16", np.float64)
    hi = cache_values((trunc + 1).astype(np.uint16), "bf16", np.float64)
    dlo, dhi = np.abs(f32 - lo), np.abs(f32 - hi)
    best = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(trunc % 2 == 0, lo, hi)))
    assert np.array_equal(got, best)


def test_q4_fixture_and_exactness():
    for row in _gold("q4_blocks.json")["rows"]:
        nib = np.array([[int(b, 16) for b in row["bytes"]]], dtype=np.uint8)
        sc = np.array([[int(row["scale_f16"], 16)]], dtype=np.uint16).view(np.float16)
        assert float(sc[0, 0]) == row["scale_value"]
        w = oracle.q4_dequant(nib, sc, np.float64)[0]
        assert w.shape == (32,)
        np.testing.assert_array_equal(w[:8], row["values_first8"])
        if "value_31" in row:
            assert w[31] == row["value_31"]
    st = synth.rand_matrix((1, 1, 10), 64, 256, "q4")
    w64 = oracle.dequant(st, np.float64)
    w32 = oracle.dequant(st, np.float32)
    assert np.array_equal(w64, w32.astype(np.float64))          # exact in fp32
    codes = w64.reshape(64, 8, 32) / st.scales.astype(np.float64)[:, :, None]
    assert np.array_equal(codes, np.round(codes)) and codes.min() >= -8 and codes.max() <= 7


# ------------------------------------------------------------------ attention

def test_attention_length_one_returns_v():
    q = synth.rand_f32((1, 2, 1), (8, 64)).astype(np.float64)
    K = synth.rand_f32((1, 2, 2), (2, 1, 64)).astype(np.float64)
    V = synth.rand_f32((1, 2, 3), (2, 1, 64)).astype(np.float64)
    a = oracle.attend(q, K, V, 4)
    for h in range(8):
        assert np.array_equal(a[h], V[h // 4, 0])


def test_attention_zero_keys_give_mean_and_dominant_key_selects():
    q = synth.rand_f32((1, 2, 4), (4, 16)).astype(np.float64)
    V = synth.rand_f32((1, 2, 5), (1, 9, 16)).astype(np.float64)
    a = oracle.attend(q, np.zeros((1, 9, 16)), V, 4)
    np.testing.assert_allclose(a, np.broadcast_to(V[0].mean(0), (4, 16)), rtol=1e-14, atol=1e-15)
    K = np.zeros((1, 9, 16))
    K[0, 6] = 1e3 * q[0]            # position 6 dominates head 0 only
    a = oracle.attend(q, K, V, 4)
    np.testing.assert_allclose(a[0], V[0, 6], rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_gqa():
    n_q, n_kv, T, d = 8, 2, 37, 64
    q = synth.rand_f32((1, 2, 6), (n_q, d)).astype(np.float64)
    K = synth.rand_f32((1, 2, 7), (n_kv, T, d)).astype(np.float64)
    V = synth.rand_f32((1, 2, 8), (n_kv, T, d)).astype(np.float64)
    tq = torch.from_numpy(q)[:, None, :]                        # [n_q, 1, d]
    tk = torch.from_numpy(K).repeat_interleave(n_q // n_kv, 0)  # [n_q, T, d]
    tv = torch.from_numpy(V).repeat_interleave(n_q // n_kv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0]
    np.testing.assert_allclose(oracle.attend(q, K, V, n_q // n_kv), ref.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ SwiGLU

def test_silu_fixture_and_swiglu_zero():
    for case in _gold("silu.json")["cases"]:
        got = float(oracle.silu(np.float64(case["z"])))
        assert abs(got - case["silu"]) <= 1e-15 * max(1.0, abs(case["silu"])), case["why"]
    u = synth.rand_f32((1, 3, 1), (100,)).astype(np.float64)
    assert np.all(oracle.swiglu(np.zeros(100), u) == 0.0)
    assert np.all(oracle.swiglu(u, np.zeros(100)) == 0.0)


def test_silu_matches_torch():
    z = synth.rand_f32((1, 3, 2), (1000,), std=8.0).astype(np.float64)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(),
                               rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ whole layer

def test_i8_cache_row_fixture():
    """Hand-computed int8 cache rows: a row whose largest magnitude is 127
    has scale 1 and inverse 1, so its codes are the values rounded to the
    nearest integer, ties to even; largest magnitude 254: scale 2, inverse
    0.5, both exact; a row of zeros: scale 0, codes 0."""
    codes, scale = oracle.quantize_i8(np.array([[127.0, -63.5, 0.5, 1.5, -2.5, 0.0, 2.49, -126.6]]))
    assert scale[0] == np.float32(1.0)
    assert codes.tolist() == [[127, -64, 0, 2, -2, 0, 2, -127]]
    codes, scale = oracle.quantize_i8(np.array([[-254.0, 3.0, 5.0, 1.0]]))
    assert scale[0] == np.float32(2.0)
    assert codes.tolist() == [[-127, 2, 2, 0]]      # 1.5 -> 2, 2.5 -> 2, 0.5 -> 0
    codes, scale = oracle.quantize_i8(np.zeros((3, 8)))
    assert (codes == 0).all() and (scale == 0).all()
    got = cache_values(np.array([[3, -127]], np.int8), "i8", np.float64, np.array([0.5], np.float32))
    assert got.tolist() == [[1.5, -63.5]]


def test_i8_cache_rows_round_to_nearest_step():
    """On 4000 random rows of 128 (magnitudes 0.01 to 100): the scale is the
    row maximum / 127 in binary32; the largest element becomes +-127; away
    from a half (1e-4, the binary32 product's error), every code is the
    nearest integer to x * 127 / m computed exactly; the value code * scale
    is within half a step of x; negating a row negates its codes, and
    scaling it by 8 scales only its scale."""
    rng = np.random.default_rng(7)
    v = rng.standard_normal((4000, 128)) * rng.uniform(0.01, 100, (4000, 1))
    codes, scale = oracle.quantize_i8(v)
    x = v.astype(np.float32).astype(np.float64)
    m = np.abs(x).max(1)
    assert np.array_equal(scale, (m / 127).astype(np.float32))
    rows = np.arange(len(v))
    i = np.abs(x).argmax(1)
    assert np.array_equal(codes[rows, i], (127 * np.sign(x[rows, i])).astype(np.int8))
    exact = x * 127.0 / m[:, None]
    far = np.abs(exact - np.floor(exact) - 0.5) > 1e-4
    assert far.mean() > 0.99
    assert np.array_equal(codes[far], np.rint(exact[far]).astype(np.int8))
    err = np.abs(codes * scale[:, None].astype(np.float64) - x)
    assert (err <= 0.5 * scale[:, None].astype(np.float64) * (1 + 1e-5)).all()
    c2, s2 = oracle.quantize_i8(-v)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)
    c3, s3 = oracle.quantize_i8(v * 8.0)
    assert np.array_equal(c3, codes) and np.array_equal(s3, scale * np.float32(8))


def _integer_layer_cfg():
    return synth.tiny(hidden=8, n_q_heads=2, n_kv_heads=1, head_dim=4, ffn=16,
                      rms_eps=0.0, ctx=0, steps=1)


def test_integer_exact_append():
    """x in {+-1}, eps 0, g 1, integer weights, position 0: u = x exactly,
    RoPE is the identity, so the cache slot holds the integer products W_k x,
    W_v x computed here in int64."""
    cfg = _integer_layer_cfg()
    rng = np.random.default_rng(123)
    wqkv = rng.integers(-4, 5, size=(cfg.n_qkv, cfg.hidden)).astype(np.float32)
    layer = {k: synth.Stored("f32", v) for k, v in {
        "attn_norm": np.ones(8, np.float32), "ffn_norm": np.ones(8, np.float32),
        "wqkv": wqkv, "wo": np.zeros((8, 8), np.float32),
        "wgate": np.zeros((16, 8), np.float32), "wup": np.zeros((16, 8), np.float32),
        "wdown": np.zeros((8, 16), np.float32)}.items()}
    o = oracle.Oracle(cfg, [layer])
    x = rng.choice([-1.0, 1.0], size=8)
    q = o.qkv_rope_append(0, x, 0)
    y = wqkv.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(q.reshape(-1), y[:8].astype(np.float64))
    assert np.array_equal(o.K[0][0, 0], y[8:12].astype(np.float32))
    assert np.array_equal(o.V[0][0, 0], y[12:16].astype(np.float32))
    # zero output projections leave the residual stream unchanged
    assert np.array_equal(o.layer(0, x, 0), x)


def _dense_causal_forward(cfg, layers, X):
    """All T tokens at once with torch CPU ops in float64: rms_norm,
    rotate_half RoPE, scaled_dot_product_attention(is_causal) with GQA by
    repeat_interleave, silu. K and V are rounded to the cache type with
    torch's own conversions before attention."""
    T, H = X.shape
    d, nq, nkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    pos = torch.arange(T, dtype=torch.float64)[:, None]
    inv = 1.0 / (cfg.rope_theta ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.cat([pos * inv, pos * inv], dim=-1)           # [T, d]
    cos, sin = torch.cos(ang)[None], torch.sin(ang)[None]

    def rot(t):                                                # t [heads, T, d]
        return t * cos + torch.cat([-t[..., d // 2:], t[..., : d // 2]], -1) * sin

    def to_cache(t):
        t = t.to(torch.float32)
        if cfg.kvtype == "i8":
            # per row (kv head, position): binary32 scale and inverse, codes
            # rounded half to even by torch.round, clamped
            m = t.abs().amax(-1, keepdim=True)
            inv = torch.where(m == 0, torch.zeros_like(m), torch.tensor(127.0, dtype=torch.float32) / m)
            code = torch.round(t * inv).clamp(-127, 127)
            scale = torch.where(m == 0, torch.zeros_like(m), m / torch.tensor(127.0, dtype=torch.float32))
            return code.to(torch.float64) * scale.to(torch.float64)
        if cfg.kvtype == "bf16":
            t = t.to(torch.bfloat16)
        return t.to(torch.float64)

    x = torch.from_numpy(X)
    for lw in layers:
        W = {k: torch.from_numpy(oracle.dequant(v)) for k, v in lw.items()}
        u = torch.nn.functional.rms_norm(x, (H,), weight=W["attn_norm"], eps=cfg.rms_eps)
        y = u @ W["wqkv"].T
        q = y[:, : nq * d].reshape(T, nq, d).transpose(0, 1)
        k = y[:, nq * d: (nq + nkv) * d].reshape(T, nkv, d).transpose(0, 1)
        v = y[:, (nq + nkv) * d:].reshape(T, nkv, d).transpose(0, 1)
        q, k = rot(q), to_cache(rot(k))
        v = to_cache(v)
        g = nq // nkv
        a = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(g, 0), v.repeat_interleave(g, 0), is_causal=True)
        x = x + a.transpose(0, 1).reshape(T, nq * d) @ W["wo"].T
        u2 = torch.nn.functional.rms_norm(x, (H,), weight=W["ffn_norm"], eps=cfg.rms_eps)
        h = torch.nn.functional.silu(u2 @ W["wgate"].T) * (u2 @ W["wup"].T)
        x = x + h @ W["wdown"].T
    return x.numpy()


@pytest.mark.parametrize("kind,nq,nkv,kv", [("f32", 4, 4, "f32"), ("f32", 4, 2, "f32"), ("bf16", 8, 2, "bf16"),
                                            ("q4", 4, 1, "bf16"), ("bf16", 8, 2, "i8"), ("q4", 4, 2, "i8")])
def test_decode_equals_dense_causal_forward(kind, nq, nkv, kv):
    cfg = synth.tiny(n_layers=2, hidden=64, n_q_heads=nq, n_kv_heads=nkv, head_dim=16, ffn=96,
                     wtype=kind, ntype="f32" if kind == "f32" else "bf16", kvtype=kv,
                     rope_theta=10000.0, ctx=0, steps=9, seed=21)
    o = oracle.Oracle.from_config(cfg, with_globals=False)
    T = cfg.steps
    X = synth.rand_f32((21, 7, 7), (T, cfg.hidden)).astype(np.float64)
    out = np.stack([_run_layers(o, X[t], t) for t in range(T)])
    ref = _dense_causal_forward(cfg, o.layers, X)
    assert _rel(out, ref) < 1e-12


@pytest.mark.parametrize("kind,kv", [("bf16", "bf16"), ("q4", "i8")])
def test_greedy_sequence_equals_dense_forward_greedy(kind, kv):
    """The greedy token sequence as a whole: the oracle decoding token by
    token (embedding, layers, final norm, head, argmax fed back) against a
    loop that re-runs the dense causal forward over the whole prefix each
    step and takes torch's final rms_norm, the head product and
    torch.argmax (first index of the maximum). Tokens equal, logits within
    1e-12."""
    cfg = synth.tiny(n_layers=2, hidden=64, n_q_heads=8, n_kv_heads=2, head_dim=16, ffn=96, wtype=kind,
                     ntype="bf16", kvtype=kv, htype="bf16", rope_theta=10000.0, ctx=0, steps=10, seed=23)
    o = oracle.Oracle.from_config(cfg)
    T = cfg.steps
    tok = int(synth.tokens(cfg)[0])
    got, got_logits = [tok], []
    for p in range(T - 1):
        x = o.step(got[-1], p)[-1]
        got_logits.append(o.logits(x))
        got.append(o.greedy(x)[0])
    E = torch.from_numpy(np.asarray(o.glob["embed"].data, dtype=np.float64))
    head = torch.from_numpy(oracle.dequant(o.glob["head"]))
    gfin = torch.from_numpy(oracle.dequant(o.glob["final_norm"]))
    ref = [tok]
    for p in range(T - 1):
        X = E[torch.tensor(ref)].numpy()
        h = torch.from_numpy(_dense_causal_forward(cfg, o.layers, X)[-1])
        z = head @ torch.nn.functional.rms_norm(h, (cfg.hidden,), weight=gfin, eps=cfg.rms_eps)
        assert _rel(got_logits[p], z.numpy()) < 1e-12, f"step {p}"
        ref.append(int(torch.argmax(z)))
    assert got == ref


def test_decode_equals_dense_causal_forward_at_depth():
    """The same over 40 layers (the 9B-shaped stacks' depth) at small widths,
    4-bit weights and a bf16 cache: depth is repetition, and the agreement
    holds through it."""
    cfg = synth.tiny(n_layers=40, hidden=64, n_q_heads=8, n_kv_heads=2, head_dim=16, ffn=96, wtype="q4",
                     ntype="bf16", kvtype="bf16", rope_theta=10000.0, ctx=0, steps=6, seed=25)
    o = oracle.Oracle.from_config(cfg, with_globals=False)
    X = synth.rand_f32((25, 7, 7), (cfg.steps, cfg.hidden)).astype(np.float64)
    out = np.stack([_run_layers(o, X[t], t) for t in range(cfg.steps)])
    assert _rel(out, _dense_causal_forward(cfg, o.layers, X)) < 1e-11


def _run_layers(o, x, p):
    for l in range(len(o.layers)):
        x = o.layer(l, x, p)
    return x


def test_fp32_oracle_agrees_with_fp64_on_the_single_layer_workload():
    cfg = synth.CONFIGS["C1"]
    toks = synth.tokens(cfg)
    runs = []
    for dt in (np.float64, np.float32):
        o = oracle.Oracle.from_config(cfg, dtype=dt)
        xs = [o.step(t, p)[-1] for p, t in enumerate(toks)]
        runs.append(np.stack(xs).astype(np.float64))
    assert _rel(runs[1], runs[0]) < 1e-6


def test_greedy_ties_take_lowest_index():
    cfg = synth.tiny(vocab=6)
    glob = {"final_norm": synth.Stored("f32", np.ones(8, np.float32)),
            "head": synth.Stored("f32", np.array([[0] * 8, [1] * 8, [1] * 8, [0] * 8, [1] * 8, [-1] * 8],
                                                 dtype=np.float32)),
            "embed": synth.Stored("f32", np.ones((6, 8), np.float32))}
    o = oracle.Oracle(cfg, [], glob)
    i, margin = o.greedy(np.ones(8))
    assert i == 1 and margin == 0.0
