"""The int8 KV cache on the GPU, layer by layer against the oracle.

The cache holds int8 codes and one float scale per row ("Vulkan Command
Buffer Reuse vs CUDA Graphs: RDNA4 Decode Overhead", section "What I am
building next": a leaner KV cache as a bytes-per-token lever; the scheme is
the oracle's quantize_i8). Each decoded row is checked as a quantization of
the oracle's exact k or v (codes may differ from the oracle's only where the
float32 row and the float64 one straddle a rounding point), then the
oracle's cache row is set to the GPU's, so that every layer output compares
float32 against float64 arithmetic on the same cache (1e-4 relative L2, as
for the other fused-layer tests).

Cases: bf16 weights (the attention combine inside the output projection)
and 4-bit weights (the attention's own combine), fused and per-op (the
per-op RoPE kernel stages the rows instead of the QKV epilogue), decoding
from an empty cache; and a 9B-shaped 4-bit stack at 8192 cached positions,
two layers, one token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import rel_l2
from transformer_layer_amd import lib as L
from transformer_layer_amd.engine import DecodeStack

pytestmark = pytest.mark.gpu
TOL = 1e-4


def check_i8_slot(codes, scale, exact, rel_tol=1e-5):
    """A GPU-written int8 row against the oracle's exact row: the scale is
    max|x| / 127 of a row within rel_tol of the exact one, every value
    code * scale lies within half a step (plus that tolerance) of the exact
    value, and at least 95% of the codes equal the oracle's own. Returns the
    number of codes that differ."""
    exact = np.asarray(exact, dtype=np.float64)
    codes = np.asarray(codes)
    scale = np.asarray(scale, dtype=np.float64)
    delta = rel_tol * np.abs(exact).max(axis=-1)
    assert np.all(np.abs(scale * 127 - np.abs(exact).max(axis=-1)) <= delta * 2 + 1e-30), "scale"
    err = np.abs(codes * scale[..., None] - exact)
    assert np.all(err <= 0.5 * scale[..., None] * (1 + 1e-6) + delta[..., None] * 2), "a code is not a nearest step"
    ora, _ = oracle.quantize_i8(exact)
    diff = codes != ora
    assert diff.mean() < 0.05, f"{diff.sum()} of {diff.size} codes differ"
    return int(diff.sum())


def _cfg(kind, **kw):
    if kind == "bf16":
        base = dict(n_layers=2, hidden=1040, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=344, wtype="bf16",
                    ntype="bf16", kvtype="i8", htype="bf16", ctx=0, steps=24, seed=41)
    else:
        base = dict(n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=4, head_dim=128, ffn=384, wtype="q4",
                    ntype="bf16", kvtype="i8", htype="bf16", ctx=0, steps=24, seed=43)
    base.update(kw)
    return synth.tiny(**base)


def _decode_and_compare(cfg, st, o, positions, toks):
    """Decode the given positions on the GPU (recording every layer's
    output) and on the oracle, layer by layer with the cache row set to the
    GPU's after it is checked. Returns (worst relative L2, codes that
    differed)."""
    nl = cfg.n_layers
    rec = torch.zeros(nl + 1, cfg.hidden, dtype=torch.float32, device="cuda")
    worst, flips = 0.0, 0
    for i, p in enumerate(positions):
        st.set_pos(p)
        st.set_token(int(toks[i]))
        st.token_step(record=rec)
        got = rec.cpu().numpy()
        x = o.embed(int(toks[i]))
        for l in range(nl):
            c = cfg
            u = oracle.rmsnorm(x, o.w(l, "attn_norm"), c.rms_eps)
            y = o.proj(l, "wqkv", u)
            d = c.head_dim
            q = oracle.rope(y[: c.q_dim].reshape(c.n_q_heads, d), p, c.rope_theta)
            k = oracle.rope(y[c.q_dim: c.q_dim + c.kv_dim].reshape(c.n_kv_heads, d), p, c.rope_theta)
            v = y[c.q_dim + c.kv_dim:].reshape(c.n_kv_heads, d)
            gk, gks = st.K[l, :, p].cpu().numpy(), st.Ks[l, :, p].cpu().numpy()
            gv, gvs = st.V[l, :, p].cpu().numpy(), st.Vs[l, :, p].cpu().numpy()
            flips += check_i8_slot(gk, gks, k) + check_i8_slot(gv, gvs, v)
            # the oracle's cache row becomes the GPU's (checked above)
            o.K[l][:, p], o.Ks[l][:, p], o.V[l][:, p], o.Vs[l][:, p] = gk, gks, gv, gvs
            o.Kd[l][:, p] = oracle.ref.cache_values(gk, "i8", np.float64, gks)
            o.Vd[l][:, p] = oracle.ref.cache_values(gv, "i8", np.float64, gvs)
            a = o.attention(l, q, p)
            x = x + o.proj(l, "wo", a)
            x = x + o.proj(l, "wdown", o.ffn(l, x))
            worst = max(worst, rel_l2(got[l + 1], x))
    return worst, flips


@pytest.mark.parametrize("kind", ["bf16", "q4"])
@pytest.mark.parametrize("path", ["fused", "per-op"])
def test_layer_steps_with_int8_cache_match_oracle(gpu, kind, path):
    cfg = _cfg(kind)
    st = DecodeStack(cfg, flags=L.DEC_UNFUSED if path == "per-op" else 0)
    layers = [synth.layer_weights(cfg, l) for l in range(cfg.n_layers)]
    for l, lw in enumerate(layers):
        st.set_layer(l, lw)
    embed = synth.embedding(cfg)
    st.set_embedding(embed)
    o = oracle.Oracle(cfg, layers, glob={"embed": embed})
    toks = synth.tokens(cfg)
    worst, flips = _decode_and_compare(cfg, st, o, list(range(cfg.steps)), toks)
    print(f"int8 cache, {kind} weights, {path}: worst layer relative L2 {worst:.2e}, {flips} codes differed")
    assert st.check_err() == 0
    assert worst <= TOL


def test_int8_cache_fused_and_per_op_4bit_agree_bit_for_bit(gpu):
    """4-bit weights: the per-op kernels keep the fused kernels' arithmetic,
    so the staged rows, and with them every code, scale and layer output,
    are the same bits."""
    cfg = _cfg("q4", steps=12)
    out = []
    for flags in (0, L.DEC_UNFUSED):
        st = DecodeStack(cfg, flags=flags)
        for l in range(cfg.n_layers):
            st.set_layer(l, synth.layer_weights(cfg, l))
        st.set_embedding(synth.embedding(cfg))
        toks = synth.tokens(cfg)
        rec = torch.zeros(cfg.n_layers + 1, cfg.hidden, dtype=torch.float32, device="cuda")
        xs = []
        for p in range(cfg.steps):
            st.set_pos(p)
            st.set_token(int(toks[p]))
            st.token_step(record=rec)
            xs.append(rec.cpu().numpy().copy())
        assert st.check_err() == 0
        out.append((np.stack(xs), st.Kraw.cpu(), st.Vraw.cpu()))
    (xa, Ka, Va), (xb, Kb, Vb) = out
    assert np.array_equal(xa.view(np.uint32), xb.view(np.uint32))
    assert torch.equal(Ka, Kb) and torch.equal(Va, Vb)


def test_9b_shaped_bf16_stack_with_int8_cache_at_4096_positions(gpu):
    """Two layers of the 9B-shaped bf16 stack with an int8 cache prefilled
    over 4096 positions, three tokens (the streaming attention kernel, its
    partials combined in the output projection), layer by layer."""
    cfg = synth.CONFIGS["C4"].with_(kvtype="i8", n_layers=2)
    st = DecodeStack(cfg)
    layers = [synth.layer_weights(cfg, l) for l in range(cfg.n_layers)]
    embed = synth.embedding(cfg)
    o = oracle.Oracle(cfg, layers, glob={"embed": embed})
    for l, lw in enumerate(layers):
        st.set_layer(l, lw)
        K, V = synth.prefill(cfg, l)
        st.set_prefill(l, K, V)
        o.load_prefill(l, K, V)
    st.set_embedding(embed)
    st.attn.fill_(float("nan"))
    toks = synth.tokens(cfg)
    worst, flips = _decode_and_compare(cfg, st, o, [cfg.ctx, cfg.ctx + 1, cfg.ctx + 2], toks)
    print(f"9B-shaped bf16, int8 cache at {cfg.ctx}: worst layer relative L2 {worst:.2e}, {flips} codes differed")
    assert st.check_err() == 0
    assert worst <= TOL
    # the combine ran in the output projection: the attention output buffer was never written
    assert bool(torch.isnan(st.attn).all())


def test_9b_shaped_4bit_stack_with_int8_cache_at_8192_positions(gpu):
    """Two layers of the 9B-shaped 4-bit stack with an int8 cache prefilled
    over 8192 positions, one token at 8192, layer by layer."""
    cfg = synth.CONFIGS["C5"].with_(kvtype="i8", n_layers=2)
    st = DecodeStack(cfg)
    layers = [synth.layer_weights(cfg, l) for l in range(cfg.n_layers)]
    embed = synth.embedding(cfg)
    o = oracle.Oracle(cfg, layers, glob={"embed": embed})
    for l, lw in enumerate(layers):
        st.set_layer(l, lw)
        K, V = synth.prefill(cfg, l)
        st.set_prefill(l, K, V)
        o.load_prefill(l, K, V)
    st.set_embedding(embed)
    toks = synth.tokens(cfg)
    worst, flips = _decode_and_compare(cfg, st, o, [cfg.ctx], toks)
    print(f"9B-shaped 4-bit, int8 cache at {cfg.ctx}: worst layer relative L2 {worst:.2e}, {flips} codes differed")
    assert st.check_err() == 0
    assert worst <= TOL
