"""The KV-cache append, bit for bit against the oracle, on the GPU.

A case whose every intermediate is an exact integer: position 0 (RoPE's
angle is zero, so the rotation is the identity), x in {-1, +1}^H, RMSNorm
epsilon 0 and norm weights 1 (so the normalized input equals x: mean(x^2)
is exactly 1), and integer projection weights that every storage type holds
exactly (f32, bf16, and 4-bit codes with block scale 1.0). Each k and v is
then an integer dot product, exact in float32 on both sides, and what the
cache stores is its rounding to the cache type: the integer itself in an f32
cache, its round-to-nearest-even bf16 value in a bf16 cache. The weight rows
are built so the sums hit values that need that rounding, ties included
(257 and 259 lie halfway between two bf16 neighbours and round to 256 and
260). The slot's bits must equal the oracle's bit for bit, through the
fused QKV kernel, through dec_layer_step, and through the per-op path; and
every other slot keeps its sentinel.

The general case, on random weights at any position (DEC_DEBUG_EXPORT_KV:
the QKV step also writes its float32 k and v rows before they are rounded):
every appended cache value is the oracle's rounding of the exported row, bit
for bit (f32 and bf16 caches; int8 codes and scales from the oracle's
quantize_i8), and the exported rows match the oracle's float64 k and v.
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
SENT16, SENT32 = 0x7FC1, 0x7FC00001

H, NQ, NKV, D, F = 256, 4, 2, 64, 256
# sums that need bf16 rounding (ties first), then a spread of others
TARGETS = [257, 259, 261, 263, -257, -259, 513, 515, 517, 1025, 1027, 1029, 300, 301, 302, 303]


def _integer_rows(x, targets, amax, rng):
    """Rows w with w . x == target, |w_c| <= amax, built as w_c = x_c a_c
    with nonnegative integers a_c (or their negatives) summing to |target|."""
    rows = []
    for t in targets:
        a = np.zeros(H, dtype=np.int64)
        left = abs(int(t))
        assert left <= amax * H
        idx = rng.permutation(H)
        i = 0
        while left:
            step = min(amax - a[idx[i % H]], left, int(rng.integers(1, amax + 1)))
            a[idx[i % H]] += step
            left -= step
            i += 1
        rows.append(np.sign(t) * a * x.astype(np.int64))
    return np.stack(rows)


def _case(wtype, kvtype):
    rng = np.random.default_rng(7)
    x = rng.choice([-1, 1], size=H).astype(np.int64)
    amax = 7 if wtype == "q4" else 8
    nqkv = (NQ + 2 * NKV) * D
    W = rng.integers(-amax, amax + 1, size=(nqkv, H)).astype(np.int64)
    kv0 = NQ * D
    specials = _integer_rows(x, TARGETS, amax, rng)
    W[kv0: kv0 + len(TARGETS)] = specials                     # k of kv head 0
    W[kv0 + NKV * D: kv0 + NKV * D + len(TARGETS)] = specials[::-1]   # v of kv head 0
    big = _integer_rows(x, rng.integers(-1700, 1700, size=2 * NKV * D - 2 * len(TARGETS)), amax, rng)
    rest = [r for r in range(kv0, nqkv) if not (kv0 <= r < kv0 + len(TARGETS) or
                                                 kv0 + NKV * D <= r < kv0 + NKV * D + len(TARGETS))]
    W[rest] = big
    cfg = synth.tiny(hidden=H, n_q_heads=NQ, n_kv_heads=NKV, head_dim=D, ffn=F, wtype=wtype, ntype="f32",
                     kvtype=kvtype, rms_eps=0.0, ctx=0, steps=4, seed=9)
    return cfg, x, W


def _stored(wtype, W):
    if wtype == "f32":
        return synth.Stored("f32", W.astype(np.float32))
    if wtype == "bf16":
        return synth.Stored("bf16", (W.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    codes = W.astype(np.int8).view(np.uint8) & 0x0F            # two's-complement nibbles
    nib = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = np.ones((W.shape[0], W.shape[1] // 32), dtype=np.float16)
    return synth.Stored("q4", nib, scales)


def _layer(cfg, wtype, W):
    zeros = lambda r, c: _stored(wtype, np.zeros((r, c), dtype=np.int64))  # noqa: E731
    return {"attn_norm": synth.Stored("f32", np.ones(H, np.float32)), "wqkv": _stored(wtype, W),
            "wo": zeros(H, NQ * D), "ffn_norm": synth.Stored("f32", np.ones(H, np.float32)),
            "wgate": zeros(F, H), "wup": zeros(F, H), "wdown": zeros(H, F)}


@pytest.mark.parametrize("route", ["qkv_kernel", "layer_step", "per_op"])
@pytest.mark.parametrize("kvtype", ["f32", "bf16"])
@pytest.mark.parametrize("wtype", ["f32", "bf16", "q4"])
def test_integer_exact_append_is_bitwise(gpu, wtype, kvtype, route):
    cfg, x, W = _case(wtype, kvtype)
    lw = _layer(cfg, wtype, W)
    # the oracle's slot, and the same integers computed here in int64
    o = oracle.Oracle(cfg, [lw])
    o.qkv_rope_append(0, x.astype(np.float64), 0)
    y = W @ x
    kv0 = NQ * D
    k_int, v_int = y[kv0: kv0 + NKV * D].reshape(NKV, D), y[kv0 + NKV * D:].reshape(NKV, D)
    assert np.array_equal(o.K[0][:, 0], oracle.round_to_cache(k_int.astype(np.float64), kvtype))
    assert np.array_equal(o.V[0][:, 0], oracle.round_to_cache(v_int.astype(np.float64), kvtype))
    if kvtype == "bf16":
        assert o.K[0][0, 0, 0] == 0x4380 and o.K[0][0, 0, 1] == 0x4382   # 257 -> 256, 259 -> 260

    flags = L.DEC_UNFUSED if route == "per_op" else 0
    st = DecodeStack(cfg, n_layers=1, flags=flags)
    st.set_layer(0, lw)
    sent = SENT16 if kvtype == "bf16" else SENT32
    (st.K.view(torch.int16) if kvtype == "bf16" else st.K.view(torch.int32)).fill_(sent)
    (st.V.view(torch.int16) if kvtype == "bf16" else st.V.view(torch.int32)).fill_(sent)
    st.x.copy_(torch.from_numpy(x.astype(np.float32)))
    st.set_pos(0)
    if route == "qkv_kernel":
        L.dec_rmsnorm_gemv_qkv_rope(st.desc, st.wstruct[0], st.state[0])
    else:
        st.layer(0)
    torch.cuda.synchronize()
    assert st.check_err() == 0
    view = np.uint16 if kvtype == "bf16" else np.uint32
    K = st.K[0].cpu().numpy().view(view)
    V = st.V[0].cpu().numpy().view(view)
    ko = o.K[0][:, 0].view(view) if kvtype == "bf16" else o.K[0][:, 0].astype(np.float32).view(view)
    vo = o.V[0][:, 0].view(view) if kvtype == "bf16" else o.V[0][:, 0].astype(np.float32).view(view)
    assert np.array_equal(K[:, 0], ko), "k slot bits differ from the oracle's"
    assert np.array_equal(V[:, 0], vo), "v slot bits differ from the oracle's"
    assert np.all(K[:, 1:] == np.array(sent).astype(view)) and np.all(V[:, 1:] == np.array(sent).astype(view))
    # q is exact too (float32 integers)
    if route == "qkv_kernel":
        assert np.array_equal(st.q.cpu().numpy(), y[:kv0].astype(np.float32))


EXPORT_CASES = {
    # the 9B-shaped layer's QKV step (bf16 weights), and small ragged shapes
    "9b_bf16": lambda kv: synth.CONFIGS["C4"].with_(kvtype=kv, n_layers=1, ctx=0),
    "ragged_bf16": lambda kv: synth.tiny(n_layers=1, hidden=1040, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=344,
                                         wtype="bf16", ntype="bf16", kvtype=kv, htype="bf16", ctx=0, steps=8,
                                         seed=47),
    "ragged_q4": lambda kv: synth.tiny(n_layers=1, hidden=1024, n_q_heads=8, n_kv_heads=4, head_dim=128, ffn=384,
                                       wtype="q4", ntype="f32", kvtype=kv, htype="bf16", ctx=0, steps=8, seed=53),
}


@pytest.mark.parametrize("path", ["fused", "per-op"])
@pytest.mark.parametrize("kvtype", ["f32", "bf16", "i8"])
@pytest.mark.parametrize("case", list(EXPORT_CASES))
def test_every_appended_value_is_its_exported_row_rounded(gpu, case, kvtype, path):
    cfg = EXPORT_CASES[case](kvtype)
    flags = L.DEC_DEBUG_EXPORT_KV | (L.DEC_UNFUSED if path == "per-op" else 0)
    st = DecodeStack(cfg, n_layers=1, flags=flags)
    lw = synth.layer_weights(cfg, 0)
    st.set_layer(0, lw)
    embed = synth.embedding(cfg)
    st.set_embedding(embed)
    o = oracle.Oracle(cfg, [lw], glob={"embed": embed})
    off, nkv, d = L.dec_scratch_kv_offset(st.desc), cfg.n_kv_heads, cfg.head_dim
    toks = synth.tokens(cfg)
    for i, p in enumerate(sorted({0, 1, 2, cfg.max_ctx // 2 + 1, cfg.max_ctx - 1})):
        st.scratch.fill_(float("nan"))
        st.set_pos(p)
        st.set_token(int(toks[i]))
        st.token_step()
        torch.cuda.synchronize()
        assert st.check_err() == 0
        ex = st.scratch[off: off + 2 * nkv * d].cpu().numpy().reshape(2, nkv, d)
        assert not np.isnan(ex).any(), "export incomplete"
        # the exported rows against the oracle's float64 k and v
        u = oracle.rmsnorm(o.embed(int(toks[i])), o.w(0, "attn_norm"), cfg.rms_eps)
        y = o.proj(0, "wqkv", u)
        k = oracle.rope(y[cfg.q_dim: cfg.q_dim + cfg.kv_dim].reshape(nkv, d), p, cfg.rope_theta)
        v = y[cfg.q_dim + cfg.kv_dim:].reshape(nkv, d)
        assert rel_l2(ex[0], k) <= 1e-5 and rel_l2(ex[1], v) <= 1e-5, f"position {p}"
        # every appended value is the rounding of its exported float32
        for src, cache, sc in ((ex[0], st.K, getattr(st, "Ks", None)), (ex[1], st.V, getattr(st, "Vs", None))):
            got = cache[0, :, p].cpu()
            if kvtype == "f32":
                assert np.array_equal(got.numpy().view(np.uint32), src.view(np.uint32)), f"position {p}"
            elif kvtype == "bf16":
                assert np.array_equal(got.view(torch.int16).numpy().view(np.uint16),
                                      oracle.round_to_cache(src, "bf16")), f"position {p}"
            else:
                codes, scales = oracle.quantize_i8(src)
                assert np.array_equal(got.numpy(), codes), f"position {p}: codes"
                assert np.array_equal(sc[0, :, p].cpu().numpy().view(np.uint32), scales.view(np.uint32)), \
                    f"position {p}: scales"
