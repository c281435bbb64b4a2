"""Fusion switches, determinism, the split attention entry points, and the
parity gates run against violations, on the GPU.

* Per-operation switches (DEC_NO_FUSE_QKV, DEC_NO_FUSE_FFN,
  DEC_NO_FUSE_ATTN_O) and DEC_DETERMINISTIC each compute the same layer:
  against the oracle, and for f32 and 4-bit weights bit for bit against the
  fused path ("backend-specific kernel fusion", section "A practical
  engineering example": global and per-operation controls).
* DEC_DETERMINISTIC: two runs of the same steps give the same bits.
* dec_attn_partials followed by dec_attn_o_residual, called directly, equal
  the oracle's x + Wo attention(q).
* Gates against violations ("Kernel fusion and block bridging", section
  "What it keeps"): with a test-only fault planted in the kernels (q and k
  left unrotated, k and v appended one slot late, the last attention split
  left out of the combine) every kernel still completes with a clean error
  word, and the same parity check that passes without the fault fails.
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


def _bf16_cfg(**kw):
    base = dict(n_layers=2, hidden=1040, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=344, wtype="bf16",
                ntype="bf16", kvtype="bf16", htype="bf16", ctx=0, steps=40, seed=29)
    base.update(kw)
    return synth.tiny(**base)


def _q4_cfg():
    return synth.tiny(n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=384, wtype="q4",
                      ntype="bf16", kvtype="bf16", htype="bf16", ctx=0, steps=24, seed=31)


def _run(cfg, flags=0, attn_chunk=0, steps=None):
    """Decode `steps` tokens from an empty cache; every layer's output of
    every step, the caches, and the error word."""
    st = DecodeStack(cfg, flags=flags, attn_chunk=attn_chunk)
    for l in range(cfg.n_layers):
        st.set_layer(l, synth.layer_weights(cfg, l))
    st.set_embedding(synth.embedding(cfg))
    toks = synth.tokens(cfg)
    n = cfg.steps if steps is None else steps
    rec = torch.zeros(cfg.n_layers + 1, cfg.hidden, dtype=torch.float32, device="cuda")
    out = []
    for p in range(n):
        st.set_pos(p)
        st.set_token(int(toks[p]))
        st.token_step(record=rec)
        out.append(rec.cpu().numpy().copy())
    torch.cuda.synchronize()
    return np.stack(out), st.K.cpu(), st.V.cpu(), st.check_err()


_ORACLE = {}


def _oracle_run(cfg, steps=None):
    key = (cfg, steps)
    if key not in _ORACLE:
        o = oracle.Oracle.from_config(cfg)
        toks = synth.tokens(cfg)
        n = cfg.steps if steps is None else steps
        _ORACLE[key] = np.stack([np.stack(o.step(int(toks[p]), p)) for p in range(n)])
    return _ORACLE[key]


def _worst(got, ref):
    return max(rel_l2(got[s, l], ref[s, l]) for s in range(got.shape[0]) for l in range(1, got.shape[1]))


@pytest.mark.parametrize("flag", ["DEC_NO_FUSE_QKV", "DEC_NO_FUSE_FFN", "DEC_NO_FUSE_ATTN_O", "DEC_DETERMINISTIC"])
@pytest.mark.parametrize("kind", ["f32", "q4", "bf16"])
def test_per_op_switch_computes_the_same_layer(gpu, flag, kind):
    cfg = {"f32": synth.CONFIGS["C1"].with_(real_prefill=False, ctx=0, steps=20), "q4": _q4_cfg(),
           "bf16": _bf16_cfg(steps=24)}[kind]
    fused, Kf, Vf, e0 = _run(cfg)
    split, Ks, Vs, e1 = _run(cfg, flags=getattr(L, flag))
    assert e0 == 0 and e1 == 0
    ref = _oracle_run(cfg)
    assert _worst(split, ref) <= (1e-5 if kind == "f32" else TOL)
    if kind != "bf16":
        # the per-op kernels keep the fused kernels' summation order
        assert np.array_equal(split.view(np.uint32), fused.view(np.uint32)), f"{flag}: differs from fused"
        assert torch.equal(Kf, Ks) and torch.equal(Vf, Vs)
    else:
        assert _worst(split, fused) <= 2e-5


@pytest.mark.parametrize("cfg_name", ["bf16", "bf16_64"])
def test_deterministic_flag_repeats_bit_for_bit(gpu, cfg_name):
    cfg = _bf16_cfg(steps=24) if cfg_name == "bf16" else _bf16_cfg(head_dim=64, hidden=1000, steps=24)
    a, Ka, Va, ea = _run(cfg, flags=L.DEC_DETERMINISTIC)
    b, Kb, Vb, eb = _run(cfg, flags=L.DEC_DETERMINISTIC)
    assert ea == 0 and eb == 0
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert torch.equal(Ka, Kb) and torch.equal(Va, Vb)
    assert _worst(a, _oracle_run(cfg)) <= TOL


@pytest.mark.parametrize("kernel", ["DEC_ATTN_BATCHED", "DEC_ATTN_STREAM", "DEC_ATTN_LOCAL"])
@pytest.mark.parametrize("combine", ["in the output projection", "in the attention kernel"])
def test_layer_step_with_each_attention_kernel(gpu, kernel, combine):
    """The bf16 layer step with each attention kernel forced, its partials
    combined in the output projection or by the attention's own combiners:
    every layer of every step against the oracle (cache from position 0, so
    the splits grow from one to three)."""
    cfg = _bf16_cfg(steps=24)
    flags = getattr(L, kernel) | (L.DEC_NO_FUSE_ATTN_O if combine == "in the attention kernel" else 0)
    got, _, _, err = _run(cfg, flags=flags, attn_chunk=10)
    assert err == 0
    assert _worst(got, _oracle_run(cfg)) <= TOL


def test_split_attention_entry_points_match_oracle(gpu):
    """dec_attn_partials then dec_attn_o_residual on a layer whose cache holds
    several splits of positions: x becomes x + Wo attention(q)."""
    cfg = _bf16_cfg(n_layers=1, ctx=300, steps=20)
    lw = synth.layer_weights(cfg, 0)
    Kp, Vp = synth.prefill(cfg, 0)
    st = DecodeStack(cfg, n_layers=1, attn_chunk=64)
    st.set_layer(0, lw)
    st.set_prefill(0, Kp, Vp)
    o = oracle.Oracle(cfg, [lw])
    o.load_prefill(0, Kp, Vp)
    x = synth.rand_f32((29, 3, 1), (cfg.hidden,))
    for p in (cfg.ctx, cfg.ctx + 1):      # five splits of at most 64 positions
        st.x.copy_(torch.from_numpy(x))
        st.set_pos(p)
        st.attn.fill_(float("nan"))
        L.dec_rmsnorm_gemv_qkv_rope(st.desc, st.wstruct[0], st.state[0])
        L.dec_attn_partials(st.desc, st.state[0])
        L.dec_attn_o_residual(st.desc, st.wstruct[0].wo, st.state[0])
        torch.cuda.synchronize()
        assert st.check_err() == 0
        assert bool(torch.isnan(st.attn).all()), "the attention output was written"
        xd = x.astype(np.float64)
        q = o.qkv_rope_append(0, xd, p)
        want = xd + o.proj(0, "wo", o.attention(0, q, p))
        assert rel_l2(st.x.cpu().numpy(), want) <= 1e-5


# ------------------------------------------------------------------ gates against violations

GATES = [
    # (fault flag, workload, attention chunk, steps)
    ("DEC_TEST_SKIP_ROPE", "f32", 0, 6),
    ("DEC_TEST_SKIP_ROPE", "q4", 0, 6),
    ("DEC_TEST_APPEND_NEXT", "f32", 0, 6),
    ("DEC_TEST_APPEND_NEXT", "bf16", 0, 6),
    ("DEC_TEST_DROP_SPLIT", "f32", 16, 24),    # splits of 16 positions: two from position 16 on
    ("DEC_TEST_DROP_SPLIT", "bf16", 16, 24),   # the combine inside the output projection
]


@pytest.mark.parametrize("fault,kind,chunk,steps", GATES)
def test_parity_gate_fails_on_a_planted_kernel_fault(gpu, fault, kind, chunk, steps):
    cfg = {"f32": synth.CONFIGS["C1"].with_(real_prefill=False, ctx=0, steps=24), "q4": _q4_cfg(),
           "bf16": _bf16_cfg(steps=24)}[kind]
    ref = _oracle_run(cfg, steps)
    good, _, _, e0 = _run(cfg, attn_chunk=chunk, steps=steps)
    bad, _, _, e1 = _run(cfg, flags=getattr(L, fault), attn_chunk=chunk, steps=steps)
    assert e0 == 0 and e1 == 0, "a planted fault must not set the error word"
    tol = 1e-5 if kind == "f32" else TOL
    assert _worst(good, ref) <= tol
    worst_bad = _worst(bad, ref)
    print(f"{fault} on {kind}: relative L2 {worst_bad:.3e} (clean {_worst(good, ref):.1e})")
    assert worst_bad > 10 * tol, f"the gate did not catch {fault}"
