"""The gated FFN with the down projection folded in (4-bit weights): one
launch per layer for x += Wd (silu(Wg u) * (Wu u)), u = RMSNorm(x) g
("RDNA4 Decode Kernel Fusion: Pipeline Barriers, Not Launches, Are the Win",
section "Fusion removes the barrier by removing the write": the four-kernel
layer).

* The entry point dec_gated_ffn_down against the oracle (x and h, 1e-5
  relative L2 as for the other kernels) and against the two-kernel form
  (dec_gated_ffn, then dec_gemv_residual), over shapes that exercise the
  plans: one to eight gate/up tiles per workgroup, four and eight gate/up
  steps and four to sixteen down steps per wave, ragged rows, scales staged
  in LDS and loaded per lane, 320 workgroups (two per compute unit); twice
  in a row on the same buffers (each launch leaves the grid counter zero).
* Layer steps with DEC_FUSE_DOWN: a small 4-bit stack over 24 steps, and the
  9B-shaped 4-bit stack's first two layers at 8192+ positions, against the
  oracle (1e-4 per layer output, as for the other layer tests); graph replay
  equal to eager launches bit for bit.
* The bounded wait's failure path, forced from the host (DEC_TEST_NO_WAIT):
  each 16-row slice of x is either the full result or untouched, the error
  word says so, the counter words are zero, and the next launch is exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import rel_l2
from transformer_layer_amd import lib as L
from transformer_layer_amd.engine import DecodeStack, _mat, _upload

pytestmark = pytest.mark.gpu
TOL = 1e-5

FD_CASES = [
    # H, F, norm weight type
    (1024, 384, "bf16"),     # 64 workgroups, one gate/up tile each, one down step a wave
    (2080, 352, "f32"),      # ragged rows (65 and 11 blocks), 130 workgroups, fp32 norm weights
    (4096, 12288, "bf16"),   # the 9B-shaped layer: 256 workgroups, 6 gate/up tiles, 12 down steps a wave
    (1024, 4096, "bf16"),    # 8 gate/up tiles per workgroup
    (5120, 2048, "bf16"),    # 8 gate/up steps a wave, 320 workgroups
    (4096, 16384, "bf16"),   # the longest down rows: 16 steps a wave, scales loaded per lane
]


def _setup(H, F, ntype, seed=31):
    cfg = synth.tiny(hidden=H, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=F, wtype="q4", ntype=ntype,
                     kvtype="bf16", ctx=0, steps=8, seed=seed)
    st = DecodeStack(cfg, n_layers=1, flags=L.DEC_FUSE_DOWN)
    lw = {"attn_norm": synth.rand_norm((seed, 0, H), H, ntype),
          "wqkv": synth.rand_matrix((seed, 1, 0), 3 * 4 * 64, H, "q4"),
          "wo": synth.rand_matrix((seed, 2, 0), H, 4 * 64, "q4"),
          "ffn_norm": synth.rand_norm((seed, 3, H), H, ntype),
          "wgate": synth.rand_matrix((seed, 4, F), F, H, "q4"),
          "wup": synth.rand_matrix((seed, 5, F), F, H, "q4"),
          "wdown": synth.rand_matrix((seed, 6, H), H, F, "q4", std=0.02)}
    st.set_layer(0, lw)
    return cfg, st, lw


def _oracle(cfg, lw, x):
    u = oracle.rmsnorm(x.astype(np.float64), oracle.dequant(lw["ffn_norm"]), cfg.rms_eps)
    h = oracle.swiglu(oracle.gemv(oracle.dequant(lw["wgate"]), u), oracle.gemv(oracle.dequant(lw["wup"]), u))
    return h, x.astype(np.float64) + oracle.gemv(oracle.dequant(lw["wdown"]), h)


@pytest.mark.parametrize("H,F,ntype", FD_CASES)
def test_gated_ffn_down_matches_oracle_and_two_kernels(gpu, H, F, ntype):
    cfg, st, lw = _setup(H, F, ntype)
    for call in range(2):
        x0 = synth.rand_f32((31, 7, call), (H,))
        st.x.copy_(torch.from_numpy(x0))
        st.h.fill_(float("nan"))
        L.dec_gated_ffn_down(st.desc, st.wstruct[0], st.state[0])
        torch.cuda.synchronize()
        got_x, got_h = st.x.cpu().numpy(), st.h.cpu().numpy()
        h_ref, x_ref = _oracle(cfg, lw, x0)
        assert rel_l2(got_h, h_ref) <= TOL, f"call {call}: h"
        assert rel_l2(got_x, x_ref) <= TOL, f"call {call}: x"
        assert rel_l2(got_x.astype(np.float64) - x0, x_ref - x0) <= 4 * TOL, f"call {call}: x - x0"
        assert st.check_err() == 0
        assert int(st.counters[2:4].abs().sum().item()) == 0, "grid counter words not cleared"
        # the two-kernel form on the same input
        st.x.copy_(torch.from_numpy(x0))
        d = st.w[0]
        L.dec_gated_ffn(st.desc, d["ffn_norm"][0].data_ptr(), _mat(d["wgate"]), _mat(d["wup"]),
                        st.x.data_ptr(), st.h.data_ptr())
        L.dec_gemv_residual(st.desc, _mat(d["wdown"]), H, F, st.h.data_ptr(), st.x.data_ptr())
        torch.cuda.synchronize()
        two = st.x.cpu().numpy()
        assert rel_l2(got_x.astype(np.float64) - x0, two.astype(np.float64) - x0) <= 1e-6, f"call {call}"


def _q4_stack_cfg(**kw):
    base = dict(n_layers=2, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn=384, wtype="q4",
                ntype="bf16", kvtype="bf16", htype="bf16", ctx=0, steps=24, seed=31)
    base.update(kw)
    return synth.tiny(**base)


def _decode(cfg, flags, steps, graph=False):
    st = DecodeStack(cfg, flags=flags)
    for l in range(cfg.n_layers):
        st.set_layer(l, synth.layer_weights(cfg, l))
    st.set_embedding(synth.embedding(cfg))
    toks = synth.tokens(cfg)
    rec = torch.zeros(cfg.n_layers + 1, cfg.hidden, dtype=torch.float32, device="cuda")
    out = []
    if graph:
        st.set_token_list(toks)
        st.set_pos(0)
        st.set_token(int(toks[0]))
        g = st.capture(0, steps)
        st.set_pos(0)
        st.set_token(int(toks[0]))
        for _ in range(steps):
            g.replay()
            torch.cuda.synchronize()
            out.append(st.x.cpu().numpy().copy())
    else:
        for p in range(steps):
            st.set_pos(p)
            st.set_token(int(toks[p]))
            st.token_step(record=rec)
            out.append(rec.cpu().numpy().copy())
    assert st.check_err() == 0
    assert int(st.counters[2:4].abs().sum().item()) == 0
    return np.stack(out), st


def test_layer_steps_with_down_folded_into_ffn_match_oracle(gpu):
    cfg = _q4_stack_cfg()
    got, _ = _decode(cfg, L.DEC_FUSE_DOWN, cfg.steps)
    ora = oracle.Oracle.from_config(cfg, with_globals=False)
    ora.glob = {"embed": synth.embedding(cfg)}
    toks = synth.tokens(cfg)
    worst = 0.0
    for p in range(cfg.steps):
        ref = ora.step(int(toks[p]), p)
        for l in range(1, cfg.n_layers + 1):
            worst = max(worst, rel_l2(got[p, l], ref[l]))
    print(f"four kernels per layer, 4-bit: worst layer relative L2 {worst:.2e}")
    assert worst <= 1e-4
    five, _ = _decode(cfg, 0, cfg.steps)
    assert max(rel_l2(got[p, l], five[p, l]) for p in range(cfg.steps) for l in range(1, 3)) <= 1e-5


def test_graph_replay_with_down_folded_equals_eager(gpu):
    cfg = _q4_stack_cfg(steps=12)
    eager, _ = _decode(cfg, L.DEC_FUSE_DOWN, cfg.steps)
    replayed, _ = _decode(cfg, L.DEC_FUSE_DOWN, cfg.steps, graph=True)
    assert np.array_equal(eager[:, -1].view(np.uint32), replayed.view(np.uint32))


def test_9b_shaped_4bit_layers_with_down_folded_at_full_shape(gpu):
    cfg = synth.CONFIGS["C5"]
    nl, nsteps = 2, 3
    ora = oracle.Oracle.from_config(cfg, n_layers=nl, with_globals=False)
    st = DecodeStack(cfg, n_layers=nl, flags=L.DEC_FUSE_DOWN)
    for l in range(nl):
        st.set_layer(l, ora.layers[l])
        st.set_prefill(l, *synth.prefill(cfg, l))
    embed = synth.embedding(cfg)
    st.set_embedding(embed)
    ora.glob = {"embed": embed}
    toks = synth.tokens(cfg)
    rec = torch.zeros(nl + 1, cfg.hidden, dtype=torch.float32, device="cuda")
    worst = 0.0
    for i in range(nsteps):
        p = cfg.ctx + i
        st.set_pos(p)
        st.set_token(int(toks[i]))
        st.token_step(record=rec)
        got = rec.cpu().numpy()
        ref = ora.step(int(toks[i]), p)
        for l in range(1, nl + 1):
            worst = max(worst, rel_l2(got[l], ref[l]))
    print(f"9B-shaped 4-bit, four kernels per layer: worst layer relative L2 {worst:.2e}")
    assert st.check_err() == 0
    assert worst <= 1e-4


def test_grid_wait_give_up_sets_sync_error_and_recovers(gpu):
    """Forced from the host: with DEC_TEST_NO_WAIT a workgroup that finds the
    others still missing gives up at once. Each 16-row slice of x is then
    either the full result or untouched, the error word has DEC_ERR_SYNC
    when any slice is untouched, the counter words are zero, and the next
    normal launch on the same buffers is exact."""
    H, F = 4096, 12288
    cfg, st, lw = _setup(H, F, "bf16", seed=37)
    x0 = synth.rand_f32((37, 7, 0), (H,))
    h_ref, x_ref = _oracle(cfg, lw, x0)
    st.desc.flags = L.DEC_FUSE_DOWN | L.DEC_TEST_NO_WAIT
    st.x.copy_(torch.from_numpy(x0))
    st.err.zero_()
    L.dec_gated_ffn_down(st.desc, st.wstruct[0], st.state[0])
    torch.cuda.synchronize()
    got = st.x.cpu().numpy()
    untouched = 0
    for t in range(H // 16):
        sl = slice(16 * t, 16 * t + 16)
        if np.array_equal(got[sl], x0[sl]):
            untouched += 1
        else:
            assert rel_l2(got[sl], x_ref[sl]) <= 1e-4, f"slice {t}"
    print(f"{untouched} of {H // 16} slices gave up")
    assert (st.check_err() == L.DEC_ERR_SYNC) == (untouched > 0)
    assert int(st.counters[2:4].abs().sum().item()) == 0
    st.desc.flags = L.DEC_FUSE_DOWN
    st.err.zero_()
    st.x.copy_(torch.from_numpy(x0))
    L.dec_gated_ffn_down(st.desc, st.wstruct[0], st.state[0])
    torch.cuda.synchronize()
    assert st.check_err() == 0
    assert rel_l2(st.x.cpu().numpy(), x_ref) <= TOL
    assert int(st.counters[2:4].abs().sum().item()) == 0
