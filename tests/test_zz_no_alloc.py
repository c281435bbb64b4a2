"""dec_layer_step_static, the layer step that needs no caller scratch,
against dec_layer_step on the same inputs (GPU).

Each case builds two identical one-layer stacks (weights, cache prefill,
hidden state, position) and runs the layer once through dec_layer_step,
with the stack's own partials, counters and per-op buffers, and once
through dec_layer_step_static, whose state passes NULL for those three. The
calls follow each other on one GPU, a large shape first and then smaller
ones, so the static array still holds the previous call's partials when the
next call starts. Results must agree as the paths' own determinism allows:
bit for bit wherever no float atomics are involved (f32 and 4-bit weights,
per-op kernels, DEC_DETERMINISTIC, and every cache slot), within 1e-5
relative L2 for x on the default bf16 path, whose output projection adds
its shares with float atomics. A captured graph of the static step then
replays three times, with eager work between the replays, each replay equal
to an eager dec_layer_step.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import rel_l2
from transformer_layer_amd import lib as L
from transformer_layer_amd.engine import DecodeStack

pytestmark = pytest.mark.gpu


def _pair(cfg, flags, pos):
    """Two identical one-layer stacks at position `pos` with the same x."""
    lw = synth.layer_weights(cfg, 0)
    pre = synth.prefill(cfg, 0) if cfg.ctx else None
    x = synth.rand_f32((cfg.seed, 77, pos), (cfg.hidden,))
    out = []
    for _ in range(2):
        st = DecodeStack(cfg, n_layers=1, flags=flags)
        st.set_layer(0, lw)
        if pre is not None:
            st.set_prefill(0, *pre)
        st.x.copy_(torch.from_numpy(x))
        st.set_pos(pos)
        out.append(st)
    return out


def _static_state(st):
    s = st.state[0]
    return L.dec_layer_state(x=s.x, q=s.q, attn=s.attn, h=s.h, part=None, counters=None, k_cache=s.k_cache,
                             v_cache=s.v_cache, pos=s.pos, rope=s.rope, err=s.err, scratch=None)


CASES = [
    # (workload, flags, position, x compared bit for bit)
    ("C5", 0, 8200, True),                    # 4-bit weights, in-kernel combine (88 splits): the largest partials
    ("C4", 0, 4100, False),                   # streaming attention, 32 splits, combine in the O projection
    ("C3", 0, 2060, False),                   # wave-local attention, 8 splits of 272 positions
    ("C1", 0, 17, True),                      # smaller: f32, two splits
    ("C4", L.DEC_DETERMINISTIC, 4099, True),
    ("C2", 0, 515, False),
    ("C1", L.DEC_UNFUSED, 19, True),          # the per-op intermediates in the static array
    ("C5", L.DEC_FUSE_DOWN, 8195, True),      # the FFN + down kernel's grid counter words in the static array
]


def test_static_step_matches_layer_step(gpu):
    for name, flags, pos, bitwise in CASES:
        cfg = synth.CONFIGS[name].with_(n_layers=1)
        if cfg.real_prefill:
            cfg = cfg.with_(real_prefill=False, ctx=0, steps=24)
        print(f"case {name} flags {flags:#x} pos {pos}", flush=True)
        a, b = _pair(cfg, flags, pos)
        a.layer(0)
        L.dec_layer_step_static(b.desc, b.wstruct[0], _static_state(b))
        torch.cuda.synchronize()
        assert a.check_err() == 0 and b.check_err() == 0
        xa, xb = a.x.cpu().numpy(), b.x.cpu().numpy()
        if bitwise:
            assert np.array_equal(xa.view(np.uint32), xb.view(np.uint32)), f"{name}: x differs"
        else:
            assert rel_l2(xb, xa) <= 1e-5, f"{name}: x differs by {rel_l2(xb, xa):.2e}"
        assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V), f"{name}: caches differ"
        del a, b
        torch.cuda.empty_cache()


def test_static_step_in_a_captured_graph(gpu):
    cfg = synth.CONFIGS["C1"].with_(real_prefill=False, ctx=0, steps=24)
    a, b = _pair(cfg, 0, 0)
    sb = _static_state(b)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        L.dec_layer_step_static(b.desc, b.wstruct[0], sb)
    for rep, pos in enumerate((3, 9, 16)):
        x = synth.rand_f32((5, 78, rep), (cfg.hidden,))
        for st in (a, b):
            st.x.copy_(torch.from_numpy(x))
            st.set_pos(pos)
        a.layer(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(a.x.cpu().numpy().view(np.uint32), b.x.cpu().numpy().view(np.uint32)), rep
        assert torch.equal(a.K, b.K) and torch.equal(a.V, b.V), rep
        b.x.mul_(2.0)   # eager work between the replays
    assert a.check_err() == 0 and b.check_err() == 0
