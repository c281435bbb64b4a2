"""The benchmark's host-side logic on the CPU: the one-GPU contract, the
algorithmic byte counts behind `value` and `roofline.achieved`, and the rule
that a committed counter summary is used only for the kernel sources it was
taken from."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _by_hand(hidden, nq, nkv, d, ffn, layers, ctx, steps, wbytes, nbytes, kvbytes):
    """Bytes of one token written out from the shapes: every weight matrix,
    both norm weights, the cache read averaged over the decode window
    (ctx+1 .. ctx+steps positions) and one cache write per layer."""
    qkv = (nq + 2 * nkv) * d * hidden
    o = hidden * nq * d
    gate_up = 2 * ffn * hidden
    down = hidden * ffn
    weights = (qkv + o + gate_up + down) * wbytes + 2 * hidden * nbytes
    per_position = 2 * nkv * d * kvbytes               # one k row and one v row
    mean_len = sum(range(ctx + 1, ctx + steps + 1)) / steps
    return layers * (weights + per_position * mean_len + per_position)


@pytest.mark.parametrize("name,wbytes", [("C2", 2), ("C3", 2), ("C4", 2), ("C5", 0.5 + 2 / 32)])
def test_token_bytes_by_hand(name, wbytes):
    c = synth.CONFIGS[name]
    want = _by_hand(c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ffn, c.n_layers, c.ctx, c.steps,
                    wbytes, 2, 2)
    assert synth.token_bytes(c) == pytest.approx(want, rel=1e-12)


def test_nine_b_token_bytes_value():
    # 40 layers of 385,892,352 weight and norm bytes plus 4096 cache bytes per
    # position over a mean of 4224.5 positions, plus the write
    assert synth.token_bytes(synth.CONFIGS["C4"]) == 16_128_000_000


def test_ffn_bytes_per_launch_is_the_gate_and_up_weights_and_norm():
    c = synth.CONFIGS["C4"]
    assert synth.layer_weight_bytes(c)["ffn"] == 2 * 12288 * 4096 * 2 + 4096 * 2


def test_traffic_summary_is_used_only_for_its_sources(tmp_path, monkeypatch):
    cfg = synth.CONFIGS["C4"]
    path = tmp_path / f"gated_ffn_{cfg.name}_hbm_traffic.txt"
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.measured_traffic(cfg) is None                      # no summary
    path.write_text("# comment: ignored\nhbm_bytes_per_launch: 201771210\n"
                    f"kernel_source_sha256_16: {bench.ffn_source_hash()}\n")
    assert bench.measured_traffic(cfg) == 201771210
    path.write_text("hbm_bytes_per_launch: 201771210\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.measured_traffic(cfg) is None                      # sources changed since


@pytest.mark.parametrize("name,hbytes,nbytes", [("C1", 4, 4), ("C2", 2, 2), ("C4", 2, 2), ("C5", 2, 2)])
def test_head_bytes_by_hand(name, hbytes, nbytes):
    """The LM head step reads the [vocab, hidden] head (bf16 also for the
    4-bit workload) and the final norm weight."""
    c = synth.CONFIGS[name]
    assert synth.head_bytes(c) == c.vocab * c.hidden * hbytes + c.hidden * nbytes


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5"])
def test_timed_bytes_follow_the_positions_timed(name):
    """The bench's bytes per token average the KV read over the positions
    its timed run visits: the whole window equals token_bytes, 20 steps the
    first 20 positions, and a run longer than the window wraps to ctx."""
    c = synth.CONFIGS[name]
    assert bench.timed_token_bytes(c, c.steps) == pytest.approx(synth.token_bytes(c), rel=1e-12)
    assert bench.timed_token_bytes(c, 20) == pytest.approx(synth.token_bytes(c, 20), rel=1e-12)
    want20 = _by_hand(c.hidden, c.n_q_heads, c.n_kv_heads, c.head_dim, c.ffn, c.n_layers, c.ctx, 20,
                      synth.elem_bytes(c.wtype), 2, 2)
    assert bench.timed_token_bytes(c, 20) == pytest.approx(want20, rel=1e-12)
    # two windows and 3 more steps: the mean over ctx+1..ctx+steps twice, then ctx+1..ctx+3
    n = 2 * c.steps + 3
    lens = [c.ctx + (i % c.steps) + 1 for i in range(n)]
    per_pos = 2 * c.n_kv_heads * c.head_dim * 2
    want = synth.token_bytes(c) + c.n_layers * per_pos * (sum(lens) / n - (c.ctx + (c.steps + 1) / 2))
    assert bench.timed_token_bytes(c, n) == pytest.approx(want, rel=1e-12)
