"""Per-kernel parity: each fused kernel of the layer, called through the C
ABI, against the CPU oracle's steps on the same seeded inputs.

Shapes span several 16-byte granule tiles per lane with ragged tails (row
lengths that are not a multiple of 64 granules), odd row counts, both
column-split modes (one wave per row and four waves per row), every weight
type, both cache types, head dims 64 and 128 and GQA groups 1..8.

Tolerance: every kernel computes in float32 (exact bf16 / 4-bit weights,
float32 inputs); a dot product of length n split over 64 lanes has a relative
rounding error of order 2^-24 * sqrt(n); 1e-5 relative L2 bounds it with
margin for n <= 16384. KV-cache bits are compared exactly, except where the
oracle's exact value lies within that error of a bf16 rounding tie.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_rounded_slot, rel_l2
from transformer_layer_amd import lib as L
from transformer_layer_amd.engine import DecodeStack

pytestmark = pytest.mark.gpu
TOL = 1e-5
SENT16 = 0x7FC1           # bf16 quiet-NaN pattern never produced by the kernels
SENT32 = 0x7FC00001


def _cfg(wtype, kvtype, H, nq, nkv, d, F=64, max_ctx=37, ntype=None):
    return synth.tiny(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=F, wtype=wtype,
                      ntype=ntype or ("f32" if wtype == "f32" else "bf16"), kvtype=kvtype,
                      ctx=0, steps=max_ctx, seed=5)


def _fill_sentinel(t):
    if t.dtype == torch.int16:
        t.fill_(SENT16)
    else:
        t.view(torch.int32).fill_(SENT32)


QKV_CASES = [
    # wtype, kvtype, H, n_q, n_kv, d
    ("f32", "f32", 256, 4, 4, 64),
    ("f32", "bf16", 1000, 2, 2, 64),      # ragged: 250 granules over 64 lanes
    ("bf16", "bf16", 2176, 4, 2, 128),    # ragged: 272 granules
    ("bf16", "bf16", 4096, 32, 8, 128),   # 9B-class layer shape
    ("bf16", "bf16", 8192, 8, 1, 64),     # four waves per row
    ("q4", "bf16", 2080, 8, 1, 64),       # 65 blocks per row
    ("q4", "bf16", 4096, 32, 8, 128),
]


@pytest.mark.parametrize("wtype,kvtype,H,nq,nkv,d", QKV_CASES)
def test_rmsnorm_gemv_qkv_rope(gpu, wtype, kvtype, H, nq, nkv, d):
    cfg = _cfg(wtype, kvtype, H, nq, nkv, d)
    p = 29
    lw = synth.layer_weights(cfg, 0)
    x = synth.rand_f32((5, 1, H), (H,))
    st = DecodeStack(cfg, n_layers=1)
    st.set_layer(0, lw)
    _fill_sentinel(st.K)
    _fill_sentinel(st.V)
    st.x.copy_(torch.from_numpy(x))
    st.set_pos(p)
    L.dec_rmsnorm_gemv_qkv_rope(st.desc, st.wstruct[0], st.state[0])
    torch.cuda.synchronize()
    assert st.check_err() == 0

    o = oracle.Oracle(cfg, [lw])
    q_ora = o.qkv_rope_append(0, x.astype(np.float64), p)
    # the oracle's exact (pre-rounding) k and v
    u = oracle.rmsnorm(x.astype(np.float64), o.w(0, "attn_norm"), cfg.rms_eps)
    y = oracle.gemv(o.w(0, "wqkv"), u)
    k_ex = oracle.rope(y[cfg.q_dim: cfg.q_dim + cfg.kv_dim].reshape(nkv, d), p, cfg.rope_theta)
    v_ex = y[cfg.q_dim + cfg.kv_dim:].reshape(nkv, d)

    assert rel_l2(st.q.cpu().numpy(), q_ora.reshape(-1)) <= TOL
    K = st.K[0].cpu().numpy()
    V = st.V[0].cpu().numpy()
    if kvtype == "bf16":
        kg, vg = K[:, p].view(np.uint16), V[:, p].view(np.uint16)
    else:
        kg, vg = K[:, p], V[:, p]
    check_rounded_slot(kg, o.K[0][:, p], k_ex, kvtype, TOL)
    check_rounded_slot(vg, o.V[0][:, p], v_ex, kvtype, TOL)
    # every other slot is untouched
    sent = SENT16 if kvtype == "bf16" else SENT32
    for C in (K, V):
        bits = C.view(np.int16 if kvtype == "bf16" else np.int32)
        mask = np.ones(bits.shape[1], dtype=bool)
        mask[p] = False
        assert np.all(bits[:, mask] == np.array(sent).astype(bits.dtype))


GEMV_CASES = [
    # wtype, rows, cols
    ("f32", 777, 1000),
    ("f32", 256, 1024),
    ("bf16", 513, 2176),
    ("bf16", 4096, 4096),
    ("bf16", 1001, 11008),   # four waves per row, ragged
    ("bf16", 4096, 12288),
    ("q4", 999, 2080),
    ("q4", 4096, 12288),     # four waves per row, 1.5 blocks per lane
]


@pytest.mark.parametrize("wtype,rows,cols", GEMV_CASES)
def test_gemv_residual(gpu, wtype, rows, cols):
    cfg = _cfg(wtype, "bf16", 256 if wtype != "q4" else 256, 4, 4, 64)
    st = DecodeStack(cfg, n_layers=1)
    W = synth.rand_matrix((6, rows, cols), rows, cols, wtype)
    inp = synth.rand_f32((6, 2, cols), (cols,))
    x0 = synth.rand_f32((6, 3, rows), (rows,))
    from transformer_layer_amd.engine import _upload, _mat
    dw = _upload(W, st.dev)
    din = torch.from_numpy(inp).cuda()
    dx = torch.from_numpy(x0).cuda()
    L.dec_gemv_residual(st.desc, _mat(dw), rows, cols, din.data_ptr(), dx.data_ptr())
    torch.cuda.synchronize()
    ref = x0.astype(np.float64) + oracle.gemv(oracle.dequant(W), inp.astype(np.float64))
    assert rel_l2(dx.cpu().numpy(), ref) <= TOL
    # the residual-free part alone, so the check is not dominated by x0
    delta = dx.cpu().numpy().astype(np.float64) - x0
    assert rel_l2(delta, ref - x0) <= 4 * TOL


FFN_CASES = [
    ("f32", 256, 1024, None),
    ("bf16", 2176, 1000, None),
    ("bf16", 4096, 12288, None),
    ("bf16", 8192, 640, None),
    ("q4", 4096, 12288, None),
    ("q4", 2080, 352, None),
    ("q4", 2080, 352, "f32"),     # 4-bit weights with fp32 norm weights
    ("q4", 16384, 96, None),      # the longest rows the interface allows
]


@pytest.mark.parametrize("wtype,H,F,ntype", FFN_CASES)
def test_gated_ffn(gpu, wtype, H, F, ntype):
    cfg = _cfg(wtype, "bf16", H, 4, 4, 64, F=F, ntype=ntype)
    st = DecodeStack(cfg, n_layers=1)
    g = synth.rand_norm((7, 1, H), H, cfg.ntype)
    Wg = synth.rand_matrix((7, 2, F), F, H, wtype)
    Wu = synth.rand_matrix((7, 3, F), F, H, wtype)
    x = synth.rand_f32((7, 4, H), (H,))
    from transformer_layer_amd.engine import _upload, _mat
    dg, dwg, dwu = _upload(g, st.dev), _upload(Wg, st.dev), _upload(Wu, st.dev)
    dx = torch.from_numpy(x).cuda()
    dh = torch.zeros(F, dtype=torch.float32, device="cuda")
    L.dec_gated_ffn(st.desc, dg[0].data_ptr(), _mat(dwg), _mat(dwu), dx.data_ptr(), dh.data_ptr())
    torch.cuda.synchronize()
    u = oracle.rmsnorm(x.astype(np.float64), oracle.dequant(g), cfg.rms_eps)
    ref = oracle.swiglu(oracle.gemv(oracle.dequant(Wg), u), oracle.gemv(oracle.dequant(Wu), u))
    assert rel_l2(dh.cpu().numpy(), ref) <= TOL


ATTN_CASES = [
    # d, kvtype, n_q, n_kv, max_ctx, positions, chunk
    (64, "f32", 4, 4, 24, (0, 15, 23), 0),
    (64, "bf16", 32, 8, 640, (0, 511, 600, 639), 0),
    (128, "bf16", 32, 32, 2176, (2047, 2100), 0),
    (128, "bf16", 32, 8, 4352, (4095, 4351), 0),
    (128, "bf16", 32, 8, 8448, (8191, 8447), 0),
    (128, "bf16", 16, 2, 300, (0, 1, 16, 17, 299), 16),   # one-row and ragged splits
    (128, "f32", 8, 1, 100, (99, 50), 48),
    (64, "bf16", 8, 4, 200, (199,), 256),                 # a single split
]


@pytest.mark.parametrize("d,kvtype,nq,nkv,max_ctx,positions,chunk", ATTN_CASES)
def test_attn_splitk(gpu, d, kvtype, nq, nkv, max_ctx, positions, chunk):
    H = 256
    cfg = synth.tiny(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype=kvtype, ctx=0, steps=max_ctx, seed=8)
    st = DecodeStack(cfg, n_layers=1, attn_chunk=chunk)
    std = 0.02 * np.sqrt(4096)
    K = synth.rand_cache((8, 1, max_ctx), nkv, max_ctx, d, kvtype, std)
    V = synth.rand_cache((8, 2, max_ctx), nkv, max_ctx, d, kvtype, std)
    st.set_prefill(0, K, V)
    Kv = oracle.ref.cache_values(K.data, kvtype, np.float64)
    Vv = oracle.ref.cache_values(V.data, kvtype, np.float64)
    for i, p in enumerate(positions):
        q = synth.rand_f32((8, 3, i), (nq, d), std=std)
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.set_pos(p)
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        ref = oracle.attend(q.astype(np.float64), Kv[:, : p + 1], Vv[:, : p + 1], nq // nkv)
        assert rel_l2(st.attn.cpu().numpy(), ref.reshape(-1)) <= TOL, f"pos {p}"
        assert int(st.counters.abs().sum().item()) == 0, "arrival counters not reset"
    assert st.check_err() == 0


KERNEL_CASES = [
    # d, n_q, n_kv, max_ctx, positions, chunk (bf16 cache: every kernel runs it)
    (64, 32, 8, 640, (0, 511, 639), 0),
    (128, 32, 32, 2176, (2047,), 0),
    (128, 16, 2, 300, (0, 1, 16, 17, 299), 16),   # one-row and ragged splits
    (128, 8, 4, 700, (699, 350), 100),            # chunks that end inside a row step
    (64, 8, 8, 1000, (999, 0), 200),
    (128, 32, 8, 4352, (4351,), 0),
    (128, 16, 4, 300, (0, 1, 16, 17, 299), 16),   # four-head groups (matrix-core scores), one-row splits
    (64, 4, 2, 333, (332, 5, 32), 33),             # two-head groups, 16-row tiles ending inside a chunk
    (128, 32, 8, 1100, (1099, 600), 256),          # 256-row chunks (the long-cache plan): several load batches
]


@pytest.mark.parametrize("kernel", ["DEC_ATTN_BATCHED", "DEC_ATTN_STREAM", "DEC_ATTN_LOCAL"])
@pytest.mark.parametrize("d,nq,nkv,max_ctx,positions,chunk", KERNEL_CASES)
def test_attn_each_kernel(gpu, kernel, d, nq, nkv, max_ctx, positions, chunk):
    """Every attention kernel, forced by its flag, on the same shapes: the
    same split-K result as the oracle, the counters reset, no error."""
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype="bf16", ctx=0, steps=max_ctx, seed=9)
    st = DecodeStack(cfg, n_layers=1, attn_chunk=chunk, flags=getattr(L, kernel))
    std = 0.02 * np.sqrt(4096)
    K = synth.rand_cache((9, 1, max_ctx), nkv, max_ctx, d, "bf16", std)
    V = synth.rand_cache((9, 2, max_ctx), nkv, max_ctx, d, "bf16", std)
    st.set_prefill(0, K, V)
    Kv = oracle.ref.cache_values(K.data, "bf16", np.float64)
    Vv = oracle.ref.cache_values(V.data, "bf16", np.float64)
    for i, p in enumerate(positions):
        q = synth.rand_f32((9, 3, i), (nq, d), std=std)
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.set_pos(p)
        st.attn.fill_(float("nan"))
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        ref = oracle.attend(q.astype(np.float64), Kv[:, : p + 1], Vv[:, : p + 1], nq // nkv)
        assert rel_l2(st.attn.cpu().numpy(), ref.reshape(-1)) <= TOL, f"{kernel} pos {p}"
        assert int(st.counters.abs().sum().item()) == 0, "arrival counters not reset"
    assert st.check_err() == 0


@pytest.mark.parametrize("kernel", ["DEC_ATTN_BATCHED", "DEC_ATTN_STREAM"])
@pytest.mark.parametrize("nq,nkv", [(32, 8), (16, 8), (8, 8)])
def test_attn_matrix_core_scores_keep_the_float32_query(gpu, kernel, nq, nkv):
    """bf16 caches with up to four query heads per kv head score on the
    matrix cores with the query as three bf16 parts. Queries eight times
    larger than usual make the softmax sharp. On these inputs (measured on
    the CPU) float32 arithmetic lands within 8e-7 relative L2 of the
    oracle, while a query kept to two bf16 parts (about 2^-17 of q) lands
    5e-6 to 2e-5 away and one part 3e-3 to 1e-2: the bound is 3e-6."""
    d, max_ctx = 128, 1000
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype="bf16", ctx=0, steps=max_ctx, seed=12)
    st = DecodeStack(cfg, n_layers=1, flags=getattr(L, kernel))
    std = 0.02 * np.sqrt(4096)
    K = synth.rand_cache((12, 1, max_ctx), nkv, max_ctx, d, "bf16", std)
    V = synth.rand_cache((12, 2, max_ctx), nkv, max_ctx, d, "bf16", std)
    st.set_prefill(0, K, V)
    Kv = oracle.ref.cache_values(K.data, "bf16", np.float64)
    Vv = oracle.ref.cache_values(V.data, "bf16", np.float64)
    for i, p in enumerate((999, 500)):
        q = synth.rand_f32((12, 3, i), (nq, d), std=8 * std)
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.set_pos(p)
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        ref = oracle.attend(q.astype(np.float64), Kv[:, : p + 1], Vv[:, : p + 1], nq // nkv)
        assert rel_l2(st.attn.cpu().numpy(), ref.reshape(-1)) <= 3e-6, f"{kernel} pos {p}"
    assert st.check_err() == 0


I8_CASES = [
    # n_q, n_kv, max_ctx, positions, chunk (int8 cache, head_dim 128, batched kernel)
    (32, 8, 640, (0, 1, 255, 256, 639), 0),
    (8, 8, 300, (0, 17, 299), 16),        # one-head groups, one-row splits at 16, 32, ...
    (16, 2, 700, (699, 350, 48), 48),     # the token alone in its split at 48
    (16, 2, 2200, (2199,), 100),
    (32, 4, 4200, (4100, 4101), 0),
    (32, 8, 1100, (1099, 513), 256),     # 256-row chunks
]


@pytest.mark.parametrize("kernel", ["default", "DEC_ATTN_BATCHED", "DEC_ATTN_STREAM"])
@pytest.mark.parametrize("nq,nkv,max_ctx,positions,chunk", I8_CASES)
def test_attn_i8_cache_appends_and_matches_oracle(gpu, nq, nkv, max_ctx, positions, chunk, kernel):
    """int8 cache: the attention quantizes the staged float k and v rows of
    the token into slot p (codes and scales equal the oracle's, bit for bit:
    both decide in binary32) and its output matches the oracle's attention
    over the decoded cache, positions 0..p; with the library's plan and with
    each kernel that reads int8 caches forced."""
    d = 128
    if kernel == "DEC_ATTN_STREAM" and nq // nkv > 4:
        pytest.skip("the streaming kernel reads int8 caches for groups of at most four heads")
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype="i8", ctx=0, steps=max_ctx, seed=10)
    flags = 0 if kernel == "default" else getattr(L, kernel)
    st = DecodeStack(cfg, n_layers=1, attn_chunk=chunk, flags=flags)
    std = 0.02 * np.sqrt(4096)
    pre = synth.rand_cache((10, 1, max_ctx), nkv, max_ctx, d, "i8", std)
    prv = synth.rand_cache((10, 2, max_ctx), nkv, max_ctx, d, "i8", std)
    st.set_prefill(0, pre, prv)
    codes_k, sc_k = pre.data.copy(), pre.scales.copy()
    codes_v, sc_v = prv.data.copy(), prv.scales.copy()
    for i, p in enumerate(positions):
        q = synth.rand_f32((10, 3, i), (nq, d), std=std)
        kn = synth.rand_f32((10, 4, i), (nkv, d), std=std)
        vn = synth.rand_f32((10, 5, i), (nkv, d), std=std)
        kn[0, :] = 0.0 if i == 1 else kn[0, :]            # a zero row once: scale 0, codes 0
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.Kstage[0].copy_(torch.from_numpy(kn))
        st.Vstage[0].copy_(torch.from_numpy(vn))
        st.set_pos(p)
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        ck, sk = oracle.quantize_i8(kn)
        cv, sv = oracle.quantize_i8(vn)
        assert np.array_equal(st.K[0, :, p].cpu().numpy(), ck), f"key codes at {p}"
        assert np.array_equal(st.V[0, :, p].cpu().numpy(), cv), f"value codes at {p}"
        assert np.array_equal(st.Ks[0, :, p].cpu().numpy(), sk) and np.array_equal(st.Vs[0, :, p].cpu().numpy(), sv)
        codes_k[:, p], sc_k[:, p], codes_v[:, p], sc_v[:, p] = ck, sk, cv, sv
        Kd = oracle.ref.cache_values(codes_k[:, : p + 1], "i8", np.float64, sc_k[:, : p + 1])
        Vd = oracle.ref.cache_values(codes_v[:, : p + 1], "i8", np.float64, sc_v[:, : p + 1])
        ref = oracle.attend(q.astype(np.float64), Kd, Vd, nq // nkv)
        assert rel_l2(st.attn.cpu().numpy(), ref.reshape(-1)) <= TOL, f"pos {p}"
        assert int(st.counters.abs().sum().item()) == 0
    assert st.check_err() == 0


@pytest.mark.parametrize("kernel", ["DEC_ATTN_BATCHED", "DEC_ATTN_STREAM"])
@pytest.mark.parametrize("nq,nkv", [(32, 8), (16, 8), (8, 8)])
def test_attn_i8_matrix_core_scores_keep_22_bits_of_the_query(gpu, kernel, nq, nkv):
    """int8 caches with up to four query heads per kv head score on the
    matrix cores with each scaled query head as integers of 22 bits (three
    int8 digits). With queries eight times larger than usual (a sharp
    softmax), these inputs land within 1.4e-6 relative L2 of the oracle when
    computed in float32 with a 22-bit query and at least 1.1e-4 away with a
    14-bit one (two digits; measured on the CPU): the bound is 1e-5."""
    d, max_ctx = 128, 1000
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype="i8", ctx=0, steps=max_ctx, seed=13)
    st = DecodeStack(cfg, n_layers=1, flags=getattr(L, kernel))
    std = 0.02 * np.sqrt(4096)
    pre = synth.rand_cache((13, 1, max_ctx), nkv, max_ctx, d, "i8", std)
    prv = synth.rand_cache((13, 2, max_ctx), nkv, max_ctx, d, "i8", std)
    st.set_prefill(0, pre, prv)
    codes_k, sc_k = pre.data.copy(), pre.scales.copy()
    codes_v, sc_v = prv.data.copy(), prv.scales.copy()
    for i, p in enumerate((999, 500)):
        q = synth.rand_f32((13, 3, i), (nq, d), std=8 * std)
        kn = synth.rand_f32((13, 4, i), (nkv, d), std=std)
        vn = synth.rand_f32((13, 5, i), (nkv, d), std=std)
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.Kstage[0].copy_(torch.from_numpy(kn))
        st.Vstage[0].copy_(torch.from_numpy(vn))
        st.set_pos(p)
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        (codes_k[:, p], sc_k[:, p]), (codes_v[:, p], sc_v[:, p]) = oracle.quantize_i8(kn), oracle.quantize_i8(vn)
        Kd = oracle.ref.cache_values(codes_k[:, : p + 1], "i8", np.float64, sc_k[:, : p + 1])
        Vd = oracle.ref.cache_values(codes_v[:, : p + 1], "i8", np.float64, sc_v[:, : p + 1])
        ref = oracle.attend(q.astype(np.float64), Kd, Vd, nq // nkv)
        assert rel_l2(st.attn.cpu().numpy(), ref.reshape(-1)) <= TOL, f"{kernel} pos {p}"
    assert st.check_err() == 0


@pytest.mark.parametrize("kernel", ["DEC_ATTN_BATCHED", "DEC_ATTN_STREAM"])
@pytest.mark.parametrize("kvtype", ["bf16", "i8"])
def test_attn_matrix_core_scores_keep_a_nan_query_visible(gpu, kernel, kvtype):
    """A NaN in one query head makes that head's output NaN, as float
    arithmetic would (the int8 digits of a non-finite query poison the
    head's scores instead of rounding it to an integer); the other heads of
    the same kv head still match the oracle."""
    d, nq, nkv, max_ctx, p = 128, 16, 4, 300, 299
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype=kvtype, ctx=0, steps=max_ctx, seed=14)
    st = DecodeStack(cfg, n_layers=1, flags=getattr(L, kernel))
    std = 0.02 * np.sqrt(4096)
    K = synth.rand_cache((14, 1, max_ctx), nkv, max_ctx, d, kvtype, std)
    V = synth.rand_cache((14, 2, max_ctx), nkv, max_ctx, d, kvtype, std)
    st.set_prefill(0, K, V)
    sk = sv = None
    if kvtype == "i8":
        kn = synth.rand_f32((14, 4, 0), (nkv, d), std=std)
        vn = synth.rand_f32((14, 5, 0), (nkv, d), std=std)
        st.Kstage[0].copy_(torch.from_numpy(kn))
        st.Vstage[0].copy_(torch.from_numpy(vn))
        K.data[:, p], K.scales[:, p] = oracle.quantize_i8(kn)
        V.data[:, p], V.scales[:, p] = oracle.quantize_i8(vn)
        sk, sv = K.scales, V.scales
    q = synth.rand_f32((14, 3, 0), (nq, d), std=std)
    bad = 5                      # query head 5: kv head 1, second head of its group
    q[bad, 17] = np.nan
    st.q.copy_(torch.from_numpy(q.reshape(-1)))
    st.set_pos(p)
    L.dec_attn_splitk(st.desc, st.state[0])
    torch.cuda.synchronize()
    got = st.attn.cpu().numpy().reshape(nq, d)
    assert np.isnan(got[bad]).all(), "the NaN query head's output"
    Kd = oracle.ref.cache_values(K.data[:, : p + 1], kvtype, np.float64, None if sk is None else sk[:, : p + 1])
    Vd = oracle.ref.cache_values(V.data[:, : p + 1], kvtype, np.float64, None if sv is None else sv[:, : p + 1])
    q[bad] = 0.0
    ref = oracle.attend(q.astype(np.float64), Kd, Vd, nq // nkv)
    keep = [h for h in range(nq) if h != bad]
    assert rel_l2(got[keep].reshape(-1), ref[keep].reshape(-1)) <= TOL
    assert st.check_err() == 0


def test_combiner_give_up_sets_sync_error_and_recovers(gpu):
    """The attention combine's failure path, forced from the host:
    DEC_TEST_NO_WAIT makes every combiner but the last arrival of a kv head
    give up its wait at once. Each launch still completes; its only effects
    are the DEC_ERR_SYNC bit and output slices left unwritten (every output
    element is either untouched or the oracle's value, and each kv head group
    has both); the arrival counters are left zero, and the next normal launch
    on the same buffers is exact."""
    d, nq, nkv, max_ctx = 128, 32, 8, 4352      # the 9B-shaped layer: several combiners per kv head
    cfg = synth.tiny(hidden=256, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=256, wtype="bf16",
                     ntype="bf16", kvtype="bf16", ctx=0, steps=max_ctx, seed=9)
    st = DecodeStack(cfg, n_layers=1, flags=L.DEC_TEST_NO_WAIT)
    std = 0.02 * np.sqrt(4096)
    K = synth.rand_cache((9, 1, max_ctx), nkv, max_ctx, d, "bf16", std)
    V = synth.rand_cache((9, 2, max_ctx), nkv, max_ctx, d, "bf16", std)
    st.set_prefill(0, K, V)
    Kv = oracle.ref.cache_values(K.data, "bf16", np.float64)
    Vv = oracle.ref.cache_values(V.data, "bf16", np.float64)
    group = (nq // nkv) * d
    for i, p in enumerate((4095, 4351)):
        q = synth.rand_f32((9, 3, i), (nq, d), std=std)
        st.q.copy_(torch.from_numpy(q.reshape(-1)))
        st.set_pos(p)
        ref = oracle.attend(q.astype(np.float64), Kv[:, : p + 1], Vv[:, : p + 1], nq // nkv).reshape(-1)
        st.desc.flags = L.DEC_TEST_NO_WAIT
        st.err.zero_()
        _fill_sentinel(st.attn)
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        assert st.check_err() == L.DEC_ERR_SYNC, f"pos {p}"
        assert int(st.counters.abs().sum().item()) == 0, "arrival counters not reset"
        got = st.attn.cpu().numpy()
        untouched = got.view(np.uint32) == SENT32
        for j in range(nkv):
            sl = slice(j * group, (j + 1) * group)
            assert untouched[sl].any() and not untouched[sl].all(), f"kv head {j}"
            w = ~untouched[sl]
            assert rel_l2(got[sl][w], ref[sl][w]) <= TOL, f"kv head {j}: written slice"
        # the same buffers, the normal path
        st.desc.flags = 0
        st.err.zero_()
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        assert st.check_err() == 0
        assert rel_l2(st.attn.cpu().numpy(), ref) <= TOL, f"pos {p}: after the failure"
        assert int(st.counters.abs().sum().item()) == 0


def test_position_out_of_range_sets_error_and_stores_nothing(gpu):
    cfg = _cfg("bf16", "bf16", 256, 4, 4, 64, max_ctx=8)
    lw = synth.layer_weights(cfg, 0)
    st = DecodeStack(cfg, n_layers=1)
    st.set_layer(0, lw)
    _fill_sentinel(st.K)
    _fill_sentinel(st.V)
    st.q.fill_(7.0)
    for bad in (8, -1, 1000):
        st.err.zero_()
        st.set_pos(bad)
        L.dec_rmsnorm_gemv_qkv_rope(st.desc, st.wstruct[0], st.state[0])
        L.dec_attn_splitk(st.desc, st.state[0])
        torch.cuda.synchronize()
        assert st.check_err() & L.DEC_ERR_POS
    assert bool(torch.all(st.K == SENT16)) and bool(torch.all(st.V == SENT16))
    assert bool(torch.all(st.q == 7.0))


HEAD_CASES = [
    # head type, H, vocab
    ("f32", 256, 1000),
    ("bf16", 2048, 32000),
    ("q4", 4096, 32000),
    ("q4", 2080, 999),            # ragged: 65 blocks per row, odd row count
]


@pytest.mark.parametrize("htype,H,vocab", HEAD_CASES)
def test_lm_head_logits_and_argmax(gpu, htype, H, vocab):
    """Final RMSNorm, head GEMV and the greedy argmax into the device token."""
    cfg = _cfg("f32" if htype == "f32" else "bf16", "bf16", H, 4, 4, 64).with_(vocab=vocab)
    st = DecodeStack(cfg, n_layers=1)
    g = synth.rand_norm((8, 1, H), H, cfg.ntype)
    head = synth.rand_matrix((8, 2, vocab), vocab, H, htype)
    x = synth.rand_f32((8, 3, H), (H,))
    st.set_head(g, head)
    st.x.copy_(torch.from_numpy(x))
    st.token.fill_(-1)
    st.head_step()
    torch.cuda.synchronize()
    xf = oracle.rmsnorm(x.astype(np.float64), oracle.dequant(g), cfg.rms_eps)
    ref = oracle.gemv(oracle.dequant(head), xf)
    got = st.logits.cpu().numpy()
    assert rel_l2(got, ref) <= TOL
    # the token is the argmax of the logits the kernel wrote (lowest index on
    # ties), and the oracle's own argmax unless its top two are within the error
    tok = int(st.token.item())
    assert tok == int(np.argmax(got))
    top2 = np.sort(ref)[-2:]
    if top2[1] - top2[0] > 1e-4 * np.abs(ref).max():
        assert tok == int(np.argmax(ref))
