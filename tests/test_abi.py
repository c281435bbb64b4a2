"""The C ABI without a GPU: libdec.so loads, exports every function that
include/dec_api.h declares, the ctypes binding lays out every struct and
constant exactly as a C compiler does from the header, and the host-side
argument checks return the documented codes. No call here enqueues a kernel:
every compute entry point is called only with arguments its checks reject
before any launch, and the size queries are pure host arithmetic.
"""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dec_api.h")

DEC_OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_UNSUPPORTED = 0, -1, -2, -3, -4, -6


@pytest.fixture(scope="module")
def L():
    from transformer_layer_amd import build, lib
    if not os.path.exists(lib.LIBPATH):
        build.build()
    lib.load()
    return lib


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(dec_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_layer_kernels_and_the_step():
    names = header_functions()
    for n in ["dec_rmsnorm_gemv_qkv_rope", "dec_attn_splitk", "dec_gemv_residual", "dec_gated_ffn",
              "dec_layer_step"]:
        assert n in names


def test_every_declared_function_is_exported_and_bound(L):
    names = header_functions()
    assert sorted(L.SIGNATURES) == names
    lib = ctypes.CDLL(L.LIBPATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported by libdec.so"
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIBPATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
        assert set(names) <= exported
        assert not {s for s in exported if s.startswith("dec_")} - set(names), "exports not in the header"


def test_abi_version(L):
    assert L.dec_abi_version() == L.ABI_VERSION
    m = re.search(r"#define DEC_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == L.ABI_VERSION


PROBE = r"""
#include <stddef.h>
#include <stdio.h>
#include "dec_api.h"
#define S(T) printf(#T " size %zu\n", sizeof(T));
#define O(T, f) printf(#T " %s %zu\n", #f, offsetof(T, f));
int main(void) {
  S(dec_layer_desc) O(dec_layer_desc, hidden) O(dec_layer_desc, n_q_heads) O(dec_layer_desc, n_kv_heads)
  O(dec_layer_desc, head_dim) O(dec_layer_desc, ffn) O(dec_layer_desc, max_ctx) O(dec_layer_desc, rms_eps)
  O(dec_layer_desc, wtype) O(dec_layer_desc, ntype) O(dec_layer_desc, kvtype) O(dec_layer_desc, attn_chunk)
  O(dec_layer_desc, flags)
  S(dec_mat) O(dec_mat, w) O(dec_mat, scales)
  S(dec_layer_weights) O(dec_layer_weights, attn_norm) O(dec_layer_weights, wqkv) O(dec_layer_weights, wo)
  O(dec_layer_weights, ffn_norm) O(dec_layer_weights, wgate) O(dec_layer_weights, wup)
  O(dec_layer_weights, wdown)
  S(dec_layer_state) O(dec_layer_state, x) O(dec_layer_state, q) O(dec_layer_state, attn)
  O(dec_layer_state, h) O(dec_layer_state, part) O(dec_layer_state, counters) O(dec_layer_state, k_cache)
  O(dec_layer_state, v_cache) O(dec_layer_state, pos) O(dec_layer_state, rope) O(dec_layer_state, err)
  O(dec_layer_state, scratch)
  printf("DEC_F32 value %d\nDEC_BF16 value %d\nDEC_Q4 value %d\nDEC_I8 value %d\n", DEC_F32, DEC_BF16, DEC_Q4,
         DEC_I8);
  printf("DEC_UNFUSED value %u\nDEC_NULL_KERNELS value %u\nDEC_TEST_NO_WAIT value %u\n", DEC_UNFUSED,
         DEC_NULL_KERNELS, DEC_TEST_NO_WAIT);
  printf("DEC_NO_FUSE_QKV value %u\nDEC_NO_FUSE_FFN value %u\nDEC_NO_FUSE_ATTN_O value %u\n", DEC_NO_FUSE_QKV,
         DEC_NO_FUSE_FFN, DEC_NO_FUSE_ATTN_O);
  printf("DEC_DETERMINISTIC value %u\nDEC_TEST_SKIP_ROPE value %u\nDEC_TEST_APPEND_NEXT value %u\n",
         DEC_DETERMINISTIC, DEC_TEST_SKIP_ROPE, DEC_TEST_APPEND_NEXT);
  printf("DEC_FUSE_DOWN value %u\nDEC_DEBUG_EXPORT_KV value %u\n", DEC_FUSE_DOWN, DEC_DEBUG_EXPORT_KV);
  printf("DEC_TEST_DROP_SPLIT value %u\nDEC_E_UNSUPPORTED value %d\n", DEC_TEST_DROP_SPLIT, DEC_E_UNSUPPORTED);
  printf("DEC_ERR_POS value %u\nDEC_ERR_TOKEN value %u\nDEC_ERR_SYNC value %u\n", DEC_ERR_POS, DEC_ERR_TOKEN,
         DEC_ERR_SYNC);
  printf("DEC_COUNTER_STRIDE value %d\n", DEC_COUNTER_STRIDE);
  printf("DEC_E_NULL value %d\nDEC_E_SHAPE value %d\nDEC_E_DTYPE value %d\nDEC_E_ALIGN value %d\n",
         DEC_E_NULL, DEC_E_SHAPE, DEC_E_DTYPE, DEC_E_ALIGN);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_struct_layout_matches_a_c_compiler(L, tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(PROBE)
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o",
                    str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    seen = 0
    for ln in filter(None, lines):
        name, field, val = ln.split()
        val = int(val)
        if field == "value":
            want = {"DEC_F32": L.DEC_F32, "DEC_BF16": L.DEC_BF16, "DEC_Q4": L.DEC_Q4, "DEC_I8": L.DEC_I8,
                    "DEC_UNFUSED": L.DEC_UNFUSED, "DEC_NULL_KERNELS": L.DEC_NULL_KERNELS,
                    "DEC_TEST_NO_WAIT": L.DEC_TEST_NO_WAIT, "DEC_NO_FUSE_QKV": L.DEC_NO_FUSE_QKV,
                    "DEC_NO_FUSE_FFN": L.DEC_NO_FUSE_FFN, "DEC_NO_FUSE_ATTN_O": L.DEC_NO_FUSE_ATTN_O,
                    "DEC_DETERMINISTIC": L.DEC_DETERMINISTIC, "DEC_TEST_SKIP_ROPE": L.DEC_TEST_SKIP_ROPE,
                    "DEC_FUSE_DOWN": L.DEC_FUSE_DOWN, "DEC_DEBUG_EXPORT_KV": L.DEC_DEBUG_EXPORT_KV,
                    "DEC_TEST_APPEND_NEXT": L.DEC_TEST_APPEND_NEXT, "DEC_TEST_DROP_SPLIT": L.DEC_TEST_DROP_SPLIT,
                    "DEC_E_UNSUPPORTED": E_UNSUPPORTED,
                    "DEC_ERR_POS": L.DEC_ERR_POS, "DEC_ERR_TOKEN": L.DEC_ERR_TOKEN, "DEC_ERR_SYNC": L.DEC_ERR_SYNC,
                    "DEC_E_NULL": E_NULL, "DEC_E_SHAPE": E_SHAPE, "DEC_E_DTYPE": E_DTYPE,
                    "DEC_E_ALIGN": E_ALIGN, "DEC_COUNTER_STRIDE": L.DEC_COUNTER_STRIDE}[name]
            assert val == want, name
        elif field == "size":
            assert ctypes.sizeof(getattr(L, name)) == val, name
        else:
            assert getattr(getattr(L, name), field).offset == val, f"{name}.{field}"
        seen += 1
    assert seen == 62   # 4 sizes, 33 offsets, 25 constants


# ---- host-side checks (every call below is rejected before any launch)

FAKE = 1 << 20   # a 16-byte-aligned address that is never dereferenced: the call fails first


def desc_of(L, cfg, **over):
    d = L.dec_layer_desc(hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                         head_dim=cfg.head_dim, ffn=cfg.ffn, max_ctx=cfg.max_ctx, rms_eps=cfg.rms_eps,
                         wtype=L.DTYPES[cfg.wtype], ntype=L.DTYPES[cfg.ntype], kvtype=L.DTYPES[cfg.kvtype],
                         attn_chunk=0, flags=0)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def weights_of(L, scales=True, **over):
    m = L.dec_mat(FAKE, FAKE if scales else None)
    w = L.dec_layer_weights(attn_norm=FAKE, wqkv=m, wo=m, ffn_norm=FAKE, wgate=m, wup=m, wdown=m)
    for k, v in over.items():
        setattr(w, k, v)
    return w


def state_of(L, **over):
    s = L.dec_layer_state(x=FAKE, q=FAKE, attn=FAKE, h=FAKE, part=FAKE, counters=FAKE, k_cache=FAKE,
                          v_cache=FAKE, pos=FAKE, rope=FAKE, err=FAKE, scratch=None)
    for k, v in over.items():
        setattr(s, k, v)
    return s


def rc_step(L, d, w, s):
    lib = L.load()
    return lib.dec_layer_step(ctypes.byref(d) if d is not None else None, ctypes.byref(w), ctypes.byref(s), None)


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_buffer_sizes(L, name):
    cfg = synth.CONFIGS[name]
    d = desc_of(L, cfg)
    n = L.dec_attn_part_floats(d)
    # one (d outputs + max + sum) record per q head per split, splits >= 1
    per_split = cfg.n_q_heads * (cfg.head_dim + 2)
    assert n >= per_split and n % per_split == 0
    splits = n // per_split
    assert 1 <= splits <= 256
    p4 = lambda v: (v + 3) // 4 * 4  # noqa: E731
    assert L.dec_scratch_floats(d) == p4(cfg.hidden) + p4(cfg.n_qkv) + 2 * p4(cfg.ffn)


@pytest.mark.parametrize("field,value,code,word", [
    ("head_dim", 96, E_SHAPE, "head_dim"),
    ("n_kv_heads", 3, E_SHAPE, "heads"),
    ("n_kv_heads", 2, E_SHAPE, "group"),        # 32 / 2 = 16 q heads per kv head
    ("hidden", 4100, E_SHAPE, "length"),        # not a multiple of the bf16 granule (8)
    ("ffn", 20000, E_SHAPE, "length"),          # beyond 16384
    ("max_ctx", 0, E_SHAPE, "max_ctx"),
    ("rms_eps", float("nan"), E_SHAPE, "rms_eps"),
    ("attn_chunk", 300, E_SHAPE, "attn_chunk"),
    ("wtype", 7, E_DTYPE, "wtype"),
    ("ntype", 2, E_DTYPE, "ntype"),             # 4-bit norm weights are not a thing
    ("kvtype", 2, E_DTYPE, "kvtype"),           # a 4-bit cache is not a thing either
    ("kvtype", 4, E_DTYPE, "kvtype"),
])
def test_bad_descriptor_is_rejected(L, field, value, code, word):
    d = desc_of(L, synth.CONFIGS["C4"], **{field: value})
    assert rc_step(L, d, weights_of(L), state_of(L)) == code
    assert word in L.dec_last_error()
    assert L.load().dec_attn_part_floats(ctypes.byref(d)) == -1


@pytest.mark.parametrize("kernel,over", [
    ("DEC_ATTN_LOCAL", {"kvtype": 0}),                        # the wave-local kernel reads bf16 caches only
    ("DEC_ATTN_STREAM", {"kvtype": 0, "n_q_heads": 64, "attn_chunk": 256}),  # f32 values beyond LDS
    ("DEC_ATTN_BATCHED", {"max_ctx": 100000}),                # 391 splits of at most 256 positions
    ("DEC_ATTN_LOCAL", {"kvtype": 3}),                        # nor an int8 one
])
def test_attention_kernel_that_cannot_run_the_shape_is_refused(L, kernel, over):
    d = desc_of(L, synth.CONFIGS["C4"], flags=getattr(L, kernel), **over)
    assert rc_step(L, d, weights_of(L), state_of(L)) == E_SHAPE
    assert L.load().dec_attn_part_floats(ctypes.byref(d)) == -1


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5"])
def test_every_attention_kernel_plans_the_workloads(L, name):
    """Each kernel, forced, plans every bf16-cache workload (C2-C5) within
    256 splits, and the library default's partials fit one of them."""
    cfg = synth.CONFIGS[name]
    sizes = []
    for k in ("DEC_ATTN_BATCHED", "DEC_ATTN_STREAM", "DEC_ATTN_LOCAL"):
        n = L.dec_attn_part_floats(desc_of(L, cfg, flags=getattr(L, k)))
        assert n > 0, (name, k, L.dec_last_error())
        sizes.append(n)
    assert L.dec_attn_part_floats(desc_of(L, cfg)) in sizes


def test_int8_cache_layout_and_shapes(L):
    """An int8 cache is one buffer per layer: the codes [n_kv, max_ctx, d],
    one float scale per row from the first 256-byte boundary after them,
    and the staged newest row (n_kv * d floats) from the next one. Only
    128-wide heads are accepted; the batched kernel plans every workload
    shape with it."""
    for name in ("C3", "C4", "C5"):
        cfg = synth.CONFIGS[name]
        d = desc_of(L, cfg, kvtype=L.DEC_I8)
        codes = cfg.n_kv_heads * cfg.max_ctx * cfg.head_dim
        up = lambda v: (v + 255) // 256 * 256  # noqa: E731
        assert L.dec_cache_scale_offset(d) == up(codes)
        assert L.dec_cache_stage_offset(d) == up(up(codes) + 4 * cfg.n_kv_heads * cfg.max_ctx)
        assert L.dec_cache_bytes(d) == L.dec_cache_stage_offset(d) + 4 * cfg.n_kv_heads * cfg.head_dim
        assert L.dec_attn_part_floats(d) > 0, L.dec_last_error()
        b = desc_of(L, cfg)
        assert L.dec_cache_bytes(b) == codes * 2
        lib = L.load()
        assert lib.dec_cache_scale_offset(ctypes.byref(b)) == -1 and "not int8" in L.dec_last_error()
        assert lib.dec_cache_stage_offset(ctypes.byref(b)) == -1
    d = desc_of(L, synth.CONFIGS["C2"], kvtype=L.DEC_I8)   # 64-wide heads
    assert rc_step(L, d, weights_of(L), state_of(L)) == E_SHAPE
    assert "int8 cache needs head_dim 128" in L.dec_last_error()
    assert L.load().dec_cache_bytes(ctypes.byref(d)) == -1


def test_gated_ffn_down_refusals(L):
    """The FFN with the down projection folded in runs 4-bit weights only,
    and only shapes whose workgroups (one per 16 rows of x) can all be
    resident at once and whose rows fit its plans; each refusal is made on
    the host, before any launch."""
    lib = L.load()
    w, s = weights_of(L), state_of(L)

    def call(d):
        return lib.dec_gated_ffn_down(ctypes.byref(d), ctypes.byref(w), ctypes.byref(s), None)

    bf = desc_of(L, synth.CONFIGS["C4"])
    assert call(bf) == E_UNSUPPORTED and "4-bit" in L.dec_last_error()
    bf.flags = L.DEC_FUSE_DOWN
    assert rc_step(L, bf, w, s) == E_UNSUPPORTED
    big = desc_of(L, synth.CONFIGS["C5"], hidden=8192)           # 512 workgroups of 155 VGPRs a lane
    assert call(big) == E_SHAPE and "resident" in L.dec_last_error()
    big.flags = L.DEC_FUSE_DOWN
    assert rc_step(L, big, w, s) == E_SHAPE
    noplan = desc_of(L, synth.CONFIGS["C5"], hidden=512, ffn=16384)   # 64 gate/up tiles per workgroup
    assert call(noplan) == E_SHAPE and "no plan" in L.dec_last_error()
    assert lib.dec_gated_ffn_down(ctypes.byref(desc_of(L, synth.CONFIGS["C5"])), None, ctypes.byref(s),
                                  None) == E_NULL


def test_null_arguments_are_rejected(L):
    lib = L.load()
    cfg = synth.CONFIGS["C4"]
    d = desc_of(L, cfg)
    assert rc_step(L, None, weights_of(L), state_of(L)) == E_NULL
    assert rc_step(L, d, weights_of(L, attn_norm=None), state_of(L)) == E_NULL
    assert rc_step(L, d, weights_of(L), state_of(L, pos=None)) == E_NULL
    assert rc_step(L, d, weights_of(L), state_of(L, counters=None)) == E_NULL
    # the per-op path needs scratch
    du = desc_of(L, cfg, flags=L.DEC_UNFUSED)
    assert rc_step(L, du, weights_of(L), state_of(L)) == E_NULL and "scratch" in L.dec_last_error()
    # 4-bit weights need scales
    dq = desc_of(L, synth.CONFIGS["C5"])
    assert rc_step(L, dq, weights_of(L, scales=False), state_of(L)) == E_NULL
    assert "scales" in L.dec_last_error()
    assert lib.dec_attn_splitk(ctypes.byref(d), None, None) == E_NULL
    assert lib.dec_gated_ffn(ctypes.byref(d), None, L.dec_mat(FAKE, None), L.dec_mat(FAKE, None), FAKE, FAKE,
                             None) == E_NULL
    assert lib.dec_rope_table(1e4, 128, 16, None, None) == E_NULL
    assert lib.dec_embed(None, 32000, 4096, FAKE, FAKE, FAKE, None) == E_NULL
    assert lib.dec_advance(None, 0, 8, None, None, None) == E_NULL


@pytest.mark.parametrize("flag", ["DEC_UNFUSED", "DEC_NO_FUSE_QKV", "DEC_NO_FUSE_FFN", "DEC_DEBUG_EXPORT_KV"])
def test_per_op_paths_need_scratch(L, flag):
    d = desc_of(L, synth.CONFIGS["C4"], flags=getattr(L, flag))
    assert rc_step(L, d, weights_of(L), state_of(L)) == E_NULL and "scratch" in L.dec_last_error()


def test_debug_kv_export_sits_after_the_per_op_intermediates(L):
    """DEC_DEBUG_EXPORT_KV: the k and v rows (2 n_kv d floats) follow every
    per-op intermediate in the scratch buffer, which grows by that much; the
    QKV entry point then needs scratch too, and the static step refuses the
    flag (its scratch is the library's own)."""
    lib = L.load()
    cfg = synth.CONFIGS["C4"]
    p4 = lambda v: (v + 3) // 4 * 4  # noqa: E731
    plain, dbg = desc_of(L, cfg), desc_of(L, cfg, flags=L.DEC_DEBUG_EXPORT_KV)
    off = p4(cfg.hidden) + p4(cfg.n_qkv) + 2 * p4(cfg.ffn)
    assert L.dec_scratch_kv_offset(plain) == L.dec_scratch_kv_offset(dbg) == off
    assert L.dec_scratch_floats(plain) == off
    assert L.dec_scratch_floats(dbg) == off + p4(2 * cfg.n_kv_heads * cfg.head_dim)
    assert lib.dec_rmsnorm_gemv_qkv_rope(ctypes.byref(dbg), ctypes.byref(weights_of(L)),
                                         ctypes.byref(state_of(L)), None) == E_NULL
    assert "scratch" in L.dec_last_error()
    st = state_of(L, part=None, counters=None)
    assert lib.dec_layer_step_static(ctypes.byref(dbg), ctypes.byref(weights_of(L)), ctypes.byref(st),
                                     None) == E_UNSUPPORTED
    assert "DEC_DEBUG_EXPORT_KV" in L.dec_last_error()


def test_combine_in_output_projection_is_refused_where_it_does_not_apply(L):
    """dec_attn_o_residual needs bf16 weights and cache and at most 32
    attention splits, and cannot honour DEC_DETERMINISTIC (float atomics)."""
    lib = L.load()
    m = L.dec_mat(FAKE, None)
    call = lambda d: lib.dec_attn_o_residual(ctypes.byref(d), m, ctypes.byref(state_of(L)), None)  # noqa: E731
    assert call(desc_of(L, synth.CONFIGS["C1"])) == E_UNSUPPORTED          # f32 weights
    assert call(desc_of(L, synth.CONFIGS["C4"], max_ctx=60000)) == E_UNSUPPORTED   # too many splits
    assert "splits" in L.dec_last_error()
    assert call(desc_of(L, synth.CONFIGS["C4"], flags=L.DEC_DETERMINISTIC)) == E_UNSUPPORTED
    assert "atomics" in L.dec_last_error()
    assert lib.dec_attn_o_residual(ctypes.byref(desc_of(L, synth.CONFIGS["C4"])), L.dec_mat(None, None),
                                   ctypes.byref(state_of(L)), None) == E_NULL
    assert lib.dec_attn_partials(ctypes.byref(desc_of(L, synth.CONFIGS["C4"])), None, None) == E_NULL


def test_static_step_rejects_shapes_beyond_its_scratch(L):
    """dec_layer_step_static checks its scratch capacity before touching the
    device: a cache long enough that the split partials pass
    DEC_STATIC_SCRATCH_BYTES is refused with DEC_E_SHAPE."""
    lib = L.load()
    # 128 query heads: each split's partials take 128 x 130 floats
    cfg = synth.CONFIGS["C4"].with_(hidden=16384, n_q_heads=128, n_kv_heads=16, ffn=16384)
    ctx = cfg.max_ctx
    while 4 * L.dec_attn_part_floats(desc_of(L, cfg, max_ctx=ctx)) + (64 << 10) <= L.DEC_STATIC_SCRATCH_BYTES:
        ctx *= 2
    d = desc_of(L, cfg, max_ctx=ctx)
    st = state_of(L, part=None, counters=None)
    assert lib.dec_layer_step_static(ctypes.byref(d), ctypes.byref(weights_of(L)), ctypes.byref(st), None) == E_SHAPE
    assert "static scratch" in L.dec_last_error()
    assert lib.dec_layer_step_static(ctypes.byref(d), ctypes.byref(weights_of(L)), None, None) == E_NULL
    assert lib.dec_layer_step_static(None, ctypes.byref(weights_of(L)), ctypes.byref(st), None) == E_NULL


def test_misaligned_pointers_are_rejected(L):
    d = desc_of(L, synth.CONFIGS["C4"])
    bad = L.dec_mat(FAKE + 2, None)
    assert rc_step(L, d, weights_of(L, wo=bad), state_of(L)) == E_ALIGN
    assert rc_step(L, d, weights_of(L), state_of(L, k_cache=FAKE + 8)) == E_ALIGN
    lib = L.load()
    assert lib.dec_gemv_residual(ctypes.byref(d), L.dec_mat(FAKE, None), 4096, 4096, FAKE + 4, FAKE * 2,
                                 None) == E_ALIGN


def test_bad_sizes_are_rejected(L):
    lib = L.load()
    d = desc_of(L, synth.CONFIGS["C4"])
    m = L.dec_mat(FAKE, None)
    assert lib.dec_gemv_residual(ctypes.byref(d), m, 4096, 4100, FAKE, FAKE * 2, None) == E_SHAPE
    assert lib.dec_gemv_residual(ctypes.byref(d), m, 0, 4096, FAKE, FAKE * 2, None) == E_SHAPE
    # input and output overlapping
    assert lib.dec_gemv_residual(ctypes.byref(d), m, 4096, 4096, FAKE, FAKE + 64, None) == E_SHAPE
    assert "overlap" in L.dec_last_error()
    assert lib.dec_rope_table(-1.0, 128, 16, FAKE, None) == E_SHAPE
    assert lib.dec_rope_table(1e4, 127, 16, FAKE, None) == E_SHAPE
    assert lib.dec_advance(FAKE, 8, 8, None, None, None) == E_SHAPE
    assert lib.dec_advance(FAKE, -1, 8, None, None, None) == E_SHAPE
    assert lib.dec_embed(FAKE, 0, 4096, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert lib.dec_lm_head(ctypes.byref(d), 1, FAKE, m, 0, FAKE, FAKE, FAKE, None) == E_SHAPE
    assert lib.dec_lm_head(ctypes.byref(d), 5, FAKE, m, 32000, FAKE, FAKE, FAKE, None) == E_DTYPE


def test_error_text_is_per_thread(L):
    import threading
    lib = L.load()
    d = desc_of(L, synth.CONFIGS["C4"], head_dim=96)
    assert lib.dec_attn_part_floats(ctypes.byref(d)) == -1
    seen = []

    def other():
        seen.append(L.dec_last_error())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "head_dim" in L.dec_last_error()
    assert seen == [""]


def test_library_allocates_copies_and_synchronises_nothing(L):
    """Every buffer comes from the caller: the HIP runtime functions the
    library imports are kernel registration and launch, device and occupancy
    queries and error reporting only. No allocation, free, memset, copy or
    synchronisation can happen inside an entry point, so a decode step is
    capturable into a graph as it stands."""
    out = subprocess.run(["nm", "-D", "--undefined-only", L.LIBPATH], capture_output=True, text=True)
    if out.returncode != 0:
        pytest.skip("nm unavailable")
    imported = {ln.split()[-1].split("@")[0] for ln in out.stdout.splitlines() if ln.strip()}
    hip = {s for s in imported if s.lower().startswith(("hip", "__hip"))}
    allowed = {"__hipRegisterFatBinary", "__hipUnregisterFatBinary", "__hipRegisterFunction",
               "__hipRegisterVar", "__hipPushCallConfiguration", "__hipPopCallConfiguration",
               "hipLaunchKernel", "hipGetDevice", "hipDeviceGetAttribute", "hipGetLastError",
               "hipGetErrorString", "hipOccupancyMaxActiveBlocksPerMultiprocessor",
               # dec_layer_step_static: its array's device address, and whether the
               # caller's stream is capturing (a query, no work enqueued)
               "hipGetSymbolAddress", "hipStreamIsCapturing"}
    assert hip <= allowed, f"unexpected HIP runtime imports: {sorted(hip - allowed)}"
    assert not {s for s in imported if s in ("malloc", "calloc", "realloc") or "Malloc" in s}, \
        "the library should not allocate host memory either"
