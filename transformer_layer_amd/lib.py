"""ctypes binding of libdec (argument marshalling only).

The functions here carry the C entry points' names and pass device pointers,
sizes and the caller's HIP stream straight through; every step of the decode
layer runs in the library's HIP kernels. Loading fails loudly when the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os

LIBPATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libdec.so")

DEC_F32, DEC_BF16, DEC_Q4, DEC_I8 = 0, 1, 2, 3
DTYPES = {"f32": DEC_F32, "bf16": DEC_BF16, "q4": DEC_Q4, "i8": DEC_I8}
DEC_UNFUSED = 0x1
DEC_NULL_KERNELS = 0x2
DEC_NO_FUSE_QKV = 0x4
DEC_NO_FUSE_FFN = 0x8
DEC_NO_FUSE_ATTN_O = 0x10
DEC_DETERMINISTIC = 0x20
DEC_FUSE_DOWN = 0x40
DEC_DEBUG_EXPORT_KV = 0x80
DEC_ATTN_KERNEL_MASK = 0x3000
DEC_ATTN_BATCHED = 0x1000
DEC_ATTN_STREAM = 0x2000
DEC_ATTN_LOCAL = 0x3000
DEC_TEST_NO_WAIT = 0x100
DEC_TEST_SKIP_ROPE = 0x200
DEC_TEST_APPEND_NEXT = 0x400
DEC_TEST_DROP_SPLIT = 0x800
DEC_ERR_POS = 0x1
DEC_ERR_TOKEN = 0x2
DEC_ERR_SYNC = 0x4
ABI_VERSION = 7
DEC_COUNTER_STRIDE = 16
DEC_STATIC_SCRATCH_BYTES = 4 << 20

c_void_p, c_int32, c_uint32, c_float, c_double, c_int64 = (
    ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_double, ctypes.c_int64)


class dec_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn", c_int32), ("max_ctx", c_int32),
                ("rms_eps", c_float), ("wtype", c_int32), ("ntype", c_int32),
                ("kvtype", c_int32), ("attn_chunk", c_int32), ("flags", c_uint32)]


class dec_mat(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("scales", c_void_p)]


class dec_layer_weights(ctypes.Structure):
    _fields_ = [("attn_norm", c_void_p), ("wqkv", dec_mat), ("wo", dec_mat),
                ("ffn_norm", c_void_p), ("wgate", dec_mat), ("wup", dec_mat), ("wdown", dec_mat)]


class dec_layer_state(ctypes.Structure):
    _fields_ = [("x", c_void_p), ("q", c_void_p), ("attn", c_void_p), ("h", c_void_p),
                ("part", c_void_p), ("counters", c_void_p), ("k_cache", c_void_p),
                ("v_cache", c_void_p), ("pos", c_void_p), ("rope", c_void_p), ("err", c_void_p),
                ("scratch", c_void_p)]


P_DESC = ctypes.POINTER(dec_layer_desc)
P_W = ctypes.POINTER(dec_layer_weights)
P_ST = ctypes.POINTER(dec_layer_state)

# name -> (restype, argtypes); every symbol include/dec_api.h declares
SIGNATURES = {
    "dec_attn_part_floats": (c_int64, [P_DESC]),
    "dec_scratch_floats": (c_int64, [P_DESC]),
    "dec_scratch_kv_offset": (c_int64, [P_DESC]),
    "dec_cache_bytes": (c_int64, [P_DESC]),
    "dec_cache_scale_offset": (c_int64, [P_DESC]),
    "dec_cache_stage_offset": (c_int64, [P_DESC]),
    "dec_rmsnorm_gemv_qkv_rope": (ctypes.c_int, [P_DESC, P_W, P_ST, c_void_p]),
    "dec_attn_splitk": (ctypes.c_int, [P_DESC, P_ST, c_void_p]),
    "dec_attn_partials": (ctypes.c_int, [P_DESC, P_ST, c_void_p]),
    "dec_attn_o_residual": (ctypes.c_int, [P_DESC, dec_mat, P_ST, c_void_p]),
    "dec_gemv_residual": (ctypes.c_int, [P_DESC, dec_mat, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "dec_gated_ffn": (ctypes.c_int, [P_DESC, c_void_p, dec_mat, dec_mat, c_void_p, c_void_p, c_void_p]),
    "dec_gated_ffn_down": (ctypes.c_int, [P_DESC, P_W, P_ST, c_void_p]),
    "dec_layer_step": (ctypes.c_int, [P_DESC, P_W, P_ST, c_void_p]),
    "dec_layer_step_static": (ctypes.c_int, [P_DESC, P_W, P_ST, c_void_p]),
    "dec_lm_head": (ctypes.c_int, [P_DESC, c_int32, c_void_p, dec_mat, c_int32, c_void_p, c_void_p, c_void_p,
                                    c_void_p]),
    "dec_rope_table": (ctypes.c_int, [c_double, c_int32, c_int32, c_void_p, c_void_p]),
    "dec_embed": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dec_advance": (ctypes.c_int, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "dec_last_error": (ctypes.c_char_p, []),
    "dec_abi_version": (ctypes.c_int, []),
}

_lib = None


class DecError(RuntimeError):
    pass


def load():
    """Load libdec.so (built in-tree). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise DecError(f"{LIBPATH} is not built: run `python -m transformer_layer_amd.build`")
    import torch  # noqa: F401  (torch's HIP runtime must be the one in the process)
    lib = ctypes.CDLL(LIBPATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.dec_abi_version() != ABI_VERSION:
        raise DecError("libdec ABI version mismatch")
    _lib = lib
    return lib


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise DecError(f"{name} returned {rc}: {_lib.dec_last_error().decode()}")


def ptr(t) -> int | None:
    """Device address of a tensor (None for None)."""
    return None if t is None else t.data_ptr()


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _s(stream):
    return current_stream() if stream is None else stream


# ---- entry points (same names as the C ABI)

def dec_attn_part_floats(desc: dec_layer_desc) -> int:
    n = load().dec_attn_part_floats(ctypes.byref(desc))
    if n < 0:
        raise DecError(_lib.dec_last_error().decode())
    return n


def dec_scratch_floats(desc: dec_layer_desc) -> int:
    n = load().dec_scratch_floats(ctypes.byref(desc))
    if n < 0:
        raise DecError(_lib.dec_last_error().decode())
    return n


def dec_scratch_kv_offset(desc: dec_layer_desc) -> int:
    return _size("dec_scratch_kv_offset", desc)


def _size(name: str, desc: dec_layer_desc) -> int:
    n = getattr(load(), name)(ctypes.byref(desc))
    if n < 0:
        raise DecError(_lib.dec_last_error().decode())
    return n


def dec_cache_bytes(desc: dec_layer_desc) -> int:
    return _size("dec_cache_bytes", desc)


def dec_cache_scale_offset(desc: dec_layer_desc) -> int:
    return _size("dec_cache_scale_offset", desc)


def dec_cache_stage_offset(desc: dec_layer_desc) -> int:
    return _size("dec_cache_stage_offset", desc)


def dec_rmsnorm_gemv_qkv_rope(desc, weights, state, stream=None) -> None:
    _check(load().dec_rmsnorm_gemv_qkv_rope(ctypes.byref(desc), ctypes.byref(weights),
                                             ctypes.byref(state), _s(stream)), "dec_rmsnorm_gemv_qkv_rope")


def dec_attn_splitk(desc, state, stream=None) -> None:
    _check(load().dec_attn_splitk(ctypes.byref(desc), ctypes.byref(state), _s(stream)), "dec_attn_splitk")


def dec_attn_partials(desc, state, stream=None) -> None:
    _check(load().dec_attn_partials(ctypes.byref(desc), ctypes.byref(state), _s(stream)), "dec_attn_partials")


def dec_attn_o_residual(desc, wo: dec_mat, state, stream=None) -> None:
    _check(load().dec_attn_o_residual(ctypes.byref(desc), wo, ctypes.byref(state), _s(stream)),
           "dec_attn_o_residual")


def dec_gemv_residual(desc, w: dec_mat, rows: int, cols: int, inp: int, x: int, stream=None) -> None:
    _check(load().dec_gemv_residual(ctypes.byref(desc), w, rows, cols, inp, x, _s(stream)), "dec_gemv_residual")


def dec_gated_ffn(desc, ffn_norm: int, wgate: dec_mat, wup: dec_mat, x: int, h: int, stream=None) -> None:
    _check(load().dec_gated_ffn(ctypes.byref(desc), ffn_norm, wgate, wup, x, h, _s(stream)), "dec_gated_ffn")


def dec_gated_ffn_down(desc, weights, state, stream=None) -> None:
    _check(load().dec_gated_ffn_down(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(state),
                                     _s(stream)), "dec_gated_ffn_down")


def dec_layer_step(desc, weights, state, stream=None) -> None:
    _check(load().dec_layer_step(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(state),
                                 _s(stream)), "dec_layer_step")


def dec_layer_step_static(desc, weights, state, stream=None) -> None:
    _check(load().dec_layer_step_static(ctypes.byref(desc), ctypes.byref(weights), ctypes.byref(state),
                                        _s(stream)), "dec_layer_step_static")


def dec_lm_head(desc, head_type: int, final_norm: int, head: dec_mat, vocab: int, x: int, logits: int,
                token: int, stream=None) -> None:
    _check(load().dec_lm_head(ctypes.byref(desc), head_type, final_norm, head, vocab, x, logits, token,
                              _s(stream)), "dec_lm_head")


def dec_rope_table(theta: float, head_dim: int, max_ctx: int, table: int, stream=None) -> None:
    _check(load().dec_rope_table(theta, head_dim, max_ctx, table, _s(stream)), "dec_rope_table")


def dec_embed(embed: int, vocab: int, hidden: int, token: int, x: int, err: int, stream=None) -> None:
    _check(load().dec_embed(embed, vocab, hidden, token, x, err, _s(stream)), "dec_embed")


def dec_advance(pos: int, pos_lo: int, pos_hi: int, tokens, token, stream=None) -> None:
    _check(load().dec_advance(pos, pos_lo, pos_hi, tokens, token, _s(stream)), "dec_advance")


def dec_last_error() -> str:
    return load().dec_last_error().decode()


def dec_abi_version() -> int:
    return load().dec_abi_version()
