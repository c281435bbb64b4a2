"""Device-side state of a decode stack and its per-token HIP graph.

PyTorch provides the device memory and the stream; every computation is a
call into libdec. One ``DecodeStack`` holds, on the GPU:

* per layer: the weights in their storage encoding (fp32, bf16 bit patterns,
  or 4-bit nibbles plus fp16 scales), and a key and a value cache
  ``[n_kv][max_ctx][d]`` in the cache type;
* shared by all layers: the residual stream x ``[H]``, the rotated queries,
  the attention output, the SwiGLU output, the attention partials and
  arrival counters, the RoPE table, the position, the current token and the
  device error word.

A token is: x = E[token]; the layers in order; then the position advances (and
the next teacher-forced token is fetched). ``capture`` records exactly that
sequence into one HIP graph (via ``torch.cuda.CUDAGraph``); since the
position lives in device memory the graph replays unchanged.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import lib as L


def _upload(st, dev):
    """A stored tensor (kind f32 / bf16 / q4) as device tensors (data, scales)."""
    if st.kind == "f32":
        return torch.from_numpy(np.ascontiguousarray(st.data, dtype=np.float32)).to(dev), None
    if st.kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(st.data).view(np.int16)).to(dev), None
    if st.kind == "q4":
        return (torch.from_numpy(np.ascontiguousarray(st.data)).to(dev),
                torch.from_numpy(np.ascontiguousarray(st.scales)).to(dev))
    raise ValueError(st.kind)


def _mat(pair) -> L.dec_mat:
    w, s = pair
    return L.dec_mat(w.data_ptr(), None if s is None else s.data_ptr())


class DecodeStack:
    def __init__(self, cfg, n_layers=None, flags=0, attn_chunk=0, device="cuda"):
        L.load()
        self.cfg = cfg
        self.n_layers = cfg.n_layers if n_layers is None else n_layers
        self.dev = torch.device(device)
        c = cfg
        self.desc = L.dec_layer_desc(
            hidden=c.hidden, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
            ffn=c.ffn, max_ctx=c.max_ctx, rms_eps=c.rms_eps, wtype=L.DTYPES[c.wtype],
            ntype=L.DTYPES[c.ntype], kvtype=L.DTYPES[c.kvtype], attn_chunk=attn_chunk, flags=flags)
        dev = self.dev
        f32 = torch.float32
        self.x = torch.zeros(c.hidden, dtype=f32, device=dev)
        self.q = torch.zeros(c.q_dim, dtype=f32, device=dev)
        self.attn = torch.zeros(c.q_dim, dtype=f32, device=dev)
        self.h = torch.zeros(c.ffn, dtype=f32, device=dev)
        self.part = torch.zeros(L.dec_attn_part_floats(self.desc), dtype=f32, device=dev)
        self.counters = torch.zeros(c.n_kv_heads * L.DEC_COUNTER_STRIDE, dtype=torch.int32, device=dev)
        self.scratch = torch.zeros(L.dec_scratch_floats(self.desc), dtype=f32, device=dev)
        self.pos = torch.zeros(1, dtype=torch.int32, device=dev)
        self.token = torch.zeros(1, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.rope = torch.empty(c.max_ctx * c.head_dim, dtype=f32, device=dev)
        L.dec_rope_table(float(c.rope_theta), c.head_dim, c.max_ctx, self.rope.data_ptr())
        shape = (self.n_layers, c.n_kv_heads, c.max_ctx, c.head_dim)
        if c.kvtype == "i8":
            # per layer: int8 codes, one float scale per row, the staged newest row
            nb = L.dec_cache_bytes(self.desc)
            so, go = L.dec_cache_scale_offset(self.desc), L.dec_cache_stage_offset(self.desc)
            ncode = c.n_kv_heads * c.max_ctx * c.head_dim
            nrow = c.n_kv_heads * c.max_ctx
            self.Kraw = torch.zeros((self.n_layers, nb), dtype=torch.uint8, device=dev)
            self.Vraw = torch.zeros((self.n_layers, nb), dtype=torch.uint8, device=dev)
            self.K, self.V = (r[:, :ncode].view(torch.int8).view(shape) for r in (self.Kraw, self.Vraw))
            self.Ks, self.Vs = (r[:, so: so + 4 * nrow].view(torch.float32).view(shape[:3])
                                for r in (self.Kraw, self.Vraw))
            self.Kstage, self.Vstage = (r[:, go: go + 4 * c.n_kv_heads * c.head_dim].view(torch.float32)
                                        .view(self.n_layers, c.n_kv_heads, c.head_dim) for r in (self.Kraw, self.Vraw))
        else:
            kvdt = f32 if c.kvtype == "f32" else torch.int16
            self.K = torch.zeros(shape, dtype=kvdt, device=dev)
            self.V = torch.zeros(shape, dtype=kvdt, device=dev)
        self.w = [None] * self.n_layers
        self.wstruct = [None] * self.n_layers
        self.state = [self._state(l) for l in range(self.n_layers)]
        self.embed = None
        self.tokens_dev = None
        self.head = None
        self.logits = None

    def _state(self, l: int) -> L.dec_layer_state:
        p = L.ptr
        return L.dec_layer_state(
            x=p(self.x), q=p(self.q), attn=p(self.attn), h=p(self.h), part=p(self.part),
            counters=p(self.counters),
            k_cache=p(self.Kraw[l] if self.cfg.kvtype == "i8" else self.K[l]),
            v_cache=p(self.Vraw[l] if self.cfg.kvtype == "i8" else self.V[l]), pos=p(self.pos),
            rope=p(self.rope), err=p(self.err), scratch=p(self.scratch))

    # ---- loading inputs
    def set_layer(self, l: int, lw: dict) -> None:
        d = {k: _upload(v, self.dev) for k, v in lw.items()}
        self.w[l] = d
        self.wstruct[l] = L.dec_layer_weights(
            attn_norm=d["attn_norm"][0].data_ptr(), wqkv=_mat(d["wqkv"]), wo=_mat(d["wo"]),
            ffn_norm=d["ffn_norm"][0].data_ptr(), wgate=_mat(d["wgate"]), wup=_mat(d["wup"]),
            wdown=_mat(d["wdown"]))

    def set_prefill(self, l: int, K, V) -> None:
        n = K.data.shape[1]
        if K.kind == "i8":
            for st, codes, scales in ((K, self.K, self.Ks), (V, self.V, self.Vs)):
                codes[l, :, :n] = torch.from_numpy(np.ascontiguousarray(st.data, dtype=np.int8)).to(self.dev)
                scales[l, :, :n] = torch.from_numpy(np.ascontiguousarray(st.scales, dtype=np.float32)).to(self.dev)
            return
        self.K[l, :, :n] = _upload(K, self.dev)[0]
        self.V[l, :, :n] = _upload(V, self.dev)[0]

    def set_embedding(self, embed) -> None:
        self.embed = _upload(embed, self.dev)[0]

    def set_head(self, final_norm, head) -> None:
        """Final norm weight and LM head [vocab, H] (storage encoding)."""
        self.final_norm = _upload(final_norm, self.dev)[0]
        self.head = _upload(head, self.dev)
        self.head_type = L.DTYPES[head.kind]
        self.logits = torch.zeros(self.cfg.vocab, dtype=torch.float32, device=self.dev)

    def set_pos(self, p: int) -> None:
        self.pos.fill_(int(p))

    def set_token(self, t: int) -> None:
        self.token.fill_(int(t))

    def set_token_list(self, toks) -> None:
        self.tokens_dev = torch.as_tensor(np.asarray(toks, dtype=np.int32), device=self.dev)

    # ---- running
    def layer(self, l: int, stream=None) -> None:
        L.dec_layer_step(self.desc, self.wstruct[l], self.state[l], stream)

    def embed_token(self, stream=None) -> None:
        c = self.cfg
        L.dec_embed(self.embed.data_ptr(), c.vocab, c.hidden, self.token.data_ptr(), self.x.data_ptr(),
                    self.err.data_ptr(), stream)

    def advance(self, pos_lo: int, pos_hi: int, stream=None, use_list=True) -> None:
        toks = L.ptr(self.tokens_dev) if use_list else None
        L.dec_advance(self.pos.data_ptr(), pos_lo, pos_hi, toks, self.token.data_ptr(), stream)

    def head_step(self, stream=None) -> None:
        """Final norm, LM head and greedy argmax: writes the next token."""
        L.dec_lm_head(self.desc, self.head_type, self.final_norm.data_ptr(), _mat(self.head), self.cfg.vocab,
                      self.x.data_ptr(), self.logits.data_ptr(), self.token.data_ptr(), stream)

    def token_step(self, pos_lo=None, pos_hi=None, record=None, stream=None, greedy=False) -> None:
        """One token: embed, every layer, (greedy: LM head and argmax into
        the token), advance. With `record` (a [n_layers+1, H] float tensor) x
        is copied after the embedding and after every layer."""
        self.embed_token(stream)
        if record is not None:
            record[0].copy_(self.x)
        for l in range(self.n_layers):
            self.layer(l, stream)
            if record is not None:
                record[l + 1].copy_(self.x)
        if greedy:
            self.head_step(stream)
        if pos_lo is not None:
            self.advance(pos_lo, pos_hi, stream, use_list=not greedy)

    def capture(self, pos_lo: int, pos_hi: int, greedy: bool = False) -> torch.cuda.CUDAGraph:
        """Record one token (embed, layers, [head], advance) into a HIP graph."""
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.token_step(pos_lo, pos_hi, greedy=greedy)
        return g

    def check_err(self) -> int:
        return int(self.err.item())
