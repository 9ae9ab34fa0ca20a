"""Marshalling of torch-allocated device tensors into the libqd C structs.

torch provides device memory and streams only; `DecodeRunner.step` is one call
of qd_decode_step (every step of the path runs in libqd's kernels) and
`prefill` one call of qd_prefill_block.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, c_int32, c_void_p
from typing import List, Optional

import numpy as np
import torch

from . import qd as Q


def _dtype_code(d: str) -> int:
    return {"f32": Q.QD_F32, "bf16": Q.QD_BF16, "i8": Q.QD_I8}[d]


def make_config(shape) -> Q.qd_config:
    return Q.qd_config(n_layers=shape.n_layers, hidden=shape.hidden, n_q_heads=shape.n_q_heads,
                       n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, ffn=shape.ffn,
                       vocab=shape.vocab, page_size=shape.page_size, rms_eps=shape.rms_eps,
                       rope_theta=shape.rope_theta, qk_norm=int(shape.qk_norm),
                       w_dtype=_dtype_code(shape.w_dtype), kv_dtype=_dtype_code(shape.kv_dtype))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def make_layer(L: dict) -> Q.qd_layer:
    return Q.qd_layer(**{n: _ptr(L.get(n)) for n in Q.LAYER_FIELDS})


def _stream_handle(stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def quantize_int8(w: torch.Tensor, stream=None):
    """One matrix through qd_quantize_rows_int8: (int8 codes [rows][cols], float32
    scales [rows]) on w's device."""
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("quantize_int8 takes a contiguous 2-D matrix")
    code = Q.QD_BF16 if w.dtype == torch.bfloat16 else Q.QD_F32
    q = torch.empty(w.shape, dtype=torch.int8, device=w.device)
    sc = torch.empty(w.shape[0], dtype=torch.float32, device=w.device)
    Q.check(Q.qd_quantize_rows_int8(w.data_ptr(), code, w.shape[0], w.shape[1], q.data_ptr(), sc.data_ptr(),
                                    _stream_handle(stream)))
    return q, sc


def quantize_weights_int8(weights: dict, stream=None) -> dict:
    """The model's weights with every projection matrix and the embedding (and an
    untied lm_head) replaced by int8 codes plus row scales (keys of qd.SCALE_OF);
    norm gains and biases are kept as they are."""
    out = {k: v for k, v in weights.items() if k != "layers"}
    for k in ("embed", "lm_head"):
        if weights.get(k) is not None:
            out[k], out[Q.SCALE_OF[k]] = quantize_int8(weights[k], stream)
    out["layers"] = []
    for L in weights["layers"]:
        M = dict(L)
        for k in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            M[k], M[Q.SCALE_OF[k]] = quantize_int8(L[k], stream)
        out["layers"].append(M)
    return out


def sample(logits: torch.Tensor, temperature: float, top_k: int, top_p: float,
           uniforms: Optional[torch.Tensor], tokens: Optional[torch.Tensor] = None, stream=None,
           raise_on_error=True):
    """qd_sample over the rows of a contiguous float32 [B][V] logits tensor; returns
    the int32 token tensor (or the status when raise_on_error is False)."""
    B, V = logits.shape
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=logits.device)
    st = Q.qd_sample(_ptr(logits), B, V, float(temperature), int(top_k), float(top_p), _ptr(uniforms),
                     _ptr(tokens), _stream_handle(stream))
    if not raise_on_error:
        return st
    Q.check(st)
    return tokens


class DecodeRunner:
    """Holds the C views of one model's weights, KV pools and block table."""

    def __init__(self, shape, weights: dict, k_pools: List[torch.Tensor], v_pools: List[torch.Tensor],
                 block_table: np.ndarray, max_batch: int, max_ctx: int, device="cuda",
                 prefill_tokens: int = 0):
        self.shape = shape
        self.cfg = make_config(shape)
        self._w = weights
        L = len(weights["layers"])
        self.layers = (Q.qd_layer * L)(*[make_layer(x) for x in weights["layers"]])
        lm = weights.get("lm_head")
        emb = weights.get("embed")
        s_emb = weights.get("s_embed")
        s_lm = weights.get("s_lm_head")
        self.weights = Q.qd_weights(embed=_ptr(emb), final_norm=_ptr(weights.get("final_norm")),
                                    lm_head=_ptr(lm if lm is not None else emb),
                                    layers_host=ctypes.cast(self.layers, POINTER(Q.qd_layer)),
                                    s_embed=_ptr(s_emb), s_lm_head=_ptr(s_lm if s_lm is not None else s_emb))
        self.k_pools, self.v_pools = k_pools, v_pools
        self._kp = (c_void_p * L)(*[p.data_ptr() for p in k_pools])
        self._vp = (c_void_p * L)(*[p.data_ptr() for p in v_pools])
        self.bt_host = np.ascontiguousarray(block_table, dtype=np.int32)
        self.bt_dev = torch.from_numpy(self.bt_host).to(device)
        self.kv = Q.qd_kv(k_pages_host=ctypes.cast(self._kp, POINTER(c_void_p)),
                          v_pages_host=ctypes.cast(self._vp, POINTER(c_void_p)),
                          block_table=self.bt_dev.data_ptr(),
                          block_table_host=self.bt_host.ctypes.data_as(POINTER(c_int32)),
                          max_blocks=int(self.bt_host.shape[1]), num_pages=int(k_pools[0].shape[0]))
        nbytes = Q.qd_workspace_bytes(self.cfg, max_batch, max_ctx, 0)
        if prefill_tokens:
            nbytes = max(nbytes, Q.qd_workspace_bytes(self.cfg, 1, max_ctx, prefill_tokens))
        if nbytes == 0:
            raise Q.QdError(Q.QD_ESHAPE, "qd_workspace_bytes returned 0 for this shape")
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        self.ws_ptr = (self.ws.data_ptr() + 255) // 256 * 256
        self.ws_bytes = nbytes

    def step(self, pos_host: np.ndarray, pos_dev: torch.Tensor, tokens: Optional[torch.Tensor] = None,
             x_in: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
             next_tokens: Optional[torch.Tensor] = None, x_out: Optional[torch.Tensor] = None,
             layer_out: Optional[torch.Tensor] = None, stream=None, raise_on_error=True) -> int:
        ph = np.ascontiguousarray(pos_host, dtype=np.int32)
        B = int(ph.shape[0])
        st = Q.qd_decode_step(self.cfg, self.weights, self.kv, B, _ptr(tokens), _ptr(x_in),
                              _ptr(pos_dev), ph.ctypes.data_as(POINTER(c_int32)), _ptr(logits),
                              _ptr(next_tokens), _ptr(x_out), _ptr(layer_out), self.ws_ptr,
                              self.ws_bytes, _stream_handle(stream))
        if raise_on_error:
            Q.check(st)
        return st

    def step_noalloc(self, pos_host: np.ndarray, pos_dev: torch.Tensor, tokens: Optional[torch.Tensor] = None,
                     x_in: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                     next_tokens: Optional[torch.Tensor] = None, x_out: Optional[torch.Tensor] = None,
                     layer_out: Optional[torch.Tensor] = None, stream=None, raise_on_error=True) -> int:
        """The same step through qd_decode_step_noalloc (no workspace argument)."""
        ph = np.ascontiguousarray(pos_host, dtype=np.int32)
        B = int(ph.shape[0])
        st = Q.qd_decode_step_noalloc(self.cfg, self.weights, self.kv, B, _ptr(tokens), _ptr(x_in),
                                      _ptr(pos_dev), ph.ctypes.data_as(POINTER(c_int32)), _ptr(logits),
                                      _ptr(next_tokens), _ptr(x_out), _ptr(layer_out), _stream_handle(stream))
        if raise_on_error:
            Q.check(st)
        return st

    def prefill(self, layer_index: int, n_tokens: int, start_pos: int, x_in: torch.Tensor,
                x_out: torch.Tensor, stream=None, raise_on_error=True) -> int:
        xd = Q.QD_BF16 if x_in.dtype == torch.bfloat16 else Q.QD_F32
        st = Q.qd_prefill_block(self.cfg, self.layers[layer_index], layer_index, self.kv, n_tokens,
                                start_pos, _ptr(x_in), xd, _ptr(x_out), self.ws_ptr, self.ws_bytes,
                                _stream_handle(stream))
        if raise_on_error:
            Q.check(st)
        return st

    def kv_append(self, layer_index: int, pos_host: np.ndarray, pos_dev: torch.Tensor,
                  k: torch.Tensor, v: torch.Tensor, stream=None) -> int:
        ph = np.ascontiguousarray(pos_host, dtype=np.int32)
        st = Q.qd_kv_append(self.cfg, self.kv, layer_index, int(ph.shape[0]), _ptr(pos_dev),
                            ph.ctypes.data_as(POINTER(c_int32)), _ptr(k), _ptr(v),
                            _stream_handle(stream))
        Q.check(st)
        return st
