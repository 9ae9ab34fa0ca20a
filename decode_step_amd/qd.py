"""ctypes binding of libqd.so (include/qd.h): the same entry points, argument
marshalling only. Every step of the path runs in the library's HIP kernels.

The library must have been built (decode_step_amd/build.py); importing this
module without it raises, so nothing can fall back to a CPU path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_float, c_int32, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqd.so")

QD_OK, QD_EINVAL, QD_ESHAPE, QD_EALIGN, QD_ECAPACITY = 0, -1, -2, -3, -4
QD_EPOSITION, QD_EWORKSPACE, QD_EUNSUPPORTED, QD_EHIP = -5, -6, -7, -8
QD_F32, QD_BF16, QD_I8 = 0, 1, 2
STATUS_NAMES = {0: "QD_OK", -1: "QD_EINVAL", -2: "QD_ESHAPE", -3: "QD_EALIGN", -4: "QD_ECAPACITY",
                -5: "QD_EPOSITION", -6: "QD_EWORKSPACE", -7: "QD_EUNSUPPORTED", -8: "QD_EHIP"}

LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "bq", "bk", "bv", "q_norm", "k_norm",
                "wo", "mlp_norm", "w_gate", "w_up", "w_down",
                "s_q", "s_k", "s_v", "s_o", "s_gate", "s_up", "s_down"]
# int8 models: the row-scale field of each quantized matrix
SCALE_OF = {"wq": "s_q", "wk": "s_k", "wv": "s_v", "wo": "s_o", "w_gate": "s_gate", "w_up": "s_up",
            "w_down": "s_down", "embed": "s_embed", "lm_head": "s_lm_head"}


class qd_config(Structure):
    _fields_ = [("n_layers", c_int32), ("hidden", c_int32), ("n_q_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32),
                ("vocab", c_int32), ("page_size", c_int32), ("rms_eps", c_float),
                ("rope_theta", c_float), ("qk_norm", c_int32), ("w_dtype", c_int32),
                ("kv_dtype", c_int32)]


class qd_layer(Structure):
    _fields_ = [(n, c_void_p) for n in LAYER_FIELDS]


class qd_weights(Structure):
    _fields_ = [("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("layers_host", POINTER(qd_layer)), ("s_embed", c_void_p), ("s_lm_head", c_void_p)]


class qd_kv(Structure):
    _fields_ = [("k_pages_host", POINTER(c_void_p)), ("v_pages_host", POINTER(c_void_p)),
                ("block_table", c_void_p), ("block_table_host", POINTER(c_int32)),
                ("max_blocks", c_int32), ("num_pages", c_int32)]


class qd_decode_plan_info(Structure):
    _fields_ = [("chunk", c_int32), ("splits", c_int32), ("heads_per_wg", c_int32),
                ("matrix_core_attention", c_int32), ("qkv_partials", c_int32),
                ("merge_in_o_proj", c_int32), ("step_kernel", c_int32),
                ("fused_qkv", c_int32)]


EXPORTS = ["qd_workspace_bytes", "qd_decode_plan", "qd_decode_step", "qd_decode_step_noalloc", "qd_prefill_block", "qd_kv_append", "qd_quantize_rows_int8",
           "qd_sample",
           "qd_last_error", "qd_abi_version", "qd_profile_enable", "qd_profile_read",
           "qd_profile_reset"]

(QD_K_EMBED, QD_K_QKV, QD_K_QKV_POST, QD_K_ATTN, QD_K_MERGE, QD_K_O, QD_K_GATEUP, QD_K_DOWN,
 QD_K_LMHEAD, QD_K_ARGMAX, QD_K_PREFILL_GEMM, QD_K_PREFILL_ATTN, QD_K_OTHER, QD_K_STEP) = range(14)


class QdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


ABI_VERSION = 5   # QD_ABI_VERSION of the header this binding follows


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run decode_step_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    P = c_void_p
    lib.qd_workspace_bytes.argtypes = [POINTER(qd_config), c_int32, c_int32, c_int32]
    lib.qd_workspace_bytes.restype = c_size_t
    lib.qd_decode_plan.argtypes = [POINTER(qd_config), c_int32, c_int32, POINTER(qd_decode_plan_info)]
    lib.qd_decode_plan.restype = c_int32
    lib.qd_decode_step.argtypes = [POINTER(qd_config), POINTER(qd_weights), POINTER(qd_kv), c_int32,
                                   P, P, P, POINTER(c_int32), P, P, P, P, P, c_size_t, P]
    lib.qd_decode_step.restype = c_int32
    lib.qd_decode_step_noalloc.argtypes = [POINTER(qd_config), POINTER(qd_weights), POINTER(qd_kv), c_int32,
                                           P, P, P, POINTER(c_int32), P, P, P, P, P]
    lib.qd_decode_step_noalloc.restype = c_int32
    lib.qd_prefill_block.argtypes = [POINTER(qd_config), POINTER(qd_layer), c_int32, POINTER(qd_kv),
                                     c_int32, c_int32, P, c_int32, P, P, c_size_t, P]
    lib.qd_prefill_block.restype = c_int32
    lib.qd_kv_append.argtypes = [POINTER(qd_config), POINTER(qd_kv), c_int32, c_int32, P,
                                 POINTER(c_int32), P, P, P]
    lib.qd_kv_append.restype = c_int32
    lib.qd_quantize_rows_int8.argtypes = [P, c_int32, ctypes.c_int64, c_int32, P, P, P]
    lib.qd_quantize_rows_int8.restype = c_int32
    lib.qd_sample.argtypes = [P, c_int32, c_int32, c_float, c_int32, c_float, P, P, P]
    lib.qd_sample.restype = c_int32
    lib.qd_last_error.argtypes = []
    lib.qd_last_error.restype = c_char_p
    lib.qd_abi_version.argtypes = []
    lib.qd_abi_version.restype = c_int32
    if lib.qd_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.qd_abi_version()}, this binding expects {ABI_VERSION}: "
                          "rebuild the library")
    lib.qd_profile_enable.argtypes = [ctypes.c_uint32]
    lib.qd_profile_enable.restype = c_int32
    lib.qd_profile_read.argtypes = [c_int32, POINTER(c_int32), POINTER(ctypes.c_double)]
    lib.qd_profile_read.restype = c_int32
    lib.qd_profile_reset.argtypes = []
    lib.qd_profile_reset.restype = None
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(status: int) -> None:
    if status != QD_OK:
        raise QdError(status, lib().qd_last_error().decode())


def qd_workspace_bytes(cfg: qd_config, batch: int, max_ctx: int, prefill_tokens: int = 0) -> int:
    return int(lib().qd_workspace_bytes(ctypes.byref(cfg), batch, max_ctx, prefill_tokens))


def qd_decode_step(cfg, weights, kv, batch, tokens, x_in, pos, pos_host, logits, next_tokens,
                   x_out, layer_out, workspace, workspace_bytes, stream) -> int:
    """Raw call; pointer arguments are integers (device addresses) or None."""
    return int(lib().qd_decode_step(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv),
                                    batch, tokens, x_in, pos, pos_host, logits, next_tokens, x_out,
                                    layer_out, workspace, workspace_bytes, stream))


def qd_decode_step_noalloc(cfg, weights, kv, batch, tokens, x_in, pos, pos_host, logits, next_tokens,
                           x_out, layer_out, stream) -> int:
    """Raw call of the workspace-free step (the library's static device scratch)."""
    return int(lib().qd_decode_step_noalloc(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(kv),
                                            batch, tokens, x_in, pos, pos_host, logits, next_tokens, x_out,
                                            layer_out, stream))


QD_NOALLOC_SCRATCH_BYTES = 16 << 20   # include/qd.h


def qd_prefill_block(cfg, layer, layer_index, kv, n_tokens, start_pos, x_in, x_dtype, x_out,
                     workspace, workspace_bytes, stream) -> int:
    return int(lib().qd_prefill_block(ctypes.byref(cfg), ctypes.byref(layer), layer_index,
                                      ctypes.byref(kv), n_tokens, start_pos, x_in, x_dtype, x_out,
                                      workspace, workspace_bytes, stream))


def qd_kv_append(cfg, kv, layer_index, batch, pos, pos_host, k, v, stream) -> int:
    return int(lib().qd_kv_append(ctypes.byref(cfg), ctypes.byref(kv), layer_index, batch, pos,
                                  pos_host, k, v, stream))


def qd_quantize_rows_int8(w, w_dtype, rows, cols, q, scale, stream) -> int:
    """Raw call; pointers are integers (device addresses)."""
    return int(lib().qd_quantize_rows_int8(w, w_dtype, rows, cols, q, scale, stream))


def qd_sample(logits, batch, vocab, temperature, top_k, top_p, uniforms, tokens, stream) -> int:
    """Raw call; pointers are integers (device addresses) or None."""
    return int(lib().qd_sample(logits, batch, vocab, temperature, top_k, top_p, uniforms, tokens, stream))


def qd_decode_plan(cfg: qd_config, batch: int, max_tokens: int) -> qd_decode_plan_info:
    """The attention plan and kernel path of a decode step (host-only query)."""
    out = qd_decode_plan_info()
    check(lib().qd_decode_plan(cfg, batch, max_tokens, ctypes.byref(out)))
    return out


def qd_last_error() -> str:
    return lib().qd_last_error().decode()


def qd_abi_version() -> int:
    return int(lib().qd_abi_version())


def qd_profile_enable(kind_mask: int) -> None:
    check(lib().qd_profile_enable(kind_mask))


def qd_profile_read(kind: int):
    """(launches, total_ms) of the timed launches of one kernel kind."""
    n = c_int32(0)
    ms = ctypes.c_double(0.0)
    check(lib().qd_profile_read(kind, ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def qd_profile_reset() -> None:
    lib().qd_profile_reset()
