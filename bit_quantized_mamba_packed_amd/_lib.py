"""ctypes binding of libdfssm.so: the C structs of include/dfssm.h and the exported functions,
under the same names. Argument marshalling only: every step of the computation runs in the
HIP library. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdfssm.so")

DFSSM_OK = 0
DFSSM_EINVAL = -1
DFSSM_EUNSUPPORTED = -2
DFSSM_EWORKSPACE = -3
DFSSM_EHIP = -4

DFSSM_OP_LAYER_DECODE = 0
DFSSM_NOALLOC_SCRATCH_BYTES = 16 << 20
DFSSM_OP_LAYER_PREFILL = 1
DFSSM_OP_STACK_DECODE = 2
DFSSM_OP_STACK_PREFILL = 3
DFSSM_OP_LM_HEAD = 4

DFSSM_STACK_STATUS_OFFSET = 0
DFSSM_STATUS_OK = 0
DFSSM_STATUS_TIMEOUT = 1

DFSSM_PATH_AUTO = 0
DFSSM_PATH_FLOW = 1
DFSSM_PATH_PER_LAYER = 2
DFSSM_LAUNCH_COOPERATIVE = 0
DFSSM_LAUNCH_ORDINARY = 1

DFSSM_F32 = 0
DFSSM_BF16 = 1

# every symbol include/dfssm.h declares
EXPORTS = ("dfssm_workspace_bytes", "dfssm_layer_decode", "dfssm_layer_decode_noalloc", "dfssm_layer_prefill",
           "dfssm_layer_prefill_ex", "dfssm_stack_prefill_ex",
           "dfssm_stack_decode", "dfssm_stack_decode_ex", "dfssm_stack_prefill", "dfssm_embed", "dfssm_lm_head",
           "dfssm_state_field_words", "dfssm_state_encode", "dfssm_state_decode", "dfssm_dfw_workspace_bytes",
           "dfssm_dfw_project", "dfssm_strerror")


class dfssm_dims(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_inner", C.c_int32), ("d_state", C.c_int32),
                ("headdim", C.c_int32), ("ngroups", C.c_int32), ("d_conv", C.c_int32),
                ("n_in_proj", C.c_int32), ("rank_in", C.c_int32), ("rank_out", C.c_int32),
                ("norm_eps", C.c_float)]


class dfssm_proj(C.Structure):
    _fields_ = [("sign", C.c_void_p), ("row_scale", C.c_void_p), ("lora_dn", C.c_void_p),
                ("lora_dn_scale", C.c_void_p), ("lora_up", C.c_void_p), ("lora_up_scale", C.c_void_p)]


class dfssm_layer_weights(C.Structure):
    _fields_ = [("in_proj", dfssm_proj), ("out_proj", dfssm_proj),
                ("conv_w", C.c_void_p), ("conv_b", C.c_void_p),
                ("dt_bias", C.c_void_p), ("A_log", C.c_void_p), ("D", C.c_void_p),
                ("norm_w", C.c_void_p), ("gnorm_w", C.c_void_p)]


class dfssm_layer_state(C.Structure):
    _fields_ = [("conv", C.c_void_p), ("ssm", C.c_void_p)]


class dfssm_taps(C.Structure):
    _fields_ = [("h_in", C.c_void_p),
                ("in_u", C.c_void_p), ("in_q", C.c_void_p), ("in_s", C.c_void_p),
                ("in_acc", C.c_void_p), ("in_t", C.c_void_p),
                ("out_u", C.c_void_p), ("out_q", C.c_void_p), ("out_s", C.c_void_p),
                ("out_acc", C.c_void_p), ("out_t", C.c_void_p)]


class dfssm_stack_opts(C.Structure):
    _fields_ = [("path", C.c_int32), ("launch", C.c_int32)]


class dfssm_embedding(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("row_scale", C.c_void_p), ("vocab", C.c_int32), ("d_model", C.c_int32)]


class dfssm_head_taps(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("acc", C.c_void_p)]


class dfssm_prefill_opts(C.Structure):
    _fields_ = [("state_codec", C.c_int32), ("reserved", C.c_int32), ("chunk_state_pre", C.c_void_p),
                ("chunk_state_in", C.c_void_p)]


class dfssm_dfw_proj(C.Structure):
    _fields_ = [("planes", C.c_void_p), ("row_scale", C.c_void_p), ("lora_dn", C.c_void_p),
                ("lora_dn_scale", C.c_void_p), ("lora_up", C.c_void_p), ("lora_up_scale", C.c_void_p)]


class dfssm_dfw_taps(C.Structure):
    _fields_ = [("q", C.c_void_p), ("s", C.c_void_p), ("acc", C.c_void_p), ("t", C.c_void_p)]


_lib = None


def load() -> C.CDLL:
    """Load libdfssm.so once; raises if it is missing (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m bit_quantized_mamba_packed_amd.build`")
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    lib.dfssm_workspace_bytes.argtypes = [C.POINTER(dfssm_dims), C.c_int32, C.c_int32, C.c_int32, C.c_int32]
    lib.dfssm_workspace_bytes.restype = C.c_size_t
    lib.dfssm_layer_decode.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                       C.POINTER(dfssm_layer_state), P, P, C.c_int32, P, C.c_size_t,
                                       C.POINTER(dfssm_taps), P]
    lib.dfssm_layer_decode.restype = C.c_int
    lib.dfssm_layer_decode_noalloc.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                               C.POINTER(dfssm_layer_state), P, P, C.c_int32,
                                               C.POINTER(dfssm_taps), P]
    lib.dfssm_layer_decode_noalloc.restype = C.c_int
    lib.dfssm_layer_prefill.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                        C.POINTER(dfssm_layer_state), P, C.c_int32, P, C.c_int32,
                                        C.c_int32, C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps), P]
    lib.dfssm_layer_prefill.restype = C.c_int
    lib.dfssm_layer_prefill_ex.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                           C.POINTER(dfssm_layer_state), P, C.c_int32, P, C.c_int32,
                                           C.c_int32, C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps),
                                           C.POINTER(dfssm_prefill_opts), P]
    lib.dfssm_layer_prefill_ex.restype = C.c_int
    lib.dfssm_stack_decode.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                       C.POINTER(dfssm_layer_state), C.c_int32, P, P, P, C.c_int32,
                                       C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps), P]
    lib.dfssm_stack_decode.restype = C.c_int
    lib.dfssm_stack_decode_ex.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                          C.POINTER(dfssm_layer_state), C.c_int32, P, P, P, C.c_int32,
                                          C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps),
                                          C.POINTER(dfssm_stack_opts), P]
    lib.dfssm_stack_decode_ex.restype = C.c_int
    lib.dfssm_stack_prefill.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                        C.POINTER(dfssm_layer_state), C.c_int32, P, P, C.c_int32, P,
                                        C.c_int32, C.c_int32, C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps), P]
    lib.dfssm_stack_prefill.restype = C.c_int
    lib.dfssm_stack_prefill_ex.argtypes = [C.POINTER(dfssm_dims), C.POINTER(dfssm_layer_weights),
                                           C.POINTER(dfssm_layer_state), C.c_int32, P, P, C.c_int32, P,
                                           C.c_int32, C.c_int32, C.c_int32, P, C.c_size_t, C.POINTER(dfssm_taps),
                                           C.POINTER(dfssm_prefill_opts), P]
    lib.dfssm_stack_prefill_ex.restype = C.c_int
    lib.dfssm_embed.argtypes = [C.POINTER(dfssm_embedding), P, C.c_int32, P, P]
    lib.dfssm_embed.restype = C.c_int
    lib.dfssm_lm_head.argtypes = [C.POINTER(dfssm_embedding), P, C.c_int32, P, P, P, C.c_size_t,
                                  C.POINTER(dfssm_head_taps), P]
    lib.dfssm_lm_head.restype = C.c_int
    lib.dfssm_dfw_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int32]
    lib.dfssm_dfw_workspace_bytes.restype = C.c_size_t
    lib.dfssm_dfw_project.argtypes = [C.POINTER(dfssm_dfw_proj), C.c_int32, C.c_int32, C.c_int32, P, P, C.c_int32,
                                      P, C.c_size_t, C.POINTER(dfssm_dfw_taps), P]
    lib.dfssm_dfw_project.restype = C.c_int
    lib.dfssm_state_field_words.argtypes = [C.c_int32]
    lib.dfssm_state_field_words.restype = C.c_int32
    lib.dfssm_state_encode.argtypes = [C.POINTER(dfssm_dims), P, C.c_int32, P, P, P]
    lib.dfssm_state_encode.restype = C.c_int
    lib.dfssm_state_decode.argtypes = [C.POINTER(dfssm_dims), P, P, C.c_int32, P, P]
    lib.dfssm_state_decode.restype = C.c_int
    lib.dfssm_strerror.argtypes = [C.c_int]
    lib.dfssm_strerror.restype = C.c_char_p
    _lib = lib
    return lib


def _ref(x):
    return None if x is None else C.byref(x)


def dfssm_workspace_bytes(dims: dfssm_dims, op: int, batch: int, seqlen: int = 0, n_layers: int = 0) -> int:
    return int(load().dfssm_workspace_bytes(C.byref(dims), op, batch, seqlen, n_layers))


def dfssm_layer_decode(dims, w, state, x_in, x_out, batch, ws, ws_bytes, taps=None, stream=None) -> int:
    return int(load().dfssm_layer_decode(C.byref(dims), C.byref(w), C.byref(state), x_in, x_out, batch,
                                         ws, ws_bytes, _ref(taps), stream))


def dfssm_layer_decode_noalloc(dims, w, state, x_in, x_out, batch, taps=None, stream=None) -> int:
    return int(load().dfssm_layer_decode_noalloc(C.byref(dims), C.byref(w), C.byref(state), x_in, x_out, batch,
                                                 _ref(taps), stream))


def dfssm_layer_prefill_ex(dims, w, state, x_in, x_dtype, x_out, batch, seqlen, chunk, ws, ws_bytes,
                           taps=None, opts=None, stream=None) -> int:
    return int(load().dfssm_layer_prefill_ex(C.byref(dims), C.byref(w), C.byref(state), x_in, x_dtype, x_out,
                                             batch, seqlen, chunk, ws, ws_bytes, _ref(taps), _ref(opts), stream))


def dfssm_layer_prefill(dims, w, state, x_in, x_dtype, x_out, batch, seqlen, chunk, ws, ws_bytes,
                        taps=None, stream=None) -> int:
    return int(load().dfssm_layer_prefill(C.byref(dims), C.byref(w), C.byref(state), x_in, x_dtype, x_out,
                                          batch, seqlen, chunk, ws, ws_bytes, _ref(taps), stream))


def dfssm_stack_decode(dims, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, ws, ws_bytes,
                       taps=None, stream=None) -> int:
    """layers / states: ctypes arrays (dfssm_layer_weights * n) / (dfssm_layer_state * n)."""
    return int(load().dfssm_stack_decode(C.byref(dims), layers, states, n_layers, final_norm_w, x0, y, batch,
                                         n_steps, ws, ws_bytes, _ref(taps), stream))


def dfssm_stack_decode_ex(dims, layers, states, n_layers, final_norm_w, x0, y, batch, n_steps, ws, ws_bytes,
                          taps=None, opts=None, stream=None) -> int:
    return int(load().dfssm_stack_decode_ex(C.byref(dims), layers, states, n_layers, final_norm_w, x0, y, batch,
                                            n_steps, ws, ws_bytes, _ref(taps), _ref(opts), stream))


def dfssm_stack_prefill_ex(dims, layers, states, n_layers, final_norm_w, x_in, x_dtype, y, batch, seqlen, chunk, ws,
                           ws_bytes, taps=None, opts=None, stream=None) -> int:
    return int(load().dfssm_stack_prefill_ex(C.byref(dims), layers, states, n_layers, final_norm_w, x_in, x_dtype, y,
                                             batch, seqlen, chunk, ws, ws_bytes, _ref(taps), _ref(opts), stream))


def dfssm_stack_prefill(dims, layers, states, n_layers, final_norm_w, x_in, x_dtype, y, batch, seqlen, chunk, ws,
                        ws_bytes, taps=None, stream=None) -> int:
    return int(load().dfssm_stack_prefill(C.byref(dims), layers, states, n_layers, final_norm_w, x_in, x_dtype, y,
                                          batch, seqlen, chunk, ws, ws_bytes, _ref(taps), stream))


def dfssm_embed(emb, tokens, batch, x, stream=None) -> int:
    return int(load().dfssm_embed(C.byref(emb), tokens, batch, x, stream))


def dfssm_lm_head(emb, y, batch, logits, next_tokens, ws, ws_bytes, taps=None, stream=None) -> int:
    return int(load().dfssm_lm_head(C.byref(emb), y, batch, logits, next_tokens, ws, ws_bytes, _ref(taps), stream))


def dfssm_dfw_workspace_bytes(n_in: int, rank: int, batch: int) -> int:
    return int(load().dfssm_dfw_workspace_bytes(n_in, rank, batch))


def dfssm_dfw_project(w, n_out, n_in, rank, x, y, batch, ws, ws_bytes, taps=None, stream=None) -> int:
    return int(load().dfssm_dfw_project(C.byref(w), n_out, n_in, rank, x, y, batch, ws, ws_bytes, _ref(taps),
                                        stream))


def dfssm_state_field_words(d_state: int) -> int:
    return int(load().dfssm_state_field_words(d_state))


def dfssm_state_encode(dims, ssm, batch, fields, stats, stream=None) -> int:
    return int(load().dfssm_state_encode(C.byref(dims), ssm, batch, fields, stats, stream))


def dfssm_state_decode(dims, fields, stats, batch, ssm, stream=None) -> int:
    return int(load().dfssm_state_decode(C.byref(dims), fields, stats, batch, ssm, stream))


def dfssm_strerror(status: int) -> str:
    return load().dfssm_strerror(status).decode()


class DfssmError(RuntimeError):
    pass


def check(status: int, what: str = "dfssm call") -> None:
    if status != DFSSM_OK:
        raise DfssmError(f"{what} failed: {dfssm_strerror(status)} ({status})")
