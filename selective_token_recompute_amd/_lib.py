"""ctypes binding of libdlm.so: the C ABI of include/dlm.h and include/dlm_ops.h.

Argument marshalling only -- every step of the computation runs in the HIP
kernels behind these calls.  Loading fails loudly when the library is
missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdlm.so")

DLM_OK, DLM_E_INVALID, DLM_E_SIZE, DLM_E_HIP, DLM_E_STATE, DLM_E_UNSUPPORTED, DLM_E_NUMERIC = (
    0, -1, -2, -3, -4, -5, -6)
DLM_FP32, DLM_BF16 = 0, 1
DLM_LOCK_NONE, DLM_LOCK_TEST = 0, 1
DLM_SAMPLER_SEMI_AR, DLM_SAMPLER_SLOWFAST = 0, 1
(DLM_GET_TOKENS, DLM_GET_LOCK_BITS, DLM_GET_COUNTERS, DLM_GET_ROW_SEQ, DLM_GET_ROW_POS,
 DLM_GET_ARGMAX, DLM_GET_CONF, DLM_GET_KL, DLM_GET_HAS_KL, DLM_GET_LSE, DLM_GET_LOGITS,
 DLM_GET_ROW_REAL, DLM_GET_KCACHE, DLM_GET_VCACHE, DLM_GET_FROZEN, DLM_GET_SF_STATE,
 DLM_GET_HAS_PREV, DLM_GET_DRIFT, DLM_GET_REFRESH) = range(19)
SF_STATE_INTS = 16
KCLASSES = ["compact", "embed_norm", "rmsnorm", "gemm_qkv", "rope_kv", "attention", "gemm_o",
            "gemm_gate_up", "gemm_down", "gemm_lm_head", "vocab_stats", "commit_lock"]
DLM_EPI_STORE_F32, DLM_EPI_RESID_ADD, DLM_EPI_SWIGLU, DLM_EPI_LOGITS = 0, 1, 2, 3

# every symbol the headers declare
EXPORTS = [
    "dlm_state_bytes", "dlm_step_init", "dlm_step", "dlm_lock_update", "dlm_get",
    "dlm_last_step_info", "dlm_destroy", "dlm_error_string", "dlm_set_timing",
    "dlm_read_timing", "dlm_op_compact", "dlm_op_embed_rmsnorm", "dlm_op_rmsnorm",
    "dlm_op_gemm_ws_bytes", "dlm_op_gemm", "dlm_op_gemm_num_configs", "dlm_op_gemm_config",
    "dlm_op_gemm_qkv", "dlm_op_rope_table", "dlm_op_rope_scatter",
    "dlm_op_attention_ws_bytes", "dlm_op_attention", "dlm_op_attention_config_ws_bytes",
    "dlm_op_attention_config", "dlm_op_vocab_ws_bytes",
    "dlm_op_vocab_stats", "dlm_op_lm_head_stats_ws_bytes", "dlm_op_lm_head_stats",
    "dlm_op_commit_lock", "dlm_op_slowfast_commit", "dlm_op_gemm_noalloc_max_bytes",
    "dlm_op_gemm_noalloc", "dlm_op_attention_num_layouts", "dlm_op_attention_layout_ws_bytes",
    "dlm_op_attention_layout", "dlm_debug_poison",
    "dlm_checkpoint_bytes", "dlm_checkpoint_save", "dlm_checkpoint_load",
]

i32 = ctypes.c_int32
f32 = ctypes.c_float
vp = ctypes.c_void_p
sz = ctypes.c_size_t


class dlm_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", i32), ("d_model", i32), ("n_heads", i32), ("n_kv_heads", i32),
                ("head_dim", i32), ("d_ff", i32), ("vocab", i32), ("mask_id", i32),
                ("rope_base", f32), ("rms_eps", f32), ("dtype", i32)]


class dlm_weights(ctypes.Structure):
    _fields_ = [("tok_emb", vp), ("final_norm", vp), ("lm_head", vp),
                ("attn_norm", ctypes.POINTER(vp)), ("w_qkv", ctypes.POINTER(vp)),
                ("w_o", ctypes.POINTER(vp)), ("ffn_norm", ctypes.POINTER(vp)),
                ("w_gate", ctypes.POINTER(vp)), ("w_up", ctypes.POINTER(vp)),
                ("w_down", ctypes.POINTER(vp))]


class dlm_run_desc(ctypes.Structure):
    _fields_ = [("batch", i32), ("seq_len", i32), ("prompt_len", i32), ("steps", i32),
                ("block_len", i32), ("kl_eps", f32), ("conf_tau", f32), ("n_consec", i32),
                ("kl_dir", i32), ("lock_prompt_after_first_step", i32), ("lock_policy", i32),
                ("sampler", i32), ("sf_k", i32), ("sf_kmax", i32), ("sf_whist", i32),
                ("sf_tau_conv", f32), ("sf_tau_high", f32), ("sf_var", f32),
                ("refresh_budget", i32), ("refresh_eps", f32)]


class dlm_override(ctypes.Structure):
    _fields_ = [("commit_seq", vp), ("commit_pos", vp), ("commit_tok", vp), ("n_commit", i32),
                ("lock_bits", vp), ("counters", vp)]


class DlmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {error_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m selective_token_recompute_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.dlm_state_bytes.restype = sz
        L.dlm_state_bytes.argtypes = [P(dlm_model_desc), P(dlm_run_desc)]
        L.dlm_step_init.argtypes = [P(dlm_model_desc), P(dlm_weights), P(dlm_run_desc), vp, vp,
                                    sz, vp, P(vp)]
        L.dlm_step.argtypes = [vp, P(i32)]
        L.dlm_lock_update.argtypes = [vp, P(dlm_override)]
        L.dlm_get.argtypes = [vp, i32, P(vp), P(ctypes.c_int64)]
        L.dlm_last_step_info.argtypes = [vp, P(i32), P(i32), P(ctypes.c_double)]
        L.dlm_destroy.argtypes = [vp]
        L.dlm_debug_poison.argtypes = [vp]
        L.dlm_checkpoint_bytes.restype = sz
        L.dlm_checkpoint_bytes.argtypes = [vp]
        L.dlm_checkpoint_save.argtypes = [vp, vp, sz]
        L.dlm_checkpoint_load.argtypes = [vp, vp, sz]
        L.dlm_error_string.restype = ctypes.c_char_p
        L.dlm_error_string.argtypes = [ctypes.c_int]
        L.dlm_set_timing.argtypes = [vp, i32]
        L.dlm_read_timing.argtypes = [vp, i32, P(ctypes.c_double), P(ctypes.c_int64),
                                      P(ctypes.c_double), P(ctypes.c_double)]
        L.dlm_op_compact.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp]
        L.dlm_op_embed_rmsnorm.argtypes = [i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp,
                                           vp, vp, vp]
        L.dlm_op_rmsnorm.argtypes = [i32, i32, i32, f32, vp, vp, vp, vp]
        L.dlm_op_gemm_ws_bytes.restype = sz
        L.dlm_op_gemm_ws_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.dlm_op_gemm.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                  sz, vp]
        L.dlm_op_attention_layout_ws_bytes.restype = sz
        L.dlm_op_attention_layout_ws_bytes.argtypes = [i32] * 9
        L.dlm_op_attention_layout.argtypes = [i32] * 7 + [vp] * 5 + [i32, i32, vp, sz, vp]
        L.dlm_op_gemm_noalloc_max_bytes.restype = sz
        L.dlm_op_gemm_noalloc_max_bytes.argtypes = []
        L.dlm_op_gemm_noalloc.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32,
                                          i32, vp]
        L.dlm_op_gemm_config.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, i32,
                                         i32, i32, vp, sz, vp]
        L.dlm_op_gemm_qkv.argtypes = [i32] * 5 + [vp] * 8 + [i32, vp]
        L.dlm_op_rope_table.argtypes = [i32, i32, f32, vp, vp]
        L.dlm_op_rope_scatter.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                          vp, vp]
        L.dlm_op_attention_ws_bytes.restype = sz
        L.dlm_op_attention_ws_bytes.argtypes = [i32] * 7
        L.dlm_op_attention.argtypes = [i32] * 7 + [vp] * 5 + [vp, sz, vp]
        L.dlm_op_attention_config_ws_bytes.restype = sz
        L.dlm_op_attention_config_ws_bytes.argtypes = [i32] * 8
        L.dlm_op_attention_config.argtypes = [i32] * 7 + [vp] * 5 + [i32] * 5 + [vp, sz, vp]
        L.dlm_op_vocab_ws_bytes.restype = sz
        L.dlm_op_vocab_ws_bytes.argtypes = [i32, i32]
        L.dlm_op_vocab_stats.argtypes = [i32, i32, i32, i32, i32] + [vp] * 14 + [sz, vp]
        L.dlm_op_lm_head_stats_ws_bytes.restype = sz
        L.dlm_op_lm_head_stats_ws_bytes.argtypes = [i32] * 4
        L.dlm_op_lm_head_stats.argtypes = ([i32] * 3 + [vp] * 5 + [i32] * 3 + [vp] * 10 +
                                           [i32, vp, sz, vp])
        L.dlm_op_commit_lock.argtypes = ([i32] * 10 + [f32, f32, i32, i32] + [vp] * 11 + [vp])
        L.dlm_op_slowfast_commit.argtypes = [i32] * 7 + [f32] * 3 + [vp] * 9
        _lib = L
    return _lib


def error_string(status: int) -> str:
    return lib().dlm_error_string(status).decode()


def check(status: int, what: str) -> None:
    if status != DLM_OK:
        raise DlmError(status, what)
