"""ctypes declarations of the libtt C ABI (include/tt.h).

Loading fails loudly when the library has not been built: there is no CPU or
PyTorch fallback for any call.
"""

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# TT_LIB_PATH: another build of the same library (the host-sanitized one the
# CPU ABI tests run against); by default the in-tree libtt.so
LIB_PATH = os.environ.get("TT_LIB_PATH") or os.path.join(_PKG, "libtt.so")

vp = C.c_void_p
i32 = C.c_int
f32 = C.c_float
sz = C.c_size_t
i64 = C.c_int64
cstr = C.c_char_p


class tt_block_cfg(C.Structure):
    _fields_ = [("B", i32), ("T", i32), ("C", i32), ("NH", i32), ("F", i32),
                ("mode", i32), ("ln_eps", f32)]


_BLOCK_W = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
            "ln2_g", "ln2_b", "w_fc", "b_fc", "w_fcp", "b_fcp"]


class tt_block_w(C.Structure):
    _fields_ = [(n, vp) for n in _BLOCK_W]


class tt_block_g(C.Structure):
    _fields_ = [(n, vp) for n in _BLOCK_W]


class tt_param(C.Structure):
    _fields_ = [("w", vp), ("g", vp), ("m", vp), ("v", vp), ("w_lowp", vp),
                ("n", sz), ("wd_mult", f32)]


class tt_prof_entry(C.Structure):
    _fields_ = [("name", C.c_char_p), ("calls", i32), ("ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


class tt_model_cfg(C.Structure):
    _fields_ = [("L", i32), ("C", i32), ("NH", i32), ("F", i32), ("V", i32),
                ("V_pad", i32), ("T_max", i32), ("B_max", i32), ("mode", i32),
                ("ln_eps", f32)]


P = C.POINTER
SIGS = {
    "tt_ctx_create": (i32, [i32, vp, sz, vp, P(vp)]),
    "tt_ctx_destroy": (None, [vp]),
    "tt_ctx_set_stream": (i32, [vp, vp]),
    "tt_ctx_alloc": (i32, [vp, sz, sz, P(vp)]),
    "tt_ctx_mark": (i32, [vp]),
    "tt_ctx_reset": (i32, [vp]),
    "tt_ctx_usage": (i32, [vp, P(sz), P(sz)]),
    "tt_ctx_sync": (i32, [vp]),
    "tt_strerror": (C.c_char_p, [i32]),
    "tt_ctx_last_error": (C.c_char_p, [vp]),
    "tt_ctx_profile": (i32, [vp, i32]),
    "tt_ctx_profile_report": (i32, [vp, P(tt_prof_entry), P(i32)]),
    "tt_linear_fwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp]),
    "tt_linear_bwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32]),
    "tt_layernorm_fwd": (i32, [vp, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp]),
    "tt_layernorm_bwd": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
    "tt_layernorm_bwd_workspace": (i32, [i32, i32, P(sz)]),
    "tt_layernorm_bwd_noalloc": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
    "tt_gelu_fwd": (i32, [vp, i32, sz, vp, vp]),
    "tt_gelu_bwd": (i32, [vp, i32, sz, vp, vp, vp]),
    "tt_attn_fwd": (i32, [vp, i32, i32, i32, i32, i32, vp, vp, vp]),
    "tt_attn_bwd": (i32, [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]),
    "tt_ce_fwdbwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, f32]),
    "tt_embed_fwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
    "tt_embed_bwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp]),
    "tt_adamw_step": (i32, [vp, P(tt_param), i32, f32, f32, f32, f32, f32, i32]),
    "tt_sgd_step": (i32, [vp, vp, vp, sz, f32]),
    "tt_cast_bf16": (i32, [vp, sz, vp, vp]),
    "tt_block_saved_create": (i32, [vp, P(tt_block_cfg), P(vp)]),
    "tt_block_saved_destroy": (None, [vp]),
    "tt_block_fwd": (i32, [vp, P(tt_block_cfg), P(tt_block_w), vp, vp, vp]),
    "tt_block_bwd": (i32, [vp, P(tt_block_cfg), P(tt_block_w), vp, vp, vp, P(tt_block_g)]),
    "tt_lmhead_ce_fwdbwd": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
    "tt_model_create": (i32, [vp, P(tt_model_cfg), P(vp)]),
    "tt_model_destroy": (None, [vp]),
    "tt_model_param_table": (i32, [vp, P(tt_param), P(i32)]),
    "tt_model_num_params": (i32, [vp, P(sz), P(sz)]),
    "tt_model_refresh_shadow": (i32, [vp]),
    "tt_train_step": (i32, [vp, vp, i32, i32, vp, vp, f32, f32, f32, f32, f32, i32, vp, vp]),
    "tt_model_fwd_bwd": (i32, [vp, vp, i32, i32, vp, vp, vp]),
    "tt_model_adamw": (i32, [vp, vp, f32, f32, f32, f32, f32, i32]),
    "tt_model_loss_scale_set": (i32, [vp, vp, f32, i32, f32, f32]),
    "tt_model_loss_scale_get": (i32, [vp, vp, P(f32), P(i32), P(i32)]),
    "tt_model_clip_grad_norm": (i32, [vp, vp, f32, vp]),
    "tt_clip_grad_norm": (i32, [vp, vp, sz, f32, vp]),
    "tt_model_save": (i32, [vp, vp, cstr, i64]),
    "tt_model_load_state": (i32, [vp, vp, cstr, P(i64)]),
    "tt_mlp_step": (i32, [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp,
                          vp]),
    "tt_graph_create": (i32, [vp, P(vp)]),
    "tt_graph_destroy": (None, [vp]),
    "tt_graph_leaf": (i32, [vp, i32, i32, vp, vp, P(i32)]),
    "tt_graph_matmul": (i32, [vp, i32, i32, P(i32)]),
    "tt_graph_add": (i32, [vp, i32, i32, P(i32)]),
    "tt_graph_gelu": (i32, [vp, i32, P(i32)]),
    "tt_graph_softmax": (i32, [vp, i32, P(i32)]),
    "tt_graph_cross_entropy": (i32, [vp, i32, vp, P(i32)]),
    "tt_graph_forward": (i32, [vp, i32]),
    "tt_graph_backward": (i32, [vp, i32]),
    "tt_graph_zero_grad": (i32, [vp]),
    "tt_graph_capture_sgd_step": (i32, [vp, i32, f32]),
    "tt_graph_step": (i32, [vp]),
    "tt_graph_tensor": (i32, [vp, i32, P(vp), P(vp), P(i32), P(i32)]),
    "tt_argmax": (i32, [vp, i32, i32, i32, i32, vp, vp]),
    "tt_kvcache_create": (i32, [vp, vp, i32, P(vp)]),
    "tt_kvcache_destroy": (None, [vp]),
    "tt_model_prefill": (i32, [vp, vp, vp, i32, i32, vp, vp, vp]),
    "tt_model_decode": (i32, [vp, vp, vp, i32, i32, vp, vp, vp]),
    "tt_probe_mfma": (i32, [vp, i32, i32, i32, P(C.c_double)]),
    "tt_probe_hbm": (i32, [vp, vp, sz, i32, P(C.c_double)]),
    "tt_probe_lds": (i32, [vp, i32, P(C.c_double), P(C.c_double)]),
    "tt_probe_lds_load": (i32, [vp, vp, sz, i32, P(C.c_double)]),
    "tt_probe_issue": (i32, [vp, i32, P(C.c_double), P(C.c_double)]),
}

_lib = None


def load():
    """Load libtt.so once; raise if it is missing (build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libtt.so not found at {LIB_PATH}: build it with "
                "`python -m autograd_transformer_amd.build` (no fallback exists)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
