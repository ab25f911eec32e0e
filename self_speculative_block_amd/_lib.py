"""ctypes declarations of the C ABI in include/ssb.h (argument marshalling only)."""

import ctypes
import os

from .build import LIB

SSB_OK, SSB_EINVAL, SSB_ENOKV, SSB_EHIP, SSB_ESTATE, SSB_ENOMEM = 0, -1, -2, -3, -4, -5
SSB_F32, SSB_BF16 = 0, 1
SSB_FEAT_SAMPLE = 1
SSB_MAX_BATCH = 64
SSB_MAX_BLOCK = 64
SSB_PROFILE_IN_GRAPH = 0x100
KERNEL_KINDS = {"qkv": 0, "attention": 1, "combine": 2, "o": 3, "gate_up": 4, "down": 5, "lm_head": 6, "argmax": 7,
                "reduce": 8, "tail": 9}

c_int, c_float, c_double, c_size_t = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
c_void_p = ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_f32 = ctypes.POINTER(ctypes.c_float)


class SsbConfig(ctypes.Structure):
    _fields_ = [(n, c_int) for n in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "ffn",
                                      "vocab", "mask_id", "eos_id", "block_B", "page_tokens",
                                      "max_rows", "max_positions")] + \
               [("rms_eps", c_float), ("rope_theta", c_float), ("dtype", c_int), ("max_batch", c_int),
                ("features", c_int)]


class SsbWeights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("final_norm", c_void_p),
                ("attn_norm", ctypes.POINTER(c_void_p)), ("mlp_norm", ctypes.POINTER(c_void_p)),
                ("wq", ctypes.POINTER(c_void_p)), ("wk", ctypes.POINTER(c_void_p)),
                ("wv", ctypes.POINTER(c_void_p)), ("wo", ctypes.POINTER(c_void_p)),
                ("wg", ctypes.POINTER(c_void_p)), ("wu", ctypes.POINTER(c_void_p)),
                ("wd", ctypes.POINTER(c_void_p))]


class SsbStats(ctypes.Structure):
    _fields_ = [("rounds", c_int), ("forwards", c_int), ("tokens", c_int), ("accepted", c_int),
                ("decode_us", c_double), ("prefill_us", c_double), ("cache_forwards", c_int)]


SSB_SERVE_AR, SSB_SERVE_SPEC = 0, 1
SSB_DEBUG_POISON = 1
SSB_DEBUG_UNFUSED = 2


class SsbRequest(ctypes.Structure):
    _fields_ = [("prefix_dev", c_void_p), ("P", c_int), ("max_len", c_int), ("cont_dev", c_void_p),
                ("cont_len", c_int), ("astar", c_void_p), ("n_astar", c_int), ("out", c_void_p),
                ("n_out", c_int), ("rounds", c_int), ("finish_us", c_double)]


class SsbServeStats(ctypes.Structure):
    _fields_ = [("steps", c_int), ("prefills", c_int), ("tokens", ctypes.c_longlong), ("total_us", c_double),
                ("prefill_us", c_double), ("decode_us", c_double), ("mean_running", c_double)]


# name -> (restype, argtypes)
SIGNATURES = {
    "ssb_last_error": (ctypes.c_char_p, []),
    "ssb_check_config": (c_int, [ctypes.POINTER(SsbConfig)]),
    "ssb_init_model": (c_int, [ctypes.POINTER(SsbConfig), ctypes.POINTER(SsbWeights), c_void_p,
                               ctypes.POINTER(c_void_p)]),
    "ssb_free_model": (None, [c_void_p]),
    "ssb_model_memory": (c_int, [c_void_p, ctypes.POINTER(c_size_t), ctypes.POINTER(c_size_t)]),
    "ssb_pool_bytes": (c_int, [c_void_p, c_int, ctypes.POINTER(c_size_t)]),
    "ssb_pool_init": (c_int, [c_void_p, c_void_p, c_size_t, c_int, ctypes.POINTER(c_void_p)]),
    "ssb_pool_free": (None, [c_void_p]),
    "ssb_pool_free_pages": (c_int, [c_void_p, ctypes.POINTER(c_int)]),
    "ssb_kv_create": (c_int, [c_void_p, c_int, ctypes.POINTER(c_void_p)]),
    "ssb_kv_free": (None, [c_void_p]),
    "ssb_kv_reset": (c_int, [c_void_p]),
    "ssb_kv_rewind": (c_int, [c_void_p, c_int, ctypes.c_int32]),
    "ssb_kv_state": (c_int, [c_void_p, ctypes.POINTER(c_int), P_i32, ctypes.POINTER(c_int)]),
    "ssb_prefill": (c_int, [c_void_p, c_void_p, c_void_p, c_int, P_i32, c_void_p]),
    "ssb_round_noalloc": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, P_i32, P_i32, P_i32, c_void_p]),
    "ssb_round": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p, P_i32, P_i32, P_i32, c_void_p,
                          c_void_p, c_void_p]),
    "ssb_ar_step": (c_int, [c_void_p, c_void_p, P_i32, c_void_p, c_void_p]),
    "ssb_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_void_p, c_int, P_i32,
                           c_int, P_i32, P_i32, ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_decode_ar": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, P_i32, P_i32,
                              ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_set_debug": (c_int, [c_void_p, c_int]),
    "ssb_kv_poison": (c_int, [c_void_p, c_int, c_int, c_void_p]),
    "ssb_round_batch": (c_int, [c_void_p, ctypes.POINTER(c_void_p), c_int, c_int, P_i32, c_void_p, P_i32,
                                P_i32, P_i32, c_void_p, c_void_p, c_void_p]),
    "ssb_round_sample": (c_int, [c_void_p, c_void_p, c_int, c_int, c_float, c_void_p, P_i32, P_i32, P_i32,
                                 c_void_p, c_void_p, c_void_p]),
    "ssb_decode_sample": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_float, c_int, c_void_p, c_int,
                                  P_i32, P_i32, ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_decode_ar_sample": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_float, c_int, c_void_p, P_i32, P_i32,
                                     ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_round_multistep": (c_int, [c_void_p, c_void_p, c_int, c_int, c_float, c_int, P_i32, P_i32, P_i32, P_i32,
                                    c_void_p, c_void_p]),
    "ssb_decode_multistep": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_float, c_int, P_i32,
                                     P_i32, ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_ar_step_batch": (c_int, [c_void_p, ctypes.POINTER(c_void_p), c_int, P_i32, c_void_p]),
    "ssb_serve": (c_int, [c_void_p, c_void_p, ctypes.POINTER(SsbRequest), c_int, c_int, c_int, c_int, c_int,
                          ctypes.POINTER(SsbServeStats), c_void_p]),
    "ssb_dd_block": (c_int, [c_void_p, c_void_p, c_int, c_float, c_int, c_int, P_i32, P_i32, P_i32, P_i32,
                             P_f32, P_i32, c_void_p, c_void_p]),
    "ssb_decode_dd": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_float, c_int, P_i32, P_i32,
                              ctypes.POINTER(SsbStats), c_void_p]),
    "ssb_profile_kernel": (c_int, [c_void_p, c_int]),
    "ssb_profile_read": (c_int, [c_void_p, ctypes.POINTER(c_double), ctypes.POINTER(ctypes.c_longlong), c_int]),
    "ssb_forward_tokens": (c_int, [c_void_p, c_void_p, P_i32, c_int, c_int, c_void_p, P_i32, P_f32, P_f32,
                                   c_void_p]),
}

_lib = None


class SsbError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"ssb error {code}: {msg}")
        self.code = code


def load():
    """Load the built library; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError(f"{LIB} is missing: build it with __graft_entry__.build() "
                          "(python -m self_speculative_block_amd.build)")
    lib = ctypes.CDLL(LIB)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code):
    if code != SSB_OK:
        raise SsbError(code, load().ssb_last_error().decode(errors="replace"))
    return code
