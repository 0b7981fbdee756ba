"""ctypes declarations of include/llama_block.h (argument marshalling only)."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_block.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "llama_block.h")

LLAMA_OK, LLAMA_ERR_INVALID_ARG, LLAMA_ERR_UNSUPPORTED, LLAMA_ERR_CAPACITY, LLAMA_ERR_HIP = 0, -1, -2, -3, -4
LLAMA_F32, LLAMA_BF16 = 0, 1
LLAMA_W_DENSE, LLAMA_W_Q4 = 0, 1
LLAMA_DIAG_ATTN, LLAMA_DIAG_H, LLAMA_DIAG_FFN = 0, 1, 2

STATUS_NAMES = {0: "LLAMA_OK", -1: "LLAMA_ERR_INVALID_ARG", -2: "LLAMA_ERR_UNSUPPORTED",
                -3: "LLAMA_ERR_CAPACITY", -4: "LLAMA_ERR_HIP"}


class llama_block_config(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32), ("ffn_dim", C.c_int32),
                ("norm_eps", C.c_float), ("rope_theta", C.c_float), ("rope_traditional", C.c_int32),
                ("act_dtype", C.c_int32), ("weight_format", C.c_int32), ("group_size", C.c_int32),
                ("max_seq", C.c_int32), ("sliding_window", C.c_int32)]


class llama_linear(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scales", C.c_void_p), ("biases", C.c_void_p)]


class llama_block_weights(C.Structure):
    _fields_ = [("attention_norm", C.c_void_p), ("ffn_norm", C.c_void_p)] + \
        [(n, llama_linear) for n in ("wq", "wk", "wv", "wo", "w1", "w2", "w3")]


class llama_kvcache_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("max_batch", C.c_int32), ("max_seq", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32), ("dtype", C.c_int32)]


P, I32, SZ, F32 = C.c_void_p, C.c_int32, C.c_size_t, C.c_float
PP = C.POINTER(C.c_void_p)
PI32 = C.POINTER(C.c_int32)

# name -> (restype, argtypes), exactly the entry points of include/llama_block.h
SIGNATURES = {
    "llama_block_weight_bytes": (SZ, [C.POINTER(llama_block_config)]),
    "llama_block_create": (I32, [C.POINTER(llama_block_config), C.POINTER(llama_block_weights), P, SZ, P, PP]),
    "llama_block_destroy": (None, [P]),
    "llama_scratch_bytes": (SZ, [C.POINTER(llama_block_config), I32, I32, I32]),
    "llama_block_prefill": (I32, [P, P, I32, P, P, I32, I32, P, SZ, P]),
    "llama_block_prefill_ragged": (I32, [P, P, I32, P, P, I32, PI32, P, SZ, P]),
    "llama_block_decode": (I32, [P, P, I32, P, P, I32, P, SZ, P]),
    "llama_block_decode_noalloc": (I32, [P, P, I32, P, P, I32, P]),
    "llama_block_diag": (I32, [P, P, I32, I32, PP]),
    "llama_block_set_diag": (I32, [P, I32]),
    "llama_block_profile_start": (I32, [P, I32, C.c_uint32]),
    "llama_block_profile_read": (I32, [P, C.POINTER(C.c_float), I32, PI32, PI32]),
    "llama_kvcache_bytes": (SZ, [C.POINTER(llama_kvcache_config)]),
    "llama_kvcache_alloc": (I32, [C.POINTER(llama_kvcache_config), P, SZ, P, PP]),
    "llama_kvcache_free": (None, [P]),
    "llama_kvcache_set_block_table": (I32, [P, PI32, P]),
    "llama_kvcache_set_lens": (I32, [P, I32, PI32, I32, P]),
    "llama_kvcache_get_lens": (I32, [P, I32, PI32, I32]),
    "llama_kvcache_write": (I32, [P, I32, I32, I32, I32, P, P, P]),
    "llama_kvcache_read": (I32, [P, I32, I32, I32, I32, P, P, P]),
    "llama_embed": (I32, [P, I32, I32, I32, P, I32, P, P]),
    "llama_head_scratch_bytes": (SZ, [I32, I32, I32]),
    "llama_lm_head_argmax": (I32, [C.POINTER(llama_linear), I32, I32, I32, P, F32, P, I32, I32, I32, P, P, P, SZ, P]),
    "llama_sample": (I32, [P, I32, I32, F32, F32, P, P, P]),
    "llama_stack_create": (I32, [C.POINTER(C.c_void_p), I32, P, I32, P, C.POINTER(llama_linear), PP]),
    "llama_stack_destroy": (None, [P]),
    "llama_stack_set_sampling": (I32, [P, F32, F32, P]),
    "llama_stack_scratch_bytes": (SZ, [P, I32, I32]),
    "llama_stack_generate": (I32, [P, P, P, I32, I32, P, P, P, SZ, I32, P]),
    "llama_stack_generate_recompute": (I32, [P, P, P, I32, I32, P, P, P, SZ, P]),
    "llama_probe_mfma_bf16": (I32, [I32, I32, P, P]),
    "llama_last_error": (C.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the HIP library; raise if it was not built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m decoder_block_rmsnorm_amd.build` "
                           f"(or __graft_entry__.build()); the decoder block has no non-HIP implementation")
    # torch's HIP runtime first: the library then binds to the copy torch
    # already holds (two runtimes in one process do not share devices)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
