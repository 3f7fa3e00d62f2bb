"""ctypes binding of libleank.so (argument marshalling only).

Every step of the path runs in the HIP library; this module turns torch
tensors into device pointers and the current HIP stream, and raises
LeankError for non-zero status codes.  If the library has not been built
the first call raises RuntimeError -- there is no fallback.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libleank.so")

HEAD_DIM = 128
QUANT_GROUP = 64
PAGE_ROWS = 64
MAX_KV_HEADS = 64
MAX_GROUP = 8
CHANNEL_QUANTUM = 8
NOALLOC_SCRATCH_BYTES = 16 << 20

OK, EINVAL, EUNSUPPORTED, ECAPACITY, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5


class LeankError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class LayerCacheDesc(ctypes.Structure):
    """Mirror of the C struct leank_layer_cache."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("max_ctx", ctypes.c_int64),
        ("mid_capacity", ctypes.c_int64),
        ("n_live", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("kept_count", ctypes.c_int32 * MAX_KV_HEADS),
        ("group_order", ctypes.c_int32 * MAX_KV_HEADS),
        ("k_prun_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("v_mid_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("k_sl_bytes", ctypes.c_uint64),
        ("v_sl_bytes", ctypes.c_uint64),
        ("k_prun_bytes", ctypes.c_uint64),
        ("v_mid_bytes", ctypes.c_uint64),
        ("kept_idx", ctypes.c_void_p),
        ("k_sl", ctypes.c_void_p),
        ("v_sl", ctypes.c_void_p),
        ("k_prun", ctypes.c_void_p),
        ("v_mid", ctypes.c_void_p),
        ("quant_bits", ctypes.c_int32),
        ("quant_group", ctypes.c_int32),
        ("k_q_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("k_qp_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("k_stage_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("v_q_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("v_qp_off", ctypes.c_int64 * MAX_KV_HEADS),
        ("k_q_bytes", ctypes.c_uint64),
        ("k_qp_bytes", ctypes.c_uint64),
        ("k_stage_bytes", ctypes.c_uint64),
        ("v_q_bytes", ctypes.c_uint64),
        ("v_qp_bytes", ctypes.c_uint64),
        ("k_q", ctypes.c_void_p),
        ("k_qp", ctypes.c_void_p),
        ("k_stage", ctypes.c_void_p),
        ("v_q", ctypes.c_void_p),
        ("v_qp", ctypes.c_void_p),
        ("page_rows", ctypes.c_int32),
        ("pages_per_row", ctypes.c_int32),
        ("n_pages", ctypes.c_int64),
        ("page_bytes", ctypes.c_uint64),
        ("pool_bytes", ctypes.c_uint64),
        ("pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
    ]


_lib = None

_SIGNATURES = {
    "leank_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "leank_abi_version": (ctypes.c_int, []),
    "leank_layer_cache_size": (ctypes.c_size_t, []),
    "leank_build_mask": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "leank_build_mask_host": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "leank_plan_layer": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.POINTER(LayerCacheDesc)]),
    "leank_plan_layer_q": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.POINTER(LayerCacheDesc)]),
    "leank_plan_layer_paged": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.POINTER(LayerCacheDesc)]),
    "leank_plan_layer_paged_q": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int32,
                                                ctypes.POINTER(LayerCacheDesc)]),
    "leank_pack_k": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p]),
    "leank_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_int64,
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "leank_workspace_init": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "leank_decode_attn": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "leank_decode_bytes": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]),
    "leank_pack_k_rows": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_void_p]),
    "leank_decode_attn_rows": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                              ctypes.c_void_p]),
    "leank_decode_step": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]),
    "leank_decode_step_rows": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_float, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "leank_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(LayerCacheDesc), ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),
    "leank_pair_retention": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p]),
    "leank_head_hf_ratio": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "leank_rank_correlation": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_double)]),
}


def lib():
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m decode_attention_channel_amd.build` "
                "(there is no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (restype, argtypes) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = restype
            fn.argtypes = argtypes
        if handle.leank_layer_cache_size() != ctypes.sizeof(LayerCacheDesc):
            raise RuntimeError("leank_layer_cache layout mismatch between libleank.so and the binding")
        _lib = handle
    return _lib


def status_string(status):
    return lib().leank_status_string(int(status)).decode()


def check(status, where):
    if status != OK:
        raise LeankError(status, where)


def stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)
