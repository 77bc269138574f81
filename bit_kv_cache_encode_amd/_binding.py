"""ctypes binding of include/kvq.h.

Argument marshalling only: every step of the encode / attention / dequant
path runs in the HIP kernels of ``libkvq.so``.  There is no CPU fallback; if
the library is missing, loading it raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIB selects another build of the same sources (the host-sanitizer test);
# a missing library raises like the default one
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_ECAPACITY, KVQ_ESTATE, KVQ_EDEVICE, KVQ_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES, NOALLOC_COUNTER_BYTES = 8 << 20, 64 << 10
ATTN_AUTO, ATTN_VALU = 0, 1
KV_LIMIT, Q_LIMIT = 4096.0, 2.0 ** 96
DOMAIN_KV, DOMAIN_Q = 1, 2
MODE_PATTERN, MODE_KVARN, MODE_NSN = 0, 1, 2
F32, BF16 = 0, 1
INDEX_NONE = 0xFF
VTILE = 32

EXPORTS = ("kvq_layout_of", "kvq_cache_init", "kvq_init_patterns", "kvq_set_patterns",
           "kvq_encode_append", "kvq_attn_decode", "kvq_attn_decode_noalloc", "kvq_decode_step",
           "kvq_dequant", "kvq_cache_status", "kvq_strerror",
           "kvq_last_device_error")


class kvq_config(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("max_tokens", C.c_int32), ("bits", C.c_int32),
                ("group", C.c_int32), ("mode", C.c_int32), ("max_patterns", C.c_int32),
                ("pattern_window", C.c_int32), ("v_alpha", C.c_float), ("in_dtype", C.c_int32),
                ("max_splits", C.c_int32), ("shared_patterns", C.c_int32),
                ("k_per_channel", C.c_int32)]


class kvq_layout(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in (
        "k_codes", "v_codes", "k_sz", "v_sz", "k_idx", "v_idx", "k_t16", "v_t16",
        "k_tab", "v_tab", "k_win", "v_win", "ws", "cnt",
        "codes_bytes", "sz_bytes", "idx_bytes", "t16_bytes", "tab_bytes", "win_bytes",
        "ws_bytes", "cnt_bytes", "total")] + [(n, C.c_int32) for n in (
        "token_cap", "n_groups", "record_bytes", "max_splits")] + [
        (n, C.c_uint64) for n in ("k_bsz", "k_tail", "bsz_bytes", "tail_bytes", "k_t2", "v_t2",
                                  "t2_bytes", "status")]


class kvq_cache(C.Structure):
    _fields_ = [("cfg", kvq_config), ("base", C.c_void_p), ("n_tokens", C.c_int32),
                ("n_patterns", C.c_int32), ("win_count", C.c_int32), ("dropped", C.c_int32),
                ("rho", C.c_float), ("attn_kernel", C.c_int32), ("attn_blocks", C.c_int32)]


class KvqError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = lib().kvq_strerror(status).decode()
        extra = ""
        if status == KVQ_EDEVICE:
            extra = f" (hip error {lib().kvq_last_device_error()})"
        super().__init__(f"{call}: {msg}{extra} [status {status}]")
        self.status = status


_lib = None


def lib():
    """Load libkvq.so (built in-tree by ``bit_kv_cache_encode_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m bit_kv_cache_encode_amd.build` (no fallback exists)")
        L = C.CDLL(LIB_PATH)
        P, I = C.c_void_p, C.c_int32
        sig = {
            "kvq_layout_of": (I, [C.POINTER(kvq_config), C.POINTER(kvq_layout)]),
            "kvq_cache_init": (I, [C.POINTER(kvq_cache), C.POINTER(kvq_config), P, C.c_uint64, P]),
            "kvq_init_patterns": (I, [C.POINTER(kvq_cache), P, P, I, I, P]),
            "kvq_set_patterns": (I, [C.POINTER(kvq_cache), P, P, I, P]),
            "kvq_encode_append": (I, [C.POINTER(kvq_cache), P, P, I, I, P]),
            "kvq_attn_decode": (I, [C.POINTER(kvq_cache), P, P, C.c_float, P]),
            "kvq_attn_decode_noalloc": (I, [C.POINTER(kvq_cache), P, P, C.c_float, P]),
            "kvq_decode_step": (I, [C.POINTER(kvq_cache), P, P, P, P, C.c_float, C.c_int32, P]),
            "kvq_dequant": (I, [C.POINTER(kvq_cache), I, I, I, P, P]),
            "kvq_cache_status": (I, [C.POINTER(kvq_cache), C.POINTER(C.c_uint32), I, P]),
            "kvq_strerror": (C.c_char_p, [I]),
            "kvq_last_device_error": (I, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def check(call: str, status: int) -> None:
    if status != KVQ_OK:
        raise KvqError(call, status)


# Raw C-ABI calls, same names as the header (pointers and sizes only).
def kvq_layout_of(cfg: kvq_config) -> kvq_layout:
    out = kvq_layout()
    check("kvq_layout_of", lib().kvq_layout_of(C.byref(cfg), C.byref(out)))
    return out


def kvq_cache_init(cache: kvq_cache, cfg: kvq_config, base: int, nbytes: int, stream: int) -> int:
    return lib().kvq_cache_init(C.byref(cache), C.byref(cfg), base, nbytes, stream)


def kvq_init_patterns(cache, k_ptr, v_ptr, n_tok, n_patterns, stream) -> int:
    return lib().kvq_init_patterns(C.byref(cache), k_ptr, v_ptr, n_tok, n_patterns, stream)


def kvq_set_patterns(cache, k_tab_ptr, v_tab_ptr, n, stream) -> int:
    return lib().kvq_set_patterns(C.byref(cache), k_tab_ptr, v_tab_ptr, n, stream)


def kvq_encode_append(cache, k_ptr, v_ptr, n_new, update_patterns, stream) -> int:
    return lib().kvq_encode_append(C.byref(cache), k_ptr, v_ptr, n_new, update_patterns, stream)


def kvq_attn_decode(cache, q_ptr, out_ptr, sm_scale, stream) -> int:
    return lib().kvq_attn_decode(C.byref(cache), q_ptr, out_ptr, sm_scale, stream)


def kvq_attn_decode_noalloc(cache, q_ptr, out_ptr, sm_scale, stream) -> int:
    return lib().kvq_attn_decode_noalloc(C.byref(cache), q_ptr, out_ptr, sm_scale, stream)


def kvq_decode_step(cache, k_ptr, v_ptr, q_ptr, out_ptr, sm_scale, update_patterns, stream) -> int:
    return lib().kvq_decode_step(C.byref(cache), k_ptr, v_ptr, q_ptr, out_ptr, sm_scale,
                                 update_patterns, stream)


def kvq_dequant(cache, which, tok0, n, out_ptr, stream) -> int:
    return lib().kvq_dequant(C.byref(cache), which, tok0, n, out_ptr, stream)


def kvq_cache_status(cache, flags_ref, clear, stream) -> int:
    return lib().kvq_cache_status(C.byref(cache), flags_ref, clear, stream)


def kvq_strerror(status: int) -> str:
    return lib().kvq_strerror(status).decode()
