"""CPU oracle for the KV-cache encode / decode-attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``bit_kv_cache_encode_amd``) never imports, links or runs anything here, and
this package shares no code with it.

The arithmetic lives in ``kvqref.c`` (plain C, one IEEE binary32 operation per
step for the encode, binary64 for attention and k-means); this module only
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvqref.c")
# KVQREF_LIB selects another build of the same source (the sanitizer test)
_LIB = os.environ.get("KVQREF_LIB") or os.path.join(_HERE, "libkvqref.so")

PATTERN, KVARN, NSN = 0, 1, 2
IN_F32, IN_BF16 = 0, 1
NONE = 0xFF
KBLOCK = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE flags)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fno-unsafe-math-optimizations", "-Wall", "-Wextra", "-Wno-unused-parameter",
               "-shared", "-fPIC", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts), for a run under the ASan runtime (LD_PRELOAD)."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fno-unsafe-math-optimizations", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           "-shared", "-fPIC", "-o", out, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "max_tokens",
        "bits", "group", "mode", "max_patterns", "pattern_window")] + [
        ("v_alpha", C.c_double), ("in_dtype", C.c_int32), ("shared_patterns", C.c_int32),
        ("k_per_channel", C.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        P, I, D, F = C.c_void_p, C.c_int32, C.c_double, C.c_float
        sig = {
            "kvqref_new": (P, [P]), "kvqref_free": (None, [P]),
            "kvqref_set_patterns": (I, [P, P, P, I]),
            "kvqref_init_patterns": (I, [P, P, P, I, I]),
            "kvqref_encode_append": (I, [P, P, P, I, I]),
            "kvqref_dequant": (I, [P, I, I, I, P]),
            "kvqref_attn_decode": (I, [P, P, P, D]),
            "kvqref_attn_exact": (I, [P, P, P, I, P, P, D]),
            "kvqref_n_tokens": (I, [P]), "kvqref_n_patterns": (I, [P]),
            "kvqref_dropped": (I, [P]), "kvqref_win_count": (I, [P]),
            "kvqref_region": (P, [P, C.c_char_p, C.POINTER(C.c_int64)]),
            "kvqref_norm_ppf": (D, [D]), "kvqref_rho_star": (D, [I, D]),
            "kvqref_rho_star_f32": (F, [I, D]),
            "kvqref_f16_round": (C.c_uint16, [F, I]),
            "kvqref_f16_to_f32": (F, [C.c_uint16]),
            "kvqref_fwht_f32": (None, [P, I]),
            "kvqref_quant_group": (None, [P, I, I, P, P, P, P]),
            "kvqref_nearest": (I, [P, P, I, I, P]),
            "kvqref_kmeans": (I, [P, I, I, I, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ------------------------------------------------------------ scalar helpers
def norm_ppf(p: float) -> float:
    return lib().kvqref_norm_ppf(p)


def rho_star(d: int, alpha: float) -> float:
    return lib().kvqref_rho_star(d, alpha)


def rho_star_f32(d: int, alpha: float) -> np.float32:
    return np.float32(lib().kvqref_rho_star_f32(d, alpha))


def f16_round(x: float, mode: int) -> int:
    return int(lib().kvqref_f16_round(float(np.float32(x)), mode))


def f16_to_f32(h: int) -> float:
    return lib().kvqref_f16_to_f32(int(h))


def fwht_f32(x: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    lib().kvqref_fwht_f32(_ptr(y), y.shape[-1])
    return y


def quant_group(r: np.ndarray, bits: int):
    r = np.ascontiguousarray(r, dtype=np.float32)
    codes = np.zeros(r.size, np.uint8)
    ties = np.zeros(r.size, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    lib().kvqref_quant_group(_ptr(r), r.size, bits, _ptr(codes), _ptr(s), _ptr(z), _ptr(ties))
    return codes, int(s[0]), int(z[0]), ties


def nearest(x: np.ndarray, pats: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    p = np.ascontiguousarray(pats, dtype=np.float32)
    e = np.zeros(1, np.float32)
    k = lib().kvqref_nearest(_ptr(x), _ptr(p), p.shape[0] if p.ndim == 2 else 0, x.size, _ptr(e))
    return k, float(e[0])


def kmeans(x: np.ndarray, k: int):
    x = np.ascontiguousarray(x, dtype=np.float32)
    n, d = x.shape
    cent = np.zeros((k, d), np.float32)
    a = np.zeros(n, np.int32)
    it = lib().kvqref_kmeans(_ptr(x), n, d, k, _ptr(cent), _ptr(a))
    return cent, a, it


# ------------------------------------------------------------ cache
class RefCache:
    """The oracle's cache: same calls as the library, on host arrays."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, max_tokens, bits=2, group=32,
                 mode=PATTERN, max_patterns=64, pattern_window=128, v_alpha=0.05,
                 in_dtype=IN_F32, shared_patterns=False, k_per_channel=False):
        self.cfg = _Cfg(batch, n_q_heads, n_kv_heads, head_dim, max_tokens, bits, group, mode,
                        max_patterns, pattern_window, v_alpha, in_dtype, int(shared_patterns),
                        int(k_per_channel))
        self._h = lib().kvqref_new(C.byref(self.cfg))
        if not self._h:
            raise ValueError("invalid oracle configuration")
        self.U = batch * n_kv_heads
        self.PU = n_kv_heads if shared_patterns else self.U   # pattern-table units
        self.tcap = max_tokens
        self.nblk = (self.tcap + KBLOCK - 1) // KBLOCK

    def __del__(self):
        # at interpreter exit the module globals may already be gone; the
        # process then releases the memory anyway
        h = getattr(self, "_h", None)
        if h and lib is not None:
            lib().kvqref_free(h)
            self._h = None

    def _in(self, a):
        if self.cfg.in_dtype == IN_F32:
            return np.ascontiguousarray(a, dtype=np.float32)
        assert a.dtype == np.uint16, "bf16 inputs are passed as uint16 bit patterns"
        return np.ascontiguousarray(a)

    def set_patterns(self, k_tab, v_tab, n=None):
        k_tab = np.ascontiguousarray(k_tab, dtype=np.float32)
        v_tab = np.ascontiguousarray(v_tab, dtype=np.float32)
        n = k_tab.shape[2] if n is None and k_tab.ndim == 4 else (n or 0)
        return lib().kvqref_set_patterns(self._h, _ptr(k_tab), _ptr(v_tab), n)

    def init_patterns(self, k, v, n_patterns):
        k, v = self._in(k), self._in(v)
        return lib().kvqref_init_patterns(self._h, _ptr(k), _ptr(v), k.shape[2], n_patterns)

    def encode_append(self, k, v, update=0):
        k, v = self._in(k), self._in(v)
        return lib().kvqref_encode_append(self._h, _ptr(k), _ptr(v), k.shape[2], int(update))

    def dequant(self, which, tok0, n):
        out = np.zeros((self.U, n, self.cfg.head_dim), np.float32)
        rc = lib().kvqref_dequant(self._h, which, tok0, n, _ptr(out))
        if rc:
            raise ValueError(f"dequant rc={rc}")
        return out.reshape(self.cfg.batch, self.cfg.n_kv_heads, n, self.cfg.head_dim)

    def attn_decode(self, q, sm_scale=0.0):
        q = self._in(q)
        out = np.zeros((self.cfg.batch, self.cfg.n_q_heads, self.cfg.head_dim), np.float32)
        rc = lib().kvqref_attn_decode(self._h, _ptr(q), _ptr(out), sm_scale)
        if rc:
            raise ValueError(f"attn rc={rc}")
        return out

    @property
    def n_tokens(self):
        return lib().kvqref_n_tokens(self._h)

    @property
    def n_patterns(self):
        return lib().kvqref_n_patterns(self._h)

    @property
    def dropped(self):
        return lib().kvqref_dropped(self._h)

    @property
    def win_count(self):
        return lib().kvqref_win_count(self._h)

    def region(self, name: str) -> np.ndarray:
        """Copy of a state region as a flat uint8 array."""
        n = C.c_int64(0)
        p = lib().kvqref_region(self._h, name.encode(), C.byref(n))
        if not p:
            raise KeyError(name)
        return np.ctypeslib.as_array((C.c_uint8 * n.value).from_address(p)).copy()

    # typed views of the regions -----------------------------------------
    def k_codes_unit(self, which: int) -> np.ndarray:
        return self.region("kv"[which] + "_codes")

    def sz(self, which):
        a = self.region("kv"[which] + "_sz").view(np.uint16)
        return a.reshape(self.U, self.tcap, -1, 2)

    def idx(self, which):
        return self.region("kv"[which] + "_idx").reshape(self.U, self.tcap)

    def t16(self, which):
        """KVARN token scale, or NSN first norm n1 (binary16 bits)."""
        return self.region("kv"[which] + "_t16").view(np.uint16).reshape(self.U, self.tcap)

    def t2(self, which):
        """NSN second norm n2 (binary16 bits)."""
        return self.region("kv"[which] + "_t2").view(np.uint16).reshape(self.U, self.tcap)

    def ties(self, which):
        return self.region("kv"[which] + "_tie").reshape(self.U, self.tcap, self.cfg.head_dim)

    def patterns(self, which):
        return self.region("kv"[which] + "_pat").view(np.float32).reshape(
            self.PU, self.cfg.max_patterns, self.cfg.head_dim)

    def scales(self, which):
        return self.region("kv"[which] + "_scale").view(np.float32).reshape(
            self.U, self.cfg.head_dim)

    def block_sz(self):
        """K per channel: binary16 (s, z) [U][block][D][2]."""
        return self.region("k_bsz").view(np.uint16).reshape(self.U, self.nblk, self.cfg.head_dim, 2)

    def k_tail(self):
        """K per channel: binary16 residuals of the open block [U][128][D]."""
        return self.region("k_tail").view(np.uint16).reshape(self.U, KBLOCK, self.cfg.head_dim)

    def codes(self, which):
        """Packed code bytes [U][tcap * D * bits / 8] in the stored layout."""
        return self.region("kv"[which] + "_codes").reshape(self.U, -1)


def attn_exact(k, v, q, n_q_heads, sm_scale=0.0):
    """fp64 attention over explicit fp32 K/V [B][Hkv][T][D] and q [B][Hq][D]."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    B, H, T, D = k.shape
    cfg = _Cfg(B, n_q_heads, H, D, T, 2, D, PATTERN, 0, 0, 0.0, IN_F32, 0, 0)
    out = np.zeros((B, n_q_heads, D), np.float32)
    rc = lib().kvqref_attn_exact(C.byref(cfg), _ptr(k), _ptr(v), T, _ptr(q), _ptr(out), sm_scale)
    if rc:
        raise ValueError(f"attn_exact rc={rc}")
    return out


def unpack_codes(packed: np.ndarray, T: int, D: int, bits: int) -> np.ndarray:
    """Codes [U][T][D] from the oracle's records (K and V alike: one record
    per token, channel d at bit bits * d, little-endian)."""
    U = packed.shape[0]
    per = 8 // bits
    mask = (1 << bits) - 1
    b = packed.reshape(U, -1)
    sh = (np.arange(per) * bits).astype(np.uint8)
    vals = ((b[..., None] >> sh) & mask).reshape(U, -1)   # code stream in bit order
    return vals.reshape(U, -1, D)[:, :T]
