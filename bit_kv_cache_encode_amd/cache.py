"""Torch-facing wrapper over the C-ABI: one device buffer per cache.

PyTorch only provides the device memory (one uint8 tensor per cache) and the
stream; all computation is in libkvq.so.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _binding as B

_DT = {torch.float32: B.F32, torch.bfloat16: B.BF16}


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class KVCache:
    """A packed 2/4-bit K/V cache for one attention layer.

    mode: "pattern" (PatternKV residual encode), "kvarn" (Hadamard +
    dual-axis normalisation encode) or "nsn" (token norm, channel centre,
    token norm, Hadamard; also 1-bit codes).  shared_patterns (pattern mode): one
    pattern table and Chebyshev window per kv-head for the whole batch.
    k_per_channel (pattern mode): K quantized per channel over 128-token
    blocks, the open block's residuals held in binary16.
    Shapes follow include/kvq.h.
    """

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, max_tokens: int,
                 head_dim: int = 128, bits: int = 2, group: int = 32, mode: str = "pattern",
                 max_patterns: int = 64, pattern_window: int = 128, v_alpha: float = 0.05,
                 in_dtype: torch.dtype = torch.bfloat16, max_splits: int = 0,
                 device: str | torch.device = "cuda", buffer: torch.Tensor | None = None,
                 shared_patterns: bool = False, k_per_channel: bool = False):
        if in_dtype not in _DT:
            raise ValueError("in_dtype must be torch.float32 or torch.bfloat16")
        m = {"pattern": B.MODE_PATTERN, "kvarn": B.MODE_KVARN, "nsn": B.MODE_NSN}[mode]
        self.cfg = B.kvq_config(batch, n_q_heads, n_kv_heads, head_dim, max_tokens, bits, group,
                                m, max_patterns, pattern_window, v_alpha, _DT[in_dtype],
                                max_splits, int(shared_patterns), int(k_per_channel))
        self.layout = B.kvq_layout_of(self.cfg)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.in_dtype = in_dtype
        self.mode = mode
        self.shared_patterns = bool(shared_patterns)
        self.k_per_channel = bool(k_per_channel)
        # pattern-table units: one per kv-head when shared, else per (batch, kv-head)
        self.pattern_units = n_kv_heads if shared_patterns else batch * n_kv_heads
        if buffer is None:
            buffer = torch.zeros(self.layout.total, dtype=torch.uint8, device=self.device)
        if buffer.numel() < self.layout.total or buffer.dtype != torch.uint8:
            raise ValueError("buffer too small or not uint8")
        self.buf = buffer
        self.c = B.kvq_cache()
        B.check("kvq_cache_init", B.kvq_cache_init(self.c, self.cfg, _ptr(buffer),
                                                   buffer.numel(), _stream(self.device)))

    # ------------------------------------------------------------- checks
    def _in(self, t: torch.Tensor, name: str, rows: int | None = None) -> torch.Tensor:
        if t.device != self.device or t.dtype != self.in_dtype or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {self.in_dtype} tensor on "
                             f"{self.device}")
        c = self.cfg
        if rows is not None and tuple(t.shape) != (c.batch, c.n_kv_heads, rows, c.head_dim):
            raise ValueError(f"{name}: shape {tuple(t.shape)} != "
                             f"{(c.batch, c.n_kv_heads, rows, c.head_dim)}")
        return t

    # ------------------------------------------------------------- calls
    def set_patterns(self, k_tab: torch.Tensor, v_tab: torch.Tensor) -> None:
        for t in (k_tab, v_tab):
            if t.device != self.device or t.dtype != torch.float32 or not t.is_contiguous():
                raise ValueError("pattern tables must be contiguous fp32 on the cache device")
        c = self.cfg
        if self.mode == "pattern":
            lead = (c.n_kv_heads,) if self.shared_patterns else (c.batch, c.n_kv_heads)
            shp = tuple(k_tab.shape)
            if self.shared_patterns and len(shp) == 4 and shp[0] == 1:
                shp = shp[1:]
            if shp[:-2] != lead or shp[-1] != c.head_dim or tuple(v_tab.shape) != tuple(k_tab.shape):
                raise ValueError(f"pattern tables: expected {lead} + (n, {c.head_dim}), got "
                                 f"{tuple(k_tab.shape)} / {tuple(v_tab.shape)}")
            n = shp[-2]
        else:
            n = 0
        B.check("kvq_set_patterns", B.kvq_set_patterns(self.c, _ptr(k_tab), _ptr(v_tab), n,
                                                       _stream(self.device)))

    def init_patterns(self, k: torch.Tensor, v: torch.Tensor, n_patterns: int) -> None:
        n = k.shape[2]
        self._in(k, "k", n)
        self._in(v, "v", n)
        B.check("kvq_init_patterns", B.kvq_init_patterns(self.c, _ptr(k), _ptr(v), n, n_patterns,
                                                         _stream(self.device)))

    def encode_append(self, k: torch.Tensor, v: torch.Tensor, update_patterns: bool = False) -> None:
        n = k.shape[2]
        self._in(k, "k", n)
        self._in(v, "v", n)
        B.check("kvq_encode_append", B.kvq_encode_append(self.c, _ptr(k), _ptr(v), n,
                                                         int(update_patterns),
                                                         _stream(self.device)))

    def attn_decode(self, q: torch.Tensor, out: torch.Tensor | None = None,
                    sm_scale: float = 0.0) -> torch.Tensor:
        c = self.cfg
        if q.device != self.device or q.dtype != self.in_dtype or not q.is_contiguous() or \
                tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError("q must be contiguous [B][Hq][D] in the cache's input dtype")
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        B.check("kvq_attn_decode", B.kvq_attn_decode(self.c, _ptr(q), _ptr(out), sm_scale,
                                                     _stream(self.device)))
        return out

    def decode_step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                    out: torch.Tensor | None = None, sm_scale: float = 0.0,
                    update_patterns: bool = True) -> torch.Tensor:
        """Append one token (k, v: [B][Hkv][1][D]) and attend with q over the
        cache including it, in one launch (kvq_decode_step)."""
        c = self.cfg
        self._in(k, "k", 1)
        self._in(v, "v", 1)
        if q.device != self.device or q.dtype != self.in_dtype or not q.is_contiguous() or \
                tuple(q.shape) != (c.batch, c.n_q_heads, c.head_dim):
            raise ValueError("q must be contiguous [B][Hq][D] in the cache's input dtype")
        if out is None:
            out = torch.empty((c.batch, c.n_q_heads, c.head_dim), dtype=torch.float32,
                              device=self.device)
        B.check("kvq_decode_step", B.kvq_decode_step(self.c, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                                     sm_scale, int(update_patterns),
                                                     _stream(self.device)))
        return out

    def dequant(self, which: int, tok0: int = 0, n: int | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
        c = self.cfg
        n = self.n_tokens - tok0 if n is None else n
        if out is None:
            out = torch.empty((c.batch, c.n_kv_heads, max(n, 0), c.head_dim), dtype=torch.float32,
                              device=self.device)
        B.check("kvq_dequant", B.kvq_dequant(self.c, which, tok0, n, _ptr(out),
                                             _stream(self.device)))
        return out

    def status(self, clear: bool = True) -> int:
        """Input-domain flags (DOMAIN_KV | DOMAIN_Q bits) set by the kernels
        since init or the last clearing read; synchronises the stream."""
        flags = C.c_uint32(0)
        B.check("kvq_cache_status", B.kvq_cache_status(self.c, C.byref(flags), int(clear),
                                                       _stream(self.device)))
        return int(flags.value)

    # ------------------------------------------------------------- state
    @property
    def n_tokens(self) -> int:
        return self.c.n_tokens

    @property
    def n_patterns(self) -> int:
        return self.c.n_patterns

    @property
    def win_count(self) -> int:
        return self.c.win_count

    @property
    def dropped(self) -> int:
        return self.c.dropped

    @property
    def rho(self) -> float:
        return self.c.rho

    @property
    def attn_kernel(self) -> str:
        """Attention kernel: "auto" (the matrix-core kernel wherever it
        applies) or "valu" (the vector kernel, a cross-check).  Set from the
        environment variable KVQ_ATTN_KERNEL when the cache is created."""
        return "valu" if self.c.attn_kernel == B.ATTN_VALU else "auto"

    @attn_kernel.setter
    def attn_kernel(self, name: str) -> None:
        if name not in ("auto", "valu"):
            raise ValueError("attn_kernel must be 'auto' or 'valu'")
        self.c.attn_kernel = B.ATTN_VALU if name == "valu" else B.ATTN_AUTO

    @property
    def attn_blocks(self) -> int:
        """Target grid size of the attention, 0 = the default (256).  Set
        from the environment variable KVQ_ATTN_BLOCKS when the cache is created."""
        return self.c.attn_blocks

    @attn_blocks.setter
    def attn_blocks(self, n: int) -> None:
        if int(n) < 0:
            raise ValueError("attn_blocks must be >= 0")
        self.c.attn_blocks = int(n)

    def region(self, name: str) -> torch.Tensor:
        """uint8 view of a region of the cache buffer (e.g. "k_codes")."""
        L = self.layout
        size = {"k_codes": L.codes_bytes, "v_codes": L.codes_bytes, "k_sz": L.sz_bytes,
                "v_sz": L.sz_bytes, "k_idx": L.idx_bytes, "v_idx": L.idx_bytes,
                "k_t16": L.t16_bytes, "v_t16": L.t16_bytes, "k_tab": L.tab_bytes,
                "v_tab": L.tab_bytes, "k_win": L.win_bytes, "v_win": L.win_bytes,
                "ws": L.ws_bytes, "cnt": L.cnt_bytes, "k_bsz": L.bsz_bytes,
                "k_tail": L.tail_bytes, "k_t2": L.t2_bytes, "v_t2": L.t2_bytes}[name]
        off = getattr(L, name)
        return self.buf[off:off + size]

    def clone(self) -> "KVCache":
        """An independent cache with a copy of this one's buffer and state."""
        other = KVCache.__new__(KVCache)
        other.__dict__.update({k: v for k, v in self.__dict__.items() if k not in ("buf", "c")})
        other.buf = self.buf.clone()
        other.c = B.kvq_cache()
        C.memmove(C.addressof(other.c), C.addressof(self.c), C.sizeof(B.kvq_cache))
        other.c.base = other.buf.data_ptr()
        return other

    def state_bytes(self) -> int:
        """Bytes a checkpoint needs: the whole buffer."""
        return self.layout.total

    def snapshot(self) -> dict:
        """Host copy of the cache (buffer + host counters) for checkpointing."""
        return {"buf": self.buf.cpu(), "n_tokens": self.c.n_tokens,
                "n_patterns": self.c.n_patterns, "win_count": self.c.win_count,
                "dropped": self.c.dropped}

    def restore(self, snap: dict) -> None:
        self.buf.copy_(snap["buf"].to(self.device))
        self.c.n_tokens = snap["n_tokens"]
        self.c.n_patterns = snap["n_patterns"]
        self.c.win_count = snap["win_count"]
        self.c.dropped = snap["dropped"]
