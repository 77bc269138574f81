"""Helpers shared by the GPU parity tests: build matching oracle / GPU caches
from the same seeded inputs and compare their stored bytes.

The oracle never receives anything produced by the GPU: both sides get the
same synthetic inputs (and the oracle computes its own pattern tables).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from bit_kv_cache_encode_amd import synth

ATTN_TOL = 2e-3        # absolute, attention outputs (bf16 inputs)
DEQ_RTOL = 1e-6        # relative, dequantised values


def to_dev(x: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """fp32 numpy -> device tensor of `dtype` (bf16 by nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).to(device).contiguous()


def to_oracle(x: np.ndarray, bf16: bool) -> np.ndarray:
    """The same values as the oracle receives them (bf16 as bit patterns)."""
    return synth.f32_to_bf16_bits(x) if bf16 else np.ascontiguousarray(x, dtype=np.float32)


def dev_to_oracle(t: torch.Tensor) -> np.ndarray:
    """A device input tensor as oracle input (bf16 -> uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()


def gpu_sz(cache, which: int) -> np.ndarray:
    L = cache.layout
    a = cache.region("kv"[which] + "_sz").cpu().numpy().view(np.uint16)
    return a.reshape(cache.cfg.batch * cache.cfg.n_kv_heads, L.token_cap, L.n_groups, 2)


def gpu_idx(cache, which: int) -> np.ndarray:
    L = cache.layout
    return cache.region("kv"[which] + "_idx").cpu().numpy().reshape(-1, L.token_cap)


def gpu_t16(cache, which: int) -> np.ndarray:
    L = cache.layout
    return cache.region("kv"[which] + "_t16").cpu().numpy().view(np.uint16).reshape(-1, L.token_cap)


def unpack_gpu_codes(packed: np.ndarray, which: int, T: int, D: int, bits: int) -> np.ndarray:
    """Codes [U][T][D] from the library's byte layout, which the oracle does
    not share.  K: one record per token, channel d at bit bits * d (the
    oracle's order).  V: 32-token tiles of 32-bit words; a word holds 32 /
    bits consecutive tokens of one channel (token k at bit bits * k), and
    word w of channel d sits at byte (w * D + d) * 4 of the tile."""
    U = packed.shape[0]
    per = 8 // bits
    mask = (1 << bits) - 1
    sh = (np.arange(per) * bits).astype(np.uint8)
    vals = ((packed.reshape(U, -1)[..., None] >> sh) & mask).reshape(U, -1)   # code stream
    if which == 0:
        return vals.reshape(U, -1, D)[:, :T]
    per_word = 32 // bits
    tiles = vals.reshape(U, -1, bits, D, per_word)        # [U][tile][word][d][k]
    return tiles.transpose(0, 1, 2, 4, 3).reshape(U, -1, D)[:, :T]


def gpu_codes(cache, which: int, T: int, units=None) -> np.ndarray:
    c = cache.cfg
    packed = cache.region("kv"[which] + "_codes").cpu().numpy().reshape(c.batch * c.n_kv_heads, -1)
    if units is not None:
        packed = packed[list(units)]
    return unpack_gpu_codes(packed, which, T, c.head_dim, c.bits)


def gpu_tab(cache, which: int) -> np.ndarray:
    """Pattern tables [PU][max_patterns][D] (PU = kv-heads when the batch
    shares them) or KVarN channel scales [U][D]."""
    c = cache.cfg
    a = cache.region("kv"[which] + "_tab").cpu().numpy().view(np.float32)
    if cache.mode == "pattern":
        return a.reshape(cache.pattern_units, c.max_patterns, c.head_dim)
    return a.reshape(c.batch * c.n_kv_heads, c.head_dim)


def assert_same_encode(ref: "O.RefCache", cache, T: int, units=None, ref_units=None) -> None:
    """Codes, scales, indices (and t16) bit-exact for tokens < T.

    units: GPU unit indices to compare; ref_units: matching oracle units."""
    c = cache.cfg
    U = c.batch * c.n_kv_heads
    units = list(range(U)) if units is None else list(units)
    ref_units = units if ref_units is None else list(ref_units)
    for which in (0, 1):
        gc = gpu_codes(cache, which, T, units)
        rc = O.unpack_codes(ref.codes(which)[ref_units], T, c.head_dim, c.bits)
        bad = gc != rc
        assert not bad.any(), (f"{'KV'[which]} codes differ at {np.argwhere(bad)[:5]} "
                               f"(ties there: {ref.ties(which)[ref_units][:, :T][bad][:5]})")
        gs = gpu_sz(cache, which)[units, :T]
        rs = ref.sz(which)[ref_units, :T]
        assert np.array_equal(gs, rs), f"{'KV'[which]} scales differ at {np.argwhere(gs != rs)[:5]}"
        if cache.mode == "pattern":
            gi = gpu_idx(cache, which)[units, :T]
            ri = ref.idx(which)[ref_units, :T]
            assert np.array_equal(gi, ri), f"{'KV'[which]} idx differ at {np.argwhere(gi != ri)[:5]}"
        else:
            gt = gpu_t16(cache, which)[units, :T]
            rt = ref.t16(which)[ref_units, :T]
            assert np.array_equal(gt, rt), f"{'KV'[which]} t16 differ at {np.argwhere(gt != rt)[:5]}"
            if cache.mode == "nsn":
                L = cache.layout
                g2 = cache.region("kv"[which] + "_t2").cpu().numpy().view(np.uint16).reshape(-1, L.token_cap)
                g2, r2 = g2[units, :T], ref.t2(which)[ref_units, :T]
                assert np.array_equal(g2, r2), f"{'KV'[which]} n2 differ at {np.argwhere(g2 != r2)[:5]}"


def assert_same_kch(ref: "O.RefCache", cache, T: int, units=None, ref_units=None) -> None:
    """K per channel: K indices, the complete blocks' codes (ties excused)
    and (s, z) words, the open block's residuals, and V bit-exact for
    tokens < T.  units: GPU units to compare; ref_units: matching oracle units."""
    c = cache.cfg
    U, D = c.batch * c.n_kv_heads, c.head_dim
    units = list(range(U)) if units is None else list(units)
    ref_units = units if ref_units is None else list(ref_units)
    closed, nblk = T // O.KBLOCK * O.KBLOCK, T // O.KBLOCK
    gi, ri = gpu_idx(cache, 0)[units, :T], ref.idx(0)[ref_units, :T]
    assert np.array_equal(gi, ri), f"K idx differ at {np.argwhere(gi != ri)[:5]}"
    if closed:
        gc = gpu_codes(cache, 0, closed, units)
        rc = O.unpack_codes(ref.codes(0)[ref_units], closed, D, c.bits)
        bad = (gc != rc) & (ref.ties(0)[ref_units, :closed] == 0)
        assert not bad.any(), f"K codes differ at {np.argwhere(bad)[:5]}"
        gb = cache.region("k_bsz").cpu().numpy().view(np.uint16).reshape(U, -1, D, 2)[units, :nblk]
        rb = ref.block_sz()[ref_units, :nblk]
        assert np.array_equal(gb, rb), f"K block (s, z) differ at {np.argwhere(gb != rb)[:5]}"
    if T % O.KBLOCK:
        gt = cache.region("k_tail").cpu().numpy().view(np.uint16).reshape(U, O.KBLOCK, D)
        gt, rt = gt[units, :T % O.KBLOCK], ref.k_tail()[ref_units, :T % O.KBLOCK]
        assert np.array_equal(gt, rt), f"K residuals differ at {np.argwhere(gt != rt)[:5]}"
    gc = gpu_codes(cache, 1, T, units)
    rc = O.unpack_codes(ref.codes(1)[ref_units], T, D, c.bits)
    assert np.array_equal(gc, rc), f"V codes differ at {np.argwhere(gc != rc)[:5]}"
    assert np.array_equal(gpu_sz(cache, 1)[units, :T], ref.sz(1)[ref_units, :T]), "V scales differ"
    assert np.array_equal(gpu_idx(cache, 1)[units, :T], ref.idx(1)[ref_units, :T]), "V idx differ"


def make_pair(B, Hq, Hkv, max_tokens, *, bits=2, group=32, mode="pattern", max_patterns=32,
              pattern_window=128, v_alpha=0.05, bf16=True, shared_patterns=False,
              k_per_channel=False):
    from bit_kv_cache_encode_amd import KVCache
    dt = torch.bfloat16 if bf16 else torch.float32
    gpu = KVCache(B, Hq, Hkv, max_tokens, bits=bits, group=group, mode=mode,
                  max_patterns=max_patterns, pattern_window=pattern_window, v_alpha=v_alpha,
                  in_dtype=dt, shared_patterns=shared_patterns, k_per_channel=k_per_channel)
    ref = O.RefCache(B, Hq, Hkv, 128, max_tokens, bits=bits, group=group,
                     mode={"pattern": O.PATTERN, "kvarn": O.KVARN, "nsn": O.NSN}[mode],
                     max_patterns=max_patterns, pattern_window=pattern_window, v_alpha=v_alpha,
                     in_dtype=O.IN_BF16 if bf16 else O.IN_F32, shared_patterns=shared_patterns,
                     k_per_channel=k_per_channel)
    return gpu, ref, dt
