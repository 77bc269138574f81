"""Seeded synthetic K/V/q inputs shaped like the PatternKV / KVarN decode workloads.

This module only draws random numbers and changes their storage type. It holds
none of the quantization method's arithmetic, so both the CPU oracle and the
HIP path may consume what it produces.

Recipe (one (batch, kv-head) pair is a "unit"):

* K: i.i.d. N(0, 1) per channel; in every unit 4 channels, drawn once per
  unit, are scaled by 10 for all tokens (the fixed outlier channels that the
  PatternKV paper reports for the K cache, section 2.2.1 and Figure 2).
* V: a mixture of 16 centres c_k ~ N(0, I_D) per unit; every token picks k
  uniformly and adds N(0, 0.3^2) noise (the clustered, semantically organised
  V cache of section 2.2.2 / Figure 3b).
* q: i.i.d. N(0, 1).
* drift: one direction u ~ N(0, I_D) per unit; a streaming decode step j adds
  0.01 * j * u to the new K vector (the smooth K drift of section 2.2.1).
* bf16 inputs are the fp32 draws rounded to nearest-even bf16.

Seeds: base 20261203; K = base+0, V = base+1, q = base+2, drift = base+3;
layer l adds 1000*l.  numpy's PCG64 generator is used for reproducible small
cases; ``device_*`` helpers draw the same distributions with torch's generator
on a GPU for the large workloads (a different random stream, same recipe).
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20261203
N_OUTLIER = 4
OUTLIER_GAIN = 10.0
N_CENTRES = 16
V_NOISE = 0.3


def seed_for(kind: str, layer: int = 0, base: int = BASE_SEED) -> int:
    off = {"k": 0, "v": 1, "q": 2, "drift": 3}[kind]
    return base + off + 1000 * layer


# ---------------------------------------------------------------- bf16 storage
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest-even bf16; return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, 0x7FC0, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- numpy draws
def k_vectors(B: int, H: int, T: int, D: int, seed: int | None = None,
              t0: int = 0) -> np.ndarray:
    """fp32 [B][H][T][D]; ``t0`` selects an independent block of tokens."""
    s = seed_for("k") if seed is None else seed
    out = np.empty((B, H, T, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            ch = np.random.default_rng([s, b, h]).choice(D, N_OUTLIER, replace=False)
            tok = np.random.default_rng([s, b, h, t0, 1])
            x = tok.standard_normal((T, D), dtype=np.float32)
            x[:, ch] *= np.float32(OUTLIER_GAIN)
            out[b, h] = x
    return out


def v_vectors(B: int, H: int, T: int, D: int, seed: int | None = None,
              t0: int = 0) -> np.ndarray:
    """fp32 [B][H][T][D]: 16-centre Gaussian mixture per unit."""
    s = seed_for("v") if seed is None else seed
    out = np.empty((B, H, T, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            cen = np.random.default_rng([s, b, h]).standard_normal(
                (N_CENTRES, D), dtype=np.float32)
            tok = np.random.default_rng([s, b, h, t0, 1])
            k = tok.integers(0, N_CENTRES, size=T)
            noise = tok.standard_normal((T, D), dtype=np.float32) * np.float32(V_NOISE)
            out[b, h] = cen[k] + noise
    return out


def queries(B: int, Hq: int, D: int, seed: int | None = None, step: int = 0) -> np.ndarray:
    s = seed_for("q") if seed is None else seed
    return np.random.default_rng([s, step]).standard_normal((B, Hq, D), dtype=np.float32)


def drift_dirs(B: int, H: int, D: int, seed: int | None = None) -> np.ndarray:
    s = seed_for("drift") if seed is None else seed
    return np.random.default_rng(s).standard_normal((B, H, D), dtype=np.float32)


# ---------------------------------------------------------------- torch draws
def device_kv(B: int, H: int, T: int, D: int, layer: int = 0, device="cuda",
              dtype=None):
    """(K, V) drawn on ``device`` with torch's generator; same recipe as above."""
    import torch
    dtype = dtype or torch.bfloat16
    gk = torch.Generator(device=device).manual_seed(seed_for("k", layer))
    gv = torch.Generator(device=device).manual_seed(seed_for("v", layer))
    k = torch.randn((B, H, T, D), generator=gk, device=device, dtype=torch.float32)
    sel = torch.rand((B, H, D), generator=gk, device=device).argsort(dim=-1)[..., :N_OUTLIER]
    gain = torch.ones((B, H, D), device=device)
    gain.scatter_(-1, sel, OUTLIER_GAIN)
    k.mul_(gain[:, :, None, :])
    cen = torch.randn((B, H, N_CENTRES, D), generator=gv, device=device)
    idx = torch.randint(0, N_CENTRES, (B, H, T), generator=gv, device=device)
    v = torch.gather(cen, 2, idx[..., None].expand(B, H, T, D))
    v.add_(torch.randn((B, H, T, D), generator=gv, device=device) * V_NOISE)
    return k.to(dtype), v.to(dtype)


def device_queries(B: int, Hq: int, D: int, step: int = 0, device="cuda", dtype=None):
    import torch
    dtype = dtype or torch.bfloat16
    g = torch.Generator(device=device).manual_seed(seed_for("q") + 7919 * step)
    return torch.randn((B, Hq, D), generator=g, device=device).to(dtype)
