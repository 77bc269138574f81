"""Input domain (KVQ_KV_LIMIT, KVQ_Q_LIMIT) and the cache's domain flags.

Inside the domain, values at its edge encode bit-exactly against the oracle
(codes, scales, indices, token scales) in every mode, attention stays within
the usual bound (scaled with the data), and no flag is raised.  An element at
or beyond the K/V limit, or not finite, in any call that reads K/V inputs
(bulk encode, one-token encode, the one-launch decode step, pattern init)
sets KVQ_DOMAIN_KV; a query element with |q| * sm_scale >= 2^96, or not
finite, sets KVQ_DOMAIN_Q in both attention kernels and in the decode step.
Flags stay set until a clearing read.  Out-of-domain values only change
results: every index the kernels derive from data is bounded (a pattern
index is the argmin over the table or 0xFF, codes are clamped), so these
inputs are safe to run.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import KVCache, synth
from bit_kv_cache_encode_amd import _binding as B
from parity_util import ATTN_TOL, assert_same_encode, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu
D = 128
EDGE = np.float32(4095.5)   # the largest binary32 value used below KVQ_KV_LIMIT = 4096


def _edge_inputs(B_, H, T, off):
    """Seeded K/V scaled so that max |x| is exactly EDGE (K keeps its outlier
    channels), and the scale factors applied."""
    k = synth.k_vectors(B_, H, T, D, seed=synth.seed_for("k") + off)
    v = synth.v_vectors(B_, H, T, D, seed=synth.seed_for("v") + off)
    ck = EDGE / np.float32(np.abs(k).max())
    cv = EDGE / np.float32(np.abs(v).max())
    k = (k * ck).astype(np.float32)
    v = (v * cv).astype(np.float32)
    # pin the extremes to exactly +-EDGE (rounding of the products may miss it)
    k.reshape(-1)[np.argmax(np.abs(k))] = np.copysign(EDGE, k.reshape(-1)[np.argmax(np.abs(k))])
    v.reshape(-1)[np.argmax(np.abs(v))] = np.copysign(EDGE, v.reshape(-1)[np.argmax(np.abs(v))])
    assert np.abs(k).max() == EDGE and np.abs(v).max() == EDGE
    return k, v, float(ck), float(cv)


@pytest.mark.parametrize("mode,bits,group", [("pattern", 2, 32), ("pattern", 4, 64),
                                             ("kvarn", 2, 32), ("nsn", 2, 32)])
def test_edge_of_kv_domain_is_exact_and_unflagged(mode, bits, group):
    B_, H, Hq, T = 2, 2, 8, 300
    P = 16 if mode == "pattern" else 0
    gpu, ref, dt = make_pair(B_, Hq, H, T + 64, bits=bits, group=group, mode=mode,
                             max_patterns=P, bf16=False)
    k, v, ck, cv = _edge_inputs(B_, H, T, off=bits + group)
    assert ref.init_patterns(to_oracle(k[:, :, :128], False), to_oracle(v[:, :, :128], False), P) == 0
    print(f"domain edge {mode} bits={bits} group={group}", flush=True)
    gpu.init_patterns(to_dev(k[:, :, :128], dt), to_dev(v[:, :, :128], dt), P)
    if mode != "pattern":
        # channel statistics agree to 1e-6 relative; the encode then compares
        # on the oracle's (the pattern tables of the GPU k-means are the
        # oracle's bit for bit)
        gpu.set_patterns(torch.from_numpy(ref.scales(0).reshape(B_, H, D).copy()).cuda(),
                         torch.from_numpy(ref.scales(1).reshape(B_, H, D).copy()).cuda())
    assert ref.encode_append(to_oracle(k, False), to_oracle(v, False)) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    torch.cuda.synchronize()
    assert_same_encode(ref, gpu, T)
    # queries scaled down by K's factor keep the scores near unit scale
    q = (synth.queries(B_, Hq, D, step=3) / np.float32(ck)).astype(np.float32)
    want = ref.attn_decode(to_oracle(q, False))
    got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
    err = float(np.abs(got - want).max())
    assert err <= ATTN_TOL * cv, (err, ATTN_TOL * cv)
    assert gpu.status() == 0


def _pattern_cache(bf16=True, T0=256):
    dt = torch.bfloat16 if bf16 else torch.float32
    dev = torch.device("cuda", 0)
    c = KVCache(2, 8, 2, T0 + 64, bits=2, group=32, max_patterns=16, in_dtype=dt, device=dev)
    k, v = synth.device_kv(2, 2, T0, D, device=dev)
    k, v = k.to(dt), v.to(dt)
    c.init_patterns(k[:, :, :128].contiguous(), v[:, :, :128].contiguous(), 16)
    c.encode_append(k, v)
    assert c.status() == 0
    return c, dt, dev


@pytest.mark.parametrize("bad", [4096.0, -5000.0, float("inf"), float("nan")])
@pytest.mark.parametrize("path", ["bulk", "token", "step", "init"])
def test_kv_out_of_domain_sets_flag(path, bad):
    c, dt, dev = _pattern_cache()
    n = 1 if path in ("token", "step") else 40
    k, v = synth.device_kv(2, 2, n, D, layer=3, device=dev)
    k, v = k.to(dt).contiguous(), v.to(dt).contiguous()
    (v if path == "token" else k)[1, 0, n - 1, 77] = bad
    print(f"kv domain path={path} bad={bad}", flush=True)
    if path == "bulk":
        c.encode_append(k, v)
    elif path == "token":
        c.encode_append(k, v)
    elif path == "step":
        q = synth.device_queries(2, 8, D, device=dev).to(dt)
        c.decode_step(k, v, q)
    else:
        c.init_patterns(k, v, 8)
    assert c.status(clear=False) == B.DOMAIN_KV
    assert c.status() == B.DOMAIN_KV      # still set, cleared by this read
    assert c.status() == 0


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("bad", ["nan", "inf", "huge"])
def test_query_out_of_domain_sets_flag(kernel, bad):
    c, dt, dev = _pattern_cache()
    c.attn_kernel = kernel
    q = synth.device_queries(2, 8, D, device=dev).float()
    # |q| * sm_scale >= 2^96 with sm_scale = 1 / sqrt(128)
    q[0, 5, 3] = {"nan": float("nan"), "inf": float("inf"), "huge": 2.0 ** 96 * 128 ** 0.5 * 1.01}[bad]
    print(f"q domain kernel={kernel} bad={bad}", flush=True)
    c.attn_decode(q.to(dt).contiguous())
    assert c.status() == B.DOMAIN_Q
    # a query just inside the limit is not flagged (and the call still runs)
    q[0, 5, 3] = 2.0 ** 96 * 128 ** 0.5 * 0.98
    c.attn_decode(q.to(dt).contiguous())
    assert c.status() == 0


def test_flags_accumulate_until_read():
    """K/V and query flags OR together over calls (the decode step reads both
    kinds of input) and stay set through later in-domain calls."""
    c, dt, dev = _pattern_cache()
    k, v = synth.device_kv(2, 2, 1, D, layer=5, device=dev)
    k, v = k.to(dt).contiguous(), v.to(dt).contiguous()
    q = synth.device_queries(2, 8, D, device=dev).to(dt).contiguous()
    k[0, 1, 0, 0] = float("nan")
    q_bad = q.clone()
    q_bad[1, 2, 9] = float("inf")
    print("domain flags accumulate", flush=True)
    c.decode_step(k, v, q_bad)
    k2, v2 = synth.device_kv(2, 2, 1, D, layer=6, device=dev)
    c.decode_step(k2.to(dt).contiguous(), v2.to(dt).contiguous(), q)
    c.attn_decode(q)
    assert c.status() == B.DOMAIN_KV | B.DOMAIN_Q
    assert c.status() == 0
