"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Bar: codes, scales, pattern indices and token scales bit-exact; dequantised
values within 1e-6 relative; attention within 2e-3 absolute.  Sizes span
several 32/64-token tiles with ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_kv_cache_encode_amd import synth
from parity_util import (ATTN_TOL, DEQ_RTOL, assert_same_encode, gpu_tab, make_pair, to_dev,
                         to_oracle)

pytestmark = pytest.mark.gpu


def _inputs(B, H, T, seed_off=0):
    k = synth.k_vectors(B, H, T, 128, seed=synth.seed_for("k") + seed_off)
    v = synth.v_vectors(B, H, T, 128, seed=synth.seed_for("v") + seed_off)
    return k, v


def _check_dequant(ref, gpu, T):
    for which in (0, 1):
        g = gpu.dequant(which, 0, T).cpu().numpy()
        r = ref.dequant(which, 0, T)
        np.testing.assert_allclose(g, r, rtol=DEQ_RTOL, atol=1e-7)


def _check_attn(ref, gpu, q_np, bf16):
    dt = torch.bfloat16 if bf16 else torch.float32
    out = gpu.attn_decode(to_dev(q_np, dt)).cpu().numpy()
    want = ref.attn_decode(to_oracle(q_np, bf16))
    err = np.abs(out - want).max()
    assert err <= ATTN_TOL, f"attention max abs err {err}"
    return err


def test_tiny_reference_config():
    """1 KV head, T=256, fp32, 8 k-means patterns, 2-bit, group 32."""
    B, Hq, H, T = 1, 1, 1, 256
    gpu, ref, dt = make_pair(B, Hq, H, T, max_patterns=8, bf16=False)
    k, v = _inputs(B, H, T)
    assert ref.init_patterns(k, v, 8) == 0
    gpu.init_patterns(to_dev(k, dt), to_dev(v, dt), 8)
    torch.cuda.synchronize()
    for which in (0, 1):
        assert np.array_equal(gpu_tab(gpu, which)[:, :8], ref.patterns(which)[:, :8])
    assert ref.encode_append(k, v) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    assert_same_encode(ref, gpu, T)
    _check_dequant(ref, gpu, T)
    _check_attn(ref, gpu, synth.queries(B, Hq, 128), bf16=False)


@pytest.mark.parametrize("T", [1, 31, 64, 300])
def test_llama_shape_encode_attend(T):
    """Llama-3-8B head geometry (32 q / 8 kv, GQA 4), bf16, 32 patterns."""
    B, Hq, H = 2, 8, 2
    gpu, ref, dt = make_pair(B, Hq, H, 512, max_patterns=32)
    kp, vp = _inputs(B, H, 200, seed_off=5)
    ref.init_patterns(to_oracle(kp, True), to_oracle(vp, True), 32)
    gpu.init_patterns(to_dev(kp, dt), to_dev(vp, dt), 32)
    k, v = _inputs(B, H, T)
    ref.encode_append(to_oracle(k, True), to_oracle(v, True))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    assert_same_encode(ref, gpu, T)
    _check_dequant(ref, gpu, T)
    _check_attn(ref, gpu, synth.queries(B, Hq, 128), bf16=True)


@pytest.mark.parametrize("bits,group,gq,npat", [(4, 64, 4, 64), (2, 32, 7, 64), (2, 64, 1, 16),
                                                 (4, 32, 2, 0), (2, 128, 8, 255),
                                                 # one-hot pattern mass over five blocks of 16
                                                 # (64 prefill patterns plus window centres;
                                                 # 4-bit at 80 also leaves M^V unstaged), then
                                                 # the first count past it (LDS atomics)
                                                 (2, 32, 4, 72), (2, 32, 7, 66), (4, 64, 4, 80),
                                                 (2, 32, 4, 81)])
def test_shape_variants(bits, group, gq, npat):
    B, H, T = 1, 2, 333
    gpu, ref, dt = make_pair(B, gq * H, H, 400, bits=bits, group=group, max_patterns=max(npat, 1))
    if npat:
        rng = np.random.default_rng(npat)
        tk = rng.standard_normal((B, H, npat, 128)).astype(np.float32)
        tv = rng.standard_normal((B, H, npat, 128)).astype(np.float32)
        ref.set_patterns(tk, tv)
        gpu.set_patterns(torch.from_numpy(tk).cuda(), torch.from_numpy(tv).cuda())
    k, v = _inputs(B, H, T, seed_off=bits)
    ref.encode_append(to_oracle(k, True), to_oracle(v, True))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    assert_same_encode(ref, gpu, T)
    _check_dequant(ref, gpu, T)
    _check_attn(ref, gpu, synth.queries(B, gq * H, 128, step=3), bf16=True)


def test_kvarn_channel_scale_closed_form():
    """GPU channel scales on the oracle pin's closed-form prefix: rows built in
    the rotated space as a_t (sigma * eps_t), so c = sigma / rms(sigma)
    whatever the token magnitudes a_t (KVarN abstract, reading R12)."""
    import math
    from scipy.linalg import hadamard
    D, T = 128, 64
    rng = np.random.default_rng(77)
    sig = [rng.permutation(np.linspace(0.3, 4.0, D)) for _ in range(2)]
    rows = []
    for s_ in sig:
        y = rng.uniform(0.5, 9.0, (T, 1)) * s_ * rng.choice([-1.0, 1.0], (T, D))
        rows.append((y @ hadamard(D).T.astype(np.float64) / math.sqrt(D)).astype(np.float32))
    k, v = rows[0][None, None], rows[1][None, None]
    gpu, _, dt = make_pair(1, 4, 1, 128, mode="kvarn", max_patterns=0, bf16=False)
    print("KVarN channel scale, closed form", flush=True)
    gpu.init_patterns(to_dev(k, dt), to_dev(v, dt), 0)
    torch.cuda.synchronize()
    for which in (0, 1):
        want = sig[which] / math.sqrt((sig[which] ** 2).mean())
        np.testing.assert_allclose(gpu_tab(gpu, which).reshape(D), want, rtol=2e-6, atol=0)


def test_kvarn_mode():
    """Hadamard + dual-axis normalisation encode, with oracle channel scales."""
    B, Hq, H, T = 2, 8, 2, 150
    gpu, ref, dt = make_pair(B, Hq, H, 256, mode="kvarn", max_patterns=0)
    kp, vp = _inputs(B, H, 64, seed_off=9)
    ref.init_patterns(to_oracle(kp, True), to_oracle(vp, True), 0)
    cs_k, cs_v = ref.scales(0).reshape(B, H, 128), ref.scales(1).reshape(B, H, 128)
    # GPU channel scales agree with the oracle's within rounding (binary64 sums
    # in a different order), then the oracle's are uploaded so the encode is
    # compared on identical inputs.
    gpu.init_patterns(to_dev(kp, dt), to_dev(vp, dt), 0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(gpu_tab(gpu, 0).reshape(B, H, 128), cs_k, rtol=1e-6)
    np.testing.assert_allclose(gpu_tab(gpu, 1).reshape(B, H, 128), cs_v, rtol=1e-6)
    gpu.set_patterns(torch.from_numpy(np.ascontiguousarray(cs_k)).cuda(),
                     torch.from_numpy(np.ascontiguousarray(cs_v)).cuda())
    k, v = _inputs(B, H, T)
    ref.encode_append(to_oracle(k, True), to_oracle(v, True))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    assert_same_encode(ref, gpu, T)
    _check_dequant(ref, gpu, T)
    _check_attn(ref, gpu, synth.queries(B, Hq, 128), bf16=True)


def test_chunked_appends_equal_bulk():
    """Appending in ragged pieces stores the same bytes as one bulk append
    (V tiles shared between calls keep the other calls' bits)."""
    B, Hq, H, T = 1, 4, 1, 250
    k, v = _inputs(B, H, T)
    a, ref, dt = make_pair(B, Hq, H, 256)
    b, _, _ = make_pair(B, Hq, H, 256)
    kd, vd = to_dev(k, dt), to_dev(v, dt)
    for c in (a, b):
        c.init_patterns(kd[:, :, :128].contiguous(), vd[:, :, :128].contiguous(), 16)
    a.encode_append(kd, vd)
    pos = 0
    for n in (3, 29, 1, 64, 5, 100, 48):
        b.encode_append(kd[:, :, pos:pos + n].contiguous(), vd[:, :, pos:pos + n].contiguous())
        pos += n
    assert pos == T
    torch.cuda.synchronize()
    for name in ("k_codes", "k_sz", "k_idx", "v_sz", "v_idx"):
        L = a.layout
        per = {"k_codes": 32, "k_sz": 16, "k_idx": 1, "v_sz": 16, "v_idx": 1}[name]
        assert torch.equal(a.region(name)[:T * per], b.region(name)[:T * per]), name
    assert torch.equal(a.region("v_codes")[:T // 32 * 1024], b.region("v_codes")[:T // 32 * 1024])
    ga = a.dequant(1, 0, T)
    gb = b.dequant(1, 0, T)
    assert torch.equal(ga, gb)


def test_streaming_chebyshev_window():
    """Decode appends one token at a time: a Chebyshev centre joins the table
    after every window; later tokens use it; GPU and oracle agree bit for bit."""
    B, Hq, H, W = 2, 8, 2, 16
    gpu, ref, dt = make_pair(B, Hq, H, 256, max_patterns=6, pattern_window=W)
    kp, vp = _inputs(B, H, 64, seed_off=11)
    ref.init_patterns(to_oracle(kp, True), to_oracle(vp, True), 4)
    gpu.init_patterns(to_dev(kp, dt), to_dev(vp, dt), 4)
    ref.encode_append(to_oracle(kp, True), to_oracle(vp, True))
    gpu.encode_append(to_dev(kp, dt), to_dev(vp, dt))
    k, v = _inputs(B, H, 3 * W + 7, seed_off=12)
    drift = synth.drift_dirs(B, H, 128)
    k = k + 0.5 * np.arange(k.shape[2], dtype=np.float32)[None, None, :, None] * drift[:, :, None, :]
    for t in range(k.shape[2]):
        kt, vt = k[:, :, t:t + 1], v[:, :, t:t + 1]
        ref.encode_append(to_oracle(kt, True), to_oracle(vt, True), update=1)
        gpu.encode_append(to_dev(kt, dt), to_dev(vt, dt), update_patterns=True)
        assert gpu.n_patterns == ref.n_patterns and gpu.win_count == ref.win_count
    assert ref.n_patterns == 6 and ref.dropped == 1
    T = ref.n_tokens
    assert_same_encode(ref, gpu, T)
    for which in (0, 1):
        assert np.array_equal(gpu_tab(gpu, which)[:, :6], ref.patterns(which)[:, :6])
    _check_attn(ref, gpu, synth.queries(B, Hq, 128, step=1), bf16=True)
    # a multi-token decode append crossing a window boundary is split there
    k2, v2 = _inputs(B, H, 2 * W + 3, seed_off=13)
    ref.encode_append(to_oracle(k2, True), to_oracle(v2, True), update=1)
    gpu.encode_append(to_dev(k2, dt), to_dev(v2, dt), update_patterns=True)
    assert gpu.n_patterns == ref.n_patterns and gpu.dropped == ref.dropped
    assert_same_encode(ref, gpu, ref.n_tokens)


def test_determinism_and_checkpoint():
    """Two runs give byte-identical caches; a snapshot restored into a fresh
    buffer continues identically."""
    B, Hq, H, T = 2, 8, 2, 200
    k, v = _inputs(B, H, T)
    caches = []
    for _ in range(2):
        g, _, dt = make_pair(B, Hq, H, 512)
        g.init_patterns(to_dev(k, dt), to_dev(v, dt), 8)
        g.encode_append(to_dev(k, dt), to_dev(v, dt))
        caches.append(g)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].buf[:caches[0].layout.ws], caches[1].buf[:caches[1].layout.ws])
    snap = caches[0].snapshot()
    fresh, _, dt = make_pair(B, Hq, H, 512)
    fresh.restore(snap)
    k2, v2 = _inputs(B, H, 40, seed_off=3)
    for c in (caches[0], fresh):
        c.encode_append(to_dev(k2, dt), to_dev(v2, dt), update_patterns=True)
    q = to_dev(synth.queries(B, Hq, 128), dt)
    assert torch.equal(caches[0].attn_decode(q), fresh.attn_decode(q))
    torch.cuda.synchronize()
    assert torch.equal(caches[0].buf[:caches[0].layout.ws], fresh.buf[:fresh.layout.ws])


@pytest.mark.parametrize("bits,group,gq,mode", [
    (2, 32, 4, "pattern"), (2, 32, 1, "pattern"), (4, 64, 4, "pattern"), (4, 64, 8, "pattern"),
    (2, 64, 2, "pattern"), (4, 32, 3, "pattern"), (2, 32, 4, "kvarn"), (4, 64, 8, "kvarn"),
    # G = 64 with at most 4 q-heads: virtual half-groups fill the row block
    (2, 64, 4, "kvarn"), (2, 64, 3, "pattern"),
    # more q-heads per kv-head than one MFMA row block holds: further head blocks
    (2, 32, 7, "pattern"), (4, 32, 8, "pattern"), (2, 64, 12, "pattern"), (2, 32, 16, "pattern"),
    (2, 32, 6, "kvarn")])
@pytest.mark.parametrize("blocks", [1, 40, 4096])
@pytest.mark.parametrize("bf16", [True, False])
def test_attention_kernels_agree(bits, group, gq, mode, blocks, bf16):
    """The MFMA kernel (default) and the VALU kernel both match the oracle,
    for one block per unit up
    to many splits, ragged lengths, bfloat16 and binary32 inputs (a binary32
    query takes the binary16 hi + lo operand path)."""
    B, H, T = 2, 2, 1000
    gpu, ref, dt = make_pair(B, gq * H, H, 1024, bits=bits, group=group, mode=mode,
                             max_patterns=24, bf16=bf16)
    k, v = _inputs(B, H, T, seed_off=bits + gq)
    if mode == "pattern":
        ref.init_patterns(to_oracle(k[:, :, :256], bf16), to_oracle(v[:, :, :256], bf16), 24)
        gpu.init_patterns(to_dev(k[:, :, :256], dt), to_dev(v[:, :, :256], dt), 24)
    else:
        ref.init_patterns(to_oracle(k[:, :, :256], bf16), to_oracle(v[:, :, :256], bf16), 0)
        gpu.set_patterns(torch.from_numpy(ref.scales(0).reshape(B, H, 128).copy()).cuda(),
                         torch.from_numpy(ref.scales(1).reshape(B, H, 128).copy()).cuda())
    ref.encode_append(to_oracle(k, bf16), to_oracle(v, bf16))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    gpu.attn_blocks = blocks
    for step, qmul in ((0, 1.0), (1, 6.0)):          # flat and peaked softmax
        q = synth.queries(B, gq * H, 128, step=step) * np.float32(qmul)
        want = ref.attn_decode(to_oracle(q, bf16))
        errs = {}
        for kern in ("", "valu") if gq <= 8 else ("",):
            gpu.attn_kernel = kern or "auto"
            got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
            errs[kern or "default"] = float(np.abs(got - want).max())
        assert max(errs.values()) <= ATTN_TOL, errs


@pytest.mark.parametrize("bf16", [True, False])
def test_attention_query_dynamic_range(bf16):
    """Query heads far from unit scale: one head with |q| in the thousands,
    one around 1e-3, one with elements near 1e-9 among normal ones.  The QK
    operand's per-head exponent keeps every head in binary16 range."""
    B, H, gq, T = 2, 2, 4, 700
    gpu, ref, dt = make_pair(B, gq * H, H, 1024, max_patterns=16, bf16=bf16)
    k, v = _inputs(B, H, T, seed_off=11)
    ref.init_patterns(to_oracle(k[:, :, :256], bf16), to_oracle(v[:, :, :256], bf16), 16)
    gpu.init_patterns(to_dev(k[:, :, :256], dt), to_dev(v[:, :, :256], dt), 16)
    ref.encode_append(to_oracle(k, bf16), to_oracle(v, bf16))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    q = synth.queries(B, gq * H, 128, step=5).copy()
    q[:, 0::gq] *= np.float32(300.0)
    q[:, 1::gq] *= np.float32(1e-3)
    q[:, 2::gq, ::3] *= np.float32(1e-9)
    want = ref.attn_decode(to_oracle(q, bf16))
    got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
    assert np.abs(got - want).max() <= ATTN_TOL


def test_attention_repeated_calls_reset_counters():
    """The fused combine's arrival counters return to zero after each call, so
    repeated calls (and calls after appends) keep matching the oracle."""
    B, Hq, H = 2, 8, 2
    gpu, ref, dt = make_pair(B, Hq, H, 4096)
    k, v = _inputs(B, H, 3000)
    ref.init_patterns(to_oracle(k[:, :, :512], True), to_oracle(v[:, :, :512], True), 16)
    gpu.init_patterns(to_dev(k[:, :, :512], dt), to_dev(v[:, :, :512], dt), 16)
    gpu.attn_blocks = 64
    pos = 0
    for n in (1000, 1, 999, 1000):
        ref.encode_append(to_oracle(k[:, :, pos:pos + n], True), to_oracle(v[:, :, pos:pos + n], True))
        gpu.encode_append(to_dev(k[:, :, pos:pos + n], dt), to_dev(v[:, :, pos:pos + n], dt))
        pos += n
        q = synth.queries(B, Hq, 128, step=pos)
        want = ref.attn_decode(to_oracle(q, True))
        for _ in range(3):
            got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
            assert np.abs(got - want).max() <= ATTN_TOL
    assert int(gpu.region("cnt").view(torch.int32).abs().sum()) == 0


KVARN_CODE_SUM_TOL = 2.5e-4


@pytest.mark.parametrize("bits,group", [(2, 32), (2, 64), (4, 32), (4, 64)])
def test_kvarn_mfma_value_sums_unbiased(bits, group):
    """KVarN V sums sum_t p t s c and sum_t p t z nearly cancel in the rotated
    space, and the inverse rotation gathers any common offset into one output
    channel.  Code fields sitting low in the binary16 mantissa lost bits in
    the MFMA's own alignment (a one-signed error, 1.5e-3 here); with the
    fields moved up the default kernel stays within 2.5e-4 of the oracle, well
    inside the 2e-3 bar."""
    B, Hq, H, T = 2, 8, 2, 600
    gpu, ref, dt = make_pair(B, Hq, H, T + 8, bits=bits, group=group, mode="kvarn", max_patterns=0,
                             bf16=False)
    k, v = _inputs(B, H, T, seed_off=7 + bits + group)
    ref.init_patterns(to_oracle(k[:, :, :256], False), to_oracle(v[:, :, :256], False), 0)
    gpu.set_patterns(torch.from_numpy(ref.scales(0).reshape(B, H, 128).copy()).cuda(),
                     torch.from_numpy(ref.scales(1).reshape(B, H, 128).copy()).cuda())
    ref.encode_append(to_oracle(k, False), to_oracle(v, False))
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    errs = []
    for step in range(3):
        q = synth.queries(B, Hq, 128, step=step)
        want = ref.attn_decode(to_oracle(q, False))
        print(f"kvarn value sums bits={bits} group={group} step={step}", flush=True)
        got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
        errs.append(float(np.abs(got - want).max()))
    assert max(errs) <= KVARN_CODE_SUM_TOL, errs
