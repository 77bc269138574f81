"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (default grid, no overrides).

The GPU encodes and attends over the whole cache; the oracle reproduces a few
sampled (batch, kv-head) units one by one, each as a one-unit cache fed the
same seeded inputs (units are independent: patterns, codes, scales and the
q-heads of one kv-head depend only on that unit's inputs).  Inputs are drawn
on the device by the seeded generators and copied to the host for the oracle;
nothing the HIP path computes is fed to the oracle.

Bar: k-means tables, codes, scales, indices / token scales bit-exact;
attention within 2e-3 absolute.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_kv_cache_encode_amd import KVCache, synth
from parity_util import ATTN_TOL, assert_same_encode, dev_to_oracle, gpu_tab

pytestmark = pytest.mark.gpu
D = 128


def _unit_ref(gq, max_tokens, **kw):
    """A one-unit oracle cache: one kv-head with its gq q-heads, bf16 inputs."""
    return O.RefCache(1, gq, 1, D, max_tokens, in_dtype=O.IN_BF16, **kw)


def _unit_in(t: torch.Tensor, b: int, h: int) -> np.ndarray:
    """One unit's rows [1][1][T][D] of a device input, as oracle input."""
    return dev_to_oracle(t[b:b + 1, h:h + 1].contiguous())


def _check_unit_attn(gpu_out, ref, q, b, h, gq):
    want = ref.attn_decode(dev_to_oracle(q[b:b + 1, h * gq:(h + 1) * gq].contiguous()))
    got = gpu_out[b:b + 1, h * gq:(h + 1) * gq].cpu().numpy()
    err = float(np.abs(got - want).max())
    assert err <= ATTN_TOL, f"unit ({b},{h}) attention err {err}"
    return err


def _pattern_workload(B, Hq, H, T, bits, group, P, W, samples, n_kmeans=2048, decode_steps=2):
    dev = torch.device("cuda", 0)
    gq = Hq // H
    steps = decode_steps
    k, v = synth.device_kv(B, H, T + steps, D, device=dev, dtype=torch.bfloat16)
    gpu = KVCache(B, Hq, H, T + steps + 64, bits=bits, group=group, mode="pattern",
                  max_patterns=P, pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16)
    nk = min(n_kmeans, T)
    gpu.init_patterns(k[:, :, :nk].contiguous(), v[:, :, :nk].contiguous(), P)
    gpu.encode_append(k[:, :, :T].contiguous(), v[:, :, :T].contiguous())
    q = synth.device_queries(B, Hq, D, device=dev, dtype=torch.bfloat16)
    out0 = gpu.attn_decode(q)
    outs = []
    for s in range(steps):
        gpu.encode_append(k[:, :, T + s:T + s + 1].contiguous(), v[:, :, T + s:T + s + 1].contiguous(),
                          update_patterns=True)
        qs = synth.device_queries(B, Hq, D, step=s + 1, device=dev, dtype=torch.bfloat16)
        outs.append((qs, gpu.attn_decode(qs)))
    torch.cuda.synchronize()
    errs = []
    for (b, h) in samples:
        u = b * H + h
        ref = _unit_ref(gq, T + steps + 64, bits=bits, group=group, mode=O.PATTERN,
                        max_patterns=P, pattern_window=W, v_alpha=0.05)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :nk], vu[:, :, :nk], P) == 0
        for which in (0, 1):
            assert np.array_equal(gpu_tab(gpu, which)[u, :P], ref.patterns(which)[0, :P]), \
                f"unit {u}: {'KV'[which]} k-means table differs"
        assert ref.encode_append(ku[:, :, :T], vu[:, :, :T]) == 0
        errs.append(_check_unit_attn(out0, ref, q, b, h, gq))
        for s in range(steps):
            assert ref.encode_append(ku[:, :, T + s:T + s + 1], vu[:, :, T + s:T + s + 1], update=1) == 0
            errs.append(_check_unit_attn(outs[s][1], ref, outs[s][0], b, h, gq))
        assert_same_encode(ref, gpu, T + steps, units=[u], ref_units=[0])
    return max(errs)


@pytest.mark.parametrize("T", [4096, 32768])
def test_llama8b_decode_fullsize(T):
    """Llama-3-8B-shaped layer: batch 8, 32 q / 8 kv heads, bf16, 2-bit group
    32, 32 patterns, window 128; prefix encode, two decode steps."""
    err = _pattern_workload(8, 32, 8, T, 2, 32, 32, 128, samples=[(0, 0), (3, 5), (7, 7)])
    print(f"T={T}: max attention err {err:.2e}")


def test_long_context_4bit_fullsize():
    """Batch 1, 8 kv heads, context 131072, 4-bit group 64, 64 patterns."""
    err = _pattern_workload(1, 32, 8, 131072, 4, 64, 64, 128, samples=[(0, 0), (0, 6)],
                            decode_steps=1)
    print(f"max attention err {err:.2e}")


def test_kvarn_breadth_fullsize():
    """64 samples x 16384 tokens, 8 kv heads, 2-bit Hadamard + dual-axis
    normalisation, decode attention per sample."""
    dev = torch.device("cuda", 0)
    B, Hq, H, T, n_init = 64, 32, 8, 16384, 256
    gq = Hq // H
    k, v = synth.device_kv(B, H, T, D, device=dev, dtype=torch.bfloat16)
    gpu = KVCache(B, Hq, H, T, bits=2, group=32, mode="kvarn", max_patterns=0,
                  in_dtype=torch.bfloat16)
    gpu.init_patterns(k[:, :, :n_init].contiguous(), v[:, :, :n_init].contiguous(), 0)
    torch.cuda.synchronize()
    samples = [(0, 0), (31, 4), (63, 7)]
    refs = {}
    ks, vs = gpu_tab(gpu, 0).copy(), gpu_tab(gpu, 1).copy()
    for (b, h) in samples:
        u = b * H + h
        ref = O.RefCache(1, gq, 1, D, T, bits=2, group=32, mode=O.KVARN, max_patterns=0,
                         in_dtype=O.IN_BF16)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :n_init], vu[:, :, :n_init], 0) == 0
        # channel scales agree within rounding (binary64 sums in another order)
        np.testing.assert_allclose(ks[u], ref.scales(0)[0], rtol=1e-6)
        np.testing.assert_allclose(vs[u], ref.scales(1)[0], rtol=1e-6)
        ks[u], vs[u] = ref.scales(0)[0], ref.scales(1)[0]
        refs[(b, h)] = (ref, ku, vu)
    # the sampled units encode with the oracle's channel scales (oracle -> GPU only)
    gpu.set_patterns(torch.from_numpy(ks.reshape(B, H, D)).to(dev),
                     torch.from_numpy(vs.reshape(B, H, D)).to(dev))
    gpu.encode_append(k, v)
    q = synth.device_queries(B, Hq, D, device=dev, dtype=torch.bfloat16)
    out = gpu.attn_decode(q)
    torch.cuda.synchronize()
    for (b, h), (ref, ku, vu) in refs.items():
        assert ref.encode_append(ku, vu) == 0
        assert_same_encode(ref, gpu, T, units=[b * H + h], ref_units=[0])
        _check_unit_attn(out, ref, q, b, h, gq)


def test_streaming_qwen_fullsize():
    """Qwen2.5-7B-shaped layer (28 q / 4 kv heads), batch 32, 32768-token
    prefix then 256 append + decode steps whose K mean drifts (step j adds
    0.01 j u, u ~ N(0, I)); 2-bit group 32, 64 k-means patterns plus one
    Chebyshev centre per 128 decode steps (66 at the end).
    Parity at sampled steps; the error against exact attention over the
    unquantised inputs is reported per sampled step."""
    dev = torch.device("cuda", 0)
    B, Hq, H, T0, S, P, W = 32, 28, 4, 32768, 256, 80, 128
    gq = Hq // H
    k, v = synth.device_kv(B, H, T0 + S, D, device=dev, dtype=torch.float32)
    drift = torch.from_numpy(synth.drift_dirs(B, H, D)).to(dev)
    ramp = torch.arange(1, S + 1, device=dev, dtype=torch.float32)
    k[:, :, T0:] += 0.01 * ramp[None, None, :, None] * drift[:, :, None, :]
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    gpu = KVCache(B, Hq, H, T0 + S + 64, bits=2, group=32, mode="pattern", max_patterns=P,
                  pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16)
    gpu.init_patterns(k[:, :, :2048].contiguous(), v[:, :, :2048].contiguous(), 64)
    gpu.encode_append(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
    check_at = {0, 85, 170, 255}
    outs = {}
    for s in range(S):
        gpu.encode_append(k[:, :, T0 + s:T0 + s + 1].contiguous(),
                          v[:, :, T0 + s:T0 + s + 1].contiguous(), update_patterns=True)
        q = synth.device_queries(B, Hq, D, step=s, device=dev, dtype=torch.bfloat16)
        o = gpu.attn_decode(q)
        if s in check_at:
            outs[s] = (q, o.clone())
    torch.cuda.synchronize()
    report = []
    for (b, h) in [(0, 0), (17, 3)]:
        ref = O.RefCache(1, gq, 1, D, T0 + S + 64, bits=2, group=32, mode=O.PATTERN,
                         max_patterns=P, pattern_window=W, v_alpha=0.05, in_dtype=O.IN_BF16)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :2048], vu[:, :, :2048], 64) == 0
        assert ref.encode_append(ku[:, :, :T0], vu[:, :, :T0]) == 0
        for s in range(S):
            assert ref.encode_append(ku[:, :, T0 + s:T0 + s + 1], vu[:, :, T0 + s:T0 + s + 1],
                                     update=1) == 0
            if s in check_at:
                q, o = outs[s]
                err = _check_unit_attn(o, ref, q, b, h, gq)
                exact = O.attn_exact(synth.bf16_bits_to_f32(ku[:, :, :T0 + s + 1]),
                                     synth.bf16_bits_to_f32(vu[:, :, :T0 + s + 1]),
                                     synth.bf16_bits_to_f32(
                                         dev_to_oracle(q[b:b + 1, h * gq:(h + 1) * gq].contiguous())),
                                     gq)
                qerr = float(np.abs(o[b:b + 1, h * gq:(h + 1) * gq].cpu().numpy() - exact).max())
                report.append((b, h, s, err, qerr))
        assert ref.n_patterns == gpu.n_patterns == 66 and ref.dropped == gpu.dropped == 0
        assert_same_encode(ref, gpu, T0 + S, units=[b * H + h], ref_units=[0])
    for b, h, s, err, qerr in report:
        print(f"unit ({b},{h}) step {s}: |gpu - oracle| {err:.2e}, |gpu - exact fp32| {qerr:.3e}")


def test_kivi_fullsize():
    """The step's shapes with K per channel over 128-token blocks: batch 8,
    32 q / 8 kv heads, 32768-token prefix then 64 single-token decode appends
    (an open block), 2-bit group 32, 32 patterns, window 128."""
    from parity_util import assert_same_kch
    dev = torch.device("cuda", 0)
    B, Hq, H, T, S, P = 8, 32, 8, 32768, 64, 32
    gq = Hq // H
    k, v = synth.device_kv(B, H, T + S, D, device=dev, dtype=torch.bfloat16)
    gpu = KVCache(B, Hq, H, T + S + 64, bits=2, group=32, mode="pattern", max_patterns=P,
                  pattern_window=128, v_alpha=0.05, in_dtype=torch.bfloat16, k_per_channel=True)
    gpu.init_patterns(k[:, :, :2048].contiguous(), v[:, :, :2048].contiguous(), P)
    gpu.encode_append(k[:, :, :T].contiguous(), v[:, :, :T].contiguous())
    for s in range(S):
        gpu.encode_append(k[:, :, T + s:T + s + 1].contiguous(), v[:, :, T + s:T + s + 1].contiguous(),
                          update_patterns=True)
    q = synth.device_queries(B, Hq, D, device=dev, dtype=torch.bfloat16)
    out = gpu.attn_decode(q)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (5, 3), (7, 7)]:
        ref = _unit_ref(gq, T + S + 64, bits=2, group=32, mode=O.PATTERN, max_patterns=P,
                        pattern_window=128, v_alpha=0.05, k_per_channel=True)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :2048], vu[:, :, :2048], P) == 0
        assert ref.encode_append(ku[:, :, :T], vu[:, :, :T]) == 0
        for s in range(S):
            assert ref.encode_append(ku[:, :, T + s:T + s + 1], vu[:, :, T + s:T + s + 1], update=1) == 0
        print(f"k per channel full size unit ({b},{h})", flush=True)
        assert_same_kch(ref, gpu, T + S, units=[b * H + h], ref_units=[0])
        err = _check_unit_attn(out, ref, q, b, h, gq)
        print(f"unit ({b},{h}): attention err {err:.2e}")


def test_nsn_breadth_fullsize():
    """64 samples x 16384 tokens, 8 kv heads, the NSN scalar mode at 2 bits
    (group 32), centres from the first 256 tokens."""
    dev = torch.device("cuda", 0)
    B, Hq, H, T, n_init = 64, 32, 8, 16384, 256
    gq = Hq // H
    k, v = synth.device_kv(B, H, T, D, device=dev, dtype=torch.bfloat16)
    gpu = KVCache(B, Hq, H, T, bits=2, group=32, mode="nsn", max_patterns=0, in_dtype=torch.bfloat16)
    gpu.init_patterns(k[:, :, :n_init].contiguous(), v[:, :, :n_init].contiguous(), 0)
    torch.cuda.synchronize()
    samples = [(0, 0), (40, 2), (63, 7)]
    refs = {}
    mk, mv = gpu_tab(gpu, 0).copy(), gpu_tab(gpu, 1).copy()
    for (b, h) in samples:
        u = b * H + h
        ref = O.RefCache(1, gq, 1, D, T, bits=2, group=32, mode=O.NSN, max_patterns=0,
                         in_dtype=O.IN_BF16)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :n_init], vu[:, :, :n_init], 0) == 0
        # centres agree within rounding (binary64 sums in another order)
        np.testing.assert_allclose(mk[u], ref.scales(0)[0], rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(mv[u], ref.scales(1)[0], rtol=1e-6, atol=1e-7)
        mk[u], mv[u] = ref.scales(0)[0], ref.scales(1)[0]
        refs[(b, h)] = (ref, ku, vu)
    # the sampled units encode with the oracle's centres (oracle -> GPU only)
    gpu.set_patterns(torch.from_numpy(mk.reshape(B, H, D)).to(dev),
                     torch.from_numpy(mv.reshape(B, H, D)).to(dev))
    gpu.encode_append(k, v)
    q = synth.device_queries(B, Hq, D, device=dev, dtype=torch.bfloat16)
    out = gpu.attn_decode(q)
    torch.cuda.synchronize()
    for (b, h), (ref, ku, vu) in refs.items():
        assert ref.encode_append(ku, vu) == 0
        print(f"nsn full size unit ({b},{h})", flush=True)
        assert_same_encode(ref, gpu, T, units=[b * H + h], ref_units=[0])
        _check_unit_attn(out, ref, q, b, h, gq)


def _used_regions(cache):
    """Device views of a cache's used contents (token-indexed regions cut at
    n_tokens, tables at n_patterns, the window state whole)."""
    c, L = cache.cfg, cache.layout
    U, T, tc = c.batch * c.n_kv_heads, cache.n_tokens, L.token_cap
    rec = D * c.bits // 8
    out = {}
    for w in "kv":
        if w == "k":
            out["k_codes"] = cache.region("k_codes").view(U, tc * rec)[:, :T * rec]
        else:
            out["v_codes"] = cache.region("v_codes").view(U, tc // 32, -1)[:, :(T + 31) // 32]
        out[w + "_sz"] = cache.region(w + "_sz").view(U, tc, -1)[:, :T]
        out[w + "_idx"] = cache.region(w + "_idx").view(U, tc)[:, :T]
        out[w + "_tab"] = cache.region(w + "_tab").view(cache.pattern_units, c.max_patterns, -1)[
            :, :cache.n_patterns]
        out[w + "_win"] = cache.region(w + "_win")
    return out


@pytest.mark.parametrize("shape", ["llama8b_ctx32k_2bit", "llama8b_ctx4k_2bit", "long_ctx128k_4bit"])
def test_decode_step_fullsize(shape):
    """The kernel the benchmark times: the one-launch decode step
    (kvq_decode_step, default grid) at full size, 130 steps with the
    Chebyshev window at 128 (PatternKV section 3.1, Eq 5), so the 128th step
    closes a window and the table grows by one pattern (Llama shape: 32 -> 33,
    which moves the pattern-mass product to a wider instantiation; long
    context: 64 -> 65, past the one-hot path).  Every step also runs through a
    copy of the cache driven by the two separate calls; the two caches' used
    contents must stay byte-identical and their outputs within 2e-3.  The
    oracle reproduces sampled units at steps 0, 126, 127 (the closing step),
    128 and 129.  The Llama shape runs at 32768 and at 4096 cached tokens."""
    dev = torch.device("cuda", 0)
    if shape == "llama8b_ctx32k_2bit":
        B, Hq, H, T0, bits, group, P = 8, 32, 8, 32768, 2, 32, 32
        samples = [(0, 0), (3, 5), (7, 7)]
    elif shape == "llama8b_ctx4k_2bit":
        # the single-layer Llama-3-8B decode shape at 4096 tokens
        B, Hq, H, T0, bits, group, P = 8, 32, 8, 4096, 2, 32, 32
        samples = [(0, 3), (6, 1)]
    else:
        B, Hq, H, T0, bits, group, P = 1, 32, 8, 131072, 4, 64, 64
        samples = [(0, 1), (0, 6)]
    W, steps, gq = 128, 130, Hq // H
    check = {0, 126, 127, 128, 129}
    maxp = P + 2
    k, v = synth.device_kv(B, H, T0 + steps, D, device=dev, dtype=torch.bfloat16)
    gpu = KVCache(B, Hq, H, T0 + steps, bits=bits, group=group, mode="pattern",
                  max_patterns=maxp, pattern_window=W, v_alpha=0.05, in_dtype=torch.bfloat16)
    nk = 2048
    gpu.init_patterns(k[:, :, :nk].contiguous(), v[:, :, :nk].contiguous(), P)
    gpu.encode_append(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
    split = gpu.clone()
    outs = {}
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous()
        q = synth.device_queries(B, Hq, D, step=s + 1, device=dev, dtype=torch.bfloat16)
        out_f = gpu.decode_step(kn, vn, q)
        split.encode_append(kn, vn, update_patterns=True)
        out_s = split.attn_decode(q)
        d = float((out_f - out_s).abs().max())
        assert d <= ATTN_TOL, f"step {s}: one-launch vs two calls differ by {d}"
        if s in check:
            outs[s] = (q, out_f.clone())
    torch.cuda.synchronize()
    print(f"{shape}: {steps} steps, patterns {gpu.n_patterns}", flush=True)
    assert gpu.n_patterns == split.n_patterns == P + 1
    a, b_ = _used_regions(gpu), _used_regions(split)
    for name in a:
        assert torch.equal(a[name], b_[name]), f"{name} differs between the one-launch step and the two calls"
    errs = []
    for (b, h) in samples:
        u = b * H + h
        ref = _unit_ref(gq, T0 + steps, bits=bits, group=group, mode=O.PATTERN,
                        max_patterns=maxp, pattern_window=W, v_alpha=0.05)
        ku, vu = _unit_in(k, b, h), _unit_in(v, b, h)
        assert ref.init_patterns(ku[:, :, :nk], vu[:, :, :nk], P) == 0
        assert ref.encode_append(ku[:, :, :T0], vu[:, :, :T0]) == 0
        for s in range(steps):
            assert ref.encode_append(ku[:, :, T0 + s:T0 + s + 1], vu[:, :, T0 + s:T0 + s + 1],
                                     update=1) == 0
            if s in check:
                errs.append(_check_unit_attn(outs[s][1], ref, outs[s][0], b, h, gq))
        assert ref.n_patterns == P + 1
        for which in (0, 1):
            assert np.array_equal(gpu_tab(gpu, which)[u, :P + 1], ref.patterns(which)[0, :P + 1]), \
                f"unit {u}: {'KV'[which]} table differs after the window closure"
        assert_same_encode(ref, gpu, T0 + steps, units=[u], ref_units=[0])
    print(f"{shape}: max attention err {max(errs):.2e} over {len(errs)} checks", flush=True)
