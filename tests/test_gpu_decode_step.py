"""GPU parity of the one-launch decode step (kvq_decode_step): append one
token and attend over the cache including it.

Each case runs the same decode stream through a cache driven by
kvq_decode_step and through a copy driven by the two separate calls
(kvq_encode_append with n_new = 1, then kvq_attn_decode), and through the
oracle.  Bar: the caches' used contents (codes, scales, indices, pattern
tables, window state) byte-identical after every step; attention within
2e-3 absolute of the oracle at every step.  Window closures (a new pattern
mid-stream), ragged lengths and split counts from one to many are covered.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_kv_cache_encode_amd import KVCache, synth
from parity_util import ATTN_TOL, assert_same_encode, to_dev, to_oracle

pytestmark = pytest.mark.gpu
D = 128


def _used_bytes(cache):
    """The cache's used contents as host arrays, keyed by region."""
    c, L = cache.cfg, cache.layout
    U, T, tc = c.batch * c.n_kv_heads, cache.n_tokens, L.token_cap
    rec = D * c.bits // 8
    out = {}
    for w in "kv":
        out[w + "_codes"] = cache.region(w + "_codes").cpu().numpy().reshape(U, tc * rec)[:, :T * rec] \
            if w == "k" else \
            cache.region(w + "_codes").cpu().numpy().reshape(U, tc // 32, -1)[:, :(T + 31) // 32]
        out[w + "_sz"] = cache.region(w + "_sz").cpu().numpy().reshape(U, tc, -1)[:, :T]
        if cache.mode == "pattern":
            out[w + "_idx"] = cache.region(w + "_idx").cpu().numpy().reshape(U, tc)[:, :T]
            out[w + "_tab"] = cache.region(w + "_tab").cpu().numpy().reshape(U, c.max_patterns, -1)[
                :, :cache.n_patterns]
            out[w + "_win"] = cache.region(w + "_win").cpu().numpy()
        else:
            out[w + "_t16"] = cache.region(w + "_t16").cpu().numpy().reshape(U, tc, -1)[:, :T]
    return out


def _run(B, Hq, H, T0, steps, *, bits=2, group=32, mode="pattern", P=16, W=8, bf16=True,
         blocks=None, seed_off=0):
    dt = torch.bfloat16 if bf16 else torch.float32
    gq = Hq // H
    k = synth.k_vectors(B, H, T0 + steps, D, seed=synth.seed_for("k") + seed_off)
    v = synth.v_vectors(B, H, T0 + steps, D, seed=synth.seed_for("v") + seed_off)
    fused = KVCache(B, Hq, H, T0 + steps, bits=bits, group=group, mode=mode, max_patterns=P,
                    pattern_window=W, v_alpha=0.05, in_dtype=dt)
    if blocks is not None:
        fused.attn_blocks = blocks
    ref = O.RefCache(B, Hq, H, D, T0 + steps, bits=bits, group=group,
                     mode=O.PATTERN if mode == "pattern" else O.KVARN, max_patterns=P,
                     pattern_window=W, v_alpha=0.05, in_dtype=O.IN_BF16 if bf16 else O.IN_F32)
    n_init = min(256, T0) if T0 else 0
    p0 = min(P - 4, n_init)      # room for window centres
    if mode == "pattern" and n_init:
        assert ref.init_patterns(to_oracle(k[:, :, :n_init], bf16), to_oracle(v[:, :, :n_init], bf16),
                                 p0) == 0
        fused.init_patterns(to_dev(k[:, :, :n_init], dt), to_dev(v[:, :, :n_init], dt), p0)
    elif mode != "pattern":
        assert ref.init_patterns(to_oracle(k[:, :, :256], bf16), to_oracle(v[:, :, :256], bf16), 0) == 0
        fused.set_patterns(torch.from_numpy(ref.scales(0).reshape(B, H, D).copy()).cuda(),
                           torch.from_numpy(ref.scales(1).reshape(B, H, D).copy()).cuda())
    if T0:
        assert ref.encode_append(to_oracle(k[:, :, :T0], bf16), to_oracle(v[:, :, :T0], bf16)) == 0
        fused.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    split = fused.clone()
    errs = []
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1], v[:, :, t:t + 1]
        q = synth.queries(B, Hq, D, step=s)
        qd = to_dev(q, dt)
        out_f = fused.decode_step(to_dev(kn, dt), to_dev(vn, dt), qd)
        split.encode_append(to_dev(kn, dt), to_dev(vn, dt), update_patterns=True)
        out_s = split.attn_decode(qd)
        assert ref.encode_append(to_oracle(kn, bf16), to_oracle(vn, bf16), update=1) == 0
        want = ref.attn_decode(to_oracle(q, bf16))
        got_f, got_s = out_f.cpu().numpy(), out_s.cpu().numpy()
        err = float(np.abs(got_f - want).max())
        assert err <= ATTN_TOL, f"step {s}: fused attention err {err}"
        assert float(np.abs(got_f - got_s).max()) <= ATTN_TOL
        errs.append(err)
        assert fused.n_tokens == split.n_tokens == t + 1
        assert fused.n_patterns == split.n_patterns == ref.n_patterns
        a, b = _used_bytes(fused), _used_bytes(split)
        for name in a:
            assert np.array_equal(a[name], b[name]), f"step {s}: {name} differs"
    assert_same_encode(ref, fused, T0 + steps)
    return max(errs)


@pytest.mark.parametrize("T0", [1, 63, 300])
def test_decode_step_llama_gqa4(T0):
    """GQA 4, 2-bit group 32, window 8 (two pattern closures in 20 steps)."""
    _run(2, 8, 2, T0, 20)


@pytest.mark.parametrize("blocks", [1, 40, 4096])
def test_decode_step_split_counts(blocks):
    """One split per unit up to many; 16 patterns grow to 19 (the one-hot
    path changes width mid-stream)."""
    _run(2, 8, 2, 700, 12, P=20, W=4, blocks=blocks, seed_off=3)


def test_decode_step_4bit_gqa8_binary32():
    """4-bit group 64, GQA 8, binary32 inputs (hi + lo query operand)."""
    _run(1, 16, 2, 500, 10, bits=4, group=64, P=40, W=6, bf16=False, seed_off=5)


def test_decode_step_group64_gqa4():
    """2-bit group 64 with 4 q-heads per kv-head (each stored group read as two
    virtual groups sharing its scale and zero point)."""
    _run(2, 8, 2, 350, 8, group=64, P=20, W=4, seed_off=11)


@pytest.mark.parametrize("Hq,group,blocks", [(14, 32, None), (14, 32, 4096), (24, 64, None),
                                             (32, 32, 40)])
def test_decode_step_several_head_blocks(Hq, group, blocks):
    """More q-heads per kv-head than one MFMA row block holds (7 and 16 at
    group 32, 12 at group 64): every q-head block of split 0 appends the new
    token (the same bytes) for its own heads' partials and the first alone
    updates and closes the Chebyshev window; results and cache bytes equal
    the separate calls over window closures, from one split per unit to
    many."""
    _run(2, Hq, 2, 400, 6, group=group, P=20, W=4, blocks=blocks, seed_off=9)


def test_decode_step_kvarn_head_blocks():
    """KVarN mode with two q-head blocks per unit in one launch."""
    _run(2, 12, 2, 300, 6, mode="kvarn", P=0, W=0, seed_off=13)


@pytest.mark.parametrize("group,bf16", [(32, True), (64, False)])
def test_decode_step_kvarn(group, bf16):
    """KVarN mode in one launch: the new token's term in the rotated space
    (q' . u^ t, partial t u^); group 64 with 4 q-heads takes the virtual
    half-groups."""
    _run(2, 8, 2, 300, 6, group=group, mode="kvarn", P=0, W=0, bf16=bf16, seed_off=7)


def test_decode_step_capacity_error_writes_nothing():
    B, Hq, H, T = 1, 4, 1, 64
    k = synth.k_vectors(B, H, T, D)
    v = synth.v_vectors(B, H, T, D)
    gpu = KVCache(B, Hq, H, T, max_patterns=8, in_dtype=torch.bfloat16)
    gpu.init_patterns(to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16), 8)
    gpu.encode_append(to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16))
    before = gpu.buf.clone()
    q = to_dev(synth.queries(B, Hq, D), torch.bfloat16)
    with pytest.raises(Exception):
        gpu.decode_step(to_dev(k[:, :, :1], torch.bfloat16), to_dev(v[:, :, :1], torch.bfloat16), q)
    torch.cuda.synchronize()
    assert gpu.n_tokens == T
    assert torch.equal(before, gpu.buf)
