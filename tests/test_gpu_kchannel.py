"""GPU parity of K per channel (k_per_channel) against the oracle.

K is quantised per channel over blocks of 128 tokens (PatternKV's KIVI-style
setting); the open block's residuals wait in binary16.  Bar: K indices, the
complete blocks' codes and (s, z) words, the open block's residuals and all
of V bit-exact; dequant bit-exact; attention within 2e-3 absolute.  Cases:
bulk appends (two complete blocks and an open one), appends that complete a
block whose first tokens came earlier (residuals read back from the buffer),
single-token decode appends across a block boundary with the Chebyshev
window, 4-bit codes, binary32 inputs, and the decode step.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import synth
from parity_util import ATTN_TOL, assert_same_kch, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu
D = 128


def _kv(B, H, T, off):
    return (synth.k_vectors(B, H, T, D, seed=synth.seed_for("k") + off),
            synth.v_vectors(B, H, T, D, seed=synth.seed_for("v") + off))


def _check(gpu, ref, B, Hq, T, bf16, step):
    torch.cuda.synchronize()
    assert gpu.n_tokens == ref.n_tokens == T
    assert_same_kch(ref, gpu, T)
    for w in (0, 1):
        g = gpu.dequant(w, 0, T).cpu().numpy()
        r = ref.dequant(w, 0, T)
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"{'KV'[w]} dequant differs"
    dt = torch.bfloat16 if bf16 else torch.float32
    q = synth.queries(B, Hq, D, step=step)
    print(f"k per channel attention T={T}", flush=True)
    got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
    want = ref.attn_decode(to_oracle(q, bf16))
    err = float(np.abs(got - want).max())
    assert err <= ATTN_TOL, f"attention err {err}"


@pytest.mark.parametrize("bits,group,bf16", [(2, 32, True), (4, 64, True), (2, 32, False)])
def test_kch_bulk_encode_attend(bits, group, bf16):
    B, H, Hq, T, P = 2, 2, 8, 300, 8
    gpu, ref, dt = make_pair(B, Hq, H, 384, bits=bits, group=group, max_patterns=P, bf16=bf16,
                             k_per_channel=True)
    k, v = _kv(B, H, T, off=bits + group)
    assert ref.init_patterns(to_oracle(k[:, :, :128], bf16), to_oracle(v[:, :, :128], bf16), P) == 0
    gpu.init_patterns(to_dev(k[:, :, :128], dt), to_dev(v[:, :, :128], dt), P)
    assert ref.encode_append(to_oracle(k, bf16), to_oracle(v, bf16)) == 0
    print(f"k per channel bulk bits={bits} group={group} bf16={bf16}", flush=True)
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    _check(gpu, ref, B, Hq, T, bf16, step=1)


def test_kch_chunked_appends_across_blocks():
    """100 tokens, then 50 (completes block 0 from buffered residuals), then
    170 (completes block 1 and 2, opens block 3), then 5."""
    B, H, Hq, P = 2, 2, 8, 6
    gpu, ref, dt = make_pair(B, Hq, H, 512, max_patterns=P, k_per_channel=True)
    k, v = _kv(B, H, 325, off=11)
    assert ref.init_patterns(to_oracle(k[:, :, :64], True), to_oracle(v[:, :, :64], True), P) == 0
    gpu.init_patterns(to_dev(k[:, :, :64], dt), to_dev(v[:, :, :64], dt), P)
    t = 0
    for n in (100, 50, 170, 5):
        kk, vv = k[:, :, t:t + n].copy(), v[:, :, t:t + n].copy()
        assert ref.encode_append(to_oracle(kk, True), to_oracle(vv, True)) == 0
        print(f"k per channel append {t}..{t + n}", flush=True)
        gpu.encode_append(to_dev(kk, dt), to_dev(vv, dt))
        t += n
        _check(gpu, ref, B, Hq, t, True, step=t % 7)


@pytest.mark.parametrize("fused_call", [False, True])
def test_kch_decode_appends_with_window(fused_call):
    """Single-token decode appends across the 256 boundary with a Chebyshev
    window of 8 (new patterns mid-block), as encode_append + attn_decode or
    as the decode step (which runs the same two calls here)."""
    B, H, Hq, P, W, T0, steps = 2, 2, 8, 12, 8, 250, 12
    gpu, ref, dt = make_pair(B, Hq, H, 300, max_patterns=P, pattern_window=W, k_per_channel=True)
    k, v = _kv(B, H, T0 + steps, off=13)
    assert ref.init_patterns(to_oracle(k[:, :, :96], True), to_oracle(v[:, :, :96], True), 4) == 0
    gpu.init_patterns(to_dev(k[:, :, :96], dt), to_dev(v[:, :, :96], dt), 4)
    assert ref.encode_append(to_oracle(k[:, :, :T0], True), to_oracle(v[:, :, :T0], True)) == 0
    gpu.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1].copy(), v[:, :, t:t + 1].copy()
        q = synth.queries(B, Hq, D, step=s)
        assert ref.encode_append(to_oracle(kn, True), to_oracle(vn, True), update=1) == 0
        want = ref.attn_decode(to_oracle(q, True))
        print(f"k per channel decode step {s}", flush=True)
        if fused_call:
            got = gpu.decode_step(to_dev(kn, dt), to_dev(vn, dt), to_dev(q, dt))
        else:
            gpu.encode_append(to_dev(kn, dt), to_dev(vn, dt), update_patterns=True)
            got = gpu.attn_decode(to_dev(q, dt))
        err = float(np.abs(got.cpu().numpy() - want).max())
        assert err <= ATTN_TOL, f"step {s}: attention err {err}"
        assert gpu.n_patterns == ref.n_patterns
    _check(gpu, ref, B, Hq, T0 + steps, True, step=3)


@pytest.mark.parametrize("bits,group,gq,npat", [(2, 32, 4, 32), (2, 64, 4, 16), (2, 64, 8, 24),
                                                (4, 32, 7, 64), (4, 64, 3, 8), (2, 32, 16, 0)])
@pytest.mark.parametrize("blocks", [1, 256])
def test_kch_attention_kernels_agree(bits, group, gq, npat, blocks):
    """The matrix-core kernel (q * s operand per tile of a complete block,
    VALU scores for the open block) and the VALU kernel match the oracle:
    several blocks plus an open one, one or many splits, virtual groups at
    G = 64, several q-head blocks (7 and 16 q-heads per kv-head)."""
    B, H, T = 2, 2, 3 * 128 + 70
    gpu, ref, dt = make_pair(B, gq * H, H, 512, bits=bits, group=group, max_patterns=max(npat, 1),
                             k_per_channel=True)
    k, v = _kv(B, H, T, off=gq + bits)
    if npat:
        assert ref.init_patterns(to_oracle(k[:, :, :128], True), to_oracle(v[:, :, :128], True), npat) == 0
        gpu.init_patterns(to_dev(k[:, :, :128], dt), to_dev(v[:, :, :128], dt), npat)
    assert ref.encode_append(to_oracle(k, True), to_oracle(v, True)) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    gpu.attn_blocks = blocks
    for step, qmul in ((0, 1.0), (1, 6.0)):
        q = synth.queries(B, gq * H, D, step=step) * np.float32(qmul)
        want = ref.attn_decode(to_oracle(q, True))
        errs = {}
        for kern in ("", "valu") if gq <= 8 else ("",):
            gpu.attn_kernel = kern or "auto"
            print(f"k per channel kernels bits={bits} group={group} gq={gq} kern={kern or 'mfma'}",
                  flush=True)
            got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
            errs[kern or "mfma"] = float(np.abs(got - want).max())
        assert max(errs.values()) <= ATTN_TOL, errs


def test_kch_single_token_appends_without_patterns():
    """One-token appends store their residual from the encode itself (no
    pattern table here, so the residual is the raw vector); the 128th token
    closes the block through the block quantiser instead."""
    B, H, Hq, T0, steps = 2, 2, 8, 120, 12
    gpu, ref, dt = make_pair(B, Hq, H, 256, max_patterns=0, pattern_window=0, k_per_channel=True)
    k, v = _kv(B, H, T0 + steps, off=17)
    assert ref.encode_append(to_oracle(k[:, :, :T0], True), to_oracle(v[:, :, :T0], True)) == 0
    gpu.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1].copy(), v[:, :, t:t + 1].copy()
        assert ref.encode_append(to_oracle(kn, True), to_oracle(vn, True)) == 0
        print(f"k per channel single token {t}", flush=True)
        gpu.encode_append(to_dev(kn, dt), to_dev(vn, dt))
        _check(gpu, ref, B, Hq, t + 1, True, step=s)
