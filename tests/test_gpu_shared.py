"""GPU parity of batch-shared pattern tables (shared_patterns) against the oracle.

One table and one Chebyshev window per kv-head for the whole batch: k-means
over the B prefixes pooled batch-major, window min / max over every
sequence's decode vectors, one centre per kv-head per window.  Bar: tables,
codes, scales and indices bit-exact; attention within 2e-3 absolute.  Covers
the block-parallel and the one-block k-means (pooled rows beyond 8192), bulk
appends, window closures through single-token appends, bulk decode appends
(the block-folded window) and the one-launch decode step.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import synth
from parity_util import ATTN_TOL, assert_same_encode, gpu_tab, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu
D = 128


def _kv(B, H, T, off):
    return (synth.k_vectors(B, H, T, D, seed=synth.seed_for("k") + off),
            synth.v_vectors(B, H, T, D, seed=synth.seed_for("v") + off))


def _same_tables(gpu, ref, n):
    for w in (0, 1):
        g, r = gpu_tab(gpu, w)[:, :n], ref.patterns(w)[:, :n]
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
            f"{'KV'[w]} tables differ in {int((g != r).sum())} values"


def _attn(gpu, ref, B, Hq, bf16, step):
    dt = torch.bfloat16 if bf16 else torch.float32
    q = synth.queries(B, Hq, D, step=step)
    got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
    want = ref.attn_decode(to_oracle(q, bf16))
    err = float(np.abs(got - want).max())
    assert err <= ATTN_TOL, f"attention err {err}"


@pytest.mark.parametrize("B,n_init,P,bf16", [(3, 128, 16, True), (2, 4500, 8, True), (4, 96, 24, False)])
def test_shared_init_encode_attend(B, n_init, P, bf16):
    """Pooled k-means (B * n_init rows: 384 and 96 take the block-parallel
    kernel, 9000 the one-block kernel), bulk encode, attention."""
    H, Hq, T = 2, 8, n_init + 173
    gpu, ref, dt = make_pair(B, Hq, H, T + 8, max_patterns=P, bf16=bf16, shared_patterns=True)
    k, v = _kv(B, H, T, off=B + P)
    assert ref.init_patterns(to_oracle(k[:, :, :n_init], bf16), to_oracle(v[:, :, :n_init], bf16), P) == 0
    print(f"shared init B={B} n={n_init} P={P}", flush=True)
    gpu.init_patterns(to_dev(k[:, :, :n_init], dt), to_dev(v[:, :, :n_init], dt), P)
    torch.cuda.synchronize()
    _same_tables(gpu, ref, P)
    assert ref.encode_append(to_oracle(k, bf16), to_oracle(v, bf16)) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    assert_same_encode(ref, gpu, T)
    _attn(gpu, ref, B, Hq, bf16, step=1)


@pytest.mark.parametrize("fused", [True, False])
def test_shared_window_decode_steps(fused):
    """Decode steps with a window of 4 (centres from every sequence's vectors):
    the one-launch step or the two calls, against the oracle at every step."""
    B, H, Hq, T0, steps, P, W = 3, 2, 8, 260, 14, 12, 4
    gpu, ref, dt = make_pair(B, Hq, H, T0 + steps, max_patterns=P, pattern_window=W,
                             shared_patterns=True)
    k, v = _kv(B, H, T0 + steps, off=21)
    assert ref.init_patterns(to_oracle(k[:, :, :128], True), to_oracle(v[:, :, :128], True), 6) == 0
    gpu.init_patterns(to_dev(k[:, :, :128], dt), to_dev(v[:, :, :128], dt), 6)
    assert ref.encode_append(to_oracle(k[:, :, :T0], True), to_oracle(v[:, :, :T0], True)) == 0
    gpu.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1], v[:, :, t:t + 1]
        q = synth.queries(B, Hq, D, step=s)
        assert ref.encode_append(to_oracle(kn, True), to_oracle(vn, True), update=1) == 0
        want = ref.attn_decode(to_oracle(q, True))
        if fused:
            got = gpu.decode_step(to_dev(kn, dt), to_dev(vn, dt), to_dev(q, dt))
        else:
            gpu.encode_append(to_dev(kn, dt), to_dev(vn, dt), update_patterns=True)
            got = gpu.attn_decode(to_dev(q, dt))
        err = float(np.abs(got.cpu().numpy() - want).max())
        assert err <= ATTN_TOL, f"step {s}: attention err {err}"
        assert gpu.n_patterns == ref.n_patterns == min(6 + (s + 1) // W, P)
    assert gpu.dropped == ref.dropped == 0
    _same_tables(gpu, ref, ref.n_patterns)
    assert_same_encode(ref, gpu, T0 + steps)


def test_shared_bulk_decode_append():
    """A multi-token decode append (the block-folded window path), split at
    window boundaries, with the table filling up (dropped centres)."""
    B, H, Hq, T0, n, P, W = 2, 2, 8, 200, 23, 8, 5
    gpu, ref, dt = make_pair(B, Hq, H, T0 + n, max_patterns=P, pattern_window=W,
                             shared_patterns=True)
    k, v = _kv(B, H, T0 + n, off=33)
    assert ref.init_patterns(to_oracle(k[:, :, :64], True), to_oracle(v[:, :, :64], True), 5) == 0
    gpu.init_patterns(to_dev(k[:, :, :64], dt), to_dev(v[:, :, :64], dt), 5)
    assert ref.encode_append(to_oracle(k[:, :, :T0], True), to_oracle(v[:, :, :T0], True)) == 0
    gpu.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    kn, vn = k[:, :, T0:].copy(), v[:, :, T0:].copy()
    assert ref.encode_append(to_oracle(kn, True), to_oracle(vn, True), update=1) == 0
    gpu.encode_append(to_dev(kn, dt), to_dev(vn, dt), update_patterns=True)
    torch.cuda.synchronize()
    assert gpu.n_patterns == ref.n_patterns == P and gpu.dropped == ref.dropped == 1
    assert gpu.c.win_count == ref.win_count == n % W
    _same_tables(gpu, ref, P)
    assert_same_encode(ref, gpu, T0 + n)
    _attn(gpu, ref, B, Hq, True, step=4)
