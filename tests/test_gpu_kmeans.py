"""GPU pattern mining (kvq_init_patterns, PATTERN mode) against the oracle.

The GPU k-means runs the oracle's Lloyd iteration in binary64 with the same
operation order (channel-ordered distance sums, lowest index on ties, member
sums in token order), so the fp32 pattern tables must be bit-identical.
Cases cover prefixes that end inside a 64-token chunk, 1 / 17 / 64 patterns
(partial and several distance passes), and 16384 tokens: with 32 patterns
the block-parallel kernel's LDS layout still fits, with 64 it does not and
the one-block-per-unit kernel runs.
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import synth
from parity_util import gpu_tab, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,P,bf16", [
    (100, 1, True),
    (300, 17, False),
    (777, 64, True),
    (2048, 32, True),
    (8192, 24, True),
    (16384, 32, True),
    (16384, 64, True),
])
def test_kmeans_tables_bit_exact(n, P, bf16):
    B, Hq, H = (1, 4, 2) if n <= 4096 else (1, 4, 1)   # the oracle's k-means is O(n P) per unit
    gpu, ref, dt = make_pair(B, Hq, H, n, max_patterns=max(P, 8), bf16=bf16)
    k = synth.k_vectors(B, H, n, 128, seed=synth.seed_for("k") + n)
    v = synth.v_vectors(B, H, n, 128, seed=synth.seed_for("v") + n)
    assert ref.init_patterns(to_oracle(k, bf16), to_oracle(v, bf16), P) == 0
    print(f"k-means n={n} P={P} bf16={bf16}", flush=True)
    gpu.init_patterns(to_dev(k, dt), to_dev(v, dt), P)
    torch.cuda.synchronize()
    assert gpu.n_patterns == P
    for which in (0, 1):
        g = gpu_tab(gpu, which)[:, :P]
        r = ref.patterns(which)[:, :P]
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
            f"{'KV'[which]} table differs in {int((g != r).sum())} of {g.size} values"


def test_kmeans_empty_cluster_trace():
    """The hand-traced Lloyd run of the oracle pins (rows 5, 15, 5, 7 in every
    channel, 2 patterns): the strided start leaves cluster 1 empty on the
    first pass, it keeps its centroid, and the run ends at (15, 17/3)."""
    D = 128
    x = np.repeat(np.array([[5.0], [15.0], [5.0], [7.0]], np.float32), D, axis=1)[None, None]
    gpu, ref, dt = make_pair(1, 1, 1, 4, max_patterns=8, bf16=False)
    assert ref.init_patterns(x, x, 2) == 0
    print("k-means empty-cluster trace", flush=True)
    gpu.init_patterns(to_dev(x, dt), to_dev(x, dt), 2)
    torch.cuda.synchronize()
    want = np.stack([np.full(D, 15.0, np.float32), np.full(D, np.float32(17.0 / 3.0), np.float32)])
    for which in (0, 1):
        g = gpu_tab(gpu, which)[0, :2]
        assert np.array_equal(ref.patterns(which)[0, :2], want)
        assert np.array_equal(g.view(np.uint32), want.view(np.uint32))


def _near_tie_rows(n, kind, seed):
    """bfloat16-exact rows built to put the nearest-centroid decision on a
    knife edge: midpoints of pairs of 12 centres, shifted by a few bfloat16
    steps (kind 'mid'), or the same at norms near the input-domain bound of
    4096 with small offsets between the centres (kind 'large')."""
    rng = np.random.default_rng(seed)
    D = 128
    if kind == "mid":
        cen = rng.standard_normal((12, D))
    else:
        cen = 3000.0 + rng.standard_normal((12, D)) * 4.0
    p, q = rng.integers(0, 12, n), rng.integers(0, 12, n)
    t = 0.5 + rng.integers(-2, 3, n)[:, None] * 2.0 ** -9
    x = cen[p] + t * (cen[q] - cen[p])
    x = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    return x[None, None]


@pytest.mark.parametrize("kind,n,P", [("mid", 1024, 8), ("mid", 1024, 24), ("large", 1024, 8),
                                      ("large", 2048, 32)])
def test_kmeans_bf16_near_ties(kind, n, P):
    """Rows on or near the bisector of two centroids: the bfloat16 matrix-core
    distances must leave them to the binary64 recomputation, so the tables
    stay bit-identical to the oracle's."""
    x = _near_tie_rows(n, kind, 7 + n + P)
    gpu, ref, dt = make_pair(1, 1, 1, n, max_patterns=max(P, 8), bf16=True)
    assert ref.init_patterns(to_oracle(x, True), to_oracle(x, True), P) == 0
    print(f"k-means near ties kind={kind} n={n} P={P}", flush=True)
    gpu.init_patterns(to_dev(x, dt), to_dev(x, dt), P)
    torch.cuda.synchronize()
    for which in (0, 1):
        g = gpu_tab(gpu, which)[:, :P]
        r = ref.patterns(which)[:, :P]
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), \
            f"{'KV'[which]} table differs in {int((g != r).sum())} of {g.size} values"


@pytest.mark.parametrize("wide", [False, True])
def test_kmeans_bf16_exponent_span(wide):
    """bfloat16 prefixes take order-free binary64 member sums only when the
    values' exponent span keeps every partial sum exact; with a few values
    scaled by 2^-50 the span is too wide and the token-order sums run.  The
    tables are bit-identical to the oracle's either way."""
    n, P = 1024, 16
    x = synth.k_vectors(1, 1, n, 128, seed=synth.seed_for("k") + 99)
    if wide:
        rng = np.random.default_rng(5)
        sel = rng.random(x.shape) < 0.01
        x = np.where(sel, x * np.float32(2.0 ** -50), x).astype(np.float32)
    gpu, ref, dt = make_pair(1, 1, 1, n, max_patterns=P, bf16=True)
    assert ref.init_patterns(to_oracle(x, True), to_oracle(x, True), P) == 0
    print(f"k-means exponent span wide={wide}", flush=True)
    gpu.init_patterns(to_dev(x, dt), to_dev(x, dt), P)
    torch.cuda.synchronize()
    for which in (0, 1):
        g = gpu_tab(gpu, which)[:, :P]
        r = ref.patterns(which)[:, :P]
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
