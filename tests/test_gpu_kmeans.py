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
