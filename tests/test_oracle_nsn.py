"""Pins of the oracle's NSN scalar mode (mode NSN).

Reading (NSNQuant, abstract): a token-wise normalisation, a channel-wise
centring and a second token-wise normalisation, with a Hadamard transform;
its vector-quantisation codebook is out of scope, so the normalised rotated
vector goes through the Eq 1 quantiser (1, 2 or 4 bits).  The pins:
* the channel centre mu is the mean over the prefix of x / rms(x) (numpy,
  binary64);
* every token reconstructs within the Eq 1 bound carried through the
  transform: ||x - x^||_2 <= n1 n2 ||y - y^||_2 with |y - y^| <= s/2 per
  element (the Hadamard rotation is orthonormal), plus rounding;
* the zero vector reconstructs to zero exactly, with n1 = n2 = 0;
* scaling a token by a power of two scales n1 by it and leaves codes,
  scales and n2 unchanged;
* centring pays: with a large common component the error is far smaller
  than with mu = 0 (same codes budget).
"""
import numpy as np
import pytest

import oracle as O
from bit_kv_cache_encode_amd import synth

D = 128


def _cache(B=1, H=2, T=256, bits=2, group=32):
    return O.RefCache(B, 2 * H, H, D, T, bits=bits, group=group, mode=O.NSN, max_patterns=0)


def _f16(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def test_centre_is_mean_of_normalised_prefix(ref):
    B, H, n = 2, 2, 77
    k = synth.k_vectors(B, H, n, D, seed=synth.seed_for("k") + 40)
    v = synth.v_vectors(B, H, n, D, seed=synth.seed_for("v") + 40)
    c = _cache(B, H)
    assert c.init_patterns(k, v, 0) == 0
    for w, X in ((0, k), (1, v)):
        X = X.reshape(B * H, n, D).astype(np.float64)
        r = np.sqrt((X ** 2).mean(-1, keepdims=True))
        want = (X / r).mean(1).astype(np.float32)
        assert np.array_equal(c.scales(w), want)


@pytest.mark.parametrize("bits,group", [(1, 32), (2, 32), (4, 64), (2, 128)])
def test_reconstruction_within_quantiser_bound(ref, bits, group):
    B, H, T = 1, 2, 200
    k = synth.k_vectors(B, H, T, D, seed=synth.seed_for("k") + bits) + np.float32(2.0)
    v = synth.v_vectors(B, H, T, D, seed=synth.seed_for("v") + bits)
    c = _cache(B, H, 256, bits, group)
    assert c.init_patterns(k[:, :, :64], v[:, :, :64], 0) == 0
    assert c.encode_append(k, v) == 0
    for w, X in ((0, k), (1, v)):
        X = X.reshape(B * H, T, D).astype(np.float64)
        xh = c.dequant(w, 0, T).reshape(B * H, T, D).astype(np.float64)
        n1, n2 = _f16(c.t16(w)[:, :T]), _f16(c.t2(w)[:, :T])
        s = _f16(c.sz(w)[:, :T, :, 0])                          # [U][T][NG]
        ybound = np.sqrt((group * (s / 2) ** 2).sum(-1))         # ||y - y^||_2 bound
        err = np.sqrt(((X - xh) ** 2).sum(-1))
        scale = np.abs(X).max() + 1
        assert np.all(err <= n1 * n2 * ybound * (1 + 1e-3) + 1e-4 * scale * np.sqrt(D)), (w, bits)
        # codes within range
        codes = O.unpack_codes(c.codes(w), T, D, bits)
        assert codes.max() <= (1 << bits) - 1


def test_zero_token(ref):
    c = _cache(1, 1, 64)
    rng = np.random.default_rng(3)
    pre = (rng.standard_normal((1, 1, 32, D)) + 4.0).astype(np.float32)
    assert c.init_patterns(pre, pre, 0) == 0
    x = np.zeros((1, 1, 2, D), np.float32)
    x[0, 0, 1] = rng.standard_normal(D).astype(np.float32)
    assert c.encode_append(x, x) == 0
    xh = c.dequant(0, 0, 2)[0, 0]
    assert np.array_equal(xh[0], np.zeros(D, np.float32))
    assert c.t16(0)[0, 0] == 0 and c.t2(0)[0, 0] == 0
    assert np.all(c.sz(0)[0, 0] == 0)


def test_power_of_two_scaling(ref):
    c1, c2 = _cache(1, 1, 64), _cache(1, 1, 64)
    x = synth.k_vectors(1, 1, 40, D, seed=synth.seed_for("k") + 41)
    for c in (c1, c2):
        c.set_patterns(np.zeros((1, 1, D), np.float32), np.zeros((1, 1, D), np.float32))
    assert c1.encode_append(x, x) == 0
    assert c2.encode_append(x * np.float32(8), x * np.float32(8)) == 0
    for w in (0, 1):
        assert np.array_equal(c1.codes(w), c2.codes(w))
        assert np.array_equal(c1.sz(w), c2.sz(w))
        assert np.array_equal(c1.t2(w), c2.t2(w))
        assert np.array_equal(_f16(c1.t16(w)) * 8, _f16(c2.t16(w)))


def test_centring_reduces_error_on_a_common_component(ref):
    rng = np.random.default_rng(5)
    common = rng.standard_normal(D).astype(np.float32) * np.float32(5)
    x = (common + 0.3 * rng.standard_normal((1, 1, 300, D))).astype(np.float32)
    errs = []
    for centre in (True, False):
        c = _cache(1, 1, 320, bits=2)
        if centre:
            assert c.init_patterns(x[:, :, :64], x[:, :, :64], 0) == 0
        assert c.encode_append(x, x) == 0
        errs.append(float(np.abs(c.dequant(0, 0, 300) - x).mean()))
    assert errs[0] < 0.25 * errs[1], errs


def test_nsn_config_rules(ref):
    with pytest.raises(ValueError):
        O.RefCache(1, 2, 1, D, 64, bits=1, mode=O.PATTERN, max_patterns=4)
    with pytest.raises(ValueError):
        O.RefCache(1, 2, 1, 96, 64, mode=O.NSN, max_patterns=0)    # Hadamard needs 2^k
    O.RefCache(1, 2, 1, D, 64, bits=1, group=8, mode=O.NSN, max_patterns=0)
