"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a library routine, a closed form, an
invariant the pages state, brute force on tiny inputs, or a hand-derived
worked example (tests/golden/).  Citations are to the PatternKV paper
(arXiv 2510.05176v2) unless stated otherwise.
"""
import math
import os

import numpy as np
import pytest

import oracle as O
from bit_kv_cache_encode_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f16(bits):
    return np.array([bits], np.uint16).view(np.float16)[0]


# --------------------------------------------------------------- binary16
def _sample_f32(n, seed=1):
    rng = np.random.default_rng(seed)
    e = rng.uniform(-30, 17, n)
    x = (rng.uniform(1, 2, n) * 2.0 ** e * rng.choice([-1, 1], n)).astype(np.float32)
    edge = np.array([0.0, -0.0, 65504, 65519.99, 65520, 70000, -65520, 6.1e-5, 5.96e-8,
                     2.98e-8, 2.99e-8, 1e-9, -1e-9, 0.5 + 2 ** -12, 1 + 2 ** -11], np.float32)
    return np.concatenate([x, edge])


def test_f16_nearest_matches_numpy(ref):
    """RNE binary16 conversion equals numpy's float32->float16 cast."""
    x = _sample_f32(20000)
    ours = np.array([O.f16_round(v, 0) for v in x], np.uint16)
    lib = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, lib)


def test_f16_directed_rounding_bounds(ref):
    """fp16 rounded down is <= x with the next fp16 above it > x (and mirrored
    for rounding up); checked with numpy's float16 nextafter."""
    x = _sample_f32(20000, seed=2)
    x = x[np.abs(x) <= 65504]
    for v in x:
        dn = _f16(O.f16_round(v, -1))
        up = _f16(O.f16_round(v, +1))
        assert float(dn) <= float(v) < float(np.nextafter(dn, np.float16(np.inf))) or float(dn) == float(v)
        assert float(np.nextafter(up, np.float16(-np.inf))) < float(v) <= float(up) or float(up) == float(v)


def test_f16_decode_all_patterns(ref):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = h.view(np.float16).astype(np.float32)
    ours = np.array([O.f16_to_f32(int(b)) for b in h], np.float32)
    ok = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert ok.all()


# --------------------------------------------------------------- Eq 7-10
def test_norm_ppf_matches_scipy(ref):
    from scipy.stats import norm
    for p in [0.5, 0.9, 0.95, 0.975, 0.99, 0.999, 1e-6, 0.3]:
        assert abs(O.norm_ppf(p) - norm.ppf(p)) < 1e-12


@pytest.mark.parametrize("d", [64, 96, 128, 256])
@pytest.mark.parametrize("alpha", [0.01, 0.05, 0.1])
def test_rho_star_solves_eq10(ref, d, alpha):
    """rho* is the boundary of Eq 10's criterion: equality holds there, the
    criterion holds just below it and fails just above."""
    from scipy.stats import norm
    z = norm.ppf(1 - alpha)
    c = 2 * z / math.sqrt(5 * d)
    crit = lambda r: (1 - r * r) - c * math.sqrt(1 + r ** 4)
    r = O.rho_star(d, alpha)
    assert 0 < r < 1
    assert abs(crit(r)) < 1e-12
    assert crit(r - 1e-6) > 0 > crit(r + 1e-6)


def test_eq8_moments_and_ztest(ref):
    """Eq 8 under the high-resolution model: a quantization error uniform on
    [-D/2, D/2] has E[e^2] = D^2/12 and Var(e^2) = D^4/180.  At rho = rho*,
    the z statistic of Eq 9 built from those moments equals z_{1-alpha}."""
    from scipy.stats import norm
    rng = np.random.default_rng(7)
    e = rng.uniform(-0.5, 0.5, 4_000_000)
    assert abs(np.mean(e ** 2) - 1 / 12) < 2e-4
    assert abs(np.var(e ** 2) - 1 / 180) < 2e-5
    d, alpha = 128, 0.05
    r = O.rho_star(d, alpha)
    draw, dflat = 1.0, r
    ed = (draw ** 2 - dflat ** 2) / 12
    vd = (draw ** 4 + dflat ** 4) / (180 * d)
    assert abs(ed / math.sqrt(vd) - norm.ppf(1 - alpha)) < 1e-9


# --------------------------------------------------------------- Eq 1
def test_quant_group_invariants(ref):
    """|r - (q*s + z)| <= s/2 with the stored s and z; codes in range; z is the
    binary16 floor of the minimum and s the binary16 ceiling of (max-z)/(2^n-1)."""
    rng = np.random.default_rng(3)
    for bits in (2, 4):
        qmax = (1 << bits) - 1
        for _ in range(400):
            g = int(rng.choice([8, 32, 64]))
            r = (rng.standard_normal(g) * rng.uniform(0.01, 20) + rng.uniform(-5, 5)).astype(np.float32)
            codes, s, z, _ = O.quant_group(r, bits)
            sf, zf = float(_f16(s)), float(_f16(z))
            assert codes.max() <= qmax
            assert zf <= r.min() < float(np.nextafter(_f16(z), np.float16(np.inf)))
            s32 = np.float32(np.float32(r.max() - np.float32(zf)) / np.float32(qmax))
            assert sf >= s32 and float(np.nextafter(_f16(s), np.float16(-np.inf))) < s32
            rec = codes.astype(np.float64) * sf + zf   # exact in binary64
            err = np.abs(r.astype(np.float64) - rec)
            assert err.max() <= sf / 2 * (1 + 1e-6) + 1e-7
            # PatternKV App. C, Eq 21: per-group L2 error <= sqrt(g)/2 * width/(2^b-1)
            width = float(r.max()) - zf
            assert np.sqrt((err ** 2).sum()) <= math.sqrt(g) / 2 * width / qmax * (1 + 2 ** -10) + 1e-6


def test_quant_group_special_cases(ref):
    codes, s, z, _ = O.quant_group(np.full(32, 1.0, np.float32), 2)
    assert s == 0 and z == 0x3C00 and not codes.any()
    codes, s, z, _ = O.quant_group(np.zeros(32, np.float32), 2)
    assert s == 0 and z == 0 and not codes.any()
    codes, s, z, _ = O.quant_group(-np.zeros(32, np.float32), 2)
    assert z == 0   # a negative zero is stored as +0


# --------------------------------------------------------------- Eq 6
def test_nearest_pattern_brute_force(ref):
    """Nearest pattern under d_mm equals a numpy broadcast over all patterns
    (first minimum = lowest index), on tiny inputs."""
    rng = np.random.default_rng(4)
    for _ in range(300):
        n, d = int(rng.integers(1, 9)), int(rng.integers(2, 17))
        x = rng.integers(-4, 5, d).astype(np.float32)
        p = rng.integers(-4, 5, (n, d)).astype(np.float32)
        diff = x[None, :] - p
        e = diff.max(1) - diff.min(1)
        k, ek = O.nearest(x, p)
        assert k == int(np.argmin(e)) and ek == e.min()
    k, _ = O.nearest(np.ones(4, np.float32), np.zeros((0, 4), np.float32))
    assert k == O.NONE


def test_nearest_pattern_identities(ref):
    """d_mm(x, x) = 0 selects x's own pattern; d_mm is unchanged by adding a
    constant to every channel (exact for small integers)."""
    rng = np.random.default_rng(5)
    p = rng.standard_normal((16, 128)).astype(np.float32)
    for j in range(16):
        assert O.nearest(p[j], p)[0] == j
    x = rng.integers(-50, 50, 128).astype(np.float32)
    pi = rng.integers(-50, 50, (16, 128)).astype(np.float32)
    assert O.nearest(x, pi)[0] == O.nearest(x + 17, pi)[0]


# --------------------------------------------------------------- Hadamard
@pytest.mark.parametrize("n", [2, 8, 64, 128])
def test_fwht_is_sylvester_hadamard(ref, n):
    from scipy.linalg import hadamard
    H = np.stack([O.fwht_f32(np.eye(n, dtype=np.float32)[i]) for i in range(n)])
    assert np.array_equal(H, hadamard(n).astype(np.float32))
    assert np.array_equal(H @ H.T, n * np.eye(n))
    x = np.random.default_rng(6).integers(-8, 9, n).astype(np.float32)
    assert np.array_equal(O.fwht_f32(O.fwht_f32(x)), n * x)


# --------------------------------------------------------------- Eq 4
def test_kmeans_matches_sklearn_lloyd(ref):
    """Same local minimum as scikit-learn's Lloyd iteration from the same
    strided initial centroids (no empty cluster occurs on this data)."""
    from sklearn.cluster import KMeans
    x = synth.k_vectors(1, 1, 512, 128)[0, 0]
    k = 16
    init = x[[j * 512 // k for j in range(k)]].astype(np.float64)
    km = KMeans(n_clusters=k, init=init, n_init=1, algorithm="lloyd", tol=0.0,
                max_iter=50).fit(x.astype(np.float64))
    cent, a, it = O.kmeans(x, k)
    assert np.bincount(a, minlength=k).min() > 0
    assert np.array_equal(a, km.labels_)
    np.testing.assert_allclose(cent, km.cluster_centers_, rtol=1e-6, atol=1e-6)
    # stationarity: each centroid is its members' mean; assignment is nearest
    for j in range(k):
        np.testing.assert_allclose(cent[j], x[a == j].astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)
    d2 = ((x[:, None, :].astype(np.float64) - cent[None].astype(np.float64)) ** 2).sum(-1)
    assert np.array_equal(np.argmin(d2, 1), a)


def test_kmeans_sse_non_increasing_with_budget(ref):
    """Eq 2/4: the within-pattern variance E[Var(Z|M)] shrinks as the pattern
    budget grows (ablation direction of Table 4) and never exceeds Var(Z)."""
    x = synth.k_vectors(1, 1, 512, 128)[0, 0].astype(np.float64)
    total = ((x - x.mean(0)) ** 2).sum()
    prev = total
    for k in (1, 2, 4, 8, 16):
        cent, a, _ = O.kmeans(x.astype(np.float32), k)
        sse = ((x - cent[a].astype(np.float64)) ** 2).sum()
        assert sse <= prev * (1 + 1e-9)
        prev = sse
    assert abs(((x - O.kmeans(x.astype(np.float32), 1)[0][0]) ** 2).sum() - total) < 1e-6 * total


# --------------------------------------------------------------- goldens
def _read_gold(name):
    kv = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            kv[key] = vals
    return kv


def test_golden_pattern_2bit(ref):
    g = _read_gold("pattern_2bit_d8.txt")
    c = O.RefCache(1, 1, 1, 8, 32, bits=2, group=4, mode=O.PATTERN, max_patterns=2, v_alpha=0.05)
    pats = np.array([[float(v) for v in g["pattern0"]], [float(v) for v in g["pattern1"]]], np.float32)
    assert c.set_patterns(pats[None, None], pats[None, None]) == 0
    x = np.array([[float(v) for v in g["x0"]], [float(v) for v in g["x1"]]], np.float32)[None, None]
    assert c.encode_append(x, x) == 0
    kb = c.codes(0)[0, :4]
    assert list(kb) == [int(v, 16) for v in g["k_bytes"]]
    assert list(c.idx(0)[0, :2]) == [int(v) for v in g["k_idx"]]
    assert list(c.idx(1)[0, :2]) == [int(v) for v in g["v_idx"]]
    assert list(c.sz(0)[0, :2].ravel()) == [int(v, 16) for v in g["k_sz"]]
    assert list(c.sz(1)[0, :2].ravel()) == [int(v, 16) for v in g["v_sz"]]
    assert list(c.codes(1)[0, :4]) == [int(v, 16) for v in g["v_bytes"]]
    assert list(c.ties(0)[0, 1]) == [int(v) for v in g["k_ties_t1"]]
    deq = c.dequant(0, 0, 2)[0, 0]
    assert list(deq[0]) == [float(v) for v in g["k_dequant_t0"]]
    assert list(deq[1]) == [float(v) for v in g["k_dequant_t1"]]
    assert abs(O.rho_star(8, 0.05) - 0.658) < 1e-3


def test_golden_kvarn_2bit(ref):
    g = _read_gold("kvarn_2bit_d4.txt")
    c = O.RefCache(1, 1, 1, 4, 32, bits=2, group=4, mode=O.KVARN, max_patterns=0)
    ones = np.ones((1, 1, 4), np.float32)
    c.set_patterns(ones, ones)
    x = np.array([float(v) for v in g["x0"]], np.float32)[None, None, None]
    c.encode_append(x, x)
    assert c.t16(0)[0, 0] == int(g["t16"][0], 16)
    assert list(c.sz(0)[0, 0].ravel()) == [int(v, 16) for v in g["k_sz"]]
    assert c.codes(0)[0, 0] == int(g["k_bytes"][0], 16)
    assert list(c.dequant(0, 0, 1)[0, 0, 0]) == [float(v) for v in g["k_dequant_t0"]]


def test_golden_raw_4bit(ref):
    g = _read_gold("raw_4bit_d8.txt")
    c = O.RefCache(1, 1, 1, 8, 32, bits=4, group=8, mode=O.PATTERN, max_patterns=0)
    x = np.array([float(v) for v in g["x0"]], np.float32)[None, None, None]
    c.encode_append(x, x)
    assert list(c.sz(0)[0, 0].ravel()) == [int(v, 16) for v in g["k_sz"]]
    assert list(c.codes(0)[0, :4]) == [int(v, 16) for v in g["k_bytes"]]
    assert c.idx(0)[0, 0] == int(g["k_idx"][0])


# --------------------------------------------------------------- V threshold
def test_v_threshold_boundary(ref):
    """Section 3.3: V uses its pattern iff R_flat <= rho* R_raw (K always does)."""
    D = 128
    rho = float(O.rho_star_f32(D, 0.05))
    base = np.zeros(D, np.float32)
    base[0], base[1] = 0.0, 100.0                    # R_raw = 100
    for flat, keep in ((rho * 100 * 0.999, True), (rho * 100 * 1.001, False)):
        pat = base.copy()
        pat[1] = np.float32(100.0 - flat)            # x - M spans [0, flat]
        c = O.RefCache(1, 1, 1, D, 32, max_patterns=1, v_alpha=0.05)
        c.set_patterns(pat[None, None, None], pat[None, None, None])
        x = base[None, None, None]
        c.encode_append(x, x)
        assert c.idx(0)[0, 0] == 0                   # K: no threshold
        assert (c.idx(1)[0, 0] == 0) == keep
    c = O.RefCache(1, 1, 1, D, 32, max_patterns=1, v_alpha=0.0)
    c.set_patterns(pat[None, None, None], pat[None, None, None])
    c.encode_append(x, x)
    assert c.idx(1)[0, 0] == 0                       # threshold off


# --------------------------------------------------------------- Eq 5
def test_chebyshev_window(ref):
    """After G_pattern decode appends, a new pattern M_d = (min_i x + max_i x)/2
    is added; it minimises max_i ||x_i - M||_inf (App. C, Chebyshev centre)."""
    D, W = 128, 128
    k = synth.k_vectors(1, 2, 3 * W + 5, D)
    v = synth.v_vectors(1, 2, 3 * W + 5, D)
    c = O.RefCache(1, 2, 2, D, 4 * W, max_patterns=3, pattern_window=W)
    c.init_patterns(k[:, :, :64], v[:, :, :64], 1)
    assert c.n_patterns == 1
    for t in range(3 * W + 5):
        c.encode_append(k[:, :, t:t + 1], v[:, :, t:t + 1], update=1)
        assert c.n_patterns == min(1 + (t + 1) // W, 3)
    assert c.dropped == 1 and c.win_count == 5
    for which, X in ((0, k), (1, v)):
        for u in range(2):
            win = X[0, u, :W]
            M = c.patterns(which)[u, 1]
            expect = ((win.min(0) + win.max(0)) * np.float32(0.5)).astype(np.float32)
            assert np.array_equal(M, expect)
            rad = np.abs(win - M).max()
            half = 0.5 * (win.max(0) - win.min(0)).max()
            assert abs(rad - half) <= 1e-5 * max(1.0, half)
            rng = np.random.default_rng(u)
            for _ in range(20):
                other = M + rng.standard_normal(D).astype(np.float32) * 0.05
                assert np.abs(win - other).max() >= rad - 1e-5


# --------------------------------------------------------------- attention
def test_attention_exact_matches_sdpa(ref):
    """fp64 attention with GQA equals torch's scaled_dot_product_attention."""
    import torch
    B, Hq, H, T, D = 2, 8, 2, 77, 128
    rng = np.random.default_rng(8)
    k = rng.standard_normal((B, H, T, D)).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    ours = O.attn_exact(k, v, q, Hq)
    kt = torch.from_numpy(k).double().repeat_interleave(Hq // H, dim=1)
    vt = torch.from_numpy(v).double().repeat_interleave(Hq // H, dim=1)
    qt = torch.from_numpy(q).double()[:, :, None, :]
    lib = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, :, 0].float().numpy()
    np.testing.assert_allclose(ours, lib, rtol=0, atol=1e-6)


def test_zero_residual_cache_is_exact(ref):
    """Vectors equal to a pattern have residual 0, so s = z = 0, codes 0 and the
    reconstruction (Eq 1 inverse + pattern restore) is exact; attention over
    the cache then equals attention over the raw vectors."""
    B, Hq, H, T, D, P = 1, 4, 2, 96, 128, 8
    rng = np.random.default_rng(9)
    pk = rng.standard_normal((B, H, P, D)).astype(np.float32)
    pv = rng.standard_normal((B, H, P, D)).astype(np.float32)
    sel = rng.integers(0, P, (B, H, T))
    k = np.take_along_axis(pk, sel[..., None].repeat(D, -1), 2)
    v = np.take_along_axis(pv, sel[..., None].repeat(D, -1), 2)
    c = O.RefCache(B, Hq, H, D, T, max_patterns=P)
    c.set_patterns(pk, pv)
    c.encode_append(k, v)
    assert np.array_equal(c.dequant(0, 0, T), k) and np.array_equal(c.dequant(1, 0, T), v)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    np.testing.assert_allclose(c.attn_decode(q), O.attn_exact(k, v, q, Hq), rtol=0, atol=1e-6)


def test_attention_special_cases(ref):
    B, H, D = 1, 1, 128
    k = synth.k_vectors(B, H, 40, D)
    v = synth.v_vectors(B, H, 40, D)
    c = O.RefCache(B, 2, H, D, 64, max_patterns=4)
    c.init_patterns(k, v, 4)
    c.encode_append(k[:, :, :1], v[:, :, :1])
    q = synth.queries(B, 2, D)
    out = c.attn_decode(q)
    v0 = c.dequant(1, 0, 1)[0, 0, 0]
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)
    c.encode_append(k[:, :, 1:], v[:, :, 1:])
    out = c.attn_decode(np.zeros_like(q))
    vm = c.dequant(1, 0, 40)[0, 0].astype(np.float64).mean(0)
    np.testing.assert_allclose(out[0, 0], vm, rtol=0, atol=1e-6)


# --------------------------------------------------------------- KVarN
def test_kvarn_normalisation_and_error(ref):
    """KVarN reading: after the rotation and channel scaling, the token scale t
    makes RMS(u) = 1 up to t's binary16 rounding; the rotation is orthonormal,
    so ||x - x^||_2 = ||t c (u - u^)||_2 (Parseval)."""
    B, H, T, D = 1, 1, 64, 128
    k = synth.k_vectors(B, H, T, D)
    c = O.RefCache(B, 1, H, D, T, mode=O.KVARN, max_patterns=0)
    c.init_patterns(k, k, 0)
    cs = c.scales(0)[0].astype(np.float64)
    np.testing.assert_allclose(np.sqrt((cs ** 2).mean()), 1.0, rtol=1e-6)  # E over channels
    c.encode_append(k, k)
    from scipy.linalg import hadamard
    Hn = hadamard(D) / math.sqrt(D)
    xh = c.dequant(0, 0, T)[0, 0].astype(np.float64)
    t16 = c.t16(0)[0, :T].view(np.float16).astype(np.float64)
    for t in range(T):
        x = k[0, 0, t].astype(np.float64)
        y = Hn @ x / cs
        u = y / t16[t]
        rms_exact = math.sqrt((y ** 2).mean())
        assert abs(math.sqrt((u ** 2).mean()) - rms_exact / t16[t]) < 1e-6
        assert abs(rms_exact / t16[t] - 1) <= 2 ** -11 * 1.01
        uh = (Hn @ xh[t]) / cs / t16[t]
        lhs = np.linalg.norm(x - xh[t])
        rhs = np.linalg.norm(t16[t] * cs * (u - uh))
        assert abs(lhs - rhs) <= 1e-4 * max(1.0, lhs)


def test_config_validation(ref):
    with pytest.raises(ValueError):
        O.RefCache(1, 3, 2, 128, 64)          # Hq not a multiple of Hkv
    with pytest.raises(ValueError):
        O.RefCache(1, 1, 1, 128, 64, bits=3)
    with pytest.raises(ValueError):
        O.RefCache(1, 1, 1, 96, 64, mode=O.KVARN)
    with pytest.raises(ValueError):
        O.RefCache(1, 1, 1, 128, 64, max_patterns=256)
    c = O.RefCache(1, 1, 1, 128, 4)
    x = np.zeros((1, 1, 5, 128), np.float32)
    assert c.encode_append(x, x) == -2 and c.n_tokens == 0


# --------------------------------------------------------------- KVarN channel scale (R12)
def _sylvester_rows(sigma_rows):
    """x = H y / sqrt(D) with scipy's Sylvester Hadamard matrix, i.e. the
    orthonormal inverse of y = H x / sqrt(D) (H is symmetric, H H = D I)."""
    from scipy.linalg import hadamard
    D = sigma_rows.shape[-1]
    return (sigma_rows @ hadamard(D).T.astype(np.float64)) / math.sqrt(D)


def test_kvarn_channel_scale_closed_form(ref):
    """KVarN abstract, dual-axis variance normalisation (reading R12): the
    channel scale is the RMS over prefix tokens of the rotated row divided by
    its own RMS.  Rows built in the rotated space as y_t = a_t (prof_t * eps_t),
    with eps_t in {+1,-1}^D, a random positive token magnitude a_t and the
    profile prof_t = sigma for the first half of the tokens and tau for the
    second, have y_tj / rms(y_t) = prof_tj eps_tj / rms(prof_t), so
    c_j = sqrt((sigma_j^2 / ms(sigma) + tau_j^2 / ms(tau)) / 2) exactly
    (ms = mean square over channels).  The profiles are random permutations of
    distinct values, so a transform in another order (bit-reversed or
    sequency order), a missed or mis-signed butterfly stage, swapped channels,
    a mean |y| in place of the RMS, or a global instead of a per-token
    normalisation all move c away from this value."""
    D, T = 128, 96
    rng = np.random.default_rng(1203)
    B = 2
    k = np.zeros((B, 1, T, D), np.float32)
    v = np.zeros((B, 1, T, D), np.float32)
    want = np.zeros((2, B, D))
    for kind, arr in enumerate((k, v)):
        for b in range(B):
            sigma = rng.permutation(np.linspace(0.2, 5.0, D))
            tau = rng.permutation(np.geomspace(0.05, 8.0, D))
            prof = np.where(np.arange(T)[:, None] < T // 2, sigma[None], tau[None])
            eps = rng.choice([-1.0, 1.0], (T, D))
            a = rng.uniform(0.1, 20.0, (T, 1))
            arr[b, 0] = _sylvester_rows(a * prof * eps).astype(np.float32)
            want[kind, b] = np.sqrt((sigma ** 2 / (sigma ** 2).mean()
                                     + tau ** 2 / (tau ** 2).mean()) / 2)
    c = O.RefCache(B, 1, 1, D, T, mode=O.KVARN, max_patterns=0)
    c.init_patterns(k, v, 0)
    for kind in range(2):
        got = c.scales(kind)[:B].astype(np.float64)
        np.testing.assert_allclose(got, want[kind], rtol=2e-6, atol=0)
    # the same construction with one profile (tau = sigma): c = sigma / rms(sigma)
    sigma = rng.permutation(np.linspace(0.5, 3.0, D))
    eps = rng.choice([-1.0, 1.0], (T, D))
    x = _sylvester_rows(sigma * eps).astype(np.float32)[None, None]
    c1 = O.RefCache(1, 1, 1, D, T, mode=O.KVARN, max_patterns=0)
    c1.init_patterns(x, x, 0)
    np.testing.assert_allclose(c1.scales(0)[0], sigma / math.sqrt((sigma ** 2).mean()),
                               rtol=2e-6, atol=0)
    # an all-zero prefix has no token to normalise: every scale is 1
    z = np.zeros((1, 1, 8, D), np.float32)
    c2 = O.RefCache(1, 1, 1, D, 8, mode=O.KVARN, max_patterns=0)
    c2.init_patterns(z, z, 0)
    assert np.array_equal(c2.scales(0)[0], np.ones(D, np.float32))


# --------------------------------------------------------------- k-means empty cluster (R13)
def test_kmeans_empty_cluster_keeps_centroid(ref):
    """Eq 4 Lloyd iteration with reading R13's empty-cluster rule, traced by
    hand on one-dimensional rows x = (5, 15, 5, 7), k = 2.  Strided start:
    centroids x[0] = 5 and x[2] = 5.  Pass 1: every row is equidistant, ties
    go to index 0, so cluster 1 is empty; c0 = 32/4 = 8 and c1 keeps 5.
    Pass 2: 5 -> 1, 15 -> 0, 5 -> 1, 7 -> 0 (1 < 4); c0 = 11, c1 = 5.
    Pass 3: 7 -> 1 (16 > 4); c0 = 15, c1 = 17/3.  Pass 4 repeats pass 3's
    assignment and stops.  Resetting an empty centroid to 0 would stop at
    (8, 0) after pass 2; moving it to the farthest row would give (17/3, 15)."""
    x = np.array([[5.0], [15.0], [5.0], [7.0]], np.float32)
    cent, a, it = O.kmeans(x, 2)
    assert np.array_equal(cent[:, 0], np.array([15.0, np.float32(17.0 / 3.0)], np.float32))
    assert list(a) == [1, 0, 1, 1]
    assert it == 4
    # the same trace in every channel of a 128-wide row, so the cache's
    # pattern init (which the GPU k-means is compared with) sees it too
    D = 128
    rows = np.repeat(x, D, axis=1)[None, None]
    c = O.RefCache(1, 1, 1, D, 4, max_patterns=2)
    c.init_patterns(rows, rows, 2)
    pk = c.patterns(0)[0, :2]
    assert np.array_equal(pk[0], np.full(D, 15.0, np.float32))
    assert np.array_equal(pk[1], np.full(D, np.float32(17.0 / 3.0), np.float32))
