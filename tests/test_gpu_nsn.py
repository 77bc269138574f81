"""GPU parity of the NSN scalar mode against the oracle.

Token norm, channel centre, token norm, Hadamard rotation, then the Eq 1
quantiser at 1, 2 or 4 bits (a scalar reading of NSNQuant's double
normalisation).  Bar: codes, (s, z) words and both binary16 norms bit-exact;
the channel centres from init within 1e-6 relative (binary64 sums in a
different order; the oracle's are then uploaded so the encode compares on
identical inputs); dequant within 1e-6 relative; attention within 2e-3
absolute (the VALU kernel serves this mode).
"""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import synth
from parity_util import ATTN_TOL, DEQ_RTOL, assert_same_encode, gpu_tab, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu
D = 128


def _kv(B, H, T, off):
    k = synth.k_vectors(B, H, T, D, seed=synth.seed_for("k") + off) + np.float32(1.5)
    v = synth.v_vectors(B, H, T, D, seed=synth.seed_for("v") + off)
    return k.astype(np.float32), v


def _setup(B, Hq, H, T, bits, group, bf16, off):
    gpu, ref, dt = make_pair(B, Hq, H, T + 16, bits=bits, group=group, mode="nsn", max_patterns=0,
                             bf16=bf16)
    k, v = _kv(B, H, T, off)
    assert ref.init_patterns(to_oracle(k[:, :, :96], bf16), to_oracle(v[:, :, :96], bf16), 0) == 0
    print(f"nsn init bits={bits} group={group} bf16={bf16}", flush=True)
    gpu.init_patterns(to_dev(k[:, :, :96], dt), to_dev(v[:, :, :96], dt), 0)
    torch.cuda.synchronize()
    for w in (0, 1):
        np.testing.assert_allclose(gpu_tab(gpu, w), ref.scales(w), rtol=1e-6, atol=1e-7)
    gpu.set_patterns(torch.from_numpy(ref.scales(0).reshape(B, H, D).copy()).cuda(),
                     torch.from_numpy(ref.scales(1).reshape(B, H, D).copy()).cuda())
    return gpu, ref, dt, k, v


def _check(gpu, ref, B, Hq, T, bf16, step):
    torch.cuda.synchronize()
    assert_same_encode(ref, gpu, T)
    for w in (0, 1):
        g = gpu.dequant(w, 0, T).cpu().numpy()
        r = ref.dequant(w, 0, T)
        np.testing.assert_allclose(g, r, rtol=DEQ_RTOL, atol=1e-6)
    dt = torch.bfloat16 if bf16 else torch.float32
    q = synth.queries(B, Hq, D, step=step)
    print(f"nsn attention T={T}", flush=True)
    got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
    want = ref.attn_decode(to_oracle(q, bf16))
    err = float(np.abs(got - want).max())
    assert err <= ATTN_TOL, f"attention err {err}"


@pytest.mark.parametrize("bits,group,bf16", [(2, 32, True), (4, 64, True), (1, 8, True), (1, 32, False),
                                             (2, 128, False)])
def test_nsn_bulk_encode_attend(bits, group, bf16):
    B, H, Hq, T = 2, 2, 8, 300
    gpu, ref, dt, k, v = _setup(B, Hq, H, T, bits, group, bf16, off=bits + group)
    assert ref.encode_append(to_oracle(k, bf16), to_oracle(v, bf16)) == 0
    print(f"nsn bulk encode bits={bits}", flush=True)
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    _check(gpu, ref, B, Hq, T, bf16, step=2)


@pytest.mark.parametrize("fused_call", [False, True])
def test_nsn_token_appends(fused_call):
    """One-token appends (the single-token encode kernel) and the decode step
    (which runs the two calls in this mode)."""
    B, H, Hq, T0, steps = 2, 2, 8, 150, 6
    gpu, ref, dt, k, v = _setup(B, Hq, H, T0 + steps, 2, 32, True, off=3)
    assert ref.encode_append(to_oracle(k[:, :, :T0], True), to_oracle(v[:, :, :T0], True)) == 0
    gpu.encode_append(to_dev(k[:, :, :T0], dt), to_dev(v[:, :, :T0], dt))
    for s in range(steps):
        t = T0 + s
        kn, vn = k[:, :, t:t + 1].copy(), v[:, :, t:t + 1].copy()
        q = synth.queries(B, Hq, D, step=s)
        assert ref.encode_append(to_oracle(kn, True), to_oracle(vn, True)) == 0
        want = ref.attn_decode(to_oracle(q, True))
        print(f"nsn step {s}", flush=True)
        if fused_call:
            got = gpu.decode_step(to_dev(kn, dt), to_dev(vn, dt), to_dev(q, dt))
        else:
            gpu.encode_append(to_dev(kn, dt), to_dev(vn, dt))
            got = gpu.attn_decode(to_dev(q, dt))
        err = float(np.abs(got.cpu().numpy() - want).max())
        assert err <= ATTN_TOL, f"step {s}: attention err {err}"
    _check(gpu, ref, B, Hq, T0 + steps, True, step=5)


@pytest.mark.parametrize("bits,group,gq", [(2, 32, 4), (4, 64, 8), (2, 64, 4), (2, 32, 16)])
@pytest.mark.parametrize("blocks", [1, 256])
def test_nsn_attention_kernels_agree(bits, group, gq, blocks):
    """The matrix-core kernel (rotated query, n1 n2 token scale, q . mu_K and
    sum p n1 centre terms) and the VALU kernel match the oracle over several
    splits and q-head blocks."""
    B, H, T = 2, 2, 700
    gpu, ref, dt, k, v = _setup(B, gq * H, H, T, bits, group, True, off=gq + bits)
    assert ref.encode_append(to_oracle(k, True), to_oracle(v, True)) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    gpu.attn_blocks = blocks
    for step, qmul in ((0, 1.0), (1, 6.0)):
        q = synth.queries(B, gq * H, D, step=step) * np.float32(qmul)
        want = ref.attn_decode(to_oracle(q, True))
        errs = {}
        for kern in ("", "valu") if gq <= 8 else ("",):
            gpu.attn_kernel = kern or "auto"
            print(f"nsn kernels bits={bits} group={group} gq={gq} kern={kern or 'mfma'}", flush=True)
            got = gpu.attn_decode(to_dev(q, dt)).cpu().numpy()
            errs[kern or "mfma"] = float(np.abs(got - want).max())
        assert max(errs.values()) <= ATTN_TOL, errs
