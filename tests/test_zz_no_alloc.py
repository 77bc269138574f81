"""kvq_attn_decode_noalloc (the attention entry point for callers that cannot
allocate: its split-K workspace lives in the library's static per-GPU scratch)
against kvq_attn_decode, both called through the C ABI, on two calls in a row
with the second on a smaller cache.  Bar: within 2e-3 of each other and of the
oracle; the cache buffer's own workspace region is left untouched."""
import numpy as np
import pytest
import torch

from bit_kv_cache_encode_amd import _binding as B
from bit_kv_cache_encode_amd import synth
from parity_util import ATTN_TOL, make_pair, to_dev, to_oracle

pytestmark = pytest.mark.gpu


def _filled(B_, Hq, H, T, P, seed_off):
    gpu, ref, dt = make_pair(B_, Hq, H, T, max_patterns=P)
    k = synth.k_vectors(B_, H, T, 128, seed=synth.seed_for("k") + seed_off)
    v = synth.v_vectors(B_, H, T, 128, seed=synth.seed_for("v") + seed_off)
    assert ref.init_patterns(to_oracle(k[:, :, :256], True), to_oracle(v[:, :, :256], True), P) == 0
    gpu.init_patterns(to_dev(k[:, :, :256], dt), to_dev(v[:, :, :256], dt), P)
    assert ref.encode_append(to_oracle(k, True), to_oracle(v, True)) == 0
    gpu.encode_append(to_dev(k, dt), to_dev(v, dt))
    return gpu, ref, dt


def test_noalloc_matches_attn_decode():
    cases = [(4, 16, 4, 3000, 24, 1), (2, 8, 2, 500, 16, 2)]   # the second call is smaller
    stream = torch.cuda.current_stream().cuda_stream
    for (B_, Hq, H, T, P, off) in cases:
        print(f"noalloc case B={B_} Hq={Hq} H={H} T={T} P={P}", flush=True)
        gpu, ref, dt = _filled(B_, Hq, H, T, P, off)
        q = synth.queries(B_, Hq, 128, step=off)
        qd = to_dev(q, dt)
        want = ref.attn_decode(to_oracle(q, True))
        out_a = torch.empty((B_, Hq, 128), dtype=torch.float32, device="cuda")
        out_n = torch.full((B_, Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        assert B.kvq_attn_decode(gpu.c, qd.data_ptr(), out_a.data_ptr(), 0.0, stream) == B.KVQ_OK
        torch.cuda.synchronize()
        ws_before = gpu.region("ws").clone()
        cnt_before = gpu.region("cnt").clone()
        assert B.kvq_attn_decode_noalloc(gpu.c, qd.data_ptr(), out_n.data_ptr(), 0.0,
                                         stream) == B.KVQ_OK
        torch.cuda.synchronize()
        a, n = out_a.cpu().numpy(), out_n.cpu().numpy()
        assert np.isfinite(n).all()
        assert float(np.abs(n - a).max()) <= ATTN_TOL
        assert float(np.abs(n - want).max()) <= ATTN_TOL
        assert torch.equal(gpu.region("ws"), ws_before) and torch.equal(gpu.region("cnt"), cnt_before)
        # a second no-alloc call on the same cache (counters back at zero)
        out_n2 = torch.empty_like(out_n)
        assert B.kvq_attn_decode_noalloc(gpu.c, qd.data_ptr(), out_n2.data_ptr(), 0.0,
                                         stream) == B.KVQ_OK
        torch.cuda.synchronize()
        assert float(np.abs(out_n2.cpu().numpy() - want).max()) <= ATTN_TOL


def test_noalloc_rejects_oversized_workspace():
    """A grid whose partials exceed the scratch is rejected before any launch:
    65536 tokens of 4 units at 1024 splits each give 16 x 1024 x 130 x 4 bytes
    (8.5 MB) of partials, over the 8 MiB scratch."""
    from bit_kv_cache_encode_amd import KVCache
    B_, Hq, H, T = 2, 8, 2, 65536
    gpu = KVCache(B_, Hq, H, T, max_patterns=16, in_dtype=torch.bfloat16)
    k, v = synth.device_kv(B_, H, T, 128)
    gpu.init_patterns(k[:, :, :256].contiguous(), v[:, :, :256].contiguous(), 16)
    gpu.encode_append(k, v)
    gpu.attn_blocks = 4096
    q = synth.device_queries(B_, Hq, 128)
    out = torch.full((B_, Hq, 128), 7.0, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    print("noalloc oversized workspace", flush=True)
    assert B.kvq_attn_decode_noalloc(gpu.c, q.data_ptr(), out.data_ptr(), 0.0, stream) == B.KVQ_ESCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # the same cache at the default grid fits and matches kvq_attn_decode
    gpu.attn_blocks = 0
    want = gpu.attn_decode(q)
    assert B.kvq_attn_decode_noalloc(gpu.c, q.data_ptr(), out.data_ptr(), 0.0, stream) == B.KVQ_OK
    torch.cuda.synchronize()
    assert float((out - want).abs().max()) <= ATTN_TOL
