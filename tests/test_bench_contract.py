"""Host-side contract of bench.py (no GPU): the refusal of more than one GPU,
and the algorithmic byte counts behind `value` and `roofline`, re-derived
from the cache layout the C ABI reports (kvq_layout_of, host only) rather
than from the bench's own record-size arithmetic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_kv_cache_encode_amd import _binding as B  # noqa: E402

D = 128
MODES = {"pattern": B.MODE_PATTERN, "kvarn": B.MODE_KVARN, "nsn": B.MODE_NSN}


def _layout(c):
    mode = MODES[c["mode"]]
    cfg = B.kvq_config(batch=c["B"], n_q_heads=c["Hq"], n_kv_heads=c["H"], head_dim=D,
                       max_tokens=c["T"], bits=c["bits"], group=c["group"], mode=mode,
                       max_patterns=c["P"] if mode == B.MODE_PATTERN else 0, pattern_window=0,
                       v_alpha=0.05 if mode == B.MODE_PATTERN else 0.0, in_dtype=B.BF16,
                       max_splits=0, k_per_channel=1 if c.get("kch") else 0)
    return B.kvq_layout_of(cfg)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("name", sorted(bench.ATTN_CONFIGS))
def test_attention_bytes_follow_the_layout(name):
    """Per call: every cached token's K and V bytes (codes, scale / zero words,
    and the pattern index or token scales), the K and V pattern tables, the
    bfloat16 query and the binary32 output, with the per-token sizes taken
    from the library's region sizes."""
    c = bench.ATTN_CONFIGS[name]
    L = _layout(c)
    U, tc, T = c["B"] * c["H"], L.token_cap, c["T"]
    per_tok = lambda nbytes: nbytes // (U * tc)
    codes, sz = per_tok(L.codes_bytes), per_tok(L.sz_bytes)
    side = per_tok(L.idx_bytes) + per_tok(L.t16_bytes) + per_tok(L.t2_bytes)
    assert codes == D * c["bits"] // 8
    assert codes + sz + side == L.record_bytes
    tables = 2 * U * c["P"] * D * 4
    q_out = c["B"] * c["Hq"] * D * (2 + 4)
    if c.get("kch"):
        # K per channel: codes and index per token, one (s, z) word per channel
        # and complete 128-token block, binary16 residuals of the open block
        blocks = L.bsz_bytes // (U * D * 4)
        assert blocks * U * D * 4 == L.bsz_bytes and L.tail_bytes == U * 128 * D * 2
        closed = T // 128 * 128
        k = T * (codes + per_tok(L.idx_bytes)) + closed // 128 * D * 4 + (T - closed) * D * 2
        expect = U * (k + T * L.record_bytes) + tables + q_out
    else:
        expect = 2 * U * T * L.record_bytes + tables + q_out
    assert bench.attn_config_bytes(c) == expect


def test_step_bytes_of_the_headline_workload():
    """The bench line's bytes per launch at 32768 cached tokens: attention over
    the cache plus the new token (its K and V in, its records out), 2-bit
    PatternKV records of 49 bytes, 32-pattern tables; the figure the committed
    traffic summary is compared against."""
    c = dict(B=8, Hq=32, H=8, T=32768 + 1, bits=2, group=32, P=32, mode="pattern")
    L = _layout(c)
    U = 64
    attn = 2 * U * c["T"] * L.record_bytes + 2 * U * 32 * D * 4 + 8 * 32 * D * 6
    enc = 2 * U * D * 2 + 2 * U * L.record_bytes
    assert L.record_bytes == 49
    assert attn + enc == 207859968
