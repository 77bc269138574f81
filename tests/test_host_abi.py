"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the ctypes structs match the C layout, the cache layout is
consistent, and every argument error is reported before any launch."""
import ctypes as C
import os
import re
import subprocess

import pytest

from bit_kv_cache_encode_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _cfg(**kw):
    d = dict(batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, max_tokens=4096, bits=2,
             group=32, mode=B.MODE_PATTERN, max_patterns=32, pattern_window=128, v_alpha=0.05,
             in_dtype=B.BF16, max_splits=0)
    d.update(kw)
    return B.kvq_config(**d)


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(kvq_\w+)\s*\(", text, re.M))
    assert declared == set(B.EXPORTS)
    lib = B.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(f'''#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(kvq_config),
         sizeof(kvq_layout), sizeof(kvq_cache), offsetof(kvq_cache, base),
         offsetof(kvq_cache, rho), offsetof(kvq_layout, total), offsetof(kvq_config, max_splits),
         offsetof(kvq_config, shared_patterns), offsetof(kvq_config, k_per_channel),
         offsetof(kvq_layout, k_bsz), offsetof(kvq_layout, tail_bytes),
         offsetof(kvq_layout, status));
  return 0;
}}''')
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c11", "-o", str(exe), str(src)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    want = [C.sizeof(B.kvq_config), C.sizeof(B.kvq_layout), C.sizeof(B.kvq_cache),
            B.kvq_cache.base.offset, B.kvq_cache.rho.offset, B.kvq_layout.total.offset,
            B.kvq_config.max_splits.offset, B.kvq_config.shared_patterns.offset,
            B.kvq_config.k_per_channel.offset, B.kvq_layout.k_bsz.offset,
            B.kvq_layout.tail_bytes.offset, B.kvq_layout.status.offset]
    assert got == want


def test_layout_regions():
    L = B.kvq_layout_of(_cfg())
    U, T = 64, 4096
    assert L.token_cap == 4096 and L.n_groups == 4
    assert L.codes_bytes == U * T * 32 and L.sz_bytes == U * T * 16 and L.idx_bytes == U * T
    assert L.record_bytes == 49        # 32 B codes + 4 x (s, z) fp16 + 1 B index
    assert L.t16_bytes == 0 and L.win_bytes == U * 2 * 128 * 4
    offs = sorted((getattr(L, n), getattr(L, n.replace("k_", "").replace("v_", "") + "_bytes")
                   if n not in ("ws",) else L.ws_bytes)
                  for n in ("k_codes", "v_codes"))
    for name in ("k_codes", "v_codes", "k_sz", "v_sz", "k_idx", "v_idx", "k_tab", "v_tab",
                 "k_win", "v_win", "ws"):
        assert getattr(L, name) % 256 == 0
    assert L.ws + L.ws_bytes <= L.total
    Lk = B.kvq_layout_of(_cfg(mode=B.MODE_KVARN, max_patterns=0))
    assert Lk.record_bytes == 50 and Lk.idx_bytes == 0 and Lk.t16_bytes == U * T * 2
    L4 = B.kvq_layout_of(_cfg(bits=4, group=64))
    assert L4.record_bytes == 73
    # batch-shared tables: one table and one window per kv-head
    Ls = B.kvq_layout_of(_cfg(shared_patterns=1))
    assert Ls.tab_bytes == 8 * 32 * 128 * 4 and Ls.win_bytes == 8 * 2 * 128 * 4
    assert L.tab_bytes == U * 32 * 128 * 4 and Ls.codes_bytes == L.codes_bytes
    assert offs  # regions exist
    # K per channel: block scales and the open block's residuals, placed after
    # every other region so that the others keep their offsets
    assert L.bsz_bytes == 0 and L.tail_bytes == 0
    Lc = B.kvq_layout_of(_cfg(k_per_channel=1, max_tokens=4000))
    assert Lc.token_cap == 4032 and Lc.bsz_bytes == U * 32 * 128 * 4
    assert Lc.tail_bytes == U * 128 * 128 * 2
    assert Lc.k_bsz % 256 == 0 and Lc.k_tail % 256 == 0 and Lc.k_bsz >= Lc.cnt + Lc.cnt_bytes
    assert Lc.k_tail + Lc.tail_bytes <= Lc.total
    # NSN: the second norm after every other region; 1-bit codes allowed there
    Ln = B.kvq_layout_of(_cfg(mode=B.MODE_NSN, max_patterns=0))
    assert Ln.t2_bytes == U * T * 2 and Ln.t16_bytes == U * T * 2 and L.t2_bytes == 0
    assert Ln.record_bytes == 32 + 16 + 4 and Ln.tab_bytes == U * 128 * 4
    assert Ln.v_t2 + Ln.t2_bytes <= Ln.total
    L1 = B.kvq_layout_of(_cfg(mode=B.MODE_NSN, max_patterns=0, bits=1, group=8))
    assert L1.codes_bytes == U * T * 16 and L1.n_groups == 16
    L0 = B.kvq_layout_of(_cfg(max_tokens=4000))
    assert all(getattr(Lc, n) == getattr(L0, n) for n in ("k_codes", "v_codes", "k_sz", "ws", "cnt"))
    # the domain-flag word comes last in every mode
    for Lx in (L, Lk, L4, Ls, Lc, Ln, L1):
        assert Lx.status % 256 == 0 and Lx.status + 4 <= Lx.total
        assert Lx.status >= max(Lx.v_t2 + Lx.t2_bytes, Lx.k_tail + Lx.tail_bytes, Lx.cnt + Lx.cnt_bytes)


@pytest.mark.parametrize("bad", [
    dict(head_dim=64), dict(bits=3), dict(group=48), dict(group=4), dict(n_q_heads=12),
    dict(n_q_heads=136), dict(n_q_heads=72, group=16), dict(max_patterns=256), dict(mode=5), dict(in_dtype=7),
    dict(v_alpha=0.5), dict(max_tokens=0), dict(batch=0), dict(pattern_window=-1),
    dict(shared_patterns=2), dict(shared_patterns=1, mode=B.MODE_KVARN, max_patterns=0),
    dict(k_per_channel=2), dict(k_per_channel=1, mode=B.MODE_KVARN, max_patterns=0),
    dict(bits=1), dict(bits=1, mode=B.MODE_KVARN, max_patterns=0), dict(mode=3),
    dict(mode=B.MODE_NSN, max_patterns=0, bits=1, group=8, n_q_heads=96)])
def test_layout_rejects_bad_configs(bad):
    """(n_q_heads 136 = 17 q-heads per kv-head; 72 at group 16 = 9 q-heads on
    a shape only the VALU attention serves, which holds at most 8.)"""
    with pytest.raises(B.KvqError) as e:
        B.kvq_layout_of(_cfg(**bad))
    assert e.value.status == B.KVQ_EINVAL


def _fake_cache(n_tokens=0, **kw):
    """A cache struct bound to a fake, aligned device address.  Only host
    argument checks run; every call below must fail before any launch."""
    c = B.kvq_cache()
    c.cfg = _cfg(**kw)
    c.base = 1 << 20
    c.n_tokens = n_tokens
    return c


def test_error_paths_fail_before_launch():
    lib = B.lib()
    p = C.c_void_p(1 << 24)
    c = _fake_cache(n_tokens=4090)
    assert lib.kvq_encode_append(C.byref(c), p, p, 7, 0, None) == B.KVQ_ECAPACITY
    assert c.n_tokens == 4090
    assert lib.kvq_encode_append(C.byref(c), p, p, -1, 0, None) == B.KVQ_EINVAL
    assert lib.kvq_encode_append(C.byref(c), None, p, 1, 0, None) == B.KVQ_EINVAL
    assert lib.kvq_encode_append(C.byref(c), C.c_void_p((1 << 24) + 4), p, 1, 0, None) == B.KVQ_EINVAL
    assert lib.kvq_encode_append(C.byref(c), p, p, 0, 0, None) == B.KVQ_OK   # no-op
    empty = _fake_cache(n_tokens=0)
    assert lib.kvq_attn_decode(C.byref(empty), p, p, 0.0, None) == B.KVQ_ESTATE
    assert lib.kvq_attn_decode(C.byref(c), None, p, 0.0, None) == B.KVQ_EINVAL
    assert lib.kvq_dequant(C.byref(c), 2, 0, 1, p, None) == B.KVQ_EINVAL
    assert lib.kvq_dequant(C.byref(c), 0, 4000, 91, p, None) == B.KVQ_EINVAL
    assert lib.kvq_dequant(C.byref(c), 0, -1, 1, p, None) == B.KVQ_EINVAL
    assert lib.kvq_dequant(C.byref(c), 0, 0, 0, p, None) == B.KVQ_OK         # no-op
    assert lib.kvq_set_patterns(C.byref(c), p, p, 33, None) == B.KVQ_EINVAL  # > max_patterns
    assert lib.kvq_set_patterns(C.byref(c), None, p, 3, None) == B.KVQ_EINVAL
    assert lib.kvq_init_patterns(C.byref(c), p, p, 0, 8, None) == B.KVQ_EINVAL
    assert lib.kvq_init_patterns(C.byref(c), p, p, 64, 33, None) == B.KVQ_EINVAL
    big = _fake_cache(max_patterns=128)
    assert lib.kvq_init_patterns(C.byref(big), p, p, 64, 100, None) == B.KVQ_EINVAL  # GPU k-means <= 64
    cache = B.kvq_cache()
    cfg = _cfg()
    L = B.kvq_layout_of(cfg)
    assert lib.kvq_cache_init(C.byref(cache), C.byref(cfg), C.c_void_p((1 << 20) + 64),
                              L.total, None) == B.KVQ_EINVAL      # not 256-byte aligned
    assert lib.kvq_cache_init(C.byref(cache), C.byref(cfg), C.c_void_p(1 << 20), L.total - 1,
                              None) == B.KVQ_EINVAL               # too small
    bad = _cfg(bits=3)
    assert lib.kvq_cache_init(C.byref(cache), C.byref(bad), C.c_void_p(1 << 20), 1 << 30,
                              None) == B.KVQ_EINVAL
    for s in (0, -1, -2, -3, -4, -5, -99):
        assert B.kvq_strerror(s)
    flags = C.c_uint32(7)
    assert lib.kvq_cache_status(None, C.byref(flags), 1, None) == B.KVQ_EINVAL
    assert lib.kvq_cache_status(C.byref(c), None, 1, None) == B.KVQ_EINVAL
    assert lib.kvq_cache_status(C.byref(B.kvq_cache()), C.byref(flags), 1, None) == B.KVQ_EINVAL
    assert flags.value == 7                                     # untouched on failure


def test_noalloc_error_paths_fail_before_launch():
    """kvq_attn_decode_noalloc checks its arguments and its workspace need
    against the static scratch before touching the device."""
    lib = B.lib()
    p = C.c_void_p(1 << 24)
    empty = _fake_cache(n_tokens=0)
    assert lib.kvq_attn_decode_noalloc(C.byref(empty), p, p, 0.0, None) == B.KVQ_ESTATE
    c = _fake_cache(n_tokens=100)
    assert lib.kvq_attn_decode_noalloc(C.byref(c), None, p, 0.0, None) == B.KVQ_EINVAL
    assert lib.kvq_attn_decode_noalloc(C.byref(c), p, C.c_void_p((1 << 24) + 4), 0.0,
                                       None) == B.KVQ_EINVAL
    # 520 x 32 (batch, q-head) rows: 66560 bytes of counters and 8.65 MB of
    # partials at one split, beyond the 64 KiB + 8 MiB scratch
    wide = _fake_cache(n_tokens=100, batch=520)
    assert lib.kvq_attn_decode_noalloc(C.byref(wide), p, p, 0.0, None) == B.KVQ_ESCRATCH
    assert "scratch" in B.kvq_strerror(B.KVQ_ESCRATCH)


def test_product_path_has_no_cpu_fallback(monkeypatch, tmp_path):
    """Without libkvq.so the binding raises instead of computing anything."""
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.lib()


def test_package_does_not_import_oracle():
    """The product package never references the oracle."""
    pkg = os.path.join(ROOT, "bit_kv_cache_encode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower() or f == "synth.py", f
                assert "kvqref" not in text, f
