"""Host-code sanitizer runs (CPU only).

* The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc;
  any report aborts) runs its pin tests under the ASan runtime.
* The host side of the library's C ABI (argument checks, layout, launch
  choice: kvq_api.hip compiled with the sanitizers for the host pass only;
  device code is not instrumented) runs the host ABI tests under clang's ASan
  runtime.

Each suite runs in a subprocess with the runtime preloaded, since the Python
interpreter itself is not instrumented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"sanitizer runtime not found ({' '.join(cmd)})")
    return p


def _run_suite(files, env_extra):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-p", "no:cacheprovider", "-q", "-x",
                        "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "libkvqref_san.so"))
    asan = _runtime(["gcc", "-print-file-name=libasan.so"])
    out = _run_suite(["tests/test_oracle_pins.py", "tests/test_oracle_kchannel.py",
                      "tests/test_oracle_nsn.py", "tests/test_oracle_shared.py"],
                     {"KVQREF_LIB": lib, "LD_PRELOAD": asan})
    assert " passed" in out


def test_host_abi_under_asan_ubsan(tmp_path):
    objs = [os.path.join(ROOT, "bit_kv_cache_encode_amd", "_build", f + ".o")
            for f in ("encode", "attn", "attn_mfma", "misc")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run __graft_entry__.build() first)")
    api = str(tmp_path / "kvq_api_san.o")
    # sanitizers on the host pass only (each -fsanitize after -Xarch_host)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
                    "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
                    "-fhip-fp32-correctly-rounded-divide-sqrt",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer", "-w",
                    "-c", os.path.join(ROOT, "bit_kv_cache_encode_amd", "csrc", "kvq_api.hip"),
                    "-o", api], check=True, capture_output=True)
    lib = str(tmp_path / "libkvq_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-fno-gpu-sanitize", "-shared-libasan", "-o", lib, api, *objs],
                   check=True, capture_output=True)
    asan = _runtime([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"])
    out = _run_suite(["tests/test_host_abi.py"], {"KVQ_LIB": lib, "LD_PRELOAD": asan})
    assert " passed" in out
