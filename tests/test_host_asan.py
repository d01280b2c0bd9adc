"""The C-ABI layer under AddressSanitizer, on the CPU.

The host code of api.hip (argument validation, workspace sizing, error
strings, the per-device tables) is rebuilt with AddressSanitizer on the host
side only, linked with the regular objects of the other translation units,
and the ABI tests of tests/test_abi.py are run against that build in a
child process with the sanitizer runtime preloaded.  No GPU is used: every
call in those tests returns from validation before any HIP launch.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OTHERS = ["fwd_bf16", "fwd_fp8", "fwd_f32", "decode", "bwd", "calib"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_layer_under_host_asan(tmp_path):
    cc, rt = _hipcc(), _asan_runtime()
    if cc is None or rt is None:
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    objs = [os.path.join(BUILD, n + ".o") for n in OTHERS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("regular objects missing: run __graft_entry__.build() first")
    api_o = str(tmp_path / "api_asan.o")
    lib = str(tmp_path / "libattn_asan.so")
    # sanitizer flags on the host side only (device code is built as usual)
    subprocess.run([cc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "exact_attention_33_amd", "csrc", "api.hip"), "-o", api_o],
                   check=True, capture_output=True)
    subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-shared-libasan", api_o, *objs, "-o", lib], check=True, capture_output=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in nm, "the host code was not instrumented"

    driver = (
        "import sys\n"
        "from exact_attention_33_amd import ops\n"
        f"ops.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py', '-m', 'not gpu']))\n"
    )
    log = str(tmp_path / "asan")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS=f"detect_leaks=0:exitcode=86:log_path={log}")
    r = subprocess.run([sys.executable, "-c", driver], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in os.listdir(tmp_path) if f.startswith("asan"))
    out = r.stdout + r.stderr + reports
    assert not reports and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]
