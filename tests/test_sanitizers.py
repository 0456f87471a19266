"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two executables are built in a temporary folder and run; each must exit 0 with no sanitizer
report:
  * oracle/oracle.c with tests/sanitize/oracle_driver.c (gcc, OpenMP): every oracle entry
    point over many shapes, edge cases and error paths, every buffer allocated at exactly its
    contract size;
  * the library's sources with tests/sanitize/abi_driver.cpp (hipcc; the sanitizers apply to
    the host compilation only): every C entry point with arguments its validation rejects,
    M = 0 no-ops, workspace sizing over many shapes, every status string.
The sanitizer runtimes are linked into the executables (nothing is preloaded).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:")


def _run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, env=SAN_ENV, timeout=300)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    for r in REPORTS:
        assert r not in text, text[-4000:]
    return text


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_asan_ubsan(outdir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = os.path.join(outdir, "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-std=c99", "-Wall",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
           "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    assert "all calls returned the expected status" in _run(exe)


def test_abi_host_under_asan_ubsan(outdir):
    from rank_adapter_gemm_sgmv_amd import build as B

    hipcc = B.hipcc()
    # host-side sanitizers only: each -fsanitize= directly after -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-g"]
    objs = []
    procs = []
    for src in B.SOURCES + ["abi_driver.cpp"]:
        path = os.path.join(HERE, src) if src == "abi_driver.cpp" else os.path.join(B.CSRC, src)
        obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
        flags = [f for f in B.COMMON_FLAGS if f != "-fPIC"]
        procs.append(subprocess.Popen([hipcc, *flags, *san, "-c", path, "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out[-4000:]
    exe = os.path.join(outdir, "abi_driver")
    link = [hipcc, f"--offload-arch={B.ARCH}", *objs, "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", "-o", exe]
    res = subprocess.run(link, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all calls returned the expected status" in _run(exe)
