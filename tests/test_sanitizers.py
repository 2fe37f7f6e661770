"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle and of the C ABI's
host layer, run on the CPU (no GPU needed).

- The oracle (oracle/oracle.c) is compiled with gcc together with tests/sanitize/oracle_main.c,
  which calls every oracle function on edge-case sizes; leak detection stays on.
- The library's sources are compiled with hipcc with the sanitizers on the host side only (the
  GPU code is built as usual and never runs here), and linked with
  tests/sanitize/boundary_main.c, which drives every validation path of include/dsa.h.
Any out-of-bounds access, use after free, leak (oracle) or undefined operation aborts the
program and fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_long_lightning_amd", "csrc")
SRC = ["api.hip", "indexer.hip", "topk.hip", "mqa.hip", "cache.hip", "kl.hip", "check.hip"]


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_asan_ubsan(outdir):
    exe = os.path.join(outdir, "oracle_san")
    run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         "-fopenmp", "-ffp-contract=off", "-Wall", os.path.join(ROOT, "oracle", "oracle.c"),
         os.path.join(SAN, "oracle_main.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", OMP_NUM_THREADS="4")
    assert "ok" in run([exe], env=env)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")
def test_c_abi_host_layer_under_asan_ubsan(outdir):
    from concurrent.futures import ThreadPoolExecutor

    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + host_san
    objs = [os.path.join(outdir, s.replace(".hip", ".o")) for s in SRC]
    with ThreadPoolExecutor(4) as ex:
        list(ex.map(lambda so: run(["hipcc", *flags, "-c", os.path.join(CSRC, so[0]), "-o", so[1]]),
                    zip(SRC, objs)))
    llvm = "/opt/rocm/llvm/bin"
    main = os.path.join(outdir, "boundary_main.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    run([f"{llvm}/clang", "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
         "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(SAN, "boundary_main.c"), "-o", main])
    exe = os.path.join(outdir, "boundary_san")
    run([f"{llvm}/clang++", *san, "-o", exe, main, *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib"])
    # the HIP runtime keeps process-lifetime allocations, so leak detection is off here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    assert "ok" in run([exe], env=env)
