"""Host code under AddressSanitizer, on the CPU: the oracle (gcc) and the host
side of the HIP library (argument checks, size computations, the per-kernel
timer's setup and teardown; hipcc with the sanitizer on the host compilation
only) are rebuilt with -fsanitize=address, and their host tests are run again
against those builds in a child process that preloads the sanitizer runtime.
Any report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
ORACLE_TESTS = ["test_oracle_plan.py", "test_oracle_gather_combine.py", "test_oracle_ffn.py",
                "test_oracle_route.py", "test_oracle_formats.py"]
LIBRARY_TESTS = ["test_abi_host.py", "test_host_sizes.py"]


def run_under_asan(runtime, env_extra, tests):
    env = dict(os.environ, LD_PRELOAD=runtime, PYTHONDONTWRITEBYTECODE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=97", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(TESTS, t) for t in tests]]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


def test_oracle_under_asan(tmp_path):
    lib = str(tmp_path / "liboracle_asan.so")
    src = os.path.join(ROOT, "oracle", "oracle.c")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-fno-fast-math", "-fno-omit-frame-pointer",
                    "-fsanitize=address", "-o", lib, src, "-lm"], check=True)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    run_under_asan(runtime, {"MOE_ORACLE_LIB_OVERRIDE": lib}, ORACLE_TESTS)


def test_library_host_code_under_asan(tmp_path):
    from mixture_experts_routed_amd import build

    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    lib = build.build(host_flags=("-fsanitize=address", "-fno-omit-frame-pointer"),
                      lib=str(tmp_path / "libmoe_routed_asan.so"),
                      build_dir=str(tmp_path / "obj"))
    run_under_asan(rt[0], {"MOE_ROUTED_LIB_OVERRIDE": lib}, LIBRARY_TESTS)


def test_asan_build_reports_a_planted_overflow(tmp_path):
    """the harness above is armed: a copy of the oracle with one planted
    out-of-bounds write (the plan's count clearing runs one expert past the end
    of cnt) is reported by the same sanitizer run"""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "    for (int e = 0; e < E; ++e) cnt[e] = 0;\n"
    assert src.count(good) == 1
    bad = tmp_path / "oracle_bad.c"
    bad.write_text(src.replace(good, "    for (int e = 0; e <= E; ++e) cnt[e] = 0;\n"))
    lib = str(tmp_path / "liboracle_bad.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fno-omit-frame-pointer", "-fsanitize=address", "-o", lib, str(bad), "-lm"],
                   check=True)
    runtime = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    with pytest.raises(AssertionError) as e:
        run_under_asan(runtime, {"MOE_ORACLE_LIB_OVERRIDE": lib}, ["test_oracle_plan.py"])
    assert "heap-buffer-overflow" in str(e.value)
