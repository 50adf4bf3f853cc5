"""AddressSanitizer + UndefinedBehaviorSanitizer build of the host library,
running the C-ABI tests against it (CPU only).

Every kernel source is compiled as the library's own build does, with the
sanitizers on the host compilation only (each -fsanitize= behind
-Xarch_host; device code is built unchanged), linked into a library in a
temporary directory, and tests/test_abi.py runs against that library in a
child process with the clang ASan runtime preloaded.  Any sanitizer report
aborts the child (halt on error, no recovery), so the test fails on the
first invalid access or undefined operation in argument validation, the
workspace queries, status strings or the binding's calls.  test_abi.py
makes no device calls, so no GPU is needed.
"""

import concurrent.futures
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized(out_dir):
    from gated_delta_rule_54_amd import _build
    hipcc = _build.hipcc()
    flags = [f for f in _build.FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE

    def compile_one(src):
        obj = os.path.join(out_dir, src[:-4] + ".o")
        r = subprocess.run([hipcc, *flags, "-c", os.path.join(_build.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed on {src}:\n{r.stderr[-4000:]}"
        return obj

    srcs = _build.sources()
    with concurrent.futures.ThreadPoolExecutor(min(len(srcs), 4)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(out_dir, "libgdr_sanitized.so")
    r = subprocess.run([hipcc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-o", lib, *objs],
                       capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"
    return lib


def test_abi_tests_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if rt is None:
        pytest.skip("the clang ASan runtime is not installed")
    lib = build_sanitized(str(tmp_path))
    driver = tmp_path / "run_abi.py"
    driver.write_text(textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        from gated_delta_rule_54_amd import binding
        binding.LIB_PATH = {lib!r}
        import pytest
        sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {os.path.join(ROOT, "tests", "test_abi.py")!r}]))
    """))
    env = dict(os.environ)
    # the runtime goes first; whatever else is preloaded stays
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, str(driver)], env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-3000:] + r.stderr[-6000:]
    assert r.returncode == 0, report
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, report
    assert " passed" in r.stdout, report
