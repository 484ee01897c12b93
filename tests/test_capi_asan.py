"""CPU: the C-ABI suite (tests/test_capi_cpu.py) against a host-side
AddressSanitizer build of the library: every argument check, workspace size
and dispatch decision of the host shim runs instrumented, with the ASan
runtime preloaded into a child Python process.  No GPU is touched (device
code is built as usual and never launched here)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "_mtla_build", os.path.join(ROOT, "temporally_compressed_latent_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_capi_suite_clean_under_host_asan():
    b = _build_module()
    lib = b.build_host_asan()
    runtime = b.asan_runtime()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms, "the host code is not instrumented"
    env = dict(os.environ, MTLA_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_capi_cpu.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr, out
    assert r.returncode == 0, out
    assert " passed" in r.stdout, out
