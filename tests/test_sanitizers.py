"""The host C++ of the library (plan, rank allocation, rotation, FFN weight
preparation) and the CPU oracle, rebuilt with AddressSanitizer and
UndefinedBehaviorSanitizer: the CPU tests that reach that code pass under
them (any report aborts the run).  CPU only; the device code is unchanged."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the CPU tests that call into the host library or the oracle
SUITES = ["tests/test_abi.py", "tests/test_alloc.py", "tests/test_rotation.py", "tests/test_ffn.py",
          "tests/test_oracle_pins.py", "tests/test_binding_checks.py", "tests/test_generator.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_cpu_suites_pass_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    import importlib.util
    import oracle
    spec = importlib.util.spec_from_file_location(
        "_lr_attn_build", os.path.join(ROOT, "latent_kv_attention_lr_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    lib = b.build_sanitized()
    olib = oracle.build(sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LR_ATTN_LIB=lib, LR_ORACLE_LIB=olib)
    # the child also reports which builds it loaded
    probe = ("import latent_kv_attention_lr_amd as l, oracle; oracle.lib(); "
             "print(sorted({x.split()[-1] for x in open('/proc/self/maps') if '_san.so' in x}))")
    out = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    assert out.returncode == 0, out.stderr[-3000:]
    assert lib in out.stdout and olib in out.stdout, out.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
