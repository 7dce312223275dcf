"""The host code and the oracle under AddressSanitizer and UBSan (CPU only).

* libvga.so rebuilt with sanitized host code (argument validation,
  workspace layouts, schedules, the C ABI; the device code is built as
  usual) runs tests/test_abi_host.py;
* vga_oracle.c rebuilt with gcc's sanitizers runs the oracle's pins,
  tests/test_oracle.py.

Each suite runs in a child process that preloads its compiler's sanitizer
runtime (clang's for libvga, gcc's for the oracle; the two runtimes cannot
share a process), with UBSan set to stop at the first report and leak
detection off (the interpreter itself is not instrumented).  Both children
first check that the sanitized build is the one they loaded.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=23",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=24"}
pytestmark = pytest.mark.slow


def _builder():
    path = os.path.join(ROOT, "alternating_attention_amd", "_build.py")
    spec = importlib.util.spec_from_file_location("_vga_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(env_extra, test_file, probe):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    # the child loaded the sanitized build, with the runtime in place
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-q", "-x", "-p",
                        "no:cacheprovider", "-m", "not gpu"], env=env, cwd=ROOT,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


PROBE = r"""
import sys
sys.path.insert(0, '.')
import {module} as m
maps = open('/proc/self/maps').read()
assert {path!r} in maps, 'sanitized build not loaded'
assert 'asan' in maps, 'sanitizer runtime not loaded'
{extra}
print('ok')
"""


def test_host_abi_under_sanitizers():
    b = _builder()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    lib = b.build_sanitized()
    probe = PROBE.format(module="alternating_attention_amd", path=lib,
                         extra="assert m.LIB_PATH == %r" % lib)
    _run({"LD_PRELOAD": b.sanitizer_runtime(), "VGA_LIB_PATH": lib}, "tests/test_abi_host.py",
         probe)


def test_oracle_pins_under_sanitizers():
    out = os.path.join(ROOT, "_build", "asan", "libvga_oracle.so")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    oracle.build_sanitized(out)
    probe = PROBE.format(module="oracle", path=out, extra="m._load()")
    # the probe maps the library only once _load() ran: check after it
    probe = probe.replace("maps = open", "m._load()\nmaps = open", 1)
    _run({"LD_PRELOAD": oracle.sanitizer_runtime(), "VGA_ORACLE_LIB": out},
         "tests/test_oracle.py", probe)
