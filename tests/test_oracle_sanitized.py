"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer:
the C oracle is rebuilt with -fsanitize=address,undefined (gcc, host code
only) and the pin and property tests run against that build in a child
process with the sanitizer runtimes preloaded; any out-of-bounds access, use
after free or undefined behaviour aborts the child. A planted out-of-bounds
read in a separate tiny library must abort the same way, which shows the
sanitizer is live in that environment."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tbe_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.slow


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def san_env(tmp_path_factory):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libtbe_oracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-g", "-fPIC", "-shared", *SAN,
                           "-fno-fast-math", "-ffp-contract=off", "-o", lib, SRC, "-lm"])
    env = dict(os.environ)
    env.update(TBE_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return d, env


def test_sanitizer_is_live(san_env):
    d, env = san_env
    src = d / "oob.c"
    src.write_text("int oob(int i) { int a[4] = {1, 2, 3, 4}; volatile int *p = a; return p[i]; }\n")
    lib = str(d / "liboob.so")
    subprocess.check_call(["gcc", "-O0", "-g", "-fPIC", "-shared", *SAN, "-o", lib, str(src)])
    code = ("import ctypes, sys; L = ctypes.CDLL(sys.argv[1]); "
            "print(L.oob(1)); sys.stdout.flush(); L.oob(6)")
    r = subprocess.run([sys.executable, "-c", code, lib], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.stdout.strip().startswith("2")
    assert r.returncode != 0 and "stack-buffer-overflow" in r.stderr


def test_oracle_pins_under_sanitizers(san_env):
    _, env = san_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_properties.py")],
                       env=env, capture_output=True, text=True, cwd=ROOT, timeout=1500)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
