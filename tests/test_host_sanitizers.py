"""The host packer under AddressSanitizer and UndefinedBehaviorSanitizer.

ternary_hybrid_bit_amd/csrc/wal_host.cpp (blob layout, packer, validator,
unpacker, the INT3/4/5 packers and the workspace-size queries) is plain C++
with no HIP code, so it is compiled here with g++ and both sanitizers, next
to the driver tests/sanitize/packer_fuzz.cpp, which calls it through the C
ABI of include/wal.h with every buffer in a heap block of exactly its
declared size: round trips of random shapes of every format, rejected
inputs, truncated and corrupted blobs, lying headers.  Any out-of-bounds
access, use of freed memory, leak, signed overflow, bad shift or misaligned
access aborts the driver.  Two planted mistakes (in tiny programs of their
own, not in the library) first show that this toolchain's sanitizers do
report what they should.

The blobs' fail-closed validation follows the WAL-Ternary-8B card ("Install":
the executable cache is verified fail-closed before use).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "sanitize", "packer_fuzz.cpp")
HOST = os.path.join(ROOT, "ternary_hybrid_bit_amd", "csrc", "wal_host.cpp")

SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1:strict_string_checks=1:"
                    "detect_stack_use_after_return=1",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    return gxx


def _build(tmp_path, sources, name, extra=()):
    exe = str(tmp_path / name)
    cmd = [_gxx(), "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *SAN_FLAGS, *extra, *sources, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr) and "cannot find" in r.stderr:
        pytest.skip("the sanitizer runtimes are not installed: " + r.stderr.strip()[-200:])
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args, timeout=300):
    env = dict(os.environ, **SAN_ENV)
    return subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout, env=env)


def test_sanitizers_report_planted_mistakes(tmp_path):
    oob = tmp_path / "oob.cpp"
    oob.write_text("#include <cstdlib>\n"
                   "int main(int argc, char**) { char* p = (char*)std::malloc(16); p[15 + argc] = 1;"
                   " int r = p[0]; std::free(p); return r; }\n")
    r = _run(_build(tmp_path, [str(oob)], "oob", ["-Wno-error"]))
    # the object-size check of UBSan or the heap redzone of ASan, whichever sees it first
    assert r.returncode != 0 and ("heap-buffer-overflow" in r.stderr or "insufficient space" in r.stderr), \
        r.stderr[-2000:]

    uaf = tmp_path / "uaf.cpp"
    uaf.write_text("#include <cstdlib>\n"
                   "int main(int argc, char**) { char* p = (char*)std::malloc(16); p[0] = (char)argc;"
                   " std::free(p); return p[0]; }\n")
    r = _run(_build(tmp_path, [str(uaf)], "uaf", ["-Wno-error"]))
    assert r.returncode != 0 and "heap-use-after-free" in r.stderr, r.stderr[-2000:]

    ovf = tmp_path / "ovf.cpp"
    ovf.write_text("#include <climits>\n"
                   "int main(int argc, char**) { int v = INT_MAX - 1 + argc; v += argc; return v == 7; }\n")
    r = _run(_build(tmp_path, [str(ovf)], "ovf"))
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-2000:]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_host_packer_under_asan_ubsan(tmp_path, seed):
    exe = _build(tmp_path, [DRIVER, HOST], "packer_fuzz")
    r = _run(exe, seed, 600)
    out = r.stdout.strip().splitlines()
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert out and out[-1].startswith("packer_fuzz: ok"), r.stdout[-2000:]
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
