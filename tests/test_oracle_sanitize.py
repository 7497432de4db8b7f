"""The CPU oracle built with the address and undefined-behaviour sanitizers
(g++, host code only) and driven through every entry point on small seeded
cases, valid and invalid (tests/csrc/oracle_sanitize.cpp): no sanitizer
report and every call returns the status the case expects."""

import os
import subprocess

import oracle as oracle_pkg

HERE = os.path.dirname(os.path.abspath(__file__))
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    flags = [f for f in oracle_pkg.CXXFLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run(["g++", *flags, *SANITIZE, "-g", os.path.join(HERE, "csrc", "oracle_sanitize.cpp"),
                    oracle_pkg.SRC, "-o", exe], check=True)
    # verify_asan_link_order=0: the sanitizer runtime need not be first if the environment preloads a library
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "ok: 0 failures" in r.stdout
