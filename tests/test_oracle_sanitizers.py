"""The C oracles under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Builds oracle/attn_oracle.c and oracle/chunk_oracle.c with
-fsanitize=address,undefined (gcc, host code only) into a temporary
directory, then runs the oracle pins (test_oracle.py, test_chunk_oracle.py)
in a child process whose oracle wrappers load those builds
(ATTN_ORACLE_LIB, ATTN_CHUNK_ORACLE_LIB).  The pins must pass and no
sanitizer may report: an out-of-bounds access, a use after free, a signed
overflow or a bad shift anywhere in the oracles fails this test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins_sanitized(tmp_path, attn_source):
    """Builds the two oracles with the sanitizers (attn_oracle.c from the
    given text) and runs the pins against them in a child process."""
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    attn_c = tmp_path / "attn_oracle.c"
    attn_c.write_text(attn_source)
    libs = {}
    for src, env in ((str(attn_c), "ATTN_ORACLE_LIB"),
                     (os.path.join(ORACLE, "chunk_oracle.c"), "ATTN_CHUNK_ORACLE_LIB")):
        so = tmp_path / (os.path.basename(src)[:-2] + "_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                        src, "-lm"], check=True)
        libs[env] = str(so)
    # reports go to files: a sanitizer ends the child inside a test, where
    # pytest's own output capture would swallow what it prints
    logs = tmp_path / "reports"
    logs.mkdir()
    env = dict(os.environ, **libs,
               LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:"
                            f"verify_asan_link_order=0:log_path={logs}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_oracle.py", "tests/test_chunk_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(f.read_text() for f in sorted(logs.iterdir()))
    return r.returncode, r.stdout, reports + r.stdout + r.stderr


def test_oracle_pins_pass_under_address_and_undefined_sanitizers(tmp_path):
    rc, out, log = _run_pins_sanitized(tmp_path, open(os.path.join(ORACLE, "attn_oracle.c")).read())
    assert rc == 0, log[-4000:]
    assert "passed" in out and " failed" not in out, log[-4000:]
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in log, log[-4000:]


def test_a_planted_overrun_is_reported(tmp_path):
    # the harness itself: a copy of the oracle whose score loop reads one
    # element past each key row (past the last row's buffer for the last key)
    src = open(os.path.join(ORACLE, "attn_oracle.c")).read()
    site = "for (int d = 0; d < D; ++d)\n            dot += qrow[d] * K[j * D + d];"
    assert src.count(site) == 1
    rc, _, log = _run_pins_sanitized(tmp_path, src.replace(site, site.replace("d < D", "d <= D")))
    assert rc != 0 and "AddressSanitizer" in log, log[-4000:]
