"""The CPU oracle under the sanitizers the decode page runs its kernel under
("Paged attention for decode in C", Overview and "What the tests check": the tests
run under AddressSanitizer, UndefinedBehaviorSanitizer and ThreadSanitizer, and the
thread pool's result must equal the serial one bit for bit, also under TSan).

oracle.c is built with gcc and -fsanitize=..., loaded into a child Python process
with the sanitizer runtime preloaded, and every pin of oracle_pins.py runs against
it; any sanitizer report makes the child fail.  Each sanitizer is also shown to be
live: a copy of the oracle with one planted out-of-bounds write, or one planted data
race, must be reported.
"""
import json
import os
import subprocess
import sys

import pytest

from oracle import oracle as oracle_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def build(src_text, out, flags):
    src = out + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", *flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def run_child(code, preload, extra_env):
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(preload)
    env.update(extra_env)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600, cwd=ROOT,
                          env=env)


def all_pins(lib):
    return f"import sys; sys.path.insert(0, {ROOT!r}); from tests import oracle_pins; oracle_pins.run_all({lib!r})"


def failed_pins(proc):
    lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
    assert lines, proc.stdout + proc.stderr
    return json.loads(lines[-1])["failed"]


ASAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
# torch's own CPU kernels (the dense references of the pins) run on one thread: its
# OpenMP runtime is not built with TSan, whose reports there would not concern the
# oracle.  The oracle's thread pool is unaffected.
TSAN_ENV = {"TSAN_OPTIONS": "halt_on_error=1:report_signal_unsafe=0", "OMP_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}
ASAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def asan_runtimes():
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's ASan / UBSan runtimes are not installed")
    return [asan, ubsan]


@pytest.fixture(scope="module")
def tsan_runtime():
    tsan = runtime("libtsan.so")
    if tsan is None:
        pytest.skip("gcc's TSan runtime is not installed")
    return [tsan]


def test_pins_clean_under_asan_and_ubsan(tmp_path, asan_runtimes):
    lib = build(open(oracle_mod.SOURCE).read(), str(tmp_path / "liborc_asan.so"), ASAN_FLAGS)
    proc = run_child(all_pins(lib), asan_runtimes, ASAN_ENV)
    assert proc.returncode == 0, proc.stderr[-4000:]
    assert "AddressSanitizer" not in proc.stderr and "runtime error" not in proc.stderr, proc.stderr[-4000:]
    assert failed_pins(proc) == []


def test_asan_reports_a_planted_overflow(tmp_path, asan_runtimes):
    """Control: rows written at the QK stride (192) instead of the V stride (128)
    run past the output array; ASan must stop the child with a report."""
    src = open(oracle_mod.SOURCE).read()
    old = "s, out + r * dv, &m, &l);"
    assert src.count(old) == 1
    lib = build(src.replace(old, "s, out + r * dk, &m, &l);"), str(tmp_path / "liborc_asan_bad.so"), ASAN_FLAGS)
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); from tests import oracle_pins; "
            f"from oracle.oracle import Oracle; oracle_pins.pin_attend_gathered_matches_dense(Oracle({lib!r}))")
    proc = run_child(code, asan_runtimes, ASAN_ENV)
    assert proc.returncode != 0 and "heap-buffer-overflow" in proc.stderr, proc.stderr[-3000:]


def test_pins_clean_under_tsan(tmp_path, tsan_runtime):
    """Every pin, with the oracle's thread pool at the host's core count; the
    invariance pin compares 1 thread with 8 bit for bit."""
    lib = build(open(oracle_mod.SOURCE).read(), str(tmp_path / "liborc_tsan.so"), ["-fsanitize=thread"])
    proc = run_child(all_pins(lib), tsan_runtime, TSAN_ENV)
    assert proc.returncode == 0, proc.stderr[-4000:]
    assert "ThreadSanitizer" not in proc.stderr, proc.stderr[-4000:]
    assert failed_pins(proc) == []


def test_tsan_reports_a_planted_race(tmp_path, tsan_runtime):
    """Control: every (sequence, kv head) task bumps one shared counter without
    synchronisation; TSan must stop the child with a data-race report."""
    src = open(oracle_mod.SOURCE).read()
    old = "static void attn_task(void* ctx, int64_t task) {\n"
    assert src.count(old) == 1
    bad = src.replace(old, "static int64_t racy_tasks;\n" + old + "  racy_tasks += 1;\n")
    lib = build(bad, str(tmp_path / "liborc_tsan_bad.so"), ["-fsanitize=thread"])
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); from tests import oracle_pins; "
            f"from oracle.oracle import Oracle; oracle_pins.pin_invariance(Oracle({lib!r}))")
    proc = run_child(code, tsan_runtime, TSAN_ENV)
    assert proc.returncode != 0 and "data race" in proc.stderr, proc.stderr[-3000:]
