"""The host C code -- the CPU oracle and the input generator -- built with
gcc's AddressSanitizer and UndefinedBehaviorSanitizer, running the oracle's
pin suite and the generator's tests in a child process: an out-of-bounds
access, a use after free or an undefined operation (signed overflow, a bad
shift, a misaligned access) in either library stops the run and fails here.
CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _gcc_runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _sanitized_builds(tmp_path, oracle_src):
    libasan = _gcc_runtime("libasan.so")
    if libasan is None:
        pytest.skip("gcc has no AddressSanitizer runtime")
    orc = str(tmp_path / "liboracle_san.so")
    syn = str(tmp_path / "libsynth_san.so")
    # the same flags as the regular builds, plus the sanitizers
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", *SAN, oracle_src, "-o", orc, "-lm"], check=True)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN,
                    os.path.join(ROOT, "synth", "synth.c"), "-o", syn, "-lm"], check=True)
    return dict(os.environ, MOONEP_ORACLE_LIB=orc, MOONEP_SYNTH_LIB=syn, LD_PRELOAD=libasan,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run_pins(env, *select):
    # -s: a sanitizer report goes to the child's stderr, not to pytest's capture
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p",
                           "no:cacheprovider", "-m", "not gpu", *select], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=900)


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    env = _sanitized_builds(tmp_path, os.path.join(ROOT, "oracle", "oracle.c"))
    r = _run_pins(env, "tests/test_oracle_pins.py", "tests/test_synth.py")
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """The same run over an oracle copy whose count loop reads one entry past
    the end of the routing fails with an AddressSanitizer report, so the
    sanitized libraries are the ones the child process loads."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = ("for (int64_t n = 0; n < NK; ++n) {\n        const int32_t e = topk[n];\n"
            "        if (e < 0 || e >= E)\n            return ORC_ERR_EXPERT_ID;\n        T[e] += 1;")
    assert src.count(good) == 1
    bad = tmp_path / "oracle_overflow.c"
    bad.write_text(src.replace(good, good.replace("n < NK", "n <= NK")))
    env = _sanitized_builds(tmp_path, str(bad))
    r = _run_pins(env, "tests/test_oracle_pins.py", "-k", "counts_match_bincount")
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
