"""The CPU sanitizer leg: AddressSanitizer and UndefinedBehaviorSanitizer
(errors fatal) over the C code that runs on the host.

* the oracle (oracle/oracle.c) and the seeded input generator
  (synth/synth.c), built sanitized by ``__graft_entry__.build()``, run the
  oracle's pins, its planted-mistake mutants (each mutant compiled sanitized
  too) and the generator tests in a child process with the ASan runtime
  preloaded;
* the library's host front (argument checks, device check, dispatch of
  include/q4proj.h), compiled for the CPU with recording stand-ins for the
  HIP runtime and the kernel launchers, walks every entry point's accepted
  and rejected arguments (tests/hostcheck);
* two canaries show the flags are live: an out-of-bounds read and a signed
  overflow, each in a tiny program built with the same flags, must be
  reported.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _asan_runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    assert os.path.isabs(path) and os.path.exists(path), path
    return path


def _sanitized_env() -> dict:
    env = dict(os.environ)
    env.update({"LD_PRELOAD": _asan_runtime(), "Q4P_SANITIZED_ORACLE": "1",
                # the interpreter itself never frees some of its memory
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
                "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", "")})
    return env


def test_oracle_pins_and_mutants_under_sanitizers():
    for lib in ("oracle/liboracle_san.so", "synth/libsynth_san.so"):
        assert os.path.exists(os.path.join(ROOT, lib)), f"{lib}: run __graft_entry__.build()"
    env = _sanitized_env()
    probe = subprocess.run(
        [sys.executable, "-c", "import oracle, synth; oracle.load(); synth.load(); "
                               "print(oracle.LIB); print(synth.LIB)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0, probe.stderr[-2000:]
    libs = probe.stdout.split()
    assert libs[0].endswith("liboracle_san.so") and libs[1].endswith("libsynth_san.so"), libs
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
         "tests/test_oracle.py", "tests/test_oracle_mutants.py", "tests/test_synth.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in run.stdout


def test_host_front_under_sanitizers():
    exe = os.path.join(ROOT, "tests", "hostcheck", "hostcheck")
    assert os.path.exists(exe), "tests/hostcheck/hostcheck: run __graft_entry__.build()"
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                         env={**os.environ, "ASAN_OPTIONS": "halt_on_error=1",
                              "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failed" in run.stdout, run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr


@pytest.mark.parametrize("kind,body,report", [
    ("heap read past the end", "int *p = malloc(4 * sizeof *p); int v = p[argc + 3]; free(p); return v;",
     "heap-buffer-overflow"),
    ("signed overflow", "long long v = 0x4000000000000000LL; v *= 2 * argc; return (int)(v >> 62);",
     "signed integer overflow"),
])
def test_sanitizers_are_live(tmp_path, kind, body, report):
    src = tmp_path / "canary.c"
    src.write_text(textwrap.dedent(f"""\
        #include <stdlib.h>
        int main(int argc, char **argv) {{ (void)argv; {body} }}
        """))
    exe = tmp_path / "canary"
    subprocess.run(["gcc", "-std=c11", "-O0", *SAN, str(src), "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"})
    assert run.returncode != 0, f"{kind}: not reported"
    assert report in run.stderr, run.stderr[-2000:]
