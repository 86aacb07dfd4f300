"""Build and run the host-only pool check under sanitizers.

    python paged_kv_speculative_amd/csrc/host_check/run.py [--ops N]

Two g++ builds of pool.cpp with host_check.cpp (no HIP code): one with
AddressSanitizer + UndefinedBehaviorSanitizer, one with ThreadSanitizer.
Each runs the serial random-operation phases and the threaded phase; any
sanitizer report makes the run fail.  Binaries go to a temporary directory.
"""
import argparse
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.dirname(HERE)
SOURCES = [os.path.join(CSRC, "pool.cpp"), os.path.join(HERE, "host_check.cpp")]
COMMON = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread"]
BUILDS = {
    "asan+ubsan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
    "tsan": ["-fsanitize=thread"],
}
ENV = {
    "asan+ubsan": {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
                   "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"},
    "tsan": {"TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"},
}


def run(ops=600, builds=tuple(BUILDS)):
    """Build and run every sanitizer variant; returns {build: stdout}."""
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        for name in builds:
            exe = os.path.join(tmp, "host_check_" + name.replace("+", "_"))
            cmd = ["g++"] + COMMON + BUILDS[name] + SOURCES + ["-o", exe]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"{name} build failed:\n{' '.join(cmd)}\n{r.stderr}")
            env = dict(os.environ, **ENV[name])
            r = subprocess.run([exe, str(ops)], capture_output=True, text=True, env=env, timeout=600)
            if r.returncode != 0 or "Sanitizer" in r.stderr or "runtime error" in r.stderr:
                raise RuntimeError(f"{name} run failed (rc {r.returncode}):\n{r.stdout}\n{r.stderr}")
            out[name] = r.stdout
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--ops", type=int, default=600)
    a = ap.parse_args()
    for name, text in run(a.ops).items():
        print(f"[{name}]\n{text}", end="")
    sys.exit(0)
