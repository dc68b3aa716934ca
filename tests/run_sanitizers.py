"""CPU sanitizer run of the host-side code: `python tests/run_sanitizers.py`.

Builds, into a scratch directory, AddressSanitizer + UndefinedBehaviorSanitizer copies of
  - the oracle (oracle/oracle.c) and the input generator (synth/synth.c), with clang and the same flags as their
    normal builds,
  - libmoe_q4.so with every host-side part instrumented (the C-ABI validation layer in api.hip and the launchers);
    device code is compiled as usual (each -fsanitize= goes to the host pass only),
then runs `pytest tests -m "not gpu"` with those copies loaded (MOE_Q4_ORACLE_LIB, MOE_Q4_SYNTH_LIB, MOE_Q4_LIB)
and clang's sanitizer runtime preloaded into the Python process.  UBSan findings are fatal; leak checking is off
(the interpreter itself keeps memory until exit).  Exit status: pytest's.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def run(cmd, **kw):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, **kw)


def main() -> int:
    out = tempfile.mkdtemp(prefix="moe_q4_sanitize_")
    # the oracle and the input generator: their normal flags plus the sanitizers
    orc = os.path.join(out, "liboracle.so")
    run([CLANG, "-O1", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", *SAN,
         os.path.join(ROOT, "oracle", "oracle.c"), "-o", orc, "-lm"])
    syn = os.path.join(out, "libsynth.so")
    run([CLANG, "-O1", "-std=c99", "-fPIC", "-shared", *SAN, os.path.join(ROOT, "synth", "synth.c"), "-o", syn,
         "-lm"])
    # the library: host passes instrumented
    sys.path.insert(0, os.path.join(ROOT, "quantized_moe_q4_amd"))
    import build as libbuild  # quantized_moe_q4_amd/build.py
    host = []
    for f in SAN:
        host += ["-Xarch_host", f]
    lib = libbuild.build(verbose=False, extra=host, lib=os.path.join(out, "libmoe_q4.so"),
                         objdir=os.path.join(out, "obj"))  # the runtime comes from LD_PRELOAD
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                             capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    env.update({
        "MOE_Q4_ORACLE_LIB": orc,
        "MOE_Q4_SYNTH_LIB": syn,
        "MOE_Q4_LIB": lib,
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    print(f"[sanitize] libraries in {out}; runtime {runtime}", flush=True)
    # pre-flight: the sanitized copies are the ones loaded, and the runtime is live in the process
    probe = ("import ctypes, sys; sys.path.insert(0, '.'); import oracle, synth, quantized_moe_q4_amd as mq; "
             "oracle._load(); synth._load(); mq.load_library(); "
             "maps = open('/proc/self/maps').read(); "
             "assert all(p in maps for p in (oracle._LIB_PATH, synth._LIB_PATH, mq.LIB_PATH)), 'sanitized libs'; "
             "ctypes.CDLL(None).__asan_get_report_address; print('[sanitize] runtime live, sanitized libraries loaded')")
    subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, check=True)
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q", "-x",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env)
    return res.returncode


if __name__ == "__main__":
    sys.exit(main())
