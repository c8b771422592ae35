"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two sanitized builds of the same sources, each loaded in a child process with
its sanitizer runtime preloaded:
* the oracle (gcc, -fsanitize=address,undefined, every report fatal) running
  its pin tests -- including its pthread pool over (sequence, kv head);
* the library with its host unit instrumented (hipcc -Xarch_host
  -fsanitize=address,undefined; the device code is as usual) running the
  C-ABI rejection and planning tests and the binding's argument checks --
  every call there fails validation or only plans, so no device is touched.
Either run fails on any sanitizer report (a planted heap overflow in a copy
of the oracle is reported and fails it).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_fp8.py", "tests/test_oracle_mq.py",
               "tests/test_oracle_lse.py", "tests/test_oracle_alibi.py"]
ABI_TESTS = ["tests/test_abi_cpu.py", "tests/test_binding_cpu.py"]
REPORT = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer",
          "UndefinedBehaviorSanitizer")


def run_child(tests, env_extra, preload, logdir):
    """Run `tests` in a child pytest with the sanitizer runtime preloaded; reports
    go to files under logdir (the child's stderr is captured by its own pytest)."""
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    log = os.path.join(str(logdir), "san")
    # (leak checking off: the interpreter keeps its own allocations at exit)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert not reports, reports[:4000]
    assert r.returncode == 0 and not any(k in out for k in REPORT), out[-4000:]
    return out


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    oracle.compile_source(os.path.join(ROOT, "oracle", "paged_decode_oracle.c"), lib,
                          sanitize=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True).stdout.strip()
    out = run_child(ORACLE_PINS, {"PA_ORACLE_LIB": lib}, libasan, tmp_path)
    assert " passed" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    from paged_kv_cache_v2_amd import build
    lib = str(tmp_path / "libpaged_attn_san.so")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-g"]
    host_flags = [f for flag in san for f in ("-Xarch_host", flag)]
    build.build(out=lib, host_flags=host_flags)
    out = run_child(ABI_TESTS, {"PAGED_ATTN_LIB": lib}, rts[-1], tmp_path)
    assert " passed" in out
