"""Host-side AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU only).

* The oracle (oracle/oracle.c) built by gcc with -fsanitize=address,undefined
  (any report aborts) runs every oracle pin in a child process that preloads
  gcc's ASan runtime.
* The library built with the same sanitizers on its host pass (hipcc
  -Xarch_host -fsanitize=...; device code as usual) runs the host-side ABI
  checks -- argument validation before anything is enqueued, the host
  quantisers against the oracle, partial layouts and workspace queries -- in
  a child process that preloads clang's ASan runtime.  No GPU is touched.
A sanitizer report makes the child fail; its output is shown."""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(runtime, **extra):
    env = dict(os.environ, **extra)
    old = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (" " + old if old else "")      # the ASan runtime must come first
    # leaks of the uninstrumented interpreter and runtimes are not this code's
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    return env


def _pytest(env, files, timeout=900):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    return r.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    assert os.path.isabs(asan) and os.path.exists(asan)
    files = sorted(os.path.relpath(f, ROOT) for f in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    out = _pytest(_env(asan, VW4_ORACLE_LIB=lib), files)
    print(out.strip().splitlines()[-1])


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from verify_step_w4_amd import build
    lib = build.build(out=str(tmp_path / "libvw4_san.so"), sanitize=True)
    rt = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    assert rt, "clang's ASan runtime is missing"
    out = _pytest(_env(rt[0], VW4_LIB=lib), ["tests/test_abi_host.py"])
    print(out.strip().splitlines()[-1])
