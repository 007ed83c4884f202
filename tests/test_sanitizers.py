"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each loaded into a fresh Python process with its sanitizer runtime preloaded,
then run against existing CPU tests:
- the oracle (oracle/moe_oracle.c) and the input generator (gen.c), built by gcc with
  -fsanitize=address,undefined: the oracle pins on the small workloads, which call every
  oracle function (routing, dispatch, bias rule, quantisation, expert rows, the layer,
  combine, backward);
- the C ABI's host code (csrc/abi.cpp), built by hipcc with both sanitizers on the host
  side only (-Xarch_host before each -fsanitize: the device code is the normal gfx950
  build) and linked with the other objects of libmoe.so: the host ABI tests, which drive
  every argument check and the workspace sizing without a GPU.
Any sanitizer report fails the run (halt on the first error, non-zero exit). Leak checking
is off: the Python interpreter itself holds memory until exit.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mixture_experts_layer_26_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87"}

# the oracle pins that run in seconds (the slow ones repeat the same functions at larger sizes)
ORACLE_SUBSET = ("not thread_count and not matrix_form and not exhaustive and not mid_bf16 "
                 "and not exact_invariants and not fp8_vs_bf16")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...: rc {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _pytest_in_child(tmp_path, preload, setup, args, must_map, must_not_map):
    """Run pytest on `args` in a fresh interpreter with `preload` loaded first; `setup` is
    Python code run before the tests (it points the loaders at the sanitized builds). After
    the tests the child checks its own memory map: every library of `must_map` (the
    sanitized builds) is loaded and none of `must_not_map` (the normal builds) is."""
    script = tmp_path / "run.py"
    check = (f"maps = open('/proc/self/maps').read()\n"
             f"bad = [p for p in {list(must_map)!r} if p not in maps] + [p for p in {list(must_not_map)!r} if p in maps]\n"
             f"if bad: print('library map check failed:', bad); sys.exit(3)\n")
    script.write_text(f"import sys\nsys.path.insert(0, {ROOT!r})\n{setup}\nimport pytest\n"
                      f"rc = pytest.main({args!r})\n{check}sys.exit(rc)\n")
    env = dict(os.environ, LD_PRELOAD=preload, OMP_NUM_THREADS="4", **SAN_ENV)
    r = subprocess.run([sys.executable, str(script)], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    libasan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    flags = ["-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]
    orc = tmp_path / "libmoe_oracle_san.so"
    gen = tmp_path / "libmoe_inputs_san.so"
    _run(["gcc", "-std=c11", "-Wall"] + flags + ["-o", str(orc), os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    _run(["gcc"] + flags + ["-o", str(gen), os.path.join(PKG, "inputs", "gen.c"), "-lm"])
    setup = (f"import oracle\noracle._LIB_PATH = {str(orc)!r}\n"
             f"from mixture_experts_layer_26_amd import inputs\ninputs._LIB_PATH = {str(gen)!r}\n")
    out = _pytest_in_child(tmp_path, libasan, setup,
                           [os.path.join(ROOT, "tests", "test_oracle.py"),
                            os.path.join(ROOT, "tests", "test_oracle_backward.py"),
                            "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", "-k", ORACLE_SUBSET],
                           [str(orc), str(gen)],
                           [os.path.join(ROOT, "oracle", "libmoe_oracle.so"),
                            os.path.join(PKG, "inputs", "libmoe_inputs.so")])
    assert " passed" in out and " failed" not in out


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_host_code_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    if not any(o.endswith("abi.o") for o in objs):
        pytest.skip("libmoe.so has not been built here (no objects)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    abi_o = tmp_path / "abi_san.o"
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip",
          "-I", os.path.join(ROOT, "include")] + san + ["-c", os.path.join(PKG, "csrc", "abi.cpp"),
                                                        "-o", str(abi_o)])
    lib = tmp_path / "libmoe_san.so"
    others = [o for o in objs if not o.endswith("abi.o")]
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-o", str(lib), str(abi_o)] + others)
    setup = f"from mixture_experts_layer_26_amd import abi\nabi.LIB_PATH = {str(lib)!r}\n"
    out = _pytest_in_child(tmp_path, rt, setup, [os.path.join(ROOT, "tests", "test_abi_host.py"), "-q", "-x",
                                                 "-p", "no:cacheprovider"],
                           [str(lib)], [os.path.join(PKG, "libmoe.so")])
    assert " passed" in out and " failed" not in out
