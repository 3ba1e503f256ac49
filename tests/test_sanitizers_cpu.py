"""The CPU oracle and the host side of the HIP library under AddressSanitizer and UBSan.

Each check builds an instrumented copy, then runs an existing CPU suite in a child process
that loads that copy (MOE_ORACLE_LIB for the oracle, MOE_LATENT_LIB for the library) with
the matching sanitizer runtime preloaded; the child stops at the first report. The copies
are only loadable with their runtime present (their instrumentation leaves its symbols
undefined), so a child that loaded one ran instrumented code. Leak checking is off: the
Python interpreter keeps allocations until exit by design.

- The oracle is built with gcc and runs the oracle's pins and one forward of every workload
  (one row each), whose bits must equal the uninstrumented build's.
- A control: an oracle copy with a planted one-element overflow must be reported.
- The library is built with hipcc, instrumenting host code only (each sanitizer flag behind
  -Xarch_host; the device code is the ordinary build), and runs the C ABI tests that need no
  GPU: every refusal of a bad configuration or descriptor and the library's bookkeeping.
"""
import glob
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PKG = os.path.join(ROOT, "latent_mixture_experts_bf16_amd")

GCC_SAN = ["-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-g"]
HOST_SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
            "-shared-libasan", "-fno-omit-frame-pointer", "-g"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(args, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    return out


def _undefined_sanitizer_symbols(path):
    syms = subprocess.run(["nm", "-D", "--undefined-only", path], check=True, capture_output=True,
                          text=True).stdout
    return [s for s in syms.split() if s.startswith(("__asan_report", "__ubsan_handle"))]


def _build_oracle_san(src, out):
    # the oracle's own floating-point flags, with the sanitizers added
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
                    *GCC_SAN, "-Wall", "-shared", "-fPIC", src, "-o", out, "-lm"], check=True)
    assert _undefined_sanitizer_symbols(out), "the oracle copy is not instrumented"
    return out


@pytest.fixture(scope="module")
def oracle_san(tmp_path_factory):
    return _build_oracle_san(ORACLE_SRC, str(tmp_path_factory.mktemp("oracle_san") / "libmoe_oracle_san.so"))


def _gcc_asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                          text=True).stdout.strip()
    assert os.path.isabs(path) and os.path.exists(path), path
    return path


def test_oracle_pins_under_sanitizers(oracle_san):
    out = _run_child(["-m", "pytest", "tests/test_oracle_pins.py", "-q", "-p", "no:cacheprovider"],
                     {"LD_PRELOAD": _gcc_asan_runtime(), "MOE_ORACLE_LIB": oracle_san})
    assert " passed" in out and " failed" not in out, out[-3000:]


_FORWARD_CHILD = r"""
import sys
import numpy as np
from latent_mixture_experts_bf16_amd import synth
from oracle import oracle as O
res = {}
for cfg in range(len(synth.WORKLOADS)):
    dims, arrays = next(synth.workload_layers(cfg, rows=1))
    ref = O.forward(dims, arrays)
    res[f"out{cfg}"] = ref["out"]
    res[f"idx{cfg}"] = ref["idx"]
    res[f"w{cfg}"] = ref["w"].view(np.uint32)
np.savez(sys.argv[1], **res)
"""


def test_oracle_forward_under_sanitizers_matches_plain_build(oracle_san, tmp_path):
    from latent_mixture_experts_bf16_amd import synth
    from oracle import oracle as O

    dest = str(tmp_path / "san_forward.npz")
    _run_child(["-c", _FORWARD_CHILD, dest],
               {"LD_PRELOAD": _gcc_asan_runtime(), "MOE_ORACLE_LIB": oracle_san})
    got = np.load(dest)
    for cfg in range(len(synth.WORKLOADS)):
        dims, arrays = next(synth.workload_layers(cfg, rows=1))
        ref = O.forward(dims, arrays)
        assert np.array_equal(got[f"idx{cfg}"], ref["idx"]), cfg
        assert np.array_equal(got[f"w{cfg}"], ref["w"].view(np.uint32)), cfg
        assert np.array_equal(got[f"out{cfg}"], ref["out"]), cfg


def test_planted_overflow_is_reported(tmp_path):
    """A control: a copy of the oracle whose latent buffer is allocated one element short
    writes past it on every row, which the sanitized child must report and stop on."""
    with open(ORACLE_SRC) as f:
        text = f.read()
    passage = "float *u = malloc(sizeof(float) * D);"
    assert text.count(passage) == 1
    src = tmp_path / "moe_oracle_short_u.c"
    src.write_text(text.replace(passage, "float *u = malloc(sizeof(float) * (D - 1));"))
    lib = _build_oracle_san(str(src), str(tmp_path / "libmoe_oracle_short_u.so"))
    child = ("from latent_mixture_experts_bf16_amd import synth\n"
             "from oracle import oracle as O\n"
             "dims, arrays = next(synth.workload_layers(0, rows=1))\n"
             "O.forward(dims, arrays)\n")
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update({"LD_PRELOAD": _gcc_asan_runtime(), "MOE_ORACLE_LIB": lib})
    r = subprocess.run([sys.executable, "-c", child], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer: heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def _sources_digest():
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
                   + [os.path.join(PKG, "build.py")])
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("hipcc's AddressSanitizer runtime is not installed")
    return found[-1]


@pytest.fixture(scope="module")
def library_san():
    from latent_mixture_experts_bf16_amd import build as hip_build

    # kept beside the ordinary objects, one build per source state
    folder = os.path.join(hip_build.OBJ, "host-asan-" + _sources_digest())
    lib = os.path.join(folder, "libmoe_latent_host_asan.so")
    if not os.path.exists(lib):
        extra = []
        for f in HOST_SAN:
            extra += ["-Xarch_host", f]
        hip_build.build(extra, lib=lib, obj=folder)
    assert _undefined_sanitizer_symbols(lib), "the library copy is not instrumented"
    return lib


def test_library_host_code_under_sanitizers(library_san):
    out = _run_child(["-m", "pytest", "tests/test_abi_cpu.py", "-q", "-p", "no:cacheprovider"],
                     {"LD_PRELOAD": _clang_asan_runtime(), "MOE_LATENT_LIB": library_san})
    assert " passed" in out and " failed" not in out, out[-3000:]
