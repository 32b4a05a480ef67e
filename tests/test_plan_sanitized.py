"""The host-side plan and validation code (plan.cpp: descriptor checks, path
choice, tile shapes, workspace layout) built on its own with AddressSanitizer
and UndefinedBehaviorSanitizer, driven over named, edge-case and random
descriptors in a subprocess with the sanitizer runtimes preloaded.  Every call
must run clean and return what the in-tree library returns (CPU only)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLAN = os.path.join(ROOT, "sparse_mixture_experts_histogram_amd", "csrc", "plan.cpp")
LIBPY = os.path.join(ROOT, "sparse_mixture_experts_histogram_amd", "_lib.py")

DRIVER = textwrap.dedent('''
    import ctypes, importlib.util, math, random, sys
    spec = importlib.util.spec_from_file_location("moe_lib", sys.argv[2])
    m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)
    L = ctypes.CDLL(sys.argv[1])
    D = ctypes.POINTER(m.MoeDesc)
    L.moe_validate.argtypes = [D]
    L.moe_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_resolve_path.argtypes = [D]
    L.moe_grouped_rows.argtypes = [D]
    L.moe_grouped_rows.restype = ctypes.c_int64
    L.moe_status_str.restype = ctypes.c_char_p
    named = [(64, 256, 8, 2, 512, 0, 0, 0), (4096, 4096, 8, 2, 14336, 0, 0, 1),
             (16, 4096, 8, 2, 14336, 0, 0, 1), (8192, 2048, 32, 2, 1024, 0, 0, 1),
             (4096, 7168, 256, 8, 2048, 1, 2048, 1)] + \\
            [(t, 2880, 128, 4, 2880, 0, 0, 1) for t in (1, 8, 32, 128, 512)]
    edge = [(0, 64, 8, 2, 64, 0, 0, 1), (1, 64, 1, 1, 64, 0, 0, 1), (1 << 29, 64, 8, 2, 64, 0, 0, 1),
            (1 << 31, 64, 8, 1, 64, 0, 0, 1), (5, 64, 512, 32, 64, 8, 64, 1),
            (5, 64, 513, 2, 64, 0, 0, 1), (5, 64, 8, 9, 64, 0, 0, 1), (-1, 64, 8, 2, 64, 0, 0, 1),
            (5, 0, 8, 2, 64, 0, 0, 1), (5, 100, 8, 2, 64, 0, 0, 1), (5, 100, 8, 2, 64, 0, 0, 0),
            (5, 64, 8, 2, 64, 1, 0, 1), (5, 64, 8, 2, 64, 9, 64, 1), (70000, 65536, 8, 2, 65536, 0, 0, 1)]
    rng = random.Random(5)
    rand = []
    for _ in range(3000):
        q = rng.choice([1, 4, 64])
        rand.append((rng.choice([0, 1, 3, 16, 17, 300, 4096, 100000, 1 << 26]),
                     q * rng.randint(0, 200), rng.randint(-1, 600), rng.randint(-1, 40),
                     q * rng.randint(0, 300), rng.randint(-1, 9), q * rng.randint(0, 60),
                     rng.choice([0, 1, 1, 2])))
    for (T, d, E, k, f, ns, fs, dt) in named + edge + rand:
        for path, sc, wt, fmt, cap in ((0, 0, 0, 0, 0.0), (1, 1, 1, 0, 1.25), (2, 0, 0, 1, 0.0),
                                       (0, 0, 1, 2, float("nan")), (0, 2, 0, 0, -1.0)):
            desc = m.MoeDesc(T=T, d=d, E=E, k=k, ffn=f, n_shared=ns, ffn_shared=fs, dtype=dt,
                             y_dtype=0, path=path, scoring=sc, weighting=wt,
                             expert_format=fmt, flags=0, capacity_factor=cap)
            n = ctypes.c_size_t(0)
            st = L.moe_workspace_size(ctypes.byref(desc), ctypes.byref(n))
            print(L.moe_validate(ctypes.byref(desc)), st, n.value if st == 0 else -1,
                  L.moe_resolve_path(ctypes.byref(desc)), L.moe_grouped_rows(ctypes.byref(desc)))
    for s in range(-6, 2):
        L.moe_status_str(s)
''')


def _run(lib, env=None):
    return subprocess.run([sys.executable, "-c", DRIVER, lib, LIBPY], capture_output=True,
                          text=True, env=env, timeout=600)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_under_address_and_ub_sanitizers(tmp_path):
    lib = str(tmp_path / "libmoe_plan_sanitized.so")
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-shared",
                        "-fPIC", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-I", os.path.join(ROOT, "include"), PLAN, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    runtimes = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                           text=True).stdout.strip()
        assert os.path.isabs(p), name
        runtimes.append(p)
    env = dict(os.environ, LD_PRELOAD=":".join(runtimes),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    san = _run(lib, env)
    assert san.returncode == 0, san.stderr[-4000:]
    assert "runtime error" not in san.stderr and "AddressSanitizer" not in san.stderr, \
        san.stderr[-4000:]
    # the same answers as the library the tests and the benchmark load
    built = os.path.join(ROOT, "sparse_mixture_experts_histogram_amd", "libmoe_mi355x.so")
    if not os.path.exists(built):
        pytest.skip("libmoe_mi355x.so is not built")
    ref = _run(built)
    assert ref.returncode == 0, ref.stderr[-2000:]
    assert san.stdout == ref.stdout
    assert len(san.stdout.splitlines()) > 10000
