"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only,
no GPU code is built with them):

* the descriptor validation of libmlra (validate.cpp), built with g++ beside a
  driver that sets every descriptor field, and every pair of integer fields,
  to boundary and extreme values (tests/sanitize/validate_fuzz.cpp);
* the C oracle (oracle.c), built as a shared library with both sanitizers and
  loaded by a child Python process with the ASan runtime preloaded, run on
  small inputs of every cache type and page layout and every entry point.

Any invalid access or undefined behaviour aborts the child
(-fno-sanitize-recover=all), which fails the test."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_kv_cache_mlra_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_fuzz")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "sanitize", "validate_fuzz.cpp"),
                           os.path.join(CSRC, "validate.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "inconsistent 0" in r.stdout, r.stdout


_ORACLE_RUN = textwrap.dedent('''
    import numpy as np
    import oracle, synth
    oracle.lib()
    assert oracle._LIB_PATH.endswith("liboracle_san.so"), oracle._LIB_PATH
    def run(shape, lens, seed, **kw):
        inp = synth.make_inputs(shape, lens, seed, **kw)
        oracle.decode_unabsorbed(inp)
        oracle.decode_absorbed(inp)
        if inp.x is not None:
            oracle.append(inp, inp.pool.copy())
            oracle.append(inp, inp.pool.copy(), c_out=False)
        return inp
    S = synth.Shape
    run(S(batch=1, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype="f32", paged=False), ("fixed", 70), 1)
    run(S(batch=3, n_heads=8, d_h=32, d_c=128, n_blocks=4, d_r=32, dtype="bf16"), ("list", [5, 0, 130]), 2)
    run(S(batch=2, n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=32, dtype="bf16", blocks_per_head=2,
          page_size=16), ("list", [40, 17]), 3)
    run(S(batch=2, n_heads=4, d_h=32, d_c=64, n_blocks=1, d_r=0, dtype="bf16"), ("list", [33, 1]), 4)
    run(S(batch=3, n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=32, dtype="fp8", cache_scale=0.5),
        ("list", [100, 0, 7]), 5, fp8_codes="full")
    run(S(batch=3, n_heads=8, d_h=32, d_c=128, n_blocks=4, d_r=32, dtype="fp8b"), ("list", [64, 3, 65]), 6,
        fp8_codes="full", scale_exp=(-8.0, 8.0))
    for dt, kw in (("bf16", {}), ("f32", {}), ("fp8", dict(cache_scale=0.25)), ("fp8b", {})):
        inp = run(S(batch=3, n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=32, dtype=dt, d_model=96, d_cq=48, **kw),
                  ("list_append", [0, 63, 64]), 7)
        oracle.rope_key(inp)
        oracle.project_query(inp)
    for c in range(256):
        oracle.e4m3_decode(c)
    oracle.e4m3_encode_array(np.array([0.0, -0.0, 1e-9, 0.001953125, 447.9, 448.0, 1e6, np.inf, -np.inf, np.nan],
                                      dtype=np.float32))
    oracle.fp8_block_encode(np.linspace(-3, 3, 64).astype(np.float32))
    oracle.fp8_block_encode(np.zeros(16, dtype=np.float32))
    oracle.rope(np.arange(8.0), 5, 100.0)
    for m in oracle.METHODS:
        oracle.cache_elems_per_token(m, h=64, d_h=128, g=8, beta_kv=2, d_c=512, d_r=64)
        for tp in (1, 2, 4, 8):
            oracle.cache_elems_per_device(m, h=64, d_h=128, g=8, beta_kv=2, d_c=512, d_r=64, n_blocks=4, tp=tp)
    oracle.decode_flops_bytes(8192, 16, 128, 64)
    print("oracle under sanitizers: ok", flush=True)
''')


def test_oracle_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc has no ASan runtime")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-fopenmp", "-fPIC", "-shared", "-o", lib,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ, MLRA_ORACLE_LIB=lib, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", _ORACLE_RUN], env=env, capture_output=True, text=True, timeout=600,
                       cwd=ROOT)
    assert r.returncode == 0 and "oracle under sanitizers: ok" in r.stdout, (r.stdout[-3000:], r.stderr[-6000:])
