"""Parity of the steps on either side of the attention with the oracle: the
RoPE key of the new token and the query path (c^Q, q^C, RoPE'd q^R), through
the C ABI, and the whole step chained on the device: project the query,
rotate and append the new token, decode, combine.

Outputs are rounded once from an fp32 accumulation, so the bf16 bar is
elementwise: |gpu - oracle| <= 2^-8 |oracle| + 1e-3 RMS(oracle) (one bf16
rounding is at most 2^-9 relative; the RMS term covers fp32 accumulation
over d_model and d_cq terms). fp32: 1e-5 of max(|oracle|, RMS).
"""
import sys

import numpy as np
import pytest

import compressed_kv_cache_mlra_amd as mlra
import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _check(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what
    r = _gpu.rms(ref)
    if dtype == "f32":
        err = float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), r)))
        assert err <= 1e-5, f"{what}: max rel err {err:.3e}"
    else:
        excess = np.abs(gpu - ref) - (2.0 ** -8 * np.abs(ref) + 1e-3 * r)
        assert float(excess.max()) <= 0, f"{what}: bound exceeded by {float(excess.max()):.3e}"
    return float(np.max(np.abs(gpu - ref))) / r


QP_SHAPES = {
    # MFMA path: several column tiles, 11 sequences (a partial row tile)
    "bf16-mlra4": dict(batch=11, n_heads=16, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16",
                       d_model=1096, d_cq=192),
    # MFMA path: two groups of 32 sequences; d_model and d_cq end in a partial
    # 32-row k-step (2504 = 78 x 32 + 8, 1064 = 33 x 32 + 8)
    "bf16-wide": dict(batch=37, n_heads=4, d_h=64, d_c=128, n_blocks=1, d_r=32, dtype="bf16",
                      d_model=2504, d_cq=1064),
    # d_model not a multiple of 8: the fp32 VALU kernel, x staged in several chunks
    "bf16-valu": dict(batch=3, n_heads=4, d_h=64, d_c=128, n_blocks=1, d_r=32, dtype="bf16",
                      d_model=2500, d_cq=1064),
    "f32": dict(batch=9, n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=16, dtype="f32",
                d_model=300, d_cq=40),
    "fp8-cache": dict(batch=5, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8",
                      cache_scale=0.125, d_model=512, d_cq=256, rope_base=500.0),
    # one scale per token and latent block
    "fp8b-cache": dict(batch=5, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8b",
                       d_model=512, d_cq=256, rope_base=500.0),
}


def _problem(name, lens=(0, 1, 63, 64, 8191), **over):
    kw = dict(QP_SHAPES[name])
    kw.update(over)
    B = kw.pop("batch")
    lens = [lens[i % len(lens)] + 7 * i for i in range(B)]
    s = synth.Shape(batch=B, **kw)
    inp = synth.make_inputs(s, ("list_append", lens), 4300 + len(name))
    return s, inp


@pytest.mark.parametrize("name", list(QP_SHAPES))
def test_rope_key(name):
    _say(f"case: rope_key {name}")
    t = _gpu.torch()
    s, inp = _problem(name)
    prob = _gpu.GpuProblem(inp)
    desc = prob.desc
    kr = t.empty((s.batch, s.d_r), dtype=mlra._elem_dtype(desc), device="cuda")
    mlra.rope_key(desc, prob.x, _gpu.to_dev(inp.w_kr), prob.positions, kr, prob.ws)
    t.cuda.synchronize()
    got = _bits_to_f64(_gpu.from_dev_bits(kr), s.arrays_dtype)
    err = _check(got, oracle.rope_key(inp), s.arrays_dtype, "k^R")
    _say(f"  k^R max err/rms {err:.2e}")


@pytest.mark.parametrize("name", list(QP_SHAPES))
def test_project_query(name):
    _say(f"case: project_query {name}")
    t = _gpu.torch()
    s, inp = _problem(name)
    prob = _gpu.GpuProblem(inp)
    desc = prob.desc
    et = mlra._elem_dtype(desc)
    cq = t.empty((s.batch, s.d_cq), dtype=t.float32, device="cuda")
    qc = t.empty((s.batch, s.n_heads, s.d_h), dtype=et, device="cuda")
    qr = t.empty((s.batch, s.n_heads, s.d_r), dtype=et, device="cuda")
    mlra.project_query(desc, prob.x, _gpu.to_dev(inp.w_dq), _gpu.to_dev(inp.w_uq),
                       _gpu.to_dev(inp.w_qr), prob.positions, cq, qc, qr, prob.ws)
    t.cuda.synchronize()
    ref_c, ref_r = oracle.project_query(inp)
    e1 = _check(_bits_to_f64(_gpu.from_dev_bits(qc), s.arrays_dtype), ref_c, s.arrays_dtype, "q^C")
    e2 = _check(_bits_to_f64(_gpu.from_dev_bits(qr), s.arrays_dtype), ref_r, s.arrays_dtype, "q^R")
    _say(f"  q^C {e1:.2e}  q^R {e2:.2e}")


@pytest.mark.parametrize("d_model", [1096, 1100])
def test_whole_step_chained_on_device(d_model):
    """project_query -> rope_key -> append_latent -> decode -> combine with
    every intermediate left on the device, against the oracle run on the
    oracle's own q^C, q^R and k^R (rounded to bf16 as the device stores them).
    d_model = 1100 (not a multiple of 8) takes the fp32 VALU projections."""
    _say(f"case: chained step, d_model {d_model}")
    t = _gpu.torch()
    s, inp = _problem("bf16-mlra4", lens=(5, 200, 64, 1000), d_model=d_model)
    prob = _gpu.GpuProblem(inp)
    desc = prob.desc
    et = mlra._elem_dtype(desc)
    cq = t.empty((s.batch, s.d_cq), dtype=t.float32, device="cuda")
    qc = t.empty((s.batch, s.n_heads, s.d_h), dtype=et, device="cuda")
    qr = t.empty((s.batch, s.n_heads, s.d_r), dtype=et, device="cuda")
    kr = t.empty((s.batch, s.d_r), dtype=et, device="cuda")
    mlra.project_query(desc, prob.x, _gpu.to_dev(inp.w_dq), _gpu.to_dev(inp.w_uq),
                       _gpu.to_dev(inp.w_qr), prob.positions, cq, qc, qr, prob.ws)
    mlra.rope_key(desc, prob.x, _gpu.to_dev(inp.w_kr), prob.positions, kr, prob.ws)
    mlra.append_latent(desc, prob.pool, prob.page_table, prob.positions, prob.x, prob.w_dkv, kr,
                       None, prob.ws)
    mlra.decode(desc, prob.pool, prob.page_table, prob.seq_lens, prob.max_seq_len, qc, qr,
                prob.w_uk, prob.ws)
    mlra.combine(desc, prob.ws, prob.w_uv, prob.out, prob.lse)
    t.cuda.synchronize()
    out = prob.out.cpu().numpy().astype(np.float64)

    # the oracle's own chain: its q^C, q^R, k^R rounded to bf16 like the cache
    # and the queries the device keeps, its own append, then its decode
    ref_c, ref_r = oracle.project_query(inp)
    inp.q_c = synth.f32_to_bf16_bits(ref_c.astype(np.float32))
    inp.q_r = synth.f32_to_bf16_bits(ref_r.astype(np.float32))
    inp.kr_new = synth.f32_to_bf16_bits(oracle.rope_key(inp).astype(np.float32))
    pool_ref = inp.pool.copy()
    oracle.append(inp, pool_ref)
    inp.pool = pool_ref
    pairs = [(b, i) for b in range(s.batch) for i in range(s.n_heads)]
    ref, _ = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    err = _gpu.check_outputs(g, ref, "bf16")
    _say(f"  chained out max err/rms {err:.2e}")


def test_full_size_layer_workload():
    """The whole-layer workload at its full size, as the benchmark launches
    it: k^R, q^C and q^R against the oracle (every element), then the decode
    on the device's own queries for sampled (sequence, head) pairs."""
    _say("case: whole-layer workload, full size")
    t = _gpu.torch()
    inp = synth.workload_inputs(7)
    s = inp.shape
    prob = _gpu.GpuProblem(inp)
    desc = prob.desc
    et = mlra._elem_dtype(desc)
    cq = t.empty((s.batch, s.d_cq), dtype=t.float32, device="cuda")
    qc = t.empty((s.batch, s.n_heads, s.d_h), dtype=et, device="cuda")
    qr = t.empty((s.batch, s.n_heads, s.d_r), dtype=et, device="cuda")
    kr = t.empty((s.batch, s.d_r), dtype=et, device="cuda")
    mlra.project_query(desc, prob.x, _gpu.to_dev(inp.w_dq), _gpu.to_dev(inp.w_uq),
                       _gpu.to_dev(inp.w_qr), prob.positions, cq, qc, qr, prob.ws)
    mlra.rope_key(desc, prob.x, _gpu.to_dev(inp.w_kr), prob.positions, kr, prob.ws)
    mlra.append_latent(desc, prob.pool, prob.page_table, prob.positions, prob.x, prob.w_dkv, kr, None, prob.ws)
    mlra.decode(desc, prob.pool, prob.page_table, prob.seq_lens, prob.max_seq_len, qc, qr,
                prob.w_uk, prob.ws)
    mlra.combine(desc, prob.ws, prob.w_uv, prob.out, prob.lse)
    t.cuda.synchronize()
    kr_b = _gpu.from_dev_bits(kr)
    qc_b, qr_b = _gpu.from_dev_bits(qc), _gpu.from_dev_bits(qr)
    _check(_bits_to_f64(kr_b, "bf16"), oracle.rope_key(inp), "bf16", "k^R")
    ref_c, ref_r = oracle.project_query(inp)
    _check(_bits_to_f64(qc_b, "bf16"), ref_c, "bf16", "q^C")
    _check(_bits_to_f64(qr_b, "bf16"), ref_r, "bf16", "q^R")
    # decode on the device's own q^C, q^R and k^R: the oracle's append and
    # attention on exactly those inputs
    inp.q_c, inp.q_r, inp.kr_new = qc_b, qr_b, kr_b
    pool_ref = inp.pool.copy()
    oracle.append(inp, pool_ref)
    inp.pool = pool_ref
    out = prob.out.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(7)
    pairs = [(int(b), int(i)) for b, i in zip(rng.integers(0, s.batch, 24), rng.integers(0, s.n_heads, 24))]
    ref, _ = oracle.decode_unabsorbed(inp, pairs)
    err = _gpu.check_outputs(np.stack([out[b, i] for b, i in pairs]), ref, "bf16")
    _say(f"  full-size layer step: out max err/rms {err:.2e}")


@pytest.mark.parametrize("name", ["bf16-mlra4", "bf16-wide", "fp8-cache", "fp8b-cache"])
def test_project_token_fused(name):
    """mlra_project_token: the latent append, the RoPE key and the query path
    of the new token in one call. k^R, q^C and q^R against the oracle; the
    appended row's latent within one bf16 ulp of the oracle's (FP8: the codes
    of the kernel's own fp32 latent, which is within 1e-5 of the oracle's);
    the row's RoPE part equal to k^R; every other pool byte unchanged."""
    _say(f"case: project_token {name}")
    t = _gpu.torch()
    s, inp = _problem(name)
    prob = _gpu.GpuProblem(inp)
    desc = prob.desc
    et = mlra._elem_dtype(desc)
    fp8 = s.is_fp8
    cq = t.empty((s.batch, s.d_cq), dtype=t.float32, device="cuda")
    qc = t.empty((s.batch, s.n_heads, s.d_h), dtype=et, device="cuda")
    qr = t.empty((s.batch, s.n_heads, s.d_r), dtype=et, device="cuda")
    kr = t.empty((s.batch, s.d_r), dtype=et, device="cuda")
    c_out = t.empty((s.batch, s.d_c), dtype=t.float32 if fp8 else et, device="cuda")
    before = _gpu.from_dev_bits(prob.pool).copy()
    mlra.project_token(desc, prob.x, prob.positions, prob.pool, prob.page_table, prob.w_dkv,
                       _gpu.to_dev(inp.w_kr), kr, c_out, _gpu.to_dev(inp.w_dq), _gpu.to_dev(inp.w_uq),
                       _gpu.to_dev(inp.w_qr), cq, qc, qr, prob.ws)
    t.cuda.synchronize()
    after = _gpu.from_dev_bits(prob.pool)
    kr_b = _gpu.from_dev_bits(kr)
    _check(_bits_to_f64(kr_b, s.arrays_dtype), oracle.rope_key(inp), s.arrays_dtype, "k^R")
    ref_c, ref_r = oracle.project_query(inp)
    _check(_bits_to_f64(_gpu.from_dev_bits(qc), s.arrays_dtype), ref_c, s.arrays_dtype, "q^C")
    _check(_bits_to_f64(_gpu.from_dev_bits(qr), s.arrays_dtype), ref_r, s.arrays_dtype, "q^R")
    # the oracle's append with the device's k^R
    inp.kr_new = kr_b
    c_ref = oracle.append(inp, inp.pool.copy())
    c_gpu = _gpu.from_dev_bits(c_out)
    P = s.page_size
    changed = np.zeros(before.shape[:2], dtype=bool)
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // P], pos % P
        changed[pg, off] = True
        row = after[pg, off]
        if fp8:
            err = np.abs(c_gpu[b].astype(np.float64) - c_ref[b]) / max(_gpu.rms(c_ref), 1e-30)
            assert err.max() <= 1e-5, err.max()
            if s.dtype == "fp8b":
                # each block: the oracle's block encoding of the kernel's own fp32 latent
                o = s.d_c + 2 * s.d_r
                for j in range(s.n_blocks):
                    codes, sc = oracle.fp8_block_encode(c_gpu[b, j * s.w:(j + 1) * s.w])
                    assert np.array_equal(row[j * s.w:(j + 1) * s.w], codes)
                    assert row[o + 4 * j:o + 4 * j + 4].view(np.float32)[0] == sc
                assert np.all(row[o + 4 * s.n_blocks:] == 0)
                assert np.array_equal(row[s.d_c:o].view(np.uint16), kr_b[b])
            else:
                codes = oracle.e4m3_encode_array(c_gpu[b] * np.float32(1.0 / s.cache_scale))
                assert np.array_equal(row[:s.d_c], codes)
                assert np.array_equal(row[s.d_c:].view(np.uint16), kr_b[b])
        else:
            assert np.abs(c_gpu[b].astype(np.int32) - c_ref[b].astype(np.int32)).max() <= 1
            assert np.array_equal(row[:s.d_c], c_gpu[b])
            assert np.array_equal(row[s.d_c:], kr_b[b])
    assert np.array_equal(before[~changed], after[~changed])
