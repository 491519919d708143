"""The one-call decode step (mlra_decode_step) on the GPU: it must reproduce
the three separate calls (absorb_query, attend, combine) bit for bit and match
the oracle within the usual bars, on every kernel family."""
import numpy as np
import pytest

import oracle
import synth

from tests import _gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


MLRA4 = dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64)
STEP_SHAPES = {
    "mlra4-bf16": dict(MLRA4, dtype="bf16"),
    "mlra4-fp8": dict(MLRA4, dtype="fp8", cache_scale=0.5),
    "mlra4-fp8b": dict(MLRA4, dtype="fp8b"),                         # per-token block scales
    "mla-bf16": dict(MLRA4, n_blocks=1, dtype="bf16"),
    "mlra4-k2-bf16": dict(MLRA4, dtype="bf16", blocks_per_head=2),  # two blocks per head
    "mlra4-f32": dict(MLRA4, dtype="f32"),                          # generic kernels
}
# sequences 4..7 are all empty (a combine workgroup with no partials to merge)
LENS = [300, 45, 0, 5, 0, 0, 0, 0, 1000, 64, 1, 129]


def _bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


@pytest.mark.parametrize("name", list(STEP_SHAPES))
def test_step_equals_separate_calls_and_oracle(name):
    _say(f"case: decode step {name}, lengths {LENS}")
    s = synth.Shape(batch=len(LENS), **STEP_SHAPES[name])
    inp = synth.make_inputs(s, ("list", LENS), 700 + len(name))
    prob = _gpu.GpuProblem(inp)
    out_sep, lse_sep = prob.run()
    prob.out.fill_(float("nan"))
    prob.lse.fill_(float("nan"))
    out, lse = prob.run(one_call=True)
    import compressed_kv_cache_mlra_amd as mlra
    assert mlra.read_flags(prob.ws) == 0
    assert _bits_equal(out, out_sep), "decode_step differs from decode + combine"
    assert _bits_equal(lse, lse_sep)
    pairs = [(b, i) for b in range(s.batch) for i in (0, 21, s.n_heads - 1)]
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    _gpu.check_lse(np.stack([lse[b, i] for b, i in pairs]), rl, s.dtype)
    for k, (b, _) in enumerate(pairs):
        if LENS[b] == 0:
            assert np.all(g[k] == 0)
    worst = _gpu.check_outputs(g, ref, s.dtype)
    _say(f"  max err / rms {worst:.2e}")


def test_repeated_steps_with_changing_lengths():
    """Three steps on one workspace, the lengths changing in between: each step
    plans afresh, so no step reads a previous step's partials."""
    _say("case: repeated steps")
    s = synth.Shape(batch=9, dtype="bf16", **MLRA4)
    t = _gpu.torch()
    inp = synth.make_inputs(s, ("list", [700, 30, 0, 255, 1, 64, 900, 2, 511]), 750)
    prob = _gpu.GpuProblem(inp)
    # each length at most the drawn one (rows past it hold NaN canaries)
    for lens in ([700, 30, 0, 255, 1, 64, 900, 2, 511], [5, 6, 0, 8, 0, 0, 0, 0, 3], [699, 1, 0, 200, 1, 60, 17, 2, 511]):
        prob.seq_lens.copy_(t.tensor(lens, dtype=t.int32))
        out_sep, lse_sep = prob.run()
        out, lse = prob.run(one_call=True)
        assert np.all(np.isfinite(out)), lens
        assert _bits_equal(out, out_sep) and _bits_equal(lse, lse_sep), lens
    import compressed_kv_cache_mlra_amd as mlra
    assert mlra.read_flags(prob.ws) == 0


def test_full_size_mlra4_step():
    """MLRA-4, B = 32, 8192 tokens each, 64-token pages (the benchmark's
    launch): the step equals the separate calls everywhere and matches
    the oracle on sampled (sequence, head) pairs."""
    _say("case: full-size MLRA-4 decode step")
    inp = synth.workload_inputs(2)
    prob = _gpu.GpuProblem(inp)
    out_sep, lse_sep = prob.run()
    out, lse = prob.run(one_call=True)
    assert _bits_equal(out, out_sep) and _bits_equal(lse, lse_sep)
    s = inp.shape
    rng = np.random.default_rng(2)
    pairs = [(int(rng.integers(s.batch)), int(rng.integers(s.n_heads))) for _ in range(6)]
    pairs += [(s.batch // 2, i) for i in range(s.n_heads)]
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    err = _gpu.check_outputs(np.stack([out[b, i] for b, i in pairs]), ref, "bf16")
    _gpu.check_lse(np.stack([lse[b, i] for b, i in pairs]), rl, "bf16")
    _say(f"  max err/rms {err:.2e}")
