"""Edge cases of the decode path on the GPU: the largest batch the plan takes,
lengths outside [0, capacity], head widths that select the other absorption
kernels and the generic combine, and a cache without a RoPE key."""
import numpy as np
import pytest

import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _check_pairs(inp, out, lse, pairs):
    """Outputs against the oracle on one RMS over every compared output;
    empty sequences must give exactly 0."""
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    _gpu.check_lse(np.stack([lse[b, i] for b, i in pairs]), rl, inp.shape.dtype)
    for k, (b, _) in enumerate(pairs):
        if int(inp.seq_lens[b]) <= 0:
            assert np.all(g[k] == 0), f"sequence {b} is empty but has non-zero outputs"
    return _gpu.check_outputs(g, ref, inp.shape.dtype)


def test_largest_batch():
    """4096 sequences (the most the plan keeps in LDS) of 0..40 tokens in
    16-token pages: thousands of sequences per work unit, many units per
    sequence boundary; sampled sequences against the oracle, both through the
    separate calls and the one-call step."""
    _say("case: batch 4096")
    rng = np.random.default_rng(4096)
    lens = [int(v) for v in rng.integers(0, 41, 4096)]
    lens[0], lens[4095] = 40, 0
    s = synth.Shape(batch=4096, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16", page_size=16)
    inp = synth.make_inputs(s, ("list", lens), 4096)
    prob = _gpu.GpuProblem(inp)
    out, lse = prob.run()
    picks = [0, 1, 2, 1000, 2047, 2048, 3333, 4094, 4095] + [int(v) for v in rng.integers(0, 4096, 8)]
    pairs = [(b, i) for b in picks for i in (0, 63)]
    worst = _check_pairs(inp, out, lse, pairs)
    out2, lse2 = prob.run(one_call=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    _say(f"  max err / rms {worst:.2e}")


def test_lengths_outside_capacity_are_clamped():
    """A length above max_pages_per_seq * page_size attends the whole capacity
    and a negative one nothing (out = 0, lse = -inf), as documented."""
    _say("case: clamped lengths")
    t = _gpu.torch()
    s = synth.Shape(batch=3, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16")
    # sequence 0 fills its two pages exactly, so its capacity holds no canary rows
    inp = synth.make_inputs(s, ("list", [128, 50, 77]), 61)
    prob = _gpu.GpuProblem(inp)
    out_ref, lse_ref = prob.run()
    prob.seq_lens.copy_(t.tensor([10 ** 6, -5, 77], dtype=t.int32))
    out, lse = prob.run()
    assert np.array_equal(out[0], out_ref[0]) and np.array_equal(lse[0], lse_ref[0])
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    assert np.array_equal(out[2], out_ref[2])
    assert _gpu.mlra.read_flags(prob.ws) == 0


@pytest.mark.parametrize("d_h", [64, 256, 512])
def test_head_widths(d_h):
    """d_h other than 128: the absorption's other compile-time k-step counts
    (d_h <= 128, 256, 512) and the generic combine; every output checked."""
    _say(f"case: d_h = {d_h}")
    s = synth.Shape(batch=3, n_heads=16, d_h=d_h, d_c=512, n_blocks=4, d_r=64, dtype="bf16")
    inp = synth.make_inputs(s, ("list", [300, 1, 97]), 70 + d_h)
    prob = _gpu.GpuProblem(inp)
    out, lse = prob.run()
    pairs = [(b, i) for b in range(s.batch) for i in range(s.n_heads)]
    worst = _check_pairs(inp, out, lse, pairs)
    _say(f"  max err / rms {worst:.2e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_rope_key(dtype):
    """d_r = 0 (no decoupled RoPE key): the generic kernels."""
    _say(f"case: d_r = 0, {dtype}")
    s = synth.Shape(batch=2, n_heads=8, d_h=64, d_c=256, n_blocks=2, d_r=0, dtype=dtype)
    inp = synth.make_inputs(s, ("list", [200, 33]), 90)
    prob = _gpu.GpuProblem(inp)
    out, lse = prob.run()
    pairs = [(b, i) for b in range(s.batch) for i in range(s.n_heads)]
    _check_pairs(inp, out, lse, pairs)
