"""Seeded random sweep over the tuned attention kernels: each case draws a
kernel shape (bf16 and FP8 caches, readings A and B, TP shares), a page size,
a batch of 1-4 sequences and a ragged length mix (empty and one-token
sequences included), and compares every output and lse with the oracle at the
same bars as the other parity tests."""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

_MLRA4 = dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64)
SHAPES = [
    ("mlra4", dict(_MLRA4, dtype="bf16")),
    ("mla", dict(_MLRA4, n_blocks=1, dtype="bf16")),
    ("tp-share", dict(n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16")),
    ("mlra2", dict(_MLRA4, n_blocks=2, dtype="bf16")),
    ("mlra2-tp2", dict(n_heads=32, d_h=128, d_c=256, n_blocks=1, d_r=64, dtype="bf16")),
    ("mla-tp-share", dict(n_heads=16, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16")),
    ("k2", dict(_MLRA4, dtype="bf16", blocks_per_head=2)),
    ("k4", dict(_MLRA4, dtype="bf16", blocks_per_head=4)),
    ("h24", dict(_MLRA4, n_heads=24, dtype="bf16")),
    ("mlra4-fp8", dict(_MLRA4, dtype="fp8", cache_scale=0.75)),
    ("mlra4-fp8b", dict(_MLRA4, dtype="fp8b")),
    ("k2-fp8", dict(_MLRA4, dtype="fp8", cache_scale=0.5, blocks_per_head=2)),
    ("mla-fp8", dict(_MLRA4, n_blocks=1, dtype="fp8", cache_scale=0.25)),
    ("tp2-fp8b", dict(n_heads=32, d_h=128, d_c=256, n_blocks=1, d_r=64, dtype="fp8b")),
]
N_CASES = 24


def _case(i):
    rng = np.random.default_rng(7000 + i)
    name, kw = SHAPES[i % len(SHAPES)]
    page = int(rng.choice([16, 32, 64, 128, 256]))
    batch = int(rng.integers(1, 5))
    lens = []
    for _ in range(batch):
        r = rng.random()
        lens.append(0 if r < 0.12 else 1 if r < 0.2 else int(rng.integers(2, 700)))
    return name, kw, page, lens, 7000 + i


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    name, kw, page, lens, seed = _case(i)
    print(f"case {i}: {name} page {page} lengths {lens} seed {seed}", flush=True)
    sys.stdout.flush()
    s = synth.Shape(batch=len(lens), page_size=page, **kw)
    inp = synth.make_inputs(s, ("list", lens), seed)
    prob = _gpu.GpuProblem(inp)
    out, l = prob.run()
    pairs = [(b, h) for b in range(s.batch) for h in range(s.n_heads)]
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, h] for b, h in pairs])
    for k, (b, _) in enumerate(pairs):
        if int(inp.seq_lens[b]) <= 0:
            assert np.all(g[k] == 0)
    if np.any(inp.seq_lens > 0):
        _gpu.check_outputs(g, ref, s.dtype)
    _gpu.check_lse(np.stack([l[b, h] for b, h in pairs]), rl, s.dtype)
