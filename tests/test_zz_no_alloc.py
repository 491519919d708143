"""The allocation-free decode step (mlra_decode_step_noalloc, whose workspace
is the library's static device scratch) against mlra_decode_step with an
allocated workspace, through the C ABI: two calls in a row on the same
scratch, the second with a smaller input (fewer sequences, shorter and empty
ones), so nothing the first call left in the scratch may leak into the second.
Both run the same kernels on the same plan, so the outputs must agree bit for
bit (stricter than the 2e-2 parity bar); the second call is also checked
against the oracle."""
import numpy as np
import pytest

import compressed_kv_cache_mlra_amd as mlra
import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

_MLRA4 = dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16")


def _noalloc(prob):
    t = _gpu.torch()
    out = t.full_like(prob.out, float("nan"))
    lse = t.full_like(prob.lse, float("nan"))
    mlra.decode_step_noalloc(prob.desc, prob.pool, prob.page_table, prob.seq_lens, prob.max_seq_len, prob.q_c,
                             prob.q_r, prob.w_uk, prob.w_uv, out, lse)
    t.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_noalloc_step_matches_decode_step_twice():
    big = synth.make_inputs(synth.Shape(batch=12, **_MLRA4),
                            ("list", [4000, 3000, 2500, 100, 1, 0, 5000, 777, 64, 65, 2048, 1500]), 1201)
    small = synth.make_inputs(synth.Shape(batch=3, **_MLRA4), ("list", [100, 0, 37]), 1202)
    for step, inp in enumerate((big, small)):
        print(f"case: noalloc call {step}, lengths {list(inp.seq_lens)}", flush=True)
        prob = _gpu.GpuProblem(inp)
        need = mlra.workspace_bytes(prob.desc, prob.max_seq_len)
        assert need <= mlra.NOALLOC_SCRATCH_BYTES
        ref_out, ref_lse = prob.run(one_call=True)
        out, lse = _noalloc(prob)
        assert np.array_equal(_bits(out), _bits(ref_out)), f"call {step}: outputs differ from decode_step"
        assert np.array_equal(_bits(lse), _bits(ref_lse)), f"call {step}: lse differ from decode_step"
    # the second (smaller) call against the oracle as well
    s = small.shape
    pairs = [(b, i) for b in range(s.batch) for i in range(s.n_heads)]
    ref, _ = oracle.decode_unabsorbed(small, pairs)
    _gpu.check_outputs(np.stack([out[b, i] for b, i in pairs]), ref, "bf16")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    """A shape whose workspace exceeds MLRA_NOALLOC_SCRATCH_BYTES is refused
    with MLRA_ERR_SCRATCH before anything is enqueued."""
    t = _gpu.torch()
    s = synth.Shape(batch=4096, n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16", page_size=16)
    desc = mlra.make_desc(batch=s.batch, n_heads=s.n_heads, d_h=s.d_h, d_c=s.d_c, n_blocks=s.n_blocks, d_r=s.d_r,
                          max_pages_per_seq=1, num_pages=1, dtype="bf16", page_size=16)
    assert mlra.workspace_bytes(desc, 16) > mlra.NOALLOC_SCRATCH_BYTES
    z = lambda *shape, dt=t.bfloat16: t.zeros(shape, dtype=dt, device="cuda")
    with pytest.raises(mlra.MlraError) as e:
        mlra.decode_step_noalloc(desc, z(1, 16, s.row), None, z(s.batch, dt=t.int32), 16, z(s.batch, 64, 128),
                                 z(s.batch, 64, 64), z(64, 1, 512, 128), z(64, 1, 512, 128),
                                 z(s.batch, 64, 128, dt=t.float32))
    assert e.value.status == mlra.ERR_SCRATCH
