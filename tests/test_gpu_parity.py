"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small cases compare every output element; the five full-size workloads (in
the launch configuration the benchmark times) compare sampled (b, head)
outputs that the oracle computes one by one. Tolerances: fp32 max relative
error 1e-5 (floor: output RMS), bf16 max error 2e-2 of the output RMS,
indexing and page-permutation results bit-exact.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

SMALL = {
    # workload id -> (shape, lengths): same head/latent structure, short ragged contexts
    2: (dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16"), [1, 33, 64, 650]),
    3: (dict(n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16"), [31, 96, 200]),
    4: (dict(n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16"), [5, 128, 129, 900, 2049]),
    5: (dict(n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="bf16"), [100, 0, 333]),
}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_and_compare(inp, pairs=None, lse=True, per_sequence=False):
    """per_sequence: each sequence's outputs against that sequence's own RMS
    (ragged batches, where a short sequence's outputs are many times larger)."""
    prob = _gpu.GpuProblem(inp)
    out, l = prob.run()
    s = inp.shape
    if pairs is None:
        pairs = [(b, i) for b in range(s.batch) for i in range(s.n_heads)]
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    gl = np.stack([l[b, i] for b, i in pairs])
    if per_sequence:
        err = 0.0
        for b in sorted({b for b, _ in pairs}):
            rows = [k for k, (bb, _) in enumerate(pairs) if bb == b]
            if int(inp.seq_lens[b]) == 0:
                assert np.all(g[rows] == 0)
                continue
            err = max(err, _gpu.check_outputs(g[rows], ref[rows], s.dtype, f"sequence {b}"))
    else:
        err = _gpu.check_outputs(g, ref, s.dtype)
    if lse:
        _gpu.check_lse(gl, rl, s.dtype)
    return prob, err


def test_workload1_full_fp32():
    """Tiny MLRA-4, fp32, contiguous cache: every output to 1e-5."""
    _say("case: workload 1 fp32")
    inp = synth.workload_inputs(1)
    _, err = _run_and_compare(inp)
    _say(f"workload 1 max rel err {err:.2e}")


@pytest.mark.parametrize("wl", [2, 3, 4, 5])
def test_small_all_outputs(wl):
    kw, lens = SMALL[wl]
    _say(f"case: small shape of workload {wl}, lengths {lens}")
    s = synth.Shape(batch=len(lens), **kw)
    inp = synth.make_inputs(s, ("list", lens), 4000 + wl)
    _, err = _run_and_compare(inp)
    _say(f"workload {wl} small: max err/rms {err:.2e}")


@pytest.mark.parametrize("wl", [2, 3, 4])
def test_full_size_sampled(wl):
    _say(f"case: full-size workload {wl}")
    inp = synth.workload_inputs(wl)
    rng = np.random.default_rng(wl)
    s = inp.shape
    pairs = [(int(rng.integers(s.batch)), int(rng.integers(s.n_heads))) for _ in range(6)]
    pairs += [(0, 0), (s.batch - 1, s.n_heads - 1)]
    _, err = _run_and_compare(inp, pairs)
    _say(f"workload {wl} full: max err/rms {err:.2e}")


def test_full_size_workload5_with_append():
    """Ragged MLRA-2 with the latent append of one token per sequence."""
    _say("case: full-size workload 5 (append + ragged decode)")
    inp = synth.workload_inputs(5)
    prob = _gpu.GpuProblem(inp)
    prob.append()
    out, l = prob.run()
    pool_after = _gpu.from_dev_bits(prob.pool)
    c_gpu = _gpu.from_dev_bits(prob.c_out)
    # oracle append on the host copy, then sampled decode on the appended pool
    pool_ref = inp.pool.copy()
    c_ref = oracle.append(inp, pool_ref)
    ulp = np.abs(c_gpu.astype(np.int32) - c_ref.astype(np.int32))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99
    s = inp.shape
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // s.page_size], pos % s.page_size
        assert np.array_equal(pool_after[pg, off, :s.d_c], c_gpu[b])
        assert np.array_equal(pool_after[pg, off, s.d_c:], inp.kr_new[b])
    inp.pool = pool_after  # decode parity on the GPU's own appended cache
    rng = np.random.default_rng(5)
    short = np.argsort(inp.seq_lens)[:4]
    pairs = [(int(b), int(rng.integers(s.n_heads))) for b in short] + [(int(short[0]), 0)]
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    err = _gpu.check_outputs(g, ref, "bf16")
    _gpu.check_lse(np.stack([l[b, i] for b, i in pairs]), rl, "bf16")
    _say(f"workload 5 full: max err/rms {err:.2e}")


APPEND_SHAPES = [
    dict(n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=32, dtype="bf16", d_model=256),
    dict(n_heads=8, d_h=32, d_c=128, n_blocks=2, d_r=32, dtype="f32", d_model=256),
    # x staged in LDS in several chunks, partial last chunk
    dict(n_heads=8, d_h=32, d_c=512, n_blocks=2, d_r=64, dtype="bf16", d_model=5000),
    # fp32 latent whose last 8-column group holds 4 columns
    dict(n_heads=8, d_h=32, d_c=132, n_blocks=1, d_r=16, dtype="f32", d_model=4100),
]


@pytest.mark.parametrize("kw", APPEND_SHAPES)
def test_append_exact_and_canary(kw):
    """Append writes exactly the target rows; every other pool byte is unchanged."""
    _say(f"case: append exactness {kw}")
    dtype = kw["dtype"]
    if True:
        s = synth.Shape(batch=5, **kw)
        inp = synth.make_inputs(s, ("list_append", [0, 63, 64, 127, 500]), 77)
        prob = _gpu.GpuProblem(inp)
        before = _gpu.from_dev_bits(prob.pool).copy()
        prob.append()
        after = _gpu.from_dev_bits(prob.pool)
        c_gpu = _gpu.from_dev_bits(prob.c_out)
        pool_ref = inp.pool.copy()
        c_ref = oracle.append(inp, pool_ref)
        if dtype == "bf16":
            d = np.abs(c_gpu.astype(np.int32) - c_ref.astype(np.int32))
            assert d.max() <= 1
        else:
            err = np.abs(c_gpu.astype(np.float64) - c_ref) / np.maximum(np.abs(c_ref), _gpu.rms(c_ref))
            assert err.max() <= 1e-5, err.max()
        changed = np.zeros(before.shape[:2], dtype=bool)
        for b in range(s.batch):
            pos = int(inp.positions[b])
            pg, off = inp.page_table[b, pos // 64], pos % 64
            changed[pg, off] = True
            assert np.array_equal(after[pg, off, :s.d_c], c_gpu[b])
            assert np.array_equal(after[pg, off, s.d_c:], inp.kr_new[b])
        bv = before.view(np.uint16 if dtype == "bf16" else np.uint32)
        av = after.view(bv.dtype)
        assert np.array_equal(bv[~changed], av[~changed])


def test_page_permutation_bit_exact():
    """Same logical tokens under a permuted and an identity page layout give
    bit-identical outputs."""
    _say("case: page permutation")
    s = synth.Shape(batch=3, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16")
    inp = synth.make_inputs(s, ("list", [300, 77, 1000]), 91)
    prob = _gpu.GpuProblem(inp)
    out1, l1 = prob.run()
    mp = inp.max_pages_per_seq
    pool2 = np.empty((3 * mp, 64, s.row), dtype=np.uint16)
    for b in range(3):
        for p in range(mp):
            pool2[b * mp + p] = inp.pool[inp.page_table[b, p]]
    ident = synth.Inputs(**{**inp.__dict__, "page_table": None})
    ident.pool = pool2
    out2, l2 = _gpu.GpuProblem(ident).run()
    assert np.array_equal(out1, out2) and np.array_equal(l1, l2)


def test_repeat_is_deterministic():
    _say("case: determinism")
    s = synth.Shape(batch=2, n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="bf16")
    inp = synth.make_inputs(s, ("list", [3000, 17]), 92)
    prob = _gpu.GpuProblem(inp)
    o1, l1 = prob.run()
    o2, l2 = prob.run()
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("k,n_blocks,n_heads,d_c", [(2, 4, 64, 512), (4, 4, 64, 512), (1, 4, 24, 512),
                                                     (4, 4, 24, 512), (2, 4, 24, 512)])
def test_blocks_per_head_and_head_counts(k, n_blocks, n_heads, d_c):
    """Heads attending several blocks (separate softmaxes, outputs summed times
    1/sqrt(k)) and the 24-head model shape (partial 16-head tiles)."""
    _say(f"case: k={k} b={n_blocks} h={n_heads}")
    s = synth.Shape(batch=2, n_heads=n_heads, d_h=128, d_c=d_c, n_blocks=n_blocks, d_r=64, dtype="bf16",
                    blocks_per_head=k)
    inp = synth.make_inputs(s, ("list", [257, 40]), 93 + k)
    _run_and_compare(inp)


@pytest.mark.parametrize("dtype,d_c,n_blocks,d_r,d_h", [("bf16", 256, 4, 32, 64), ("f32", 512, 4, 64, 128),
                                                        ("bf16", 64, 1, 64, 256)])
def test_generic_path(dtype, d_c, n_blocks, d_r, d_h):
    """Shapes without a tuned MFMA kernel run on the generic kernel."""
    _say(f"case: generic {dtype} d_c={d_c} b={n_blocks}")
    s = synth.Shape(batch=2, n_heads=8, d_h=d_h, d_c=d_c, n_blocks=n_blocks, d_r=d_r, dtype=dtype)
    inp = synth.make_inputs(s, ("list", [130, 3]), 95)
    _run_and_compare(inp)


def test_page_sizes():
    _say("case: page sizes")
    for ps, lens in ((16, [40, 17]), (128, [300, 129]), (256, [513, 5])):
        s = synth.Shape(batch=2, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16", page_size=ps)
        inp = synth.make_inputs(s, ("list", lens), 96)
        _run_and_compare(inp)
        s4 = synth.Shape(batch=2, n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16", page_size=ps)
        _run_and_compare(synth.make_inputs(s4, ("list", lens), 97))


def test_bad_page_id_is_flagged_not_dereferenced():
    _say("case: bad page id")
    s = synth.Shape(batch=2, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16")
    inp = synth.make_inputs(s, ("list", [100, 70]), 98)
    inp.page_table = inp.page_table.copy()
    inp.page_table[1, 1] = 10 ** 6
    prob = _gpu.GpuProblem(inp)
    out, _ = prob.run()
    import compressed_kv_cache_mlra_amd as mlra
    assert mlra.read_flags(prob.ws) & mlra.FLAG_BAD_PAGE
    # the sequence with valid pages is unaffected
    ref, _ = oracle.decode_unabsorbed(inp, [(0, i) for i in range(64)])
    _gpu.check_outputs(out[0], ref, "bf16")
    # a clean step clears the flag
    inp2 = synth.make_inputs(s, ("list", [100, 70]), 98)
    prob2 = _gpu.GpuProblem(inp2)
    prob2.run()
    assert mlra.read_flags(prob2.ws) == 0


def test_side_stream():
    _say("case: side stream")
    t = _gpu.torch()
    s = synth.Shape(batch=2, n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16")
    inp = synth.make_inputs(s, ("list", [700, 64]), 99)
    prob = _gpu.GpuProblem(inp)
    st = t.cuda.Stream()
    with t.cuda.stream(st):
        prob.step(st)
    st.synchronize()
    out = prob.out.cpu().numpy().astype(np.float64)
    ref, _ = oracle.decode_unabsorbed(inp)
    _gpu.check_outputs(out.reshape(-1, 128), ref, "bf16")


def test_graph_replay_matches_eager():
    """A decode step (absorb, attend, combine) captured in a HIP graph and
    replayed several times, with eager work and synchronisations between the
    replays, gives the eager result bit for bit every time (no memset nodes:
    the plan and partials are written by kernels)."""
    _say("case: graph replay, small MLRA-4 shape")
    t = _gpu.torch()
    kw, lens = SMALL[2]
    s = synth.Shape(batch=len(lens), **kw)
    inp = synth.make_inputs(s, ("list", lens), 4101)
    prob = _gpu.GpuProblem(inp)
    eager, eager_l = prob.run()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        prob.step(t.cuda.current_stream())
    for rep in range(3):
        prob.out.zero_()
        prob.lse.zero_()
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(prob.out.cpu().numpy().astype(np.float64), eager), rep
        assert np.array_equal(prob.lse.cpu().numpy().astype(np.float64), eager_l), rep
        # eager work between replays
        junk = t.randn(1 << 20, device="cuda")
        junk.mul_(2.0).sum().item()
        prob.step()
        t.cuda.synchronize()



@pytest.mark.parametrize("wl", [9, 10, 11, 12])
def test_reading_b_and_h24_full_size_sampled(wl):
    """Reading B (k = 2, 4) and the 24-head width at full size (B = 32, 8192
    tokens, the launches bench.py times): sampled (sequence, head) pairs,
    including the last head, against the oracle; outputs and every block's lse."""
    _say(f"case: full-size workload {wl}")
    inp = synth.workload_inputs(wl)
    s = inp.shape
    rng = np.random.default_rng(wl)
    pairs = [(int(rng.integers(s.batch)), int(rng.integers(s.n_heads))) for _ in range(6)]
    pairs += [(0, 0), (s.batch - 1, s.n_heads - 1)]
    _, err = _run_and_compare(inp, pairs)
    _say(f"workload {wl} full: max err/rms {err:.2e}")


# ------------------------------------------------------------------ FP8 cache

FP8_SHAPES = {
    # same head/latent structure as the bf16 workloads, E4M3FN latent codes
    "mlra4": (dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8", cache_scale=0.5),
              [1, 33, 64, 650]),
    "mla": (dict(n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="fp8", cache_scale=0.25), [31, 96]),
    "tp_share": (dict(n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="fp8", cache_scale=1.0),
                 [5, 129, 900, 2049]),
    "mlra2": (dict(n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="fp8", cache_scale=1.25),
              [100, 0, 333]),
}


@pytest.mark.parametrize("name", list(FP8_SHAPES))
def test_fp8_small_all_outputs(name):
    """FP8 caches against the oracle on the same codes (every output and lse;
    NaN canaries in unused rows)."""
    kw, lens = FP8_SHAPES[name]
    _say(f"case: fp8 {name}, lengths {lens}")
    s = synth.Shape(batch=len(lens), **kw)
    inp = synth.make_inputs(s, ("list", lens), 4200 + len(name))
    _, err = _run_and_compare(inp)
    _say(f"fp8 {name}: max err/rms {err:.2e}")


def test_fp8_full_size_sampled():
    _say("case: full-size fp8 workload (MLRA-4 shape, B=32, 8K)")
    inp = synth.workload_inputs(6)
    rng = np.random.default_rng(6)
    s = inp.shape
    pairs = [(int(rng.integers(s.batch)), int(rng.integers(s.n_heads))) for _ in range(6)]
    pairs += [(0, 0), (s.batch - 1, s.n_heads - 1)]
    _, err = _run_and_compare(inp, pairs)
    _say(f"fp8 full: max err/rms {err:.2e}")


def test_fp8_append_encodes_kernel_latent():
    """FP8 append: the fp32 latent (c_out) matches the oracle's to the fp32 bar,
    every code is bit-identical to the oracle's encoding of that same fp32
    latent times the reciprocal scale, the RoPE key lands as bf16 and no
    other byte changes."""
    _say("case: fp8 append")
    s = synth.Shape(batch=5, n_heads=8, d_h=32, d_c=512, n_blocks=4, d_r=64, dtype="fp8",
                    cache_scale=0.125, d_model=1000)
    inp = synth.make_inputs(s, ("list_append", [0, 63, 64, 127, 500]), 78)
    prob = _gpu.GpuProblem(inp)
    before = prob.pool.cpu().numpy().copy()
    prob.append()
    after = prob.pool.cpu().numpy()
    c_gpu = prob.c_out.cpu().numpy()
    pool_ref = inp.pool.copy()
    c_ref = oracle.append(inp, pool_ref)
    err = np.abs(c_gpu.astype(np.float64) - c_ref) / np.maximum(np.abs(c_ref), _gpu.rms(c_ref))
    assert err.max() <= 1e-5, err.max()
    codes_want = oracle.e4m3_encode_array(c_gpu * np.float32(1.0 / 0.125))
    changed = np.zeros(before.shape[:2], dtype=bool)
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // 64], pos % 64
        changed[pg, off] = True
        assert np.array_equal(after[pg, off, :s.d_c], codes_want[b])
        assert np.array_equal(after[pg, off, s.d_c:].view(np.uint16), inp.kr_new[b])
    assert np.array_equal(before[~changed], after[~changed])


# ------------------------------------ FP8 cache, one scale per token and block

@pytest.mark.parametrize("name", list(FP8_SHAPES))
def test_fp8b_small_all_outputs(name):
    """Block-scaled FP8 caches (scales 2^u, u in [-3, 1), per token and block;
    NaN codes, keys and scales in unused rows) against the oracle on every
    output and lse, for each of the four kernel shapes. Sequence by sequence:
    p_t s_t is rounded to bf16 even for a one-token sequence (a power-of-two
    cache scale made that exact), and such a sequence's outputs are many times
    the batch RMS."""
    kw, lens = FP8_SHAPES[name]
    kw = dict(kw, dtype="fp8b")
    kw.pop("cache_scale")
    _say(f"case: fp8b {name}, lengths {lens}")
    s = synth.Shape(batch=len(lens), **kw)
    inp = synth.make_inputs(s, ("list", lens), 4300 + len(name))
    _, err = _run_and_compare(inp, per_sequence=True)
    _say(f"fp8b {name}: max err/rms {err:.2e}")


def test_fp8b_full_size_sampled():
    _say("case: full-size fp8b workload (MLRA-4 shape, B=32, 8K)")
    inp = synth.workload_inputs(8)
    rng = np.random.default_rng(8)
    s = inp.shape
    pairs = [(int(rng.integers(s.batch)), int(rng.integers(s.n_heads))) for _ in range(6)]
    pairs += [(0, 0), (s.batch - 1, s.n_heads - 1)]
    _, err = _run_and_compare(inp, pairs)
    _say(f"fp8b full: max err/rms {err:.2e}")


def test_fp8b_append_encodes_each_block():
    """Block-scaled append: c_out within the fp32 bar of the oracle's latent;
    every block's codes and scale bit-identical to the oracle's block encoding
    of the kernel's own fp32 latent; RoPE key, zero pad, no other byte changed.
    One token's latent is all zero in one block (scale 1, zero codes)."""
    _say("case: fp8b append")
    s = synth.Shape(batch=5, n_heads=8, d_h=32, d_c=512, n_blocks=4, d_r=64, dtype="fp8b", d_model=1000)
    inp = synth.make_inputs(s, ("list_append", [0, 63, 64, 127, 500]), 79)
    inp.w_dkv[:, 128:256] = 0  # block 1 of every token is exactly zero
    prob = _gpu.GpuProblem(inp)
    before = prob.pool.cpu().numpy().copy()
    prob.append()
    after = prob.pool.cpu().numpy()
    c_gpu = prob.c_out.cpu().numpy()
    c_ref = oracle.append(inp, inp.pool.copy())
    err = np.abs(c_gpu.astype(np.float64) - c_ref) / np.maximum(np.abs(c_ref), _gpu.rms(c_ref))
    assert err.max() <= 1e-5, err.max()
    o = s.d_c + 2 * s.d_r
    changed = np.zeros(before.shape[:2], dtype=bool)
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // 64], pos % 64
        changed[pg, off] = True
        row = after[pg, off]
        for j in range(s.n_blocks):
            codes, sc = oracle.fp8_block_encode(c_gpu[b, j * s.w:(j + 1) * s.w])
            assert np.array_equal(row[j * s.w:(j + 1) * s.w], codes), (b, j)
            assert row[o + 4 * j:o + 4 * j + 4].view(np.float32)[0] == sc, (b, j)
        assert row[o + 4:o + 8].view(np.float32)[0] == 1.0 and np.all(row[s.w:2 * s.w] & 0x7F == 0)
        assert np.all(row[o + 4 * s.n_blocks:] == 0)
        assert np.array_equal(row[s.d_c:o].view(np.uint16), inp.kr_new[b])
    assert np.array_equal(before[~changed], after[~changed])


# The tuned kernel of each configured shape (step order, two-tile prologue and
# column splits differ between them), on inputs that stress the unit plan:
# many short and empty sequences, so work units span several sequences (the
# prologue's page-id gather falls back beyond two), and pages smaller than a
# tile.
VARIANT_SHAPES = {
    "mlra4": dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16"),
    "mla": dict(n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16"),
    "tp-share": dict(n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16"),
    "mlra2": dict(n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="bf16"),
    "mlra4-fp8": dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8", cache_scale=0.5),
    "mlra4-fp8b": dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8b"),
}


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("name", list(VARIANT_SHAPES))
def test_variants_many_short_sequences(name, page_size):
    """Forty sequences of 0..300 tokens on every tuned kernel variant: many
    tiles that start or end mid-page, empty and one-token sequences.

    Outputs are compared sequence by sequence against that sequence's own RMS:
    a short sequence averages few latent rows, so its outputs are several times
    larger than a long one's and a batch-wide RMS would judge them on the wrong
    scale (a numpy emulation of only the kernel's bf16 roundings of q~ and P
    reaches 2.55e-2 of the batch RMS on this input at page size 64, and 1.3e-2
    of the sequence RMS)."""
    _say(f"case: variant {name}, page size {page_size}")
    rng = np.random.default_rng(500 + page_size)
    lens = [int(v) for v in rng.integers(0, 300, 40)]
    lens[3] = 0
    lens[17] = 1
    lens[30] = 0
    s = synth.Shape(batch=len(lens), page_size=page_size, **VARIANT_SHAPES[name])
    inp = synth.make_inputs(s, ("list", lens), 600 + len(name))
    heads = sorted({0, s.n_heads // 4 + 1, s.n_heads // 2 + 6, s.n_heads - 1})
    pairs = [(b, i) for b in range(s.batch) for i in heads]
    prob = _gpu.GpuProblem(inp)
    out, l = prob.run()
    ref, rl = oracle.decode_unabsorbed(inp, pairs)
    g = np.stack([out[b, i] for b, i in pairs])
    _gpu.check_lse(np.stack([l[b, i] for b, i in pairs]), rl, s.dtype)
    worst = 0.0
    for b in range(s.batch):
        rows = [k for k, (bb, _) in enumerate(pairs) if bb == b]
        if lens[b] == 0:
            assert np.all(g[rows] == 0), f"sequence {b} is empty but has non-zero outputs"
            continue
        worst = max(worst, _gpu.check_outputs(g[rows], ref[rows], s.dtype, f"sequence {b} (n={lens[b]})"))
    _say(f"  max err / sequence rms {worst:.2e}")
