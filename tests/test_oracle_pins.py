"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/), closed forms, textbook attention over explicitly
materialised keys and values (numpy), brute force in pure Python, and
structural properties (block independence, page-permutation invariance).
"""
import ast
import math
import operator
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kv_file(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split()
        out[k] = v
    return out


def _f(a):
    """Storage array (bf16 bits or fp32) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _small(dtype="f32", lengths=("list", [37, 130]), batch=2, n_heads=8, d_h=16, d_c=64,
           n_blocks=4, d_r=16, k=1, page_size=64, paged=True, seed=5, **kw):
    s = synth.Shape(batch=batch, n_heads=n_heads, d_h=d_h, d_c=d_c, n_blocks=n_blocks, d_r=d_r,
                    dtype=dtype, page_size=page_size, blocks_per_head=k, paged=paged, **kw)
    return synth.make_inputs(s, lengths, seed)


def _gather_rows(inp, b):
    """Rows of sequence b in logical order, via the page table (numpy indexing)."""
    s = inp.shape
    n = int(inp.seq_lens[b])
    t = np.arange(n)
    if inp.page_table is None:
        phys = b * inp.max_pages_per_seq + t // s.page_size
    else:
        phys = inp.page_table[b, t // s.page_size]
    return _f(inp.pool[phys, t % s.page_size, :])


def _textbook(inp, b, i, sigma=None, alpha=None):
    """Textbook attention per attended block over materialised K and V.

    K_t = [W^UK_i^T c_t | k^R_t], V_t = W^UV_i^T c_t, q = [q^C_i | q^R_i],
    softmax(sigma q K^T) V; per-block outputs summed times alpha."""
    s = inp.shape
    sigma = 1.0 / math.sqrt(s.d_h + s.d_r) if sigma is None else sigma
    alpha = 1.0 / math.sqrt(s.blocks_per_head) if alpha is None else alpha
    rows = _gather_rows(inp, b)
    q = np.concatenate([_f(inp.q_c[b, i]), _f(inp.q_r[b, i])])
    w = s.w
    heads_per_group = s.n_heads * s.blocks_per_head // s.n_blocks
    out = np.zeros(s.d_h)
    lses = []
    for jj in range(s.blocks_per_head):
        j = (i // heads_per_group) * s.blocks_per_head + jj
        c = rows[:, j * w:(j + 1) * w]
        kr = rows[:, s.d_c:s.d_c + s.d_r]
        Kc = c @ _f(inp.w_uk[i, jj])  # [n, d_h]
        V = c @ _f(inp.w_uv[i, jj])
        Kfull = np.concatenate([Kc, kr], axis=1)
        logits = sigma * (Kfull @ q)
        m = logits.max()
        e = np.exp(logits - m)
        out += alpha * (e / e.sum()) @ V
        lses.append(m + math.log(e.sum()))
    return out, np.array(lses)


# ---------------------------------------------------------------- counters

def test_table1_loading_per_device():
    """All 24 printed cells of Table 1 (loading per token per device)."""
    P = dict(h=64, d_h=128, g=8, beta_kv=2, d_c=512, d_r=64)
    n_cells = 0
    for line in open(os.path.join(GOLDEN, "table1_loading.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        method, *vals = line.split()
        for tp, v in zip((1, 2, 4, 8), vals):
            got = oracle.cache_elems_per_device(method, tp=tp, **P) / P["d_h"]
            assert got == pytest.approx(float(v), rel=0, abs=1e-12), (method, tp)
            n_cells += 1
    assert n_cells == 24


def test_mlra_loading_derived():
    """MLRA-4 under 4-way TP loads d_c/4 + d_R = 192 elements = 1.5 d_h per
    device: 3x fewer than MLA's 4.5 d_h (derived from Table 1's MLA row)."""
    mlra = oracle.cache_elems_per_device("MLRA", d_c=512, d_r=64, n_blocks=4, tp=4)
    mla = oracle.cache_elems_per_device("MLA", d_c=512, d_r=64, tp=4)
    assert mlra == 192 and mla == 576 and mla / mlra == 3.0
    # on one device the latent blocks together are as wide as MLA's latent
    assert oracle.cache_elems_per_device("MLRA", d_c=512, d_r=64, n_blocks=4, tp=1) == 576


def test_p4_demo_counts():
    g = _kv_file("p4_demo.txt")
    H, dh, dc = int(g["demo_H"]), int(g["demo_d_head"]), int(g["demo_d_c"])
    std = oracle.cache_elems_per_token("MHA", h=H, d_h=dh)
    mla = oracle.cache_elems_per_token("MLA", d_c=dc, d_r=0)
    assert std == int(g["demo_standard_floats_per_token"])
    assert mla == int(g["demo_mla_floats_per_token"])
    assert std // mla == int(g["demo_reduction"])
    H2, dh2, dc2 = int(g["dsv2_H"]), int(g["dsv2_d_head"]), int(g["dsv2_d_c"])
    std2 = oracle.cache_elems_per_token("MHA", h=H2, d_h=dh2)
    mla2 = oracle.cache_elems_per_token("MLA", d_c=dc2, d_r=0)
    gqa = oracle.cache_elems_per_token("GQA", h=H2, d_h=dh2, g=8)
    assert std2 == int(g["dsv2_standard_floats"]) and mla2 == int(g["dsv2_mla_floats"])
    assert std2 / mla2 == int(g["dsv2_mla_reduction"])
    assert std2 / gqa == int(g["dsv2_gqa8_reduction"])
    assert round(gqa / mla2) == int(g["dsv2_mla_vs_gqa"])


def test_p4_demo_reconstruction_shape():
    """The demo's K and V per token have shape (H, d_head)."""
    g = _kv_file("p4_demo.txt")
    H, dh, dc = int(g["demo_H"]), int(g["demo_d_head"]), int(g["demo_d_c"])
    inp = _small(batch=1, n_heads=H, d_h=dh, d_c=dc, n_blocks=1, d_r=8, lengths=("list", [1]))
    out, _ = oracle.decode_unabsorbed(inp)
    assert out.shape == tuple(int(v) for v in g["demo_K_shape"].split(","))


def test_p3_counts():
    g = _kv_file("p3_counts.txt")
    per_layer = oracle.cache_elems_per_token("MHA", h=int(g["mha_heads"]), d_h=int(g["mha_d_head"]))
    assert per_layer * int(g["mha_layers"]) * int(g["mha_bytes_per_elem"]) == int(g["mha_bytes_per_token"])
    assert oracle.cache_elems_per_token("MLA", d_c=int(g["mla_d_c"]), d_r=int(g["mla_d_r"])) == \
        int(g["mla_dims_per_token"])


_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul, ast.Div: operator.truediv}


def _eval(expr, env):
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.Name):
            return env[node.id]
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return node.value
        raise ValueError(ast.dump(node))
    return ev(ast.parse(expr, mode="eval"))


@pytest.mark.parametrize("env", [dict(n=1, h=64, d_c=512, d_R=64), dict(n=8192, h=24, d_c=512, d_R=64),
                                 dict(n=3, h=16, d_c=128, d_R=32)])
def test_table2_intensity(env):
    rows = 0
    for line in open(os.path.join(GOLDEN, "table2_intensity.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        method, uh, uw, num, den = [x.strip() for x in line.split("|")]
        flops, nbytes = oracle.decode_flops_bytes(env["n"], _eval(uh, env), _eval(uw, env), env["d_R"], 2.0)
        assert flops == pytest.approx(_eval(num, env), rel=1e-15), method
        assert nbytes == pytest.approx(_eval(den, env), rel=1e-15), method
        rows += 1
    assert rows == 4


def test_intensity_of_workloads():
    """MLA at h = 64 is 120.9 FLOP/B; one MLRA-4 block with 16 heads is 26.67."""
    f, b = oracle.decode_flops_bytes(1, 64, 512, 64)
    assert f / b == pytest.approx((4 * 64 * 512 + 2 * 64 * 64) / (2 * 576))
    assert f / b == pytest.approx(120.888, abs=1e-3)
    f, b = oracle.decode_flops_bytes(1, 16, 128, 64)
    assert f / b == pytest.approx(26.667, abs=1e-3)


# ---------------------------------------------------------------- rounding

@pytest.mark.parametrize("v,bits", [
    (1.0, 0x3F80), (-2.5, 0xC020), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2 ** -8, 0x3F80),            # tie -> even (1.0)
    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie -> even (1 + 2^-6)
    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),  # just above the tie -> up
    (3.0e38, 0x7F62),
    (2 ** -126, 0x0080),
])
def test_round_bf16(v, bits):
    assert oracle.round_bf16(v) == bits


def test_round_bf16_matches_fp32_path_off_ties():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000).astype(np.float32)
    ref = synth.f32_to_bf16_bits(v)
    got = np.array([oracle.round_bf16(float(x)) for x in v], dtype=np.uint16)
    assert np.array_equal(ref, got)


# ------------------------------------------------------ attention identities

WORKLOAD_SHAPES = {
    1: dict(n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype="f32"),
    2: dict(n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16"),
    3: dict(n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16"),
    4: dict(n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16"),
    5: dict(n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="bf16"),
}


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5])
def test_absorbed_equals_unabsorbed(wl):
    """Absorption is exact algebra: q.(W^UK c) = (W^UK^T q).c and
    sum p W^UV c = W^UV (sum p c) (lesty.tech section 5; ai360xpert
    "Absorbing the up-projection")."""
    inp = _small(batch=2, lengths=("list", [150, 70]), seed=10 + wl, **WORKLOAD_SHAPES[wl])
    pairs = [(b, i) for b in range(2) for i in range(0, inp.shape.n_heads, max(1, inp.shape.n_heads // 6))]
    o1, l1 = oracle.decode_unabsorbed(inp, pairs)
    o2, l2 = oracle.decode_absorbed(inp, pairs)
    assert np.abs(o1 - o2).max() <= 1e-12 * np.abs(o1).max()
    assert np.abs(l1 - l2).max() <= 1e-12 * np.abs(l1).max()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mla_b1_equals_textbook(dtype):
    """b = 1 is MLA with decoupled RoPE: textbook attention over
    K = [W^UK c | k^R], V = W^UV c (lesty.tech section 4)."""
    inp = _small(dtype=dtype, n_blocks=1, lengths=("list", [65, 200]), seed=3)
    out, lse = oracle.decode_unabsorbed(inp)
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(8)]):
        ref, rl = _textbook(inp, b, i)
        assert np.allclose(out[p], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
        assert abs(lse[p, 0] - rl[0]) <= 1e-12 * abs(rl[0])


@pytest.mark.parametrize("k,n_blocks,n_heads", [(1, 4, 8), (1, 2, 8), (2, 4, 8), (4, 4, 8)])
def test_mlra_equals_textbook_per_block(k, n_blocks, n_heads):
    """MLRA: head i attends its latent block(s) with their own softmax; the
    per-block outputs are summed times out_scale."""
    inp = _small(k=k, n_blocks=n_blocks, n_heads=n_heads, lengths=("list", [33, 129]), seed=4)
    out, lse = oracle.decode_unabsorbed(inp)
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(n_heads)]):
        ref, rl = _textbook(inp, b, i)
        assert np.allclose(out[p], ref, rtol=0, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(lse[p], rl, rtol=1e-12)


def test_head_to_block_map():
    """Reading A (k = 1): head i reads block floor(i b / h); reading B groups."""
    inp = _small(n_heads=8, n_blocks=4, k=1)
    assert [oracle.block_of(inp, i, 0) for i in range(8)] == [0, 0, 1, 1, 2, 2, 3, 3]
    inp = _small(n_heads=8, n_blocks=4, k=2)
    assert [[oracle.block_of(inp, i, jj) for jj in range(2)] for i in range(8)] == \
        [[0, 1]] * 4 + [[2, 3]] * 4
    inp = _small(n_heads=8, n_blocks=4, k=4)
    assert all([oracle.block_of(inp, i, jj) for jj in range(4)] == [0, 1, 2, 3] for i in range(8))


def test_block_independence():
    """Latent heads are independent ("sections don't talk to each other during
    lookup", alanhou.org "Key Concepts"): MLRA-b equals b separate MLA problems
    on the latent slices, and perturbing block j's latent changes only the
    outputs of block j's heads."""
    inp = _small(dtype="f32", n_heads=8, n_blocks=4, lengths=("list", [90, 17]), seed=8)
    out, _ = oracle.decode_unabsorbed(inp)
    s = inp.shape
    w = s.w
    for j in range(4):
        heads = list(range(2 * j, 2 * j + 2))
        sub_shape = synth.Shape(batch=2, n_heads=2, d_h=s.d_h, d_c=w, n_blocks=1, d_r=s.d_r,
                                dtype="f32", page_size=s.page_size,
                                softmax_scale=1.0 / math.sqrt(s.d_h + s.d_r))
        sub = synth.Inputs(
            shape=sub_shape, seq_lens=inp.seq_lens, page_table=inp.page_table,
            max_pages_per_seq=inp.max_pages_per_seq,
            pool=np.ascontiguousarray(np.concatenate(
                [inp.pool[:, :, j * w:(j + 1) * w], inp.pool[:, :, s.d_c:]], axis=2)),
            q_c=np.ascontiguousarray(inp.q_c[:, heads]), q_r=np.ascontiguousarray(inp.q_r[:, heads]),
            w_uk=np.ascontiguousarray(inp.w_uk[heads]), w_uv=np.ascontiguousarray(inp.w_uv[heads]))
        sub_out, _ = oracle.decode_unabsorbed(sub)
        for b in range(2):
            for hi, i in enumerate(heads):
                assert np.array_equal(sub_out[b * 2 + hi], out[b * 8 + i])
    pool2 = inp.pool.copy()
    pool2[:, :, 1 * w:2 * w] += 1.0  # perturb block 1 only
    out2, _ = oracle.decode_unabsorbed(inp, pool=pool2)
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(8)]):
        if i in (2, 3):
            assert not np.array_equal(out2[p], out[p])
        else:
            assert np.array_equal(out2[p], out[p])


def test_zero_query_is_mean():
    """q = 0: uniform weights, so o_i = W^UV_i^T mean_t c_t and lse = ln n."""
    inp = _small(lengths=("list", [77, 5]), seed=11)
    inp.q_c[...] = 0
    inp.q_r[...] = 0
    out, lse = oracle.decode_unabsorbed(inp)
    s = inp.shape
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(8)]):
        rows = _gather_rows(inp, b)
        j = i // 2
        ref = rows[:, j * s.w:(j + 1) * s.w].mean(axis=0) @ _f(inp.w_uv[i, 0])
        assert np.allclose(out[p], ref, rtol=0, atol=1e-13)
        assert lse[p, 0] == pytest.approx(math.log(inp.seq_lens[b]), abs=1e-13)


def test_single_token():
    """n = 1: the only weight is 1, so o_i = W^UV_i^T c_0 whatever q is."""
    inp = _small(lengths=("list", [1, 1]), seed=12)
    out, _ = oracle.decode_unabsorbed(inp)
    s = inp.shape
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(8)]):
        c0 = _gather_rows(inp, b)[0]
        j = i // 2
        assert np.allclose(out[p], c0[j * s.w:(j + 1) * s.w] @ _f(inp.w_uv[i, 0]), rtol=0, atol=1e-13)


def test_one_hot():
    """A score gap of ~60 nats on one token: the output is that token's value."""
    inp = _small(lengths=("list", [50, 100]), seed=13)
    s = inp.shape
    inp.q_r[...] = 0
    inp.q_r[:, :, 0] = 1.0
    tstar = {0: 17, 1: 64}
    for b, t in tstar.items():
        rows_b = np.arange(inp.seq_lens[b])
        phys = inp.page_table[b, rows_b // s.page_size]
        inp.pool[phys, rows_b % s.page_size, s.d_c] = 0.0
        inp.pool[inp.page_table[b, t // s.page_size], t % s.page_size, s.d_c] = 60.0 * math.sqrt(s.d_h + s.d_r)
    inp.q_c[...] = 0  # only the RoPE term scores
    out, _ = oracle.decode_unabsorbed(inp)
    for p, (b, i) in enumerate([(b, i) for b in range(2) for i in range(8)]):
        c = _gather_rows(inp, b)[tstar[b]]
        j = i // 2
        ref = c[j * s.w:(j + 1) * s.w] @ _f(inp.w_uv[i, 0])
        assert np.allclose(out[p], ref, rtol=0, atol=1e-14 * np.abs(ref).max())


def test_brute_force_pure_python():
    """n <= 8, tiny shape: everything recomputed with Python floats and
    math.fsum, without numpy."""
    inp = _small(batch=2, n_heads=4, d_h=3, d_c=4, n_blocks=2, d_r=2, lengths=("list", [8, 3]), seed=21)
    out, lse = oracle.decode_unabsorbed(inp)
    s = inp.shape
    sigma = 1.0 / math.sqrt(s.d_h + s.d_r)
    pool = inp.pool.tolist()
    p = 0
    for b in range(2):
        n = int(inp.seq_lens[b])
        rows = [pool[int(inp.page_table[b][t // 64])][t % 64] for t in range(n)]
        for i in range(4):
            j = i // 2
            wk = inp.w_uk[i][0].tolist()
            wv = inp.w_uv[i][0].tolist()
            q = inp.q_c[b][i].tolist()
            qr = inp.q_r[b][i].tolist()
            logits = []
            vals = []
            for r in rows:
                c = r[j * 2:(j + 1) * 2]
                K = [math.fsum(wk[cc][d] * c[cc] for cc in range(2)) for d in range(3)]
                V = [math.fsum(wv[cc][d] * c[cc] for cc in range(2)) for d in range(3)]
                logits.append(sigma * (math.fsum(q[d] * K[d] for d in range(3)) +
                                       math.fsum(qr[e] * r[4 + e] for e in range(2))))
                vals.append(V)
            m = max(logits)
            ex = [math.exp(x - m) for x in logits]
            den = math.fsum(ex)
            ref = [math.fsum(ex[t] / den * vals[t][d] for t in range(n)) for d in range(3)]
            assert np.allclose(out[p], ref, rtol=1e-13, atol=1e-15)
            assert lse[p, 0] == pytest.approx(m + math.log(den), rel=1e-14)
            p += 1


def test_empty_sequence():
    inp = _small(lengths=("list", [0, 9]), seed=22)
    out, lse = oracle.decode_unabsorbed(inp)
    assert np.all(out[:8] == 0) and np.all(np.isneginf(lse[:8]))
    assert np.all(np.isfinite(out[8:]))


def test_page_permutation_invariance():
    """The result depends on the logical token order only: a contiguous copy of
    each sequence and the permuted paged pool give bit-identical outputs."""
    inp = _small(dtype="bf16", lengths=("list", [200, 129]), seed=23)
    s = inp.shape
    out, lse = oracle.decode_unabsorbed(inp)
    mp = inp.max_pages_per_seq
    pool2 = np.zeros((2 * mp, s.page_size, s.row), dtype=inp.pool.dtype)
    for b in range(2):
        for pg in range(mp):
            pool2[b * mp + pg] = inp.pool[inp.page_table[b, pg]]
    ident = synth.Inputs(**{**inp.__dict__, "page_table": None})
    ident.pool = pool2
    out2, lse2 = oracle.decode_unabsorbed(ident)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_softmax_scale_default():
    inp = _small(seed=24)
    o1, _ = oracle.decode_unabsorbed(inp)
    o2, _ = oracle.decode_unabsorbed(inp, softmax_scale=1.0 / math.sqrt(16 + 16))
    assert np.array_equal(o1, o2)
    o3, _ = oracle.decode_unabsorbed(inp, softmax_scale=0.5)
    assert not np.allclose(o1, o3)


def test_no_canary_read():
    """Rows outside the sequences hold NaN; the oracle never reads them."""
    inp = _small(dtype="bf16", lengths=("list", [3, 130]), seed=25)
    assert np.isnan(_f(inp.pool)).any()
    out, lse = oracle.decode_unabsorbed(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# ------------------------------------------------------------------- append

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append(dtype):
    """c_new = x W^DKV (ai360xpert "The two projections"), rounded once; the
    row [c_new | k^R_new] lands at pt[b][pos / P] P + pos % P and nothing else
    in the pool changes."""
    s = synth.Shape(batch=3, n_heads=8, d_h=16, d_c=64, n_blocks=2, d_r=16, dtype=dtype, d_model=96)
    inp = synth.make_inputs(s, ("list_append", [5, 64, 130]), 31)
    pool = inp.pool.copy()
    c = oracle.append(inp, pool)
    ref = _f(inp.x) @ _f(inp.w_dkv)  # float64 library matmul
    if dtype == "bf16":
        ref_bits = np.array([[oracle.round_bf16(v) for v in r] for r in ref], dtype=np.uint16)
        assert np.array_equal(c, ref_bits)
    else:
        assert np.array_equal(c, ref.astype(np.float32))
    changed = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(3):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // 64], pos % 64
        assert oracle.row_index(inp, b, pos) == pg * 64 + off
        assert np.array_equal(pool[pg, off, :64], c[b])
        assert np.array_equal(pool[pg, off, 64:], inp.kr_new[b])
        changed[pg, off] = True
    before = inp.pool.view(np.uint16 if dtype == "bf16" else np.uint32)
    after = pool.view(before.dtype)
    assert np.array_equal(before[~changed], after[~changed])


# -------------------------------------------------------------------- synth

def test_synth_deterministic():
    a = synth.make_inputs(synth.WORKLOADS[5]["shape"], ("uniform_append", 1024, 4096), 99)
    b = synth.make_inputs(synth.WORKLOADS[5]["shape"], ("uniform_append", 1024, 4096), 99)
    for k in ("seq_lens", "page_table", "pool", "q_c", "q_r", "w_uk", "w_uv", "x", "w_dkv", "kr_new"):
        assert np.array_equal(getattr(a, k).view(np.uint8), getattr(b, k).view(np.uint8)), k
    assert np.all(a.seq_lens == a.positions + 1)
    assert a.seq_lens.min() >= 1025 and a.seq_lens.max() <= 4097


# ---------------------------------------------------------------- FP8 cache
# The lesty.tech MLA explainer (section 5) notes that the cached latent can be
# quantised with FP8 frameworks; the encoding here is OCP FP8 E4M3FN with one
# scale per cache (the readings are listed in the design notes).

E4M3_KNOWN = {  # code -> value, from the OCP 8-bit floating point specification's E4M3 table
    0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 0.875 * 2.0 ** -6, 0x08: 2.0 ** -6,
    0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0,
}


def test_e4m3_decode_known_values_and_library():
    for code, v in E4M3_KNOWN.items():
        assert oracle.e4m3_decode(code) == v and math.copysign(1, oracle.e4m3_decode(code)) == math.copysign(1, v)
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    torch = pytest.importorskip("torch")
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    mine = np.array([oracle.e4m3_decode(c) for c in range(256)])
    same = (mine == lib) | (np.isnan(mine) & np.isnan(lib))
    assert same.all(), np.nonzero(~same)


def test_e4m3_encode_roundtrip_ties_and_saturation():
    # every finite code is a fixed point of encode(decode(.))
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c, hex(c)
    # midpoints between neighbouring positive codes go to the even code
    for c in range(0x00, 0x7E):
        lo, hi = oracle.e4m3_decode(c), oracle.e4m3_decode(c + 1)
        mid = np.float32((lo + hi) / 2)
        if float(mid) != (lo + hi) / 2:
            continue  # not exactly representable in fp32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(float(mid)) == want, hex(c)
    # saturation (the reading chosen for values past the largest finite code) and NaN
    for v, code in ((448.0, 0x7E), (463.9, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE)):
        assert oracle.e4m3_encode(v) == code, v
    assert oracle.e4m3_encode(float("nan")) == 0x7F


def test_e4m3_encode_matches_library_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.1, 1.0, 30.0, 150.0)]).astype(np.float32)
    x = x[np.abs(x) < 464.0]  # the library rounds past the largest code to NaN; the oracle saturates
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_array(x), lib)


def _fp8_and_bf16_twin(seed, lengths, cache_scale, **kw):
    """An FP8 problem and a bf16 problem whose latents hold exactly the FP8
    problem's dequantised values (E4M3 values times a power of two are bf16)."""
    s8 = synth.Shape(dtype="fp8", cache_scale=cache_scale, **kw)
    inp8 = synth.make_inputs(s8, lengths, seed)
    codes = inp8.pool[..., :s8.d_c]
    table = np.array([oracle.e4m3_decode(c) for c in range(256)]) * (cache_scale or 1.0)
    lat = synth.f32_to_bf16_bits(table[codes].astype(np.float32))
    rope = np.ascontiguousarray(inp8.pool[..., s8.d_c:]).view(np.uint16)
    s16 = synth.Shape(dtype="bf16", **kw)
    inp16 = synth.make_inputs(s16, lengths, seed)
    inp16.pool = np.ascontiguousarray(np.concatenate([lat, rope], axis=-1))
    for f in ("page_table", "seq_lens", "q_c", "q_r", "w_uk", "w_uv", "max_pages_per_seq"):
        setattr(inp16, f, getattr(inp8, f))
    return inp8, inp16


def test_fp8_cache_decodes_like_its_bf16_twin():
    """An FP8 cache reads as (decoded code) x cache_scale for the latent and as
    bf16 for the RoPE key: the oracle's result equals the bf16 path's (itself
    pinned to textbook attention) on the dequantised twin, canaries included."""
    inp8, inp16 = _fp8_and_bf16_twin(21, ("list", [150, 1, 70]), 0.5, batch=3, n_heads=8, d_h=16,
                                     d_c=64, n_blocks=4, d_r=16)
    o8, l8 = oracle.decode_unabsorbed(inp8)
    o16, l16 = oracle.decode_unabsorbed(inp16)
    assert np.all(np.isfinite(o8))
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
    a8, al8 = oracle.decode_absorbed(inp8)
    assert np.abs(a8 - o8).max() <= 1e-12 * np.abs(o8).max()


def test_fp8_append_encodes_the_fp32_latent():
    """FP8 append: c = x W^DKV (numpy float64 matmul), rounded to fp32, times
    the fp32 reciprocal of cache_scale, encoded by the library's E4M3 rounding;
    c_out holds the fp32 latent; the RoPE key lands as bf16; nothing else moves."""
    torch = pytest.importorskip("torch")
    s = synth.Shape(batch=3, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype="fp8",
                    cache_scale=0.25, d_model=96)
    inp = synth.make_inputs(s, ("list_append", [0, 63, 200]), 8)
    pool = inp.pool.copy()
    c = oracle.append(inp, pool)
    x = _f(inp.x)
    w = _f(inp.w_dkv)
    c_ref = (x @ w).astype(np.float32)
    # summation order may move the fp32 rounding of a sum by one unit in the last place
    assert np.all(np.abs(c - c_ref) <= 2 * np.spacing(np.abs(c_ref)))
    want = torch.from_numpy(c * np.float32(1.0 / 0.25)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    changed = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // s.page_size], pos % s.page_size
        changed[pg, off] = True
        assert np.array_equal(pool[pg, off, :s.d_c], want[b])
        assert np.array_equal(pool[pg, off, s.d_c:].view(np.uint16), inp.kr_new[b])
    assert np.array_equal(pool[~changed], inp.pool[~changed])


def _fp8b_dequantised(inp):
    """The block-scaled pool's rows as float64 [pages][P][d_c + d_r]: codes
    decoded by the library's E4M3FN type times the row's per-block fp32 scale
    (read as raw float32 bytes), the RoPE key from its bf16 bits."""
    torch = pytest.importorskip("torch")
    s = inp.shape
    pool = inp.pool
    codes = torch.from_numpy(np.ascontiguousarray(pool[..., :s.d_c])).view(torch.float8_e4m3fn).double().numpy()
    o = s.d_c + 2 * s.d_r
    scales = np.ascontiguousarray(pool[..., o:o + 4 * s.n_blocks]).view(np.float32).astype(np.float64)
    lat = codes * np.repeat(scales, s.w, axis=-1)
    rope = synth.bf16_bits_to_f32(np.ascontiguousarray(pool[..., s.d_c:o]).view(np.uint16)).astype(np.float64)
    return np.concatenate([lat, rope], axis=-1)


def test_fp8b_row_layout():
    """Block-scaled rows: codes, bf16 RoPE key, one fp32 scale per block, zero
    pad to a multiple of 16 bytes."""
    for d_c, d_r, nb, want in ((512, 64, 4, 656), (512, 64, 1, 656), (128, 64, 1, 272), (512, 64, 2, 656),
                               (64, 16, 4, 112)):
        s = synth.Shape(batch=1, n_heads=8, d_h=16, d_c=d_c, n_blocks=nb, d_r=d_r, dtype="fp8b")
        assert s.row_bytes == want
        inp = synth.make_inputs(s, ("list", [20]), 1)
        assert oracle.fp8_row_bytes(inp) == want
        assert inp.pool.shape[-1] == want
        assert np.all(inp.pool[..., d_c + 2 * d_r + 4 * nb:] == 0)


def test_fp8b_cache_equals_textbook_on_dequantised_rows():
    """A block-scaled FP8 cache reads latent (row, col) as decoded code x the
    scale of col's block in that row: the oracle equals textbook attention over
    the dequantised rows, on every (sequence, head) pair, blocks_per_head 1 and 2."""
    for k in (1, 2):
        inp = _small("fp8b", lengths=("list", [130, 1, 77]), batch=3, k=k, seed=40 + k)
        rows = _fp8b_dequantised(inp)
        o, l = oracle.decode_unabsorbed(inp)
        twin = synth.make_inputs(inp.shape, ("list", [130, 1, 77]), 40 + k)
        twin.pool = np.ascontiguousarray(rows)
        for b in range(3):
            for i in range(inp.shape.n_heads):
                ref, rl = _textbook(twin, b, i)
                r = b * inp.shape.n_heads + i
                assert np.abs(o[r] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), (k, b, i)
                assert np.abs(l[r] - rl).max() <= 1e-12 * max(1.0, np.abs(rl).max())
        a, _ = oracle.decode_absorbed(inp)
        assert np.abs(a - o).max() <= 1e-12 * np.abs(o).max()


def test_fp8b_equal_scales_equal_per_cache_scale():
    """Every block scale set to 0.5 reads exactly like the per-cache-scaled
    FP8 cache of the same codes with cache_scale 0.5."""
    kw = dict(batch=3, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16)
    sb = synth.Shape(dtype="fp8b", **kw)
    inp_b = synth.make_inputs(sb, ("list", [150, 1, 70]), 23)
    o = kw["d_c"] + 2 * kw["d_r"]
    sc = inp_b.pool[..., o:o + 16].view(np.float32)
    finite = np.isfinite(sc)
    sc[finite] = 0.5  # canary rows keep their NaN scales
    s8 = synth.Shape(dtype="fp8", cache_scale=0.5, **kw)
    inp8 = synth.make_inputs(s8, ("list", [150, 1, 70]), 23)
    inp8.pool = np.ascontiguousarray(inp_b.pool[..., :o])
    for f in ("page_table", "seq_lens", "q_c", "q_r", "w_uk", "w_uv", "max_pages_per_seq"):
        setattr(inp8, f, getattr(inp_b, f))
    ob, lb = oracle.decode_unabsorbed(inp_b)
    o8, l8 = oracle.decode_unabsorbed(inp8)
    assert np.all(np.isfinite(ob))
    assert np.array_equal(ob, o8) and np.array_equal(lb, l8)


def test_fp8b_block_encode_closed_forms():
    torch = pytest.importorskip("torch")
    # the largest magnitude gets the largest code; scale = amax / 448 in fp32
    codes, sc = oracle.fp8_block_encode(np.array([1.0, -2.0, 0.25, 0.0], np.float32))
    assert sc == np.float32(2.0) / np.float32(448.0)
    assert codes[1] == 0xFE and oracle.e4m3_decode(int(codes[0])) * float(sc) == pytest.approx(1.0, rel=2 ** -4)
    assert codes[3] == 0x00
    # all zero: scale 1, zero codes; a NaN is skipped and encodes to 0x7F
    codes, sc = oracle.fp8_block_encode(np.zeros(8, np.float32))
    assert sc == 1.0 and np.all(codes == 0)
    codes, sc = oracle.fp8_block_encode(np.array([np.nan, 3.5, -7.0], np.float32))
    assert sc == np.float32(7.0) / np.float32(448.0) and codes[0] == 0x7F and codes[2] == 0xFE
    # an infinite value: scale 1, the values saturate
    codes, sc = oracle.fp8_block_encode(np.array([np.inf, 1.0], np.float32))
    assert sc == 1.0 and codes[0] == 0x7E and codes[1] == 0x38
    # a block too small for a normal scale: scale 1
    codes, sc = oracle.fp8_block_encode(np.array([1e-39, -2e-39], np.float32))
    assert sc == 1.0
    # random blocks: codes = the library's E4M3 rounding of c x fp32(1 / scale);
    # the decoded value is within half a code spacing of c (relative 2^-4 above
    # the subnormal range)
    rng = np.random.default_rng(9)
    for mag in (1e-3, 1.0, 1e4):
        c = (rng.standard_normal(128) * mag).astype(np.float32)
        codes, sc = oracle.fp8_block_encode(c)
        amax = np.float32(np.abs(c).max())
        assert sc == amax / np.float32(448.0)
        inv = np.float32(1.0) / sc
        want = torch.from_numpy(c * inv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes, want)
        dec = np.array([oracle.e4m3_decode(int(v)) for v in codes]) * float(sc)
        err = np.abs(dec - c.astype(np.float64))
        bound = np.maximum(2.0 ** -4 * np.abs(c), 2.0 ** -10 * float(sc)) * (1 + 1e-6)
        assert np.all(err <= bound)


def test_fp8b_append_encodes_each_block_with_its_own_scale():
    """Block-scaled append: c = x W^DKV (numpy float64 matmul) rounded to
    fp32; each block's scale is its fp32 largest magnitude / 448 and its codes
    the library's E4M3 rounding of c x fp32(1 / scale); the RoPE key lands as
    bf16, the pad bytes are zero, and nothing else moves."""
    torch = pytest.importorskip("torch")
    s = synth.Shape(batch=3, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype="fp8b", d_model=96)
    inp = synth.make_inputs(s, ("list_append", [0, 63, 200]), 8)
    pool = inp.pool.copy()
    c = oracle.append(inp, pool)
    c_ref = (_f(inp.x) @ _f(inp.w_dkv)).astype(np.float32)
    assert np.all(np.abs(c - c_ref) <= 2 * np.spacing(np.abs(c_ref)))
    o = s.d_c + 2 * s.d_r
    changed = np.zeros(pool.shape[:2], dtype=bool)
    for b in range(s.batch):
        pos = int(inp.positions[b])
        pg, off = inp.page_table[b, pos // s.page_size], pos % s.page_size
        changed[pg, off] = True
        row = pool[pg, off]
        for j in range(s.n_blocks):
            blk = c[b, j * s.w:(j + 1) * s.w]
            sc = np.float32(np.abs(blk).max()) / np.float32(448.0)
            assert row[o + 4 * j:o + 4 * j + 4].view(np.float32)[0] == sc
            want = torch.from_numpy(blk * (np.float32(1.0) / sc)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(row[j * s.w:(j + 1) * s.w], want)
        assert np.array_equal(row[s.d_c:o].view(np.uint16), inp.kr_new[b])
        assert np.all(row[o + 4 * s.n_blocks:] == 0)
    assert np.array_equal(pool[~changed], inp.pool[~changed])


# ------------------------------------------------- RoPE and the query path
# lesty.tech section 4: k^R = RoPE(h W^KR), the query split the same way; the
# rotation is RoFormer's (cited by the MLRA index page). Readings in the design notes.

def test_rope_closed_forms():
    # position 0 is the identity
    v = np.random.default_rng(1).standard_normal(64)
    assert np.array_equal(oracle.rope(v, 0), v)
    # d = 2: theta_0 = 1, so (1, 0) turns by pos radians, counter-clockwise
    for pos in (1, 2, 7, 1000):
        r = oracle.rope(np.array([1.0, 0.0]), pos)
        assert abs(r[0] - math.cos(pos)) < 1e-12 and abs(r[1] - math.sin(pos)) < 1e-12
    # d = 4, base 10000: pair 1 turns at 10000^(-1/2) = 0.01 rad per position
    r = oracle.rope(np.array([0.0, 0.0, 0.0, 1.0]), 100)
    assert np.allclose(r, [0.0, 0.0, -math.sin(1.0), math.cos(1.0)], atol=1e-12)
    # adjacent pairs: a unit vector stays inside its own pair
    e1 = np.zeros(8)
    e1[5] = 1.0
    r = oracle.rope(e1, 33)
    assert np.all(r[[0, 1, 2, 3, 6, 7]] == 0.0) and abs(np.hypot(r[4], r[5]) - 1.0) < 1e-12
    # another base
    r = oracle.rope(np.array([0.0, 0.0, 1.0, 0.0]), 10, base=100.0)
    assert np.allclose(r, [0.0, 0.0, math.cos(1.0), math.sin(1.0)], atol=1e-12)


def test_rope_is_a_rotation_with_relative_positions():
    """Norms are preserved and <RoPE(q, m), RoPE(k, n)> depends only on m - n
    (RoFormer's defining property)."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m in (0, 5, 1234):
        assert abs(np.linalg.norm(oracle.rope(q, m)) - np.linalg.norm(q)) < 1e-10
    base = float(oracle.rope(q, 40) @ oracle.rope(k, 25))
    for shift in (1, 17, 9000):
        assert abs(float(oracle.rope(q, 40 + shift) @ oracle.rope(k, 25 + shift)) - base) < 1e-9
    assert abs(float(oracle.rope(q, 15) @ oracle.rope(k, 0)) - base) < 1e-9


def _proj_inputs(dtype="f32", seed=31):
    s = synth.Shape(batch=3, n_heads=4, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype=dtype, d_model=48,
                    d_cq=24, rope_base=500.0)
    return synth.make_inputs(s, ("list_append", [0, 70, 300]), seed)


def test_rope_key_is_rotated_projection():
    inp = _proj_inputs()
    kr = oracle.rope_key(inp)
    xw = _f(inp.x) @ _f(inp.w_kr)  # numpy matmul
    for b in range(inp.shape.batch):
        assert np.allclose(kr[b], oracle.rope(xw[b], int(inp.positions[b]), base=500.0), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_project_query_against_numpy(dtype):
    inp = _proj_inputs(dtype)
    qc, qr = oracle.project_query(inp)
    cq = _f(inp.x) @ _f(inp.w_dq)
    s = inp.shape
    for b in range(s.batch):
        for i in range(s.n_heads):
            assert np.allclose(qc[b, i], cq[b] @ _f(inp.w_uq)[i], rtol=1e-12, atol=1e-12)
            want = oracle.rope(cq[b] @ _f(inp.w_qr)[i], int(inp.positions[b]), base=500.0)
            assert np.allclose(qr[b, i], want, rtol=1e-12, atol=1e-12)
