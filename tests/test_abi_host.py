"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import compressed_kv_cache_mlra_amd as mlra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlra.h")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlra_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = mlra.lib()
    names = _declared_symbols()
    assert {"mlra_append_latent", "mlra_decode", "mlra_combine"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    assert mlra.lib().mlra_abi_version() == mlra.ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5):
        assert mlra.status_string(code) != "unknown status"
    assert mlra.status_string(7) == "unknown status"


def _desc(**kw):
    base = dict(batch=2, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, max_pages_per_seq=4,
                num_pages=8, dtype="f32", page_size=64)
    base.update(kw)
    return mlra.make_desc(**base)


def _decode(desc, ws_bytes=1 << 30, pool=FAKE, seq_lens=FAKE, q_c=FAKE, q_r=FAKE, w_uk=FAKE,
            ws=FAKE, max_seq_len=10):
    return mlra.lib().mlra_decode(ctypes.byref(desc), pool, None, seq_lens, max_seq_len, q_c, q_r,
                                  w_uk, ws, ctypes.c_size_t(ws_bytes), None)


BAD_DESCS = [
    (dict(batch=0), mlra.ERR_INVALID_ARG),
    (dict(n_heads=0), mlra.ERR_INVALID_ARG),
    (dict(d_c=66), mlra.ERR_INVALID_ARG),            # d_c not divisible by n_blocks
    (dict(n_heads=6), mlra.ERR_INVALID_ARG),         # h not divisible by b / k
    (dict(blocks_per_head=3), mlra.ERR_INVALID_ARG),  # k does not divide b
    (dict(page_size=48), mlra.ERR_INVALID_ARG),      # not a power of two
    (dict(page_size=8), mlra.ERR_INVALID_ARG),
    (dict(page_size=512), mlra.ERR_INVALID_ARG),
    (dict(d_r=2), mlra.ERR_INVALID_ARG),             # row bytes not a multiple of 16
    (dict(dtype="bf16", d_c=4 * 12, d_r=16), mlra.ERR_INVALID_ARG),  # bf16 block width % 8
    (dict(dtype=7), mlra.ERR_UNSUPPORTED),
    (dict(d_h=1024), mlra.ERR_UNSUPPORTED),
    (dict(d_c=4 * 1024), mlra.ERR_UNSUPPORTED),      # block wider than 512
    (dict(max_pages_per_seq=0), mlra.ERR_INVALID_ARG),
    (dict(num_pages=0), mlra.ERR_INVALID_ARG),
    (dict(d_r=-8), mlra.ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), mlra.ERR_INVALID_ARG),
    (dict(batch=4097), mlra.ERR_UNSUPPORTED),          # the plan keeps the batch in LDS
    (dict(batch=4096, max_pages_per_seq=1 << 18, page_size=256), mlra.ERR_UNSUPPORTED),  # int32 tile count
]


@pytest.mark.parametrize("kw,code", BAD_DESCS)
def test_bad_descriptor(kw, code):
    if kw.get("dtype") == 7:
        d = _desc()
        d.dtype = 7
    else:
        d = _desc(**kw)
    assert _decode(d) == code
    assert mlra.lib().mlra_workspace_bytes(ctypes.byref(d), 10) == 0


def test_null_descriptor():
    L = mlra.lib()
    assert L.mlra_decode(None, FAKE, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == mlra.ERR_INVALID_ARG
    assert L.mlra_workspace_bytes(None, 1) == 0


@pytest.mark.parametrize("field", ["pool", "seq_lens", "q_c", "q_r", "w_uk", "ws"])
def test_null_pointers(field):
    d = _desc()
    assert _decode(d, **{field: None}) == mlra.ERR_INVALID_ARG


def test_max_seq_len_range():
    d = _desc()
    assert _decode(d, max_seq_len=-1) == mlra.ERR_INVALID_ARG
    assert _decode(d, max_seq_len=4 * 64 + 1) == mlra.ERR_INVALID_ARG
    assert mlra.lib().mlra_workspace_bytes(ctypes.byref(d), 4 * 64 + 1) == 0


def test_workspace_too_small():
    d = _desc()
    need = mlra.workspace_bytes(d, 100)
    assert need > 0
    assert _decode(d, ws_bytes=need - 1) == mlra.ERR_WORKSPACE
    L = mlra.lib()
    assert L.mlra_combine(ctypes.byref(d), FAKE, ctypes.c_size_t(need - 1), FAKE, FAKE, None, None) == \
        mlra.ERR_WORKSPACE
    assert L.mlra_attend(ctypes.byref(d), FAKE, None, FAKE, ctypes.c_size_t(need - 1), None) == \
        mlra.ERR_WORKSPACE


def test_workspace_independent_of_lengths():
    d = _desc()
    assert mlra.workspace_bytes(d, 0) == mlra.workspace_bytes(d, 256)


def test_combine_and_append_validation():
    L = mlra.lib()
    d = _desc()
    assert L.mlra_combine(ctypes.byref(d), None, 1 << 30, FAKE, FAKE, None, None) == mlra.ERR_INVALID_ARG
    assert L.mlra_combine(ctypes.byref(d), FAKE, 1 << 30, FAKE, None, None, None) == mlra.ERR_INVALID_ARG
    # append needs d_model >= 1
    A = L.mlra_append_latent
    ws = (FAKE, ctypes.c_size_t(16), None)  # a workspace far too small: nothing valid gets past it
    assert A(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, *ws) == mlra.ERR_INVALID_ARG
    d2 = _desc(d_model=32)
    assert A(ctypes.byref(d2), None, None, FAKE, FAKE, FAKE, FAKE, None, *ws) == mlra.ERR_INVALID_ARG
    assert A(ctypes.byref(d2), FAKE, None, FAKE, FAKE, FAKE, None, None, *ws) == \
        mlra.ERR_INVALID_ARG  # k^R_new required when d_r > 0
    assert A(ctypes.byref(d2), FAKE, None, FAKE, FAKE, ctypes.c_void_p(0x1008), FAKE, None, *ws) == \
        mlra.ERR_INVALID_ARG  # W^DKV not 16-byte aligned
    # the workspace is part of the contract on every path
    assert A(ctypes.byref(d2), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, ctypes.c_size_t(1 << 30), None) == \
        mlra.ERR_INVALID_ARG
    d3 = _desc(d_model=32, dtype="bf16", n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16)
    assert A(ctypes.byref(d3), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, *ws) == mlra.ERR_WORKSPACE


def test_decode_step_validation():
    """The one-call step checks everything the three calls it stands for check."""
    L = mlra.lib()
    d = _desc()
    need = mlra.workspace_bytes(d, 100)

    def step(pool=FAKE, seq_lens=FAKE, max_seq_len=100, q_c=FAKE, q_r=FAKE, w_uk=FAKE, w_uv=FAKE, out=FAKE,
             lse=None, ws=FAKE, ws_bytes=need):
        return L.mlra_decode_step(ctypes.byref(d), pool, None, seq_lens, max_seq_len, q_c, q_r, w_uk, w_uv, out,
                                  lse, ws, ctypes.c_size_t(ws_bytes), None)

    for field in ("pool", "seq_lens", "q_c", "q_r", "w_uk", "w_uv", "out", "ws"):
        assert step(**{field: None}) == mlra.ERR_INVALID_ARG, field
    assert step(max_seq_len=-1) == mlra.ERR_INVALID_ARG
    assert step(max_seq_len=4 * 64 + 1) == mlra.ERR_INVALID_ARG
    assert step(ws_bytes=need - 1) == mlra.ERR_WORKSPACE
    assert L.mlra_decode_step(None, FAKE, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                              ctypes.c_size_t(need), None) == mlra.ERR_INVALID_ARG


def test_decode_step_noalloc_validation():
    """The allocation-free step validates like mlra_decode_step and rejects a
    shape whose workspace exceeds the static scratch, all before any HIP call."""
    L = mlra.lib()
    d = _desc()

    def step(desc=d, pool=FAKE, seq_lens=FAKE, max_seq_len=100, q_c=FAKE, q_r=FAKE, w_uk=FAKE, w_uv=FAKE,
             out=FAKE, lse=None):
        return L.mlra_decode_step_noalloc(ctypes.byref(desc), pool, None, seq_lens, max_seq_len, q_c, q_r, w_uk,
                                          w_uv, out, lse, None)

    for field in ("pool", "seq_lens", "q_c", "q_r", "w_uk", "w_uv", "out"):
        assert step(**{field: None}) == mlra.ERR_INVALID_ARG, field
    assert step(max_seq_len=-1) == mlra.ERR_INVALID_ARG
    assert step(max_seq_len=4 * 64 + 1) == mlra.ERR_INVALID_ARG
    assert L.mlra_decode_step_noalloc(None, FAKE, None, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                      None) == mlra.ERR_INVALID_ARG
    big = _desc(batch=4096, n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16", max_pages_per_seq=1,
                num_pages=4096)
    assert mlra.workspace_bytes(big, 64) > mlra.NOALLOC_SCRATCH_BYTES
    assert step(desc=big, max_seq_len=64) == mlra.ERR_SCRATCH
    assert "scratch" in mlra.status_string(mlra.ERR_SCRATCH)


def test_attend_timed_validation():
    """The timed attention helper validates like mlra_attend and needs both events."""
    L = mlra.lib()
    d = _desc()
    need = mlra.workspace_bytes(d, 100)

    def call(pool=FAKE, ws=FAKE, ws_bytes=need, t0=FAKE, t1=FAKE):
        return L.mlra_attend_timed(ctypes.byref(d), pool, None, ws, ctypes.c_size_t(ws_bytes), t0, t1, None)

    for field in ("pool", "ws", "t0", "t1"):
        assert call(**{field: None}) == mlra.ERR_INVALID_ARG, field
    assert call(ws_bytes=need - 1) == mlra.ERR_WORKSPACE


def test_project_token_validation():
    L = mlra.lib()
    d = _desc(d_model=64, d_cq=32, dtype="bf16")

    def call(desc=d, x=FAKE, pos=FAKE, pool=FAKE, wdkv=FAKE, wkr=FAKE, kr=FAKE, wdq=FAKE, wuq=FAKE, wqr=FAKE,
             cq=FAKE, qc=FAKE, qr=FAKE, ws=FAKE, ws_bytes=16):
        return L.mlra_project_token(ctypes.byref(desc), x, pos, pool, None, wdkv, wkr, kr, None, wdq, wuq, wqr,
                                    cq, qc, qr, ws, ctypes.c_size_t(ws_bytes), None)

    for k in ("x", "pos", "pool", "wdkv", "wkr", "kr", "wdq", "wuq", "wqr", "cq", "qc", "qr"):
        assert call(**{k: None}) == mlra.ERR_INVALID_ARG, k
    for k in ("wdkv", "wkr", "wdq", "wuq", "wqr"):
        assert call(**{k: ctypes.c_void_p(0x1004)}) == mlra.ERR_INVALID_ARG, k
    assert call() == mlra.ERR_WORKSPACE
    assert call(ws=None) == mlra.ERR_INVALID_ARG
    # no query path: its arrays may be NULL
    nq = _desc(d_model=64, dtype="bf16")
    assert call(desc=nq, wdq=None, wuq=None, wqr=None, cq=None, qc=None, qr=None) == mlra.ERR_WORKSPACE
    assert call(desc=_desc(d_model=0, d_cq=32, dtype="bf16")) == mlra.ERR_INVALID_ARG


def test_read_flags_validation():
    v = ctypes.c_uint32(0)
    assert mlra.lib().mlra_read_flags(None, 256, ctypes.byref(v), None) == mlra.ERR_INVALID_ARG
    assert mlra.lib().mlra_read_flags(FAKE, 16, ctypes.byref(v), None) == mlra.ERR_INVALID_ARG


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    d = _desc()
    with pytest.raises(ValueError):
        mlra.attend(d, torch.zeros(10), None, torch.zeros(10, dtype=torch.uint8))



def test_absorb_query_validation():
    """The planning call validates like the others before launching."""
    L = mlra.lib()
    d = _desc()
    need = mlra.workspace_bytes(d, 100)
    absorb = L.mlra_absorb_query
    assert absorb(None, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(need), None) == mlra.ERR_INVALID_ARG
    for i in (1, 2, 4, 5):  # seq_lens, q_c, w_uk, workspace
        args = [ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(need), None]
        args[i] = None
        assert absorb(*args) == mlra.ERR_INVALID_ARG, i
    assert absorb(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(need - 1), None) == \
        mlra.ERR_WORKSPACE


def test_stream_read_validation():
    L = mlra.lib()
    assert L.mlra_stream_read(None, 1024, FAKE, 1 << 20, None) == mlra.ERR_INVALID_ARG
    assert L.mlra_stream_read(FAKE, 1024, None, 1 << 20, None) == mlra.ERR_INVALID_ARG
    assert L.mlra_stream_read(FAKE, 1000, FAKE, 1 << 20, None) == mlra.ERR_INVALID_ARG  # not a multiple of 16
    assert L.mlra_stream_read(FAKE, 1024, FAKE, 4, None) == mlra.ERR_INVALID_ARG        # sink too small


def test_fp8_needs_an_mfma_variant_and_aligned_rows():
    """FP8 caches run on the MFMA variants only; other shapes are rejected
    before any launch, as are rows that are not whole 16-byte chunks."""
    ok = _desc(dtype="fp8", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, cache_scale=0.5)
    assert mlra.lib().mlra_workspace_bytes(ctypes.byref(ok), 10) > 0
    no_variant = _desc(dtype="fp8", n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16)
    assert _decode(no_variant) == mlra.ERR_UNSUPPORTED
    bad_row = _desc(dtype="fp8", n_heads=8, d_h=16, d_c=72, n_blocks=1, d_r=16)
    assert _decode(bad_row) == mlra.ERR_INVALID_ARG
    nan_scale = _desc(dtype="fp8", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, cache_scale=float("nan"))
    assert _decode(nan_scale) == mlra.ERR_INVALID_ARG


def test_fp8_block_scaled_descriptor():
    """Block-scaled FP8 caches: the four MFMA shapes are accepted and other
    shapes rejected like per-cache FP8; cache_scale is ignored (even NaN); the
    append's workspace also holds the fp32 latents [B][d_c]; without the MFMA
    product (d_model not a multiple of 8) the append is unsupported."""
    L = mlra.lib()
    for kw in (dict(n_heads=64, d_c=512, n_blocks=4), dict(n_heads=64, d_c=512, n_blocks=1),
               dict(n_heads=16, d_c=128, n_blocks=1), dict(n_heads=64, d_c=512, n_blocks=2)):
        ok = _desc(dtype="fp8b", d_h=128, d_r=64, cache_scale=float("nan"), **kw)
        assert L.mlra_workspace_bytes(ctypes.byref(ok), 10) > 0, kw
    assert _decode(_desc(dtype="fp8b", n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16)) == mlra.ERR_UNSUPPORTED
    assert _decode(_desc(dtype="fp8b", n_heads=8, d_h=16, d_c=72, n_blocks=1, d_r=16)) == mlra.ERR_INVALID_ARG
    per_cache = _desc(dtype="fp8", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, d_model=512)
    blocked = _desc(dtype="fp8b", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, d_model=512)
    extra = L.mlra_workspace_bytes(ctypes.byref(blocked), 10) - L.mlra_workspace_bytes(ctypes.byref(per_cache), 10)
    assert 4 * blocked.batch * 512 <= extra <= 4 * blocked.batch * 512 + 256
    assert mlra.fp8_row_bytes(blocked) == 656 and mlra.fp8_row_bytes(per_cache) == 640
    valu = _desc(dtype="fp8b", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, d_model=500)
    ws = ctypes.c_size_t(L.mlra_workspace_bytes(ctypes.byref(valu), 10))
    st = L.mlra_append_latent(ctypes.byref(valu), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert st == mlra.ERR_UNSUPPORTED


def test_rope_key_validation():
    L = mlra.lib()
    d = _desc(d_model=64)

    def call(desc=d, x=FAKE, w=FAKE, pos=FAKE, out=FAKE, ws=FAKE, ws_bytes=16):
        # ws_bytes far too small: a call that passes every other check stops there
        return L.mlra_rope_key(ctypes.byref(desc), x, w, pos, out, ws, ctypes.c_size_t(ws_bytes), None)

    for kw in (dict(x=None), dict(w=None), dict(pos=None), dict(out=None)):
        assert call(**kw) == mlra.ERR_INVALID_ARG, kw
    assert call(w=ctypes.c_void_p(0x1008)) == mlra.ERR_INVALID_ARG  # W^KR not 16-byte aligned
    assert call(desc=_desc(d_model=0)) == mlra.ERR_INVALID_ARG
    assert call(desc=_desc(d_model=64, d_r=4, d_c=64 + 8)) != mlra.OK  # row or d_r % 8 rejected
    assert call(desc=_desc(d_model=64, rope_base=float("nan"))) == mlra.ERR_INVALID_ARG
    assert call(desc=_desc(d_model=64, rope_base=float("inf"))) == mlra.ERR_INVALID_ARG
    # no RoPE key: nothing to do, nothing dereferenced
    assert call(desc=_desc(d_model=64, d_r=0), x=None, w=None, pos=None, out=None) == mlra.OK
    assert call() == mlra.ERR_WORKSPACE
    assert call(ws=None) == mlra.ERR_INVALID_ARG


def test_project_query_validation():
    L = mlra.lib()
    d = _desc(d_model=64, d_cq=32)

    def call(desc=d, x=FAKE, wdq=FAKE, wuq=FAKE, wqr=FAKE, pos=FAKE, cq=FAKE, qc=FAKE, qr=FAKE, ws=FAKE,
             ws_bytes=16):
        return L.mlra_project_query(ctypes.byref(desc), x, wdq, wuq, wqr, pos, cq, qc, qr, ws,
                                    ctypes.c_size_t(ws_bytes), None)

    assert call(desc=_desc(d_model=64, d_cq=0)) == mlra.ERR_INVALID_ARG
    assert call(desc=_desc(d_model=64, d_cq=-8)) == mlra.ERR_INVALID_ARG
    assert call(desc=_desc(d_model=0, d_cq=32)) == mlra.ERR_INVALID_ARG
    assert call(desc=_desc(d_model=64, d_cq=36)) == mlra.ERR_UNSUPPORTED  # d_cq % 8
    assert call(desc=_desc(d_model=64, d_cq=32, d_h=12)) == mlra.ERR_UNSUPPORTED  # d_h % 8
    for k in ("x", "wdq", "wuq", "wqr", "pos", "cq", "qc", "qr"):
        assert call(**{k: None}) == mlra.ERR_INVALID_ARG, k
    for k in ("wdq", "wuq", "wqr"):
        assert call(**{k: ctypes.c_void_p(0x1004)}) == mlra.ERR_INVALID_ARG, k
    assert call() == mlra.ERR_WORKSPACE
    assert call(ws=None) == mlra.ERR_INVALID_ARG


def test_projection_scratch_is_part_of_the_workspace():
    """bf16 layers with a query path need split-K scratch beyond the decode's
    regions; fp32 layers (VALU path) need none."""
    L = mlra.lib()
    kw = dict(dtype="bf16", n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64)
    plain = _desc(**kw)
    layer = _desc(d_model=4096, d_cq=1536, **kw)
    assert L.mlra_workspace_bytes(ctypes.byref(layer), 10) > L.mlra_workspace_bytes(ctypes.byref(plain), 10)
    f32 = _desc(d_model=4096, d_cq=64)
    f32_plain = _desc()
    assert L.mlra_workspace_bytes(ctypes.byref(f32), 10) == L.mlra_workspace_bytes(ctypes.byref(f32_plain), 10)
