"""ctypes front end of the C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
the CPU-baseline leg of bench.py. The product path never imports this package.

Inputs are numpy arrays exactly as synth produces them (bf16 as uint16 bit
patterns, fp32 as float32); outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MLRA_ORACLE_LIB: another build of oracle.c to load (the sanitizer test's)
_LIB_PATH = os.environ.get("MLRA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8, FP8_BS = 0, 1, 2, 3
METHODS = {"MHA": 0, "MQA": 1, "GQA": 2, "MLA": 3, "MFA": 4, "TPA": 5, "MLRA": 6}


class OracleShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("d_c", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("blocks_per_head", ctypes.c_int32),
        ("d_r", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("d_model", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_double), ("out_scale", ctypes.c_double),
        ("cache_scale", ctypes.c_double),
        ("d_cq", ctypes.c_int32), ("rope_base", ctypes.c_double),
    ]


def build(force: bool = True) -> str:
    """Compiles oracle.c into liboracle.so with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, os.path.join(_HERE, "oracle.c"), "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        vp, ip, dp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)
        sp = ctypes.POINTER(OracleShape)
        for name in ("oracle_decode_unabsorbed", "oracle_decode_absorbed"):
            f = getattr(L, name)
            f.argtypes = [sp, vp, ip, ip, vp, vp, vp, vp, ctypes.c_int32, ip, ip, dp, dp]
            f.restype = None
        L.oracle_append.argtypes = [sp, vp, ip, ip, vp, vp, vp, vp]
        L.oracle_append.restype = None
        L.oracle_block_of.argtypes = [sp, ctypes.c_int32, ctypes.c_int32]
        L.oracle_block_of.restype = ctypes.c_int32
        L.oracle_row_index.argtypes = [sp, ip, ctypes.c_int32, ctypes.c_int32]
        L.oracle_row_index.restype = ctypes.c_int64
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_uint16
        L.oracle_rope.argtypes = [dp, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        L.oracle_rope.restype = None
        L.oracle_rope_key.argtypes = [sp, vp, vp, ip, dp]
        L.oracle_rope_key.restype = None
        L.oracle_project_query.argtypes = [sp, vp, vp, vp, vp, ip, dp, dp]
        L.oracle_project_query.restype = None
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_fp8_block_encode.argtypes = [vp, ctypes.c_int32, vp, ctypes.POINTER(ctypes.c_float)]
        L.oracle_fp8_block_encode.restype = None
        L.oracle_fp8_row_bytes.argtypes = [sp]
        L.oracle_fp8_row_bytes.restype = ctypes.c_int64
        L.oracle_cache_elems_per_token.argtypes = [ctypes.c_int32] * 7
        L.oracle_cache_elems_per_token.restype = ctypes.c_double
        L.oracle_cache_elems_per_device.argtypes = [ctypes.c_int32] * 9
        L.oracle_cache_elems_per_device.restype = ctypes.c_double
        L.oracle_decode_flops_bytes.argtypes = [ctypes.c_double] * 5 + [dp, dp]
        L.oracle_decode_flops_bytes.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int32
        L.oracle_set_num_threads.argtypes = [ctypes.c_int32]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def shape_of(inp, softmax_scale: Optional[float] = None, out_scale: Optional[float] = None) -> OracleShape:
    s = inp.shape
    return OracleShape(
        batch=s.batch, n_heads=s.n_heads, d_h=s.d_h, d_c=s.d_c, n_blocks=s.n_blocks,
        blocks_per_head=s.blocks_per_head, d_r=s.d_r, page_size=s.page_size,
        max_pages_per_seq=inp.max_pages_per_seq, d_model=s.d_model,
        dtype={"bf16": BF16, "f32": F32, "fp8": FP8, "fp8b": FP8_BS}[s.dtype],
        softmax_scale=s.softmax_scale if softmax_scale is None else softmax_scale,
        out_scale=s.out_scale if out_scale is None else out_scale,
        cache_scale=getattr(s, "cache_scale", 0.0), d_cq=getattr(s, "d_cq", 0),
        rope_base=getattr(s, "rope_base", 0.0))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _iptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _pairs(inp, pairs):
    if pairs is None:
        pairs = [(b, i) for b in range(inp.shape.batch) for i in range(inp.shape.n_heads)]
    pb = np.ascontiguousarray([p[0] for p in pairs], dtype=np.int32)
    ph = np.ascontiguousarray([p[1] for p in pairs], dtype=np.int32)
    return pb, ph


def _decode(fn, inp, pairs, pool, seq_lens, page_table, softmax_scale, out_scale):
    s = inp.shape
    pb, ph = _pairs(inp, pairs)
    out = np.zeros((pb.size, s.d_h), dtype=np.float64)
    lse = np.zeros((pb.size, s.blocks_per_head), dtype=np.float64)
    shp = shape_of(inp, softmax_scale, out_scale)
    pool = inp.pool if pool is None else pool
    seq_lens = inp.seq_lens if seq_lens is None else np.ascontiguousarray(seq_lens, dtype=np.int32)
    pt = inp.page_table if page_table is None else page_table
    fn(ctypes.byref(shp), _ptr(pool), _iptr(pt), _iptr(seq_lens), _ptr(inp.q_c), _ptr(inp.q_r),
       _ptr(inp.w_uk), _ptr(inp.w_uv), ctypes.c_int32(pb.size), _iptr(pb), _iptr(ph),
       out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
       lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out, lse


def decode_unabsorbed(inp, pairs: Optional[Sequence] = None, pool=None, seq_lens=None,
                      page_table=None, softmax_scale=None, out_scale=None):
    """Un-absorbed MLRA decode for (b, head) pairs (all pairs when None).
    Returns (out [npairs][d_h], lse [npairs][k]) in float64, lse in natural log."""
    return _decode(lib().oracle_decode_unabsorbed, inp, pairs, pool, seq_lens, page_table,
                   softmax_scale, out_scale)


def decode_absorbed(inp, pairs: Optional[Sequence] = None, pool=None, seq_lens=None,
                    page_table=None, softmax_scale=None, out_scale=None):
    return _decode(lib().oracle_decode_absorbed, inp, pairs, pool, seq_lens, page_table,
                   softmax_scale, out_scale)


def append(inp, pool: np.ndarray, c_out: bool = True):
    """Applies the latent append to `pool` in place; returns c_new [B][d_c]."""
    s = inp.shape
    shp = shape_of(inp)
    c_dtype = np.float32 if s.dtype in ("fp8", "fp8b") else pool.dtype  # fp8: the latent before encoding
    c = np.zeros((s.batch, s.d_c), dtype=c_dtype) if c_out else None
    lib().oracle_append(ctypes.byref(shp), _ptr(pool), _iptr(inp.page_table), _iptr(inp.positions),
                        _ptr(inp.x), _ptr(inp.w_dkv), _ptr(inp.kr_new), _ptr(c))
    return c


def fp8_block_encode(c: np.ndarray):
    """Block-scaled E4M3FN encoding of one block of fp32 latent values:
    returns (codes uint8 [n], scale float32)."""
    c = np.ascontiguousarray(c, dtype=np.float32)
    codes = np.zeros(c.size, dtype=np.uint8)
    sc = ctypes.c_float(0.0)
    lib().oracle_fp8_block_encode(_ptr(c), c.size, _ptr(codes), ctypes.byref(sc))
    return codes, np.float32(sc.value)


def fp8_row_bytes(inp) -> int:
    return int(lib().oracle_fp8_row_bytes(ctypes.byref(shape_of(inp))))


def block_of(inp, head: int, jj: int) -> int:
    shp = shape_of(inp)
    return int(lib().oracle_block_of(ctypes.byref(shp), head, jj))


def row_index(inp, b: int, t: int, page_table=None) -> int:
    shp = shape_of(inp)
    pt = inp.page_table if page_table is None else page_table
    return int(lib().oracle_row_index(ctypes.byref(shp), _iptr(pt), b, t))


def round_bf16(v: float) -> int:
    return int(lib().oracle_round_bf16(float(v)))


def rope(v: np.ndarray, pos: int, base: float = 10000.0) -> np.ndarray:
    """RoPE of one vector (a rotated copy)."""
    out = np.ascontiguousarray(v, dtype=np.float64).copy()
    lib().oracle_rope(out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), out.size, int(pos), float(base))
    return out


def rope_key(inp) -> np.ndarray:
    """k^R [B][d_r] for the new token of every sequence (inp.w_kr, inp.positions)."""
    s = inp.shape
    out = np.zeros((s.batch, s.d_r))
    lib().oracle_rope_key(ctypes.byref(shape_of(inp)), _ptr(inp.x), _ptr(inp.w_kr), _iptr(inp.positions),
                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def project_query(inp):
    """(q^C [B][h][d_h], q^R [B][h][d_r]) from x and the query-path weights."""
    s = inp.shape
    qc = np.zeros((s.batch, s.n_heads, s.d_h))
    qr = np.zeros((s.batch, s.n_heads, s.d_r))
    dp = ctypes.POINTER(ctypes.c_double)
    lib().oracle_project_query(ctypes.byref(shape_of(inp)), _ptr(inp.x), _ptr(inp.w_dq), _ptr(inp.w_uq),
                               _ptr(inp.w_qr), _iptr(inp.positions), qc.ctypes.data_as(dp),
                               qr.ctypes.data_as(dp))
    return qc, qr


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def e4m3_encode_array(a: np.ndarray) -> np.ndarray:
    """Encodes every fp32 value of `a` (a loop over the scalar oracle encoder)."""
    flat = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    enc = lib().oracle_e4m3_encode
    for i, v in enumerate(flat.tolist()):
        out[i] = enc(v)
    return out.reshape(np.shape(a))


def cache_elems_per_token(method: str, h=0, d_h=0, g=0, beta_kv=0, d_c=0, d_r=0) -> float:
    return lib().oracle_cache_elems_per_token(METHODS[method], h, d_h, g, beta_kv, d_c, d_r)


def cache_elems_per_device(method: str, h=0, d_h=0, g=0, beta_kv=0, d_c=0, d_r=0,
                           n_blocks=1, tp=1) -> float:
    return lib().oracle_cache_elems_per_device(METHODS[method], h, d_h, g, beta_kv, d_c, d_r,
                                               n_blocks, tp)


def decode_flops_bytes(n, heads_u, w_u, d_r, elem_bytes=2.0):
    f, b = ctypes.c_double(), ctypes.c_double()
    lib().oracle_decode_flops_bytes(float(n), float(heads_u), float(w_u), float(d_r),
                                    float(elem_bytes), ctypes.byref(f), ctypes.byref(b))
    return f.value, b.value


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))
