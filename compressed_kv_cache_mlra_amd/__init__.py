"""Python binding of libmlra: MLRA decode attention over a paged latent cache
on AMD Instinct MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libmlra.so,
reached through its C ABI (include/mlra.h) with ctypes. PyTorch provides device
memory and streams. There is no CPU fallback: importing works anywhere, but
every call raises if the library is not built or no GPU is present.

Entry points (same names as the C ABI, without the mlra_ prefix):
  workspace_bytes, append_latent, absorb_query, attend, decode, combine,
  decode_step, decode_step_noalloc, rope_key, project_query, project_token,
  read_flags, status_string; and the measurement helper stream_read.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmlra.so")

F32, BF16, FP8_E4M3, FP8_E4M3_BS = 0, 1, 2, 3
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5
FLAG_BAD_PAGE = 1
ABI_VERSION = 9
NOALLOC_SCRATCH_BYTES = 32 << 20  # MLRA_NOALLOC_SCRATCH_BYTES


class MlraError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class MlraDesc(ctypes.Structure):
    """Mirror of mlra_desc (include/mlra.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("d_c", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("blocks_per_head", ctypes.c_int32),
        ("d_r", ctypes.c_int32), ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("d_model", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("out_scale", ctypes.c_float),
        ("cache_scale", ctypes.c_float), ("d_cq", ctypes.c_int32), ("rope_base", ctypes.c_float),
    ]


def make_desc(batch, n_heads, d_h, d_c, n_blocks, d_r, max_pages_per_seq, num_pages, dtype,
              page_size=64, blocks_per_head=1, d_model=0, softmax_scale=0.0, out_scale=0.0,
              cache_scale=0.0, d_cq=0, rope_base=0.0) -> MlraDesc:
    if isinstance(dtype, str):
        dtype = {"f32": F32, "bf16": BF16, "fp8": FP8_E4M3, "fp8b": FP8_E4M3_BS}[dtype]
    return MlraDesc(batch=batch, n_heads=n_heads, d_h=d_h, d_c=d_c, n_blocks=n_blocks,
                    blocks_per_head=blocks_per_head, d_r=d_r, page_size=page_size,
                    max_pages_per_seq=max_pages_per_seq, num_pages=num_pages, d_model=d_model,
                    dtype=dtype, softmax_scale=softmax_scale, out_scale=out_scale,
                    cache_scale=cache_scale, d_cq=d_cq, rope_base=rope_base)


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libmlra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with compressed_kv_cache_mlra_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, ip, dp = ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(MlraDesc)
        L.mlra_abi_version.restype = ctypes.c_int
        L.mlra_status_string.argtypes = [ctypes.c_int]
        L.mlra_status_string.restype = ctypes.c_char_p
        L.mlra_workspace_bytes.argtypes = [dp, ctypes.c_int32]
        L.mlra_workspace_bytes.restype = ctypes.c_size_t
        L.mlra_append_latent.argtypes = [dp, vp, ip, ip, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mlra_project_token.argtypes = [dp, vp, ip, vp, ip, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        L.mlra_absorb_query.argtypes = [dp, ip, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mlra_attend.argtypes = [dp, vp, ip, vp, ctypes.c_size_t, vp]
        L.mlra_attend_timed.argtypes = [dp, vp, ip, vp, ctypes.c_size_t, vp, vp, vp]
        L.mlra_decode.argtypes = [dp, vp, ip, ip, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.mlra_combine.argtypes = [dp, vp, ctypes.c_size_t, vp, vp, vp, vp]
        L.mlra_decode_step.argtypes = [dp, vp, ip, ip, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.c_size_t, vp]
        L.mlra_decode_step_noalloc.argtypes = [dp, vp, ip, ip, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp]
        L.mlra_read_flags.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_uint32), vp]
        L.mlra_stream_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, vp]
        L.mlra_rope_key.argtypes = [dp, vp, vp, ip, vp, vp, ctypes.c_size_t, vp]
        L.mlra_project_query.argtypes = [dp, vp, vp, vp, vp, ip, vp, vp, vp, vp, ctypes.c_size_t, vp]
        for f in ("mlra_append_latent", "mlra_absorb_query", "mlra_attend", "mlra_attend_timed", "mlra_decode",
                  "mlra_combine", "mlra_decode_step", "mlra_decode_step_noalloc", "mlra_read_flags",
                  "mlra_stream_read", "mlra_rope_key", "mlra_project_query", "mlra_project_token"):
            getattr(L, f).restype = ctypes.c_int
        if L.mlra_abi_version() != ABI_VERSION:
            raise ImportError("libmlra ABI version mismatch; rebuild the library")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().mlra_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise MlraError(status, where)


# ----------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def _elem_dtype(desc: MlraDesc):
    """Element type of queries, weights and append inputs (bf16 for FP8 caches)."""
    torch = _torch()
    return torch.float32 if desc.dtype == F32 else torch.bfloat16


def _ptr(t, desc: Optional[MlraDesc] = None, kind: str = "float", name: str = "tensor",
         numel: Optional[int] = None, nullable: bool = False):
    """Device pointer of a contiguous CUDA tensor, after checking dtype and size."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if kind == "float":
        want = _elem_dtype(desc)
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}, got {t.dtype}")
    elif kind == "int32":
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32, got {t.dtype}")
    elif kind == "f32":
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")
    elif kind == "bytes":
        pass
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def workspace_bytes(desc: MlraDesc, max_seq_len: int) -> int:
    n = lib().mlra_workspace_bytes(ctypes.byref(desc), int(max_seq_len))
    if n == 0:
        raise MlraError(ERR_INVALID_ARG, "workspace_bytes")
    return int(n)


def alloc_workspace(desc: MlraDesc, max_seq_len: int, device="cuda"):
    torch = _torch()
    return torch.empty(workspace_bytes(desc, max_seq_len), dtype=torch.uint8, device=device)


def _row(desc):
    return desc.d_c + desc.d_r


def _pool_ptr(pool, desc):
    """The cache pool: elements of desc.dtype, or bytes for FP8 caches."""
    if desc.dtype in (FP8_E4M3, FP8_E4M3_BS):
        return _ptr(pool, kind="bytes", name="pool",
                    numel=desc.num_pages * desc.page_size * fp8_row_bytes(desc) // pool.element_size())
    return _ptr(pool, desc, name="pool", numel=desc.num_pages * desc.page_size * _row(desc))


def fp8_row_bytes(desc):
    """Bytes of one FP8 cache row: codes, bf16 k^R, (block-scaled) one fp32
    scale per block, rounded up to a multiple of 16."""
    rb = desc.d_c + 2 * desc.d_r + (4 * desc.n_blocks if desc.dtype == FP8_E4M3_BS else 0)
    return (rb + 15) // 16 * 16


def _w(desc):
    return desc.d_c // desc.n_blocks


def append_latent(desc, pool, page_table, positions, x, w_dkv, kr_new, c_out, workspace, stream=None):
    B = desc.batch
    _check(lib().mlra_append_latent(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=B * desc.max_pages_per_seq, nullable=True),
        _ptr(positions, kind="int32", name="positions", numel=B),
        _ptr(x, desc, name="x", numel=B * desc.d_model),
        _ptr(w_dkv, desc, name="w_dkv", numel=desc.d_model * desc.d_c),
        _ptr(kr_new, desc, name="kr_new", numel=B * desc.d_r, nullable=desc.d_r == 0),
        _c_out_ptr(c_out, desc),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "append_latent")


def _c_out_ptr(c_out, desc):
    """c_out: fp32 for FP8 caches (the latent before encoding), else the element type; optional."""
    if desc.dtype in (FP8_E4M3, FP8_E4M3_BS):
        return _ptr(c_out, kind="f32", name="c_out", numel=desc.batch * desc.d_c, nullable=True)
    return _ptr(c_out, desc, name="c_out", numel=desc.batch * desc.d_c, nullable=True)


def project_token(desc, x, positions, pool, page_table, w_dkv, w_kr, kr_out, c_out, w_dq, w_uq, w_qr, c_q, q_c,
                  q_r, workspace, stream=None):
    """rope_key + append_latent + project_query of the new token in one call."""
    B, H, DQ = desc.batch, desc.n_heads, desc.d_cq
    no_q, no_r = DQ == 0, desc.d_r == 0
    _check(lib().mlra_project_token(
        ctypes.byref(desc),
        _ptr(x, desc, name="x", numel=B * desc.d_model),
        _ptr(positions, kind="int32", name="positions", numel=B),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=B * desc.max_pages_per_seq, nullable=True),
        _ptr(w_dkv, desc, name="w_dkv", numel=desc.d_model * desc.d_c),
        _ptr(w_kr, desc, name="w_kr", numel=desc.d_model * desc.d_r, nullable=no_r),
        _ptr(kr_out, desc, name="kr_out", numel=B * desc.d_r, nullable=no_r),
        _c_out_ptr(c_out, desc),
        _ptr(w_dq, desc, name="w_dq", numel=desc.d_model * DQ, nullable=no_q),
        _ptr(w_uq, desc, name="w_uq", numel=H * DQ * desc.d_h, nullable=no_q),
        _ptr(w_qr, desc, name="w_qr", numel=H * DQ * desc.d_r, nullable=no_q or no_r),
        _ptr(c_q, kind="f32", name="c_q", numel=B * DQ, nullable=no_q),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h, nullable=no_q),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=no_q or no_r),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "project_token")


def rope_key(desc, x, w_kr, positions, kr_out, workspace, stream=None):
    """kr_out[b] = RoPE(x[b] W^KR, positions[b]) (feeds append_latent's kr_new)."""
    B = desc.batch
    _check(lib().mlra_rope_key(
        ctypes.byref(desc),
        _ptr(x, desc, name="x", numel=B * desc.d_model),
        _ptr(w_kr, desc, name="w_kr", numel=desc.d_model * desc.d_r),
        _ptr(positions, kind="int32", name="positions", numel=B),
        _ptr(kr_out, desc, name="kr_out", numel=B * desc.d_r),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "rope_key")


def project_query(desc, x, w_dq, w_uq, w_qr, positions, c_q, q_c, q_r, workspace, stream=None):
    """c_q = x W^DQ (fp32), q_c[:, i] = c_q W^UQ[i], q_r[:, i] = RoPE(c_q W^QR[i])."""
    B, H, DQ = desc.batch, desc.n_heads, desc.d_cq
    no_r = desc.d_r == 0
    _check(lib().mlra_project_query(
        ctypes.byref(desc),
        _ptr(x, desc, name="x", numel=B * desc.d_model),
        _ptr(w_dq, desc, name="w_dq", numel=desc.d_model * DQ),
        _ptr(w_uq, desc, name="w_uq", numel=H * DQ * desc.d_h),
        _ptr(w_qr, desc, name="w_qr", numel=H * DQ * desc.d_r, nullable=no_r),
        _ptr(positions, kind="int32", name="positions", numel=B, nullable=no_r),
        _ptr(c_q, kind="f32", name="c_q", numel=B * DQ),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=no_r),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "project_query")


def absorb_query(desc, seq_lens, q_c, q_r, w_uk, workspace, stream=None):
    B, H, K = desc.batch, desc.n_heads, desc.blocks_per_head
    _check(lib().mlra_absorb_query(
        ctypes.byref(desc),
        _ptr(seq_lens, kind="int32", name="seq_lens", numel=B),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=desc.d_r == 0),
        _ptr(w_uk, desc, name="w_uk", numel=H * K * _w(desc) * desc.d_h),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "absorb_query")


def attend(desc, pool, page_table, workspace, stream=None):
    _check(lib().mlra_attend(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=desc.batch * desc.max_pages_per_seq,
             nullable=True),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "attend")


def attend_timed(desc, pool, page_table, workspace, start, stop, stream=None):
    """Measurement helper: attend, with the kernel's own start and stop times
    recorded into the torch.cuda.Event pair (start, stop) by its dispatch."""
    for e in (start, stop):
        if e.cuda_event == 0:  # torch creates the HIP event on its first record
            e.record(_torch().cuda.current_stream() if stream is None else stream)
    _check(lib().mlra_attend_timed(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=desc.batch * desc.max_pages_per_seq,
             nullable=True),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event),
        _stream(stream)), "attend_timed")


def decode(desc, pool, page_table, seq_lens, max_seq_len, q_c, q_r, w_uk, workspace, stream=None):
    B, H, K = desc.batch, desc.n_heads, desc.blocks_per_head
    _check(lib().mlra_decode(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=B * desc.max_pages_per_seq, nullable=True),
        _ptr(seq_lens, kind="int32", name="seq_lens", numel=B), ctypes.c_int32(int(max_seq_len)),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=desc.d_r == 0),
        _ptr(w_uk, desc, name="w_uk", numel=H * K * _w(desc) * desc.d_h),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "decode")


def combine(desc, workspace, w_uv, out, lse=None, stream=None):
    B, H, K = desc.batch, desc.n_heads, desc.blocks_per_head
    _check(lib().mlra_combine(
        ctypes.byref(desc),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _ptr(w_uv, desc, name="w_uv", numel=H * K * _w(desc) * desc.d_h),
        _ptr(out, kind="f32", name="out", numel=B * H * desc.d_h),
        _ptr(lse, kind="f32", name="lse", numel=B * H * K, nullable=True),
        _stream(stream)), "combine")


def decode_step(desc, pool, page_table, seq_lens, max_seq_len, q_c, q_r, w_uk, w_uv, out, workspace, lse=None,
                stream=None):
    """absorb_query + attend + combine in one call."""
    B, H, K = desc.batch, desc.n_heads, desc.blocks_per_head
    _check(lib().mlra_decode_step(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=B * desc.max_pages_per_seq, nullable=True),
        _ptr(seq_lens, kind="int32", name="seq_lens", numel=B), ctypes.c_int32(int(max_seq_len)),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=desc.d_r == 0),
        _ptr(w_uk, desc, name="w_uk", numel=H * K * _w(desc) * desc.d_h),
        _ptr(w_uv, desc, name="w_uv", numel=H * K * _w(desc) * desc.d_h),
        _ptr(out, kind="f32", name="out", numel=B * H * desc.d_h),
        _ptr(lse, kind="f32", name="lse", numel=B * H * K, nullable=True),
        _ptr(workspace, kind="bytes", name="workspace"), ctypes.c_size_t(workspace.numel()),
        _stream(stream)), "decode_step")


def decode_step_noalloc(desc, pool, page_table, seq_lens, max_seq_len, q_c, q_r, w_uk, w_uv, out, lse=None,
                        stream=None):
    """decode_step with the library's static device scratch as its workspace
    (for callers that cannot allocate; calls that overlap on one GPU race)."""
    B, H, K = desc.batch, desc.n_heads, desc.blocks_per_head
    _check(lib().mlra_decode_step_noalloc(
        ctypes.byref(desc),
        _pool_ptr(pool, desc),
        _ptr(page_table, kind="int32", name="page_table", numel=B * desc.max_pages_per_seq, nullable=True),
        _ptr(seq_lens, kind="int32", name="seq_lens", numel=B), ctypes.c_int32(int(max_seq_len)),
        _ptr(q_c, desc, name="q_c", numel=B * H * desc.d_h),
        _ptr(q_r, desc, name="q_r", numel=B * H * desc.d_r, nullable=desc.d_r == 0),
        _ptr(w_uk, desc, name="w_uk", numel=H * K * _w(desc) * desc.d_h),
        _ptr(w_uv, desc, name="w_uv", numel=H * K * _w(desc) * desc.d_h),
        _ptr(out, kind="f32", name="out", numel=B * H * desc.d_h),
        _ptr(lse, kind="f32", name="lse", numel=B * H * K, nullable=True),
        _stream(stream)), "decode_step_noalloc")


def read_flags(workspace, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().mlra_read_flags(_ptr(workspace, kind="bytes", name="workspace"),
                                 ctypes.c_size_t(workspace.numel()), ctypes.byref(v), _stream(stream)),
           "read_flags")
    return int(v.value)


@dataclasses.dataclass
class DecodeStep:
    """Convenience wrapper holding a descriptor and a workspace for repeated
    decode steps: append (optional) -> absorb + attend -> combine."""
    desc: MlraDesc
    workspace: object
    max_seq_len: int

    @classmethod
    def create(cls, desc: MlraDesc, max_seq_len: int, device="cuda"):
        return cls(desc, alloc_workspace(desc, max_seq_len, device), int(max_seq_len))

    def __call__(self, pool, page_table, seq_lens, q_c, q_r, w_uk, w_uv, out, lse=None, stream=None):
        decode(self.desc, pool, page_table, seq_lens, self.max_seq_len, q_c, q_r, w_uk,
               self.workspace, stream)
        combine(self.desc, self.workspace, w_uv, out, lse, stream)
        return out


def stream_read(src, sink, stream=None):
    """Measurement helper: reads all of `src` (a GPU tensor whose size in bytes
    is a multiple of 16) once, as the attention reads the cache; `sink` is a
    GPU tensor of at least 16 KiB that receives a checksum."""
    nbytes = src.numel() * src.element_size()
    _check(lib().mlra_stream_read(
        _ptr(src, kind="bytes", name="src"), ctypes.c_size_t(nbytes),
        _ptr(sink, kind="bytes", name="sink"), ctypes.c_size_t(sink.numel() * sink.element_size()),
        _stream(stream)), "stream_read")


def default_softmax_scale(desc: MlraDesc) -> float:
    return desc.softmax_scale if desc.softmax_scale > 0 else 1.0 / math.sqrt(desc.d_h + desc.d_r)
