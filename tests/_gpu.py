"""Helpers of the GPU tests: upload synth inputs, run the HIP path through the
C ABI, and compare with the oracle to the stated tolerances."""
from __future__ import annotations

import numpy as np

import compressed_kv_cache_mlra_amd as mlra
import synth


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        h = t.from_numpy(a.view(np.int16)).view(t.bfloat16)
    else:
        h = t.from_numpy(a)
    return h.to("cuda")


def from_dev_bits(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


class GpuProblem:
    """One decode problem resident on the GPU."""

    def __init__(self, inp: synth.Inputs, pool=None):
        t = torch()
        s = inp.shape
        self.inp = inp
        pool_np = inp.pool if pool is None else pool
        self.pool = to_dev(pool_np)
        self.page_table = None if inp.page_table is None else to_dev(inp.page_table)
        self.seq_lens = to_dev(inp.seq_lens)
        self.q_c, self.q_r = to_dev(inp.q_c), to_dev(inp.q_r)
        self.w_uk, self.w_uv = to_dev(inp.w_uk), to_dev(inp.w_uv)
        self.desc = mlra.make_desc(
            batch=s.batch, n_heads=s.n_heads, d_h=s.d_h, d_c=s.d_c, n_blocks=s.n_blocks, d_r=s.d_r,
            max_pages_per_seq=inp.max_pages_per_seq, num_pages=pool_np.shape[0], dtype=s.dtype,
            page_size=s.page_size, blocks_per_head=s.blocks_per_head, d_model=s.d_model,
            softmax_scale=s.softmax_scale, out_scale=s.out_scale, cache_scale=s.cache_scale,
            d_cq=s.d_cq, rope_base=s.rope_base)
        self.max_seq_len = inp.max_seq_len
        self.ws = mlra.alloc_workspace(self.desc, self.max_seq_len)
        self.out = t.empty((s.batch, s.n_heads, s.d_h), dtype=t.float32, device="cuda")
        self.lse = t.empty((s.batch, s.n_heads, s.blocks_per_head), dtype=t.float32, device="cuda")
        if inp.x is not None:
            self.positions = to_dev(inp.positions)
            self.x, self.w_dkv, self.kr_new = to_dev(inp.x), to_dev(inp.w_dkv), to_dev(inp.kr_new)
            c_dtype = t.float32 if s.is_fp8 else self.pool.dtype  # fp8: latent before encoding
            self.c_out = t.empty((s.batch, s.d_c), dtype=c_dtype, device="cuda")

    def append(self, stream=None):
        mlra.append_latent(self.desc, self.pool, self.page_table, self.positions, self.x, self.w_dkv,
                           self.kr_new, self.c_out, self.ws, stream)

    def step(self, stream=None):
        mlra.decode(self.desc, self.pool, self.page_table, self.seq_lens, self.max_seq_len, self.q_c,
                    self.q_r, self.w_uk, self.ws, stream)
        mlra.combine(self.desc, self.ws, self.w_uv, self.out, self.lse, stream)

    def step_one_call(self, stream=None):
        """The whole step through mlra_decode_step."""
        mlra.decode_step(self.desc, self.pool, self.page_table, self.seq_lens, self.max_seq_len, self.q_c,
                         self.q_r, self.w_uk, self.w_uv, self.out, self.ws, self.lse, stream)

    def run(self, stream=None, one_call=False):
        (self.step_one_call if one_call else self.step)(stream)
        torch().cuda.synchronize()
        return self.out.cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def check_outputs(gpu: np.ndarray, ref: np.ndarray, dtype: str, what: str = "out"):
    """bf16 and FP8 caches: max |g - r| / RMS(r) <= 2e-2, the RMS taken over
    every output compared; fp32: max |g - r| / max(|r|, RMS(r)) <= 1e-5.

    The FP8 bar equals the bf16 one, fixed before any run: the oracle decodes
    the same E4M3 codes exactly, and the FP8 kernels round less than the bf16
    ones (fp16 query and weights P, 11 significant bits, against the bf16
    path's P at 8 bits; a 16-bit query on both)."""
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    r = rms(ref)
    if dtype in ("bf16", "fp8", "fp8b"):
        err = float(np.max(np.abs(gpu - ref))) / max(r, 1e-30)
        assert err <= 2e-2, f"{what}: max err / rms = {err:.3e}"
    else:
        err = float(np.max(np.abs(gpu - ref) / np.maximum(np.abs(ref), r)))
        assert err <= 1e-5, f"{what}: max rel err = {err:.3e}"
    return err


def check_lse(gpu: np.ndarray, ref: np.ndarray, dtype: str):
    finite = np.isfinite(ref)
    assert np.array_equal(finite, np.isfinite(gpu))
    assert np.all(gpu[~finite] == ref[~finite])
    if finite.any():
        d = np.abs(gpu[finite] - ref[finite])
        tol = 5e-2 if dtype in ("bf16", "fp8", "fp8b") else 1e-5 * max(1.0, float(np.max(np.abs(ref[finite]))))
        assert float(np.max(d)) <= tol, f"lse: max abs err {float(np.max(d)):.3e}"


def plan_geometry(shape: "synth.Shape"):
    """(work units, tokens per tile) of the attention launch for this shape on
    the current device, read from the workspace header after planning a
    single long sequence (header: magic, flags, tiles, units, tile tokens)."""
    t = torch()
    s = synth.Shape(**{**shape.__dict__, "batch": 1, "d_model": 0, "d_cq": 0})
    n = 1 << 20
    desc = mlra.make_desc(batch=1, n_heads=s.n_heads, d_h=s.d_h, d_c=s.d_c, n_blocks=s.n_blocks, d_r=s.d_r,
                          max_pages_per_seq=n // s.page_size, num_pages=1, dtype=s.dtype, page_size=s.page_size,
                          blocks_per_head=s.blocks_per_head, cache_scale=s.cache_scale)
    ws = mlra.alloc_workspace(desc, n)
    et = t.float32 if s.dtype == "f32" else t.bfloat16
    q_c = t.zeros((1, s.n_heads, s.d_h), dtype=et, device="cuda")
    q_r = t.zeros((1, s.n_heads, max(s.d_r, 1)), dtype=et, device="cuda")
    w_uk = t.zeros((s.n_heads, s.blocks_per_head, s.w, s.d_h), dtype=et, device="cuda")
    lens = t.tensor([n], dtype=t.int32, device="cuda")
    mlra.absorb_query(desc, lens, q_c, q_r, w_uk, ws)
    t.cuda.synchronize()
    hdr = ws[:32].cpu().numpy().view(np.int32)
    return int(hdr[3]), int(hdr[4])


def tile_begin(u: int, n_tiles: int, units: int) -> int:
    """First tile of work unit u (the plan's balanced split)."""
    return (u * n_tiles) // units
