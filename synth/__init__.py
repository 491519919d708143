"""Seeded synthetic inputs for MLRA decode, shared by the tests and the benchmark.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic. Both the HIP path and the CPU oracle consume exactly the
arrays produced here (bf16 values are produced once, by round-to-nearest-even
from fp32, and handed to both sides as bit patterns).

Recipe (one generator per call, numpy Philox keyed by the seed, fixed order):
  1. sequence lengths (ragged workloads only), uniform integers, inclusive;
  2. the physical page permutation (Fisher-Yates inside numpy's permutation);
  3. the cache pool rows [c | k^R], N(0, 1);
  4. q^C [B][h][d_h] and q^R [B][h][d_r], N(0, 1);
  5. W^UK and W^UV [h][k][w][d_h], N(0, 1) / sqrt(w) (w = latent block width);
  6. append only: x [B][d_model] N(0, 1), W^DKV [d_model][d_c] N(0, 1) /
     sqrt(d_model), k^R_new [B][d_r] N(0, 1);
  7. append with a query width d_cq > 0 only (the steps on either side of the
     attention): W^KR [d_model][d_r] and W^DQ [d_model][d_cq] N(0, 1) /
     sqrt(d_model), W^UQ [h][d_cq][d_h] and W^QR [h][d_cq][d_r] N(0, 1) / sqrt(d_cq).
Rows of the pool that hold no token (the tail of each sequence's last page, a
spare page per sequence for the append target, and one guard page that unused
page-table entries point at) are filled with a NaN canary so that a kernel that
reads outside the sequence shows up as NaN in its outputs.

FP8 caches (dtype "fp8"): a row is d_c bytes of OCP E4M3FN codes followed by the
RoPE key as d_r bf16 values. Step 3 then draws each code's fields directly as
integers (sign uniform in {0, 1}, exponent field uniform in 3..7, mantissa field
uniform in 0..7: magnitudes between 1/16 and 1.875, RMS about 0.8 like the
N(0, 1) latents of the bf16 workloads; no zeros or NaN) and the RoPE
key N(0, 1) in bf16; every other array is bf16. The NaN canary is code 0x7F and
the bf16 NaN.

Block-scaled FP8 caches (dtype "fp8b"): each row further holds one fp32 scale
per latent block after the RoPE key, then zero bytes up to a multiple of 16.
Step 3 draws the codes and RoPE key as for "fp8", then each scale as
2^u, u uniform in [-3, 1) (fp32), so scales differ by up to 16x between tokens
and blocks. Canary rows hold NaN scales.

make_inputs(fp8_codes="full") instead draws every latent code uniformly from
all 254 finite E4M3FN codes (zero, both signed zeros, the subnormals 0x01..0x07
and the largest magnitude 448, code 0x7E), and scale_exp=(lo, hi) sets the
range of u for block scales.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
F32_NAN = np.float32(np.nan)


@dataclasses.dataclass
class Shape:
    batch: int
    n_heads: int
    d_h: int
    d_c: int
    n_blocks: int
    d_r: int
    dtype: str  # "f32", "bf16", "fp8" (E4M3FN latent codes, bf16 everything else) or
    # "fp8b" (as fp8, plus an fp32 scale per token and latent block in each row)
    page_size: int = 64
    blocks_per_head: int = 1
    d_model: int = 0
    paged: bool = True  # False: identity page layout (page table omitted)
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(d_h + d_r)
    out_scale: float = 0.0  # 0 -> 1/sqrt(blocks_per_head)
    cache_scale: float = 0.0  # fp8: latent value = decoded code x cache_scale (0 -> 1)
    d_cq: int = 0  # query-path width (0: no query-path weights drawn)
    rope_base: float = 0.0  # RoPE base (0 -> 10000)

    @property
    def w(self) -> int:
        return self.d_c // self.n_blocks

    @property
    def row(self) -> int:
        return self.d_c + self.d_r

    @property
    def row_bytes(self) -> int:
        if self.dtype == "fp8":
            return self.d_c + 2 * self.d_r
        if self.dtype == "fp8b":
            return (self.d_c + 2 * self.d_r + 4 * self.n_blocks + 15) // 16 * 16
        return self.row * (2 if self.dtype == "bf16" else 4)

    @property
    def is_fp8(self) -> bool:
        return self.dtype in ("fp8", "fp8b")

    @property
    def arrays_dtype(self) -> str:
        """Encoding of queries, weights and append inputs."""
        return "bf16" if self.is_fp8 else self.dtype

    @property
    def heads_per_block(self) -> int:
        return self.n_heads * self.blocks_per_head // self.n_blocks


# The five workloads: shapes, dtypes and length mixes.
WORKLOADS = {
    1: dict(name="tiny MLRA-4 fp32, B=1 h=8 d_c=64(4x16) d_r=16 d_h=16 n=256 contiguous",
            shape=Shape(batch=1, n_heads=8, d_h=16, d_c=64, n_blocks=4, d_r=16, dtype="f32",
                        paged=False),
            lengths=("fixed", 256)),
    2: dict(name="MLRA-4 bf16, B=32 h=64 d_h=128 d_c=512(4x128) d_r=64 ctx=8192 paged",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16"),
            lengths=("fixed", 8192)),
    3: dict(name="MLA (b=1) bf16, B=32 h=64 d_h=128 d_c=512 d_r=64 ctx=8192 paged",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16"),
            lengths=("fixed", 8192)),
    4: dict(name="MLRA-4 one TP rank share, bf16, B=64 h=16 d_h=128 d_c=128 d_r=64 ctx=32768 paged",
            shape=Shape(batch=64, n_heads=16, d_h=128, d_c=128, n_blocks=1, d_r=64, dtype="bf16"),
            lengths=("fixed", 32768)),
    5: dict(name="ragged MLRA-2 + append, bf16, B=16 h=64 d_c=512(2x256) d_r=64 L~U[1024,131072] d_model=4096",
            shape=Shape(batch=16, n_heads=64, d_h=128, d_c=512, n_blocks=2, d_r=64, dtype="bf16",
                        d_model=4096),
            lengths=("uniform_append", 1024, 131072)),
    # the FP8 latent cache of the next-step list: workload 2's shape with E4M3FN codes
    6: dict(name="MLRA-4 fp8-e4m3 cache (scale 1.25), B=32 h=64 d_h=128 d_c=512(4x128) d_r=64 ctx=8192 paged",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8",
                        cache_scale=1.25),
            lengths=("fixed", 8192)),
    # the whole layer step around the attention (next-step list): workload 2's
    # cache and heads plus the query path and the RoPE'd append of the new token
    7: dict(name="MLRA-4 step with query path + RoPE append, bf16, B=32 h=64 d_h=128 d_c=512(4x128) d_r=64 "
                 "ctx=8191+1 d_model=4096 d_cq=1536",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16",
                        d_model=4096, d_cq=1536),
            lengths=("uniform_append", 8191, 8191)),
    8: dict(name="MLRA-4 fp8-e4m3 cache, one scale per token and block, B=32 h=64 d_h=128 d_c=512(4x128) "
                 "d_r=64 ctx=8192 paged",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="fp8b"),
            lengths=("fixed", 8192)),
    9: dict(name="MLRA-4 reading B (k=2: each head attends 2 blocks), bf16, B=32 h=64 d_h=128 d_c=512(4x128) "
                 "d_r=64 ctx=8192 paged",
            shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16", blocks_per_head=2),
            lengths=("fixed", 8192)),
    10: dict(name="MLRA-4 reading B (k=4: each head attends all 4 blocks), bf16, B=32 h=64 d_h=128 "
                  "d_c=512(4x128) d_r=64 ctx=8192 paged",
             shape=Shape(batch=32, n_heads=64, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16", blocks_per_head=4),
             lengths=("fixed", 8192)),
    11: dict(name="MLRA-4 at the paper's model width h=24 (6 heads per block), bf16, B=32 d_h=128 "
                  "d_c=512(4x128) d_r=64 ctx=8192 paged",
             shape=Shape(batch=32, n_heads=24, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16"),
             lengths=("fixed", 8192)),
    12: dict(name="MLRA-4 reading B (k=4) at h=24 (24 heads per block), bf16, B=32 d_h=128 d_c=512(4x128) "
                  "d_r=64 ctx=8192 paged",
             shape=Shape(batch=32, n_heads=24, d_h=128, d_c=512, n_blocks=4, d_r=64, dtype="bf16", blocks_per_head=4),
             lengths=("fixed", 8192)),
    # one rank's share of MLRA-2 under 2-way tensor parallelism: one 256-wide
    # latent block and the RoPE key serving its 32 query heads, at the batch and
    # context of the MLRA-4 share above
    13: dict(name="MLRA-2 one TP-2 rank share, bf16, B=64 h=32 d_h=128 d_c=256 d_r=64 ctx=32768 paged",
             shape=Shape(batch=64, n_heads=32, d_h=128, d_c=256, n_blocks=1, d_r=64, dtype="bf16"),
             lengths=("fixed", 32768)),
    # MLA's share under the same 4-way tensor parallelism as workload 4: the
    # latent cannot be split, so each rank reads the whole 512 + 64 row for its
    # 16 heads (the one-GPU stand-in for the MLRA-against-MLA decode comparison)
    14: dict(name="MLA one TP-4 rank share, bf16, B=64 h=16 d_h=128 d_c=512 d_r=64 ctx=32768 paged",
             shape=Shape(batch=64, n_heads=16, d_h=128, d_c=512, n_blocks=1, d_r=64, dtype="bf16"),
             lengths=("fixed", 32768)),
}


def default_seed(workload: int) -> int:
    return 1000 + workload


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32).astype(np.uint32)
        nan = np.isnan(flat_in[s:s + step])
        u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        r = (u >> np.uint32(16)).astype(np.uint16)
        r[nan] = BF16_NAN
        flat_out[s:s + step] = r
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    shape: Shape
    seq_lens: np.ndarray  # int32 [B], lengths the decode attends
    page_table: Optional[np.ndarray]  # int32 [B][max_pages] or None (identity layout)
    max_pages_per_seq: int
    pool: np.ndarray  # [pages][page_size][row], uint16 (bf16 bits) or float32; fp8: uint8 [..][row_bytes]
    q_c: np.ndarray
    q_r: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    # append (None unless the workload appends one token per sequence)
    positions: Optional[np.ndarray] = None  # int32 [B], slot the new token goes to
    x: Optional[np.ndarray] = None
    w_dkv: Optional[np.ndarray] = None
    kr_new: Optional[np.ndarray] = None
    # query path and RoPE key (None unless the shape has d_cq > 0)
    w_kr: Optional[np.ndarray] = None
    w_dq: Optional[np.ndarray] = None
    w_uq: Optional[np.ndarray] = None
    w_qr: Optional[np.ndarray] = None

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


def _fp8_pool(rng: np.random.Generator, pages_rows, d_c: int, d_r: int, codes: str = "narrow") -> np.ndarray:
    """FP8 cache rows: E4M3FN code fields drawn as integers, then the bf16 RoPE key."""
    size = tuple(pages_rows) + (d_c,)
    if codes == "full":
        # every finite code: 0x00..0x7E and 0x80..0xFE (0x7F and 0xFF are NaN)
        v = rng.integers(0, 254, size=size, dtype=np.int32)
        lat = np.where(v < 127, v, v + 1).astype(np.uint8)
    else:
        sign = rng.integers(0, 2, size=size, dtype=np.uint8)
        expo = rng.integers(3, 8, size=size, dtype=np.uint8)
        mant = rng.integers(0, 8, size=size, dtype=np.uint8)
        lat = (sign << np.uint8(7)) | (expo << np.uint8(3)) | mant
    rope = _normal(rng, tuple(pages_rows) + (d_r,), 1.0, "bf16")
    pool = np.empty(tuple(pages_rows) + (d_c + 2 * d_r,), dtype=np.uint8)
    pool[..., :d_c] = lat
    pool[..., d_c:] = rope.view(np.uint8).reshape(tuple(pages_rows) + (2 * d_r,))
    return pool


def _fp8b_pool(rng: np.random.Generator, pages_rows, shape: "Shape", codes: str = "narrow",
               scale_exp=(-3.0, 1.0)) -> np.ndarray:
    """Block-scaled FP8 rows: the fp8 row, n_blocks fp32 scales 2^u, zero pad."""
    d_c, d_r, nb = shape.d_c, shape.d_r, shape.n_blocks
    base = _fp8_pool(rng, pages_rows, d_c, d_r, codes)
    u = rng.uniform(float(scale_exp[0]), float(scale_exp[1]), size=tuple(pages_rows) + (nb,))
    scales = np.exp2(u).astype(np.float32)
    pool = np.zeros(tuple(pages_rows) + (shape.row_bytes,), dtype=np.uint8)
    pool[..., :d_c + 2 * d_r] = base
    pool[..., d_c + 2 * d_r:d_c + 2 * d_r + 4 * nb] = scales.view(np.uint8).reshape(tuple(pages_rows) + (4 * nb,))
    return pool


def _FP8_NAN_ROW(d_c: int, d_r: int, row_bytes: int = 0, n_scales: int = 0) -> np.ndarray:
    row = np.zeros(max(row_bytes, d_c + 2 * d_r), dtype=np.uint8)
    row[:d_c] = 0x7F
    row[d_c:d_c + 2 * d_r] = np.full(d_r, BF16_NAN, dtype=np.uint16).view(np.uint8)
    row[d_c + 2 * d_r:d_c + 2 * d_r + 4 * n_scales] = np.full(n_scales, F32_NAN, dtype=np.float32).view(np.uint8)
    return row


def _normal(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def make_inputs(shape: Shape, lengths, seed: int, canary: bool = True,
                pool_copies: int = 1, fp8_codes: str = "narrow", scale_exp=(-3.0, 1.0)) -> Inputs:
    """Draws one workload.

    lengths: ("fixed", n) | ("uniform", lo, hi) | ("uniform_append", lo, hi) |
             ("list", [n_0, ...]) | ("list_append", [L_0, ...]).
    The *_append kinds draw/hold pre-append lengths L_b; the new token goes to
    slot L_b and the decode attends n_b = L_b + 1 tokens.
    pool_copies > 1 returns a list of independent pools in Inputs.pool (same
    page table), for benchmarks that rotate cache instances.
    fp8_codes ("narrow" | "full") and scale_exp: FP8 code and block-scale
    draws (module docstring).
    """
    rng = np.random.Generator(np.random.Philox(seed))
    B, P = shape.batch, shape.page_size
    kind = lengths[0]
    append = kind.endswith("_append")
    if kind in ("fixed",):
        pre = np.full(B, int(lengths[1]), dtype=np.int64)
    elif kind in ("uniform", "uniform_append"):
        pre = rng.integers(int(lengths[1]), int(lengths[2]), size=B, endpoint=True).astype(np.int64)
    elif kind in ("list", "list_append"):
        pre = np.asarray(lengths[1], dtype=np.int64)
        assert pre.shape == (B,)
    else:
        raise ValueError(kind)
    n = pre + 1 if append else pre
    pages_per_seq = np.array([max(1, math.ceil(int(v) / P)) for v in n], dtype=np.int64)
    if not shape.paged:
        # identity layout: page p of sequence b is b * max_pages + p
        max_pages = int(pages_per_seq.max())
        n_pages = B * max_pages
        page_table = None
        phys_of = [np.arange(b * max_pages, b * max_pages + pages_per_seq[b]) for b in range(B)]
        guard = None
    else:
        max_pages = int(pages_per_seq.max())
        used = int(pages_per_seq.sum())
        n_pages = used + 1  # + one guard page
        perm = rng.permutation(used).astype(np.int64)
        page_table = np.full((B, max_pages), used, dtype=np.int32)  # unused -> guard page
        phys_of = []
        off = 0
        for b in range(B):
            k = int(pages_per_seq[b])
            page_table[b, :k] = perm[off:off + k]
            phys_of.append(perm[off:off + k])
            off += k
        guard = used
    row = shape.row
    pools = []
    for _ in range(pool_copies):
        if shape.dtype == "fp8":
            pool = _fp8_pool(rng, (n_pages, P), shape.d_c, shape.d_r, fp8_codes)
            nanv = _FP8_NAN_ROW(shape.d_c, shape.d_r)
        elif shape.dtype == "fp8b":
            pool = _fp8b_pool(rng, (n_pages, P), shape, fp8_codes, scale_exp)
            nanv = _FP8_NAN_ROW(shape.d_c, shape.d_r, shape.row_bytes, shape.n_blocks)
        else:
            pool = _normal(rng, (n_pages, P, row), 1.0, shape.dtype)
            nanv = BF16_NAN if shape.dtype == "bf16" else F32_NAN
        if canary:
            for b in range(B):
                valid = int(n[b]) - (1 if append else 0)  # rows written so far
                for pi, page in enumerate(phys_of[b]):
                    s0 = valid - pi * P
                    if s0 < P:
                        pool[page, max(0, s0):, :] = nanv
            if guard is not None:
                pool[guard] = nanv
            elif not shape.paged:
                for b in range(B):
                    for pi in range(int(pages_per_seq[b]), max_pages):
                        pool[b * max_pages + pi] = nanv
        pools.append(pool)
    H, DH, DR, K, W = shape.n_heads, shape.d_h, shape.d_r, shape.blocks_per_head, shape.w
    adt = shape.arrays_dtype
    q_c = _normal(rng, (B, H, DH), 1.0, adt)
    q_r = _normal(rng, (B, H, DR), 1.0, adt)
    w_uk = _normal(rng, (H, K, W, DH), 1.0 / math.sqrt(W), adt)
    w_uv = _normal(rng, (H, K, W, DH), 1.0 / math.sqrt(W), adt)
    inp = Inputs(shape=shape, seq_lens=n.astype(np.int32), page_table=page_table,
                 max_pages_per_seq=max_pages, pool=pools[0] if pool_copies == 1 else pools,
                 q_c=q_c, q_r=q_r, w_uk=w_uk, w_uv=w_uv)
    if append:
        DM = shape.d_model
        inp.positions = pre.astype(np.int32)
        inp.x = _normal(rng, (B, DM), 1.0, adt)
        inp.w_dkv = _normal(rng, (DM, shape.d_c), 1.0 / math.sqrt(DM), adt)
        inp.kr_new = _normal(rng, (B, DR), 1.0, adt)
        if shape.d_cq > 0:
            DQ = shape.d_cq
            inp.w_kr = _normal(rng, (DM, DR), 1.0 / math.sqrt(DM), adt)
            inp.w_dq = _normal(rng, (DM, DQ), 1.0 / math.sqrt(DM), adt)
            inp.w_uq = _normal(rng, (H, DQ, DH), 1.0 / math.sqrt(DQ), adt)
            inp.w_qr = _normal(rng, (H, DQ, DR), 1.0 / math.sqrt(DQ), adt)
    return inp


def workload_inputs(workload: int, seed: Optional[int] = None, **kw) -> Inputs:
    w = WORKLOADS[workload]
    return make_inputs(w["shape"], w["lengths"], default_seed(workload) if seed is None else seed, **kw)
