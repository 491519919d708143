// Split-K latent attention over the paged cache, bf16 MFMA path for gfx950.
//
// What it computes (per work unit, per query head i and attended block j):
//   l_t = q~_{i,j} . c_{t,j} + q^R~_i . k^R_t          (base-2 logits; the
//         query was absorbed into latent space, lesty.tech section 5)
//   m = max_t l_t,  l = sum_t 2^(l_t - m),  o~ = sum_t 2^(l_t - m) c_{t,j}
// over the unit's tokens, written as (m, l, o~) partials for the combine.
//
// How (MI355X-first):
//  - One workgroup per compute unit streams a contiguous range of tiles of TT
//    tokens. While tile x is computed from LDS, tile x+1 goes from registers
//    into the other LDS buffer and tile x+2 is in flight from HBM into those
//    registers (coalesced 16-byte global loads). One barrier per tile publishes
//    the new tile and retires the old buffer. Rows past the sequence end are
//    written as zeros on the way in. (Register staging rather than LDS-DMA:
//    on gfx950 the DMA writes into LDS stall the MFMA operand reads.)
//  - Every wave owns one (latent block, 16-head tile) task; all waves read the
//    same LDS tile, so k^R and (for MLA) the latent are fetched from HBM once
//    and shared by every head.
//  - Scores: S^T[token][head] = K_ext[token] . Q_ext[head] with
//    v_mfma_f32_16x16x32_bf16 (tokens as MFMA rows). Its output layout puts
//    four tokens of one head in each lane, which is exactly the B-operand
//    layout of the value product, so P never leaves registers. Per-head max
//    and sum reduce across the four lanes of a head with v_permlane16/32_swap.
//  - Precision: the latent part of the absorbed query enters the score MFMAs
//    as two bf16 parts (hi + lo, about 16 significant bits); the RoPE part is
//    the bf16 query as given; the fp32 sums are then scaled by softmax_scale
//    log2(e). (One bf16 rounding of the absorbed query moves the outputs by up
//    to ~2% of their RMS on short contexts; P stays bf16, ~0.8%.)
//  - Values: O^T[col][head] += C^T[col][token] P^T[token][head], again
//    16x16x32 bf16 MFMA; C^T operands come from 128-bit LDS reads of 8 token
//    rows, transposed in registers with v_perm_b32.
//  - Rows are XOR-swizzled in 16-byte chunks inside each 128-byte group
//    (chunk ^ (row & 7)) so both read patterns avoid LDS bank conflicts.
//  - Page ids of the whole unit are gathered into LDS once, so the tile loop
//    issues no scalar loads.
//  - FP8 caches: rows enter LDS as stored (E4M3FN latent codes, then the bf16
//    k^R), 44% fewer LDS bytes per tile than widened rows; each latent operand
//    is an 8-byte LDS read widened to 8 fp16 values in registers (exact: every
//    E4M3 value is an fp16 value), so the latent products run on
//    v_mfma_f32_16x16x32_f16 with the absorbed query in fp16 (scaled per row
//    by a power of two into [1, 2), 11 significant bits) and P in fp16; with
//    block scales the value side takes P s 2^-E (E a running exponent of the
//    largest scale, folded back into the partial's max).
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int W_, int DR_, int NBR_, int HT_, int G_, int TT_, int OCC_, bool F8_ = false, bool CF_ = false,
          int CS_ = 1, bool P2_ = false, bool TS_ = false, int HPW_ = 1, bool QL_ = false>
struct Cfg {
  static constexpr int W = W_;      // latent block width
  static constexpr int DR = DR_;    // RoPE key width
  static constexpr int NBR = NBR_;  // latent blocks in a cache row
  static constexpr int HT = HT_;    // 16-head tiles per block
  static constexpr int G = G_;      // waves sharing one task (token groups)
  static constexpr int TT = TT_;    // tokens per tile
  static constexpr int OCC = OCC_;  // workgroups resident per compute unit
  static constexpr int ROW = NBR * W + DR;
  static constexpr bool F8 = F8_;     // cache rows hold E4M3FN latent codes, then bf16 k^R
  // Step order: CF computes tile x before storing tile x+1 (so the first tile
  // is computed without waiting for the second); otherwise x+1 is stored and
  // x+2 requested before tile x is computed. Chosen per shape by measurement.
  static constexpr bool CF = CF_;
  // Column splits: CS waves share a (block, 16-head tile, token group) task,
  // each accumulating W / CS of the value columns and scoring over 1 / CS of
  // the query dimensions; the partial scores are summed through LDS. This
  // divides the accumulator and query registers by CS.
  static constexpr int CS = CS_;
  // Prologue: P2 requests the unit's first two tiles together (a second
  // register set, live only before the loop); otherwise the second is
  // requested once the first is in LDS. Chosen per shape by measurement.
  static constexpr bool P2 = P2_;
  // TS (FP8 only): every row also holds one fp32 scale per latent block after
  // the RoPE key (at byte SCO), then zero bytes up to a multiple of 16
  static constexpr bool TS = TS_;
  static constexpr int SCO = NBR * W + 2 * DR;
  static constexpr int ROWG = F8 ? (SCO + (TS ? 4 * NBR : 0) + 15) / 16 * 16 : ROW * 2;  // bytes of a row in HBM
  // bytes of a row in LDS: rows are stored as they come from HBM (FP8: the
  // E4M3 codes, widened to bf16 when the MFMA operands are read), padded to
  // whole 128-byte groups for the swizzle
  static constexpr int ROWB = (ROWG + 127) / 128 * 128;
  static constexpr int CPRG = ROWG / 16;                     // 16-byte HBM chunks per row
  static constexpr int LATC = F8 ? NBR * W / 16 : 0;         // HBM chunks of latent codes per row
  // Head tiles per wave: HPW > 1 gives each wave HPW of its block's 16-head
  // tiles, so every LDS operand read serves HPW MFMAs and the workgroup needs
  // HPW times fewer waves (more registers each).
  static constexpr int HPW = HPW_;
  static constexpr int TASKS = NBR * HT / HPW;
  static constexpr int NWAVES = TASKS * G * CS;
  static constexpr int NTHREADS = NWAVES * 64;
  // waves per SIMD when OCC workgroups share a compute unit, rounded up (the
  // second __launch_bounds__ argument, which bounds the registers per wave)
  static constexpr int WAVES_PER_SIMD = (OCC * NWAVES + 3) / 4;
  static constexpr int TILE_BYTES = TT * ROWB;
  static constexpr int TILE_CHUNKS = TT * CPRG;  // HBM chunks of one tile
  // Loader threads: the largest multiple of 64 not above NTHREADS that divides
  // the tile's chunk count, so every loader moves the same number of chunks;
  // all threads, the last round partly idle (TAIL), where none divides it.
  static constexpr int loaders() {
    for (int n = NTHREADS; n >= 64; n -= 64)
      if (TILE_CHUNKS % n == 0) return n;
    return NTHREADS;
  }
  static constexpr int NLT = loaders();
  static constexpr bool TAIL = TILE_CHUNKS % NLT != 0;
  static constexpr int NL = (TILE_CHUNKS + NLT - 1) / NLT;  // 16-byte chunks per loader per tile
  static constexpr int KK = (W + DR) / 32;       // score k-steps
  static constexpr int KKC = W / 32;             // k-steps over the latent part
  static constexpr int KKH = KK / CS;            // score k-steps of one wave
  // absorbed-query row in the workspace: 4 W + 2 DR bytes; bf16 caches
  // [hi (W) | lo (W) | q^R (DR)] in bf16, FP8 caches [fp16 (W) | q^R bf16 (DR) | 2^e fp32]
  static constexpr int QWB = 4 * W + 2 * DR;
  // registers for the lo parts of one head tile (bf16 caches): the wave's
  // latent k-steps (the first KKC without column splits; with them the share
  // depends on the wave's split)
  // QL (bf16 caches): the lo parts live in LDS instead of registers, one
  // 1 KB row (64 lanes x 16 bytes) per (task, head tile, latent k-step), read
  // next to the tile operands; for kernels whose registers are full
  static constexpr bool QL = QL_ && !F8;
  static constexpr int NLO = (F8 || QL) ? 1 : (CS > 1 ? KKH : KKC);
  static constexpr int QLO_BYTES = QL ? TASKS * HPW * KKC * 1024 : 0;
  static constexpr int NSUB = TT / 32;
  static constexpr int SUBW = NSUB / G;          // 32-token sub-tiles per wave per tile
  static constexpr int NQ = W / 128 / CS;        // 128-column groups per wave on the value side
  static constexpr int MAXPG = TT / 16;          // pages a tile can span (page_size >= 16)
  static constexpr int SEQ_WIN = 64;
  static constexpr int XCH_BYTES = CS > 1 ? NWAVES * 64 * 8 * 4 : 0;  // partial-score exchange
  static constexpr int PT_CAP_RAW =
      (160 * 1024 / OCC - 2 * TILE_BYTES - SEQ_WIN * 4 - NWAVES * 64 - XCH_BYTES - QLO_BYTES - 256) / 4;
  static constexpr int PT_CAP = PT_CAP_RAW > 4096 ? 4096 : PT_CAP_RAW;
  static_assert(ROWB % 128 == 0, "rows must be whole 128-byte groups (the LDS swizzle)");
  static_assert(W % (128 * CS) == 0 && DR % 32 == 0 && KK % CS == 0, "");
  static_assert(TT % 32 == 0 && NSUB % G == 0, "");
  static_assert(!TS || (F8 && NBR <= 4 && CS == 1 && SCO % 16 == 0), "token scales: one chunk, no splits");
  static_assert(PT_CAP >= 64, "LDS: room for the page-id table");
  static_assert(NTHREADS <= 1024, "");
  static_assert(HT % HPW == 0 && (HPW == 1 || CS == 1), "head tiles per wave: whole tiles, no column splits");
  static_assert(!F8 || CS == 1, "FP8: the per-row query scale applies after the latent k-steps of one wave");
};

__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// s_waitcnt immediate for vmcnt(0) alone on gfx9: vmcnt bits [3:0] and
// [15:14] zero, expcnt [6:4] and lgkmcnt [11:8] at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Uniform 32-bit load through the scalar cache (constant address space).
typedef __attribute__((address_space(4))) const int32_t cint32_t;
__device__ __forceinline__ int32_t cload(const int32_t* p) { return *(cint32_t*)(p); }

// Work unit of workgroup b in a grid of n. The dispatcher deals workgroups to
// the 8 XCDs in turn (b -> XCD b % 8); numbering units XCD-major puts runs of
// consecutive units, which share a sequence's query rows, page-table row and
// partial slots, on one XCD and its L2. XCD x runs units
// [x*q + min(x, r), (x+1)*q + min(x+1, r)) with q = n / 8, r = n % 8: a
// bijection for any n.
__device__ __forceinline__ int xcd_major_unit(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

__device__ __forceinline__ floatx4_t mfma_bf16(u32x4_t a, u32x4_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ floatx4_t mfma_f16(u32x4_t a, u32x4_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const half2_t v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // v_cvt_pk_bf16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, v);
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the lanes holding one head).
__device__ __forceinline__ float max_4lanes(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_4lanes(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 16-byte load from global memory (explicit address space: a generic pointer
// would compile to a flat load, which the compiler must also wait for with
// lgkmcnt before any LDS result can be used).
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;
__device__ __forceinline__ u32x4_t gload16(const uint8_t* p) { return *(const gu32x4_t*)(p); }
typedef __attribute__((address_space(1))) const float gfloat_t;
__device__ __forceinline__ float gload4f(const uint8_t* p) { return *(const gfloat_t*)(p); }
// The same load marked nontemporal, for the cache stream: every cache row is
// read once per step, and the streaming hint lets HBM reads run measurably
// closer to peak than plain loads do.
__device__ __forceinline__ u32x4_t gload16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load((const gu32x4_t*)(p));
}

__device__ __forceinline__ u32x4_t lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// 8 E4M3FN codes (8 bytes of LDS) -> 8 fp16 values (exact: E4M3 values are fp16 values)
__device__ __forceinline__ u32x4_t widen8(const uint8_t* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t c = *reinterpret_cast<const u32x2_t*>(p);
  u32x4_t r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    r[2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[h], 1.0f, false));
    r[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[h], 1.0f, true));
  }
  return r;
}

constexpr int kNoExp = -100000;  // block scales: no running exponent yet

template <class C>
__global__ __launch_bounds__(C::NTHREADS, C::WAVES_PER_SIMD) void attend_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * C::TILE_BYTES];
  __shared__ int32_t ptab[C::PT_CAP];      // physical page of (tile - x0, page in tile)
  __shared__ int32_t seq_end[C::SEQ_WIN];  // cum[lo + 1 + i]
  __shared__ float amax_sh[C::CS > 1 ? C::NWAVES : 1][16];  // segment ends: row maxima of the column splits
  __shared__ float xch[C::CS > 1 ? C::NWAVES : 1][8][64];     // partial scores of the column splits
  __shared__ __attribute__((aligned(16))) uint8_t qlo[C::QL ? C::QLO_BYTES : 16];  // QL: lo query parts

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int task = wave % C::TASKS;
  const int tgrp = C::CS > 1 ? (wave / C::TASKS) % C::G : wave / C::TASKS;
  // column split: value columns [cs W / CS, (cs + 1) W / CS) (a constant 0 without splits)
  const int cs = C::CS > 1 ? wave / (C::TASKS * C::G) : 0;
  constexpr int HW = C::HPW;
  const int blk = task / (C::HT / HW);
  const int ht0 = (task % (C::HT / HW)) * HW;  // this wave's first head tile
  const int hgrp = blk / a.k;
  const int jj = blk - hgrp * a.k;
  const int m16 = lane & 15;
  const int g4 = lane >> 4;
  const int HK = a.n_heads * a.k;
  bool head_ok[HW];
  int hk[HW];
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const int hloc = (ht0 + hw) * 16 + m16;
    head_ok[hw] = hloc < a.hpb;
    hk[hw] = (hgrp * a.hpb + hloc) * a.k + jj;
  }
  const int P = a.page_size;
  const bool loader = tid < C::NLT;

  WsHeader* hdr = reinterpret_cast<WsHeader*>(a.ws);
  const int32_t* cum = reinterpret_cast<const int32_t*>(a.ws + a.off_cum);
  const int32_t* nlen = reinterpret_cast<const int32_t*>(a.ws + a.off_nlen);
  const int unit = xcd_major_unit(blockIdx.x, gridDim.x);
  // The unit's descriptor from the plan (one scalar fetch): tile range, the
  // sequence owning its first tile and that sequence's tile range and length.
  const int32_t* ud = reinterpret_cast<const int32_t*>(a.ws + a.off_udesc) + unit * kUnitDescInts;
  const int32_t x0 = cload(ud + 0);
  const int32_t x1 = cload(ud + 1);
  if (x0 >= x1) return;
  const int lo = cload(ud + 2);

  const uint8_t* pool = static_cast<const uint8_t*>(a.pool);
  uint32_t bad_page = 0;
  const int npt = P >= C::TT ? 1 : C::TT >> a.log2_page;  // pages per tile

  // ---- load cursor: runs two tiles ahead of the compute cursor
  int pb = lo;
  int32_t pb_start = cload(ud + 3), pb_end = cload(ud + 4), pb_n = cload(ud + 5);
  bool use_tab = false;
  auto lookup = [&](int b, int32_t pidx) __attribute__((always_inline)) -> int32_t {
    int32_t phys = a.page_table ? cload(a.page_table + static_cast<int64_t>(b) * a.max_pages + pidx)
                                : b * a.max_pages + pidx;
    if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) {
      phys = 0;
      bad_page = 1;
    }
    return phys;
  };
  auto checked = [&](int32_t phys) __attribute__((always_inline)) -> int32_t {
    if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) {
      phys = 0;
      bad_page = 1;
    }
    return phys;
  };
  // Physical page of the j-th page of tile x (x at the load cursor).
  auto page_of = [&](int32_t x, int j) __attribute__((always_inline)) -> int32_t {
    if (use_tab) return __builtin_amdgcn_readfirstlane(ptab[(x - x0) * npt + j]);
    const int32_t npg = (pb_n + P - 1) >> a.log2_page;
    const int32_t pg = ((((x - pb_start) * C::TT)) >> a.log2_page) + j;
    return lookup(pb, pg < npg ? pg : npg - 1);
  };
  // Issues the global loads of tile x into ring slot `ring`.
  auto load_tile = [&](int32_t x, u32x4_t* ring) __attribute__((always_inline)) {
    while (x >= pb_end) {
      ++pb;
      pb_start = pb_end;
      pb_end = cload(cum + pb + 1);
      pb_n = cload(nlen + pb);
    }
    if (!loader) return;
    const int32_t tok0 = (x - pb_start) * C::TT;
    if (P >= C::TT) {
      // the whole tile sits in one page: one base, per-lane offsets
      const uint8_t* base = reinterpret_cast<const uint8_t*>(uniform64(reinterpret_cast<uint64_t>(
          pool + (static_cast<int64_t>(page_of(x, 0)) * P + (tok0 & (P - 1))) * C::ROWG)));
      // rows are contiguous inside a page: chunk p of the tile is at 16 p, a
      // 32-bit offset from the uniform base (scalar base + vector offset)
#pragma unroll
      for (int k = 0; k < C::NL; ++k) {
        if (C::TAIL && k * C::NLT + tid >= C::TILE_CHUNKS) break;
        const uint32_t off = 16u * static_cast<uint32_t>(k * C::NLT + tid);
        ring[k] = gload16_stream(base + off);
      }
    } else {
      // tile spans npt pages (tok0 is page aligned): per-lane page select
      int32_t ph[C::MAXPG];
#pragma unroll
      for (int j = 0; j < C::MAXPG; ++j) ph[j] = j < npt ? page_of(x, j) : 0;
#pragma unroll
      for (int k = 0; k < C::NL; ++k) {
        const int p = k * C::NLT + tid;
        if (C::TAIL && p >= C::TILE_CHUNKS) break;
        const int r = p / C::CPRG, lc = p % C::CPRG;
        const int j = r >> a.log2_page;
        int32_t phys = ph[0];
#pragma unroll
        for (int q = 1; q < C::MAXPG; ++q) phys = j == q ? ph[q] : phys;
        ring[k] = gload16_stream(pool + (static_cast<int64_t>(phys) * P + (r & (P - 1))) * C::ROWG + 16 * lc);
      }
    }
  };
  // Writes ring slot `ring` (tile with `valid` token rows) into LDS buffer `dst`.
  auto store_tile = [&](const u32x4_t* ring, uint8_t* dst, int valid) __attribute__((always_inline)) {
    if (!loader) return;
#pragma unroll
    for (int k = 0; k < C::NL; ++k) {
      const int p = k * C::NLT + tid;
      if (C::TAIL && p >= C::TILE_CHUNKS) break;
      const int r = p / C::CPRG, lc = p % C::CPRG;
      u32x4_t v = ring[k];
      if (r >= valid) v = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(dst + r * C::ROWB + 16 * (lc ^ (r & 7))) = v;
    }
  };

  // ---- compute state
  floatx4_t O[HW][C::NQ][8];
  float m_run[HW], l_run[HW];
  int e_run = kNoExp;  // block scales: the value side accumulates P s 2^-e_run
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
#pragma unroll
    for (int q = 0; q < C::NQ; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) O[hw][q][e] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_run[hw] = -INFINITY;
    l_run[hw] = 0.f;
  }
  u32x4_t Qb[HW][C::KKH];   // this wave's score k-steps [cs KKH, (cs + 1) KKH), per head tile
  u32x4_t Ql[HW][C::NLO];   // bf16 caches: lo parts of its latent k-steps (zero for RoPE k-steps)
  float qn[HW];             // FP8 caches: the row scale 2^e of the fp16 query

  int cb = lo;
  int32_t cb_start = pb_start, cb_end = pb_end, cb_n = pb_n;

  float* pm = reinterpret_cast<float*>(a.ws + a.off_pm);
  float* pl = reinterpret_cast<float*>(a.ws + a.off_pl);
  uint16_t* po = reinterpret_cast<uint16_t*>(a.ws + a.off_po);  // fp16 weighted latent sums
  const uint8_t* qext = reinterpret_cast<const uint8_t*>(a.ws + a.off_qext);

  auto load_q = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int hw = 0; hw < HW; ++hw) {
      const uint8_t* qe = qext + (static_cast<int64_t>(b) * HK + hk[hw]) * C::QWB;
      // byte offsets: latent parts, then the RoPE part after them
      constexpr int kRope = C::F8 ? 2 * C::W : 4 * C::W;
#pragma unroll
      for (int u = 0; u < C::KKH; ++u) {
        const int kk = cs * C::KKH + u;
        const bool lat = kk < C::KKC;
        const int off = lat ? 2 * (32 * kk + 8 * g4) : kRope + 2 * (32 * (kk - C::KKC) + 8 * g4);
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (head_ok[hw]) v = gload16(qe + off);
        Qb[hw][u] = v;
        if constexpr (C::QL) {
          // every wave of a task writes the same values into its rows, before
          // any of them reads them (a new sequence starts after the tile barrier)
          if (lat) {
            u32x4_t vl = u32x4_t{0u, 0u, 0u, 0u};
            if (head_ok[hw]) vl = gload16(qe + 2 * C::W + off);
            *reinterpret_cast<u32x4_t*>(qlo + ((task * HW + hw) * C::KKC + kk) * 1024 + 16 * lane) = vl;
          }
        } else if constexpr (!C::F8) {
          if (u < C::NLO) {
            u32x4_t vl = u32x4_t{0u, 0u, 0u, 0u};
            if (head_ok[hw] && lat) vl = gload16(qe + 2 * C::W + off);
            Ql[hw][u] = vl;
          }
        }
      }
      if constexpr (C::F8) qn[hw] = head_ok[hw] ? gload4f(qe + 2 * C::W + 2 * C::DR) : 1.f;
    }
  };
  load_q(cb);

  // ---- store cursor: the tile written into LDS next
  int sc_b = lo;
  int32_t sc_start = pb_start, sc_end = pb_end, sc_n = pb_n;
  auto store_valid = [&](int32_t x) __attribute__((always_inline)) -> int {
    while (x >= sc_end) {
      ++sc_b;
      sc_start = sc_end;
      sc_end = cload(cum + sc_b + 1);
      sc_n = cload(nlen + sc_b);
    }
    return min(C::TT, sc_n - (x - sc_start) * C::TT);
  };

  // ---- prologue: with the descriptor in hand, tile x0 (its page looked up
  // with a scalar load), the query and the page ids of the rest of the unit
  // are requested together; tile x0+1 follows once x0 is in LDS.
  u32x4_t ring0[C::P2 ? C::NL : 1], ring[C::NL];
  if constexpr (C::P2) {
    load_tile(x0, ring0);
    if (x0 + 1 < x1) load_tile(x0 + 1, ring);
  } else {
    load_tile(x0, ring);
  }

  const int32_t nx_end = cload(ud + 6), nx_n = cload(ud + 7);  // the sequence after lo
  const int32_t ntab = (x1 - x0) * npt;
  if (ntab <= C::PT_CAP && x1 <= nx_end) {
    // every tile of the unit lies in sequence lo or lo + 1. lo's range comes
    // from the compute cursor (cb_*), which still holds it: with the two-tile
    // prologue the load cursor has already moved on when x0 is lo's last tile
    for (int i = tid; i < ntab; i += C::NTHREADS) {
      const int32_t x = x0 + i / npt;
      const int j = i % npt;
      const bool first = x < cb_end;
      const int b = first ? lo : lo + 1;
      const int32_t start = first ? cb_start : cb_end;
      const int32_t n = first ? cb_n : nx_n;
      const int32_t npg = (n + P - 1) >> a.log2_page;
      const int32_t pg0 = (((x - start) * C::TT) >> a.log2_page) + j;
      const int32_t pg = pg0 < npg ? pg0 : npg - 1;
      ptab[i] = checked(a.page_table ? a.page_table[static_cast<int64_t>(b) * a.max_pages + pg]
                                     : b * a.max_pages + pg);
    }
    __syncthreads();
    use_tab = true;
  } else {
    const int win = min(C::SEQ_WIN, a.batch - lo);
    if (tid < win) seq_end[tid] = cum[lo + 1 + tid];
    __syncthreads();
    if (ntab <= C::PT_CAP && x1 <= seq_end[win - 1]) {
      const int32_t lo_start = cb_start;
      for (int i = tid; i < ntab; i += C::NTHREADS) {
        const int32_t x = x0 + i / npt;
        const int j = i % npt;
        int k = 0;
        while (seq_end[k] <= x) ++k;
        const int b = lo + k;
        const int32_t start = k == 0 ? lo_start : seq_end[k - 1];
        const int32_t n = nlen[b];
        const int32_t npg = (n + P - 1) >> a.log2_page;
        const int32_t pg0 = (((x - start) * C::TT) >> a.log2_page) + j;
        const int32_t pg = pg0 < npg ? pg0 : npg - 1;
        ptab[i] = checked(a.page_table ? a.page_table[static_cast<int64_t>(b) * a.max_pages + pg]
                                       : b * a.max_pages + pg);
      }
      use_tab = true;
    }
    __syncthreads();
  }
  if constexpr (C::P2) {
    store_tile(ring0, lds, store_valid(x0));
  } else {
    store_tile(ring, lds, store_valid(x0));
    if (x0 + 1 < x1) load_tile(x0 + 1, ring);
  }

  auto step = [&](int32_t x) __attribute__((always_inline)) {
    const int t = x - x0;
    uint8_t* sb = lds + (t & 1) * C::TILE_BYTES;

    bool need_q = false;
    while (x >= cb_end) {
      ++cb;
      cb_start = cb_end;
      cb_end = cload(cum + cb + 1);
      cb_n = cload(nlen + cb);
      need_q = true;
    }
    const int valid = min(C::TT, cb_n - (x - cb_start) * C::TT);
    // Tile x is in its buffer for every wave and every wave is done with
    // tile x-1: tile x+1 goes registers -> the other buffer (before or after
    // tile x is computed), tile x+2 is requested into the registers.
    lds_barrier();
    if constexpr (C::CF) {
      if (need_q) {
        // a new sequence starts inside this unit: its query before any MFMA
        load_q(cb);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
    } else if constexpr (C::OCC == 1) {
      // One workgroup per compute unit: nothing else hides this workgroup's
      // memory waits, so tile x+2 stays in flight while tile x is computed.
      // The query of a new sequence is loaded and waited for first, so no
      // path into the MFMAs has it outstanding.
      if (x + 1 < x1) store_tile(ring, lds + ((t + 1) & 1) * C::TILE_BYTES, store_valid(x + 1));
      if (need_q) {
        load_q(cb);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
      if (x + 2 < x1) load_tile(x + 2, ring);
    } else {
      // Several workgroups per compute unit: each waits for its loads before
      // computing and the others fill the wait.
      if (x + 1 < x1) {
        store_tile(ring, lds + ((t + 1) & 1) * C::TILE_BYTES, store_valid(x + 1));
        if (x + 2 < x1) load_tile(x + 2, ring);
      }
      if (need_q) load_q(cb);  // a new sequence starts inside this unit
    }

#pragma unroll
    for (int si = 0; si < C::SUBW; ++si) {
      const int rowbase = 32 * (si * C::G + tgrp);
      // ---- scores: S_h[i] = token rowbase + 16 h + 4 g4 + i, head m16
      const int r0 = rowbase + m16;
      const uint8_t* rp0 = sb + r0 * C::ROWB;
      const uint8_t* rp1 = rp0 + 16 * C::ROWB;
      const int key = m16 & 7;
      floatx4_t S0[HW], S1[HW];
#pragma unroll
      for (int hw = 0; hw < HW; ++hw) S0[hw] = S1[hw] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      // TS: the scales of this wave's block for its eight tokens (rows past
      // the sequence end were stored as zeros)
      float sc0[4], sc1[4];
      if constexpr (C::TS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t0 = rowbase + 4 * g4 + i, t1 = t0 + 16;
          sc0[i] = *reinterpret_cast<const float*>(sb + t0 * C::ROWB + 16 * ((C::SCO / 16) ^ (t0 & 7)) + 4 * blk);
          sc1[i] = *reinterpret_cast<const float*>(sb + t1 * C::ROWB + 16 * ((C::SCO / 16) ^ (t1 & 7)) + 4 * blk);
        }
      }
      // score k-steps whose operands are read ahead together (two with two head
      // tiles per wave: fewer live operands where registers spill; 1-2% faster)
      constexpr int KB = C::HPW > 1 ? 2 : 3;
#pragma unroll
      for (int kb = 0; kb < C::KKH; kb += KB) {
        u32x4_t A0[KB], A1[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int kl = kb + u;
          if (kl < C::KKH) {
            const int kk = cs * C::KKH + kl;
            if (C::F8 && kk < C::KKC) {
              // 8 latent codes of the row: half of a 16-byte chunk
              const int ch = blk * (C::W / 16) + 2 * kk + (g4 >> 1);
              const int co = 16 * (ch ^ key) + 8 * (g4 & 1);
              A0[u] = widen8(rp0 + co);
              A1[u] = widen8(rp1 + co);
            } else {
              const int lat = C::F8 ? C::NBR * C::W / 16 : C::NBR * (C::W / 8);  // chunks before k^R
              const int chunk = kk < C::KKC ? blk * (C::W / 8) + 4 * kk + g4 : lat + 4 * (kk - C::KKC) + g4;
              const int co = 16 * (chunk ^ key);
              A0[u] = lds_read16(rp0 + co);
              A1[u] = lds_read16(rp1 + co);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int kl = kb + u;
          if (kl < C::KKH) {
            const bool lat = cs * C::KKH + kl < C::KKC;
#pragma unroll
            for (int hw = 0; hw < HW; ++hw) {
              if (C::F8 && lat) {
                S0[hw] = mfma_f16(A0[u], Qb[hw][kl], S0[hw]);
                S1[hw] = mfma_f16(A1[u], Qb[hw][kl], S1[hw]);
              } else {
                S0[hw] = mfma_bf16(A0[u], Qb[hw][kl], S0[hw]);
                S1[hw] = mfma_bf16(A1[u], Qb[hw][kl], S1[hw]);
              }
              if constexpr (C::QL) {
                if (lat) {
                  const u32x4_t ql = lds_read16(qlo + ((task * HW + hw) * C::KKC + cs * C::KKH + kl) * 1024 + 16 * lane);
                  S0[hw] = mfma_bf16(A0[u], ql, S0[hw]);
                  S1[hw] = mfma_bf16(A1[u], ql, S1[hw]);
                }
              } else if constexpr (!C::F8) {
                if (kl < C::NLO && lat) {
                  S0[hw] = mfma_bf16(A0[u], Ql[hw][kl], S0[hw]);
                  S1[hw] = mfma_bf16(A1[u], Ql[hw][kl], S1[hw]);
                }
              }
              if constexpr (C::F8) {
                if (kl == C::KKC - 1) {
                  // the latent part is complete: the query's row scale (and the
                  // token's block scale) before the RoPE k-steps add theirs
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    S0[hw][i] *= C::TS ? qn[hw] * sc0[i] : qn[hw];
                    S1[hw][i] *= C::TS ? qn[hw] * sc1[i] : qn[hw];
                  }
                }
              }
            }
          }
        }
      }
      if constexpr (C::CS > 1) {
        // sum the column splits' partial scores (the same order-free sum in
        // every split, so all of them see identical scores)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xch[wave][i][lane] = S0[0][i];
          xch[wave][4 + i][lane] = S1[0][i];
        }
        __syncthreads();
#pragma unroll
        for (int c2 = 0; c2 < C::CS; ++c2) {
          if (c2 == cs) continue;
          const int w2 = task + C::TASKS * (tgrp + C::G * c2);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            S0[0][i] += xch[w2][i][lane];
            S1[0][i] += xch[w2][4 + i][lane];
          }
        }
      }
      // base-2 logits: the query parts were not scaled by softmax_scale log2(e)
#pragma unroll
      for (int hw = 0; hw < HW; ++hw)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S0[hw][i] *= a.qscale;
          S1[hw][i] *= a.qscale;
        }
      // block scales: the value side takes P s 2^-e_run. e_run follows the
      // largest scale of the sub-tile (the same for every lane: it depends on
      // the tokens only); when that moves up, or more than 2^8 below, O is
      // rescaled, so the fp16 weights of the sub-tile's largest terms keep
      // their precision (s 2^-e_run < 1). A downward move is capped at 2^100
      // so that O (at most ~2^20 in these units) stays finite.
      int pexp = 0;  // P s is multiplied by 2^pexp
      if constexpr (C::TS) {
        float smax = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) smax = fmaxf(smax, fmaxf(sc0[i], sc1[i]));
        smax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(max_4lanes(smax))));
        if (smax > 0.f && smax <= 3.0e38f) {
          int et;
          frexpf(smax, &et);  // smax < 2^et
          if (e_run == kNoExp) {
            e_run = et;  // O is still zero
          } else if (et > e_run || et < e_run - 8) {
            const int en = et > e_run ? et : max(et, e_run - 100);
#pragma unroll
            for (int hw = 0; hw < HW; ++hw)
#pragma unroll
              for (int q = 0; q < C::NQ; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                  for (int i = 0; i < 4; ++i) O[hw][q][e][i] = ldexpf(O[hw][q][e][i], e_run - en);
            e_run = en;
          }
        }
        if (e_run != kNoExp) pexp = -e_run;
      }
      // value-side rows: 8 columns (col group 16 q' + m16 of the block, q' the
      // 128-column group) of 8 token rows
      auto read_rows = [&](int qg, u32x4_t* R) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int tr = rowbase + (v < 4 ? 4 * g4 + v : 16 + 4 * g4 + (v - 4));
          if constexpr (C::F8) {
            const int ch = blk * (C::W / 16) + 8 * qg + (m16 >> 1);
            R[v] = widen8(sb + tr * C::ROWB + 16 * (ch ^ (tr & 7)) + 8 * (m16 & 1));
          } else {
            const int chunk = blk * (C::W / 8) + 16 * qg + m16;
            R[v] = lds_read16(sb + tr * C::ROWB + 16 * (chunk ^ (tr & 7)));
          }
        }
      };
      // the first 128-column group, read while the scores finish
      u32x4_t R[8];
      read_rows(cs * C::NQ, R);
      u32x4_t pb[HW];
#pragma unroll
      for (int hw = 0; hw < HW; ++hw) {
        if (valid < C::TT) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (rowbase + 4 * g4 + i >= valid) S0[hw][i] = -INFINITY;
            if (rowbase + 16 + 4 * g4 + i >= valid) S1[hw][i] = -INFINITY;
          }
        }
        // ---- online softmax (per head m16; lanes m16, m16+16, +32, +48 share a head)
        float mx = fmaxf(fmaxf(fmaxf(S0[hw][0], S0[hw][1]), fmaxf(S0[hw][2], S0[hw][3])),
                         fmaxf(fmaxf(S1[hw][0], S1[hw][1]), fmaxf(S1[hw][2], S1[hw][3])));
        mx = max_4lanes(mx);
        const float m_new = fmaxf(m_run[hw], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float scale = fast_exp2(m_run[hw] - m_use);
        float p0[4], p1[4];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p0[i] = fast_exp2(S0[hw][i] - m_use);
          p1[i] = fast_exp2(S1[hw][i] - m_use);
          psum += p0[i] + p1[i];
        }
        l_run[hw] = l_run[hw] * scale + psum;
        m_run[hw] = m_new;
        if (__any(scale != 1.f)) {
#pragma unroll
          for (int q = 0; q < C::NQ; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) O[hw][q][e] *= scale;
        }
        if constexpr (C::TS) {
          // value side: sum_t p_t (s_t code_t) = sum_t (p_t s_t) code_t; the
          // softmax sum above keeps the unscaled p_t
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p0[i] *= ldexpf(sc0[i], pexp);
            p1[i] *= ldexpf(sc1[i], pexp);
          }
        }
        if constexpr (C::F8)
          pb[hw] = u32x4_t{pack_f16x2(p0[0], p0[1]), pack_f16x2(p0[2], p0[3]), pack_f16x2(p1[0], p1[1]),
                           pack_f16x2(p1[2], p1[3])};
        else
          pb[hw] = u32x4_t{pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]), pack_bf16x2(p1[0], p1[1]),
                           pack_bf16x2(p1[2], p1[3])};
      }
      // ---- values: O^T[col][head] += C^T[col][tokens] P^T[tokens][head]
#pragma unroll
      for (int q = 0; q < C::NQ; ++q) {
        if (q > 0) read_rows(cs * C::NQ + q, R);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t Av;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            Av[u] = __builtin_amdgcn_perm(R[2 * u + 1][e >> 1], R[2 * u][e >> 1], sel);
#pragma unroll
          for (int hw = 0; hw < HW; ++hw)
            O[hw][q][e] = C::F8 ? mfma_f16(Av, pb[hw], O[hw][q][e]) : mfma_bf16(Av, pb[hw], O[hw][q][e]);
        }
      }
    }

    if (x + 1 == cb_end || x + 1 == x1) {
      // ---- segment end: write this wave's partials and reset.
      const int64_t slot = static_cast<int64_t>(unit + cb) * C::G + tgrp;
#pragma unroll
      for (int hw = 0; hw < HW; ++hw) {
        const float l_tot = sum_4lanes(l_run[hw]);
        // The head's row of weighted sums is scaled by 2^-s, s the exponent of
        // its largest magnitude, and stored as fp16 (values in (-1, 1), 11-bit
        // precision); m + s and l 2^-s go with it, which leaves every ratio the
        // combine forms unchanged.
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < C::NQ; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(O[hw][q][e][i]));
        amax = max_4lanes(amax);
        if constexpr (C::CS > 1) {
          // the column splits of a head agree on one scale
          if (g4 == 0) amax_sh[wave][m16] = amax;
          __syncthreads();
#pragma unroll
          for (int c2 = 0; c2 < C::CS; ++c2) amax = fmaxf(amax, amax_sh[task + C::TASKS * (tgrp + C::G * c2)][m16]);
        }
        int sexp = 0;
        if (amax > 0.f) frexpf(amax, &sexp);
        const float rs = ldexpf(1.f, -sexp);
        if (head_ok[hw]) {
          // column 128 q + 8 (4 g4 + i) + e holds O[q][e][i]: 8 consecutive
          // columns per (q, i), one 16-byte store
          uint16_t* dst = po + (slot * HK + hk[hw]) * C::W;
#pragma unroll
          for (int q = 0; q < C::NQ; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const u32x4_t v = {pack_f16x2(O[hw][q][0][i] * rs, O[hw][q][1][i] * rs),
                                 pack_f16x2(O[hw][q][2][i] * rs, O[hw][q][3][i] * rs),
                                 pack_f16x2(O[hw][q][4][i] * rs, O[hw][q][5][i] * rs),
                                 pack_f16x2(O[hw][q][6][i] * rs, O[hw][q][7][i] * rs)};
              *reinterpret_cast<u32x4_t*>(dst + 128 * (cs * C::NQ + q) + 8 * (4 * g4 + i)) = v;
            }
          if (g4 == 0 && cs == 0) {
            // block scales: the sums are O 2^e_run, so the stored row's scale
            // exponent is sexp + e_run
            const int tot = C::TS && e_run != kNoExp ? sexp + e_run : sexp;
            pm[slot * HK + hk[hw]] = m_run[hw] + static_cast<float>(tot);
            pl[slot * HK + hk[hw]] = ldexpf(l_tot, -tot);
          }
        }
#pragma unroll
        for (int q = 0; q < C::NQ; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) O[hw][q][e] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        m_run[hw] = -INFINITY;
        l_run[hw] = 0.f;
      }
      e_run = kNoExp;
    }
    if constexpr (C::CF) {
      // tile x+1 has been in flight since the previous step; its buffer was
      // left by every wave at this step's barrier, the next barrier publishes it
      if (x + 1 < x1) {
        store_tile(ring, lds + ((t + 1) & 1) * C::TILE_BYTES, store_valid(x + 1));
        if (x + 2 < x1) load_tile(x + 2, ring);
      }
    }
  };

  for (int32_t x = x0; x < x1; ++x) step(x);
  if (__any(bad_page) && lane == 0) atomicOr(&hdr->flags, kFlagBadPage);
}

template <class C>
hipError_t run_variant(const DecodeArgs& a, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  if (t0 || t1)  // the dispatch records the kernel's own start and stop times
    hipExtLaunchKernelGGL(attend_mfma_kernel<C>, dim3(a.units), dim3(C::NTHREADS), 0, stream, t0, t1, 0, a);
  else
    attend_mfma_kernel<C><<<a.units, C::NTHREADS, 0, stream>>>(a);
  return hipGetLastError();
}

struct Entry {
  MfmaVariant v;
  hipError_t (*fn)(const DecodeArgs&, hipStream_t, hipEvent_t, hipEvent_t);
};

template <int W, int DR, int NBR, int HT, int G, int TT, int OCC, bool F8 = false, bool CF = false, int CS = 1,
          bool P2 = false, bool TS = false, int HPW = 1, bool QL = false>
constexpr Entry entry() {
  using C = Cfg<W, DR, NBR, HT, G, TT, OCC, F8, CF, CS, P2, TS, HPW, QL>;
  return Entry{MfmaVariant{W, DR, NBR, HT, G, TT, OCC, F8 ? (TS ? 2 : 1) : 0, C::NTHREADS, 2 * C::TILE_BYTES},
               &run_variant<C>};
}

// Shapes with a tuned MFMA kernel. Key: (w, d_r, blocks per row, 16-head tiles per block).
// Each tuning was chosen by same-box A/B timing of the candidates (step
// order, prologue, column splits, head tiles per wave, occupancy, where the
// query's lo parts live). Compute-first is 4-7% faster for the TP shares,
// MLRA-2, FP8 MLRA-4 and the column-split MLA kernels and 2-6% slower for bf16
// MLRA-4; the two-tile prologue 4-6% faster for the TP shares and FP8 MLRA-4,
// 22% for MLRA-2.
const Entry kVariants[] = {
    // MLRA-4: 4 x 128 latent, <= 16 heads per block; 64-token tiles in two
    // 32-token groups (eight waves, one workgroup per compute unit),
    // compute-first (interleaved at B = 32, 8K: step 67.1 -> 64.8 us against
    // four waves on 32-token tiles at two workgroups per unit; 65.3-65.4 with
    // the two-tile prologue or store-first)
    entry<128, 64, 4, 1, 2, 64, 1, false, true>(),
    // MLA: one 512 latent, 64 heads; column-split waves (half the value
    // columns and half the score dimensions each), compute-first; the lo query
    // parts in LDS (in registers they spilled 65 VGPRs: 137.5 vs 103.7 us at
    // B = 32, 8K)
    entry<512, 64, 1, 4, 1, 32, 1, false, true, 2, false, false, 1, true>(),
    // one MLRA-4 block (a TP rank's share), <= 16 heads: one-wave workgroups,
    // four per compute unit, each streaming its own 32-token tiles (measured
    // 1.8x faster than four waves sharing 128-token tiles at one per unit)
    entry<128, 64, 1, 1, 1, 32, 4, false, true, 1, true>(),
    // MLRA-2: 2 x 256 latent, <= 32 heads per block; column-split waves, one
    // workgroup per compute unit (no spills), two-tile prologue: the fastest
    // step of the four combinations of split and prologue measured
    entry<256, 64, 2, 2, 1, 32, 1, false, true, 2, true>(),
    // 4 x 128 latent, <= 32 heads per block (reading B with k = 2): eight
    // one-tile waves, compute-first, two-tile prologue (82.6 -> 61.5 us at
    // B = 32, 8K against store-first with a one-tile prologue; two head tiles
    // per wave spilled 82 VGPRs over 64-token tiles, and at 32-token tiles
    // with the lo parts in LDS measured 75.7 us)
    entry<128, 64, 4, 2, 1, 32, 1, false, true, 1, true>(),
    // 4 x 128 latent, <= 64 heads per block (reading B with k = 4): two head
    // tiles per wave, eight waves, the lo query parts in LDS (sixteen one-tile
    // waves spill; 112.8 us with the lo parts in registers, 99.6 in LDS)
    entry<128, 64, 4, 4, 1, 32, 1, false, false, 1, false, false, 2, true>(),
    // MLA's share under 4-way tensor parallelism: the whole 512 latent and the
    // RoPE key for <= 16 heads; column-split waves, two workgroups per compute
    // unit, compute-first, two-tile prologue (362.7 us at B = 64, 32K; 446.4
    // store-first with a one-tile prologue, 422.4 with 64-token tiles in two
    // token groups at one workgroup per unit)
    entry<512, 64, 1, 1, 1, 32, 2, false, true, 2, true>(),
    // one MLRA-2 block (a TP-2 rank's share), <= 32 heads: column-split waves,
    // two workgroups per compute unit, compute-first, two-tile prologue
    // (406 -> 235 us at B = 64, 32K against one workgroup of four waves)
    entry<256, 64, 1, 2, 1, 32, 2, false, true, 2, true>(),
    // FP8 (E4M3FN) caches of the same shapes and tunings
    entry<128, 64, 4, 1, 1, 32, 2, true, true, 1, true>(),
    entry<512, 64, 1, 4, 1, 32, 1, true>(),
    entry<128, 64, 1, 1, 1, 32, 4, true, true>(),
    entry<256, 64, 2, 2, 1, 32, 2, true, true>(),
    // FP8 reading B (32 and 64 heads per block) and the TP-2 share of MLRA-2
    // (no column splits on FP8 caches; MLA's TP-4 share would spill over 500
    // registers without them and has no FP8 kernel)
    entry<128, 64, 4, 2, 1, 32, 1, true, true, 1, true>(),
    entry<128, 64, 4, 4, 1, 32, 1, true, false, 1, false, false, 2>(),
    entry<256, 64, 1, 2, 1, 32, 2, true, true, 1, true>(),
    // FP8 with one scale per token and latent block (the same tunings)
    entry<128, 64, 4, 1, 1, 32, 2, true, true, 1, true, true>(),
    entry<512, 64, 1, 4, 1, 32, 1, true, false, 1, false, true>(),
    entry<128, 64, 1, 1, 1, 32, 4, true, true, 1, false, true>(),
    entry<256, 64, 2, 2, 1, 32, 2, true, true, 1, false, true>(),
    entry<128, 64, 4, 2, 1, 32, 1, true, true, 1, true, true>(),
    entry<128, 64, 4, 4, 1, 32, 1, true, false, 1, false, true, 2>(),
    entry<256, 64, 1, 2, 1, 32, 2, true, true, 1, true, true>(),
};

}  // namespace

const MfmaVariant* find_mfma_variant(int w, int d_r, int n_blocks, int head_tiles, int fp8) {
  for (const Entry& e : kVariants)
    if (e.v.w == w && e.v.d_r == d_r && e.v.n_blocks == n_blocks && e.v.head_tiles == head_tiles &&
        e.v.fp8 == fp8)
      return &e.v;
  return nullptr;
}

hipError_t launch_attend_mfma(const MfmaVariant* v, const DecodeArgs& a, hipStream_t stream, hipEvent_t t0,
                              hipEvent_t t1) {
  for (const Entry& e : kVariants)
    if (&e.v == v) return e.fn(a, stream, t0, t1);
  return hipErrorInvalidValue;
}

}  // namespace mlra
