// Shared definitions of libmlra's kernels and host layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "validate.h"

namespace mlra {

// Workspace layout (all offsets 256-byte aligned):
//   [0, 256)     WsHeader
//   cum          int32 [batch + 1]  prefix sums of tiles per sequence
//   nlen         int32 [batch]      clamped sequence lengths
//   qext         [batch][hk] rows of absorbed queries, by query mode (DecodeArgs::q_mode):
//                  kQueryF32   fp32 [w + d_r], latent and RoPE parts scaled by softmax_scale log2(e)
//                  kQuerySplit bf16 [hi (w) | lo (w) | q^R (d_r)]: the latent part v = W^UK^T q^C
//                              as v = hi + lo (about 16 significant bits), q^R as given; not scaled
//                  kQueryF16   [v 2^-e as fp16 (w) | q^R bf16 (d_r) | 2^e fp32], e chosen per row
//                              so the largest |v 2^-e| is in [1, 2); not scaled by softmax_scale
//                the two MFMA modes use 4 w + 2 d_r bytes per row
//   pm, pl       fp32 [slots][hk]      partial running max / sum
//   po           fp32 [slots][hk][w]   partial weighted latent sums
// hk = n_heads * blocks_per_head; slots = (units + batch) * groups + 1 (the
// last slot is kept empty: m = -inf, l = 0, o~ = 0).
struct WsHeader {
  uint32_t magic;
  uint32_t flags;
  int32_t n_tiles;
  int32_t units;
  int32_t tile_tokens;
  int32_t groups;
  int32_t batch;
  int32_t hk;
  int32_t pad[56];
};
static_assert(sizeof(WsHeader) == 256, "header is 256 bytes");

constexpr uint32_t kWsMagic = 0x4d4c5241u;  // "MLRA"
constexpr uint32_t kFlagBadPage = 1u;       // same value as MLRA_FLAG_BAD_PAGE
// Per-unit plan descriptor (ints): 0 first tile x0, 1 end tile x1, 2 sequence
// lo owning x0, 3 cum[lo], 4 cum[lo + 1], 5 length of lo, 6 cum[lo + 2] (the
// tile count when lo is the last sequence), 7 length of lo + 1 (0 if none).
constexpr int kUnitDescInts = 8;
// Absorbed-query layouts (qext rows, above).
constexpr int kQueryF32 = 0, kQuerySplit = 1, kQueryF16 = 2;

// Everything a decode kernel needs, passed by value.
struct DecodeArgs {
  const void* pool;
  const int32_t* page_table;  // nullptr: identity layout
  char* ws;
  int64_t off_cum, off_nlen, off_sunit, off_udesc, off_qext, off_pm, off_pl, off_po;
  int32_t po_f16;     // weighted latent sums of the partials stored as fp16 rows scaled by a
                      // power of two folded into m and l (MFMA path), else fp32
  int32_t q_mode;     // absorbed-query layout: kQueryF32 (generic path), kQuerySplit (bf16
                      // caches on MFMA) or kQueryF16 (FP8 caches on MFMA)
  int32_t batch;
  int32_t n_heads;
  int32_t d_h;
  int32_t w;          // latent block width
  int32_t n_blocks;   // blocks per cache row
  int32_t k;          // blocks per head
  int32_t hpb;        // heads per block (h k / b)
  int32_t d_r;
  int32_t row;        // elements per cache row (n_blocks * w + d_r)
  int32_t page_size;
  int32_t log2_page;
  int32_t max_pages;
  int32_t num_pages;
  int32_t units;
  int32_t tile_tokens;
  int32_t groups;
  int32_t empty_slot;  // partial slot kept empty (m = -inf, l = 0, o~ = 0) for the combine
  float qscale;       // softmax_scale * log2(e)
  float out_scale;
  float lat_scale;    // FP8 caches: cache_scale (folded into the latent part of q~); else 1
};

struct AppendArgs {
  void* pool;
  const int32_t* page_table;
  const int32_t* positions;
  const void* x;
  const void* w_dkv;
  const void* kr_new;
  void* c_out;
  int32_t batch, d_c, d_r, d_model, row, page_size, max_pages, num_pages;  // row: bytes for FP8
  float cache_inv;  // FP8 caches: fp32 reciprocal of cache_scale
};

struct CombineArgs {
  const char* ws;
  const void* w_uv;
  float* out;
  float* lse;
  int64_t off_sunit, off_pm, off_pl, off_po;
  int32_t po_f16;  // as DecodeArgs::po_f16
  int32_t batch, n_heads, d_h, w, k, hk;
  int32_t groups;      // head groups per work unit (partial slots per unit and sequence)
  int32_t empty_slot;  // partial slot that always reads as empty (m = -inf, l = 0, o~ = 0)
  float out_scale;
};

// y[b][m][n] = sum_k x[b][k] W_m[k][n] (+ RoPE on each output vector).
struct ProjArgs {
  const void* x;
  int64_t x_bstride;   // elements between sequences of x
  int32_t x_f32;       // x is fp32 (else bf16)
  const void* w;
  int64_t w_mstride;   // elements between the matrices W_m
  int32_t w_bf16;      // W is bf16 (else fp32)
  void* y;
  int64_t y_bstride, y_mstride;
  int32_t y_bf16;      // y is bf16 (else fp32)
  int32_t B, K, N;     // N a multiple of 8
  const int32_t* positions;
  int32_t rope;
  float rope_base;
};

// One product of a projection launch on the MFMA path (bf16 weights):
// y[b][m][n] = sum_k x[b][k] W_m[k][n], W_m stored [K][N], optional RoPE.
struct ProjJob {
  const void* x;
  int64_t x_bstride;  // elements between sequences of x (a multiple of 8)
  int32_t x_f32;      // x is fp32 (split into two bf16 operands), else bf16
  const uint16_t* w;
  int64_t w_mstride;
  void* y;
  int64_t y_bstride, y_mstride;
  int32_t y_f32;
  int32_t K, N;  // multiples of 8
  int32_t rope;
  int32_t kind;    // epilogue: kProjStore, kProjLatentRow or kProjRopeRow
  int32_t n_mats;  // matrices W_m (heads) sharing the job
  int32_t tiles;   // column tiles of N (set by the launcher)
  int32_t ksplit;  // K slices (set by the launcher); > 1: fp32 partials go to `part`
  int32_t kper;    // 32-row k-steps per slice (set by the launcher)
  int32_t wgs;     // workgroups: tiles x sequence groups x matrices x slices (set by the launcher)
  float* part;     // [ksplit][n_mats][B][N] fp32 partial sums (ksplit > 1)
};
// Epilogues of a projection job:
//   kProjStore      y[b][m][n] (fp32 or bf16), optional RoPE;
//   kProjLatentRow  the latent of token positions[b] into its pool row (bf16,
//                   or FP8 codes of value x cache_inv) and c_out; with kr_src
//                   the given RoPE key is copied into the row as well;
//   kProjRopeRow    RoPE, then the RoPE key into the row and into y (kr_out).
constexpr int kProjStore = 0, kProjLatentRow = 1, kProjRopeRow = 2;
constexpr int kProjMaxJobs = 3;
struct ProjBatch {
  ProjJob job[kProjMaxJobs];
  int32_t n_jobs;
  int32_t B;
  int32_t mgroups;  // groups of 32 sequences
  const int32_t* positions;
  float rope_base;
  // pool rows (row epilogues)
  void* pool;
  const int32_t* page_table;  // nullptr: identity layout
  int32_t page_size, max_pages, num_pages;
  int32_t row_bytes;  // bytes per pool row
  int32_t d_c, d_r;
  int32_t fp8;        // FP8 E4M3FN latent codes (else bf16): 1 one cache scale, 2 block scales
  float cache_inv;    // FP8: fp32 reciprocal of the cache scale
  void* c_out;        // latent before rounding/encoding: fp32 (FP8) or bf16; may be null
  const uint16_t* kr_src;  // bf16 RoPE keys [B][d_r] to copy into the rows; may be null
  float* lat;         // fp8 == 2: the fp32 latents [B][d_c], encoded into the rows afterwards
  int32_t n_blocks;   // fp8 == 2: latent blocks per row
};

// ------------------------------------------------------------- device helpers

// Nearest OCP E4M3FN code of x, ties to even; magnitudes of 448 and above
// saturate to 448 and NaN gives 0x7F. Codes in the binade [2^E, 2^(E+1))
// (E >= -6) are spaced 2^(E-3) and the subnormal spacing 2^-9 continues below
// 2^-6, so with E' = max(E, -6) the nearest multiple n 2^(E'-3) of |x|
// (n in 0..16) has code (E' + 6) 8 + n.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  if (x != x) return 0x7Fu;
  const uint32_t sgn = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a >= 448.f) return sgn | 0x7Eu;
  int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // floor(log2 a); zero -> -127
  if (e < -6) e = -6;
  const float n = rintf(a * __uint_as_float(static_cast<uint32_t>(130 - e) << 23));  // a 2^(3-e), exact
  return sgn | static_cast<uint32_t>((e + 6) * 8 + static_cast<int>(n));
}

// Four consecutive weighted-latent values of a partial, fp32 or fp16 storage.
template <bool PH>
__device__ __forceinline__ float4 load_partial4(const char* po, int64_t i);
template <>
__device__ __forceinline__ float4 load_partial4<false>(const char* po, int64_t i) {
  return *reinterpret_cast<const float4*>(po + 4 * i);
}
template <>
__device__ __forceinline__ float4 load_partial4<true>(const char* po, int64_t i) {
  typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
  const half4_t v = *reinterpret_cast<const half4_t*>(po + 2 * i);
  return make_float4(static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                     static_cast<float>(v[3]));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ T store_cast(float v);
template <>
__device__ __forceinline__ float store_cast<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t store_cast<uint16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work split: the concatenated tiles of all sequences are cut into `units`
// contiguous ranges of near-equal length; unit u owns [tile_begin(u), tile_begin(u+1)).
__device__ __forceinline__ int32_t tile_begin(int32_t u, int32_t n_tiles, int32_t units) {
  return static_cast<int32_t>((static_cast<int64_t>(u) * n_tiles) / units);
}
__device__ __forceinline__ bool unit_owns_tiles(int32_t u, int32_t n_tiles, int32_t units) {
  return tile_begin(u + 1, n_tiles, units) > tile_begin(u, n_tiles, units);
}
// The unit whose range contains tile x (largest u with tile_begin(u) <= x).
__device__ __forceinline__ int32_t unit_of_tile(int32_t x, int32_t n_tiles, int32_t units) {
  return static_cast<int32_t>(((static_cast<int64_t>(x) + 1) * units - 1) / n_tiles);
}

}  // namespace mlra
