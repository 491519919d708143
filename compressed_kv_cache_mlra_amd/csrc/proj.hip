// Projections on either side of the attention (lesty.tech MLA explainer,
// section 4: the decoupled RoPE key k^R = RoPE(h W^KR) and the query split the
// same way; the query path c^Q = h W^DQ, q^C_i = c^Q W^UQ_i,
// q^R_i = RoPE(c^Q W^QR_i)). One kernel shape serves all of them:
//   y[b][m][n] = sum_k x[b][k] W_m[k][n]      (W_m stored [K][N], m = head)
// optionally followed by RoPE on each output vector (RoFormer's rotation:
// pairs (2i, 2i+1) turn by pos_b * base^(-2i/N)).
//
// Workgroup: 32 output columns (4 column groups of 8, one 16-byte weight row
// load per k each) x 64 k-lanes x up to 8 sequences, so every weight element
// loaded serves 8 sequences; x is staged in LDS in chunks of 1024; the 64
// k-lanes are summed in LDS, fp32 throughout, one rounding at the end.
#include <string.h>

#include <algorithm>
#include <cfloat>
#include <initializer_list>

#include "../../include/mlra.h"
#include "common.h"
#include "launch.h"
#include "validate.h"

namespace mlra {
namespace {

constexpr int kPThreads = 256;
constexpr int kPColGroups = 4;
constexpr int kPCols = 8 * kPColGroups;
constexpr int kPKLanes = kPThreads / kPColGroups;
constexpr int kPSeq = 8;
constexpr int kPXChunk = 1024;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_w8(const void* p, bool bf16, float* w) {
  if (bf16) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t u = v[j >> 1];
      w[j] = __uint_as_float((j & 1) ? (u & 0xffff0000u) : (u << 16));
    }
  } else {
    const u32x4_t a = reinterpret_cast<const u32x4_t*>(p)[0], b = reinterpret_cast<const u32x4_t*>(p)[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = __uint_as_float(a[j]);
      w[4 + j] = __uint_as_float(b[j]);
    }
  }
}

__global__ __launch_bounds__(kPThreads) void proj_kernel(ProjArgs a) {
  __shared__ float xs[kPSeq][kPXChunk];
  __shared__ float red[kPKLanes][kPCols + 1];
  const int tid = threadIdx.x;
  const int g = tid % kPColGroups, kl = tid / kPColGroups;
  const int n0 = blockIdx.x * kPCols;
  const int b0 = blockIdx.y * kPSeq;
  const int m = blockIdx.z;
  const int nb = min(kPSeq, a.B - b0);
  const int col = n0 + 8 * g;
  const bool col_ok = col < a.N;  // N is a multiple of 8
  const size_t welem = a.w_bf16 ? 2 : 4;
  const char* wbase = static_cast<const char*>(a.w) + static_cast<int64_t>(m) * a.w_mstride * welem;

  float acc[kPSeq][8];
#pragma unroll
  for (int s = 0; s < kPSeq; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[s][j] = 0.f;

  for (int k0 = 0; k0 < a.K; k0 += kPXChunk) {
    const int kn = min(kPXChunk, a.K - k0);
    __syncthreads();
    for (int i = tid; i < kPSeq * kn; i += kPThreads) {
      const int s = i / kn, k = i % kn;
      float v = 0.f;
      if (s < nb) {
        const int64_t idx = static_cast<int64_t>(b0 + s) * a.x_bstride + k0 + k;
        v = a.x_f32 ? static_cast<const float*>(a.x)[idx]
                    : bf16_to_f32(static_cast<const uint16_t*>(a.x)[idx]);
      }
      xs[s][k] = v;
    }
    __syncthreads();
    if (col_ok) {
      for (int r0 = kl; r0 < kn; r0 += kPKLanes * 4) {
        float w[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = min(r0 + u * kPKLanes, kn - 1);  // rows past the chunk are loaded, not used
          load_w8(wbase + (static_cast<int64_t>(k0 + r) * a.N + col) * welem, a.w_bf16, w[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = r0 + u * kPKLanes;
          if (r < kn) {
#pragma unroll
            for (int s = 0; s < kPSeq; ++s) {
              const float xv = xs[s][r];
#pragma unroll
              for (int j = 0; j < 8; ++j) acc[s][j] += xv * w[u][j];
            }
          }
        }
      }
    }
  }

  // tid < 32: output column n0 + tid; s unrolled so acc stays in registers
  const int n = n0 + tid;
#pragma unroll
  for (int s = 0; s < kPSeq; ++s) {
    if (s >= nb) break;  // uniform
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) red[kl][8 * g + j] = acc[s][j];
    __syncthreads();
    float v = 0.f;
    if (tid < kPCols)
      for (int q = 0; q < kPKLanes; ++q) v += red[q][tid];
    __syncthreads();
    if (tid < kPCols) red[0][tid] = v;  // the sums, for the RoPE partner
    __syncthreads();
    if (tid < kPCols && n < a.N) {
      if (a.rope) {
        // pair (n & ~1, n | 1) turns by pos * base^(-2 i / N), i = n / 2
        const float other = red[0][tid ^ 1];
        const int i = n >> 1;
        const double ang = static_cast<double>(a.positions[b0 + s]) *
                           pow(static_cast<double>(a.rope_base), -2.0 * i / a.N);
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float cs = static_cast<float>(cd), sn = static_cast<float>(sd);
        v = (n & 1) ? other * sn + v * cs : v * cs - other * sn;
      }
      const int64_t o = static_cast<int64_t>(b0 + s) * a.y_bstride + static_cast<int64_t>(m) * a.y_mstride + n;
      if (a.y_bf16)
        static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(v);
      else
        static_cast<float*>(a.y)[o] = v;
    }
  }
}


// ---------------------------------------------------------------- MFMA path
// At decode batch sizes the products are skinny GEMMs ([B x K] x [K x N] with
// B of a few dozen) whose weights stream from HBM once; in fp32 VALU the
// multiply-adds alone would outlast the weight reads, so they go to
// v_mfma_f32_16x16x32_bf16 with the sequences as MFMA rows (A = x) and the
// weight columns as MFMA columns (B = W).
//
// The B operand wants 8 consecutive k of one column per lane, while W is
// stored [K][N] (columns contiguous). Each lane therefore loads CPL
// consecutive columns of 8 consecutive rows (8 small row loads; the 16 lanes
// of a row group cover 16 CPL contiguous columns) and transposes the 8 x CPL
// block in registers with v_perm_b32 into CPL operands. Operand e of lane c
// holds column CPL c + e, so MFMA tile e's output column c is weight column
// CPL c + e; the epilogue undoes that permutation.
//
// Workgroup: 8 waves split the K rows (k-steps of 32 rows, wave-interleaved,
// 3 or 6 k-steps of loads in flight per wave), 32 sequences (two MFMA row tiles),
// one tile of 16 CPL columns; the 8 partial accumulators are summed in LDS in
// a fixed order, then RoPE (pairs 2i, 2i+1, fp64 angles) and the store.
// An fp32 x (the compressed query) is split into bf16 hi + lo parts, two
// MFMAs each, which keeps about 16 significant bits of it.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kMW = 8;   // waves per workgroup
constexpr int kMT = 2;   // 16-sequence MFMA row tiles per workgroup

__device__ __forceinline__ floatx4_t mfma_bf16(u32x4_t a, u32x4_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // inputs here are finite
}

// hi + lo bf16 split of 8 fp32 values: hi = RNE(v), lo = RNE(v - hi).
__device__ __forceinline__ void split8(const u32x4_t& f0, const u32x4_t& f1, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float a = __uint_as_float(u < 2 ? f0[2 * u] : f1[2 * u - 4]);
    const float b = __uint_as_float(u < 2 ? f0[2 * u + 1] : f1[2 * u - 3]);
    const uint32_t ha = bf16_rne_bits(a), hb = bf16_rne_bits(b);
    hi[u] = ha | (hb << 16);
    const uint32_t la = bf16_rne_bits(a - __uint_as_float(ha << 16));
    const uint32_t lb = bf16_rne_bits(b - __uint_as_float(hb << 16));
    lo[u] = la | (lb << 16);
  }
}

template <int CPL>
struct RowBits;
template <>
struct RowBits<4> {
  typedef uint32_t v_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(1))) const v_t g_t;
};
template <>
struct RowBits<2> {
  typedef uint32_t v_t;
  typedef __attribute__((address_space(1))) const uint32_t g_t;
};

typedef __attribute__((address_space(1))) const u32x4_t gq_t;

__device__ __forceinline__ uint32_t bf16_pair(float v0, float v1) {
  return static_cast<uint32_t>(f32_to_bf16(v0)) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
}

// Byte address of the pool row of token positions[m], or nullptr when the
// position or its page is out of range (nothing is written then).
__device__ __forceinline__ uint8_t* pool_row(const ProjBatch& a, int m) {
  const int32_t pos = a.positions[m];
  if (pos < 0 || pos >= a.max_pages * a.page_size) return nullptr;
  const int32_t pidx = pos / a.page_size;
  const int32_t phys = a.page_table ? a.page_table[static_cast<int64_t>(m) * a.max_pages + pidx]
                                    : m * a.max_pages + pidx;
  if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) return nullptr;
  return static_cast<uint8_t*>(a.pool) +
         (static_cast<int64_t>(phys) * a.page_size + pos % a.page_size) * a.row_bytes;
}

// Block-scaled FP8 rows of the appended tokens (one workgroup per token, one
// wave per latent block): the block's scale is its largest magnitude over 448
// in fp32 (NaN values left out), or 1 where that is 0, below the smallest
// normal fp32 or not finite; each code is the nearest E4M3FN of c x fp32(1 /
// scale). Writes the codes, the scales and the row's zero pad; the RoPE key
// was written by the product's epilogue.
__global__ __launch_bounds__(256) void encode_block_scaled_kernel(ProjBatch a) {
  const int m = blockIdx.x;
  uint8_t* row = pool_row(a, m);
  if (!row) return;
  const int w = a.d_c / a.n_blocks;
  const float* c = a.lat + static_cast<int64_t>(m) * a.d_c;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = wave; j < a.n_blocks; j += 4) {
    float amax = 0.f;
    for (int i = lane; i < w; i += 64) amax = fmaxf(amax, fabsf(c[j * w + i]));  // fmaxf skips NaN
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    float sc = amax / 448.f;
    if (!(sc >= FLT_MIN) || isinf(sc)) sc = 1.f;
    const float inv = 1.f / sc;
    for (int i = lane; i < w; i += 64) row[j * w + i] = static_cast<uint8_t>(e4m3_encode(c[j * w + i] * inv));
    if (lane == 0) *reinterpret_cast<float*>(row + a.d_c + 2 * a.d_r + 4 * j) = sc;
  }
  for (int i = a.d_c + 2 * a.d_r + 4 * a.n_blocks + threadIdx.x; i < a.row_bytes; i += 256) row[i] = 0;
}

// Output pair (n, n + 1) of sequence m and matrix mat: RoPE (pair index n / 2,
// angle pos base^(-n / N) in fp64) if the job asks for it, then one rounding,
// into the job's destination.
__device__ __forceinline__ void proj_store(const ProjJob& jb, const ProjBatch& a, int mat, int m, int n, float v0,
                                           float v1) {
  if (jb.kind == kProjLatentRow) {
    uint8_t* row = pool_row(a, m);
    if (!row) return;
    if (a.fp8 == 2) {
      // block scales need the whole block: keep the fp32 latent for the encoder
      float* l = a.lat + static_cast<int64_t>(m) * a.d_c + n;
      l[0] = v0;
      l[1] = v1;
    } else if (a.fp8) {
      *reinterpret_cast<uint16_t*>(row + n) =
          static_cast<uint16_t>(e4m3_encode(v0 * a.cache_inv) | (e4m3_encode(v1 * a.cache_inv) << 8));
    }
    if (a.fp8) {
      if (a.c_out) {
        float* c = static_cast<float*>(a.c_out) + static_cast<int64_t>(m) * a.d_c + n;
        c[0] = v0;
        c[1] = v1;
      }
    } else {
      const uint32_t pr = bf16_pair(v0, v1);
      *reinterpret_cast<uint32_t*>(row + 2 * n) = pr;
      if (a.c_out)
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.c_out) + static_cast<int64_t>(m) * a.d_c + n) = pr;
    }
    if (a.kr_src) {
      // the given RoPE key: pairs n, n + d_c, ... of it
      uint16_t* rope = reinterpret_cast<uint16_t*>(row + (a.fp8 ? a.d_c : 2 * a.d_c));
      for (int r = n; r < a.d_r; r += a.d_c)
        *reinterpret_cast<uint32_t*>(rope + r) =
            *reinterpret_cast<const uint32_t*>(a.kr_src + static_cast<int64_t>(m) * a.d_r + r);
    }
    return;
  }
  if (jb.rope) {
    const double ang = static_cast<double>(a.positions[m]) *
                       pow(static_cast<double>(a.rope_base), -2.0 * (n >> 1) / jb.N);
    double sd, cd;
    sincos(ang, &sd, &cd);
    const float cs = static_cast<float>(cd), sn = static_cast<float>(sd);
    const float r0 = v0 * cs - v1 * sn, r1 = v0 * sn + v1 * cs;
    v0 = r0;
    v1 = r1;
  }
  if (jb.kind == kProjRopeRow) {
    uint8_t* row = pool_row(a, m);
    if (row) *reinterpret_cast<uint32_t*>(row + (a.fp8 ? a.d_c : 2 * a.d_c) + 2 * n) = bf16_pair(v0, v1);
  }
  if (!jb.y) return;
  const int64_t o = static_cast<int64_t>(m) * jb.y_bstride + static_cast<int64_t>(mat) * jb.y_mstride + n;
  if (jb.y_f32) {
    float* y = static_cast<float*>(jb.y) + o;
    y[0] = v0;
    y[1] = v1;
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(jb.y) + o) = bf16_pair(v0, v1);
  }
}

// k-steps of loads in flight per wave (at workload 7's shape 3 and 6 measured
// 30.8 us for project_token against 31.4 with 2 and 4, outputs identical)
constexpr int proj_kmd(int cpl) { return cpl == 4 ? 3 : 6; }

template <int CPL, bool XF>
__global__ __launch_bounds__(kMW * 64) void proj_mfma_kernel(ProjBatch a) {
  constexpr int TC = 16 * CPL;  // tile columns
  constexpr int NR = kMT * CPL * 4;
  constexpr int kMD = proj_kmd(CPL);  // register budget
  typedef typename RowBits<CPL>::v_t v_t;
  typedef typename RowBits<CPL>::g_t g_t;
  __shared__ float red[kMW][NR][64];
  __shared__ float fin[kMT * 16][TC + 1];

  int id = blockIdx.x;
  // the job this workgroup belongs to (id becomes the index inside it),
  // copied with constant indices so the arguments stay out of scratch memory
  int jsel = 0;
  if (a.n_jobs > 1 && id >= a.job[0].wgs) {
    id -= a.job[0].wgs;
    jsel = 1;
    if (a.n_jobs > 2 && id >= a.job[1].wgs) {
      id -= a.job[1].wgs;
      jsel = 2;
    }
  }
  ProjJob jb;
  if (jsel == 0) __builtin_memcpy(&jb, &a.job[0], sizeof(ProjJob));
  else if (jsel == 1) __builtin_memcpy(&jb, &a.job[1], sizeof(ProjJob));
  else __builtin_memcpy(&jb, &a.job[2], sizeof(ProjJob));
  const int K = jb.K, N = jb.N, B = a.B;
  const int tile = id % jb.tiles;
  int rest = id / jb.tiles;
  const int slice = rest % jb.ksplit;
  rest /= jb.ksplit;
  const int mg = rest % a.mgroups;
  const int mat = rest / a.mgroups;
  const int n0 = tile * TC, m0 = mg * (16 * kMT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const bool col_ok = n0 + CPL * c < N;
  // Every load is issued unconditionally from a clamped, valid address and
  // out-of-range operands are zeroed when used: a load whose destination is
  // zeroed on another path makes the compiler wait for all loads in flight.
  const uint16_t* wp = jb.w + static_cast<int64_t>(mat) * jb.w_mstride + (col_ok ? n0 + CPL * c : 0);
  const int k_lo = slice * jb.kper;                        // this slice's k-steps
  const int k_hi = min((K + 31) / 32, k_lo + jb.kper);
  int64_t xrow[kMT];
  bool m_ok[kMT];
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    const int m = m0 + 16 * t + c;
    m_ok[t] = m < B;
    xrow[t] = static_cast<int64_t>(m_ok[t] ? m : B - 1) * jb.x_bstride;
  }

  floatx4_t acc[kMT][CPL];
#pragma unroll
  for (int t = 0; t < kMT; ++t)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[t][e] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int ks0 = k_lo + wave; ks0 < k_hi; ks0 += kMW * kMD) {
    v_t rw[kMD][8];
    u32x4_t ax[kMD][kMT][XF ? 2 : 1];
    bool kv[kMD];
#pragma unroll
    for (int d = 0; d < kMD; ++d) {
      const int ks = ks0 + d * kMW;
      const int kb = 32 * ks + 8 * g;  // this lane's 8 rows
      kv[d] = ks < k_hi && kb < K;     // K % 8 == 0: an 8-row group is whole or absent
      const int kc = kv[d] ? kb : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) rw[d][j] = *(g_t*)(wp + static_cast<int64_t>(kc + j) * N);
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        if constexpr (XF) {
          const float* xr = static_cast<const float*>(jb.x) + xrow[t] + kc;
          ax[d][t][0] = *(gq_t*)(xr);
          ax[d][t][1] = *(gq_t*)(xr + 4);
        } else {
          ax[d][t][0] = *(gq_t*)(static_cast<const uint16_t*>(jb.x) + xrow[t] + kc);
        }
      }
    }
    // keep every load of the chunk ahead of its first use (the scheduler
    // would otherwise interleave them with the MFMAs, one k-step in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kMD; ++d) {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      u32x4_t ahi[kMT], alo[kMT];
#pragma unroll
      for (int t = 0; t < kMT; ++t) {
        if constexpr (XF) {
          split8(ax[d][t][0], ax[d][t][1], ahi[t], alo[t]);
          if (!(kv[d] && m_ok[t])) alo[t] = z;
        } else {
          ahi[t] = ax[d][t][0];
        }
        if (!(kv[d] && m_ok[t])) ahi[t] = z;
      }
      const bool bok = kv[d] && col_ok;
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t bv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint32_t r0, r1;
          if constexpr (CPL == 4) {
            r0 = rw[d][2 * u][e >> 1];
            r1 = rw[d][2 * u + 1][e >> 1];
          } else {
            r0 = rw[d][2 * u];
            r1 = rw[d][2 * u + 1];
          }
          bv[u] = bok ? __builtin_amdgcn_perm(r1, r0, sel) : 0u;
        }
#pragma unroll
        for (int t = 0; t < kMT; ++t) {
          acc[t][e] = mfma_bf16(ahi[t], bv, acc[t][e]);
          if constexpr (XF) acc[t][e] = mfma_bf16(alo[t], bv, acc[t][e]);
        }
      }
    }
  }

  // sum the waves' accumulators in a fixed order
#pragma unroll
  for (int t = 0; t < kMT; ++t)
#pragma unroll
    for (int e = 0; e < CPL; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][(t * CPL + e) * 4 + i][lane] = acc[t][e][i];
  __syncthreads();
  for (int q = threadIdx.x; q < NR * 64; q += kMW * 64) {
    const int r = q >> 6, ln = q & 63;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kMW; ++w) v += red[w][r][ln];
    const int t = r / (CPL * 4), e = (r >> 2) % CPL, i = r & 3;
    fin[16 * t + 4 * (ln >> 4) + i][CPL * (ln & 15) + e] = v;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < kMT * 16 * (TC / 2); p += kMW * 64) {
    const int ml = p / (TC / 2), np = p % (TC / 2);
    const int m = m0 + ml, n = n0 + 2 * np;
    if (m >= B || n >= N) continue;
    const float v0 = fin[ml][2 * np], v1 = fin[ml][2 * np + 1];
    if (jb.ksplit > 1) {
      float* pp = jb.part + ((static_cast<int64_t>(slice) * jb.n_mats + mat) * B + m) * N + n;
      pp[0] = v0;
      pp[1] = v1;
    } else {
      proj_store(jb, a, mat, m, n, v0, v1);
    }
  }
}

// Sums the K slices of every output pair in slice order, then the epilogue.
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjBatch a) {
  int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int B = a.B;
#pragma unroll
  for (int j = 0; j < kProjMaxJobs; ++j) {
    if (j >= a.n_jobs) return;
    const ProjJob& jb = a.job[j];
    const int half = jb.N / 2;
    const int64_t pairs = static_cast<int64_t>(jb.n_mats) * B * half;
    if (jb.ksplit > 1 && q < pairs) {
      const int np = static_cast<int>(q % half);
      const int64_t mm = q / half;
      const int m = static_cast<int>(mm % B), mat = static_cast<int>(mm / B);
      const int n = 2 * np;
      float v0 = 0.f, v1 = 0.f;
      for (int s = 0; s < jb.ksplit; ++s) {
        const float* pp = jb.part + ((static_cast<int64_t>(s) * jb.n_mats + mat) * B + m) * jb.N + n;
        v0 += pp[0];
        v1 += pp[1];
      }
      proj_store(jb, a, mat, m, n, v0, v1);
      return;
    }
    if (jb.ksplit > 1) q -= pairs;
  }
}
}  // namespace

hipError_t launch_proj(const ProjArgs& a, int n_mats, hipStream_t stream) {
  const dim3 grid((a.N + kPCols - 1) / kPCols, (a.B + kPSeq - 1) / kPSeq, n_mats);
  proj_kernel<<<grid, kPThreads, 0, stream>>>(a);
  return hipGetLastError();
}

namespace {

// About 192 workgroups per launch: the up-projection launch of a 32-sequence
// batch (192 column tiles) then needs no K split and no reduce launch, and the
// x launch splits three ways. project_token at B = 32, d_model = 4096,
// d_cq = 1536, h = 64 (interleaved, settled clocks): 35.4 us with 512, 36.5
// with 256, 31.3 with 192, 31.4 with 128, 33.6 with 64 (no split at all).
constexpr int kTargetWgs = 192;

// Tiles, K slices and workgroups of every job; returns the partial bytes.
// A job is split along K until the launch has about kTargetWgs workgroups,
// each wave of a slice then issues its loads in one go; never more slices
// than k-step groups of one wave pass (8 waves x k-steps in flight).
size_t plan_proj(ProjBatch& b, int cpl) {
  b.mgroups = (b.B + 16 * kMT - 1) / (16 * kMT);
  int64_t base = 0;
  for (int j = 0; j < b.n_jobs; ++j) {
    ProjJob& jb = b.job[j];
    jb.tiles = (jb.N + 16 * cpl - 1) / (16 * cpl);
    base += static_cast<int64_t>(jb.tiles) * b.mgroups * jb.n_mats;
  }
  const int want = static_cast<int>(std::max<int64_t>(1, (kTargetWgs + base - 1) / base));
  size_t bytes = 0;
  for (int j = 0; j < b.n_jobs; ++j) {
    ProjJob& jb = b.job[j];
    const int ks = (jb.K + 31) / 32;
    const int pass = kMW * proj_kmd(cpl);
    const int most = (ks + pass - 1) / pass;
    int split = std::min(want, most);
    jb.kper = (ks + split - 1) / split;
    jb.ksplit = (ks + jb.kper - 1) / jb.kper;  // no empty slice
    jb.wgs = jb.tiles * b.mgroups * jb.n_mats * jb.ksplit;
    if (jb.ksplit > 1)
      bytes += (sizeof(float) * static_cast<size_t>(jb.ksplit) * jb.n_mats * b.B * jb.N + 255) / 256 * 256;
  }
  return bytes;
}

}  // namespace

size_t proj_mfma_scratch_bytes(ProjBatch b, int cpl) { return plan_proj(b, cpl); }

hipError_t launch_proj_mfma(ProjBatch& b, int cpl, void* scratch, hipStream_t stream) {
  plan_proj(b, cpl);
  int total = 0;
  int64_t pairs = 0;
  char* sp = static_cast<char*>(scratch);
  for (int j = 0; j < b.n_jobs; ++j) {
    ProjJob& jb = b.job[j];
    total += jb.wgs;
    if (jb.ksplit > 1) {
      jb.part = reinterpret_cast<float*>(sp);
      const size_t n = sizeof(float) * static_cast<size_t>(jb.ksplit) * jb.n_mats * b.B * jb.N;
      sp += (n + 255) / 256 * 256;
      pairs += static_cast<int64_t>(jb.n_mats) * b.B * (jb.N / 2);
    }
  }
  const bool xf = b.job[0].x_f32 != 0;  // every job of a launch has the same x type
  if (cpl == 4 && xf)
    proj_mfma_kernel<4, true><<<total, kMW * 64, 0, stream>>>(b);
  else if (cpl == 4)
    proj_mfma_kernel<4, false><<<total, kMW * 64, 0, stream>>>(b);
  else if (xf)
    proj_mfma_kernel<2, true><<<total, kMW * 64, 0, stream>>>(b);
  else
    proj_mfma_kernel<2, false><<<total, kMW * 64, 0, stream>>>(b);
  if (pairs > 0) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    proj_reduce_kernel<<<static_cast<unsigned>((pairs + 255) / 256), 256, 0, stream>>>(b);
  }
  return hipGetLastError();
}

}  // namespace mlra

// ------------------------------------------------------------------ C ABI

namespace {

int proj_status(hipError_t e) { return e == hipSuccess ? MLRA_OK : MLRA_ERR_HIP; }

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

float rope_base_of(const mlra_desc* d) { return d->rope_base > 0.f ? d->rope_base : 10000.f; }

// Element type of x, the weights and the outputs (bf16 for FP8 caches).
bool elems_bf16(const mlra_desc* d) { return d->dtype != MLRA_F32; }

// The MFMA path needs bf16 weights, rows of x in whole 16-byte chunks and
// 16-byte aligned arrays; anything else runs on the fp32 VALU kernel.
bool mfma_path(const mlra_desc* d, std::initializer_list<const void*> ptrs) {
  if (!elems_bf16(d) || d->d_model % 8 != 0) return false;
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return false;
  return true;
}

mlra::ProjJob job(const void* x, int64_t x_bstride, bool x_f32, const void* w, int64_t w_mstride, void* y,
                  int64_t y_bstride, int64_t y_mstride, bool y_f32, int K, int N, bool rope, int n_mats) {
  mlra::ProjJob j;
  memset(&j, 0, sizeof(j));
  j.x = x;
  j.x_bstride = x_bstride;
  j.x_f32 = x_f32;
  j.w = static_cast<const uint16_t*>(w);
  j.w_mstride = w_mstride;
  j.y = y;
  j.y_bstride = y_bstride;
  j.y_mstride = y_mstride;
  j.y_f32 = y_f32;
  j.K = K;
  j.N = N;
  j.rope = rope;
  j.n_mats = n_mats;
  return j;
}

// The MFMA launches of the two entry points (pointers may be null when sizing).
mlra::ProjBatch rope_batch(const mlra_desc* d, const void* x, const void* w_kr, const int32_t* pos, void* kr) {
  mlra::ProjBatch b;
  memset(&b, 0, sizeof(b));
  b.job[0] = job(x, d->d_model, false, w_kr, 0, kr, d->d_r, 0, false, d->d_model, d->d_r, true, 1);
  b.n_jobs = 1;
  b.B = d->batch;
  b.positions = pos;
  b.rope_base = rope_base_of(d);
  return b;
}

// c^Q = x W^DQ, kept in fp32
mlra::ProjBatch query_batch1(const mlra_desc* d, const void* x, const void* w_dq, float* c_q) {
  mlra::ProjBatch b;
  memset(&b, 0, sizeof(b));
  b.job[0] = job(x, d->d_model, false, w_dq, 0, c_q, d->d_cq, 0, true, d->d_model, d->d_cq, false, 1);
  b.n_jobs = 1;
  b.B = d->batch;
  return b;
}

// q^C_i = c^Q W^UQ_i and q^R_i = RoPE(c^Q W^QR_i), every head, one launch
mlra::ProjBatch query_batch2(const mlra_desc* d, const float* c_q, const void* w_uq, const void* w_qr,
                             const int32_t* pos, void* q_c, void* q_r) {
  const int H = d->n_heads, DQ = d->d_cq, DH = d->d_h, DR = d->d_r;
  mlra::ProjBatch b;
  memset(&b, 0, sizeof(b));
  b.job[0] = job(c_q, DQ, true, w_uq, static_cast<int64_t>(DQ) * DH, q_c, static_cast<int64_t>(H) * DH, DH, false,
                 DQ, DH, false, H);
  b.n_jobs = 1;
  if (DR > 0) {
    b.job[1] = job(c_q, DQ, true, w_qr, static_cast<int64_t>(DQ) * DR, q_r, static_cast<int64_t>(H) * DR, DR, false,
                   DQ, DR, true, H);
    b.n_jobs = 2;
  }
  b.B = d->batch;
  b.positions = pos;
  b.rope_base = rope_base_of(d);
  return b;
}

// The latent append (kProjLatentRow) into the pool rows of positions[b];
// kr_new (bf16) is copied into the rows' RoPE part.
void set_pool(mlra::ProjBatch& b, const mlra_desc* d, void* pool, const int32_t* page_table, void* c_out) {
  b.pool = pool;
  b.page_table = page_table;
  b.page_size = d->page_size;
  b.max_pages = d->max_pages_per_seq;
  b.num_pages = d->num_pages;
  b.fp8 = mlra::fp8_mode(d);
  b.row_bytes = b.fp8 ? mlra::fp8_row_bytes(d) : 2 * (d->d_c + d->d_r);
  b.n_blocks = d->n_blocks;
  b.d_c = d->d_c;
  b.d_r = d->d_r;
  b.cache_inv = 1.0f / (d->cache_scale > 0.f ? d->cache_scale : 1.0f);
  b.c_out = c_out;
}

mlra::ProjBatch append_batch(const mlra_desc* d, const void* x, const void* w_dkv, const int32_t* pos, void* pool,
                             const int32_t* page_table, const void* kr_new, void* c_out) {
  mlra::ProjBatch b;
  memset(&b, 0, sizeof(b));
  b.job[0] = job(x, d->d_model, false, w_dkv, 0, nullptr, 0, 0, false, d->d_model, d->d_c, false, 1);
  b.job[0].kind = mlra::kProjLatentRow;
  b.n_jobs = 1;
  b.B = d->batch;
  b.positions = pos;
  set_pool(b, d, pool, page_table, c_out);
  b.kr_src = static_cast<const uint16_t*>(kr_new);
  return b;
}

// Everything the new token's hidden state x feeds, one launch: its latent into
// the pool row, its RoPE key into the row (and kr_out), and (d_cq > 0) the
// compressed query c^Q.
mlra::ProjBatch token_batch(const mlra_desc* d, const void* x, const int32_t* pos, void* pool,
                            const int32_t* page_table, const void* w_dkv, const void* w_kr, void* kr_out, void* c_out,
                            const void* w_dq, float* c_q) {
  mlra::ProjBatch b = append_batch(d, x, w_dkv, pos, pool, page_table, nullptr, c_out);
  b.rope_base = rope_base_of(d);
  if (d->d_r > 0) {
    b.job[b.n_jobs] = job(x, d->d_model, false, w_kr, 0, kr_out, d->d_r, 0, false, d->d_model, d->d_r, true, 1);
    b.job[b.n_jobs].kind = mlra::kProjRopeRow;
    ++b.n_jobs;
  }
  if (d->d_cq > 0) {
    b.job[b.n_jobs] = job(x, d->d_model, false, w_dq, 0, c_q, d->d_cq, 0, true, d->d_model, d->d_cq, false, 1);
    ++b.n_jobs;
  }
  return b;
}

// kCplToken: four columns per lane for the x launch of project_token and the
// append, so a column tile covers whole 128-byte lines of each weight row (with
// two, neighbouring tiles on different XCDs each fetched the shared lines: 36.8
// MB from HBM for 17.3 MB of weights; 30.8 -> 29.8 us for project_token)
// kCplQuery1 likewise (mlra_project_query at the same shape: 28.4 -> 27.8 us);
// kCplRope stays at two (its 64-column matrix would get fewer workgroups:
// 10.1 -> 10.9 us with four)
constexpr int kCplRope = 2, kCplQuery1 = 4, kCplQuery2 = 4, kCplToken = 4;

// Checks the workspace and returns the start of the projection region.
int proj_scratch(const mlra_desc* d, void* workspace, size_t ws_bytes, void** scratch) {
  size_t off = 0, total = 0;
  const int st = mlra::proj_workspace_region(d, &off, &total);
  if (st != MLRA_OK) return st;
  if (!workspace) return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < total) return MLRA_ERR_WORKSPACE;
  *scratch = static_cast<char*>(workspace) + off;
  return MLRA_OK;
}

size_t splitk_scratch_bytes(const mlra_desc* d) {
  if (!elems_bf16(d) || d->d_model < 1 || d->d_model % 8 != 0) return 0;  // VALU path: no scratch
  size_t need = 0;
  if (d->d_c % 8 == 0 && d->d_r % 8 == 0) {
    need = std::max(need, proj_mfma_scratch_bytes(
                              append_batch(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), kCplToken));
    if (d->d_cq % 8 == 0)
      need = std::max(need, proj_mfma_scratch_bytes(token_batch(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                                nullptr, nullptr, nullptr, nullptr),
                                                    kCplToken));
  }
  if (d->d_r > 0 && d->d_r % 8 == 0)
    need = std::max(need, proj_mfma_scratch_bytes(rope_batch(d, nullptr, nullptr, nullptr, nullptr), kCplRope));
  if (d->d_cq > 0 && d->d_cq % 8 == 0 && d->d_h % 8 == 0 && d->d_r % 8 == 0) {
    need = std::max(need, proj_mfma_scratch_bytes(query_batch1(d, nullptr, nullptr, nullptr), kCplQuery1));
    need = std::max(need, proj_mfma_scratch_bytes(
                              query_batch2(d, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), kCplQuery2));
  }
  return need;
}

// Block-scaled FP8 caches: the fp32 latents [B][d_c] between the product and
// the encoder, after the split-K scratch.
size_t lat_offset(const mlra_desc* d) { return (splitk_scratch_bytes(d) + 255) / 256 * 256; }
float* lat_scratch(const mlra_desc* d, void* scratch) {
  return reinterpret_cast<float*>(static_cast<char*>(scratch) + lat_offset(d));
}

hipError_t encode_rows(const mlra::ProjBatch& b, hipStream_t stream) {
  if (b.fp8 != 2) return hipSuccess;
  mlra::encode_block_scaled_kernel<<<b.B, 256, 0, stream>>>(b);
  return hipGetLastError();
}

}  // namespace

size_t mlra::proj_scratch_bytes(const mlra_desc* d) {
  const size_t need = splitk_scratch_bytes(d);
  // block-scaled appends run on the MFMA product only (d_model % 8 == 0), which
  // may need no split-K scratch: the latents get their room regardless
  if (fp8_mode(d) != 2 || d->d_model < 1 || d->d_model % 8 != 0) return need;
  return lat_offset(d) + sizeof(float) * static_cast<size_t>(d->batch) * d->d_c;
}

extern "C" int mlra_rope_key(const mlra_desc* desc, const void* x, const void* w_kr,
                             const int32_t* positions, void* kr_out, void* workspace, size_t ws_bytes,
                             void* stream) {
  using namespace mlra;
  int st = check_desc(desc, nullptr);
  if (st != MLRA_OK) return st;
  if (desc->d_model < 1) return MLRA_ERR_INVALID_ARG;
  if (desc->d_r == 0) return MLRA_OK;
  if (desc->d_r % 8 != 0) return MLRA_ERR_UNSUPPORTED;
  if (!x || !w_kr || !positions || !kr_out || !aligned16(w_kr)) return MLRA_ERR_INVALID_ARG;
  void* scratch = nullptr;
  st = proj_scratch(desc, workspace, ws_bytes, &scratch);
  if (st != MLRA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma_path(desc, {x, kr_out})) {
    ProjBatch b = rope_batch(desc, x, w_kr, positions, kr_out);
    return proj_status(launch_proj_mfma(b, kCplRope, scratch, s));
  }
  const bool bf = elems_bf16(desc);
  ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.x_bstride = desc->d_model;
  a.x_f32 = !bf;
  a.w = w_kr;
  a.w_bf16 = bf;
  a.y = kr_out;
  a.y_bstride = desc->d_r;
  a.y_bf16 = bf;
  a.B = desc->batch;
  a.K = desc->d_model;
  a.N = desc->d_r;
  a.positions = positions;
  a.rope = 1;
  a.rope_base = rope_base_of(desc);
  return proj_status(launch_proj(a, 1, s));
}

extern "C" int mlra_project_query(const mlra_desc* desc, const void* x, const void* w_dq,
                                  const void* w_uq, const void* w_qr, const int32_t* positions,
                                  float* c_q, void* q_c, void* q_r, void* workspace, size_t ws_bytes,
                                  void* stream) {
  using namespace mlra;
  int st = check_desc(desc, nullptr);
  if (st != MLRA_OK) return st;
  if (desc->d_model < 1 || desc->d_cq < 1) return MLRA_ERR_INVALID_ARG;
  if (desc->d_cq % 8 != 0 || desc->d_h % 8 != 0 || desc->d_r % 8 != 0) return MLRA_ERR_UNSUPPORTED;
  if (!x || !w_dq || !w_uq || !c_q || !q_c) return MLRA_ERR_INVALID_ARG;
  if (desc->d_r > 0 && (!w_qr || !q_r || !positions)) return MLRA_ERR_INVALID_ARG;
  if (!aligned16(w_dq) || !aligned16(w_uq) || (desc->d_r > 0 && !aligned16(w_qr))) return MLRA_ERR_INVALID_ARG;
  void* scratch = nullptr;
  st = proj_scratch(desc, workspace, ws_bytes, &scratch);
  if (st != MLRA_OK) return st;
  const bool bf = elems_bf16(desc);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mfma_path(desc, {x, c_q, q_c, q_r})) {
    ProjBatch b1 = query_batch1(desc, x, w_dq, c_q);
    st = proj_status(launch_proj_mfma(b1, kCplQuery1, scratch, s));
    if (st != MLRA_OK) return st;
    ProjBatch b2 = query_batch2(desc, c_q, w_uq, w_qr, positions, q_c, q_r);
    return proj_status(launch_proj_mfma(b2, kCplQuery2, scratch, s));
  }
  ProjArgs a;
  memset(&a, 0, sizeof(a));
  // c^Q = x W^DQ, kept in fp32
  a.x = x;
  a.x_bstride = desc->d_model;
  a.x_f32 = !bf;
  a.w = w_dq;
  a.w_bf16 = bf;
  a.y = c_q;
  a.y_bstride = desc->d_cq;
  a.y_bf16 = 0;
  a.B = desc->batch;
  a.K = desc->d_model;
  a.N = desc->d_cq;
  st = proj_status(launch_proj(a, 1, s));
  if (st != MLRA_OK) return st;
  // q^C_i = c^Q W^UQ_i for every head i
  a.x = c_q;
  a.x_bstride = desc->d_cq;
  a.x_f32 = 1;
  a.w = w_uq;
  a.w_mstride = static_cast<int64_t>(desc->d_cq) * desc->d_h;
  a.y = q_c;
  a.y_bstride = static_cast<int64_t>(desc->n_heads) * desc->d_h;
  a.y_mstride = desc->d_h;
  a.y_bf16 = bf;
  a.K = desc->d_cq;
  a.N = desc->d_h;
  st = proj_status(launch_proj(a, desc->n_heads, s));
  if (st != MLRA_OK || desc->d_r == 0) return st;
  // q^R_i = RoPE(c^Q W^QR_i)
  a.w = w_qr;
  a.w_mstride = static_cast<int64_t>(desc->d_cq) * desc->d_r;
  a.y = q_r;
  a.y_bstride = static_cast<int64_t>(desc->n_heads) * desc->d_r;
  a.y_mstride = desc->d_r;
  a.N = desc->d_r;
  a.positions = positions;
  a.rope = 1;
  a.rope_base = rope_base_of(desc);
  return proj_status(launch_proj(a, desc->n_heads, s));
}

// Latent append on the MFMA path (bf16 x and W^DKV, d_model % 8 == 0, 16-byte
// aligned arrays); returns kNotEligible for the fp32 kernel's inputs.
int mlra::append_latent_mfma(const mlra_desc* desc, void* pool, const int32_t* page_table,
                             const int32_t* positions, const void* x, const void* w_dkv, const void* kr_new,
                             void* c_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!mfma_path(desc, {x, w_dkv, kr_new, c_out}) || desc->d_c % 8 != 0 || desc->d_r % 8 != 0) return kNotEligible;
  void* scratch = nullptr;
  const int st = proj_scratch(desc, workspace, ws_bytes, &scratch);
  if (st != MLRA_OK) return st;
  ProjBatch b = append_batch(desc, x, w_dkv, positions, pool, page_table, kr_new, c_out);
  b.lat = lat_scratch(desc, scratch);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int st2 = proj_status(launch_proj_mfma(b, kCplToken, scratch, s));
  if (st2 != MLRA_OK) return st2;
  return proj_status(encode_rows(b, s));
}

extern "C" int mlra_project_token(const mlra_desc* desc, const void* x, const int32_t* positions, void* pool,
                                  const int32_t* page_table, const void* w_dkv, const void* w_kr, void* kr_out,
                                  void* c_out, const void* w_dq, const void* w_uq, const void* w_qr, float* c_q,
                                  void* q_c, void* q_r, void* workspace, size_t ws_bytes, void* stream) {
  using namespace mlra;
  int st = check_desc(desc, nullptr);
  if (st != MLRA_OK) return st;
  if (desc->d_model < 1 || desc->d_cq < 0) return MLRA_ERR_INVALID_ARG;
  if (!x || !positions || !pool || !w_dkv || (desc->d_r > 0 && (!w_kr || !kr_out))) return MLRA_ERR_INVALID_ARG;
  if (desc->d_cq > 0 && (!w_dq || !w_uq || !c_q || !q_c || (desc->d_r > 0 && (!w_qr || !q_r))))
    return MLRA_ERR_INVALID_ARG;
  if (!aligned16(w_dkv) || (w_kr && !aligned16(w_kr)) || (w_dq && !aligned16(w_dq)) || (w_uq && !aligned16(w_uq)) ||
      (w_qr && !aligned16(w_qr)))
    return MLRA_ERR_INVALID_ARG;
  if (desc->d_r % 8 != 0 || desc->d_cq % 8 != 0 || desc->d_h % 8 != 0) return MLRA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  st = proj_scratch(desc, workspace, ws_bytes, &scratch);
  if (st != MLRA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!mfma_path(desc, {x, kr_out, c_out, c_q, q_c, q_r}) || desc->d_c % 8 != 0) {
    // the fp32 kernels, one product at a time
    if (desc->d_r > 0) {
      st = mlra_rope_key(desc, x, w_kr, positions, kr_out, workspace, ws_bytes, stream);
      if (st != MLRA_OK) return st;
    }
    st = mlra_append_latent(desc, pool, page_table, positions, x, w_dkv, kr_out, c_out, workspace, ws_bytes, stream);
    if (st != MLRA_OK || desc->d_cq == 0) return st;
    return mlra_project_query(desc, x, w_dq, w_uq, w_qr, positions, c_q, q_c, q_r, workspace, ws_bytes, stream);
  }
  ProjBatch b1 = token_batch(desc, x, positions, pool, page_table, w_dkv, w_kr, kr_out, c_out, w_dq, c_q);
  b1.lat = lat_scratch(desc, scratch);
  st = proj_status(launch_proj_mfma(b1, kCplToken, scratch, s));
  if (st == MLRA_OK) st = proj_status(encode_rows(b1, s));
  if (st != MLRA_OK || desc->d_cq == 0) return st;
  ProjBatch b2 = query_batch2(desc, c_q, w_uq, w_qr, positions, q_c, q_r);
  return proj_status(launch_proj_mfma(b2, kCplQuery2, scratch, s));
}
