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

}  // namespace

hipError_t launch_proj(const ProjArgs& a, int n_mats, hipStream_t stream) {
  const dim3 grid((a.N + kPCols - 1) / kPCols, (a.B + kPSeq - 1) / kPSeq, n_mats);
  proj_kernel<<<grid, kPThreads, 0, stream>>>(a);
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

}  // namespace

extern "C" int mlra_rope_key(const mlra_desc* desc, const void* x, const void* w_kr,
                             const int32_t* positions, void* kr_out, void* stream) {
  using namespace mlra;
  int st = check_desc(desc, nullptr);
  if (st != MLRA_OK) return st;
  if (desc->d_model < 1) return MLRA_ERR_INVALID_ARG;
  if (desc->d_r == 0) return MLRA_OK;
  if (desc->d_r % 8 != 0) return MLRA_ERR_UNSUPPORTED;
  if (!x || !w_kr || !positions || !kr_out || !aligned16(w_kr)) return MLRA_ERR_INVALID_ARG;
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
  return proj_status(launch_proj(a, 1, static_cast<hipStream_t>(stream)));
}

extern "C" int mlra_project_query(const mlra_desc* desc, const void* x, const void* w_dq,
                                  const void* w_uq, const void* w_qr, const int32_t* positions,
                                  float* c_q, void* q_c, void* q_r, void* stream) {
  using namespace mlra;
  int st = check_desc(desc, nullptr);
  if (st != MLRA_OK) return st;
  if (desc->d_model < 1 || desc->d_cq < 1) return MLRA_ERR_INVALID_ARG;
  if (desc->d_cq % 8 != 0 || desc->d_h % 8 != 0 || desc->d_r % 8 != 0) return MLRA_ERR_UNSUPPORTED;
  if (!x || !w_dq || !w_uq || !c_q || !q_c) return MLRA_ERR_INVALID_ARG;
  if (desc->d_r > 0 && (!w_qr || !q_r || !positions)) return MLRA_ERR_INVALID_ARG;
  if (!aligned16(w_dq) || !aligned16(w_uq) || (desc->d_r > 0 && !aligned16(w_qr))) return MLRA_ERR_INVALID_ARG;
  const bool bf = elems_bf16(desc);
  const hipStream_t s = static_cast<hipStream_t>(stream);
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
