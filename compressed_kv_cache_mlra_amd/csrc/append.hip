// Latent append: c_new = x W^DKV (ai360xpert concept page, "The two
// projections"; the cache keeps the latent, not per-head keys and values),
// accumulated in fp32, rounded once to the cache type, and written with the
// already-rotated RoPE key as the row [c_new | k^R_new] of token positions[b].
// FP8 caches (the latent quantisation the lesty.tech MLA explainer mentions
// in section 5) store each latent value as the nearest OCP E4M3FN code of
// c_new times the reciprocal of the cache scale.
#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kColGroups = 4;                 // 8 columns per thread: 32 latent columns per workgroup
constexpr int kCols = 8 * kColGroups;
constexpr int kKLanes = kThreads / kColGroups;  // threads splitting d_model inside the workgroup
constexpr int kXChunk = 4096;                   // d_model elements of x staged in LDS at a time
constexpr int kRowBatch = 16;                   // W^DKV rows per thread whose loads are in flight together

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Eight consecutive W^DKV elements as floats (one 16-byte load for bf16, two for fp32).
template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {
  u32x4_t v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t u = v[j >> 1];
    return __uint_as_float((j & 1) ? (u & 0xffff0000u) : (u << 16));
  }
};
template <>
struct Row8<float> {
  u32x4_t v0, v1;
  __device__ __forceinline__ void load(const float* p) {
    v0 = *reinterpret_cast<const u32x4_t*>(p);
    v1 = *reinterpret_cast<const u32x4_t*>(p + 4);
  }
  __device__ __forceinline__ float get(int j) const { return __uint_as_float(j < 4 ? v0[j] : v1[j - 4]); }
};

// grid: n_chunks * batch, chunk fastest, so consecutive workgroups (which the
// dispatcher spreads over the 8 XCDs) cover different column chunks and each
// XCD's L2 keeps reusing one chunk of W^DKV across the batch.
// Thread (col group g, k lane kl) accumulates columns [8 g, 8 g + 8) of the
// chunk over rows k = kl (mod 64) of W^DKV; the 64 k lanes are summed in LDS.
// T: element type of x, W^DKV and k^R_new; F8: the pool is an FP8 cache
// (codes then the bf16 RoPE key per row; c_out is fp32).
template <typename T, bool F8>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, int n_chunks) {
  __shared__ float xs[kXChunk];
  __shared__ float red[kKLanes][kCols + 1];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x % n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int g = tid % kColGroups, kl = tid / kColGroups;
  const int col0 = chunk * kCols + 8 * g;
  const bool col_ok = col0 < a.d_c;  // d_c is a multiple of 8 for bf16, of 4 for fp32 (checked below)
  const int32_t pos = a.positions[b];
  if (pos < 0 || pos >= a.max_pages * a.page_size) return;  // uniform per workgroup

  const T* x = static_cast<const T*>(a.x) + static_cast<int64_t>(b) * a.d_model;
  const T* w = static_cast<const T*>(a.w_dkv);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const bool full8 = col0 + 8 <= a.d_c;
  for (int k0 = 0; k0 < a.d_model; k0 += kXChunk) {
    const int kn = min(kXChunk, a.d_model - k0);
    __syncthreads();
    for (int i = tid; i < kn; i += kThreads) xs[i] = load_elem(x, k0 + i);
    __syncthreads();
    if (col_ok && full8) {
      for (int r0 = kl; r0 < kn; r0 += kKLanes * kRowBatch) {
        Row8<T> wr[kRowBatch];
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          const int r = min(r0 + u * kKLanes, kn - 1);  // rows past the chunk are loaded, not used
          wr[u].load(w + static_cast<int64_t>(k0 + r) * a.d_c + col0);
        }
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
          const int r = r0 + u * kKLanes;
          const float xv = r < kn ? xs[r] : 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] += xv * wr[u].get(j);
        }
      }
    } else if (col_ok) {
      // fp32 latent of 4 (mod 8) columns: the last group holds 4 columns
      for (int r = kl; r < kn; r += kKLanes) {
        const float xv = xs[r];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (col0 + j < a.d_c) acc[j] += xv * load_elem(w, static_cast<int64_t>(k0 + r) * a.d_c + col0 + j);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[kl][8 * g + j] = acc[j];
  __syncthreads();
  const int32_t pidx = pos / a.page_size;
  int32_t phys = a.page_table ? a.page_table[static_cast<int64_t>(b) * a.max_pages + pidx]
                              : b * a.max_pages + pidx;
  if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) return;  // uniform
  const int64_t row_index = static_cast<int64_t>(phys) * a.page_size + (pos % a.page_size);
  const int col = chunk * kCols + tid;
  const T* kr = static_cast<const T*>(a.kr_new) + static_cast<int64_t>(b) * a.d_r;
  if constexpr (F8) {
    uint8_t* row = static_cast<uint8_t*>(a.pool) + row_index * a.row;  // a.row: bytes
    if (tid < kCols && col < a.d_c) {
      float v = 0.f;
      for (int s = 0; s < kKLanes; ++s) v += red[s][tid];
      row[col] = static_cast<uint8_t>(e4m3_encode(v * a.cache_inv));
      if (a.c_out) static_cast<float*>(a.c_out)[static_cast<int64_t>(b) * a.d_c + col] = v;
    }
    if (chunk == 0) {
      T* rope = reinterpret_cast<T*>(row + a.d_c);
      for (int r = tid; r < a.d_r; r += kThreads) rope[r] = kr[r];
    }
  } else {
    T* row = static_cast<T*>(a.pool) + row_index * a.row;
    if (tid < kCols && col < a.d_c) {
      float v = 0.f;
      for (int s = 0; s < kKLanes; ++s) v += red[s][tid];
      const T o = store_cast<T>(v);
      row[col] = o;
      if (a.c_out) static_cast<T*>(a.c_out)[static_cast<int64_t>(b) * a.d_c + col] = o;
    }
    if (chunk == 0)
      for (int r = tid; r < a.d_r; r += kThreads) row[a.d_c + r] = kr[r];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t stream) {
  const int n_chunks = (a.d_c + kCols - 1) / kCols;
  const dim3 grid(n_chunks * a.batch);
  if (dtype == 2)
    append_kernel<uint16_t, true><<<grid, kThreads, 0, stream>>>(a, n_chunks);
  else if (dtype == 1)
    append_kernel<uint16_t, false><<<grid, kThreads, 0, stream>>>(a, n_chunks);
  else
    append_kernel<float, false><<<grid, kThreads, 0, stream>>>(a, n_chunks);
  return hipGetLastError();
}

}  // namespace mlra
