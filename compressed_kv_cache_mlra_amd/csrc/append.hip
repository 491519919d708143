// Latent append: c_new = x W^DKV (ai360xpert concept page, "The two
// projections"; the cache keeps the latent, not per-head keys and values),
// accumulated in fp32, rounded once to the cache type, and written with the
// already-rotated RoPE key as the row [c_new | k^R_new] of token positions[b].
#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;                    // latent columns per workgroup
constexpr int kSlices = kThreads / kCols;    // d_model split inside the workgroup

// grid: n_chunks * batch, chunk fastest, so consecutive workgroups (which the
// dispatcher spreads over the 8 XCDs) cover different column chunks and each
// XCD's L2 keeps reusing one chunk of W^DKV across the batch.
template <typename T>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, int n_chunks) {
  __shared__ float red[kSlices][kCols];
  const int tid = threadIdx.x;
  const int chunk = blockIdx.x % n_chunks;
  const int b = blockIdx.x / n_chunks;
  const int col = chunk * kCols + (tid % kCols);
  const int slice = tid / kCols;
  const int32_t pos = a.positions[b];
  if (pos < 0 || pos >= a.max_pages * a.page_size) return;  // uniform per workgroup

  const T* x = static_cast<const T*>(a.x) + static_cast<int64_t>(b) * a.d_model;
  const T* w = static_cast<const T*>(a.w_dkv);
  float acc = 0.f;
  if (col < a.d_c) {
    int m = slice;
    for (; m + 3 * kSlices < a.d_model; m += 4 * kSlices) {
      const float x0 = load_elem(x, m), x1 = load_elem(x, m + kSlices);
      const float x2 = load_elem(x, m + 2 * kSlices), x3 = load_elem(x, m + 3 * kSlices);
      const float w0 = load_elem(w, static_cast<int64_t>(m) * a.d_c + col);
      const float w1 = load_elem(w, static_cast<int64_t>(m + kSlices) * a.d_c + col);
      const float w2 = load_elem(w, static_cast<int64_t>(m + 2 * kSlices) * a.d_c + col);
      const float w3 = load_elem(w, static_cast<int64_t>(m + 3 * kSlices) * a.d_c + col);
      acc += x0 * w0;
      acc += x1 * w1;
      acc += x2 * w2;
      acc += x3 * w3;
    }
    for (; m < a.d_model; m += kSlices) acc += load_elem(x, m) * load_elem(w, static_cast<int64_t>(m) * a.d_c + col);
  }
  red[slice][tid % kCols] = acc;
  __syncthreads();
  const int32_t pidx = pos / a.page_size;
  int32_t phys = a.page_table ? a.page_table[static_cast<int64_t>(b) * a.max_pages + pidx]
                              : b * a.max_pages + pidx;
  if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) return;  // uniform
  T* row = static_cast<T*>(a.pool) +
           (static_cast<int64_t>(phys) * a.page_size + (pos % a.page_size)) * a.row;
  if (tid < kCols && col < a.d_c) {
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < kSlices; ++s) v += red[s][tid];
    const T o = store_cast<T>(v);
    row[col] = o;
    if (a.c_out) static_cast<T*>(a.c_out)[static_cast<int64_t>(b) * a.d_c + col] = o;
  }
  if (chunk == 0) {
    const T* kr = static_cast<const T*>(a.kr_new) + static_cast<int64_t>(b) * a.d_r;
    for (int r = tid; r < a.d_r; r += kThreads) row[a.d_c + r] = kr[r];
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t stream) {
  const int n_chunks = (a.d_c + kCols - 1) / kCols;
  const dim3 grid(n_chunks * a.batch);
  if (dtype == 1)
    append_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(a, n_chunks);
  else
    append_kernel<float><<<grid, kThreads, 0, stream>>>(a, n_chunks);
  return hipGetLastError();
}

}  // namespace mlra
