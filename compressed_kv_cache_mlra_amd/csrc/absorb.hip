// Query absorption and work planning.
//
// Absorption (lesty.tech MLA explainer, section 5; ai360xpert concept page,
// "Absorbing the up-projection"): the key up-projection folds into the query,
//   q~[b][i][jj][c] = s * sum_d W^UK[i][jj][c][d] q^C[b][i][d],
// and the RoPE part of the query is only scaled, q^R~ = s * q^R, with
// s = softmax_scale * log2(e) so the attention kernels work with base-2 logits.
#include "common.h"
#include "launch.h"

namespace mlra {

namespace {

constexpr int kAbsorbThreads = 256;
constexpr int kAbsorbBatchGroup = 8;

// grid: (hk, ceil(batch / kAbsorbBatchGroup)); block: kAbsorbThreads.
// Block (0, 0) also writes the work plan into the workspace header.
template <typename TIn, typename TQ>
__global__ __launch_bounds__(kAbsorbThreads) void absorb_kernel(DecodeArgs a, const int32_t* seq_lens,
                                                                 const TIn* __restrict__ q_c,
                                                                 const TIn* __restrict__ q_r,
                                                                 const TIn* __restrict__ w_uk) {
  extern __shared__ float q_sh[];  // [kAbsorbBatchGroup][d_h]
  __shared__ int32_t scan_sh[kAbsorbThreads];
  const int tid = threadIdx.x;
  const int hk = blockIdx.x;
  const int head = hk / a.k;
  const int b0 = blockIdx.y * kAbsorbBatchGroup;
  const int nb = min(kAbsorbBatchGroup, a.batch - b0);
  const int HK = a.n_heads * a.k;
  const int QW = a.w + a.d_r;

  if (blockIdx.x == 0 && blockIdx.y == 0) {
    // Plan: clamp lengths, count tiles per sequence, exclusive prefix sum.
    int32_t* cum = reinterpret_cast<int32_t*>(a.ws + a.off_cum);
    int32_t* nlen = reinterpret_cast<int32_t*>(a.ws + a.off_nlen);
    const int32_t cap = a.max_pages * a.page_size;
    int32_t carry = 0;
    for (int base = 0; base < a.batch; base += kAbsorbThreads) {
      const int b = base + tid;
      int32_t tiles = 0;
      if (b < a.batch) {
        int32_t n = seq_lens[b];
        n = n < 0 ? 0 : (n > cap ? cap : n);
        nlen[b] = n;
        tiles = (n + a.tile_tokens - 1) / a.tile_tokens;
      }
      scan_sh[tid] = tiles;
      __syncthreads();
      for (int off = 1; off < kAbsorbThreads; off <<= 1) {
        const int32_t v = tid >= off ? scan_sh[tid - off] : 0;
        __syncthreads();
        scan_sh[tid] += v;
        __syncthreads();
      }
      if (b < a.batch) cum[b] = carry + scan_sh[tid] - tiles;
      carry += scan_sh[kAbsorbThreads - 1];
      __syncthreads();
    }
    if (tid == 0) {
      cum[a.batch] = carry;
      WsHeader* h = reinterpret_cast<WsHeader*>(a.ws);
      h->magic = kWsMagic;
      h->flags = 0;
      h->n_tiles = carry;
      h->units = a.units;
      h->tile_tokens = a.tile_tokens;
      h->groups = a.groups;
      h->batch = a.batch;
      h->hk = HK;
    }
  }

  for (int e = tid; e < nb * a.d_h; e += kAbsorbThreads) {
    const int bl = e / a.d_h, d = e % a.d_h;
    q_sh[e] = load_elem(q_c, (static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_h + d);
  }
  __syncthreads();

  TQ* qext = reinterpret_cast<TQ*>(a.ws + a.off_qext);
  const TIn* wrow_base = w_uk + static_cast<int64_t>(hk) * a.w * a.d_h;
  for (int c = tid; c < a.w; c += kAbsorbThreads) {
    float acc[kAbsorbBatchGroup];
#pragma unroll
    for (int bl = 0; bl < kAbsorbBatchGroup; ++bl) acc[bl] = 0.f;
    const TIn* wrow = wrow_base + static_cast<int64_t>(c) * a.d_h;
    for (int d = 0; d < a.d_h; ++d) {
      const float wv = load_elem(wrow, d);
#pragma unroll
      for (int bl = 0; bl < kAbsorbBatchGroup; ++bl)
        if (bl < nb) acc[bl] += wv * q_sh[bl * a.d_h + d];
    }
#pragma unroll
    for (int bl = 0; bl < kAbsorbBatchGroup; ++bl)
      if (bl < nb)
        qext[(static_cast<int64_t>(b0 + bl) * HK + hk) * QW + c] = store_cast<TQ>(acc[bl] * a.qscale);
  }
  for (int e = tid; e < nb * a.d_r; e += kAbsorbThreads) {
    const int bl = e / a.d_r, r = e % a.d_r;
    const float v = load_elem(q_r, (static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_r + r);
    qext[(static_cast<int64_t>(b0 + bl) * HK + hk) * QW + a.w + r] = store_cast<TQ>(v * a.qscale);
  }
}

}  // namespace

hipError_t launch_absorb(const DecodeArgs& a, int dtype, bool q_bf16, const int32_t* seq_lens,
                         const void* q_c, const void* q_r, const void* w_uk, hipStream_t stream) {
  const dim3 grid(a.n_heads * a.k, (a.batch + kAbsorbBatchGroup - 1) / kAbsorbBatchGroup);
  const size_t sh = sizeof(float) * kAbsorbBatchGroup * a.d_h;
  if (dtype == 1) {
    if (q_bf16)
      absorb_kernel<uint16_t, uint16_t><<<grid, kAbsorbThreads, sh, stream>>>(
          a, seq_lens, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
          static_cast<const uint16_t*>(w_uk));
    else
      absorb_kernel<uint16_t, float><<<grid, kAbsorbThreads, sh, stream>>>(
          a, seq_lens, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
          static_cast<const uint16_t*>(w_uk));
  } else {
    absorb_kernel<float, float><<<grid, kAbsorbThreads, sh, stream>>>(
        a, seq_lens, static_cast<const float*>(q_c), static_cast<const float*>(q_r),
        static_cast<const float*>(w_uk));
  }
  return hipGetLastError();
}

}  // namespace mlra
