// Log-sum-exp merge of the split partials and the absorbed value up-projection.
//
// For sequence b, head i, attended block jj (partials from every unit whose
// tile range touches b):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o~ = sum_s o~_s 2^(m_s - M) / L
//   out[b][i] = out_scale * sum_jj W^UV[i][jj]^T o~[jj]
//   lse[b][i][jj] = ln 2 * (M + log2 L)
// The value up-projection is applied once, to the merged latent (lesty.tech
// MLA explainer, section 5); per-block outputs are summed ("results get
// combined", alanhou.org "Core Mechanism").
#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kBatchGroup = 8;

// grid: (n_heads, ceil(batch / kBatchGroup)); dynamic LDS: merged latents
// [kBatchGroup][k][w] plus a reduction buffer [kThreads][kBatchGroup].
template <typename TW>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  extern __shared__ float sh[];
  float* ot = sh;                                   // [kBatchGroup][k * w]
  float* red = sh + kBatchGroup * a.k * a.w;        // [kThreads][kBatchGroup]
  __shared__ float ml_sh[2];

  const int tid = threadIdx.x;
  const int head = blockIdx.x;
  const int b0 = blockIdx.y * kBatchGroup;
  const int nb = min(kBatchGroup, a.batch - b0);
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t NT = hdr->n_tiles, units = hdr->units, G = hdr->groups;
  const int32_t* cum = reinterpret_cast<const int32_t*>(a.ws + a.off_cum);
  const float* pm = reinterpret_cast<const float*>(a.ws + a.off_pm);
  const float* pl = reinterpret_cast<const float*>(a.ws + a.off_pl);
  const float* po = reinterpret_cast<const float*>(a.ws + a.off_po);
  const int KW = a.k * a.w;

  for (int bl = 0; bl < nb; ++bl) {
    const int b = b0 + bl;
    const int32_t xa = cum[b], xb = cum[b + 1];
    for (int jj = 0; jj < a.k; ++jj) {
      const int hk = head * a.k + jj;
      float* dst = ot + bl * KW + jj * a.w;
      if (xa >= xb) {
        for (int c = tid; c < a.w; c += kThreads) dst[c] = 0.f;
        if (tid == 0 && a.lse)
          a.lse[(static_cast<int64_t>(b) * a.n_heads + head) * a.k + jj] = -INFINITY;
        continue;
      }
      const int32_t u0 = unit_of_tile(xa, NT, units), u1 = unit_of_tile(xb - 1, NT, units);
      // slot (u + b) * G + g for u in [u0, u1]; units with an empty range
      // (possible when there are fewer tiles than units) wrote nothing.
      const int nslots = (u1 - u0 + 1) * G;
      const int64_t slot0 = static_cast<int64_t>(u0 + b) * G;
      // global max over the slots, then weights 2^(m_s - M) / L
      if (tid < 64) {
        float mx = -INFINITY;
        for (int s = tid; s < nslots; s += 64)
          if (unit_owns_tiles(u0 + s / G, NT, units)) mx = fmaxf(mx, pm[(slot0 + s) * a.hk + hk]);
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        float lsum = 0.f;
        for (int s = tid; s < nslots; s += 64) {
          if (!unit_owns_tiles(u0 + s / G, NT, units)) continue;
          const float ms = pm[(slot0 + s) * a.hk + hk];
          lsum += pl[(slot0 + s) * a.hk + hk] * fast_exp2(ms - mx);
        }
        for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
        if (tid == 0) {
          ml_sh[0] = mx;
          ml_sh[1] = lsum;
          if (a.lse)
            a.lse[(static_cast<int64_t>(b) * a.n_heads + head) * a.k + jj] =
                0.69314718055994531f * (mx + __log2f(lsum));
        }
      }
      __syncthreads();
      const float M = ml_sh[0], invL = 1.f / ml_sh[1];
      for (int c = tid; c < a.w; c += kThreads) {
        float acc = 0.f;
        for (int s = 0; s < nslots; ++s) {
          if (!unit_owns_tiles(u0 + s / G, NT, units)) continue;
          const float ms = pm[(slot0 + s) * a.hk + hk];
          acc += po[((slot0 + s) * a.hk + hk) * a.w + c] * fast_exp2(ms - M);
        }
        dst[c] = acc * invL;
      }
      __syncthreads();
    }
  }
  __syncthreads();

  // out[b][head][d] = out_scale * sum_{jj, c} W^UV[head][jj][c][d] o~[b][jj][c]
  const TW* wuv = static_cast<const TW*>(a.w_uv) + static_cast<int64_t>(head) * KW * a.d_h;
  for (int d0 = 0; d0 < a.d_h; d0 += kThreads) {
    const int span = min(kThreads, a.d_h - d0);       // columns in this pass
    const int split = max(1, kThreads / span);         // threads per column
    const int d = d0 + tid % span;
    const int part = tid / span;
    float acc[kBatchGroup];
#pragma unroll
    for (int bl = 0; bl < kBatchGroup; ++bl) acc[bl] = 0.f;
    if (part < split) {
      const int e0 = static_cast<int>((static_cast<int64_t>(part) * KW) / split);
      const int e1 = static_cast<int>((static_cast<int64_t>(part + 1) * KW) / split);
      for (int e = e0; e < e1; ++e) {
        const float wv = load_elem(wuv, static_cast<int64_t>(e) * a.d_h + d);
#pragma unroll
        for (int bl = 0; bl < kBatchGroup; ++bl)
          if (bl < nb) acc[bl] += wv * ot[bl * KW + e];
      }
    }
#pragma unroll
    for (int bl = 0; bl < kBatchGroup; ++bl) red[tid * kBatchGroup + bl] = acc[bl];
    __syncthreads();
    if (tid < span) {
      for (int bl = 0; bl < nb; ++bl) {
        float v = 0.f;
        for (int p = 0; p < split; ++p) v += red[(p * span + tid) * kBatchGroup + bl];
        a.out[(static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_h + d0 + tid] = a.out_scale * v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  const dim3 grid(a.n_heads, (a.batch + kBatchGroup - 1) / kBatchGroup);
  const size_t sh = sizeof(float) * (kBatchGroup * a.k * a.w + kThreads * kBatchGroup);
  if (dtype == 1)
    combine_kernel<uint16_t><<<grid, kThreads, sh, stream>>>(a);
  else
    combine_kernel<float><<<grid, kThreads, sh, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mlra
