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
//
// One workgroup per (head, group of 8 sequences). The partials were just
// written by other compute units, so every read is an L2/MALL round trip:
// all (sequence, block) pairs are merged at once, each by 32 threads, with
// branch-free slot loops so the loads of one thread are all in flight
// together. W^UV[head] is then read once per workgroup and applied to the 8
// merged latents, which sit in LDS transposed ([k w][8]) so one W^UV element
// meets all 8 with two 16-byte LDS reads.
#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kBatchGroup = 8;
constexpr int kPairLanes = 32;                     // threads per (sequence, block) pair
constexpr int kPairsPerPass = kThreads / kPairLanes;

// Reduction over the 32 lanes of a half-wave (xor 16, 8, 4, 2, 1).
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 32));
  return v;
}
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) v += __shfl_xor(v, off, 32);
  return v;
}

template <typename TW>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  extern __shared__ float sh[];
  float* ot = sh;                             // [k * w][kBatchGroup]
  float* red = sh + kBatchGroup * a.k * a.w;  // [kThreads][2 * kBatchGroup]
  float* mstat = red + kThreads * 2 * kBatchGroup;  // [kBatchGroup * k][2]: M, 1 / L
  __shared__ int32_t sinfo[kBatchGroup][2];   // per sequence: first, last unit (last < first: empty)

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
  const int npairs = nb * a.k;

  if (tid < kBatchGroup) {
    int32_t u0 = 0, u1 = -1;
    if (tid < nb) {
      const int32_t xa = cum[b0 + tid], xb = cum[b0 + tid + 1];
      if (xa < xb) {
        u0 = unit_of_tile(xa, NT, units);
        u1 = unit_of_tile(xb - 1, NT, units);
      }
    }
    sinfo[tid][0] = u0;
    sinfo[tid][1] = u1;
  }
  __syncthreads();

  // ---- M and 1/L per (sequence, block) pair: 32 threads per pair, slots strided
  for (int p0 = 0; p0 < npairs; p0 += kPairsPerPass) {
    const int p = p0 + tid / kPairLanes;
    const int ln = tid % kPairLanes;
    const bool live = p < npairs;
    const int bl = live ? p / a.k : 0, jj = live ? p % a.k : 0;
    const int b = b0 + bl, hk = head * a.k + jj;
    const int32_t u0 = sinfo[bl][0];
    const int nslots = live ? (sinfo[bl][1] - u0 + 1) * G : 0;
    float M = -INFINITY;
    for (int s = ln; s < nslots; s += kPairLanes) {
      const int32_t u = u0 + s / G;
      const float v = pm[(static_cast<int64_t>(u + b) * G + s % G) * a.hk + hk];
      if (unit_owns_tiles(u, NT, units)) M = fmaxf(M, v);
    }
    M = half_max(M);
    const float Muse = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    for (int s = ln; s < nslots; s += kPairLanes) {
      const int32_t u = u0 + s / G;
      const int64_t idx = (static_cast<int64_t>(u + b) * G + s % G) * a.hk + hk;
      const float v = pl[idx] * fast_exp2(pm[idx] - Muse);
      if (unit_owns_tiles(u, NT, units)) L += v;
    }
    L = half_sum(L);
    if (live && ln == 0) {
      mstat[2 * p] = Muse;
      mstat[2 * p + 1] = nslots > 0 ? 1.f / L : 0.f;
      if (a.lse)
        a.lse[(static_cast<int64_t>(b) * a.n_heads + head) * a.k + jj] =
            nslots > 0 ? 0.69314718055994531f * (M + __log2f(L)) : -INFINITY;
    }
  }
  __syncthreads();

  // ---- merged latents: item = (pair, 4 columns); loads of all slots in flight
  const int w4 = a.w / 4;
  for (int it = tid; it < npairs * w4; it += kThreads) {
    const int p = it / w4, c = 4 * (it % w4);
    const int bl = p / a.k, jj = p % a.k;
    const int b = b0 + bl, hk = head * a.k + jj;
    const int32_t u0 = sinfo[bl][0];
    const int nslots = (sinfo[bl][1] - u0 + 1) * G;
    const float M = mstat[2 * p];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = 0; s < nslots; ++s) {
      const int32_t u = u0 + s / G;
      const int64_t idx = (static_cast<int64_t>(u + b) * G + s % G) * a.hk + hk;
      const float4 v = *reinterpret_cast<const float4*>(po + idx * a.w + c);
      // units with an empty range (fewer tiles than units) wrote nothing
      const float wgt = unit_owns_tiles(u, NT, units) ? fast_exp2(pm[idx] - M) : 0.f;
      const bool ok = wgt != 0.f;
      acc.x += ok ? wgt * v.x : 0.f;
      acc.y += ok ? wgt * v.y : 0.f;
      acc.z += ok ? wgt * v.z : 0.f;
      acc.w += ok ? wgt * v.w : 0.f;
    }
    const float invL = mstat[2 * p + 1];
    const int e = jj * a.w + c;
    ot[(e + 0) * kBatchGroup + bl] = acc.x * invL;
    ot[(e + 1) * kBatchGroup + bl] = acc.y * invL;
    ot[(e + 2) * kBatchGroup + bl] = acc.z * invL;
    ot[(e + 3) * kBatchGroup + bl] = acc.w * invL;
  }
  for (int it = tid; it < (kBatchGroup - nb) * KW; it += kThreads) {
    const int bl = nb + it / KW, e = it % KW;
    ot[e * kBatchGroup + bl] = 0.f;
  }
  __syncthreads();

  // ---- out[b][head][d] = out_scale * sum_e W^UV[head][e][d] o~[b][e],  e = (jj, c)
  // Each thread owns two adjacent output columns and a slice of e.
  const TW* wuv = static_cast<const TW*>(a.w_uv) + static_cast<int64_t>(head) * KW * a.d_h;
  const int pairs_d = (a.d_h + 1) / 2;
  for (int d0 = 0; d0 < pairs_d; d0 += kThreads) {
    const int span = min(kThreads, pairs_d - d0);
    const int split = max(1, kThreads / span);
    const int dp = d0 + tid % span;
    const int d = 2 * dp;
    const int part = tid / span;
    const bool two = d + 1 < a.d_h;
    float acc0[kBatchGroup], acc1[kBatchGroup];
#pragma unroll
    for (int bl = 0; bl < kBatchGroup; ++bl) acc0[bl] = acc1[bl] = 0.f;
    if (part < split) {
      const int e0 = static_cast<int>((static_cast<int64_t>(part) * KW) / split);
      const int e1 = static_cast<int>((static_cast<int64_t>(part + 1) * KW) / split);
#pragma unroll 8
      for (int e = e0; e < e1; ++e) {
        const float w0 = load_elem(wuv, static_cast<int64_t>(e) * a.d_h + d);
        const float w1 = two ? load_elem(wuv, static_cast<int64_t>(e) * a.d_h + d + 1) : 0.f;
        const float4 o0 = *reinterpret_cast<const float4*>(ot + e * kBatchGroup);
        const float4 o1 = *reinterpret_cast<const float4*>(ot + e * kBatchGroup + 4);
        acc0[0] += w0 * o0.x; acc1[0] += w1 * o0.x;
        acc0[1] += w0 * o0.y; acc1[1] += w1 * o0.y;
        acc0[2] += w0 * o0.z; acc1[2] += w1 * o0.z;
        acc0[3] += w0 * o0.w; acc1[3] += w1 * o0.w;
        acc0[4] += w0 * o1.x; acc1[4] += w1 * o1.x;
        acc0[5] += w0 * o1.y; acc1[5] += w1 * o1.y;
        acc0[6] += w0 * o1.z; acc1[6] += w1 * o1.z;
        acc0[7] += w0 * o1.w; acc1[7] += w1 * o1.w;
      }
    }
#pragma unroll
    for (int bl = 0; bl < kBatchGroup; ++bl) {
      red[tid * 2 * kBatchGroup + bl] = acc0[bl];
      red[tid * 2 * kBatchGroup + kBatchGroup + bl] = acc1[bl];
    }
    __syncthreads();
    if (tid < span) {
      for (int bl = 0; bl < nb; ++bl) {
        float v0 = 0.f, v1 = 0.f;
        for (int q = 0; q < split; ++q) {
          v0 += red[(q * span + tid) * 2 * kBatchGroup + bl];
          v1 += red[(q * span + tid) * 2 * kBatchGroup + kBatchGroup + bl];
        }
        float* o = a.out + (static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_h + d;
        o[0] = a.out_scale * v0;
        if (two) o[1] = a.out_scale * v1;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  const dim3 grid(a.n_heads, (a.batch + kBatchGroup - 1) / kBatchGroup);
  const size_t sh = sizeof(float) * (kBatchGroup * a.k * a.w + kThreads * 2 * kBatchGroup +
                                     2 * kBatchGroup * a.k);
  if (dtype == 1)
    combine_kernel<uint16_t><<<grid, kThreads, sh, stream>>>(a);
  else
    combine_kernel<float><<<grid, kThreads, sh, stream>>>(a);
  return hipGetLastError();
}

}  // namespace mlra
