// Split-K latent attention, generic VALU path (fp32 caches and shapes without
// a tuned MFMA variant). Same partial format and work split as the MFMA path:
// per (unit, head, attended block) the base-2 running max m, sum l and the
// weighted latent sum o~ = sum_t 2^(l_t - m) c_{t,j} (lesty.tech MLA explainer,
// section 5, with the MLRA block split of the alanhou.org "Core Mechanism").
// One wave per (unit, head-block pair); lane t scores token t of a 64-token
// tile, then the wave accumulates the latent columns, lane c owning column c.
#include <hip/hip_ext.h>

#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int TT = kGenericTileTokens;  // 64: one token per lane
constexpr int kMaxColsPerLane = 8;      // w <= 512

template <typename T, typename TQ>
__global__ __launch_bounds__(64) void attend_generic_kernel(DecodeArgs a) {
  extern __shared__ float sh[];  // q: [w + d_r] | p: [TT] | row offsets: [TT] int64
  float* q_sh = sh;
  float* p_sh = sh + a.w + a.d_r;
  int64_t* rowoff_sh = reinterpret_cast<int64_t*>(p_sh + TT + ((a.w + a.d_r + TT) & 1));

  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int hk = blockIdx.y;
  const int head = hk / a.k, jj = hk % a.k;
  const int blk = (head / a.hpb) * a.k + jj;
  const int HK = a.n_heads * a.k;
  const int QW = a.w + a.d_r;

  WsHeader* hdr = reinterpret_cast<WsHeader*>(a.ws);
  const int32_t NT = hdr->n_tiles, units = hdr->units;
  const int32_t* cum = reinterpret_cast<const int32_t*>(a.ws + a.off_cum);
  const int32_t* nlen = reinterpret_cast<const int32_t*>(a.ws + a.off_nlen);
  if (unit >= units) return;
  const int32_t x0 = tile_begin(unit, NT, units);
  const int32_t x1 = tile_begin(unit + 1, NT, units);
  if (x0 >= x1) return;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= x0) lo = mid; else hi = mid - 1;
  }

  const T* pool = static_cast<const T*>(a.pool);
  const TQ* qext = reinterpret_cast<const TQ*>(a.ws + a.off_qext);
  float* pm = reinterpret_cast<float*>(a.ws + a.off_pm);
  float* pl = reinterpret_cast<float*>(a.ws + a.off_pl);
  float* po = reinterpret_cast<float*>(a.ws + a.off_po);

  float O[kMaxColsPerLane];
#pragma unroll
  for (int s = 0; s < kMaxColsPerLane; ++s) O[s] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  uint32_t bad_page = 0;

  int cb = lo;
  int32_t cb_start = cum[cb], cb_end = cum[cb + 1], cb_n = nlen[cb];
  bool need_q = true;
  for (int32_t x = x0; x < x1; ++x) {
    while (x >= cb_end) {
      ++cb;
      cb_start = cb_end;
      cb_end = cum[cb + 1];
      cb_n = nlen[cb];
      need_q = true;
    }
    if (need_q) {
      __syncthreads();
      for (int e = lane; e < QW; e += 64)
        q_sh[e] = load_elem(qext, (static_cast<int64_t>(cb) * HK + hk) * QW + e);
      need_q = false;
    }
    const int32_t tok0 = (x - cb_start) * TT;
    const int valid = min(TT, cb_n - tok0);
    // row offset of this lane's token
    int64_t rowoff = 0;
    if (lane < valid) {
      const int32_t tok = tok0 + lane;
      const int32_t pidx = tok >> a.log2_page;
      int32_t phys = a.page_table ? a.page_table[static_cast<int64_t>(cb) * a.max_pages + pidx]
                                  : cb * a.max_pages + pidx;
      if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) {
        phys = 0;
        bad_page = 1;
      }
      rowoff = (static_cast<int64_t>(phys) * a.page_size + (tok & (a.page_size - 1))) * a.row;
    }
    rowoff_sh[lane] = rowoff;
    __syncthreads();
    float score = -INFINITY;
    if (lane < valid) {
      const T* rp = pool + rowoff;
      float acc = 0.f;
      for (int c = 0; c < a.w; ++c) acc += q_sh[c] * load_elem(rp, static_cast<int64_t>(blk) * a.w + c);
      for (int r = 0; r < a.d_r; ++r) acc += q_sh[a.w + r] * load_elem(rp, static_cast<int64_t>(a.n_blocks) * a.w + r);
      score = acc;
    }
    float mx = score;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float scale = fast_exp2(m_run - m_use);
    const float p = fast_exp2(score - m_use);
    float ps = p;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l_run = l_run * scale + ps;
    m_run = m_new;
    p_sh[lane] = p;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kMaxColsPerLane; ++s) {
      const int c = lane + 64 * s;
      if (c < a.w) {
        float acc = O[s] * scale;
        for (int t = 0; t < valid; ++t)
          acc += p_sh[t] * load_elem(pool + rowoff_sh[t], static_cast<int64_t>(blk) * a.w + c);
        O[s] = acc;
      }
    }
    __syncthreads();
    if (x + 1 == cb_end || x + 1 == x1) {
      const int64_t slot = unit + cb;
#pragma unroll
      for (int s = 0; s < kMaxColsPerLane; ++s) {
        const int c = lane + 64 * s;
        if (c < a.w) po[(slot * HK + hk) * a.w + c] = O[s];
        O[s] = 0.f;
      }
      if (lane == 0) {
        pm[slot * HK + hk] = m_run;
        pl[slot * HK + hk] = l_run;
      }
      m_run = -INFINITY;
      l_run = 0.f;
    }
  }
  if (__any(bad_page) && lane == 0) atomicOr(&hdr->flags, kFlagBadPage);
}

}  // namespace

hipError_t launch_attend_generic(const DecodeArgs& a, int dtype, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(a.units, a.n_heads * a.k);
  const size_t sh = sizeof(float) * (a.w + a.d_r + TT + 2) + sizeof(int64_t) * TT + 16;
  // with events, the dispatch records the kernel's own start and stop times
  if (dtype == 1) {
    if (t0 || t1)
      hipExtLaunchKernelGGL(attend_generic_kernel<uint16_t, float>, grid, dim3(64), sh, stream, t0, t1, 0, a);
    else
      attend_generic_kernel<uint16_t, float><<<grid, 64, sh, stream>>>(a);
  } else {
    if (t0 || t1)
      hipExtLaunchKernelGGL(attend_generic_kernel<float, float>, grid, dim3(64), sh, stream, t0, t1, 0, a);
    else
      attend_generic_kernel<float, float><<<grid, 64, sh, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mlra
