// Query absorption and work planning.
//
// Absorption (lesty.tech MLA explainer, section 5; ai360xpert concept page,
// "Absorbing the up-projection"): the key up-projection folds into the query,
//   q~[b][i][jj][c] = s z * sum_d W^UK[i][jj][c][d] q^C[b][i][d],
// and the RoPE part of the query is only scaled, q^R~ = s * q^R, with
// s = softmax_scale * log2(e) so the attention kernels work with base-2 logits
// and z the FP8 cache scale (1 for other caches), so that scores against the
// raw E4M3 codes are scores against the latent values they stand for.
#include "common.h"
#include "launch.h"

namespace mlra {

namespace {

constexpr int kAbsorbThreads = 256;
constexpr int kAbsorbBatchGroup = 8;

// Work plan. The absorb grid has one extra row of workgroups, which plan
// while the others absorb, so planning runs beside the absorption rather than
// before it. Every workgroup of the plan row computes the clamped lengths and
// the prefix sum of tiles per sequence (in LDS); part 0 writes them, each
// sequence's unit range, the empty partial slot and the workspace header, and
// the unit descriptors (one per attention workgroup: its tile range and first
// sequence, read with one scalar fetch) are shared out over the row's parts.
__device__ void plan_block(const DecodeArgs& a, const int32_t* seq_lens, int part, int nparts) {
  __shared__ int32_t cum_sh[kMaxBatch + 1];
  __shared__ int32_t len_sh[kMaxBatch];
  __shared__ int32_t wsum_sh[kAbsorbThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t cap = a.max_pages * a.page_size;
  const int TT = a.tile_tokens;
  // tiles per sequence -> exclusive prefix sum; thread t scans a contiguous run,
  // the runs are scanned across the wave with lane shifts and across waves in LDS
  const int per = (a.batch + kAbsorbThreads - 1) / kAbsorbThreads;
  const int bb = min(a.batch, tid * per), be = min(a.batch, bb + per);
  int32_t run = 0;
  for (int b = bb; b < be; ++b) {
    int32_t n = seq_lens[b];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    len_sh[b] = n;
    run += (n + TT - 1) / TT;
  }
  int32_t incl = run;  // inclusive scan of the runs within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum_sh[wave] = incl;
  __syncthreads();
  int32_t base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kAbsorbThreads / 64; ++w) {
    base += w < wave ? wsum_sh[w] : 0;
    total += wsum_sh[w];
  }
  run = base + incl - run;  // exclusive prefix of this thread's first sequence
  for (int b = bb; b < be; ++b) {
    cum_sh[b] = run;
    run += (len_sh[b] + TT - 1) / TT;
  }
  if (tid == 0) cum_sh[a.batch] = total;
  __syncthreads();
  const int32_t NT = total;
  // With fewer tiles than launched units only the first NT units get work (one
  // tile each), so every unit a sequence's range meets holds a partial.
  const int32_t UE = NT < a.units ? (NT > 0 ? NT : 1) : a.units;

  // in global memory for the attention and the combine
  if (part == 0) {
    int32_t* cum = reinterpret_cast<int32_t*>(a.ws + a.off_cum);
    int32_t* nlen = reinterpret_cast<int32_t*>(a.ws + a.off_nlen);
    int32_t* sunit = reinterpret_cast<int32_t*>(a.ws + a.off_sunit);
    for (int b = tid; b <= a.batch; b += kAbsorbThreads) cum[b] = cum_sh[b];
    for (int b = tid; b < a.batch; b += kAbsorbThreads) {
      nlen[b] = len_sh[b];
      // first and last unit whose tile range meets the sequence (last < first:
      // no tiles), so the combine finds its partial slots with one load
      const int32_t xa = cum_sh[b], xb = cum_sh[b + 1];
      int32_t u0 = 0, u1 = -1;
      if (xa < xb) {
        u0 = unit_of_tile(xa, NT, UE);
        u1 = unit_of_tile(xb - 1, NT, UE);
      }
      sunit[2 * b] = u0;
      sunit[2 * b + 1] = u1;
    }
    if (tid == 0) {
      WsHeader* h = reinterpret_cast<WsHeader*>(a.ws);
      h->magic = kWsMagic;
      h->flags = 0;
      h->n_tiles = NT;
      h->units = UE;  // units that may hold partials
      h->tile_tokens = a.tile_tokens;
      h->groups = a.groups;
      h->batch = a.batch;
      h->hk = a.n_heads * a.k;
    }
  }
  // the empty partial slot read by the combine for slots no unit wrote: its
  // m, l (part 0) and weighted sums (16-byte chunks shared out over the parts)
  const int hk_all = a.n_heads * a.k;
  if (part == 0) {
    float* pm = reinterpret_cast<float*>(a.ws + a.off_pm) + static_cast<int64_t>(a.empty_slot) * hk_all;
    float* pl = reinterpret_cast<float*>(a.ws + a.off_pl) + static_cast<int64_t>(a.empty_slot) * hk_all;
    for (int i = tid; i < hk_all; i += kAbsorbThreads) {
      pm[i] = -INFINITY;
      pl[i] = 0.f;
    }
  }
  {
    const int64_t esz = a.po_f16 ? 2 : 4;
    char* po = a.ws + a.off_po + static_cast<int64_t>(a.empty_slot) * hk_all * a.w * esz;
    const int64_t bytes = static_cast<int64_t>(hk_all) * a.w * esz;  // even
    // 16-byte stores when the slot is 16-byte aligned (the usual shapes), the rest 2 bytes at a time
    const int64_t n16 = (reinterpret_cast<uintptr_t>(po) & 15) == 0 ? bytes / 16 : 0;
    const int64_t c0 = n16 * part / nparts, c1 = n16 * (part + 1) / nparts;
    for (int64_t c = c0 + tid; c < c1; c += kAbsorbThreads) reinterpret_cast<int4*>(po)[c] = make_int4(0, 0, 0, 0);
    if (part == 0)
      for (int64_t i = 16 * n16 + 2 * tid; i < bytes; i += 2 * kAbsorbThreads) *reinterpret_cast<uint16_t*>(po + i) = 0;
  }
  int32_t* udesc = reinterpret_cast<int32_t*>(a.ws + a.off_udesc);
  const int u_lo = static_cast<int>(static_cast<int64_t>(a.units) * part / nparts);
  const int u_hi = static_cast<int>(static_cast<int64_t>(a.units) * (part + 1) / nparts);
  for (int u = u_lo + tid; u < u_hi; u += kAbsorbThreads) {
    const int32_t x0 = u < UE ? tile_begin(u, NT, UE) : NT, x1 = u < UE ? tile_begin(u + 1, NT, UE) : NT;
    // sequence owning tile x0: the largest b with cum_sh[b] <= x0
    int lo = 0, hi = a.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cum_sh[mid] <= x0) lo = mid; else hi = mid - 1;
    }
    const bool nxt = lo + 1 < a.batch;
    int4* dst = reinterpret_cast<int4*>(udesc + static_cast<int64_t>(u) * kUnitDescInts);
    dst[0] = make_int4(x0, x1, lo, cum_sh[lo]);
    dst[1] = make_int4(cum_sh[lo + 1], len_sh[lo], nxt ? cum_sh[lo + 2] : NT, nxt ? len_sh[lo + 1] : 0);
  }
}

// grid: (hk, ceil(batch / kAbsorbBatchGroup) + 1); block: kAbsorbThreads.
// Block (0, last row) writes the work plan; the rest of the last row is idle.
template <typename TIn, typename TQ>
__global__ __launch_bounds__(kAbsorbThreads) void absorb_kernel(DecodeArgs a, const int32_t* seq_lens,
                                                                 const TIn* __restrict__ q_c,
                                                                 const TIn* __restrict__ q_r,
                                                                 const TIn* __restrict__ w_uk) {
  extern __shared__ float q_sh[];  // [kAbsorbBatchGroup][d_h]
  const int tid = threadIdx.x;
  const int hk = blockIdx.x;
  const int head = hk / a.k;
  const int b0 = blockIdx.y * kAbsorbBatchGroup;
  const int nb = min(kAbsorbBatchGroup, a.batch - b0);
  const int HK = a.n_heads * a.k;
  const int QW = a.w + a.d_r;

  if (blockIdx.y == gridDim.y - 1) {  // the plan row: one workgroup plans
    plan_block(a, seq_lens, blockIdx.x, gridDim.x);
    return;
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
        qext[(static_cast<int64_t>(b0 + bl) * HK + hk) * QW + c] = store_cast<TQ>(acc[bl] * (a.qscale * a.lat_scale));
  }
  for (int e = tid; e < nb * a.d_r; e += kAbsorbThreads) {
    const int bl = e / a.d_r, r = e % a.d_r;
    const float v = load_elem(q_r, (static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_r + r);
    qext[(static_cast<int64_t>(b0 + bl) * HK + hk) * QW + a.w + r] = store_cast<TQ>(v * a.qscale);
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int kAbsorbMaxKD = 16;       // d_h / 32 for d_h <= 512
constexpr int kAbsorbTilesPerWg = 8;   // 16-row W^UK tiles per workgroup (grid z splits the rest)
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 absorption on MFMA: for head-block pair hk and a 16-sequence tile,
//   D[c][b] = sum_d W^UK[hk][c][d] q^C[b][head][d]   (v_mfma_f32_16x16x32_bf16)
// with W^UK rows as the A operand and queries as the B operand, both read
// straight from global memory 16 bytes per lane. grid: (hk, ceil(batch / 16)
// + 1, ceil(w / 128)): z splits the 16-row tiles of W^UK eight to a workgroup
// (two per wave); the last y row is the plan row. Every load of a workgroup
// (query operands, both W^UK tiles of each wave, the RoPE part) is issued
// before the first MFMA, so the kernel waits for one memory round trip.
// KD: 32-wide k-steps (d_h <= 32 KD).
template <int KD>
__global__ __launch_bounds__(kAbsorbThreads) void absorb_mfma_kernel(DecodeArgs a, const int32_t* seq_lens,
                                                                      const uint16_t* __restrict__ q_c,
                                                                      const uint16_t* __restrict__ q_r,
                                                                      const uint16_t* __restrict__ w_uk) {
  constexpr int kWaves = kAbsorbThreads / 64;
  constexpr int kTilesPerWave = kAbsorbTilesPerWg / kWaves;
  constexpr int kRope = 4;  // RoPE elements per thread loaded up front (16 sequences x d_r <= 64)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = blockIdx.x;
  const int head = hk / a.k;
  const int b0 = blockIdx.y * 16;
  const int HK = a.n_heads * a.k;
  const int QW = a.w + a.d_r;
  if (blockIdx.y == gridDim.y - 1) {  // the plan row
    plan_block(a, seq_lens, blockIdx.x + gridDim.x * blockIdx.z, gridDim.x * gridDim.z);
    return;
  }

  const int m16 = lane & 15, g4 = lane >> 4;
  const int b = b0 + m16;
  const bool b_ok = b < a.batch;
  const uint16_t* qrow = q_c + (static_cast<int64_t>(b) * a.n_heads + head) * a.d_h;
  const uint16_t* wbase = w_uk + static_cast<int64_t>(hk) * a.w * a.d_h;
  uint16_t* qext = reinterpret_cast<uint16_t*>(a.ws + a.off_qext);
  const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
  // the query operands of this lane's sequence
  u32x4_t bq[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    const int d = 32 * kk + 8 * g4;
    bq[kk] = (d < a.d_h && b_ok) ? *reinterpret_cast<const u32x4_t*>(qrow + d) : zero;
  }
  // this wave's 16-row tiles of W^UK: mt = 8 z + wave + 4 j
  const int n_mt = a.w / 16;
  const int mt_end = min(n_mt, static_cast<int>(blockIdx.z + 1) * kAbsorbTilesPerWg);
  u32x4_t aw[kTilesPerWave][KD];
#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
    const int mt = blockIdx.z * kAbsorbTilesPerWg + wave + kWaves * j;
    const uint16_t* wrow = wbase + static_cast<int64_t>(mt * 16 + m16) * a.d_h;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int d = 32 * kk + 8 * g4;
      aw[j][kk] = (mt < mt_end && d < a.d_h) ? *reinterpret_cast<const u32x4_t*>(wrow + d) : zero;
    }
  }
  // the RoPE part, once per (head-block pair, 16 sequences): only scaled
  const int nb = min(16, a.batch - b0);
  const int nr = blockIdx.z == 0 ? nb * a.d_r : 0;
  uint16_t rv[kRope];
#pragma unroll
  for (int j = 0; j < kRope; ++j) {
    const int e = tid + kAbsorbThreads * j;
    rv[j] = e < nr ? q_r[(static_cast<int64_t>(b0 + e / a.d_r) * a.n_heads + head) * a.d_r + e % a.d_r] : 0;
  }

#pragma unroll
  for (int j = 0; j < kTilesPerWave; ++j) {
    const int mt = blockIdx.z * kAbsorbTilesPerWg + wave + kWaves * j;
    if (mt >= mt_end) break;
    floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw[j][kk]),
                                                    __builtin_bit_cast(bf16x8_t, bq[kk]), acc, 0, 0, 0);
    if (b_ok) {
      // lane holds rows c = mt*16 + 4 g4 + i of sequence b: 4 consecutive outputs
      // the latent part carries the FP8 cache scale (1 otherwise)
      const float qs = a.qscale * a.lat_scale;
      const uint32_t lo = static_cast<uint32_t>(f32_to_bf16(acc[0] * qs)) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[1] * qs)) << 16);
      const uint32_t hi = static_cast<uint32_t>(f32_to_bf16(acc[2] * qs)) |
                          (static_cast<uint32_t>(f32_to_bf16(acc[3] * qs)) << 16);
      uint2* dst = reinterpret_cast<uint2*>(qext + (static_cast<int64_t>(b) * HK + hk) * QW + mt * 16 + 4 * g4);
      *dst = make_uint2(lo, hi);
    }
  }
#pragma unroll
  for (int j = 0; j < kRope; ++j) {
    const int e = tid + kAbsorbThreads * j;
    if (e < nr)
      qext[(static_cast<int64_t>(b0 + e / a.d_r) * HK + hk) * QW + a.w + e % a.d_r] =
          f32_to_bf16(bf16_to_f32(rv[j]) * a.qscale);
  }
  for (int e = tid + kAbsorbThreads * kRope; e < nr; e += kAbsorbThreads) {
    const int bl = e / a.d_r, r = e % a.d_r;
    const float v = bf16_to_f32(q_r[(static_cast<int64_t>(b0 + bl) * a.n_heads + head) * a.d_r + r]);
    qext[(static_cast<int64_t>(b0 + bl) * HK + hk) * QW + a.w + r] = f32_to_bf16(v * a.qscale);
  }
}

}  // namespace

hipError_t launch_absorb(const DecodeArgs& a, int dtype, bool q_bf16, const int32_t* seq_lens,
                         const void* q_c, const void* q_r, const void* w_uk, hipStream_t stream) {
  // the last row of every absorb grid is the plan row
  const dim3 grid(a.n_heads * a.k, (a.batch + kAbsorbBatchGroup - 1) / kAbsorbBatchGroup + 1);
  const size_t sh = sizeof(float) * kAbsorbBatchGroup * a.d_h;
  if (dtype == 1) {
    if (q_bf16 && a.d_h % 8 == 0 && a.w % 16 == 0) {
      const dim3 g(a.n_heads * a.k, (a.batch + 15) / 16 + 1, (a.w / 16 + kAbsorbTilesPerWg - 1) / kAbsorbTilesPerWg);
      const uint16_t *qc = static_cast<const uint16_t*>(q_c), *qr = static_cast<const uint16_t*>(q_r),
                     *wk = static_cast<const uint16_t*>(w_uk);
      if (a.d_h <= 128)
        absorb_mfma_kernel<4><<<g, kAbsorbThreads, 0, stream>>>(a, seq_lens, qc, qr, wk);
      else if (a.d_h <= 256)
        absorb_mfma_kernel<8><<<g, kAbsorbThreads, 0, stream>>>(a, seq_lens, qc, qr, wk);
      else
        absorb_mfma_kernel<kAbsorbMaxKD><<<g, kAbsorbThreads, 0, stream>>>(a, seq_lens, qc, qr, wk);
    } else if (q_bf16)
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
