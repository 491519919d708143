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

// Work plan. The absorb grid has one extra row of workgroups; the first of
// them plans while the others absorb, so planning runs beside the absorption
// rather than before it: clamped lengths, tiles per sequence and their prefix
// sum (built in LDS), each sequence's unit range, the empty partial slot and
// the workspace header, and one descriptor per work unit so an attention
// workgroup learns its tile range and first sequence with one scalar fetch.
__device__ void plan_block(const DecodeArgs& a, const int32_t* seq_lens) {
  __shared__ int32_t cum_sh[kMaxBatch + 1];
  __shared__ int32_t len_sh[kMaxBatch];
  __shared__ int32_t part_sh[kAbsorbThreads];
  const int tid = threadIdx.x;
  const int32_t cap = a.max_pages * a.page_size;
  const int TT = a.tile_tokens;
  // tiles per sequence -> exclusive prefix sum; thread t scans a contiguous run
  const int per = (a.batch + kAbsorbThreads - 1) / kAbsorbThreads;
  const int bb = min(a.batch, tid * per), be = min(a.batch, bb + per);
  int32_t run = 0;
  for (int b = bb; b < be; ++b) {
    int32_t n = seq_lens[b];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    len_sh[b] = n;
    run += (n + TT - 1) / TT;
  }
  part_sh[tid] = run;
  __syncthreads();
  for (int off = 1; off < kAbsorbThreads; off <<= 1) {
    const int32_t v = tid >= off ? part_sh[tid - off] : 0;
    __syncthreads();
    part_sh[tid] += v;
    __syncthreads();
  }
  run = part_sh[tid] - run;
  for (int b = bb; b < be; ++b) {
    cum_sh[b] = run;
    run += (len_sh[b] + TT - 1) / TT;
  }
  if (tid == kAbsorbThreads - 1) cum_sh[a.batch] = part_sh[kAbsorbThreads - 1];
  __syncthreads();
  const int32_t NT = cum_sh[a.batch];
  // With fewer tiles than launched units only the first NT units get work (one
  // tile each), so every unit a sequence's range meets holds a partial.
  const int32_t UE = NT < a.units ? (NT > 0 ? NT : 1) : a.units;

  {  // in global memory for the attention and the combine
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
    // the empty partial slot read by the combine for slots no unit wrote
    const int hk_all = a.n_heads * a.k;
    float* pm = reinterpret_cast<float*>(a.ws + a.off_pm) + static_cast<int64_t>(a.empty_slot) * hk_all;
    float* pl = reinterpret_cast<float*>(a.ws + a.off_pl) + static_cast<int64_t>(a.empty_slot) * hk_all;
    const int64_t po0 = static_cast<int64_t>(a.empty_slot) * hk_all * a.w;  // first element of the empty slot
    for (int i = tid; i < hk_all; i += kAbsorbThreads) {
      pm[i] = -INFINITY;
      pl[i] = 0.f;
    }
    if (a.po_f16) {
      uint16_t* po = reinterpret_cast<uint16_t*>(a.ws + a.off_po) + po0;
      for (int i = tid; i < hk_all * a.w; i += kAbsorbThreads) po[i] = 0;
    } else {
      float* po = reinterpret_cast<float*>(a.ws + a.off_po) + po0;
      for (int i = tid; i < hk_all * a.w; i += kAbsorbThreads) po[i] = 0.f;
    }
    int32_t* udesc = reinterpret_cast<int32_t*>(a.ws + a.off_udesc);
    for (int u = tid; u < a.units; u += kAbsorbThreads) {
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
    if (blockIdx.x == 0) plan_block(a, seq_lens);
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
// straight from global memory 16 bytes per lane (the query operands once per
// lane). grid: (hk, ceil(batch / 16) + 1, ceil(w / 128)): z splits the 16-row
// tiles of W^UK eight to a workgroup; the last y row is the plan row.
__global__ __launch_bounds__(kAbsorbThreads) void absorb_mfma_kernel(DecodeArgs a, const int32_t* seq_lens,
                                                                      const uint16_t* __restrict__ q_c,
                                                                      const uint16_t* __restrict__ q_r,
                                                                      const uint16_t* __restrict__ w_uk) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = blockIdx.x;
  const int head = hk / a.k;
  const int b0 = blockIdx.y * 16;
  const int HK = a.n_heads * a.k;
  const int QW = a.w + a.d_r;
  if (blockIdx.y == gridDim.y - 1) {  // the plan row: one workgroup plans
    if (blockIdx.x == 0 && blockIdx.z == 0) plan_block(a, seq_lens);
    return;
  }

  const int m16 = lane & 15, g4 = lane >> 4;
  const int b = b0 + m16;
  const bool b_ok = b < a.batch;
  const uint16_t* qrow = q_c + (static_cast<int64_t>(b) * a.n_heads + head) * a.d_h;
  const uint16_t* wbase = w_uk + static_cast<int64_t>(hk) * a.w * a.d_h;
  uint16_t* qext = reinterpret_cast<uint16_t*>(a.ws + a.off_qext);
  // the query operands of this lane's sequence, loaded once (d_h <= 512)
  const int KD = (a.d_h + 31) / 32;
  u32x4_t bq[kAbsorbMaxKD];
#pragma unroll
  for (int kk = 0; kk < kAbsorbMaxKD; ++kk) {
    const int d = 32 * kk + 8 * g4;
    bq[kk] = (kk < KD && d < a.d_h && b_ok) ? *reinterpret_cast<const u32x4_t*>(qrow + d) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // this workgroup's 16-row tiles of W^UK: kAbsorbTilesPerWg of them, one per wave at a time
  const int n_mt = a.w / 16;
  const int mt_end = min(n_mt, static_cast<int>(blockIdx.z + 1) * kAbsorbTilesPerWg);
  for (int mt = blockIdx.z * kAbsorbTilesPerWg + wave; mt < mt_end; mt += kAbsorbThreads / 64) {
    floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* wrow = wbase + static_cast<int64_t>(mt * 16 + m16) * a.d_h;
    u32x4_t aw[kAbsorbMaxKD];
#pragma unroll
    for (int kk = 0; kk < kAbsorbMaxKD; ++kk) {
      const int d = 32 * kk + 8 * g4;
      aw[kk] = (kk < KD && d < a.d_h) ? *reinterpret_cast<const u32x4_t*>(wrow + d) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int kk = 0; kk < kAbsorbMaxKD; ++kk)
      if (kk < KD)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw[kk]),
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
  if (blockIdx.z != 0) return;  // the RoPE part once per (head-block pair, 16 sequences)
  const int nb = min(16, a.batch - b0);
  for (int e = tid; e < nb * a.d_r; e += kAbsorbThreads) {
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
    if (q_bf16 && a.d_h % 8 == 0 && a.w % 16 == 0)
      absorb_mfma_kernel<<<dim3(a.n_heads * a.k, (a.batch + 15) / 16 + 1,
                                (a.w / 16 + kAbsorbTilesPerWg - 1) / kAbsorbTilesPerWg),
                           kAbsorbThreads, 0, stream>>>(
          a, seq_lens, static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(q_r),
          static_cast<const uint16_t*>(w_uk));
    else if (q_bf16)
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
