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
// written by other compute units, so every read is an L2/MALL round trip; the
// kernel is organised so that each thread has all its reads in flight at once:
// the W^UV slice a thread needs is requested first, then each thread merges
// four columns of one (sequence, block) pair from 16 partial slots per batch
// (it recomputes the pair's max and sum itself rather than waiting on other
// threads). The merged latents sit in LDS transposed ([k w][8]) so each W^UV
// element meets all 8 sequences with two 16-byte LDS reads.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

constexpr int kThreads = 256;
constexpr int kBatchGroup = 8;
constexpr int kSlotBatch = 16;  // partial slots whose loads are in flight together
constexpr int kWPrefetch = 32;  // W^UV rows per thread loaded ahead of the merge

// Two adjacent W^UV elements (d, d+1) as floats. EVEN: d_h is even, so the
// pair is one aligned 4-byte (bf16) or 8-byte (fp32) load; otherwise two
// scalar loads, the second from a clamped index. No branches, so every load
// of a loop can be in flight at once.
template <typename TW, bool EVEN>
__device__ __forceinline__ float2 load_pair(const TW* p, int64_t i, int64_t i2);
template <>
__device__ __forceinline__ float2 load_pair<uint16_t, true>(const uint16_t* p, int64_t i, int64_t) {
  const uint32_t v = *reinterpret_cast<const uint32_t*>(p + i);
  return make_float2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}
template <>
__device__ __forceinline__ float2 load_pair<uint16_t, false>(const uint16_t* p, int64_t i, int64_t i2) {
  return make_float2(bf16_to_f32(p[i]), bf16_to_f32(p[i2]));
}
template <>
__device__ __forceinline__ float2 load_pair<float, true>(const float* p, int64_t i, int64_t) {
  return *reinterpret_cast<const float2*>(p + i);
}
template <>
__device__ __forceinline__ float2 load_pair<float, false>(const float* p, int64_t i, int64_t i2) {
  return make_float2(p[i], p[i2]);
}

template <typename TW, bool EVEN, bool PB>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  extern __shared__ float sh[];
  float* ot = sh;                             // [k * w][kBatchGroup]
  float* red = sh + kBatchGroup * a.k * a.w;  // [kThreads][2 * kBatchGroup]

  const int tid = threadIdx.x;
  const int head = blockIdx.x;
  const int b0 = blockIdx.y * kBatchGroup;
  const int nb = min(kBatchGroup, a.batch - b0);
  const int KW = a.k * a.w;

  // ---- W^UV slice of this thread, requested before anything else
  // thread -> (output column pair dp, e-slice part); passes over column pairs
  // beyond the first 256 reload inside the product loop.
  const TW* wuv = static_cast<const TW*>(a.w_uv) + static_cast<int64_t>(head) * KW * a.d_h;
  const int pairs_d = (a.d_h + 1) / 2;
  const int span0 = min(kThreads, pairs_d);
  const int split0 = max(1, kThreads / span0);
  const int part0 = tid / span0;
  const int d_0 = 2 * (tid % span0);
  const int e0_0 = static_cast<int>((static_cast<int64_t>(part0) * KW) / split0);
  const int d_0b = min(d_0 + 1, a.d_h - 1);
  float2 wpre[kWPrefetch];
#pragma unroll
  for (int u = 0; u < kWPrefetch; ++u) {
    const int e = min(e0_0 + u, KW - 1);  // rows past the slice are loaded but not used
    wpre[u] = load_pair<TW, EVEN>(wuv, static_cast<int64_t>(e) * a.d_h + d_0,
                                  static_cast<int64_t>(e) * a.d_h + d_0b);
  }

  // header through the scalar cache, so using it does not wait for the W^UV loads
  typedef __attribute__((address_space(4))) const int32_t cint32_t;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t NT = *(cint32_t*)(&hdr->n_tiles), units = *(cint32_t*)(&hdr->units);
  const int32_t G = *(cint32_t*)(&hdr->groups);
  const int32_t* sunit = reinterpret_cast<const int32_t*>(a.ws + a.off_sunit);
  const float* pm = reinterpret_cast<const float*>(a.ws + a.off_pm);
  const float* pl = reinterpret_cast<const float*>(a.ws + a.off_pl);
  const char* po = a.ws + a.off_po;
  const int64_t empty_hk = static_cast<int64_t>(a.empty_slot) * a.hk;  // first entry of the empty slot


  // ---- merge: item = (pair, 4 columns); 16 slots of loads in flight per batch
  const int w4 = a.w / 4;
  const int npairs = nb * a.k;
  // When there are at least as many tiles as units every unit owns tiles and
  // the per-slot check (64-bit divisions) is skipped.
  auto merge = [&](auto check_units) __attribute__((always_inline)) {
    constexpr bool kCheck = decltype(check_units)::value;
  for (int it = tid; it < npairs * w4; it += kThreads) {
      const int p = it / w4, c = 4 * (it % w4);
      const int bl = p / a.k, jj = p % a.k;
      const int b = b0 + bl, hk = head * a.k + jj;
      const int2 su = *reinterpret_cast<const int2*>(sunit + 2 * b);  // first, last unit
      const int32_t u0 = su.x;
      const int nslots = (su.y - u0 + 1) * G;
      float M = -INFINITY, L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s0 = 0; s0 < nslots; s0 += kSlotBatch) {
        float ms[kSlotBatch], ls[kSlotBatch];
        float4 vs[kSlotBatch];
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
          const int s = s0 + u;
          const int32_t uu = u0 + s / G;
          // units with an empty range (fewer tiles than units) wrote nothing
          const bool ok = s < nslots && (!kCheck || unit_owns_tiles(uu, NT, units));
          // invalid slots read the empty partial (m = -inf, l = 0, o~ = 0)
          const int64_t idx = ok ? (static_cast<int64_t>(uu + b) * G + s % G) * a.hk + hk : empty_hk + hk;
          ms[u] = pm[idx];
          ls[u] = pl[idx];
          vs[u] = load_partial4<PB>(po, idx * a.w + c);
        }
        float mb = M;
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) mb = fmaxf(mb, ms[u]);
        const float mu = mb == -INFINITY ? 0.f : mb;
        const float r = fast_exp2(M - mu);
        L *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
#pragma unroll
        for (int u = 0; u < kSlotBatch; ++u) {
          const float wgt = fast_exp2(ms[u] - mu);  // 0 for empty slots (m = -inf)
          L += wgt * ls[u];
          acc.x += wgt * vs[u].x;
          acc.y += wgt * vs[u].y;
          acc.z += wgt * vs[u].z;
          acc.w += wgt * vs[u].w;
        }
        M = mb;
      }
      const float invL = nslots > 0 ? 1.f / L : 0.f;
      if (c == 0 && a.lse)
        a.lse[(static_cast<int64_t>(b) * a.n_heads + head) * a.k + jj] =
            nslots > 0 ? 0.69314718055994531f * (M + __log2f(L)) : -INFINITY;
      const int e = jj * a.w + c;
      ot[(e + 0) * kBatchGroup + bl] = acc.x * invL;
      ot[(e + 1) * kBatchGroup + bl] = acc.y * invL;
      ot[(e + 2) * kBatchGroup + bl] = acc.z * invL;
      ot[(e + 3) * kBatchGroup + bl] = acc.w * invL;
    }
  };
  if (NT >= units)
    merge(std::false_type{});
  else
    merge(std::true_type{});
  for (int it = tid; it < (kBatchGroup - nb) * KW; it += kThreads) {
    const int bl = nb + it / KW, e = it % KW;
    ot[e * kBatchGroup + bl] = 0.f;
  }
  __syncthreads();

  // ---- out[b][head][d] = out_scale * sum_e W^UV[head][e][d] o~[b][e],  e = (jj, c)
  // Each thread owns two adjacent output columns and a slice of e.
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
      const int db = two ? d + 1 : d;
      for (int e = e0; e < e1; e += kWPrefetch) {
        float2 wl[kWPrefetch];
        if (d0 == 0 && e == e0) {
#pragma unroll
          for (int u = 0; u < kWPrefetch; ++u) wl[u] = wpre[u];
        } else {
#pragma unroll
          for (int u = 0; u < kWPrefetch; ++u) {
            const int ee = min(e + u, KW - 1);
            wl[u] = load_pair<TW, EVEN>(wuv, static_cast<int64_t>(ee) * a.d_h + d,
                                        static_cast<int64_t>(ee) * a.d_h + db);
          }
        }
#pragma unroll
        for (int u = 0; u < kWPrefetch; ++u) {
          if (e + u < e1) {
            const float2 wv = wl[u];
            const float4 o0 = *reinterpret_cast<const float4*>(ot + (e + u) * kBatchGroup);
            const float4 o1 = *reinterpret_cast<const float4*>(ot + (e + u) * kBatchGroup + 4);
            acc0[0] += wv.x * o0.x; acc1[0] += wv.y * o0.x;
            acc0[1] += wv.x * o0.y; acc1[1] += wv.y * o0.y;
            acc0[2] += wv.x * o0.z; acc1[2] += wv.y * o0.z;
            acc0[3] += wv.x * o0.w; acc1[3] += wv.y * o0.w;
            acc0[4] += wv.x * o1.x; acc1[4] += wv.y * o1.x;
            acc0[5] += wv.x * o1.y; acc1[5] += wv.y * o1.y;
            acc0[6] += wv.x * o1.z; acc1[6] += wv.y * o1.z;
            acc0[7] += wv.x * o1.w; acc1[7] += wv.y * o1.w;
          }
        }
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


// ---------------------------------------------------------------------------
// Combine for bf16 W^UV with d_h = 128 and compile-time block width / blocks
// per head: the shapes the MFMA attention runs. Same arithmetic as
// combine_kernel; the work is laid out so that a workgroup needs two dependent
// memory round trips (unit ranges, then all partial slots at once):
//   * one workgroup per (head, 4 sequences), 256 threads;
//   * merge: item = (sequence, K / 32 latent columns, half), one per thread;
//     the two halves of an item take alternate partial slots (a batch of
//     slots per half in flight at once) and are merged with one lane exchange;
//   * product: thread = (8 output columns, row residue r mod 16); its first
//     16 W^UV rows are requested with 16-byte loads before the merge starts,
//     each further batch before the previous one is multiplied (both before
//     the merge would hold too many registers for two workgroups per unit);
//     each wave
//     multiplies its rows on MFMA and the four waves are summed in LDS.
constexpr int kFastThreads = 256;
// sequences per workgroup (a multiple of 4; 8 measured slower on every
// workload: fewer workgroups outweigh the fewer W^UV re-reads)
constexpr int kFastSeq = 4;
// partial slots per half in flight together, 4-column items (eight: step
// 64.1 -> 63.4 us at MLRA-4 B = 32 8K against twelve, where a sequence has
// about nine slots, four or five per half)
constexpr int kFastSlots = 8;
constexpr int kFastDh = 128;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
static_assert(kFastSeq % 4 == 0 && kFastSeq <= 16, "sequences are MFMA rows, four per lane group");

template <int W, int KB, bool PB>
__global__ __launch_bounds__(kFastThreads) void combine_fast_kernel(CombineArgs a) {
  constexpr int K = W * KB;               // merged latent columns per head
  // merge item = (sequence, CW latent columns, half): every thread holds one
  // item, so all partial slots of a batch are requested in one round trip
  constexpr int CW = K * kFastSeq * 2 / kFastThreads;
  static_assert(CW >= 4 && CW % 4 == 0 && W % CW == 0, "whole 4-column loads inside one block");
  constexpr int CG = K / CW;              // column groups per sequence
  // partial slots per half whose loads are in flight together (the loaded
  // values take CW / 2 registers a slot)
  constexpr int NSL = CW <= 4 ? kFastSlots : (CW <= 8 ? 8 : 6);
  constexpr int ROWS = K / 16;            // W^UV rows per thread
  constexpr int RB = ROWS < 16 ? ROWS : 16;  // rows per load batch
  constexpr int NBAT = ROWS / RB;         // load batches, double-buffered
  static_assert(ROWS % RB == 0, "");
  __shared__ __attribute__((aligned(16))) float ot[K][kFastSeq];        // merged latents, transposed
  __shared__ __attribute__((aligned(16))) float red[4][16][8][kFastSeq];  // per-wave partial outputs

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x;
  const int b0 = blockIdx.y * kFastSeq;
  const int nb = min(kFastSeq, a.batch - b0);

  // ---- W^UV rows of this thread: e = rr + 16 i, columns [8 dc, 8 dc + 8);
  // the first batch is requested before the merge
  const int dc = tid & 15, rr = tid >> 4;
  const uint16_t* wuv = static_cast<const uint16_t*>(a.w_uv) + static_cast<int64_t>(head) * K * kFastDh + 8 * dc;
  typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;
  u32x4_t wr[2][RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) wr[0][i] = *(const gu32x4_t*)(wuv + static_cast<int64_t>(rr + 16 * i) * kFastDh);

  typedef __attribute__((address_space(4))) const int32_t cint32_t;
  const WsHeader* hdr = reinterpret_cast<const WsHeader*>(a.ws);
  const int32_t NT = *(cint32_t*)(&hdr->n_tiles), units = *(cint32_t*)(&hdr->units);
  const int32_t G = a.groups;
  const int32_t* sunit = reinterpret_cast<const int32_t*>(a.ws + a.off_sunit);
  const float* pm = reinterpret_cast<const float*>(a.ws + a.off_pm);
  const float* pl = reinterpret_cast<const float*>(a.ws + a.off_pl);
  const char* po = a.ws + a.off_po;
  const int64_t empty_hk = static_cast<int64_t>(a.empty_slot) * a.hk;

  // ---- merge
  // the lse value is stored after the outputs: a store issued here would be
  // waited for (stores count in vmcnt) before the W^UV registers are used
  float lse_v = 0.f;
  int64_t lse_i = -1;
  auto merge = [&](auto check_units) __attribute__((always_inline)) {
    constexpr bool kCheck = decltype(check_units)::value;
    const int half = tid & 1;
    const int cgi = (tid >> 1) % CG, bl = (tid >> 1) / CG;
    const int e = CW * cgi, jj = e / W, c = e % W;
    const int b = min(b0 + bl, a.batch - 1);  // rows past the batch merge a real sequence, unused
    const int hk = head * KB + jj;
    const int2 su = *reinterpret_cast<const int2*>(sunit + 2 * b);  // first, last unit
    const int nslots = (su.y - su.x + 1) * G;
    float M = -INFINITY, L = 0.f;
    float acc[CW];
#pragma unroll
    for (int q = 0; q < CW; ++q) acc[q] = 0.f;
    for (int s0 = half; s0 < nslots; s0 += 2 * NSL) {
      float ms[NSL], ls[NSL];
      float4 vs[NSL][CW / 4];
#pragma unroll
      for (int u = 0; u < NSL; ++u) {
        const int sl = s0 + 2 * u;
        const int32_t uu = su.x + sl / G;
        const bool ok = sl < nslots && (!kCheck || unit_owns_tiles(uu, NT, units));
        const int64_t idx = ok ? (static_cast<int64_t>(uu + b) * G + sl % G) * a.hk + hk : empty_hk + hk;
        ms[u] = pm[idx];
        ls[u] = pl[idx];
#pragma unroll
        for (int q = 0; q < CW / 4; ++q) vs[u][q] = load_partial4<PB>(po, idx * W + c + 4 * q);
      }
      float mb = M;
#pragma unroll
      for (int u = 0; u < NSL; ++u) mb = fmaxf(mb, ms[u]);
      const float mu = mb == -INFINITY ? 0.f : mb;
      const float r = fast_exp2(M - mu);
      L *= r;
#pragma unroll
      for (int q = 0; q < CW; ++q) acc[q] *= r;
#pragma unroll
      for (int u = 0; u < NSL; ++u) {
        const float wgt = fast_exp2(ms[u] - mu);  // 0 for empty slots (m = -inf)
        L += wgt * ls[u];
#pragma unroll
        for (int q = 0; q < CW / 4; ++q) {
          acc[4 * q + 0] += wgt * vs[u][q].x;
          acc[4 * q + 1] += wgt * vs[u][q].y;
          acc[4 * q + 2] += wgt * vs[u][q].z;
          acc[4 * q + 3] += wgt * vs[u][q].w;
        }
      }
      M = mb;
    }
    // merge the two halves (lanes 2t and 2t+1)
    const float Mo = __shfl_xor(M, 1), Lo = __shfl_xor(L, 1);
    const float Mt = fmaxf(M, Mo);
    const float mu = Mt == -INFINITY ? 0.f : Mt;
    const float r0 = fast_exp2(M - mu), r1 = fast_exp2(Mo - mu);
    const float Lt = L * r0 + Lo * r1;
    const float invL = nslots > 0 ? 1.f / Lt : 0.f;
#pragma unroll
    for (int q = 0; q < CW; ++q) {
      const float ao = __shfl_xor(acc[q], 1);
      if (half == 0) ot[e + q][bl] = (acc[q] * r0 + ao * r1) * invL;
    }
    if (half == 0 && c == 0 && a.lse && bl < nb) {
      lse_i = (static_cast<int64_t>(b) * a.n_heads + head) * KB + jj;
      lse_v = nslots > 0 ? 0.69314718055994531f * (Mt + __log2f(Lt)) : -INFINITY;
    }
  };
  if (NT >= units)
    merge(std::false_type{});
  else
    merge(std::true_type{});
  __syncthreads();

  // ---- product on MFMA: out[bl][d] = sum_e o~[bl][e] W^UV[e][d] with
  // v_mfma_f32_16x16x32_bf16, the sequences as MFMA rows (kFastSeq of 16 used).
  // A k-step of a wave covers the 32 rows e = rr + 16 i (rr = 4 wave + lane / 16,
  // i = 8 s .. 8 s + 7) whose W^UV columns [8 dc, 8 dc + 8) this thread loaded:
  // the columns are transposed in registers with v_perm_b32 (MFMA j, column dc
  // = output column 8 dc + j), and o~ enters as bf16 hi + lo parts (about 16
  // significant bits). Each wave sums its rows; the waves meet in LDS.
  const int g4 = lane >> 4;
  floatx4_t pacc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pacc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int bt = 0; bt < NBAT; ++bt) {
    const int i0 = bt * RB;
    // the next batch is requested before this one is multiplied
    if (bt + 1 < NBAT) {
#pragma unroll
      for (int i = 0; i < RB; ++i)
        wr[(bt + 1) & 1][i] = *(const gu32x4_t*)(wuv + static_cast<int64_t>(rr + 16 * (i0 + RB + i)) * kFastDh);
    }
#pragma unroll
    for (int s8 = 0; s8 < RB; s8 += 8) {
      // A: row dc is sequence dc (zero past kFastSeq), k = this lane's 8 rows
      u32x4_t ahi, alo;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float v2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          v2[h] = dc < kFastSeq ? ot[rr + 16 * (i0 + s8 + 2 * u + h)][dc] : 0.f;
        const uint16_t h0 = f32_to_bf16(v2[0]), h1 = f32_to_bf16(v2[1]);
        const uint16_t l0 = f32_to_bf16(v2[0] - bf16_to_f32(h0)), l1 = f32_to_bf16(v2[1] - bf16_to_f32(h1));
        ahi[u] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        alo[u] = static_cast<uint32_t>(l0) | (static_cast<uint32_t>(l1) << 16);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4_t bv;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          bv[u] = __builtin_amdgcn_perm(wr[bt & 1][s8 + 2 * u + 1][j >> 1], wr[bt & 1][s8 + 2 * u][j >> 1], sel);
        pacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ahi),
                                                          __builtin_bit_cast(bf16x8_t, bv), pacc[j], 0, 0, 0);
        pacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, alo),
                                                          __builtin_bit_cast(bf16x8_t, bv), pacc[j], 0, 0, 0);
      }
    }
  }
  // lane group g4 holds output rows (sequences) 4 g4 .. 4 g4 + 3 of column 8 dc + j
  if (g4 < kFastSeq / 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<float4*>(&red[wave][dc][j][4 * g4]) =
          make_float4(pacc[j][0], pacc[j][1], pacc[j][2], pacc[j][3]);
  }
  __syncthreads();
  // outputs: f = (bl, d), d fastest
#pragma unroll
  for (int f0 = 0; f0 < kFastSeq * kFastDh; f0 += kFastThreads) {
    const int f = f0 + tid;
    const int bl = f / kFastDh, d = f % kFastDh;
    if (bl < nb) {
      const float v = red[0][d >> 3][d & 7][bl] + red[1][d >> 3][d & 7][bl] + red[2][d >> 3][d & 7][bl] +
                      red[3][d >> 3][d & 7][bl];
      a.out[(static_cast<int64_t>(b0 + bl) * a.n_heads + head) * kFastDh + d] = a.out_scale * v;
    }
  }
  if (lse_i >= 0) a.lse[lse_i] = lse_v;
}

template <int W, int KB>
void launch_fast(const CombineArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_heads, (a.batch + kFastSeq - 1) / kFastSeq);
  if (a.po_f16)
    combine_fast_kernel<W, KB, true><<<grid, kFastThreads, 0, stream>>>(a);
  else
    combine_fast_kernel<W, KB, false><<<grid, kFastThreads, 0, stream>>>(a);
}

// Runs the specialised combine when the shape has one; false otherwise.
bool try_launch_fast(const CombineArgs& a, int dtype, hipStream_t stream) {
  if (dtype != 1 || a.d_h != kFastDh) return false;
  switch (a.w * 8 + a.k) {
    case 128 * 8 + 1: launch_fast<128, 1>(a, stream); return true;
    case 128 * 8 + 2: launch_fast<128, 2>(a, stream); return true;
    case 128 * 8 + 4: launch_fast<128, 4>(a, stream); return true;
    case 256 * 8 + 1: launch_fast<256, 1>(a, stream); return true;
    case 256 * 8 + 2: launch_fast<256, 2>(a, stream); return true;
    case 256 * 8 + 4: launch_fast<256, 4>(a, stream); return true;
    case 512 * 8 + 1: launch_fast<512, 1>(a, stream); return true;
    case 512 * 8 + 2: launch_fast<512, 2>(a, stream); return true;
    default: return false;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream) {
  if (try_launch_fast(a, dtype, stream)) return hipGetLastError();
  const dim3 grid(a.n_heads, (a.batch + kBatchGroup - 1) / kBatchGroup);
  const size_t sh = sizeof(float) * (kBatchGroup * a.k * a.w + kThreads * 2 * kBatchGroup);
  const bool even = a.d_h % 2 == 0;
  if (dtype == 1) {
    if (a.po_f16) {
      if (even) combine_kernel<uint16_t, true, true><<<grid, kThreads, sh, stream>>>(a);
      else combine_kernel<uint16_t, false, true><<<grid, kThreads, sh, stream>>>(a);
    } else {
      if (even) combine_kernel<uint16_t, true, false><<<grid, kThreads, sh, stream>>>(a);
      else combine_kernel<uint16_t, false, false><<<grid, kThreads, sh, stream>>>(a);
    }
  } else {
    // fp32 arrays run the generic attention, which keeps fp32 partials
    if (even) combine_kernel<float, true, false><<<grid, kThreads, sh, stream>>>(a);
    else combine_kernel<float, false, false><<<grid, kThreads, sh, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mlra
