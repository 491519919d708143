// Split-K latent attention over the paged cache, bf16 MFMA path for gfx950.
//
// What it computes (per work unit, per query head i and attended block j):
//   l_t = q~_{i,j} . c_{t,j} + q^R~_i . k^R_t          (base-2 logits; the
//         query was absorbed into latent space, lesty.tech section 5)
//   m = max_t l_t,  l = sum_t 2^(l_t - m),  o~ = sum_t 2^(l_t - m) c_{t,j}
// over the unit's tokens, written as (m, l, o~) partials for the combine.
//
// How (MI355X-first):
//  - One workgroup per compute unit streams a contiguous range of 32- or
//    128-token tiles. Each tile [c | k^R] is copied HBM -> LDS once with
//    LDS-DMA (global_load_lds_dwordx4) into a ring of STAGES buffers, so
//    STAGES-1 tiles are in flight while one is consumed. The waits are
//    explicit (s_waitcnt vmcnt), the loads are issued from inline asm so the
//    compiler does not serialise them behind its own LDS alias checks.
//  - Every wave owns one (latent block, 16-head tile) task; all waves read the
//    same LDS tile, so k^R and (for MLA) the latent are fetched from HBM once
//    and shared by every head.
//  - Scores: S^T[token][head] = K_ext[token] . Q_ext[head] with
//    v_mfma_f32_16x16x32_bf16 (tokens as MFMA rows). Its output layout puts
//    four tokens of one head in each lane, which is exactly the B-operand
//    layout of the value product, so P never leaves registers.
//  - Values: O^T[col][head] += C^T[col][token] P^T[token][head], again
//    16x16x32 bf16 MFMA; C^T operands come from 128-bit LDS reads of 8 token
//    rows, transposed in registers with v_perm_b32.
//  - Rows are XOR-swizzled in 16-byte chunks inside each 128-byte group
//    (chunk ^ (row & 7)) so both read patterns are free of LDS bank conflicts.
#include "common.h"
#include "launch.h"

namespace mlra {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int W_, int DR_, int NBR_, int HT_, int G_, int TT_, int ST_>
struct Cfg {
  static constexpr int W = W_;      // latent block width
  static constexpr int DR = DR_;    // RoPE key width
  static constexpr int NBR = NBR_;  // latent blocks in a cache row
  static constexpr int HT = HT_;    // 16-head tiles per block
  static constexpr int G = G_;      // waves sharing one task (token groups)
  static constexpr int TT = TT_;    // tokens per tile
  static constexpr int ST = ST_;    // LDS ring stages
  static constexpr int ROW = NBR * W + DR;
  static constexpr int ROWB = ROW * 2;
  static constexpr int CPR = ROW / 8;  // 16-byte chunks per row
  static constexpr int TASKS = NBR * HT;
  static constexpr int NWAVES = TASKS * G;
  static constexpr int NTHREADS = NWAVES * 64;
  static constexpr int TILE_BYTES = TT * ROWB;
  static constexpr int NI = TT * CPR / 64;  // DMA instructions per tile
  // Waves that issue DMA: the largest divisor of NI not above NWAVES, so every
  // issuing wave has the same count (its vmcnt arithmetic stays static).
  static constexpr int largest_divisor(int n, int cap) {
    for (int d = cap; d > 1; --d)
      if (n % d == 0) return d;
    return 1;
  }
  static constexpr int NWD = largest_divisor(NI, NWAVES);
  static constexpr int NI_W = NI / NWD;
  static constexpr int KK = (W + DR) / 32;  // score k-steps
  static constexpr int KKC = W / 32;        // k-steps over the latent part
  static constexpr int NSUB = TT / 32;
  static constexpr int SUBW = NSUB / G;     // 32-token sub-tiles per wave per tile
  static constexpr int NQ = W / 128;        // 128-column groups on the value side
  static_assert(ROW % 64 == 0, "rows must be whole 128-byte groups");
  static_assert(W % 128 == 0 && DR % 32 == 0, "");
  static_assert(TT % 32 == 0 && NSUB % G == 0, "");
  static_assert(NI * 64 == TT * CPR && NI % NWD == 0, "");
  static_assert((ST - 1) * NI_W <= 63, "vmcnt range");
  static_assert(ST * TILE_BYTES <= 160 * 1024, "LDS");
  static_assert(NTHREADS <= 1024, "");
};

// One LDS-DMA instruction: lane l copies 16 bytes from base + off to LDS
// address lds_addr + 16 l. m0 is saved and restored around it.
__device__ __forceinline__ void dma16(uint64_t base, uint32_t off, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_addr)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int STAGES, int NIW>
__device__ __forceinline__ void wait_tile(int tiles_after) {
  // Each wave issued NIW loads per tile; waiting until at most
  // tiles_after * NIW remain guarantees this tile has landed.
  switch (tiles_after) {
    case 0: wait_vmcnt_barrier<0>(); break;
    case 1: wait_vmcnt_barrier<NIW>(); break;
    case 2: if constexpr (STAGES > 2) wait_vmcnt_barrier<2 * NIW>(); break;
    case 3: if constexpr (STAGES > 3) wait_vmcnt_barrier<3 * NIW>(); break;
    case 4: if constexpr (STAGES > 4) wait_vmcnt_barrier<4 * NIW>(); break;
    case 5: if constexpr (STAGES > 5) wait_vmcnt_barrier<5 * NIW>(); break;
    default: wait_vmcnt_barrier<0>(); break;
  }
}

__device__ __forceinline__ floatx4_t mfma32(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

template <class C>
__global__ __launch_bounds__(C::NTHREADS, 1) void attend_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::ST * C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int task = wave % C::TASKS;
  const int tgrp = wave / C::TASKS;
  const int blk = task / C::HT;
  const int ht = task % C::HT;
  const int hgrp = blk / a.k;
  const int jj = blk - hgrp * a.k;
  const int m16 = lane & 15;
  const int g4 = lane >> 4;
  const int hloc = ht * 16 + m16;
  const bool head_ok = hloc < a.hpb;
  const int head = hgrp * a.hpb + hloc;
  const int HK = a.n_heads * a.k;
  const int hk = head * a.k + jj;
  const int P = a.page_size;

  WsHeader* hdr = reinterpret_cast<WsHeader*>(a.ws);
  const int32_t NT = hdr->n_tiles;
  const int32_t* cum = reinterpret_cast<const int32_t*>(a.ws + a.off_cum);
  const int32_t* nlen = reinterpret_cast<const int32_t*>(a.ws + a.off_nlen);
  const int unit = blockIdx.x;
  const int32_t x0 = tile_begin(unit, NT, a.units);
  const int32_t x1 = tile_begin(unit + 1, NT, a.units);
  if (x0 >= x1) return;

  // Sequence owning tile x0: the largest b with cum[b] <= x0.
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cum[mid] <= x0) lo = mid; else hi = mid - 1;
  }

  // Per-lane byte offsets of this wave's DMA slots inside a contiguous tile image.
  uint32_t loff[C::NI_W];
#pragma unroll
  for (int k = 0; k < C::NI_W; ++k) {
    const int p = (k * C::NWD + wave) * 64 + lane;
    const int r = p / C::CPR;
    const int lc = (p % C::CPR) ^ (r & 7);
    loff[k] = static_cast<uint32_t>(r * C::ROWB + 16 * lc);
  }
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  const uint64_t pool = reinterpret_cast<uint64_t>(a.pool);

  // Issue cursor (runs STAGES-1 tiles ahead of the compute cursor).
  int ib = lo;
  int32_t ib_start = cum[ib], ib_end = cum[ib + 1], ib_n = nlen[ib];
  uint32_t bad_page = 0;

  auto issue = [&](int32_t x, int stage) {
    while (x >= ib_end) {
      ++ib;
      ib_start = ib_end;
      ib_end = cum[ib + 1];
      ib_n = nlen[ib];
    }
    if (wave >= C::NWD) return;
    const int32_t tok0 = (x - ib_start) * C::TT;
    const int32_t npg = (ib_n + P - 1) >> a.log2_page;
#pragma unroll
    for (int k = 0; k < C::NI_W; ++k) {
      const int inst = k * C::NWD + wave;
      const int row0 = (inst * 64) / C::CPR;
      const int32_t pg_unclamped = (tok0 + row0) >> a.log2_page;
      const int32_t pidx = pg_unclamped < npg ? pg_unclamped : npg - 1;
      int32_t phys = a.page_table ? a.page_table[static_cast<int64_t>(ib) * a.max_pages + pidx]
                                  : ib * a.max_pages + pidx;
      if (static_cast<uint32_t>(phys) >= static_cast<uint32_t>(a.num_pages)) {
        phys = 0;
        bad_page = 1;
      }
      uint32_t off;
      if (P >= C::TT) {
        off = loff[k] + static_cast<uint32_t>((tok0 & (P - 1)) * C::ROWB);
      } else {
        const int32_t first_pg = tok0 >> a.log2_page;
        off = loff[k] - static_cast<uint32_t>((pg_unclamped - first_pg) * P * C::ROWB);
      }
      const uint64_t base = pool + static_cast<uint64_t>(phys) * static_cast<uint64_t>(P) * C::ROWB;
      const uint32_t b_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base));
      const uint32_t b_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base >> 32));
      dma16((static_cast<uint64_t>(b_hi) << 32) | b_lo, off,
            __builtin_amdgcn_readfirstlane(lds_base + stage * C::TILE_BYTES + inst * 1024));
    }
  };

  // Compute state.
  floatx4_t O[C::NQ][8];
#pragma unroll
  for (int q = 0; q < C::NQ; ++q)
#pragma unroll
    for (int e = 0; e < 8; ++e) O[q][e] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bf16x8_t Qb[C::KK];

  int cb = lo;
  int32_t cb_start = cum[cb], cb_end = cum[cb + 1], cb_n = nlen[cb];
  bool need_q = true;

  float* pm = reinterpret_cast<float*>(a.ws + a.off_pm);
  float* pl = reinterpret_cast<float*>(a.ws + a.off_pl);
  float* po = reinterpret_cast<float*>(a.ws + a.off_po);
  const uint16_t* qext = reinterpret_cast<const uint16_t*>(a.ws + a.off_qext);

#pragma unroll
  for (int s = 0; s < C::ST - 1; ++s)
    if (x0 + s < x1) issue(x0 + s, s);

  for (int32_t x = x0; x < x1; ++x) {
    const int t = x - x0;
    const int st = t % C::ST;
    if (x + C::ST - 1 < x1) issue(x + C::ST - 1, (t + C::ST - 1) % C::ST);
    const int after = wave < C::NWD ? min(C::ST - 1, x1 - 1 - x) : 0;
    wait_tile<C::ST, C::NI_W>(after);

    while (x >= cb_end) {
      ++cb;
      cb_start = cb_end;
      cb_end = cum[cb + 1];
      cb_n = nlen[cb];
      need_q = true;
    }
    const int valid = min(C::TT, cb_n - (x - cb_start) * C::TT);
    uint8_t* sb = lds + st * C::TILE_BYTES;
    if (valid < C::TT) {
      // Rows past the sequence end may hold anything: zero them so that the
      // value product sees 0 * 0 there.
      const int nz = (C::TT - valid) * C::CPR;
      for (int idx = tid; idx < nz; idx += C::NTHREADS) {
        const int r = valid + idx / C::CPR;
        *reinterpret_cast<u32x4_t*>(sb + r * C::ROWB + 16 * (idx % C::CPR)) = u32x4_t{0u, 0u, 0u, 0u};
      }
      lds_barrier();
    }
    if (need_q) {
      const uint16_t* qe = qext + (static_cast<int64_t>(cb) * HK + hk) * (C::W + C::DR);
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const int off = kk < C::KKC ? 32 * kk + 8 * g4 : C::W + 32 * (kk - C::KKC) + 8 * g4;
        u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
        if (head_ok) v = *reinterpret_cast<const u32x4_t*>(qe + off);
        Qb[kk] = __builtin_bit_cast(bf16x8_t, v);
      }
      need_q = false;
    }

#pragma unroll
    for (int si = 0; si < C::SUBW; ++si) {
      const int rowbase = 32 * (si * C::G + tgrp);
      // ---- scores: S_h[i] = token rowbase + 16 h + 4 g4 + i, head m16
      floatx4_t S0 = floatx4_t{0.f, 0.f, 0.f, 0.f}, S1 = S0;
      const int r0 = rowbase + m16;
      const uint8_t* rp0 = sb + r0 * C::ROWB;
      const uint8_t* rp1 = rp0 + 16 * C::ROWB;
      const int key = m16 & 7;
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
        const int chunk = kk < C::KKC ? blk * (C::W / 8) + 4 * kk + g4
                                      : C::NBR * (C::W / 8) + 4 * (kk - C::KKC) + g4;
        const int co = 16 * (chunk ^ key);
        const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(rp0 + co));
        const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(rp1 + co));
        S0 = mfma32(a0, Qb[kk], S0);
        S1 = mfma32(a1, Qb[kk], S1);
      }
      if (valid < C::TT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (rowbase + 4 * g4 + i >= valid) S0[i] = -INFINITY;
          if (rowbase + 16 + 4 * g4 + i >= valid) S1[i] = -INFINITY;
        }
      }
      // ---- online softmax (per head m16; lanes m16, m16+16, +32, +48 share a head)
      float mx = fmaxf(fmaxf(fmaxf(S0[0], S0[1]), fmaxf(S0[2], S0[3])),
                       fmaxf(fmaxf(S1[0], S1[1]), fmaxf(S1[2], S1[3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float scale = fast_exp2(m_run - m_use);
      float p0[4], p1[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p0[i] = fast_exp2(S0[i] - m_use);
        p1[i] = fast_exp2(S1[i] - m_use);
        psum += p0[i] + p1[i];
      }
      l_run = l_run * scale + psum;
      m_run = m_new;
      if (__any(scale != 1.f)) {
#pragma unroll
        for (int q = 0; q < C::NQ; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e) O[q][e] *= scale;
      }
      const u32x4_t pbu = u32x4_t{pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]),
                                  pack_bf16x2(p1[0], p1[1]), pack_bf16x2(p1[2], p1[3])};
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pbu);
      // ---- values: O^T[col][head] += C^T[col][tokens] P^T[tokens][head]
#pragma unroll
      for (int q = 0; q < C::NQ; ++q) {
        const int chunk = blk * (C::W / 8) + 16 * q + m16;
        u32x4_t R[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int tr = rowbase + (v < 4 ? 4 * g4 + v : 16 + 4 * g4 + (v - 4));
          R[v] = *reinterpret_cast<const u32x4_t*>(sb + tr * C::ROWB + 16 * (chunk ^ (tr & 7)));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          u32x4_t A;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            A[u] = __builtin_amdgcn_perm(R[2 * u + 1][e >> 1], R[2 * u][e >> 1], sel);
          O[q][e] = mfma32(__builtin_bit_cast(bf16x8_t, A), pb, O[q][e]);
        }
      }
    }

    if (x + 1 == cb_end || x + 1 == x1) {
      // ---- segment end: write this wave's partial and reset.
      float l_tot = l_run + __shfl_xor(l_run, 16);
      l_tot += __shfl_xor(l_tot, 32);
      const int64_t slot = static_cast<int64_t>(unit + cb) * C::G + tgrp;
      if (head_ok) {
        float* dst = po + (slot * HK + hk) * C::W;
#pragma unroll
        for (int q = 0; q < C::NQ; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[128 * q + 8 * (4 * g4 + i) + e] = O[q][e][i];
        if (g4 == 0) {
          pm[slot * HK + hk] = m_run;
          pl[slot * HK + hk] = l_tot;
        }
      }
#pragma unroll
      for (int q = 0; q < C::NQ; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[q][e] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    lds_barrier();
  }
  if (bad_page && lane == 0) atomicOr(&hdr->flags, kFlagBadPage);
}

template <class C>
hipError_t run_variant(const DecodeArgs& a, hipStream_t stream) {
  attend_mfma_kernel<C><<<a.units, C::NTHREADS, 0, stream>>>(a);
  return hipGetLastError();
}

struct Entry {
  MfmaVariant v;
  hipError_t (*fn)(const DecodeArgs&, hipStream_t);
};

template <int W, int DR, int NBR, int HT, int G, int TT, int ST>
constexpr Entry entry() {
  using C = Cfg<W, DR, NBR, HT, G, TT, ST>;
  return Entry{MfmaVariant{W, DR, NBR, HT, G, TT, ST, C::NTHREADS, C::ST * C::TILE_BYTES},
               &run_variant<C>};
}

// Shapes with a tuned MFMA kernel. Key: (w, d_r, blocks per row, 16-head tiles per block).
const Entry kVariants[] = {
    entry<128, 64, 4, 1, 1, 32, 4>(),   // MLRA-4: 4 x 128 latent, <= 16 heads per block
    entry<512, 64, 1, 4, 1, 32, 4>(),   // MLA: one 512 latent, 64 heads
    entry<128, 64, 1, 1, 4, 128, 3>(),  // one MLRA-4 block (a TP rank's share), <= 16 heads
    entry<256, 64, 2, 2, 1, 32, 4>(),   // MLRA-2: 2 x 256 latent, <= 32 heads per block
    entry<128, 64, 4, 2, 1, 32, 4>(),   // 4 x 128 latent, <= 32 heads per block
    entry<128, 64, 4, 4, 1, 32, 4>(),   // 4 x 128 latent, <= 64 heads per block
    entry<256, 64, 1, 2, 2, 64, 4>(),   // one 256 block + RoPE, <= 32 heads
};

}  // namespace

const MfmaVariant* find_mfma_variant(int w, int d_r, int n_blocks, int head_tiles) {
  for (const Entry& e : kVariants)
    if (e.v.w == w && e.v.d_r == d_r && e.v.n_blocks == n_blocks && e.v.head_tiles == head_tiles)
      return &e.v;
  return nullptr;
}

hipError_t launch_attend_mfma(const MfmaVariant* v, const DecodeArgs& a, hipStream_t stream) {
  for (const Entry& e : kVariants)
    if (&e.v == v) return e.fn(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mlra
