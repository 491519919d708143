// Kernel launchers of libmlra (internal; the public interface is include/mlra.h).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace mlra {

// Tuning of one MFMA attention variant (see attend_mfma.hip).
struct MfmaVariant {
  int w, d_r, n_blocks, head_tiles;  // shape key
  int groups, tile_tokens, occupancy;  // tuning (occupancy: workgroups per compute unit)
  int fp8;                             // the cache holds E4M3FN latent codes
  int threads;
  int lds_bytes;
};

// Returns the MFMA variant for this shape, or nullptr when only the generic
// path can run it.
const MfmaVariant* find_mfma_variant(int w, int d_r, int n_blocks, int head_tiles, bool fp8);

hipError_t launch_absorb(const DecodeArgs& a, int dtype, bool q_bf16, const int32_t* seq_lens,
                         const void* q_c, const void* q_r, const void* w_uk, hipStream_t stream);

hipError_t launch_attend_mfma(const MfmaVariant* v, const DecodeArgs& a, hipStream_t stream);

// Generic VALU attention for any supported shape (fp32 or bf16 cache).
constexpr int kGenericTileTokens = 64;
hipError_t launch_attend_generic(const DecodeArgs& a, int dtype, hipStream_t stream);

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream);

hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t stream);

// n_mats matrices W_m share one launch (the heads of a per-head projection).
hipError_t launch_proj(const ProjArgs& a, int n_mats, hipStream_t stream);

}  // namespace mlra
