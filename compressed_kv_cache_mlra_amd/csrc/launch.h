// Kernel launchers of libmlra (internal; the public interface is include/mlra.h).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/mlra.h"
#include "common.h"

namespace mlra {

// Tuning of one MFMA attention variant (see attend_mfma.hip).
struct MfmaVariant {
  int w, d_r, n_blocks, head_tiles;  // shape key
  int groups, tile_tokens, occupancy;  // tuning (occupancy: workgroups per compute unit)
  int fp8;                             // E4M3FN latent codes: 1 one scale per cache, 2 per token and block
  int threads;
  int lds_bytes;
};

// Returns the MFMA variant for this shape, or nullptr when only the generic
// path can run it.
// fp8: 0 bf16 cache, 1 FP8 with one scale per cache, 2 FP8 with per-token block scales
const MfmaVariant* find_mfma_variant(int w, int d_r, int n_blocks, int head_tiles, int fp8);

hipError_t launch_absorb(const DecodeArgs& a, int dtype, bool q_bf16, const int32_t* seq_lens,
                         const void* q_c, const void* q_r, const void* w_uk, hipStream_t stream);

// t0, t1 (optional): events that the dispatch fills with the kernel's own
// start and stop times (measurement helper mlra_attend_timed)
hipError_t launch_attend_mfma(const MfmaVariant* v, const DecodeArgs& a, hipStream_t stream,
                              hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// Generic VALU attention for any supported shape (fp32 or bf16 cache).
constexpr int kGenericTileTokens = 64;
hipError_t launch_attend_generic(const DecodeArgs& a, int dtype, hipStream_t stream, hipEvent_t t0 = nullptr,
                                 hipEvent_t t1 = nullptr);

hipError_t launch_combine(const CombineArgs& a, int dtype, hipStream_t stream);

hipError_t launch_append(const AppendArgs& a, int dtype, hipStream_t stream);

// n_mats matrices W_m share one launch (the heads of a per-head projection).
hipError_t launch_proj(const ProjArgs& a, int n_mats, hipStream_t stream);

// MFMA projection launch: every job's workgroups in one grid. cpl (2 or 4)
// is the columns each lane loads per weight row; tiles are 16 cpl wide.
// Products whose column tiles give too few workgroups are split along K;
// their fp32 partial sums go to `scratch` (bytes from proj_scratch_bytes for
// the same jobs) and a second kernel sums them in a fixed order and applies
// the epilogue.
size_t proj_mfma_scratch_bytes(ProjBatch b, int cpl);
hipError_t launch_proj_mfma(ProjBatch& b, int cpl, void* scratch, hipStream_t stream);
// Workspace bytes the projection entry points need for this descriptor, and
// where that region starts in the workspace (after the decode's regions).
size_t proj_scratch_bytes(const mlra_desc* d);
// mlra_append_latent on MFMA; kNotEligible when its inputs need the fp32 kernel.
constexpr int kNotEligible = 1;
int append_latent_mfma(const mlra_desc* desc, void* pool, const int32_t* page_table, const int32_t* positions,
                       const void* x, const void* w_dkv, const void* kr_new, void* c_out, void* workspace,
                       size_t ws_bytes, void* stream);
int proj_workspace_region(const mlra_desc* d, size_t* offset, size_t* total);

}  // namespace mlra
