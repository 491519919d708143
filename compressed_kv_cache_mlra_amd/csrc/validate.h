// Host-side descriptor validation of libmlra (no HIP calls: runs before any
// launch, and on machines without a GPU).
#pragma once

#include "../../include/mlra.h"

namespace mlra {

constexpr int kMaxBatch = 4096;    // sequences per call (the plan keeps them in LDS)
constexpr int kMaxLatent = 65536;  // latent width d_c of a cache row

struct ShapeInfo {
  int w;           // latent block width d_c / n_blocks
  int hpb;         // heads per block h k / b
  int head_tiles;  // ceil(hpb / 16)
  int hk;          // head-block pairs h k
  int log2_page;
};

// Checks a descriptor; fills `s` on success. Returns an mlra_status.
int check_desc(const mlra_desc* d, ShapeInfo* s);

// Extra checks of the append entry point.
int check_append(const mlra_desc* d);

// FP8 caches: 1 per-cache scale, 2 one scale per token and latent block; 0 otherwise.
int fp8_mode(const mlra_desc* d);

// Bytes of one FP8 cache row (codes, bf16 k^R, block scales, pad to 16).
int fp8_row_bytes(const mlra_desc* d);

}  // namespace mlra
