// Host-side descriptor validation of libmlra.
#include "validate.h"

#include <math.h>
#include <stdint.h>

namespace mlra {

int fp8_mode(const mlra_desc* d) {
  return d->dtype == MLRA_FP8_E4M3 ? 1 : d->dtype == MLRA_FP8_E4M3_BS ? 2 : 0;
}

int fp8_row_bytes(const mlra_desc* d) {
  const int rb = d->d_c + 2 * d->d_r + (d->dtype == MLRA_FP8_E4M3_BS ? 4 * d->n_blocks : 0);
  return (rb + 15) / 16 * 16;
}

int check_desc(const mlra_desc* d, ShapeInfo* s) {
  if (!d) return MLRA_ERR_INVALID_ARG;
  if (d->dtype != MLRA_F32 && d->dtype != MLRA_BF16 && d->dtype != MLRA_FP8_E4M3 && d->dtype != MLRA_FP8_E4M3_BS)
    return MLRA_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->n_heads < 1 || d->d_h < 1 || d->d_c < 1 || d->n_blocks < 1 ||
      d->blocks_per_head < 1 || d->d_r < 0 || d->max_pages_per_seq < 1 || d->num_pages < 1)
    return MLRA_ERR_INVALID_ARG;
  // widths bounded before any arithmetic on them (no int overflow below)
  if (d->d_c > kMaxLatent || d->d_r > 512 || d->d_h > 512) return MLRA_ERR_UNSUPPORTED;
  if (d->d_c % d->n_blocks != 0) return MLRA_ERR_INVALID_ARG;
  if (d->n_blocks % d->blocks_per_head != 0) return MLRA_ERR_INVALID_ARG;
  const int groups = d->n_blocks / d->blocks_per_head;  // head groups
  if (d->n_heads % groups != 0) return MLRA_ERR_INVALID_ARG;
  const int ps = d->page_size;
  if (ps < 16 || ps > 256 || (ps & (ps - 1)) != 0) return MLRA_ERR_INVALID_ARG;
  const int elem = d->dtype == MLRA_F32 ? 4 : 2;
  const int64_t row = static_cast<int64_t>(d->d_c) + d->d_r;
  if ((row * elem) % 16 != 0) return MLRA_ERR_INVALID_ARG;
  const int w = d->d_c / d->n_blocks;
  if (d->dtype != MLRA_F32 && (w % 8 != 0 || d->d_r % 8 != 0)) return MLRA_ERR_INVALID_ARG;
  // FP8 rows: d_c code bytes in whole 16-byte chunks, then the bf16 RoPE key
  if (fp8_mode(d) && d->d_c % 16 != 0) return MLRA_ERR_INVALID_ARG;
  if (d->dtype == MLRA_FP8_E4M3 && (!(d->cache_scale == d->cache_scale) || isinf(d->cache_scale)))
    return MLRA_ERR_INVALID_ARG;
  if (d->dtype == MLRA_F32 && (w % 4 != 0 || d->d_r % 4 != 0)) return MLRA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(d->max_pages_per_seq) * ps > INT32_MAX) return MLRA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(d->batch) * d->max_pages_per_seq > INT32_MAX) return MLRA_ERR_INVALID_ARG;
  // the plan counts tiles (>= 16 tokens) of all sequences in int32
  if (static_cast<int64_t>(d->batch) * d->max_pages_per_seq * ps / 16 > INT32_MAX) return MLRA_ERR_UNSUPPORTED;
  if (!(d->softmax_scale == d->softmax_scale) || !(d->out_scale == d->out_scale) ||
      isinf(d->softmax_scale) || isinf(d->out_scale))
    return MLRA_ERR_INVALID_ARG;
  if (d->d_cq < 0 || !(d->rope_base == d->rope_base) || isinf(d->rope_base)) return MLRA_ERR_INVALID_ARG;
  // Kernel limits of this build.
  if (d->batch > kMaxBatch) return MLRA_ERR_UNSUPPORTED;
  if (d->d_h > 512 || d->d_r > 512 || w > 512) return MLRA_ERR_UNSUPPORTED;
  if (d->blocks_per_head * w > 1024 || d->blocks_per_head > 32) return MLRA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->n_heads) * d->blocks_per_head > 65535) return MLRA_ERR_UNSUPPORTED;
  if (s) {
    s->w = w;
    s->hpb = d->n_heads / groups;
    s->head_tiles = (s->hpb + 15) / 16;
    s->hk = d->n_heads * d->blocks_per_head;
    int l = 0;
    while ((1 << l) < ps) ++l;
    s->log2_page = l;
  }
  return MLRA_OK;
}

int check_append(const mlra_desc* d) {
  if (!d) return MLRA_ERR_INVALID_ARG;
  if (d->d_model < 1) return MLRA_ERR_INVALID_ARG;
  return MLRA_OK;
}

}  // namespace mlra
