/*
 * mlra.h: C ABI of libmlra, MLRA decode attention over a paged latent cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Method (sources are the pages this library follows):
 *  - The cache keeps, per token, the compressed latent c = W^DKV x and a
 *    d_r-wide RoPE key k^R shared by all heads ("Multi-Head Latent Attention
 *    (MLA): How Low-Rank KV Compression Crushes Transformer Memory Footprints
 *    by 93%", lesty.tech, sections 3 and 4; "Multi-Head Latent Attention",
 *    ai360xpert, "The two projections").
 *  - MLRA splits the latent into n_blocks independent latent heads, each
 *    serving a subset of the query heads; per-subset results are combined
 *    ("Multi-Head Low-Rank Attention: Making Compressed Attention Actually
 *    Parallelizable", alanhou.org, "Core Mechanism"). With blocks_per_head > 1
 *    a head attends several blocks with separate softmaxes and the outputs are
 *    summed times out_scale (the alpha_attn of Tables 16 and 17 on the
 *    "Multi-Head Low-Rank Attention" paper page, thelatestinai.com).
 *  - The up-projections are absorbed: the query is mapped into latent space
 *    once, scores are dot products with the raw cached latent, and W^UV is
 *    applied once to the softmax-weighted latent sum (lesty.tech, section 5).
 *
 * Notation: h = n_heads query heads of width d_h; latent width d_c per cache
 * row cut into b = n_blocks blocks of width w = d_c / b; k = blocks_per_head;
 * head i belongs to group g = i / (h k / b) and attends blocks g k + jj,
 * jj = 0 .. k-1. The softmax scale defaults to 1 / sqrt(d_h + d_r).
 *
 * Memory and ownership (every entry point):
 *  - Every pointer argument is a caller-owned DEVICE pointer (except `desc`,
 *    which is host memory read during the call). Arrays are dense, row-major,
 *    16-byte aligned. The library allocates nothing and keeps no state across
 *    calls (the one exception is the static scratch of
 *    mlra_decode_step_noalloc, below); it is safe to call from several host
 *    threads on different streams with different workspaces.
 *  - `stream` is a hipStream_t (NULL = the default stream). All work is
 *    enqueued on it asynchronously; results are ready when the stream is.
 *  - Element type: every floating-point input (pool, queries, weights, x,
 *    k^R_new, c_out) uses desc->dtype; outputs `out` and `lse` are fp32.
 *    MLRA_FP8_E4M3 is a quantised cache (the FP8 latent quantisation the
 *    lesty.tech MLA explainer mentions in section 5): the pool holds the latent
 *    as OCP FP8 E4M3FN codes, each standing for (decoded code) x cache_scale,
 *    and the RoPE key in bf16; queries, weights, x and k^R_new are bf16 and
 *    c_out is fp32. It is supported for the shapes with an MFMA attention
 *    variant (MLRA_ERR_UNSUPPORTED otherwise).
 *    MLRA_FP8_E4M3_BS is the same quantised cache with one fp32 scale per
 *    token and latent block instead of cache_scale (which it ignores): latent
 *    value (token, col) = (decoded code) x the scale of col's block in that
 *    token's row. Same shapes and array types as MLRA_FP8_E4M3.
 *
 * Cache layout (all entry points):
 *  - pool: [num_pages][page_size][d_c + d_r]; row = [c (d_c) | k^R (d_r)].
 *    MLRA_FP8_E4M3: rows of d_c + 2 d_r bytes, [codes (d_c bytes) | k^R (d_r
 *    bf16)]. MLRA_FP8_E4M3_BS: rows of d_c + 2 d_r + 4 n_blocks bytes rounded
 *    up to a multiple of 16, [codes | k^R (bf16) | n_blocks fp32 scales |
 *    zero pad].
 *  - page_table: int32 [batch][max_pages_per_seq]; token t of sequence b lives
 *    in row page_table[b][t / page_size] * page_size + t % page_size.
 *    NULL means the identity layout: page p of sequence b is
 *    b * max_pages_per_seq + p.
 *  - Only page-table entries for pages that hold tokens are read. A page id
 *    outside [0, num_pages) is never dereferenced: that page is read as page 0
 *    instead and the error flag MLRA_FLAG_BAD_PAGE is raised in the workspace.
 *
 * Errors: every entry point validates its arguments on the host before
 * enqueuing anything. On failure it returns a negative mlra_status and touches
 * no buffer. A failed launch returns MLRA_ERR_HIP. Faults during execution
 * surface at the caller's next synchronisation, as usual for HIP.
 */
#ifndef MLRA_H
#define MLRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLRA_OK = 0,
  MLRA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shape */
  MLRA_ERR_UNSUPPORTED = -2, /* a shape or dtype this build has no kernel for */
  MLRA_ERR_WORKSPACE = -3,   /* workspace smaller than mlra_workspace_bytes() */
  MLRA_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  MLRA_ERR_SCRATCH = -5      /* mlra_decode_step_noalloc: the shape's workspace exceeds
                                MLRA_NOALLOC_SCRATCH_BYTES */
} mlra_status;

typedef enum { MLRA_F32 = 0, MLRA_BF16 = 1, MLRA_FP8_E4M3 = 2, MLRA_FP8_E4M3_BS = 3 } mlra_dtype;

/* Error flags a kernel can raise in the workspace (see mlra_read_flags). */
#define MLRA_FLAG_BAD_PAGE 1u

typedef struct {
  int32_t batch;             /* B, number of sequences (1 .. 4096) */
  int32_t n_heads;           /* h */
  int32_t d_h;               /* query / value head width (1 .. 512) */
  int32_t d_c;               /* latent width stored in each cache row (1 .. 65536) */
  int32_t n_blocks;          /* b: latent blocks per row (1 = MLA); divides d_c */
  int32_t blocks_per_head;   /* k: blocks each head attends (divides b) */
  int32_t d_r;               /* RoPE key width (0 .. 512) */
  int32_t page_size;         /* tokens per page: power of two in [16, 256] */
  int32_t max_pages_per_seq; /* page-table row length (batch * max_pages_per_seq * page_size
                                <= 16 * INT32_MAX, else MLRA_ERR_UNSUPPORTED) */
  int32_t num_pages;         /* pages in the pool */
  int32_t d_model;           /* append only: width of x */
  int32_t dtype;             /* mlra_dtype */
  float softmax_scale;       /* <= 0 selects 1 / sqrt(d_h + d_r) */
  float out_scale;           /* <= 0 selects 1 / sqrt(blocks_per_head) */
  float cache_scale;         /* MLRA_FP8_E4M3: latent value of a code = decoded code x
                                cache_scale (<= 0 selects 1); ignored otherwise (also by
                                MLRA_FP8_E4M3_BS, whose rows carry their scales) */
  int32_t d_cq;              /* mlra_project_query only: query latent width d_c' */
  float rope_base;           /* RoPE frequency base (<= 0 selects 10000) */
} mlra_desc;

/* Bytes of device workspace mlra_decode / mlra_combine need for this shape,
 * plus, with d_model (and d_cq) set, the split-K scratch of mlra_rope_key and
 * mlra_project_query: one workspace serves every entry point of a layer.
 * Depends on the shape and on the number of compute units of the current
 * device, not on the sequence lengths. Returns 0 for an invalid descriptor.
 * max_seq_len: upper bound of the lengths the workspace will be used with
 * (validated to be >= 0 and <= max_pages_per_seq * page_size). */
size_t mlra_workspace_bytes(const mlra_desc* desc, int32_t max_seq_len);

/* Latent append (the down-projection c = W^DKV x of ai360xpert, "The two
 * projections"; W^DKV stored [d_model][d_c]):
 *   c_new[b] = x[b] W^DKV, accumulated in fp32 and rounded once to dtype
 *   (round to nearest, ties to even), then the row [c_new[b] | kr_new[b]] is
 *   written to the pool slot of token positions[b] of sequence b.
 *   x: [batch][d_model]; w_dkv: [d_model][d_c], 16-byte aligned (else
 *   MLRA_ERR_INVALID_ARG); kr_new: [batch][d_r] (already rotated); positions:
 *   int32 [batch] (device); c_out: [batch][d_c] or NULL.
 * MLRA_FP8_E4M3: the fp32 latent is multiplied by the fp32 reciprocal of
 *   cache_scale and encoded to the nearest E4M3FN code (ties to even,
 *   magnitudes of 448 and above saturate to 448, NaN to 0x7F); c_out receives
 *   the fp32 latent before encoding.
 * MLRA_FP8_E4M3_BS: each latent block of the fp32 latent gets the scale
 *   (largest magnitude of the block) / 448 in fp32, or 1 where that quotient
 *   is 0, below the smallest normal fp32 or not finite (NaN values are left
 *   out of the largest magnitude), and is encoded as above with that scale;
 *   the row's scales and zero pad are written too. Needs the MFMA product
 *   (bf16 arrays, d_model % 8 == 0, the alignments below), else
 *   MLRA_ERR_UNSUPPORTED. The workspace also holds the fp32 latents between
 *   the product and the encoding.
 * A position outside [0, max_pages_per_seq * page_size) writes nothing. The
 * caller advances its sequence lengths itself.
 * workspace: at least mlra_workspace_bytes(desc, .) bytes (the decode's
 * workspace, which then also holds this call's split-K scratch; calls sharing
 * it must be ordered on one stream), else MLRA_ERR_WORKSPACE. With bf16
 * arrays, d_model % 8 == 0 and 16-byte aligned x, kr_new and c_out the product
 * runs on MFMA (bf16 operands, fp32 accumulation); otherwise on an fp32 VALU
 * kernel. */
int mlra_append_latent(const mlra_desc* desc, void* pool, const int32_t* page_table,
                       const int32_t* positions, const void* x, const void* w_dkv,
                       const void* kr_new, void* c_out, void* workspace, size_t ws_bytes,
                       void* stream);

/* Query absorption (lesty.tech section 5; ai360xpert "Absorbing the
 * up-projection") and work planning:
 *   q~[b][i][jj] = s * W^UK[i][jj]^T q_c[b][i],  q^R~[b][i] = s * q_r[b][i],
 *   s = softmax_scale * log2(e) (scores are then base-2 logits),
 * written into the workspace, plus the split of all sequences' tokens into
 * balanced work units, computed on the device from seq_lens.
 *   q_c: [batch][h][d_h]; q_r: [batch][h][d_r]; w_uk: [h][k][w][d_h];
 *   seq_lens: int32 [batch] (device), lengths the decode attends; values above
 *   max_pages_per_seq * page_size are clamped to it, negative values read as 0. */
int mlra_absorb_query(const mlra_desc* desc, const int32_t* seq_lens, const void* q_c,
                      const void* q_r, const void* w_uk, void* workspace, size_t ws_bytes,
                      void* stream);

/* Split-K latent attention over the paged cache (the kernel that streams the
 * cache; lesty.tech section 6 describes the MLA analogue): for every work unit
 * and every (head, attended block), base-2 scores q~ . c_j + q^R~ . k^R,
 * online max and sum, and the weighted latent sum sum_t 2^(l_t - m) c_{t,j},
 * written as (m, l, o~) partials into the workspace. Needs the workspace
 * filled by mlra_absorb_query for the same descriptor. */
int mlra_attend(const mlra_desc* desc, const void* pool, const int32_t* page_table, void* workspace,
                size_t ws_bytes, void* stream);

/* mlra_absorb_query followed by mlra_attend. */
int mlra_decode(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                const void* w_uk, void* workspace, size_t ws_bytes, void* stream);

/* Log-sum-exp merge of the partials of each sequence and the absorbed value
 * up-projection (lesty.tech section 5; "results get combined", alanhou.org
 * "Core Mechanism"):
 *   o~[b][i][jj] = merged softmax-weighted latent sum of block J(i)[jj];
 *   out[b][i] = out_scale * sum_jj W^UV[i][jj]^T o~[b][i][jj]   (fp32 [batch][h][d_h])
 *   lse[b][i][jj] = natural-log log-sum-exp of the scaled logits (fp32
 *   [batch][h][k]; NULL to skip). An empty sequence gives out = 0, lse = -inf.
 *   w_uv: [h][k][w][d_h]. */
int mlra_combine(const mlra_desc* desc, const void* workspace, size_t ws_bytes, const void* w_uv,
                 float* out, float* lse, void* stream);

/* One whole decode step: mlra_absorb_query, mlra_attend and mlra_combine
 * enqueued on `stream` by one call, with the same arguments, results and
 * errors as those three calls (every argument is validated before anything is
 * enqueued). It stays three launches: with the combine's workgroups appended
 * to the attention's launch, waiting on per-unit completion flags, the MLRA-4
 * step (B = 32, 8192 tokens) measured about 7 us slower on MI355X. */
int mlra_decode_step(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                     const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                     const void* w_uk, const void* w_uv, float* out, float* lse, void* workspace,
                     size_t ws_bytes, void* stream);

/* Bytes of the static device scratch of mlra_decode_step_noalloc. */
#define MLRA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* mlra_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, results and errors minus the workspace, which is a
 * static device array of MLRA_NOALLOC_SCRATCH_BYTES inside the library (one
 * copy per GPU the library runs on, held until the process ends; its device
 * address is looked up on the first call on each device). The call allocates
 * nothing and frees nothing. Shapes whose mlra_workspace_bytes(desc,
 * max_seq_len) exceeds MLRA_NOALLOC_SCRATCH_BYTES return MLRA_ERR_SCRATCH
 * before anything is enqueued. Every call on one GPU uses that GPU's single
 * scratch copy: calls that overlap in time on one GPU (different streams or
 * host threads without ordering between them) race and give undefined results;
 * calls ordered on one stream are safe. Nothing in the scratch needs to start
 * at zero: each step writes its plan before reading it. The error flags of the
 * step (MLRA_FLAG_*) live in the scratch and cannot be read back through
 * mlra_read_flags. */
int mlra_decode_step_noalloc(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                             const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                             const void* w_uk, const void* w_uv, float* out, float* lse, void* stream);

/* RoPE key of the new token (the decoupled key of lesty.tech section 4,
 * computed from the token's hidden state and rotated for its position):
 *   kr_out[b] = RoPE(x[b] W^KR, positions[b]),  W^KR stored [d_model][d_r].
 * RoPE (RoFormer's rotary embedding): coordinates (2i, 2i+1) of a d-wide
 * vector turn by the angle pos * rope_base^(-2i / d), i = 0 .. d/2 - 1.
 * The product is accumulated in fp32, the angles are evaluated in fp64 and
 * the rotated value is rounded once to the element type.
 *   x: [batch][d_model]; w_kr: 16-byte aligned; positions: int32 [batch]
 *   (device); kr_out: [batch][d_r], ready to be passed to mlra_append_latent
 *   as kr_new. Element type: desc->dtype (bf16 for MLRA_FP8_E4M3).
 *   workspace: at least mlra_workspace_bytes(desc, .) bytes (the decode's
 *   workspace; calls sharing it must be ordered on one stream), else
 *   MLRA_ERR_WORKSPACE; its contents before the call do not matter.
 * With bf16 weights, d_model % 8 == 0 and 16-byte aligned x and kr_out the
 * products run on MFMA (bf16 x and W, fp32 accumulation); otherwise on an fp32
 * VALU kernel. Results are deterministic (fixed summation order).
 * d_r == 0 does nothing; d_r % 8 != 0 is MLRA_ERR_UNSUPPORTED. */
int mlra_rope_key(const mlra_desc* desc, const void* x, const void* w_kr,
                  const int32_t* positions, void* kr_out, void* workspace, size_t ws_bytes,
                  void* stream);

/* The query path (lesty.tech section 4: the query is compressed and split like
 * the key; MLA's parameter count on the "Multi-Head Low-Rank Attention" paper
 * page, thelatestinai.com, lists W^DQ, W^UQ and W^QR):
 *   c_q[b]     = x[b] W^DQ                   (fp32 [batch][d_cq], W^DQ [d_model][d_cq])
 *   q_c[b][i]  = c_q[b] W^UQ[i]              ([batch][h][d_h], W^UQ [h][d_cq][d_h])
 *   q_r[b][i]  = RoPE(c_q[b] W^QR[i], positions[b])  ([batch][h][d_r], W^QR [h][d_cq][d_r])
 * c_q is caller-owned device memory that receives the unrounded fp32
 * compressed query and is read back by the second and third products; q_c
 * and q_r are rounded once to the element type (desc->dtype, bf16 for
 * MLRA_FP8_E4M3) and feed mlra_absorb_query / mlra_decode directly.
 * Weights 16-byte aligned; d_cq, d_h and d_r multiples of 8 (else
 * MLRA_ERR_UNSUPPORTED); with d_r == 0, w_qr, q_r and positions may be NULL.
 * workspace as for mlra_rope_key. On the MFMA path (same conditions as
 * mlra_rope_key, with c_q, q_c and q_r 16-byte aligned) c_q enters the second
 * and third products as two bf16 parts (c_q = hi + lo, about 16 significant
 * bits). */
int mlra_project_query(const mlra_desc* desc, const void* x, const void* w_dq, const void* w_uq,
                       const void* w_qr, const int32_t* positions, float* c_q, void* q_c,
                       void* q_r, void* workspace, size_t ws_bytes, void* stream);

/* Everything the new token's hidden state x feeds before the attention, in
 * one call: the same results as mlra_rope_key (into kr_out), then
 * mlra_append_latent with kr_new = kr_out, then (d_cq > 0) mlra_project_query.
 * On the MFMA path the three products over x (W^DKV, W^KR, W^DQ) share one
 * launch and the pool row, k^R and c^Q are written by its epilogue (a
 * block-scaled FP8 cache's codes and scales by a small encoding launch right
 * after it); the query up-projections take a second launch. w_dq, w_uq, w_qr, c_q, q_c and q_r may
 * be NULL when d_cq == 0; c_out may be NULL. Same layouts, element types and
 * workspace as the three calls. */
int mlra_project_token(const mlra_desc* desc, const void* x, const int32_t* positions, void* pool,
                       const int32_t* page_table, const void* w_dkv, const void* w_kr, void* kr_out,
                       void* c_out, const void* w_dq, const void* w_uq, const void* w_qr, float* c_q,
                       void* q_c, void* q_r, void* workspace, size_t ws_bytes, void* stream);

/* Copies the workspace's error flags (MLRA_FLAG_*) to *flags (host memory),
 * after the work already enqueued on `stream` (synchronises it). The flags are
 * reset by mlra_absorb_query / mlra_decode / mlra_decode_step at the start of each step and raised
 * by the kernels of that step; reading does not clear them. */
int mlra_read_flags(const void* workspace, size_t ws_bytes, uint32_t* flags, void* stream);

/* Measurement helper, not part of the decode path: reads `bytes` (a multiple
 * of 16) of device memory at `src` once, with the 16-byte nontemporal loads
 * and the two-workgroups-per-compute-unit launch that mlra_attend uses for
 * the cache, so the attention's bandwidth can be stated against a plain read
 * on the same device. `sink` (device, >= 16 KiB suffices: 4 bytes per
 * workgroup) receives a checksum so the reads cannot be elided.
 * Errors: MLRA_ERR_INVALID_ARG for NULL pointers, a size not a multiple of 16
 * or a sink that is too small. Asynchronous on `stream`. */
int mlra_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/* Measurement helper, not part of the decode path: mlra_attend, with the
 * attention kernel dispatched through hipExtLaunchKernel so that start_event
 * and stop_event (hipEvent_t, created by the caller) receive the kernel's own
 * start and stop times, as a kernel trace would, rather than the times at
 * which the stream reached two event markers around the launch. Same
 * arguments, results and errors as mlra_attend, plus MLRA_ERR_INVALID_ARG for
 * a NULL event. */
int mlra_attend_timed(const mlra_desc* desc, const void* pool, const int32_t* page_table, void* workspace,
                      size_t ws_bytes, void* start_event, void* stop_event, void* stream);

/* Text for a status code. Never NULL. */
const char* mlra_status_string(int status);

/* ABI version: bumped when a signature or the descriptor changes. */
int mlra_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLRA_H */
