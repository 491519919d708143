/*
 * CPU oracle for MLRA decode attention over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this code: only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header or constant with the HIP library.
 *
 * Everything here is plain, slow and written to be read against the pages:
 * double-precision accumulation, explicit reconstruction of per-head keys and
 * values from the cached latent, a two-pass softmax, no tiling or fusion.
 */
#ifndef MLRA_ORACLE_H
#define MLRA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings the oracle reads: IEEE fp32 values, or bf16 bit patterns
 * (upper half of an fp32), which widen to double exactly. ORACLE_FP8_E4M3
 * selects a quantised cache (the FP8 latent quantisation the lesty.tech MLA
 * explainer mentions in section 5): cache rows hold the latent as OCP FP8
 * E4M3FN codes followed by the RoPE key in bf16, every latent value being
 * (decoded code) x cache_scale; all other arrays are then bf16.
 * ORACLE_FP8_E4M3_BS is the same cache with one fp32 scale per token and
 * latent block instead of cache_scale: a row is the d_c codes, the d_r bf16
 * RoPE values, n_blocks fp32 scales, then zero bytes up to a multiple of 16
 * (oracle_fp8_row_bytes), and latent value (row, col) = decoded code x the
 * scale of col's block in that row. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 2, ORACLE_FP8_E4M3_BS = 3 };

/* Problem shape, in the notation of the MLRA paper page (Table 6 notation):
 * h query heads of width d_h; a latent of width d_c cut into n_blocks blocks of
 * width d_c / n_blocks; a RoPE key of width d_r shared by all heads. Head i
 * attends blocks_per_head blocks (1 = each head reads exactly one block). */
typedef struct {
  int32_t batch;
  int32_t n_heads;
  int32_t d_h;
  int32_t d_c;             /* latent width stored in each cache row */
  int32_t n_blocks;        /* b */
  int32_t blocks_per_head; /* k */
  int32_t d_r;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t d_model;         /* append only */
  int32_t dtype;           /* ORACLE_F32, ORACLE_BF16 (every input array) or an FP8 cache */
  double softmax_scale;    /* <= 0 selects 1 / sqrt(d_h + d_r) */
  double out_scale;        /* <= 0 selects 1 / sqrt(blocks_per_head) */
  double cache_scale;      /* FP8 caches: scale of every latent code (<= 0 selects 1) */
  int32_t d_cq;            /* query path: width of the query latent c^Q */
  double rope_base;        /* RoPE base (<= 0 selects 10000) */
} oracle_shape;

/* Block attended by head `head` in its `jj`-th slot (0 <= jj < k). */
int32_t oracle_block_of(const oracle_shape* s, int32_t head, int32_t jj);

/* Physical row index of token t of sequence b in the pool. page_table may be
 * NULL (identity layout: page p of sequence b is b * max_pages_per_seq + p). */
int64_t oracle_row_index(const oracle_shape* s, const int32_t* page_table, int32_t b, int32_t t);

/* Un-absorbed decode. For each requested (b, head) pair, reconstructs
 * K = W^UK c and V = W^UV c per cached token, scores with the content and the
 * decoupled RoPE terms, applies a two-pass softmax per attended block and sums
 * the per-block outputs times out_scale.
 *   pool:       [pages][page_size][d_c + d_r] elements; for FP8 caches
 *               [pages][page_size] rows of d_c code bytes then d_r bf16
 *   q_c:        [batch][h][d_h], q_r: [batch][h][d_r]
 *   w_uk, w_uv: [h][k][d_c / n_blocks][d_h]
 *   out:        [npairs][d_h] doubles, lse: [npairs][k] doubles (natural log) */
void oracle_decode_unabsorbed(const oracle_shape* s, const void* pool, const int32_t* page_table,
                              const int32_t* seq_lens, const void* q_c, const void* q_r,
                              const void* w_uk, const void* w_uv, int32_t npairs,
                              const int32_t* pair_b, const int32_t* pair_head, double* out,
                              double* lse);

/* The same result computed the absorbed way: the query is mapped into latent
 * space once, scores are dot products with the raw latent, the softmax-weighted
 * latent sum is up-projected once. Exists to check the absorption identity. */
void oracle_decode_absorbed(const oracle_shape* s, const void* pool, const int32_t* page_table,
                            const int32_t* seq_lens, const void* q_c, const void* q_r,
                            const void* w_uk, const void* w_uv, int32_t npairs,
                            const int32_t* pair_b, const int32_t* pair_head, double* out,
                            double* lse);

/* Latent append: c = x W^DKV accumulated in double and rounded once to the
 * storage type (round to nearest, ties to even), written with kr_new into the
 * row of token positions[b]; c_out (nullable) receives the rounded latent.
 * FP8 caches: c is rounded to fp32, multiplied in fp32 by the fp32 reciprocal
 * of cache_scale and encoded; c_out then receives the fp32 c (before encoding).
 * Block-scaled FP8 caches: c is rounded to fp32 and every latent block of the
 * row is encoded with oracle_fp8_block_encode (its own scale).
 *   x: [batch][d_model], w_dkv: [d_model][d_c], kr_new: [batch][d_r] */
void oracle_append(const oracle_shape* s, void* pool, const int32_t* page_table,
                   const int32_t* positions, const void* x, const void* w_dkv, const void* kr_new,
                   void* c_out);

/* Rotary position embedding (RoFormer, cited by the MLRA index page; the
 * lesty.tech explainer's section 4 applies it to the decoupled key and query):
 * pairs (v[2i], v[2i+1]) of a d-wide vector rotate by the angle pos theta_i,
 * theta_i = base^(-2i/d). In place, d even. */
void oracle_rope(double* v, int32_t d, int32_t pos, double base);

/* The steps on either side of the attention (lesty.tech section 4; MLA's
 * query compression), for the token at positions[b]:
 *   k^R[b] = RoPE(x[b] W^KR)                       W^KR: [d_model][d_r]
 *   c^Q[b] = x[b] W^DQ                             W^DQ: [d_model][d_cq]
 *   q^C[b][i] = c^Q[b] W^UQ[i]                     W^UQ: [h][d_cq][d_h]
 *   q^R[b][i] = RoPE(c^Q[b] W^QR[i])               W^QR: [h][d_cq][d_r]
 * in double; arrays use the shape's array encoding; outputs are doubles
 * (kr_out [batch][d_r], q_c_out [batch][h][d_h], q_r_out [batch][h][d_r]). */
void oracle_rope_key(const oracle_shape* s, const void* x, const void* w_kr, const int32_t* positions,
                     double* kr_out);
void oracle_project_query(const oracle_shape* s, const void* x, const void* w_dq, const void* w_uq,
                          const void* w_qr, const int32_t* positions, double* q_c_out,
                          double* q_r_out);

/* Rounds a double to a bf16 bit pattern, nearest with ties to even. */
uint16_t oracle_round_bf16(double v);

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, subnormals,
 * no infinities, S.1111.111 is NaN, largest finite magnitude 448.
 * decode: the exact value of a code (NaN for the NaN codes).
 * encode: nearest code to an fp32 value, ties to even, magnitudes of 448 and
 * above saturate to 448, NaN gives 0x7F. */
double oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float x);

/* Bytes of one cache row of an FP8 cache: d_c + 2 d_r, plus for the
 * block-scaled layout 4 n_blocks, rounded up to a multiple of 16. */
int64_t oracle_fp8_row_bytes(const oracle_shape* s);

/* Block-scaled encoding of n fp32 latent values (one block of one token): the
 * block's scale is its largest magnitude divided by 448 in fp32 (so that value
 * gets the largest code), or 1 where that quotient is 0, below the smallest
 * normal fp32 or not finite; each code is oracle_e4m3_encode(c[i] x (1 / scale)),
 * the reciprocal and the product rounded to fp32. NaN values are skipped in
 * the largest magnitude (and encode to 0x7F). */
void oracle_fp8_block_encode(const float* c, int32_t n, uint8_t* codes, float* scale);

/* KV-cache elements loaded per token per device (Table 1 of the MLRA paper
 * page), for the methods listed there plus MLRA's block split.
 * method: 0 MHA, 1 MQA, 2 GQA, 3 MLA, 4 MFA, 5 TPA, 6 MLRA. */
double oracle_cache_elems_per_device(int32_t method, int32_t h, int32_t d_h, int32_t g,
                                     int32_t beta_kv, int32_t d_c, int32_t d_r,
                                     int32_t n_blocks, int32_t tp);

/* Elements cached per token (Table 1 "KV Cache" column; p4's demo counts). */
double oracle_cache_elems_per_token(int32_t method, int32_t h, int32_t d_h, int32_t g,
                                    int32_t beta_kv, int32_t d_c, int32_t d_r);

/* Absorbed-decode work for one unit of heads_u query heads reading a w_u-wide
 * latent block plus the d_r-wide RoPE key over n tokens (Table 2 accounting):
 * flops = n heads_u (4 w_u + 2 d_r), bytes = elem_bytes n (w_u + d_r). */
void oracle_decode_flops_bytes(double n, double heads_u, double w_u, double d_r,
                               double elem_bytes, double* flops, double* bytes);

/* Number of OpenMP threads the oracle's parallel loops use. */
int32_t oracle_num_threads(void);
/* Sets that number (n > 0; for timing the oracle on fewer threads). */
void oracle_set_num_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
