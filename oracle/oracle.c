/*
 * CPU oracle for MLRA decode attention over a paged latent cache.
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path. It shares no
 * code with the HIP library.
 *
 * Sources (the pages this follows):
 *  - "Multi-Head Latent Attention" concept page (ai360xpert), "The two
 *    projections": the cache keeps c = W^DKV x per token; per-head keys and
 *    values are rebuilt as K_h = W^UK_h c and V_h = W^UV_h c. "Show Me the
 *    Code" stores the up-projections as (H, d_c, d_head).
 *  - "Multi-Head Latent Attention (MLA): How Low-Rank KV Compression Crushes
 *    Transformer Memory Footprints by 93%" (lesty.tech), section 4 "The
 *    Decoupled RoPE Mechanism": the attention logit is the content dot product
 *    plus the dot product of the query's RoPE part with a d_r-wide key that all
 *    heads share; the cache holds [c, k^R]. Section 5 "On-The-Fly Matrix
 *    Absorption": q W^UK^T against raw c, and the value up-projection applied
 *    once to the softmax-weighted latent sum.
 *  - "Multi-Head Low-Rank Attention: Making Compressed Attention Actually
 *    Parallelizable" (alanhou.org), "Core Mechanism" and "Key Concepts": the
 *    latent is split into independent latent heads, each serving a subset of
 *    the query heads, with per-subset attention whose results are combined.
 *  - "Multi-Head Low-Rank Attention" paper page (thelatestinai.com), Table 1
 *    (cache and loading per token per device) and Table 2 (decode arithmetic
 *    intensity): the counters at the end of this file.
 *
 * Readings where the pages leave a step open (all listed with reasons in the
 * repository's design notes): softmax scale 1/sqrt(d_h + d_r); head i of h
 * reads blocks J(i) = {g k + jj : jj < k} with g = i / (h k / b); each
 * attended block has its own softmax and the per-block outputs are summed
 * times out_scale (1/sqrt(k), which is 1 when k = 1); an empty sequence gives
 * a zero output and lse = -inf.
 *
 * parity pins: every function here is pinned by tests/test_oracle_*.py
 * (closed forms, brute force, textbook attention, Table 1 / Table 2 values).
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- elements */

static double elem(int32_t dtype, const void* base, int64_t idx) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  return (double)((const float*)base)[idx];
}

uint16_t oracle_round_bf16(double v) {
  /* bf16 keeps 8 significant bits. Scale the magnitude so those bits are the
   * integer part, round half to even with rint (default rounding mode), scale
   * back: the result is exactly representable in fp32, whose top half is the
   * bf16 pattern. */
  if (v != v) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
  double r = ldexp(rint(ldexp(m, 8)), e - 8);
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u >> 16) | sign);
}

/* OCP FP8 E4M3FN (see oracle.h). A normal code e.m (e >= 1) is
 * (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); a subnormal (e = 0) is m 2^-9. */
double oracle_e4m3_decode(uint8_t code) {
  const int sgn = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return sgn ? -v : v;
}

/* Codes in the binade [2^E, 2^(E+1)) (E >= -6) are spaced 2^(E-3); below 2^-6
 * the subnormal spacing 2^-9 continues. With E' = max(E, -6) the nearest
 * multiple n 2^(E'-3) of |x| (n in 0..16) has code (E' + 6) 8 + n, which also
 * covers n = 16 (the next binade) and the subnormal range (E' = -6). */
uint8_t oracle_e4m3_encode(float x) {
  if (x != x) return 0x7F;
  const uint8_t sgn = signbit(x) ? 0x80 : 0;
  const double a = fabs((double)x);
  if (a >= 448.0) return sgn | 0x7E;
  int e2;
  frexp(a, &e2); /* a = f 2^e2 with f in [0.5, 1): floor(log2 a) = e2 - 1 */
  int E = a == 0.0 ? -6 : e2 - 1;
  if (E < -6) E = -6;
  const double n = rint(ldexp(a, 3 - E)); /* exact scaling, ties to even */
  return sgn | (uint8_t)((E + 6) * 8 + (int)n);
}

static int is_fp8(const oracle_shape* s) {
  return s->dtype == ORACLE_FP8_E4M3 || s->dtype == ORACLE_FP8_E4M3_BS;
}

int64_t oracle_fp8_row_bytes(const oracle_shape* s) {
  int64_t rb = s->d_c + 2 * (int64_t)s->d_r;
  if (s->dtype == ORACLE_FP8_E4M3_BS) rb += 4 * (int64_t)s->n_blocks;
  return (rb + 15) / 16 * 16;
}

void oracle_fp8_block_encode(const float* c, int32_t n, uint8_t* codes, float* scale) {
  float amax = 0.0f;
  for (int32_t i = 0; i < n; ++i)
    if (fabsf(c[i]) > amax) amax = fabsf(c[i]); /* false for NaN */
  float sc = amax / 448.0f;
  if (!(sc >= FLT_MIN) || isinf(sc)) sc = 1.0f;
  const float inv = 1.0f / sc;
  for (int32_t i = 0; i < n; ++i) codes[i] = oracle_e4m3_encode(c[i] * inv);
  *scale = sc;
}

/* Latent value `col` and RoPE value `r` of pool row `row_idx`. */
static double pool_latent(const oracle_shape* s, const void* pool, int64_t row_idx, int32_t col) {
  if (is_fp8(s)) {
    const uint8_t* row = (const uint8_t*)pool + row_idx * oracle_fp8_row_bytes(s);
    double sc = s->cache_scale > 0 ? s->cache_scale : 1.0;
    if (s->dtype == ORACLE_FP8_E4M3_BS) {
      float f; /* the scale of col's block in this row */
      memcpy(&f, row + s->d_c + 2 * (int64_t)s->d_r + 4 * (int64_t)(col / (s->d_c / s->n_blocks)), 4);
      sc = f;
    }
    return oracle_e4m3_decode(row[col]) * sc;
  }
  return elem(s->dtype, pool, row_idx * (s->d_c + s->d_r) + col);
}

static double pool_rope(const oracle_shape* s, const void* pool, int64_t row_idx, int32_t r) {
  if (is_fp8(s)) {
    const int64_t rb = oracle_fp8_row_bytes(s);
    uint16_t v;
    memcpy(&v, (const uint8_t*)pool + row_idx * rb + s->d_c + 2 * (int64_t)r, 2);
    return elem(ORACLE_BF16, &v, 0);
  }
  return elem(s->dtype, pool, row_idx * (s->d_c + s->d_r) + s->d_c + r);
}

/* Encoding of the non-cache arrays (queries, weights, x, k^R_new). */
static int32_t arrays_dtype(const oracle_shape* s) {
  return is_fp8(s) ? ORACLE_BF16 : s->dtype;
}

static void store_elem(int32_t dtype, void* base, int64_t idx, double v) {
  if (dtype == ORACLE_BF16)
    ((uint16_t*)base)[idx] = oracle_round_bf16(v);
  else
    ((float*)base)[idx] = (float)v;
}

/* ------------------------------------------------------------------ shape */

static double scale_of(const oracle_shape* s) {
  return s->softmax_scale > 0 ? s->softmax_scale : 1.0 / sqrt((double)(s->d_h + s->d_r));
}

static double out_scale_of(const oracle_shape* s) {
  return s->out_scale > 0 ? s->out_scale : 1.0 / sqrt((double)s->blocks_per_head);
}

int32_t oracle_block_of(const oracle_shape* s, int32_t head, int32_t jj) {
  /* b / k head groups; each group owns k consecutive blocks and h k / b heads. */
  int32_t heads_per_group = s->n_heads * s->blocks_per_head / s->n_blocks;
  int32_t group = head / heads_per_group;
  return group * s->blocks_per_head + jj;
}

int64_t oracle_row_index(const oracle_shape* s, const int32_t* page_table, int32_t b, int32_t t) {
  int32_t logical_page = t / s->page_size;
  int32_t offset = t % s->page_size;
  int64_t phys = page_table ? (int64_t)page_table[(int64_t)b * s->max_pages_per_seq + logical_page]
                            : (int64_t)b * s->max_pages_per_seq + logical_page;
  return phys * s->page_size + offset;
}

/* ------------------------------------------------------ un-absorbed decode */

void oracle_decode_unabsorbed(const oracle_shape* s, const void* pool, const int32_t* page_table,
                              const int32_t* seq_lens, const void* q_c, const void* q_r,
                              const void* w_uk, const void* w_uv, int32_t npairs,
                              const int32_t* pair_b, const int32_t* pair_head, double* out,
                              double* lse) {
  const int32_t H = s->n_heads, DH = s->d_h, DR = s->d_r, K = s->blocks_per_head;
  const int32_t W = s->d_c / s->n_blocks;
  const double sigma = scale_of(s), alpha = out_scale_of(s);
  const int32_t dt = arrays_dtype(s);

#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t p = 0; p < npairs; ++p) {
    const int32_t b = pair_b[p], i = pair_head[p];
    const int32_t n = seq_lens[b];
    double* o = out + (int64_t)p * DH;
    for (int32_t d = 0; d < DH; ++d) o[d] = 0.0;
    if (n <= 0) {
      for (int32_t jj = 0; jj < K; ++jj) lse[(int64_t)p * K + jj] = -INFINITY;
      continue;
    }
    double* q = (double*)malloc(sizeof(double) * (DH + DR));
    double* wk = (double*)malloc(sizeof(double) * (size_t)W * DH);
    double* wv = (double*)malloc(sizeof(double) * (size_t)W * DH);
    double* c = (double*)malloc(sizeof(double) * W);
    double* kvec = (double*)malloc(sizeof(double) * DH);
    double* score = (double*)malloc(sizeof(double) * n);
    for (int32_t d = 0; d < DH; ++d) q[d] = elem(dt, q_c, ((int64_t)b * H + i) * DH + d);
    for (int32_t r = 0; r < DR; ++r) q[DH + r] = elem(dt, q_r, ((int64_t)b * H + i) * DR + r);

    for (int32_t jj = 0; jj < K; ++jj) {
      const int32_t j = oracle_block_of(s, i, jj);
      const int64_t wbase = ((int64_t)i * K + jj) * W * DH;
      for (int64_t e = 0; e < (int64_t)W * DH; ++e) {
        wk[e] = elem(dt, w_uk, wbase + e);
        wv[e] = elem(dt, w_uv, wbase + e);
      }
      /* pass 1: reconstruct the key of every token and score it */
      double m = -INFINITY;
      for (int32_t t = 0; t < n; ++t) {
        const int64_t row = oracle_row_index(s, page_table, b, t);
        for (int32_t cc = 0; cc < W; ++cc) c[cc] = pool_latent(s, pool, row, j * W + cc);
        for (int32_t d = 0; d < DH; ++d) kvec[d] = 0.0;
        for (int32_t cc = 0; cc < W; ++cc) /* K_t = W^UK_{i,j}^T c_{t,j} */
          for (int32_t d = 0; d < DH; ++d) kvec[d] += wk[(int64_t)cc * DH + d] * c[cc];
        double content = 0.0, rope = 0.0;
        for (int32_t d = 0; d < DH; ++d) content += q[d] * kvec[d];
        for (int32_t r = 0; r < DR; ++r) rope += q[DH + r] * pool_rope(s, pool, row, r);
        score[t] = sigma * (content + rope);
        if (score[t] > m) m = score[t];
      }
      /* pass 2: softmax weights, reconstruct every value, accumulate */
      double denom = 0.0;
      for (int32_t t = 0; t < n; ++t) denom += exp(score[t] - m);
      for (int32_t t = 0; t < n; ++t) {
        const double pt = exp(score[t] - m) / denom;
        const int64_t row = oracle_row_index(s, page_table, b, t);
        for (int32_t cc = 0; cc < W; ++cc) c[cc] = pool_latent(s, pool, row, j * W + cc);
        for (int32_t d = 0; d < DH; ++d) kvec[d] = 0.0; /* reused as V_t */
        for (int32_t cc = 0; cc < W; ++cc)
          for (int32_t d = 0; d < DH; ++d) kvec[d] += wv[(int64_t)cc * DH + d] * c[cc];
        for (int32_t d = 0; d < DH; ++d) o[d] += alpha * pt * kvec[d];
      }
      lse[(int64_t)p * K + jj] = m + log(denom);
    }
    free(q); free(wk); free(wv); free(c); free(kvec); free(score);
  }
}

/* -------------------------------------------------------- absorbed decode */

void oracle_decode_absorbed(const oracle_shape* s, const void* pool, const int32_t* page_table,
                            const int32_t* seq_lens, const void* q_c, const void* q_r,
                            const void* w_uk, const void* w_uv, int32_t npairs,
                            const int32_t* pair_b, const int32_t* pair_head, double* out,
                            double* lse) {
  const int32_t H = s->n_heads, DH = s->d_h, DR = s->d_r, K = s->blocks_per_head;
  const int32_t W = s->d_c / s->n_blocks;
  const double sigma = scale_of(s), alpha = out_scale_of(s);
  const int32_t dt = arrays_dtype(s);

#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t p = 0; p < npairs; ++p) {
    const int32_t b = pair_b[p], i = pair_head[p];
    const int32_t n = seq_lens[b];
    double* o = out + (int64_t)p * DH;
    for (int32_t d = 0; d < DH; ++d) o[d] = 0.0;
    if (n <= 0) {
      for (int32_t jj = 0; jj < K; ++jj) lse[(int64_t)p * K + jj] = -INFINITY;
      continue;
    }
    double* qt = (double*)malloc(sizeof(double) * W);   /* W^UK^T q, in latent space */
    double* acc = (double*)malloc(sizeof(double) * W);  /* sum_t p_t c_t */
    double* score = (double*)malloc(sizeof(double) * n);
    for (int32_t jj = 0; jj < K; ++jj) {
      const int32_t j = oracle_block_of(s, i, jj);
      const int64_t wbase = ((int64_t)i * K + jj) * W * DH;
      for (int32_t cc = 0; cc < W; ++cc) {
        double v = 0.0;
        for (int32_t d = 0; d < DH; ++d)
          v += elem(dt, w_uk, wbase + (int64_t)cc * DH + d) * elem(dt, q_c, ((int64_t)b * H + i) * DH + d);
        qt[cc] = v;
      }
      double m = -INFINITY;
      for (int32_t t = 0; t < n; ++t) {
        const int64_t row = oracle_row_index(s, page_table, b, t);
        double v = 0.0;
        for (int32_t cc = 0; cc < W; ++cc) v += qt[cc] * pool_latent(s, pool, row, j * W + cc);
        for (int32_t r = 0; r < DR; ++r)
          v += elem(dt, q_r, ((int64_t)b * H + i) * DR + r) * pool_rope(s, pool, row, r);
        score[t] = sigma * v;
        if (score[t] > m) m = score[t];
      }
      double denom = 0.0;
      for (int32_t t = 0; t < n; ++t) denom += exp(score[t] - m);
      for (int32_t cc = 0; cc < W; ++cc) acc[cc] = 0.0;
      for (int32_t t = 0; t < n; ++t) {
        const double pt = exp(score[t] - m) / denom;
        const int64_t row = oracle_row_index(s, page_table, b, t);
        for (int32_t cc = 0; cc < W; ++cc) acc[cc] += pt * pool_latent(s, pool, row, j * W + cc);
      }
      for (int32_t d = 0; d < DH; ++d) {
        double v = 0.0;
        for (int32_t cc = 0; cc < W; ++cc) v += elem(dt, w_uv, wbase + (int64_t)cc * DH + d) * acc[cc];
        o[d] += alpha * v;
      }
      lse[(int64_t)p * K + jj] = m + log(denom);
    }
    free(qt); free(acc); free(score);
  }
}

/* ----------------------------------------------------------------- append */

void oracle_append(const oracle_shape* s, void* pool, const int32_t* page_table,
                   const int32_t* positions, const void* x, const void* w_dkv, const void* kr_new,
                   void* c_out) {
  const int32_t DC = s->d_c, DR = s->d_r, DM = s->d_model, ROW = s->d_c + s->d_r;
  if (is_fp8(s)) {
    const int64_t rb = oracle_fp8_row_bytes(s);
    const float inv = 1.0f / (float)(s->cache_scale > 0 ? s->cache_scale : 1.0);
    float* cf = (float*)malloc(sizeof(float) * (size_t)(DC > 0 ? DC : 1));
    for (int32_t b = 0; b < s->batch; ++b) {
      uint8_t* row = (uint8_t*)pool + oracle_row_index(s, page_table, b, positions[b]) * rb;
      for (int32_t cc = 0; cc < DC; ++cc) {
        double v = 0.0;
        for (int32_t m = 0; m < DM; ++m)
          v += elem(ORACLE_BF16, x, (int64_t)b * DM + m) * elem(ORACLE_BF16, w_dkv, (int64_t)m * DC + cc);
        cf[cc] = (float)v;
        if (c_out) ((float*)c_out)[(int64_t)b * DC + cc] = cf[cc];
      }
      if (s->dtype == ORACLE_FP8_E4M3_BS) {
        const int32_t W = DC / s->n_blocks;
        memset(row, 0, (size_t)rb); /* the pad bytes */
        for (int32_t j = 0; j < s->n_blocks; ++j) {
          float sc;
          oracle_fp8_block_encode(cf + (int64_t)j * W, W, row + (int64_t)j * W, &sc);
          memcpy(row + DC + 2 * (int64_t)DR + 4 * (int64_t)j, &sc, 4);
        }
      } else {
        for (int32_t cc = 0; cc < DC; ++cc) row[cc] = oracle_e4m3_encode(cf[cc] * inv);
      }
      memcpy(row + DC, (const uint16_t*)kr_new + (int64_t)b * DR, 2 * (size_t)DR);
    }
    free(cf);
    return;
  }
  const int32_t dt = s->dtype;
  for (int32_t b = 0; b < s->batch; ++b) {
    const int64_t row = oracle_row_index(s, page_table, b, positions[b]) * ROW;
    for (int32_t cc = 0; cc < DC; ++cc) {
      double v = 0.0; /* c = x W^DKV, W^DKV stored [d_model][d_c] */
      for (int32_t m = 0; m < DM; ++m)
        v += elem(dt, x, (int64_t)b * DM + m) * elem(dt, w_dkv, (int64_t)m * DC + cc);
      store_elem(dt, pool, row + cc, v);
      if (c_out) store_elem(dt, c_out, (int64_t)b * DC + cc, v);
    }
    for (int32_t r = 0; r < DR; ++r)
      store_elem(dt, pool, row + DC + r, elem(dt, kr_new, (int64_t)b * DR + r));
  }
}

/* ------------------------------------------------ RoPE and the query path */

static double rope_base_of(const oracle_shape* s) { return s->rope_base > 0 ? s->rope_base : 10000.0; }

void oracle_rope(double* v, int32_t d, int32_t pos, double base) {
  for (int32_t i = 0; i < d / 2; ++i) {
    const double theta = pow(base, -2.0 * i / d);
    const double a = (double)pos * theta, c = cos(a), sn = sin(a);
    const double x0 = v[2 * i], x1 = v[2 * i + 1];
    v[2 * i] = x0 * c - x1 * sn;
    v[2 * i + 1] = x0 * sn + x1 * c;
  }
}

void oracle_rope_key(const oracle_shape* s, const void* x, const void* w_kr, const int32_t* positions,
                     double* kr_out) {
  const int32_t DM = s->d_model, DR = s->d_r, dt = arrays_dtype(s);
  for (int32_t b = 0; b < s->batch; ++b) {
    double* k = kr_out + (int64_t)b * DR;
    for (int32_t r = 0; r < DR; ++r) { /* h W^KR, W^KR stored [d_model][d_r] */
      double v = 0.0;
      for (int32_t m = 0; m < DM; ++m) v += elem(dt, x, (int64_t)b * DM + m) * elem(dt, w_kr, (int64_t)m * DR + r);
      k[r] = v;
    }
    oracle_rope(k, DR, positions[b], rope_base_of(s));
  }
}

void oracle_project_query(const oracle_shape* s, const void* x, const void* w_dq, const void* w_uq,
                          const void* w_qr, const int32_t* positions, double* q_c_out,
                          double* q_r_out) {
  const int32_t DM = s->d_model, DQ = s->d_cq, H = s->n_heads, DH = s->d_h, DR = s->d_r;
  const int32_t dt = arrays_dtype(s);
  double* cq = (double*)malloc(sizeof(double) * (size_t)DQ);
  for (int32_t b = 0; b < s->batch; ++b) {
    for (int32_t c = 0; c < DQ; ++c) { /* c^Q = h W^DQ */
      double v = 0.0;
      for (int32_t m = 0; m < DM; ++m) v += elem(dt, x, (int64_t)b * DM + m) * elem(dt, w_dq, (int64_t)m * DQ + c);
      cq[c] = v;
    }
    for (int32_t i = 0; i < H; ++i) {
      double* qc = q_c_out + ((int64_t)b * H + i) * DH;
      double* qr = q_r_out + ((int64_t)b * H + i) * DR;
      for (int32_t d = 0; d < DH; ++d) { /* q^C_i = c^Q W^UQ_i */
        double v = 0.0;
        for (int32_t c = 0; c < DQ; ++c) v += cq[c] * elem(dt, w_uq, ((int64_t)i * DQ + c) * DH + d);
        qc[d] = v;
      }
      for (int32_t r = 0; r < DR; ++r) { /* q^R_i = RoPE(c^Q W^QR_i) */
        double v = 0.0;
        for (int32_t c = 0; c < DQ; ++c) v += cq[c] * elem(dt, w_qr, ((int64_t)i * DQ + c) * DR + r);
        qr[r] = v;
      }
      oracle_rope(qr, DR, positions[b], rope_base_of(s));
    }
  }
  free(cq);
}

/* --------------------------------------------------------------- counters */

double oracle_cache_elems_per_token(int32_t method, int32_t h, int32_t d_h, int32_t g,
                                    int32_t beta_kv, int32_t d_c, int32_t d_r) {
  switch (method) {
    case 0: return 2.0 * h * d_h;                     /* MHA: K and V of every head */
    case 1: return 2.0 * d_h;                         /* MQA: one shared K/V head */
    case 2: return 2.0 * g * d_h;                     /* GQA: one K/V head per group */
    case 3: return (double)d_c + d_r;                 /* MLA: latent + shared RoPE key */
    case 4: return 2.0 * 2.0 * d_h;                   /* MFA: one K/V head of width 2 d_h */
    case 5: return 2.0 * beta_kv * ((double)h + d_h); /* TPA: rank-beta_kv factors of K and V */
    case 6: return (double)d_c + d_r;                 /* MLRA: the blocks together are d_c wide */
    default: return -1.0;
  }
}

double oracle_cache_elems_per_device(int32_t method, int32_t h, int32_t d_h, int32_t g,
                                     int32_t beta_kv, int32_t d_c, int32_t d_r,
                                     int32_t n_blocks, int32_t tp) {
  /* Tensor parallelism over heads: whatever is per-head is split, whatever is
   * shared by all heads is replicated on every device. */
  switch (method) {
    case 0: return 2.0 * ((double)h / tp) * d_h;
    case 1: return 2.0 * d_h;
    case 2: return 2.0 * ((double)g / (tp < g ? tp : g)) * d_h;
    case 3: return (double)d_c + d_r;
    case 4: return 2.0 * 2.0 * d_h;
    case 5: return 2.0 * beta_kv * ((double)h / tp + d_h);
    case 6: { /* each device holds its share of the latent blocks plus the RoPE key */
      int32_t shards = tp < n_blocks ? tp : n_blocks;
      return (double)d_c / shards + d_r;
    }
    default: return -1.0;
  }
}

void oracle_decode_flops_bytes(double n, double heads_u, double w_u, double d_r,
                               double elem_bytes, double* flops, double* bytes) {
  /* per token and head: score q~ . c (2 w_u) + q^R . k^R (2 d_r), weighted sum
   * p c (2 w_u); every cached element of the unit is loaded once per token. */
  *flops = n * heads_u * (2.0 * (w_u + d_r) + 2.0 * w_u);
  *bytes = elem_bytes * n * (w_u + d_r);
}

void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int32_t oracle_num_threads(void) {
#ifdef _OPENMP
  return (int32_t)omp_get_max_threads();
#else
  return 1;
#endif
}
