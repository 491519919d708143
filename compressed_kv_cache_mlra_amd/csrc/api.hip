// C ABI of libmlra: argument validation, work planning, workspace layout and
// kernel launches. The public contract is documented in include/mlra.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/mlra.h"
#include "common.h"
#include "launch.h"
#include "validate.h"

namespace mlra {
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

struct Plan {
  ShapeInfo s;
  const MfmaVariant* variant;  // nullptr: generic path
  int tile_tokens;
  int groups;
  int units;
  int64_t slots;
  size_t off_cum, off_nlen, off_sunit, off_udesc, off_qext, off_pm, off_pl, off_po, off_proj, total;
  bool q_bf16;
};

int make_plan(const mlra_desc* d, Plan* p) {
  int st = check_desc(d, &p->s);
  if (st != MLRA_OK) return st;
  const ShapeInfo& s = p->s;
  const int fp8 = fp8_mode(d);
  p->variant = d->dtype != MLRA_F32 ? find_mfma_variant(s.w, d->d_r, d->n_blocks, s.head_tiles, fp8)
                                    : nullptr;
  if (fp8 && !p->variant) return MLRA_ERR_UNSUPPORTED;  // FP8 caches run on the MFMA variants only
  if (p->variant) {
    p->tile_tokens = p->variant->tile_tokens;
    p->groups = p->variant->groups;
    p->q_bf16 = true;
  } else {
    p->tile_tokens = kGenericTileTokens;
    p->groups = 1;
    p->q_bf16 = false;
  }
  p->units = compute_units() * (p->variant ? p->variant->occupancy : 1);
  p->slots = static_cast<int64_t>(p->units + d->batch) * p->groups + 1;  // + the empty slot
  // absorbed-query row: 4 w + 2 d_r bytes on the MFMA path (bf16 hi + lo, or
  // fp16 + a row scale, and the bf16 RoPE part), fp32 [w + d_r] otherwise
  const size_t qrow = p->q_bf16 ? 4 * static_cast<size_t>(s.w) + 2 * static_cast<size_t>(d->d_r)
                                : 4 * static_cast<size_t>(s.w + d->d_r);
  size_t off = align_up(sizeof(WsHeader));
  p->off_cum = off;
  off = align_up(off + sizeof(int32_t) * (d->batch + 1));
  p->off_nlen = off;
  off = align_up(off + sizeof(int32_t) * d->batch);
  p->off_sunit = off;
  off = align_up(off + sizeof(int32_t) * 2 * d->batch);
  p->off_udesc = off;
  off = align_up(off + sizeof(int32_t) * kUnitDescInts * static_cast<size_t>(p->units));
  p->off_qext = off;
  off = align_up(off + qrow * static_cast<size_t>(d->batch) * s.hk);
  p->off_pm = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p->slots) * s.hk);
  p->off_pl = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p->slots) * s.hk);
  p->off_po = off;
  // weighted latent sums: fp16 on the MFMA path (rows scaled into (-1, 1) by a
  // power of two folded into m and l), fp32 on the generic path
  off = align_up(off + (p->variant ? 2 : 4) * static_cast<size_t>(p->slots) * s.hk * s.w);
  p->off_proj = off;  // split-K partials of the projections (rope key, query path)
  off = align_up(off + proj_scratch_bytes(d));
  p->total = off;
  return MLRA_OK;
}

}  // namespace

int proj_workspace_region(const mlra_desc* d, size_t* offset, size_t* total) {
  Plan p;
  const int st = make_plan(d, &p);
  if (st != MLRA_OK) return st;
  *offset = p.off_proj;
  *total = p.total;
  return MLRA_OK;
}

namespace {

// FP8 caches: the value one code unit stands for (1 for other caches).
float cache_scale_of(const mlra_desc* d) {
  return d->dtype == MLRA_FP8_E4M3 && d->cache_scale > 0.f ? d->cache_scale : 1.0f;
}

DecodeArgs decode_args(const mlra_desc* d, const Plan& p, const void* pool, const int32_t* pt,
                       void* ws) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.pool = pool;
  a.page_table = pt;
  a.ws = static_cast<char*>(ws);
  a.off_cum = static_cast<int64_t>(p.off_cum);
  a.off_nlen = static_cast<int64_t>(p.off_nlen);
  a.off_sunit = static_cast<int64_t>(p.off_sunit);
  a.off_udesc = static_cast<int64_t>(p.off_udesc);
  a.off_qext = static_cast<int64_t>(p.off_qext);
  a.off_pm = static_cast<int64_t>(p.off_pm);
  a.off_pl = static_cast<int64_t>(p.off_pl);
  a.off_po = static_cast<int64_t>(p.off_po);
  a.po_f16 = p.variant ? 1 : 0;
  a.q_mode = !p.variant ? kQueryF32 : (fp8_mode(d) ? kQueryF16 : kQuerySplit);
  a.batch = d->batch;
  a.n_heads = d->n_heads;
  a.d_h = d->d_h;
  a.w = p.s.w;
  a.n_blocks = d->n_blocks;
  a.k = d->blocks_per_head;
  a.hpb = p.s.hpb;
  a.d_r = d->d_r;
  a.row = d->d_c + d->d_r;
  a.page_size = d->page_size;
  a.log2_page = p.s.log2_page;
  a.max_pages = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.units = p.units;
  a.tile_tokens = p.tile_tokens;
  a.groups = p.groups;
  a.empty_slot = static_cast<int32_t>(p.slots - 1);
  const float sigma = d->softmax_scale > 0.f ? d->softmax_scale
                                             : 1.0f / sqrtf(static_cast<float>(d->d_h + d->d_r));
  a.qscale = sigma * 1.4426950408889634f;
  a.out_scale = d->out_scale > 0.f ? d->out_scale
                                   : 1.0f / sqrtf(static_cast<float>(d->blocks_per_head));
  a.lat_scale = cache_scale_of(d);
  return a;
}

CombineArgs combine_args(const mlra_desc* d, const Plan& p, const void* ws, const void* w_uv, float* out,
                         float* lse) {
  CombineArgs c;
  memset(&c, 0, sizeof(c));
  c.ws = static_cast<const char*>(ws);
  c.w_uv = w_uv;
  c.out = out;
  c.lse = lse;
  c.off_sunit = static_cast<int64_t>(p.off_sunit);
  c.off_pm = static_cast<int64_t>(p.off_pm);
  c.off_pl = static_cast<int64_t>(p.off_pl);
  c.off_po = static_cast<int64_t>(p.off_po);
  c.po_f16 = p.variant ? 1 : 0;
  c.batch = d->batch;
  c.n_heads = d->n_heads;
  c.d_h = d->d_h;
  c.w = p.s.w;
  c.k = d->blocks_per_head;
  c.hk = p.s.hk;
  c.groups = p.groups;
  c.empty_slot = static_cast<int32_t>(p.slots - 1);
  c.out_scale = d->out_scale > 0.f ? d->out_scale : 1.0f / sqrtf(static_cast<float>(d->blocks_per_head));
  c.out_scale *= cache_scale_of(d);  // FP8 caches: the partials sum codes, not latent values
  return c;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MLRA_OK : MLRA_ERR_HIP; }

// ------------------------------------------------------- allocation-free step
// The workspace of mlra_decode_step_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends. Host code
// never uses the array's name as an address: the device address of each GPU's
// copy is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept here.
constexpr size_t kScratchBytes = MLRA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch copy.
int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLRA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLRA_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLRA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MLRA_OK;
}

// Element type of queries, weights and append inputs (bf16 for FP8 caches).
int arrays_dtype(const mlra_desc* d) { return fp8_mode(d) ? MLRA_BF16 : d->dtype; }

}  // namespace
}  // namespace mlra

using namespace mlra;

extern "C" {

int mlra_abi_version(void) { return 9; }

const char* mlra_status_string(int status) {
  switch (status) {
    case MLRA_OK: return "ok";
    case MLRA_ERR_INVALID_ARG: return "invalid argument";
    case MLRA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLRA_ERR_WORKSPACE: return "workspace too small";
    case MLRA_ERR_HIP: return "HIP runtime error";
    case MLRA_ERR_SCRATCH: return "shape needs more workspace than the static scratch (MLRA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t mlra_workspace_bytes(const mlra_desc* desc, int32_t max_seq_len) {
  Plan p;
  if (make_plan(desc, &p) != MLRA_OK) return 0;
  if (max_seq_len < 0 || static_cast<int64_t>(max_seq_len) >
                             static_cast<int64_t>(desc->max_pages_per_seq) * desc->page_size)
    return 0;
  return p.total;
}

int mlra_absorb_query(const mlra_desc* desc, const int32_t* seq_lens, const void* q_c,
                      const void* q_r, const void* w_uk, void* workspace, size_t ws_bytes,
                      void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!seq_lens || !q_c || !w_uk || !workspace || (desc->d_r > 0 && !q_r)) return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  DecodeArgs a = decode_args(desc, p, nullptr, nullptr, workspace);
  return hip_status(launch_absorb(a, arrays_dtype(desc), p.q_bf16, seq_lens, q_c, q_r, w_uk,
                                  static_cast<hipStream_t>(stream)));
}

int mlra_attend(const mlra_desc* desc, const void* pool, const int32_t* page_table, void* workspace,
                size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!pool || !workspace) return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  DecodeArgs a = decode_args(desc, p, pool, page_table, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.variant) return hip_status(launch_attend_mfma(p.variant, a, s));
  return hip_status(launch_attend_generic(a, desc->dtype, s));
}

int mlra_attend_timed(const mlra_desc* desc, const void* pool, const int32_t* page_table, void* workspace,
                      size_t ws_bytes, void* start_event, void* stop_event, void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!pool || !workspace || !start_event || !stop_event) return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  DecodeArgs a = decode_args(desc, p, pool, page_table, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = static_cast<hipEvent_t>(start_event), t1 = static_cast<hipEvent_t>(stop_event);
  if (p.variant) return hip_status(launch_attend_mfma(p.variant, a, s, t0, t1));
  return hip_status(launch_attend_generic(a, desc->dtype, s, t0, t1));
}

int mlra_decode(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                const void* w_uk, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!pool || !seq_lens || !q_c || !w_uk || !workspace || (desc->d_r > 0 && !q_r))
    return MLRA_ERR_INVALID_ARG;
  if (max_seq_len < 0 || static_cast<int64_t>(max_seq_len) >
                             static_cast<int64_t>(desc->max_pages_per_seq) * desc->page_size)
    return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  st = mlra_absorb_query(desc, seq_lens, q_c, q_r, w_uk, workspace, ws_bytes, stream);
  if (st != MLRA_OK) return st;
  return mlra_attend(desc, pool, page_table, workspace, ws_bytes, stream);
}

int mlra_combine(const mlra_desc* desc, const void* workspace, size_t ws_bytes, const void* w_uv,
                 float* out, float* lse, void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!workspace || !w_uv || !out) return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  const CombineArgs c = combine_args(desc, p, workspace, w_uv, out, lse);
  return hip_status(launch_combine(c, arrays_dtype(desc), static_cast<hipStream_t>(stream)));
}

int mlra_decode_step(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                     const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                     const void* w_uk, const void* w_uv, float* out, float* lse, void* workspace,
                     size_t ws_bytes, void* stream) {
  Plan p;
  int st = make_plan(desc, &p);
  if (st != MLRA_OK) return st;
  if (!pool || !seq_lens || !q_c || !w_uk || !w_uv || !out || !workspace || (desc->d_r > 0 && !q_r))
    return MLRA_ERR_INVALID_ARG;
  if (max_seq_len < 0 || static_cast<int64_t>(max_seq_len) >
                             static_cast<int64_t>(desc->max_pages_per_seq) * desc->page_size)
    return MLRA_ERR_INVALID_ARG;
  if (ws_bytes < p.total) return MLRA_ERR_WORKSPACE;
  const CombineArgs c = combine_args(desc, p, workspace, w_uv, out, lse);
  st = mlra_decode(desc, pool, page_table, seq_lens, max_seq_len, q_c, q_r, w_uk, workspace, ws_bytes, stream);
  if (st != MLRA_OK) return st;
  return hip_status(launch_combine(c, arrays_dtype(desc), static_cast<hipStream_t>(stream)));
}

int mlra_decode_step_noalloc(const mlra_desc* desc, const void* pool, const int32_t* page_table,
                             const int32_t* seq_lens, int32_t max_seq_len, const void* q_c, const void* q_r,
                             const void* w_uk, const void* w_uv, float* out, float* lse, void* stream) {
  const size_t need = mlra_workspace_bytes(desc, max_seq_len);
  if (need == 0) return MLRA_ERR_INVALID_ARG;
  if (!pool || !seq_lens || !q_c || !w_uk || !w_uv || !out || (desc->d_r > 0 && !q_r)) return MLRA_ERR_INVALID_ARG;
  if (need > kScratchBytes) return MLRA_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st != MLRA_OK) return st;
  // nothing in the workspace has to start at zero: each step writes its plan
  // and header before anything reads them
  return mlra_decode_step(desc, pool, page_table, seq_lens, max_seq_len, q_c, q_r, w_uk, w_uv, out, lse, ws,
                          kScratchBytes, stream);
}

int mlra_append_latent(const mlra_desc* desc, void* pool, const int32_t* page_table,
                       const int32_t* positions, const void* x, const void* w_dkv,
                       const void* kr_new, void* c_out, void* workspace, size_t ws_bytes, void* stream) {
  ShapeInfo s;
  int st = check_desc(desc, &s);
  if (st != MLRA_OK) return st;
  st = check_append(desc);
  if (st != MLRA_OK) return st;
  if (!pool || !positions || !x || !w_dkv || (desc->d_r > 0 && !kr_new)) return MLRA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(w_dkv) % 16 != 0) return MLRA_ERR_INVALID_ARG;  // 16-byte row loads
  st = append_latent_mfma(desc, pool, page_table, positions, x, w_dkv, kr_new, c_out, workspace, ws_bytes, stream);
  if (st != kNotEligible) return st;
  if (!workspace) return MLRA_ERR_INVALID_ARG;  // the same contract on every path
  if (fp8_mode(desc) == 2) return MLRA_ERR_UNSUPPORTED;  // block scales: the MFMA product only
  AppendArgs a;
  memset(&a, 0, sizeof(a));
  a.pool = pool;
  a.page_table = page_table;
  a.positions = positions;
  a.x = x;
  a.w_dkv = w_dkv;
  a.kr_new = kr_new;
  a.c_out = c_out;
  a.batch = desc->batch;
  a.d_c = desc->d_c;
  a.d_r = desc->d_r;
  a.d_model = desc->d_model;
  a.row = fp8_mode(desc) ? fp8_row_bytes(desc) : desc->d_c + desc->d_r;
  a.page_size = desc->page_size;
  a.max_pages = desc->max_pages_per_seq;
  a.num_pages = desc->num_pages;
  a.cache_inv = 1.0f / cache_scale_of(desc);
  return hip_status(launch_append(a, desc->dtype, static_cast<hipStream_t>(stream)));
}

int mlra_read_flags(const void* workspace, size_t ws_bytes, uint32_t* flags, void* stream) {
  if (!workspace || !flags || ws_bytes < sizeof(WsHeader)) return MLRA_ERR_INVALID_ARG;
  const WsHeader* h = static_cast<const WsHeader*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(flags, &h->flags, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MLRA_ERR_HIP;
  return hip_status(hipStreamSynchronize(s));
}

}  // extern "C"
