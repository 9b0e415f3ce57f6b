// C ABI of libtilemix.so: host-side argument validation, workspace layout and
// launches on the caller's stream.  Validation is plain C++ and runs before any
// HIP call, so every error path can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "internal.hpp"
#include "tilemix.h"

namespace tilemix {
namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t ok() {
  g_last_error.clear();
  return TILEMIX_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TILEMIX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxTokens = (int64_t)1 << 31;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t check_common(int32_t batch, int32_t max_seqlen, const int32_t* cu) {
  if (!cu) return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (batch < 1 || batch > (1 << 22)) return fail(TILEMIX_ERR_INVALID_ARG, "batch %d out of range [1, 2^22]", batch);
  if (max_seqlen < 1) return fail(TILEMIX_ERR_INVALID_ARG, "max_seqlen %d must be >= 1", max_seqlen);
  return TILEMIX_OK;
}

// Route groups of one row: the key tiles of max_seqlen_k (chunked) or of max_seqlen.
int32_t check_groups(int32_t max_seqlen_keys, int32_t g) {
  if (g < 1) return fail(TILEMIX_ERR_INVALID_ARG, "g = %d must be >= 1", g);
  const int64_t T = cdiv(max_seqlen_keys, kTile);
  if (cdiv(T, g) > 64)
    return fail(TILEMIX_ERR_TOO_MANY_GROUPS, "ceil(T/g) = %lld groups (T = %lld, g = %d) exceed one 64-bit word",
                (long long)cdiv(T, g), (long long)T, g);
  return TILEMIX_OK;
}

// Query heads per work item.  fp16 K/V: up to 3.  INT8 KV cache: 3 when the
// GQA ratio is a multiple of 3 or above 4 (the 3-head kernel stages tiles
// through LDS, a serialized widening step per tile, but each K/V tile then
// serves more heads: 7 heads as 3 + 3 + 1 run 11 % faster than as
// 2 + 2 + 2 + 1, 8 as 3 + 3 + 2 5 % faster than 2 + 2 + 2 + 2, 5 as 3 + 2 4 %),
// else 2 (tiles staged in registers).  A partial last chunk runs the kernel
// body for its own head count.
int32_t max_heads_per_chunk(const tilemix_attn_params* p) {
  if (!p->kv_int8) return 3;
  const int32_t G = p->num_kv_heads > 0 ? p->num_q_heads / p->num_kv_heads : 1;
  return G % 3 == 0 || G > 4 ? 3 : 2;
}

int32_t validate_attn_params(const tilemix_attn_params* p) {
  if (!p) return fail(TILEMIX_ERR_INVALID_ARG, "params is NULL");
  if (p->batch < 1 || p->batch > (1 << 22)) return fail(TILEMIX_ERR_INVALID_ARG, "batch %d out of range", p->batch);
  if (p->max_seqlen < 1) return fail(TILEMIX_ERR_INVALID_ARG, "max_seqlen %d must be >= 1", p->max_seqlen);
  if (p->num_kv_heads < 1 || p->num_kv_heads > 256)
    return fail(TILEMIX_ERR_INVALID_ARG, "num_kv_heads %d out of range [1, 256]", p->num_kv_heads);
  if (p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(TILEMIX_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads > 4096) return fail(TILEMIX_ERR_INVALID_ARG, "num_q_heads %d > 4096", p->num_q_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(TILEMIX_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  if (p->blk_q != 64 && p->blk_q != 128)
    return fail(TILEMIX_ERR_UNSUPPORTED, "blk_q %d not supported (64 or 128)", p->blk_q);
  if (p->causal != 1) return fail(TILEMIX_ERR_UNSUPPORTED, "causal = %d: only causal prefill is implemented", p->causal);
  if (p->kv_int8 != 0 && p->kv_int8 != 1) return fail(TILEMIX_ERR_INVALID_ARG, "kv_int8 must be 0 or 1");
  if (p->out_fp32 != 0 && p->out_fp32 != 1) return fail(TILEMIX_ERR_INVALID_ARG, "out_fp32 must be 0 or 1");
  if (p->otf_quant < 0 || p->otf_quant > 2) return fail(TILEMIX_ERR_INVALID_ARG, "otf_quant must be 0, 1 or 2");
  if (p->otf_quant && p->kv_int8)
    return fail(TILEMIX_ERR_UNSUPPORTED, "otf_quant = %d cannot be combined with kv_int8 = 1", p->otf_quant);
  if (p->max_seqlen_k < 0) return fail(TILEMIX_ERR_INVALID_ARG, "max_seqlen_k %d must be >= 0", p->max_seqlen_k);
  if (p->max_seqlen_k > 0 && p->max_seqlen_k < p->max_seqlen)
    return fail(TILEMIX_ERR_INVALID_ARG, "max_seqlen_k %d < max_seqlen %d: a chunk has no more queries than keys",
                p->max_seqlen_k, p->max_seqlen);
  if (!(p->sm_scale > 0.0f) || !std::isfinite(p->sm_scale))
    return fail(TILEMIX_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  int32_t st = check_groups(p->max_seqlen_k > 0 ? p->max_seqlen_k : p->max_seqlen, p->g);
  if (st != TILEMIX_OK) return st;
  // one workgroup per work item: the grid (256 threads each) must stay below 2^32 threads
  const int64_t items = (int64_t)p->batch * cdiv(p->max_seqlen, kTile) * p->num_kv_heads *
                        cdiv(p->num_q_heads / p->num_kv_heads, max_heads_per_chunk(p));
  if (items > (int64_t)1 << 24)
    return fail(TILEMIX_ERR_UNSUPPORTED, "%lld work items exceed one launch (2^24); split the batch",
                (long long)items);
  return TILEMIX_OK;
}

struct Derived {
  int32_t T, Tk, G, nch, hc, nbq;   // T query tiles, Tk key tiles
  WorkspaceLayout ws;
};

Derived derive(const tilemix_attn_params* p) {
  Derived d;
  d.T = (int32_t)cdiv(p->max_seqlen, kTile);
  d.Tk = (int32_t)cdiv(p->max_seqlen_k > 0 ? p->max_seqlen_k : p->max_seqlen, kTile);
  d.G = p->num_q_heads / p->num_kv_heads;
  d.nch = (int32_t)cdiv(d.G, max_heads_per_chunk(p));
  d.hc = (int32_t)cdiv(d.G, d.nch);       // heads per chunk (balanced)
  d.nbq = (int32_t)cdiv(p->max_seqlen, p->blk_q);
  d.ws = workspace_layout(p->batch, d.T, p->num_kv_heads, d.nch);
  return d;
}

int32_t validate_tensors(const tilemix_attn_params* p, const tilemix_attn_tensors* t) {
  if (!t) return fail(TILEMIX_ERR_INVALID_ARG, "tensors is NULL");
  if (!t->q || !t->k || !t->v) return fail(TILEMIX_ERR_INVALID_ARG, "q, k and v must be non-NULL");
  const bool otf = p->otf_quant == 1;              // Q and K made on chip
  const bool qotf = p->otf_quant != 0;             // Q made on chip
  if (!qotf && (!t->q_q || !t->q_scale)) return fail(TILEMIX_ERR_INVALID_ARG, "q_q and q_scale must be non-NULL");
  if (!otf && !t->k_scale) return fail(TILEMIX_ERR_INVALID_ARG, "k_scale must be non-NULL");
  if (!otf && !p->kv_int8 && !t->k_q)
    return fail(TILEMIX_ERR_INVALID_ARG, "k_q must be non-NULL when kv_int8 = 0");
  if (p->kv_int8 && !t->v_scale) return fail(TILEMIX_ERR_INVALID_ARG, "v_scale must be non-NULL when kv_int8 = 1");
  if (!t->cu_seqlens || !t->route_words || !t->out)
    return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens, route_words and out must be non-NULL");
  if ((p->max_seqlen_k > 0) != (t->cu_seqlens_k != nullptr))
    return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens_k must be given exactly when max_seqlen_k > 0 (chunked prefill)");
  if ((t->cu_seqlens_k && !aligned(t->cu_seqlens_k, 4)) || (t->lse && !aligned(t->lse, 4)))
    return fail(TILEMIX_ERR_INVALID_ARG, "misaligned cu_seqlens_k or lse pointer");
  if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(t->v, 16) || (!qotf && !aligned(t->q_q, 16)) ||
      (!otf && t->k_q && !aligned(t->k_q, 16)) || !aligned(t->out, 16))
    return fail(TILEMIX_ERR_INVALID_ARG, "q, k, v, q_q, k_q and out must be 16-byte aligned");
  if (!aligned(t->route_words, 8) || (!qotf && !aligned(t->q_scale, 4)) || (!otf && !aligned(t->k_scale, 4)) ||
      !aligned(t->cu_seqlens, 4) || (t->v_scale && !aligned(t->v_scale, 4)))
    return fail(TILEMIX_ERR_INVALID_ARG, "misaligned scale, cu_seqlens or route_words pointer");
  const int64_t kv_mult = p->kv_int8 ? 16 : 8;
  if (t->q_stride_tok % 8 || t->q_stride_head % 8 || t->q_stride_tok <= 0 || t->q_stride_head <= 0)
    return fail(TILEMIX_ERR_INVALID_ARG, "q strides must be positive multiples of 8 elements");
  if (t->kv_stride_tok % kv_mult || t->kv_stride_head % kv_mult || t->kv_stride_tok <= 0 || t->kv_stride_head <= 0)
    return fail(TILEMIX_ERR_INVALID_ARG, "k/v strides must be positive multiples of %lld elements", (long long)kv_mult);
  if (t->q_stride_head < p->head_dim && t->q_stride_tok < p->head_dim)
    return fail(TILEMIX_ERR_INVALID_ARG, "q strides overlap the channel dimension");
  // a K/V tile (64 rows at the token stride) is read through one buffer
  // descriptor whose byte range is 32-bit
  const int64_t tile_span = t->kv_stride_tok * (p->kv_int8 ? 1 : 2) * kTile;
  if (tile_span >= ((int64_t)1 << 32))
    return fail(TILEMIX_ERR_UNSUPPORTED, "k/v token stride of %lld elements: 64 rows span %lld bytes, 4 GiB or more",
                (long long)t->kv_stride_tok, (long long)tile_span);
  return TILEMIX_OK;
}

enum class Mode { kPlanAndRun, kPlanOnly, kRunOnly };

// Calls the decode kernel takes (see launch_attn): it needs no work list.
bool decode_call(const tilemix_attn_params* p, const int32_t* cu_k, bool debug) {
  return cu_k && p->max_seqlen == 1 && p->num_q_heads / p->num_kv_heads <= 16 && !p->otf_quant && !debug;
}

int32_t attn_common(const tilemix_attn_params* p, const tilemix_attn_tensors* t, const int32_t* cu_seqlens,
                    const int32_t* cu_seqlens_k, void* workspace, size_t workspace_bytes, const tilemix_debug* dbg,
                    hipStream_t stream, Mode mode) {
  int32_t st = validate_attn_params(p);
  if (st != TILEMIX_OK) return st;
  if (mode != Mode::kPlanOnly) {
    st = validate_tensors(p, t);
    if (st != TILEMIX_OK) return st;
    cu_seqlens = t->cu_seqlens;
    cu_seqlens_k = t->cu_seqlens_k;
  } else {
    if (!cu_seqlens || !aligned(cu_seqlens, 4))
      return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens must be a non-NULL, 4-byte aligned device pointer");
    if ((p->max_seqlen_k > 0) != (cu_seqlens_k != nullptr) || (cu_seqlens_k && !aligned(cu_seqlens_k, 4)))
      return fail(TILEMIX_ERR_INVALID_ARG,
                  "cu_seqlens_k must be a 4-byte aligned device pointer exactly when max_seqlen_k > 0");
  }
  const Derived d = derive(p);
  if (!workspace || workspace_bytes < d.ws.total)
    return fail(TILEMIX_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", d.ws.total, workspace_bytes,
                workspace ? "" : " (NULL)");
  if (!aligned(workspace, 256)) return fail(TILEMIX_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (dbg) {
    if (dbg->s32_tiles && (dbg->seq < 0 || dbg->seq >= p->batch || dbg->q_head < 0 ||
                           dbg->q_head >= p->num_q_heads || dbg->m_begin < 0 || dbg->m_end <= dbg->m_begin ||
                           dbg->m_end > d.T))
      return fail(TILEMIX_ERR_INVALID_ARG, "debug window (seq %d, head %d, m %d..%d) out of range", dbg->seq,
                  dbg->q_head, dbg->m_begin, dbg->m_end);
    if ((dbg->s32_tiles && !aligned(dbg->s32_tiles, 16)) || (dbg->visit_count && !aligned(dbg->visit_count, 4)))
      return fail(TILEMIX_ERR_INVALID_ARG, "misaligned debug buffer");
  }

  char* ws = static_cast<char*>(workspace);
  SchedArgs sa;
  sa.cu = cu_seqlens;
  sa.cu_k = cu_seqlens_k;
  sa.batch = p->batch;
  sa.T = d.T;
  sa.Hk = p->num_kv_heads;
  sa.nch = d.nch;
  {
    // upper bound of the summed cost of all groups: every sequence at T query
    // tiles, each also behind up to Tk key tiles of earlier keys (chunked)
    const uint64_t rows = (uint64_t)p->batch * p->num_kv_heads * d.nch * (uint64_t)d.T;
    const uint64_t total = rows * (d.T + 1) / 2 + (p->max_seqlen_k > 0 ? rows * (uint64_t)d.Tk : 0);
    int shift = 0;
    while ((total >> shift) >= ((uint64_t)1 << 28)) ++shift;
    sa.cost_shift = shift;
  }
  sa.nslots = d.ws.nslots;
  sa.segmax = d.ws.segmax;
  sa.items = reinterpret_cast<WorkItem*>(ws + d.ws.items_off);
  sa.seg = reinterpret_cast<int32_t*>(ws + d.ws.seg_off);
  sa.segidx = reinterpret_cast<int32_t*>(ws + d.ws.segidx_off);
  sa.order = reinterpret_cast<int32_t*>(ws + d.ws.order_off);
  hipError_t e = hipSuccess;
  if (mode == Mode::kPlanOnly || (mode == Mode::kPlanAndRun && !decode_call(p, cu_seqlens_k, dbg != nullptr))) {
    e = launch_schedule(sa, stream);
    if (e != hipSuccess) return hip_status(e, "work-list launch");
    if (mode == Mode::kPlanOnly) return ok();
  }

  AttnArgs a{};
  a.q = t->q;
  a.k = t->k;
  a.v = t->v;
  a.q_st = t->q_stride_tok;
  a.q_sh = t->q_stride_head;
  a.kv_st = t->kv_stride_tok;
  a.kv_sh = t->kv_stride_head;
  a.q_q = t->q_q;
  a.q_scale = t->q_scale;
  a.k_q = t->k_q;
  a.k_scale = t->k_scale;
  a.v_scale = t->v_scale;
  a.cu = t->cu_seqlens;
  a.cu_k = t->cu_seqlens_k;
  a.words = t->route_words;
  a.out = t->out;
  a.lse = t->lse;
  a.items = sa.items;
  a.batch = p->batch;
  a.max_seqlen = p->max_seqlen;
  a.Hq = p->num_q_heads;
  a.Hk = p->num_kv_heads;
  a.D = p->head_dim;
  a.g = p->g;
  a.blk_q = p->blk_q;
  a.T = d.T;
  a.Tk = d.Tk;
  a.G = d.G;
  a.nch = d.nch;
  a.hc = d.hc;
  a.nbq = d.nbq;
  a.sm_log2 = (float)((double)p->sm_scale * 1.4426950408889634);
  a.out_fp32 = p->out_fp32;
  a.kv_int8 = p->kv_int8;
  a.otf = p->otf_quant;
  if (a.otf) {   // not read in these modes
    a.q_q = nullptr;
    a.q_scale = nullptr;
  }
  if (a.otf == 1) {
    a.k_q = nullptr;
    a.k_scale = nullptr;
  }
  a.dbg_seq = -1;
  if (dbg) {
    const int64_t tiles = (int64_t)p->batch * p->num_q_heads * d.T * d.Tk;
    if (dbg->visit_count) {
      e = launch_fill_u32(dbg->visit_count, 0u, tiles, stream);
      if (e != hipSuccess) return hip_status(e, "debug fill");
    }
    if (dbg->route_used) {
      e = launch_fill_u8(dbg->route_used, 0xFF, tiles, stream);
      if (e != hipSuccess) return hip_status(e, "debug fill");
    }
    if (dbg->s32_tiles) {
      e = launch_fill_u32(reinterpret_cast<uint32_t*>(dbg->s32_tiles), 0x80000000u,
                          (int64_t)(dbg->m_end - dbg->m_begin) * d.Tk * kTile * kTile, stream);
      if (e != hipSuccess) return hip_status(e, "debug fill");
    }
    a.dbg_seq = dbg->s32_tiles ? dbg->seq : -1;
    a.dbg_head = dbg->q_head;
    a.dbg_m0 = dbg->m_begin;
    a.dbg_m1 = dbg->m_end;
    a.dbg_s32 = dbg->s32_tiles;
    a.dbg_visits = dbg->visit_count;
    a.dbg_route = dbg->route_used;
  }
  e = launch_attn(a, d.ws.nslots, dbg != nullptr, stream);
  return hip_status(e, "attention launch");
}

}  // namespace

int32_t validate_attn_call(const tilemix_attn_params* p, const tilemix_attn_tensors* t) {
  int32_t st = validate_attn_params(p);
  if (st != TILEMIX_OK) return st;
  return validate_tensors(p, t);
}

int32_t set_last_error(int32_t status, const char* text) {
  g_last_error = text;
  return status;
}

WorkspaceLayout workspace_layout(int32_t batch, int32_t T, int32_t Hk, int32_t nch) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  WorkspaceLayout w;
  const int64_t items = (int64_t)batch * T * Hk * nch;
  w.nslots = ((items + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (w.nslots == 0) w.nslots = kNumXcd;
  w.segmax = (int64_t)batch * Hk + 2 * kNumXcd;
  size_t off = 0;
  w.items_off = off;
  off = up(off + (size_t)w.nslots * sizeof(WorkItem));
  w.seg_off = off;
  off = up(off + (size_t)w.segmax * 6 * sizeof(int32_t));
  w.segidx_off = off;
  off = up(off + (kNumXcd + 1) * sizeof(int32_t));
  w.order_off = off;
  off = up(off + (size_t)batch * 2 * sizeof(int32_t));
  w.total = off;
  return w;
}

hipError_t launch_attn_d64_kv0(const AttnArgs&, int64_t, bool, hipStream_t);
hipError_t launch_attn_d64_kv1(const AttnArgs&, int64_t, bool, hipStream_t);
hipError_t launch_attn_d128_kv0(const AttnArgs&, int64_t, bool, hipStream_t);
hipError_t launch_attn_d128_kv1(const AttnArgs&, int64_t, bool, hipStream_t);
hipError_t launch_attn_d64_otf(const AttnArgs&, int64_t, bool, hipStream_t);
hipError_t launch_attn_d128_otf(const AttnArgs&, int64_t, bool, hipStream_t);

hipError_t launch_attn_decode(const AttnArgs&, hipStream_t);

// Decode (chunked with one query per sequence: max_seqlen = 1) with the query
// heads of a KV head fitting one 16-row MFMA block goes to the decode kernel
// (heads as rows, waves splitting the keys); everything else, and the debug
// products, to the fused prefill kernel.
bool decode_shape(const AttnArgs& a, bool debug) {
  return a.cu_k && a.max_seqlen == 1 && a.G <= 16 && !a.otf && !debug;
}

hipError_t launch_attn(const AttnArgs& a, int64_t nslots, bool debug, hipStream_t s) {
  if (decode_shape(a, debug)) return launch_attn_decode(a, s);
  if (a.D == 64) {
    if (a.kv_int8) return launch_attn_d64_kv1(a, nslots, debug, s);
    return a.otf ? launch_attn_d64_otf(a, nslots, debug, s) : launch_attn_d64_kv0(a, nslots, debug, s);
  }
  if (a.kv_int8) return launch_attn_d128_kv1(a, nslots, debug, s);
  return a.otf ? launch_attn_d128_otf(a, nslots, debug, s) : launch_attn_d128_kv0(a, nslots, debug, s);
}

}  // namespace tilemix

using namespace tilemix;

extern "C" {

const char* tilemix_status_string(int32_t s) {
  switch (s) {
    case TILEMIX_OK: return "TILEMIX_OK";
    case TILEMIX_ERR_INVALID_ARG: return "TILEMIX_ERR_INVALID_ARG";
    case TILEMIX_ERR_UNSUPPORTED: return "TILEMIX_ERR_UNSUPPORTED";
    case TILEMIX_ERR_TOO_MANY_GROUPS: return "TILEMIX_ERR_TOO_MANY_GROUPS";
    case TILEMIX_ERR_WORKSPACE: return "TILEMIX_ERR_WORKSPACE";
    case TILEMIX_ERR_HIP: return "TILEMIX_ERR_HIP";
    default: return "TILEMIX_UNKNOWN_STATUS";
  }
}

const char* tilemix_last_error(void) { return g_last_error.c_str(); }

const char* tilemix_version(void) { return "tilemix-gfx950 0.1"; }

int32_t tilemix_quantize_blockwise(const void* x, int64_t stride_tok, int64_t stride_head, const int32_t* cu_seqlens,
                                   int32_t batch, int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                                   int32_t blk, int8_t* x_q, float* scales, void* stream) {
  int32_t st = check_common(batch, max_seqlen, cu_seqlens);
  if (st != TILEMIX_OK) return st;
  if (!x || !x_q || !scales) return fail(TILEMIX_ERR_INVALID_ARG, "x, x_q and scales must be non-NULL");
  if (num_heads < 1 || num_heads > 65535 * 4) return fail(TILEMIX_ERR_INVALID_ARG, "num_heads %d out of range", num_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(TILEMIX_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (blk != 64 && blk != 128) return fail(TILEMIX_ERR_UNSUPPORTED, "blk %d not supported (64 or 128)", blk);
  if (!aligned(x, 16) || !aligned(x_q, 8) || !aligned(scales, 4))
    return fail(TILEMIX_ERR_INVALID_ARG, "x must be 16-byte, x_q 8-byte and scales 4-byte aligned");
  if (stride_tok <= 0 || stride_head <= 0 || stride_tok % 8 || stride_head % 8)
    return fail(TILEMIX_ERR_INVALID_ARG, "strides must be positive multiples of 8 elements");
  if (cdiv(max_seqlen, blk) * batch > 0x7fffffffLL)
    return fail(TILEMIX_ERR_INVALID_ARG, "too many blocks for one launch");
  QuantArgs a{x, stride_tok, stride_head, cu_seqlens, batch, max_seqlen, num_heads, head_dim, blk, x_q, scales};
  return hip_status(launch_quantize(a, static_cast<hipStream_t>(stream)), "quantize launch");
}

static int32_t check_route_args(int32_t batch, int32_t max_seqlen, const int32_t* cu, const int32_t* cu_k,
                         int32_t max_seqlen_k, int32_t num_kv_heads, int32_t g) {
  int32_t st = check_common(batch, max_seqlen, cu);
  if (st != TILEMIX_OK) return st;
  if (num_kv_heads < 1) return fail(TILEMIX_ERR_INVALID_ARG, "num_kv_heads %d must be >= 1", num_kv_heads);
  if ((cu_k != nullptr) != (max_seqlen_k > 0))
    return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens_k must be given exactly when max_seqlen_k > 0 (chunked prefill)");
  if (max_seqlen_k < 0 || (max_seqlen_k > 0 && max_seqlen_k < max_seqlen))
    return fail(TILEMIX_ERR_INVALID_ARG, "max_seqlen_k %d must be 0 or >= max_seqlen %d", max_seqlen_k, max_seqlen);
  if (cu_k && !aligned(cu_k, 4)) return fail(TILEMIX_ERR_INVALID_ARG, "cu_seqlens_k must be 4-byte aligned");
  return check_groups(max_seqlen_k > 0 ? max_seqlen_k : max_seqlen, g);
}

int32_t tilemix_build_route_mask(const uint8_t* tile_route, const int32_t* cu_seqlens, const int32_t* cu_seqlens_k,
                                 int32_t batch, int32_t max_seqlen, int32_t max_seqlen_k, int32_t num_kv_heads,
                                 int32_t g, uint64_t* route_words, void* stream) {
  if (!tile_route || !route_words) return fail(TILEMIX_ERR_INVALID_ARG, "tile_route and route_words must be non-NULL");
  if (!aligned(route_words, 8)) return fail(TILEMIX_ERR_INVALID_ARG, "route_words must be 8-byte aligned");
  int32_t st = check_route_args(batch, max_seqlen, cu_seqlens, cu_seqlens_k, max_seqlen_k, num_kv_heads, g);
  if (st != TILEMIX_OK) return st;
  RouteArgs a{};
  a.tile_route = tile_route;
  a.words_out = route_words;
  a.cu = cu_seqlens;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.T = (int32_t)cdiv(max_seqlen, kTile);
  a.Tk = (int32_t)cdiv(max_seqlen_k > 0 ? max_seqlen_k : max_seqlen, kTile);
  a.num_kv_heads = num_kv_heads;
  a.g = g;
  return hip_status(launch_build_route(a, static_cast<hipStream_t>(stream)), "route-mask launch");
}

int32_t tilemix_decode_route_mask(const uint64_t* route_words, const int32_t* cu_seqlens,
                                  const int32_t* cu_seqlens_k, int32_t batch, int32_t max_seqlen,
                                  int32_t max_seqlen_k, int32_t num_kv_heads, int32_t g, uint8_t* tile_route_out,
                                  void* stream) {
  if (!route_words || !tile_route_out)
    return fail(TILEMIX_ERR_INVALID_ARG, "route_words and tile_route_out must be non-NULL");
  if (!aligned(route_words, 8)) return fail(TILEMIX_ERR_INVALID_ARG, "route_words must be 8-byte aligned");
  int32_t st = check_route_args(batch, max_seqlen, cu_seqlens, cu_seqlens_k, max_seqlen_k, num_kv_heads, g);
  if (st != TILEMIX_OK) return st;
  RouteArgs a{};
  a.words_in = route_words;
  a.tile_route_out = tile_route_out;
  a.cu = cu_seqlens;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.T = (int32_t)cdiv(max_seqlen, kTile);
  a.Tk = (int32_t)cdiv(max_seqlen_k > 0 ? max_seqlen_k : max_seqlen, kTile);
  a.num_kv_heads = num_kv_heads;
  a.g = g;
  return hip_status(launch_decode_route(a, static_cast<hipStream_t>(stream)), "route-decode launch");
}

int32_t tilemix_template_route_words(int32_t template_kind, int32_t int8_permille, uint64_t seed,
                                     const int32_t* cu_seqlens, const int32_t* cu_seqlens_k, int32_t batch,
                                     int32_t max_seqlen, int32_t max_seqlen_k, int32_t num_kv_heads,
                                     int32_t g, uint64_t* route_words, void* stream) {
  if (template_kind < TILEMIX_TEMPLATE_ALL_FP16 || template_kind > TILEMIX_TEMPLATE_SPTRANS)
    return fail(TILEMIX_ERR_INVALID_ARG, "template kind %d unknown", template_kind);
  if (int8_permille < 0 || int8_permille > 1000)
    return fail(TILEMIX_ERR_INVALID_ARG, "int8_permille %d out of [0, 1000]", int8_permille);
  if (!route_words) return fail(TILEMIX_ERR_INVALID_ARG, "route_words must be non-NULL");
  if (!aligned(route_words, 8)) return fail(TILEMIX_ERR_INVALID_ARG, "route_words must be 8-byte aligned");
  int32_t st = check_route_args(batch, max_seqlen, cu_seqlens, cu_seqlens_k, max_seqlen_k, num_kv_heads, g);
  if (st != TILEMIX_OK) return st;
  RouteArgs a{};
  a.words_out = route_words;
  a.cu = cu_seqlens;
  a.cu_k = cu_seqlens_k;
  a.batch = batch;
  a.T = (int32_t)cdiv(max_seqlen, kTile);
  a.Tk = (int32_t)cdiv(max_seqlen_k > 0 ? max_seqlen_k : max_seqlen, kTile);
  a.num_kv_heads = num_kv_heads;
  a.g = g;
  return hip_status(launch_template_route(a, template_kind, int8_permille, seed, static_cast<hipStream_t>(stream)),
                    "template launch");
}

int32_t tilemix_attn_workspace_size(const tilemix_attn_params* params, size_t* bytes) {
  if (!bytes) return fail(TILEMIX_ERR_INVALID_ARG, "bytes is NULL");
  int32_t st = validate_attn_params(params);
  if (st != TILEMIX_OK) return st;
  *bytes = derive(params).ws.total;
  return ok();
}

int32_t tilemix_attn_prefill(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return attn_common(params, tensors, nullptr, nullptr, workspace, workspace_bytes, nullptr,
                     static_cast<hipStream_t>(stream), Mode::kPlanAndRun);
}

int32_t tilemix_attn_plan(const tilemix_attn_params* params, const int32_t* cu_seqlens, const int32_t* cu_seqlens_k,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return attn_common(params, nullptr, cu_seqlens, cu_seqlens_k, workspace, workspace_bytes, nullptr,
                     static_cast<hipStream_t>(stream), Mode::kPlanOnly);
}

int32_t tilemix_attn_run(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return attn_common(params, tensors, nullptr, nullptr, workspace, workspace_bytes, nullptr,
                     static_cast<hipStream_t>(stream), Mode::kRunOnly);
}

int32_t tilemix_attn_prefill_debug(const tilemix_attn_params* params, const tilemix_attn_tensors* tensors,
                                   void* workspace, size_t workspace_bytes, const tilemix_debug* dbg, void* stream) {
  if (!dbg) return fail(TILEMIX_ERR_INVALID_ARG, "dbg is NULL");
  return attn_common(params, tensors, nullptr, nullptr, workspace, workspace_bytes, dbg,
                     static_cast<hipStream_t>(stream), Mode::kPlanAndRun);
}

}  // extern "C"
