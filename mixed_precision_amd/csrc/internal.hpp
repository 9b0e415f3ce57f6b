// Internal interfaces between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tilemix.h"

namespace tilemix {

constexpr int kTile = 64;    // score tile edge (BLOCK_M = BLOCK_N)
constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin

struct QuantArgs {
  const void* x;
  int64_t stride_tok, stride_head;
  const int32_t* cu;
  int32_t batch, max_seqlen, num_heads, head_dim, blk;
  int8_t* xq;
  float* scales;
};

struct RouteArgs {
  const uint8_t* tile_route;
  const uint64_t* words_in;
  uint64_t* words_out;
  uint8_t* tile_route_out;
  const int32_t* cu;
  const int32_t* cu_k;   // key prefix sums (chunked prefill), or nullptr: keys = queries
  int32_t batch, T, Tk, num_kv_heads, g;   // T query tiles, Tk key tiles
};

// Last key tile that query tile m reaches when the Lq queries are the last Lq of
// Lk positions (bottom-right causal alignment; prefill has Lq = Lk and gives m).
__host__ __device__ inline int last_key_tile(int m, int Lq, int Lk) {
  const int q = m * kTile + kTile - 1 < Lq - 1 ? m * kTile + kTile - 1 : Lq - 1;
  const int r = (Lk - Lq) + q;
  return r < 0 ? 0 : r / kTile;
}

// Work item of the fused kernel: one query-tile row m of one sequence b for one
// chunk of the query heads that share KV head hk.  b < 0 marks an empty slot.
struct WorkItem {
  int32_t b, hk, m, chunk;
};

// Placement of the work list in the caller's workspace.
struct WorkspaceLayout {
  int64_t nslots;     // grid size of the fused kernel (multiple of 8)
  int64_t segmax;     // capacity of the segment table
  size_t items_off, seg_off, segidx_off, order_off, total;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_st, q_sh, kv_st, kv_sh;
  const int8_t* q_q;
  const float* q_scale;
  const int8_t* k_q;
  const float* k_scale;
  const float* v_scale;
  const int32_t* cu;
  const int32_t* cu_k;   // key prefix sums (chunked prefill), or nullptr: keys = queries
  const uint64_t* words;
  void* out;
  float* lse;            // optional [N][Hq] log-sum-exp of each query row's scores
  const WorkItem* items;
  int32_t batch, max_seqlen, Hq, Hk, D, g, blk_q, T, G, nch, hc, nbq;
  int32_t Tk;            // key tiles (T in prefill)
  float sm_log2;     // fl32(sm_scale * log2(e))
  int32_t out_fp32;
  int32_t kv_int8;
  int32_t otf;       // 1: Q and K quantised inside the kernel (q_q, q_scale, k_q, k_scale unused);
                     // 2: Q alone (q_q, q_scale unused)
  // debug products (fused kernel with DBG = true only)
  int32_t dbg_seq, dbg_head, dbg_m0, dbg_m1;
  int32_t* dbg_s32;
  uint32_t* dbg_visits;
  uint8_t* dbg_route;
};

struct SchedArgs {
  const int32_t* cu;
  const int32_t* cu_k;  // key prefix sums (chunked prefill), or nullptr
  int32_t batch, T, Hk, nch;
  int32_t cost_shift;   // group costs >> cost_shift keep every XCD load below 2^28
  int64_t nslots, segmax;
  WorkItem* items;
  int32_t* seg;      // int32 [segmax][6]: xcd, slot_begin, count, item_begin, b, hk
  int32_t* segidx;   // int32 [1 + kNumXcd]: segment count, then slots used per XCD
  int32_t* order;    // int32 [2 * batch]: sequences by decreasing tile count, then tile counts
                     // (used only when batch exceeds what the plan kernel keeps in LDS)
};

WorkspaceLayout workspace_layout(int32_t batch, int32_t T, int32_t Hk, int32_t nch);

// Host-side validation of an attention call's params and tensors (no HIP call).
int32_t validate_attn_call(const tilemix_attn_params* p, const tilemix_attn_tensors* t);
// Sets the calling thread's tilemix_last_error() text; returns status.
int32_t set_last_error(int32_t status, const char* text);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);
hipError_t launch_build_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_decode_route(const RouteArgs& a, hipStream_t s);
hipError_t launch_template_route(const RouteArgs& a, int32_t kind, int32_t permille, uint64_t seed, hipStream_t s);
hipError_t launch_schedule(const SchedArgs& a, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, uint32_t value, int64_t count, hipStream_t s);
hipError_t launch_fill_u8(uint8_t* p, uint8_t value, int64_t count, hipStream_t s);
hipError_t launch_attn(const AttnArgs& a, int64_t nslots, bool debug, hipStream_t s);

}  // namespace tilemix
