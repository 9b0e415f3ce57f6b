// Route-word packer and decoder.
//
// One 64-bit word per (KV head, sequence, query-tile row); bit j covers key
// tiles [j*g, j*g+g), least significant bit first, 1 = INT8 path.  With key
// prefix sums (chunked prefill) a sequence's Lq queries are its last Lq of Lk
// positions, and row m's legal key tiles run to last_key_tile(m, Lq, Lk).
// Decoding is the constant-time shift-and-mask R = (w >> floor(n/g)) & 1.  (paperlayer.ai
// summary of arXiv 2608.17336, "TileMix: Tile-Centric Mixed-Precision Attention
// for LLM Inference Acceleration", §3 Preliminaries, §4 and App. D; gist.science
// technical summary, compact-bitmask routing.)
//
// The packer takes per-tile decisions; a group's bit is the AND of its legal
// tiles (FP16 wins on disagreement) and bits of groups without a legal tile are
// 0, so equal decisions give equal words.  Both kernels are tiny (one wave per
// word, one thread per tile) and run once per routing template.
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {

// Sequence b's query and key counts (keys = queries unless cu_k is given).
TM_DEV void seq_lengths(const RouteArgs& a, int b, int& Lq, int& Lk) {
  Lq = a.cu[b + 1] - a.cu[b];
  Lk = a.cu_k ? a.cu_k[b + 1] - a.cu_k[b] : Lq;
}

// One wavefront per word: lane j reduces group j (key tiles j*g .. j*g+g-1 up to
// the row's last legal tile; at most 64 groups per word) and a ballot packs the
// 64 group bits.
__global__ __launch_bounds__(256) void build_route_kernel(RouteArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // word [hk][b][m]
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T;
  if (idx >= total) return;
  const int m = (int)(idx % a.T);
  const int b = (int)((idx / a.T) % a.batch);
  int Lq, Lk;
  seq_lengths(a, b, Lq, Lk);
  const int Tb = (Lq + kTile - 1) / kTile;
  bool bit = false;
  if (m < Tb) {
    const uint8_t* row = a.tile_route + idx * a.Tk;  // [hk][b][m][:]
    const int n0 = lane * a.g;
    // (clamped to the row: lengths beyond max_seqlen_k must not read past it)
    const int n1 = min(n0 + a.g, min(last_key_tile(m, Lq, Lk) + 1, a.Tk));
    if (n0 < n1) {                                   // the group has a legal tile: AND over them
      bool all = true;
      for (int n = n0; n < n1; ++n) all = all && (row[n] != 0);
      bit = all;
    }
  }
  const uint64_t w = __ballot(bit);
  if (lane == 0) a.words_out[idx] = w;
}

__global__ __launch_bounds__(256) void decode_route_kernel(RouteArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T * a.Tk;
  if (idx >= total) return;
  const int n = (int)(idx % a.Tk);
  const int64_t wi = idx / a.Tk;                 // [hk][b][m]
  const int m = (int)(wi % a.T);
  const int b = (int)((wi / a.T) % a.batch);
  int Lq, Lk;
  seq_lengths(a, b, Lq, Lk);
  const int Tb = (Lq + kTile - 1) / kTile;
  uint8_t out = 0xFF;
  if (m < Tb && n <= last_key_tile(m, Lq, Lk)) out = (uint8_t)((a.words_in[wi] >> (n / a.g)) & 1ull);
  a.tile_route_out[idx] = out;
}

hipError_t launch_build_route(const RouteArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T;
  const unsigned blocks = (unsigned)((total + 3) / 4);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(build_route_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_route(const RouteArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T * a.Tk;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_route_kernel, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tilemix
