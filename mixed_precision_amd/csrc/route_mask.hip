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

// ---- static routing templates (All-FP16, All-INT8, Band, Global, Row-Random,
// Aligned-Sparse, BigBird, SpTrans; paperlayer.ai summary, App. B; gist.science
// summary).  The pages name the layouts and their INT8 coverage of legal tile
// groups but print no definitions; per query-tile row with n legal groups,
// F = round((1 - p) n) groups (p in per mille, integer arithmetic) are FP16:
//   band: the F groups nearest the diagonal; global: the first F;
//   row_random: the F smallest SplitMix64 keys (Steele, Lea and Flood, 2014) of
//     seed ^ (((hk B + b) Tq + m) 64 + j), ties by j;
//   aligned_sparse: F evenly spaced groups floor(k n / F);
//   bigbird: ceil(F/3) band groups, ceil((F - that)/2) first groups, then
//     random (key order) among the rest up to F;
//   sptrans: ceil(F/2) band groups, the rest evenly spaced before the band.
// One wave per word: lane j decides group j.
TM_DEV uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// does group j (< n) hold one of the positions floor(i n / k), i = 0 .. k-1?
TM_DEV bool evenly_spaced_hit(int j, int n, int k) {
  if (k <= 0) return false;
  const int imin = (j * k + n - 1) / n;   // ceil(j k / n)
  return imin < k && imin * n < (j + 1) * k;
}

// rank of (key, j) among the lanes i < n with cand_i set, by (key_i, i)
TM_DEV int key_rank(uint64_t key, int j, int n, bool cand_j, uint64_t cand_mask) {
  int rank = 0;
  for (int i = 0; i < n; ++i) {
    if (!((cand_mask >> i) & 1ull)) continue;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key, i);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), i);
    const uint64_t ki = ((uint64_t)hi << 32) | lo;
    rank += (ki < key) || (ki == key && i < j);
  }
  return cand_j ? rank : 64;
}

__global__ __launch_bounds__(256) void template_route_kernel(RouteArgs a, int32_t kind, int32_t permille,
                                                             uint64_t seed) {
  const int64_t idx = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // word [hk][b][m]
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T;
  if (idx >= total) return;
  const int m = (int)(idx % a.T);
  const int b = (int)((idx / a.T) % a.batch);
  const int hk = (int)(idx / ((int64_t)a.T * a.batch));
  int Lq, Lk;
  seq_lengths(a, b, Lq, Lk);
  const int Tb = (Lq + kTile - 1) / kTile;
  // legal groups of this row (0 past the sequence end), clamped to the row's tiles
  const int n = m < Tb ? min(last_key_tile(m, Lq, Lk), a.Tk - 1) / a.g + 1 : 0;
  const int j = lane;
  const bool legal = j < n;
  const int F = ((1000 - permille) * n + 500) / 1000;
  const uint64_t key = splitmix64(seed ^ ((((uint64_t)hk * a.batch + b) * a.T + m) * 64 + j));
  bool fp16 = false;
  switch (kind) {
    case TILEMIX_TEMPLATE_ALL_FP16: fp16 = true; break;
    case TILEMIX_TEMPLATE_ALL_INT8: fp16 = false; break;
    case TILEMIX_TEMPLATE_BAND: fp16 = j >= n - F; break;
    case TILEMIX_TEMPLATE_GLOBAL: fp16 = j < F; break;
    case TILEMIX_TEMPLATE_ROW_RANDOM: {
      const uint64_t cand = __ballot(legal);
      fp16 = key_rank(key, j, n, legal, cand) < F;
      break;
    }
    case TILEMIX_TEMPLATE_ALIGNED_SPARSE: fp16 = evenly_spaced_hit(j, n, F); break;
    case TILEMIX_TEMPLATE_BIGBIRD: {
      const int w = (F + 2) / 3;
      const bool fixed = legal && (j >= n - w || j < (F - w + 1) / 2);
      const uint64_t fixed_mask = __ballot(fixed);
      const int left = F - (int)__builtin_popcountll(fixed_mask);
      const bool cand = legal && !fixed;
      fp16 = fixed || key_rank(key, j, n, cand, __ballot(cand)) < left;
      break;
    }
    case TILEMIX_TEMPLATE_SPTRANS: {
      const int w = (F + 1) / 2;
      fp16 = j >= n - w || (j < n - w && evenly_spaced_hit(j, n - w, F - w));
      break;
    }
    default: break;
  }
  const uint64_t word = __ballot(legal && !fp16);
  if (lane == 0) a.words_out[idx] = word;
}

hipError_t launch_template_route(const RouteArgs& a, int32_t kind, int32_t permille, uint64_t seed,
                                 hipStream_t s) {
  const int64_t total = (int64_t)a.num_kv_heads * a.batch * a.T;
  const unsigned blocks = (unsigned)((total + 3) / 4);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(template_route_kernel, dim3(blocks), dim3(256), 0, s, a, kind, permille, seed);
  return hipGetLastError();
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
