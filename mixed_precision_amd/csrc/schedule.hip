// Varlen / GQA work scheduler for the fused attention kernel.
//
// The fused kernel runs one workgroup per work item = (sequence b, KV head hk,
// query-tile row m, chunk of the query heads that share hk).  Sequences are
// unpadded, described only by cu_seqlens prefix sums (paperlayer.ai summary of
// arXiv 2608.17336, "TileMix: Tile-Centric Mixed-Precision Attention for LLM
// Inference Acceleration", §4: GQA heads share routing decisions, prefix-sum
// metadata gives padding-free execution).
//
// MI355X deals workgroups to its 8 XCDs round-robin (workgroup i -> XCD i % 8)
// and each XCD has its own L2.  The plan therefore gives every (b, hk) group of
// items to one XCD where possible, so the K/V of a group is fetched from HBM
// once into that XCD's L2 and reused by all of its query-tile rows:
//   * groups are placed greedily, most expensive first (cost = sum over rows of
//     the legal key tiles, T_b (T_b + 1) / 2 per head chunk, plus T_b times the
//     whole key tiles before the first query in chunked prefill), on the XCD with
//     the least accumulated cost that still has free slots; a group that fits
//     nowhere whole is split over the XCDs with the most free slots;
//   * inside an XCD's list, groups follow each other and a group's items are in
//     decreasing m (longest causal rows first), so the short rows fill the tail.
// Slot i of the grid then takes entry i / 8 of XCD (i % 8)'s list.
//
// plan: one workgroup.  Tile counts and the rank sort live in LDS (global
//   scratch past kPlanLdsBatch sequences); the greedy placement runs in wave 0
//   with one XCD per lane and writes each segment to the segment table without
//   reading it back, then the segment count and per-XCD fill levels.  A
//   sequence's KV-head groups are identical jobs; up to eight of them are
//   placed in one step where that gives the same result as one at a time.
// emit: one workgroup per segment writes that segment's items; 8 more
//   workgroups mark each XCD's unused slots empty (b = -1).
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {

namespace {
constexpr int kSegFields = 6;
// min / max over each group of 8 lanes (all 8 end with the result)
TM_DEV uint32_t min8(uint32_t k) {
  k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  k = min(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x141, 0xF, 0xF, false));   // row_half_mirror
  return k;
}
TM_DEV uint32_t max8(uint32_t k) {
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x4E, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x141, 0xF, 0xF, false));
  return k;
}           // xcd, slot_begin, count, item_begin, b, hk
constexpr int kPlanLdsBatch = 4096;     // sequences whose tile counts / order fit in LDS
}  // namespace

template <bool kLds>
__global__ __launch_bounds__(256) void schedule_plan_kernel(SchedArgs a) {
  __shared__ int32_t s_tiles[kLds ? kPlanLdsBatch : 1];
  __shared__ int32_t s_order[kLds ? kPlanLdsBatch : 1];
  int32_t* tiles = kLds ? s_tiles : a.order + a.batch;
  int32_t* order = kLds ? s_order : a.order;

  for (int b = threadIdx.x; b < a.batch; b += 256) tiles[b] = (a.cu[b + 1] - a.cu[b] + kTile - 1) / kTile;
  __syncthreads();
  // 1) sequences ordered by decreasing tile count (ties by index): rank sort.
  for (int b = threadIdx.x; b < a.batch; b += 256) {
    const int tb = tiles[b];
    int rank = 0;
    for (int o = 0; o < a.batch; ++o) {
      const int to = tiles[o];
      rank += (to > tb) || (to == tb && o < b);
    }
    order[rank] = b;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;

  // 2) greedy placement of (b, hk) groups on XCDs, by wave 0: lane x < 8
  //    holds XCD x's used slots and load; the least-loaded XCD with room is a
  //    min over 8 lanes of (load << 3 | x) (DPP quad swaps and a half-row
  //    mirror), so each placement is a few instructions with no memory trip.
  //    Costs are shifted right by cost_shift so loads stay below 2^28.
  const int lane = threadIdx.x;
  const uint32_t cap = (uint32_t)(a.nslots / kNumXcd);
  uint32_t used = 0, load = 0;
  uint32_t nseg = 0;
  const uint32_t segmax = (uint32_t)a.segmax;
  for (int r = 0; r < a.batch; ++r) {
    const int b = uniform(order[r]);
    const uint32_t tb = (uint32_t)uniform(tiles[b]);
    if (tb == 0) break;                           // sorted: the rest are empty too
    const uint32_t cnt = tb * (uint32_t)a.nch;
    uint64_t tiles_b = (uint64_t)tb * (tb + 1) / 2;
    if (a.cu_k) {                                 // chunked: queries start (Lk - Lq) keys in
      const int lead = (uniform(a.cu_k[b + 1]) - uniform(a.cu_k[b])) - (uniform(a.cu[b + 1]) - uniform(a.cu[b]));
      tiles_b += (uint64_t)tb * (uint32_t)max(lead, 0) / kTile;
    }
    const uint32_t cost = (uint32_t)(((uint64_t)a.nch * tiles_b) >> a.cost_shift);
    for (int hk = 0; hk < a.Hk;) {
      // The sequence's Hk groups are identical jobs.  When every XCD has room
      // for a whole group and one group's cost moves the least-loaded XCD's key
      // past the k-th smallest key, placing k groups one by one gives group
      // hk + i to the XCD of rank i: all k are placed at once.
      {
        const int k = min(a.Hk - hk, kNumXcd);
        const uint32_t key = lane < kNumXcd ? (load << 3) | (uint32_t)lane : 0xFFFFFFFFu;
        uint32_t rank = 0, kmin = 0xFFFFFFFFu;
#pragma unroll
        for (int y = 0; y < kNumXcd; ++y) {
          const uint32_t ky = (uint32_t)__builtin_amdgcn_readlane((int)key, y);
          rank += ky < key;
          kmin = min(kmin, ky);
        }
        const bool room = lane >= kNumXcd || cap - used >= cnt;
        const uint64_t kth = __ballot(lane < kNumXcd && rank == (uint32_t)(k - 1));
        const uint32_t keyk = (uint32_t)__builtin_amdgcn_readlane((int)key, (int)__builtin_ctzll(kth));
        if (k > 1 && __all(room) && (uint64_t)kmin + ((uint64_t)cost << 3) > keyk &&
            nseg + (uint32_t)k <= segmax) {
          if (lane < kNumXcd && rank < (uint32_t)k) {
            int32_t* sg = a.seg + (int64_t)(nseg + rank) * kSegFields;
            sg[0] = lane;
            sg[1] = (int32_t)used;
            sg[2] = (int32_t)cnt;
            sg[3] = 0;
            sg[4] = b;
            sg[5] = hk + (int)rank;
            used += cnt;
            load += cost;
          }
          nseg += (uint32_t)k;
          hk += k;
          continue;
        }
      }
      uint32_t remaining = cnt, ib = 0;
      while (remaining > 0 && nseg < segmax) {
        const bool fits = lane < kNumXcd && cap - used >= remaining;
        const uint32_t kmin = uniform(min8(fits ? (load << 3) | (uint32_t)lane : 0xFFFFFFFFu));
        int best;
        uint32_t take;
        if (kmin != 0xFFFFFFFFu) {
          best = (int)(kmin & 7u);
          take = remaining;
        } else {                                  // split: XCD with the most free slots (lowest index on ties)
          const uint32_t kmax =
              uniform(max8(lane < kNumXcd ? ((cap - used) << 3) | (uint32_t)(7 - lane) : 0u));
          best = 7 - (int)(kmax & 7u);
          take = kmax >> 3;
          if (take == 0) break;                   // cannot happen: slots >= items
        }
        const uint32_t slot_begin = (uint32_t)__builtin_amdgcn_readlane((int)used, best);
        if (lane == 0) {
          int32_t* sg = a.seg + (int64_t)nseg * kSegFields;
          sg[0] = best;
          sg[1] = (int32_t)slot_begin;
          sg[2] = (int32_t)take;
          sg[3] = (int32_t)ib;
          sg[4] = b;
          sg[5] = hk;
        }
        const uint32_t add = (take == cnt) ? cost : (uint32_t)((uint64_t)cost * take / cnt);
        if (lane == best) {
          used += take;
          load += add;
        }
        ++nseg;
        ib += take;
        remaining -= take;
      }
      ++hk;
    }
  }
  if (lane == 0) a.segidx[0] = (int32_t)nseg;
  if (lane < kNumXcd) a.segidx[1 + lane] = (int32_t)used;
}

__global__ __launch_bounds__(256) void schedule_emit_kernel(SchedArgs a) {
  const int64_t w = blockIdx.x;
  const int64_t cap = a.nslots / kNumXcd;
  if (w >= a.segmax) {                              // empty tail of XCD x
    const int x = (int)(w - a.segmax);
    const int64_t used = uniform(a.segidx[1 + x]);
    for (int64_t pos = used + threadIdx.x; pos < cap; pos += 256)
      a.items[pos * kNumXcd + x] = WorkItem{-1, 0, 0, 0};
    return;
  }
  if (w >= uniform(a.segidx[0])) return;
  const int32_t* sg = a.seg + w * kSegFields;
  const int x = uniform(sg[0]);
  const int64_t slot_begin = uniform(sg[1]);
  const int count = uniform(sg[2]);
  const int item_begin = uniform(sg[3]);
  const int b = uniform(sg[4]);
  const int hk = uniform(sg[5]);
  const int tb = (uniform(a.cu[b + 1]) - uniform(a.cu[b]) + kTile - 1) / kTile;
  for (int i = threadIdx.x; i < count; i += 256) {
    const int t = item_begin + i;                   // item index inside the group: m descending, chunks inner
    a.items[(slot_begin + i) * kNumXcd + x] = WorkItem{b, hk, tb - 1 - t / a.nch, t % a.nch};
  }
}

hipError_t launch_schedule(const SchedArgs& a, hipStream_t s) {
  if (a.batch <= kPlanLdsBatch)
    hipLaunchKernelGGL(schedule_plan_kernel<true>, dim3(1), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(schedule_plan_kernel<false>, dim3(1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(schedule_emit_kernel, dim3((unsigned)(a.segmax + kNumXcd)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Small fills used by the debug entry point (kernels rather than memsets so the
// call sequence stays capturable in a HIP graph).
__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}
__global__ __launch_bounds__(256) void fill_u8_kernel(uint8_t* p, uint8_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

static unsigned fill_blocks(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(fill_blocks(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t launch_fill_u8(uint8_t* p, uint8_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u8_kernel, dim3(fill_blocks(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace tilemix
