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
//     the legal key tiles, T_b (T_b + 1) / 2 per head chunk), on the XCD with
//     the least accumulated cost that still has free slots; a group that fits
//     nowhere whole is split over the XCDs with the most free slots;
//   * inside an XCD's list, groups follow each other and a group's items are in
//     decreasing m (longest causal rows first), so the short rows fill the tail.
// Slot i of the grid then takes entry i / 8 of XCD (i % 8)'s list.
//
// plan: one workgroup (the greedy placement is sequential, O(groups * 8)).
// emit: one thread per slot, binary search of its XCD's segment table.
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {

namespace {
constexpr int kSegFields = 6;   // xcd, slot_begin, count, item_begin, b, hk

__device__ __forceinline__ int tiles_of(const int32_t* cu, int b) {
  return (cu[b + 1] - cu[b] + kTile - 1) / kTile;
}
}  // namespace

__global__ __launch_bounds__(256) void schedule_plan_kernel(SchedArgs a) {
  // 1) sequences ordered by decreasing tile count (ties by index): rank sort.
  for (int b = threadIdx.x; b < a.batch; b += 256) {
    const int tb = tiles_of(a.cu, b);
    int rank = 0;
    for (int o = 0; o < a.batch; ++o) {
      const int to = tiles_of(a.cu, o);
      rank += (to > tb) || (to == tb && o < b);
    }
    a.order[rank] = b;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;

  // 2) greedy placement of (b, hk) groups on XCDs, raw segments in creation order.
  const int64_t cap = a.nslots / kNumXcd;
  int64_t used[kNumXcd];
  int64_t load[kNumXcd];
  for (int x = 0; x < kNumXcd; ++x) used[x] = load[x] = 0;
  int32_t* raw = a.seg;                                   // [segmax][6]
  int32_t* sorted = a.seg + a.segmax * kSegFields;        // [segmax][6]
  int64_t nseg = 0;
  for (int r = 0; r < a.batch; ++r) {
    const int b = a.order[r];
    const int tb = tiles_of(a.cu, b);
    if (tb == 0) continue;
    const int64_t cnt = (int64_t)tb * a.nch;
    const int64_t cost = (int64_t)a.nch * tb * (tb + 1) / 2;
    for (int hk = 0; hk < a.Hk; ++hk) {
      int64_t remaining = cnt, ib = 0;
      while (remaining > 0 && nseg < a.segmax) {
        int best = -1;
        for (int x = 0; x < kNumXcd; ++x)
          if (cap - used[x] >= remaining && (best < 0 || load[x] < load[best])) best = x;
        int64_t take = remaining;
        if (best < 0) {
          best = 0;
          for (int x = 1; x < kNumXcd; ++x)
            if (cap - used[x] > cap - used[best]) best = x;
          take = cap - used[best];
          if (take <= 0) break;      // cannot happen: slots >= items
        }
        int32_t* s = raw + nseg * kSegFields;
        s[0] = best;
        s[1] = (int32_t)used[best];
        s[2] = (int32_t)take;
        s[3] = (int32_t)ib;
        s[4] = b;
        s[5] = hk;
        ++nseg;
        used[best] += take;
        load[best] += cost * take / cnt;
        ib += take;
        remaining -= take;
      }
    }
  }
  // 3) per-XCD segment lists (increasing slot_begin inside each XCD).
  int64_t k = 0;
  for (int x = 0; x < kNumXcd; ++x) {
    a.segidx[x] = (int32_t)k;
    for (int64_t i = 0; i < nseg; ++i) {
      const int32_t* s = raw + i * kSegFields;
      if (s[0] != x) continue;
      int32_t* d = sorted + k * kSegFields;
      for (int f = 0; f < kSegFields; ++f) d[f] = s[f];
      ++k;
    }
  }
  a.segidx[kNumXcd] = (int32_t)k;
}

__global__ __launch_bounds__(256) void schedule_emit_kernel(SchedArgs a) {
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot >= a.nslots) return;
  const int x = (int)(slot % kNumXcd);
  const int64_t pos = slot / kNumXcd;
  const int32_t* sorted = a.seg + a.segmax * kSegFields;
  int lo = a.segidx[x], hi = a.segidx[x + 1] - 1;
  WorkItem it{-1, 0, 0, 0};
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int32_t* s = sorted + (int64_t)mid * kSegFields;
    if (pos < s[1]) {
      hi = mid - 1;
    } else if (pos >= (int64_t)s[1] + s[2]) {
      lo = mid + 1;
    } else {
      const int b = s[4];
      const int tb = tiles_of(a.cu, b);
      const int64_t t = s[3] + (pos - s[1]);
      it.b = b;
      it.hk = s[5];
      it.m = tb - 1 - (int)(t / a.nch);
      it.chunk = (int)(t % a.nch);
      break;
    }
  }
  a.items[slot] = it;
}

hipError_t launch_schedule(const SchedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(schedule_plan_kernel, dim3(1), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((a.nslots + 255) / 256);
  hipLaunchKernelGGL(schedule_emit_kernel, dim3(blocks), dim3(256), 0, s, a);
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
