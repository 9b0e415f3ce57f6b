// Decode over a KV cache (one query per sequence and head) for gfx950.
//
// Same method as the fused prefill kernel (paperlayer.ai summary of arXiv
// 2608.17336, "TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
// Acceleration", §3 Preliminaries, §4, App. C): key tile n of the row takes the
// FP16 or the INT8 score path by bit (w >> floor(n/g)) & 1 of the row's route
// word, both feed one online softmax, P.V in fp16.  The pages evaluate prefill
// only; decode is the single-query case of bottom-right causal alignment (the
// query sits at position Lk - 1 and sees every key).
//
// Layout for one query per head: a workgroup owns one (sequence, KV head); the
// G query heads that share the KV head are the rows of one 16-row MFMA block
// (GQA: they share K/V and the route word), and the four waves split every
// 64-key tile into 16-key slices.  Per wave and tile: S^T = K Q^T for its 16
// keys (v_mfma_f32_16x16x32_f16, or v_mfma_i32_16x16x64_i8), a 4-score online
// softmax per lane, and O^T += V^T P^T on v_mfma_f32_16x16x16_f16, whose B
// operand is exactly the lane's 4 probabilities.  K/V tiles stream through the
// prefill kernel's double-buffered LDS stages; at the end the four waves' softmax
// states (m, l, acc) are merged through LDS exactly as tiles merge.
#pragma once
#include "attn_kernel.hpp"

namespace tilemix {

template <int D, bool KVI8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_decode_kernel(const AttnArgs a) {
  using A = Attn<D, 1, KVI8>;
  constexpr int NDS = A::NDS, NDS8 = A::NDS8, NDB = A::NDB;
  constexpr float kSlack = A::kSlack;
  __shared__ __attribute__((aligned(1024))) char stA[A::KBYTES + A::VBYTES];
  __shared__ __attribute__((aligned(1024))) char stB[A::KBYTES + A::VBYTES];

  // Workgroups are dealt round-robin to the 8 XCDs.  Each XCD takes a
  // contiguous range of the (sequence, KV head) pairs, ordered as the cache is
  // (a sequence's heads together for a token-major cache, a head's sequences
  // together for a head-major one), so that its L2 and address translation
  // cover one compact slice of the cache.
  int b, hk;
  {
    const int total = (int)gridDim.x, x = (int)(blockIdx.x & 7), slot = (int)(blockIdx.x >> 3);
    const int q = total >> 3, r = total & 7;
    const int w = x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    if (a.kv_sh > a.kv_st) {
      hk = w / a.batch;
      b = w - hk * a.batch;
    } else {
      b = w / a.Hk;
      hk = w - b * a.Hk;
    }
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);   // 16-key slice of every tile
  const int c = lane & 15;              // query row = query head hk*G + c
  const int gq = lane >> 4;
  const int seq0 = uniform(a.cu[b]);
  const int Lq = uniform(a.cu[b + 1]) - seq0;
  const int kseq0 = uniform(a.cu_k[b]);
  const int Lk = uniform(a.cu_k[b + 1]) - kseq0;
  if (Lq != 1 || Lk < 1) return;        // (the host sends only decode calls here)
  const int n_last = (Lk - 1) / kTile;
  const bool row_ok = c < a.G;
  const int head = hk * a.G + c;
  const int64_t tok = seq0;

  // ---- Q operands of the row's head, its block scale times sm_scale log2(e)
  f16x8 qf[1][NDS];
  i32x4 q8[1][NDS8];
  const f16* qptr = static_cast<const f16*>(a.q);
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds)
    qf[0][ds] = row_ok ? *reinterpret_cast<const f16x8*>(qptr + tok * a.q_st + (int64_t)head * a.q_sh + ds * 32 + gq * 8)
                       : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int ds = 0; ds < NDS8; ++ds)
    q8[0][ds] = row_ok ? *reinterpret_cast<const i32x4*>(a.q_q + (tok * a.Hq + head) * D + ds * 64 + gq * 16)
                       : i32x4{0, 0, 0, 0};
  const float sqs = (row_ok ? a.q_scale[((int64_t)head * a.batch + b) * a.nbq] : 1.0f) * a.sm_log2;

  // ---- K/V sources (rows >= Lk read as zero), scales, route word
  const int64_t esz = KVI8 ? 1 : 2;
  const char* kbase = static_cast<const char*>(a.k) + ((int64_t)kseq0 * a.kv_st + (int64_t)hk * a.kv_sh) * esz;
  const char* vbase = static_cast<const char*>(a.v) + ((int64_t)kseq0 * a.kv_st + (int64_t)hk * a.kv_sh) * esz;
  const uint32_t kv_stride = (uint32_t)(a.kv_st * esz);
  const uint32_t k8_stride = KVI8 ? kv_stride : (uint32_t)(a.Hk * D);
  const char* k8base = KVI8 ? kbase : reinterpret_cast<const char*>(a.k_q + ((int64_t)kseq0 * a.Hk + hk) * D);
  auto tile_rsrc = [&](const char* base, uint32_t stride, int n, bool empty) __attribute__((always_inline)) {
    // (min after a readfirstlane: as one min/max pair the clamp becomes a VALU
    // med3, and the descriptor built from it a waterfall loop per load)
    const int rows = empty ? 0 : min(__builtin_amdgcn_readfirstlane(max(Lk - n * kTile, 0)), kTile);
    return make_rsrc(base + (int64_t)n * kTile * stride, (uint32_t)rows * stride);
  };
  typename A::Dma dma;
  if (!KVI8) A::dma_offsets(dma, wave, lane, kv_stride, k8_stride);
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* kscale_row = (cfloat*)(a.k_scale + ((int64_t)hk * a.batch + b) * a.Tk);
  cfloat* vscale_row = KVI8 ? (cfloat*)(a.v_scale + ((int64_t)hk * a.batch + b) * a.Tk) : nullptr;
  uint64_t wsh = uniform64(a.words[((int64_t)hk * a.batch + b) * a.T]);
  int left = a.g;
  auto fetch = [&](int n, int route, typename A::Stage& st, char* sg, bool empty) __attribute__((always_inline)) {
    if (KVI8) {
      A::stage_load(st, tid, tile_rsrc(kbase, kv_stride, n, empty), tile_rsrc(vbase, kv_stride, n, empty),
                    kv_stride);
    } else {
      A::dma_tile(route, wave, dma, kv_stride, k8_stride, tile_rsrc(kbase, kv_stride, n, empty),
                  tile_rsrc(k8base, k8_stride, n, empty), tile_rsrc(vbase, kv_stride, n, empty), sg,
                  sg + A::KBYTES);
    }
  };

  // ---- per-wave online-softmax state (log2 units), O^T block of 16 channels x 16 rows per db
  f32x4 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x4{0, 0, 0, 0};
  float mref = -INFINITY, lsum = 0.0f;

  {
    typename A::Stage st;
    fetch(0, (int)(wsh & 1), st, stA, false);
    if (KVI8) {
      const typename A::VSplit v0 = A::vsplit(vscale_row[0]);
      wait_vmem();
      A::stage_store(st, (int)(wsh & 1), tid, stA, stA + A::KBYTES, v0.s2, v0.b2);
    }
  }
  wait_vmem();
  __syncthreads();

  auto tile = [&](int n, const char* cur, char* next) __attribute__((always_inline)) {
    const int rc = (int)(wsh & 1);
    const int rnext = (left == 1) ? (int)((wsh >> 1) & 1) : rc;
    const bool last = (n == n_last);
    typename A::Stage st;
    fetch(n + 1, rnext, st, next, last);
    const float ksc = kscale_row[n];
    // INT8 V: the tile's scale split as in the prefill kernel (the power of two
    // widened into V, the mantissa into P, the row sum from the same fp16 P)
    float lmv = 0.0f, rmv = 1.0f;
    if (KVI8) {
      const typename A::VSplit vs = A::vsplit(vscale_row[n]);
      lmv = vs.lmv;
      rmv = vs.rmv;
    }
    // S^T for keys 64n + 16 wave + 4 gq + i of row c (raw: float bits or int32)
    i32x4 S;
    if (rc == 0) {
      f32x4 acc = {0, 0, 0, 0};
      const char* base = cur + A::L16::lane(c) + gq * 16 + wave * A::L16::step16;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const f16x8*>(base + ds * 64), qf[0][ds], acc,
                                                     0, 0, 0);
      S = __builtin_bit_cast(i32x4, acc);
    } else {
      i32x4 acc = {0, 0, 0, 0};
      const char* base = cur + A::L8::lane(c) + gq * 16 + wave * A::L8::step16;
#pragma unroll
      for (int ds = 0; ds < NDS8; ++ds)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const i32x4*>(base + ds * 64), q8[0][ds], acc,
                                                    0, 0, 0);
      S = __builtin_bit_cast(i32x4, __builtin_convertvector(acc, f32x4));
    }
    // score factor (> 0, so a zero scale cannot turn a masked -inf into NaN)
    const float cj = __builtin_elementwise_maximum(rc ? sqs * ksc : (KVI8 ? ksc * a.sm_log2 : a.sm_log2),
                                                   1.17549435e-38f);
    f32x4 x = __builtin_bit_cast(f32x4, S);
    if (last) {   // keys at or past Lk (the query sits at Lk - 1)
      const int key0 = n * kTile + wave * 16 + gq * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + i > Lk - 1) x[i] = -INFINITY;
    }
    const float lm = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]),
                                                   __builtin_elementwise_maximum(x[2], x[3]));
    if (__any(lm * cj > mref + kSlack)) {
      const float tmax = rows4_max(lm) * cj;
      const bool moved = tmax > mref + kSlack;
      const float alpha = moved ? __builtin_amdgcn_exp2f(mref - tmax) : 1.0f;
      mref = moved ? tmax : mref;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[db] *= alpha;
    }
    f16x4 P;
    {
      // a wave whose keys so far are all masked (short caches) still has
      // m = -inf: its masked scores must give p = 0, not exp2(-inf + inf)
      const float mm = (mref == -INFINITY) ? 0.0f : mref;
      const float add = lmv - mm;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[0], cj, add));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[1], cj, add));
      const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2], cj, add));
      const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[3], cj, add));
      P = f16x4{(f16)p0, (f16)p1, (f16)p2, (f16)p3};
      // the wave's 16-key slice sum of P for the lane's query (all-ones A
      // operand), divided by the INT8 V mantissa
      const f16x4 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
      const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x16f16(ones, P, f32x4{0, 0, 0, 0}, 0, 0, 0);
      lsum = __builtin_fmaf(t[0], rmv, lsum);
    }
    // O^T += V^T P^T: lane (c, gq) reads channel db*16 + c of keys 16 wave + 4 gq .. +3
    const int jl = lane & 15;
    const char* vb = cur + A::KBYTES + A::LV::lane(4 * gq + (jl >> 2)) + 8 * (jl & 3) + wave * A::LV::step16;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      O[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(read_tr16(vb + db * 32), P, O[db], 0, 0, 0);
    if (KVI8) {
      const typename A::VSplit vn = A::vsplit(last ? 1.0f : vscale_row[n + 1]);
      wait_vmem();
      A::stage_store(st, rnext, tid, next, next + A::KBYTES, vn.s2, vn.b2);
    }
    wait_vmem();
    __syncthreads();
    if (--left == 0) {
      left = a.g;
      wsh >>= 1;
    }
  };
#pragma unroll 1
  for (int n = 0;; n += 2) {
    tile(n, stA, stB);
    if (n + 1 > n_last) break;
    tile(n + 1, stB, stA);
    if (n + 2 > n_last) break;
  }

  // ---- merge the four waves' states (the stages are free after the last barrier):
  // per row, M = max m_w, L = sum l_w 2^(m_w - M), acc = sum acc_w 2^(m_w - M)
  float* red = reinterpret_cast<float*>(stA);          // [4][16] m, then [4][16] l
  float* acc = reinterpret_cast<float*>(stB);          // [4][16 rows][D]
  const float lrow = lsum;   // (every lane of the query holds the slice sum)
  if (gq == 0) {
    red[wave * 16 + c] = mref;
    red[64 + wave * 16 + c] = lrow;
  }
  __syncthreads();
  float M = red[c];
#pragma unroll
  for (int w = 1; w < 4; ++w) M = __builtin_elementwise_maximum(M, red[w * 16 + c]);
  const float sc = __builtin_amdgcn_exp2f(mref - M);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[(wave * 16 + c) * D + db * 16 + gq * 4 + i] = O[db][i] * sc;
  __syncthreads();
  // thread t: row t / 16, channels (t % 16) * D/16 ..
  {
    const int r = tid >> 4;
    if (r < a.G) {
      float Mr = red[r];
#pragma unroll
      for (int w = 1; w < 4; ++w) Mr = __builtin_elementwise_maximum(Mr, red[w * 16 + r]);
      float L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) L += red[64 + w * 16 + r] * __builtin_amdgcn_exp2f(red[w * 16 + r] - Mr);
      const float inv = 1.0f / L;
      const int hq = hk * a.G + r;
      const int64_t obase = (tok * a.Hq + hq) * D;
      constexpr int CH = D / 16;
      const int c0 = (tid & 15) * CH;
#pragma unroll
      for (int e = 0; e < CH; ++e) {
        const float o = (acc[(0 * 16 + r) * D + c0 + e] + acc[(1 * 16 + r) * D + c0 + e] +
                         acc[(2 * 16 + r) * D + c0 + e] + acc[(3 * 16 + r) * D + c0 + e]) * inv;
        if (a.out_fp32)
          static_cast<float*>(a.out)[obase + c0 + e] = o;
        else
          static_cast<f16*>(a.out)[obase + c0 + e] = (f16)o;
      }
      if (a.lse && (tid & 15) == 0) a.lse[tok * a.Hq + hq] = (Mr + __builtin_amdgcn_logf(L)) * 0.6931471805599453f;
    }
  }
}

template <int D, bool KVI8>
hipError_t launch_decode_inst(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_kernel<D, KVI8>), dim3((unsigned)((int64_t)a.batch * a.Hk)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tilemix
