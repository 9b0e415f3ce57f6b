// Fused causal routed FP16/INT8 prefill attention for gfx950 (MI355X).
//
// Method (paperlayer.ai summary of arXiv 2608.17336, "TileMix: Tile-Centric
// Mixed-Precision Attention for LLM Inference Acceleration": §1, §3
// Preliminaries, §4, App. C; ainews.surl.tw article on TileMix): for each query
// tile the legal key tiles are streamed (chunked prefill: the Lq queries are
// the last Lq of Lk positions, so a query tile's keys start (Lk - Lq) earlier
// and the causal edge may cut two tiles); a bit of the row's packed 64-bit word,
// (w >> floor(n/g)) & 1, sends tile n through an FP16 or an INT8 QK^T (INT32
// accumulation, then the block scales); both update one online-softmax state
// (running max, sum, output accumulator) and P.V runs in FP16.
//
// gfx950 design (the pages' A100/Triton kernel is prior art, not followed):
//  * Workgroup = 4 wavefronts = one work item (sequence b, KV head hk, query
//    tile m, up to 3 of the query heads that share hk); two workgroups share a
//    CU (2 waves per SIMD) so one wave's softmax overlaps the other's MFMAs.
//    All of the item's query heads take the same route bit and read the same
//    K/V tiles, so one LDS copy of each tile feeds 4*nh query blocks of 16
//    rows; wave w owns nh of them (nh = heads in the chunk), which balances
//    GQA ratios such as 3 over the 4 SIMDs.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_f16
//    or v_mfma_i32_16x16x64_i8: A = K rows from LDS, B = Q^T from registers
//    (loaded once per item).  In the 16x16 accumulator layout each lane then
//    holds one query column and a quarter of the keys, so the softmax
//    statistics need one max over 4 lanes, and the exponentials are already
//    laid out as the B operand (P^T) of the P.V MFMA: O^T += V^T P^T.  The A
//    operand V^T comes straight from V's natural [key][d] layout through
//    ds_read_b64_tr_b16 (within each 16-lane group the 16x4 block of b16 the
//    lanes address is handed back transposed).  O^T has one query per lane,
//    so the rescale and the final 1/l are lane-local.
//  * Tiles are processed in 32-key halves (QK, softmax, P.V per half) to keep
//    the live score registers small; the online softmax is exact at any
//    granularity.
//  * The route bit is wave-uniform (SGPR shift and mask), so the FP16/INT8
//    choice is a scalar branch around the QK^T only; one loop body serves every
//    tile (duplicating it per route costs the register allocator dearly).
//  * FP16 K/V tiles move HBM -> LDS with buffer_load ... lds (no staging
//    registers); the next tile's loads are in flight while the current tile
//    computes from the other half of a double-buffered stage.  K is fetched
//    in the form its route needs (fp16 16 KB or int8 8 KB at d = 128).  An
//    INT8 KV cache is widened int8 -> fp16 exactly where the FP16 path or P.V
//    needs it; the next tile waits in registers (up to 2 heads per item) or, as
//    raw int8, in LDS (3 heads per item, whose q-blocks leave no room for the
//    staging registers).  Buffer range checks return zeros past the sequence
//    end, so ragged tails need no branches.
//  * Scores live in the log2 domain: t = raw * c with c = sm_scale*log2(e)
//    (FP16 path) or q_scale*k_scale*sm_scale*log2(e) (INT8 path), so both paths
//    meet in one running max and p = exp2(raw*c - m) is one FMA plus v_exp_f32.
//    The reference max only moves when a half-tile's max exceeds it by more
//    than kSlack, so the accumulator is rescaled on few tiles (per q-block,
//    only where it moved); acc / l is unchanged.  Raw scores are held in
//    integer-typed registers (INT8 results as int32, FP16 results as their
//    float bits) so no float transformation ever touches an int32 bit pattern.
//  * On-the-fly mode (OTF; the pages' second operand preparation, App. C and
//    App. D): no Q8/K8 in HBM.  The Q block scales and INT8 Q fragments are made
//    once per item from fp16 Q; every tile's K arrives as fp16, and only an
//    INT8-routed tile is quantised, cooperatively, into a separate LDS tile.  Each
//    wave reads back the K chunks its own lds-loads brought in and publishes
//    their max |k| before the end-of-tile barrier, so the scale costs no barrier
//    of its own; one LDS-only barrier separates the quantised tile from its use.
//    Scales and int8 values equal those of the quantise-once kernel bit for bit,
//    so both modes give the same output.  The Q-only variant makes Q's operands
//    the same way and takes K quantised once: it saves the step's Q pass (Q is
//    read here anyway) without quantising a K tile once per query tile.
//  * The normaliser l sums the fp16-rounded probabilities that actually enter
//    P.V, on the MFMA (an all-ones A operand times P^T), so O is an exact
//    weighted mean of V rows with slightly perturbed weights and the dominant
//    term's rounding cancels.  With an INT8 V the v scale's power of two is
//    widened into V exactly and its mantissa enters P (see VSplit).
//  * The kernel is bound by the SIMD's VALU issue port, which the MFMAs share
//    (each 16x16x32 f16 MFMA takes about 7 cycles of the other wave's VALU
//    issue); the softmax is written for the fewest VALU instructions per score.
#pragma once
#include "device_common.hpp"
#include "internal.hpp"

namespace tilemix {


typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

TM_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
TM_DEV u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// 16 bytes per lane from global straight into LDS at lds_base + lane*16.
TM_DEV void bload16_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, 0);
}
TM_DEV f16x4 read_tr16(const char* p) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}
TM_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0) only
// Workgroup barrier that waits for this wave's LDS operations only, not for
// its global loads in flight (which __syncthreads would also drain).
TM_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int QB, bool KVI8>
struct Attn {
  // The reference max may lag the true running max by up to kSlack (log2
  // units), so p <= 2^kSlack.  FP16 V: p itself must stay finite in fp16
  // (2^15 < 65504).  INT8 V: P = p mv carries the v scale's mantissa mv
  // (VSplit), below 16.2 for any scale of fp16 data (s_v <= 65504 / 127), so
  // 2^11 keeps P below 2^15.
  static constexpr float kSlack = KVI8 ? 11.0f : 15.0f;
  // When the reference moves, FP16 V sets it kOver above the new maximum, so
  // the row's maximum can grow by kOver + kSlack before the next rescale
  // (fewer O rescales on rows whose maximum keeps rising).  The largest p is
  // then >= 2^-kOver: the terms within 14 - kOver of the maximum keep fp16's
  // full precision, and the smaller ones fall into its subnormal range, whose
  // absolute step is 2^-24.  With near one-hot rows (outlier channels) an
  // overshoot of 8 doubled the worst output error; 4 left it unchanged.
  static constexpr float kOver = 4.0f;
  // Row sums: with three q-blocks over an fp16 cache, one all-ones MFMA per
  // q-block and half accumulates them in a 4-register accumulator (lacc);
  // otherwise each half's sum, from a transient MFMA result, is added to one
  // register per q-block (lrow), 3 fewer registers per q-block.
  static constexpr bool kLacc = !KVI8 && QB == 3;
  static constexpr int NDS = D / 32;       // fp16 MFMA k-steps over d
  static constexpr int NDS8 = D / 64;      // int8 MFMA k-steps over d
  static constexpr int NDB = D / 16;       // 16-row blocks of d in O^T
  static constexpr int RB16 = 2 * D;       // bytes of one fp16 row (K or V)
  static constexpr int RB8 = D;            // bytes of one int8 K row
  // LDS tile layout: a tile's 64 rows are spread over NB = 64 / (1024/RB)
  // blocks of 1 KB (padded to 1040 B); row r sits in block r % NB at slot
  // r / NB.  The 16 consecutive rows one MFMA operand read touches then fall in
  // 16 different 16-byte bank groups, every operand address is a per-lane base
  // plus an immediate, and one lds-load instruction fills one whole block.
  //
  // K blocks are padded to 1040 B: a K operand read (16 rows x 16 B per lane
  // group) then covers all 64 banks once.  V blocks are padded to 1056 B: a
  // ds_read_b64_tr_b16 has each 16-lane group read 4 consecutive keys x 32 B,
  // and the 32-byte skew puts the 8 keys of 32 lanes on 256 distinct bytes.
  template <int RB, int BLK>
  struct Lay {
    static constexpr int NB = 64 / (1024 / RB);
    static constexpr int BLOCK = BLK;
    static TM_DEV int row(int r) { return (r % NB) * BLK + (r / NB) * RB; }
    // row 16*k + c16 (c16 < 16): per-lane part and compile-time part
    static TM_DEV int lane(int c16) { return (c16 % NB) * BLK + (c16 / NB) * RB; }
    static constexpr int step16 = (16 / NB) * RB;
    static constexpr int BYTES = NB * BLK;
  };
  using L16 = Lay<RB16, 1040>;
  using L8 = Lay<RB8, 1040>;
  using LV = Lay<RB16, 1056>;
  static constexpr int KBYTES = L16::BYTES;                // one K stage (int8 K uses half)
  static constexpr int VBYTES = LV::BYTES;                 // one V stage
  static constexpr int LDS_BYTES = 2 * (KBYTES + VBYTES);  // K and V, double-buffered
  static constexpr int NI16 = L16::NB / 4;                 // lds-load instructions per wave, fp16 tile
  static constexpr int NI8 = L8::NB / 4;                   // ... int8 tile

  static TM_DEV int k16_off(int R, int C) { return L16::row(R) + C * 16; }
  static TM_DEV int k8_off(int R, int C) { return L8::row(R) + C * 16; }
  static TM_DEV int v_off(int key, int d) { return LV::row(key) + d * 2; }

  // Per-lane global byte offsets (relative to the tile's first row) of the
  // lds-loads.  Instruction i of wave w fills block w*NI + i, whose lanes
  // hold rows w*NI + i + NB*s (slot s = lane*16 / RB): offset = base + i*stride.
  struct Dma {
    uint32_t b16, b8;
  };
  static TM_DEV void dma_offsets(Dma& o, int wave, int lane, uint32_t k16_stride, uint32_t k8_stride) {
    o.b16 = (uint32_t)(wave * NI16 + L16::NB * ((lane * 16) / RB16)) * k16_stride + ((lane * 16) % RB16);
    o.b8 = (uint32_t)(wave * NI8 + L8::NB * ((lane * 16) / RB8)) * k8_stride + ((lane * 16) % RB8);
  }

  // --- FP16 KV: issue the lds-loads of tile n (K in its route's form, and V).
  // K and V rows share one stride.
  static TM_DEV void dma_tile(int route, int wave, const Dma& o, uint32_t s16, uint32_t s8,
                              __amdgpu_buffer_rsrc_t rk16, __amdgpu_buffer_rsrc_t rk8, __amdgpu_buffer_rsrc_t rv,
                              char* kl, char* vl) {
    if (route == 0) {
#pragma unroll
      for (int i = 0; i < NI16; ++i) bload16_lds(rk16, o.b16 + i * s16, kl + (wave * NI16 + i) * L16::BLOCK);
    } else {
#pragma unroll
      for (int i = 0; i < NI8; ++i) bload16_lds(rk8, o.b8 + i * s8, kl + (wave * NI8 + i) * L8::BLOCK);
    }
#pragma unroll
    for (int i = 0; i < NI16; ++i) bload16_lds(rv, o.b16 + i * s16, vl + (wave * NI16 + i) * LV::BLOCK);
  }

  // --- the same loads, K and V apart (single V stage: V's loads are issued
  // later than K's)
  static TM_DEV void dma_k(int route, int wave, const Dma& o, uint32_t s16, uint32_t s8, __amdgpu_buffer_rsrc_t rk16,
                           __amdgpu_buffer_rsrc_t rk8, char* kl) {
    if (route == 0) {
#pragma unroll
      for (int i = 0; i < NI16; ++i) bload16_lds(rk16, o.b16 + i * s16, kl + (wave * NI16 + i) * L16::BLOCK);
    } else {
#pragma unroll
      for (int i = 0; i < NI8; ++i) bload16_lds(rk8, o.b8 + i * s8, kl + (wave * NI8 + i) * L8::BLOCK);
    }
  }
  static TM_DEV void dma_v(int wave, const Dma& o, uint32_t s16, __amdgpu_buffer_rsrc_t rv, char* vl) {
#pragma unroll
    for (int i = 0; i < NI16; ++i) bload16_lds(rv, o.b16 + i * s16, vl + (wave * NI16 + i) * LV::BLOCK);
  }

  // --- on-the-fly K quantisation.  Load i of wave w fills LDS block
  // w*NI16 + i of the stage's K; its lane l holds channels 8 (l % (RB16/16))
  // .. +7 of row w*NI16 + i + NB (16 l / RB16), at block + 16 l.  A wave can
  // read back the chunks of its own loads as soon as they have landed.
  static constexpr int AMAX_OFF = KBYTES + VBYTES;   // the stage's 4 per-wave maxima
  static TM_DEV void k_partial_amax(char* st, int wave, int lane) {
    u16x2 mx = {0, 0};
#pragma unroll
    for (int i = 0; i < NI16; ++i)
      mx = absmax_acc(mx, *reinterpret_cast<const u32x4*>(st + (wave * NI16 + i) * L16::BLOCK + lane * 16));
    const uint32_t am = wave_max_u32(absmax_bits(mx));
    if (lane == 0) *reinterpret_cast<uint32_t*>(st + AMAX_OFF + wave * 4) = am;
  }
  static TM_DEV float k_tile_scale(const char* st) {
    const u32x4 p = *reinterpret_cast<const u32x4*>(st + AMAX_OFF);
    return block_scale(max(max(p[0], p[1]), max(p[2], p[3])));
  }
  static TM_DEV void quant_k(const char* st, char* k8, float scale, int wave, int lane) {
    const float rs = __fdiv_rn(1.0f, scale);
#pragma unroll
    for (int i = 0; i < NI16; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + (wave * NI16 + i) * L16::BLOCK + lane * 16);
      const int R = wave * NI16 + i + L16::NB * ((lane * 16) / RB16);
      *reinterpret_cast<u32x2*>(k8 + L8::row(R) + ((lane * 16) % RB16) / 2) = quant8(v, scale, rs);
    }
  }

  // --- INT8 KV cache: register staging (16 int8 of one row per thread and load)
  struct Stage {
    u32x4 k[D / 64];   // K: 64 x D bytes = D/64 loads of 16 B per thread
    u32x4 v[D / 64];
  };
  static TM_DEV void stage_load(Stage& r, int tid, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                uint32_t stride) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int id = tid + 256 * i;
      const uint32_t off = (id / (D / 16)) * stride + (id % (D / 16)) * 16;
      r.k[i] = bload16(rk, off);
      r.v[i] = bload16(rv, off);
    }
  }
  // INT8 KV cache, LDS staging: the raw int8 K and V tiles land in LDS by
  // lds-loads in their natural [row][D] layout (RAW_BYTES: K, then V).  The
  // loads cover the same 16-byte chunks stage_load does: instruction i of wave
  // w fills bytes 1024 w + 4096 i .. +1023 of each, lane l chunk id =
  // tid + 256 i at 16 id.  The widening pass then reads them back
  // (stage_from_lds) and stage_store writes the stage, so no staging registers
  // stay live while a tile is computed.
  static constexpr int RAW_BYTES = 2 * 64 * D;
  static TM_DEV void raw_dma(char* raw, int tid, int wave, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                             uint32_t stride) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int id = tid + 256 * i;
      const uint32_t off = (id / (D / 16)) * stride + (id % (D / 16)) * 16;
      bload16_lds(rk, off, raw + 1024 * wave + 4096 * i);
      bload16_lds(rv, off, raw + 64 * D + 1024 * wave + 4096 * i);
    }
  }
  static TM_DEV void stage_from_lds(Stage& r, int tid, const char* raw) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      r.k[i] = *reinterpret_cast<const u32x4*>(raw + 16 * (tid + 256 * i));
      r.v[i] = *reinterpret_cast<const u32x4*>(raw + 64 * D + 16 * (tid + 256 * i));
    }
  }
  // INT8 V: the tile's scale s_v = mv 2^E.  V is widened exactly to v8 2^E,
  // the mantissa mv goes into P (log2 mv added in the exponent) and the row
  // sum adds P / mv: the P.V numerator and the row sum then use the same
  // rounded weights, as with fp16 V.
  //  * s_v >= 2^-24: E = min(exponent, 5) and mv in [1, 16.2) for every scale
  //    up to 65504/127, the largest the quantiser makes from fp16 data (larger
  //    scales would let P overflow fp16 and are outside the supported range);
  //  * 0 < s_v < 2^-24: E = -24 (v8 2^-24 is still exact in fp16) and
  //    mv = s_v 2^24 < 1 (at least 2^-7 for any scale the quantiser makes:
  //    fp16 data give s_v >= 2^-24 / 127);
  //  * s_v = 0 (an all-zero block, as a caller may store it): V widens to zeros
  //    and mv = 1, so the block's probabilities still count in the row sum.
  struct VSplit {
    float lmv, rmv;   // log2 mv, 1 / mv
    f16x2 s2, b2;     // 2^E and -1152 2^E for the widening fma
  };
  static TM_DEV VSplit vsplit(float vsc) {
    // (selects, not branches: the split sits between a tile's loads and its
    // barrier)
    const bool big = vsc >= 0x1p-24f;
    const int E = big ? min((int)((__builtin_bit_cast(uint32_t, vsc) >> 23) & 0xFF) - 127, 5) : -24;
    const float tiny = vsc > 0.0f ? vsc * 0x1p24f : 1.0f;   // (exact)
    const float mv = big ? __builtin_ldexpf(vsc, -E) : tiny;
    const float p2 = vsc > 0.0f ? __builtin_ldexpf(1.0f, E) : 0.0f;
    VSplit v;
    v.lmv = __builtin_amdgcn_logf(mv);
    v.rmv = 1.0f / mv;
    v.s2 = f16x2{(f16)p2, (f16)p2};
    v.b2 = f16x2{(f16)(-1152.0f * p2), (f16)(-1152.0f * p2)};
    return v;
  }
  static TM_DEV void stage_store(const Stage& r, int route, int tid, char* kl, char* vl,
                                 f16x2 vs2 = f16x2{(f16)1.0f, (f16)1.0f},
                                 f16x2 vb2 = f16x2{(f16)-1152.0f, (f16)-1152.0f}) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int id = tid + 256 * i;
      const int R = id / (D / 16), col = id % (D / 16);   // 16 int8 channels: col*16 ..
      u32x4 c0, c1;
      if (route == 1) {
        *reinterpret_cast<u32x4*>(kl + k8_off(R, col)) = r.k[i];
      } else {
        i8x16_to_f16x16(r.k[i], c0, c1);
        *reinterpret_cast<u32x4*>(kl + k16_off(R, 2 * col)) = c0;
        *reinterpret_cast<u32x4*>(kl + k16_off(R, 2 * col + 1)) = c1;
      }
      i8x16_to_f16x16(r.v[i], c0, c1, vs2, vb2);
      *reinterpret_cast<u32x4*>(vl + v_off(R, col * 16)) = c0;
      *reinterpret_cast<u32x4*>(vl + v_off(R, col * 16 + 8)) = c1;
    }
  }

  // --- raw S^T for the 32-key half h: FP16 path (float bits in int registers)
  static TM_DEV void qk16(const char* kl, int h, const f16x8 (&qf)[QB][NDS], i32x4 (&S)[QB][2], int c, int gq) {
    f32x4 acc[QB][2];
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc[j][kk] = f32x4{0, 0, 0, 0};
    const char* base = kl + L16::lane(c) + gq * 16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const f16x8 ak = *reinterpret_cast<const f16x8*>(base + (2 * h + kk) * L16::step16 + ds * 64);
#pragma unroll
        for (int j = 0; j < QB; ++j)
          acc[j][kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, qf[j][ds], acc[j][kk], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) S[j][kk] = __builtin_bit_cast(i32x4, acc[j][kk]);
  }

  // --- raw S^T for the 32-key half h: INT8 path (exact int32 accumulation)
  static TM_DEV void qk8(const char* kl, int h, const i32x4 (&q8)[QB][NDS8], i32x4 (&S)[QB][2], int c, int gq) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) S[j][kk] = i32x4{0, 0, 0, 0};
    const char* base = kl + L8::lane(c) + gq * 16;
#pragma unroll
    for (int ds = 0; ds < NDS8; ++ds) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i32x4 ak = *reinterpret_cast<const i32x4*>(base + (2 * h + kk) * L8::step16 + ds * 64);
#pragma unroll
        for (int j = 0; j < QB; ++j)
          S[j][kk] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ak, q8[j][ds], S[j][kk], 0, 0, 0);
      }
    }
  }

  // --- INT8 results -> float bits, in place (the registers stay int-typed)
  static TM_DEV void int_to_float_bits(i32x4 (&S)[QB][2]) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) S[j][kk] = __builtin_bit_cast(i32x4, __builtin_convertvector(S[j][kk], f32x4));
  }

  // --- diagonal tile: a key may not come after the query (key0 = first key
  // of this lane's rows in the half, qpos[j] = query position)
  static TM_DEV void mask_diag(i32x4 (&S)[QB][2], int key0, const int (&qpos)[QB]) {
#pragma unroll
    for (int j = 0; j < QB; ++j)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 16 * kk + i > qpos[j]) S[j][kk][i] = __builtin_bit_cast(int32_t, -INFINITY);
  }

  // --- shared online-softmax update for half h from raw scores (float bits).
  // Each lane first compares its own keys' max with its reference max; only
  // when some lane of the wave exceeds it by more than kSlack does the wave
  // take the reduction over the query's 4 lanes, move the reference and
  // rescale l and the accumulator (the same decision as reducing first, since
  // the reduced max exceeds the bound exactly when some lane's max does).
  // Row sums on the MFMA: an all-ones A operand times P^T gives, in every row,
  // the query's sum over the half's 32 keys.  kLacc accumulates it into lacc;
  // otherwise it is added to lrow (INT8 V: divided by the tile's mv, see
  // VSplit).
  // The reference max is kept negated (nref = -m_ref) so that every exponent
  // is one fma with it as the addend.
  static TM_DEV void softmax(const i32x4 (&S)[QB][2], const float (&cj)[QB], float lmv, float (&nref)[QB],
                             float (&lrow)[QB], f32x4 (&lacc)[QB], f32x4 (&O)[QB][NDB], f16x8 (&P)[QB]) {
    float lm[QB];
    bool up = false, upj[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      // Whole-vector bit casts: clang mis-lowers __builtin_bit_cast applied to
      // a single element of an ext_vector (it reads element 0).
      const f32x4 a = __builtin_bit_cast(f32x4, S[j][0]);
      const f32x4 b = __builtin_bit_cast(f32x4, S[j][1]);
      // three-input max tree (v_maximum3): 4 instructions for 8 values
      const float t0 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[0], a[1]), a[2]);
      const float t1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(a[3], b[0]), b[1]);
      const float t2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(b[2], b[3]), t0);
      lm[j] = __builtin_elementwise_maximum(t1, t2);
      // lm c - m_ref > kSlack in one fma (m_ref = -inf gives +inf: a first
      // finite score always moves the reference)
      upj[j] = __builtin_fmaf(lm[j], cj[j], nref[j]) > kSlack;
      up |= upj[j];
    }
    // A wave skips the reduction of each q-block none of whose rows moved
    // (measured faster with three q-blocks and with two over an fp16 cache;
    // slower with two over the INT8 cache).
    constexpr bool kGate = QB == 3 || (QB == 2 && !KVI8);
    if (__any(up)) {
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        if (kGate && !__any(upj[j])) continue;
        float mx = lm[j];
        mx = rows4_max(mx);
        const float tmax = mx * cj[j];
        const bool moved = tmax + nref[j] > kSlack;
        const float tnew = tmax + kOver;
        const float alpha = moved ? __builtin_amdgcn_exp2f(-(nref[j] + tnew)) : 1.0f;
        nref[j] = moved ? -tnew : nref[j];
        if (!kLacc) lrow[j] *= alpha;
        if (kGate || __any(moved)) {
          if (kLacc) lacc[j] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) O[j][db] *= alpha;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const f32x4 a = __builtin_bit_cast(f32x4, S[j][0]);
      const f32x4 b = __builtin_bit_cast(f32x4, S[j][1]);
      const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      // INT8 V: p mv = exp2(x c - m_ref + log2 mv)
      const float add = KVI8 ? nref[j] + lmv : nref[j];
      u32x4 pk;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * t], cj[j], add));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[2 * t + 1], cj[j], add));
        const f16x2 hv = {(f16)p0, (f16)p1};
        pk[t] = __builtin_bit_cast(uint32_t, hv);
      }
      P[j] = __builtin_bit_cast(f16x8, pk);
    }
  }

  // --- O^T += V^T P^T for half h.  Lane (c, gq) needs, for channel db*16+c,
  // keys 32h+4gq+0..3 (lo) and 32h+16+4gq+0..3 (hi); each comes from one
  // ds_read_b64_tr_b16 whose 16 lanes address 4 keys x 16 channels.
  static TM_DEV void pv(const char* vl, int h, const f16x8 (&P)[QB], f32x4 (&O)[QB][NDB], f32x4 (&lacc)[QB],
                        float (&lrow)[QB], float rmv, int lane) {
    const int gq = lane >> 4, jl = lane & 15;
    // key 32h + 16e + (4gq + jl/4), channels db*16 + 4*(jl%4) .. +3
    const char* base = vl + LV::lane(4 * gq + (jl >> 2)) + 8 * (jl & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f16x4 lo = read_tr16(base + (2 * h) * LV::step16 + db * 32);
      const f16x4 hi = read_tr16(base + (2 * h + 1) * LV::step16 + db * 32);
      const f16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int j = 0; j < QB; ++j) O[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, P[j], O[j][db], 0, 0, 0);
    }
    const f16x8 ones = {(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      if (kLacc) {
        lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, P[j], lacc[j], 0, 0, 0);
      } else {
        const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, P[j], f32x4{0, 0, 0, 0}, 0, 0, 0);
        lrow[j] = __builtin_fmaf(t[0], rmv, lrow[j]);
      }
    }
  }
};

// Operand preparation of the prefill kernel: Q and K quantised beforehand, both
// quantised in the kernel, or Q in the kernel and K beforehand.
enum OtfMode : int { kOtfNone = 0, kOtfQK = 1, kOtfQ = 2 };

// Waves per SIMD each prefill kernel is built for.  d = 64 (34-38 KB of LDS):
// 3 with three q-blocks, or two over the INT8 cache, which fit 168 VGPRs; 4
// with fewer (128 VGPRs).  From 2, 3 waves per SIMD took the d = 64 kernels
// 13-15 % less time, 4 another 5-8 %.  d = 128: three q-blocks take 248 of 256
// VGPRs, so 2.  With one or two q-blocks over an fp16 cache, 3 (single V
// stage, below), except with K quantised in the kernel (its INT8 K tile needs
// 8 KB more LDS); otherwise 2, because the double-buffered K/V stages take
// 67 KB of LDS.
//
// Single V stage: K stays double-buffered but V gets one stage, so a
// workgroup takes 50 KB of LDS and three fit a CU.  Tile n+1's V loads are
// issued after the end-of-tile barrier (every wave is done with tile n's V)
// and awaited, behind a second barrier, just before the first P.V of tile
// n+1, i.e. behind half a tile of QK^T and softmax; the third workgroup
// covers the rest.  The two-head kernel fits 168 VGPRs with Q's operands made
// in the kernel (row sums in one register per q-block, Attn::kLacc) and
// spills 7 with quantise-once operands; both run faster than with two stages
// (5-10 %).
template <int D, int QB, bool KVI8, int OTFM>
constexpr bool attn_single_v() {
  return D == 128 && QB <= 2 && !KVI8 && OTFM != kOtfQK;
}
template <int D, int QB, bool KVI8, int OTFM>
constexpr int attn_waves_per_simd() {
  return D == 128 ? (attn_single_v<D, QB, KVI8, OTFM>() ? 3 : 2) : (QB == 3 || (QB == 2 && KVI8)) ? 3 : 4;
}

// LDS objects of a prefill workgroup.  Two stages (K tile, then V tile) as two
// LDS objects: with a fixed object per access the compiler can tell the loads
// into one stage from reads of the other and does not make those reads wait
// for the loads.
//   INT8 KV cache, up to 2 heads per item: the next tile travels through
//   registers (staged while the current one is computed) into the other stage.
//   INT8 KV cache, 3 heads per item (RAWST): those 16 staging registers do not
//   fit beside three q-blocks, so lds-loads bring the raw int8 tile into `raw`
//   while the one stage is computed, and it is widened into the stage between
//   two barriers.
//   Single V stage (attn_single_v): stage A holds K and the one V, stage B K
//   only.
// On-the-fly mode: the current INT8 tile's K, and per-wave Q-block maxima.
struct AttnLds {
  char *stA, *stB, *raw, *k8s;
  uint32_t* qam;
};
template <int D, int QB, bool KVI8, int OTFM>
TM_DEV __attribute__((always_inline)) AttnLds attn_lds() {
  using A = Attn<D, QB, KVI8>;
  constexpr bool OTF = OTFM == kOtfQK;
  constexpr bool QOTF = OTFM != kOtfNone;
  constexpr bool RAWST = KVI8 && QB == 3;
  constexpr int STAGE = A::KBYTES + A::VBYTES + (OTF ? 16 : 0);
  __shared__ __attribute__((aligned(1024))) char stA[STAGE];
  constexpr bool VS1 = attn_single_v<D, QB, KVI8, OTFM>();
  __shared__ __attribute__((aligned(1024))) char stB[RAWST ? 16 : VS1 ? A::KBYTES : STAGE];
  __shared__ __attribute__((aligned(1024))) char raw[RAWST ? A::RAW_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char k8s[OTF ? A::L8::BYTES : 16];
  __shared__ uint32_t qam[QOTF ? 3 * 4 : 1];
  return AttnLds{stA, stB, raw, k8s, qam};
}

// The prefill kernel: one work item (a query tile of one sequence, the query
// heads of one chunk of a KV head's GQA group) per workgroup.
template <int D, int QB, bool KVI8, int OTFM, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd<D, QB, KVI8, OTFM>(),
                                                                     attn_waves_per_simd<D, QB, KVI8, OTFM>())))
void attn_prefill_kernel(const AttnArgs a) {
  constexpr bool OTF = OTFM == kOtfQK;    // K (and Q) quantised in the kernel
  constexpr bool QOTF = OTFM != kOtfNone; // Q quantised in the kernel
  static_assert(!(KVI8 && OTF), "on-the-fly quantisation applies to an fp16 K");
  using A = Attn<D, QB, KVI8>;            // tile layout, DMA and staging
  constexpr int NDS = A::NDS, NDS8 = A::NDS8, NDB = A::NDB;
  constexpr bool RAWST = KVI8 && QB == 3;
  constexpr bool VS1 = attn_single_v<D, QB, KVI8, OTFM>();
  const AttnLds lds = attn_lds<D, QB, KVI8, OTFM>();
  char* const stA = lds.stA;
  char* const stB = lds.stB;
  char* const raw = lds.raw;
  char* const k8s = lds.k8s;
  uint32_t* const qam = lds.qam;
  const WorkItem item = a.items[blockIdx.x];
  const int b = uniform(item.b);
  const int hk = uniform(item.hk);
  const int m = uniform(item.m);
  const int chunk = uniform(item.chunk);
  // empty slot (b < 0), or an item outside the problem (work list not built
  // for these parameters): nothing to do
  if (b < 0 || b >= a.batch || hk < 0 || hk >= a.Hk || m < 0 || m >= a.T || chunk < 0 || chunk >= a.nch) return;
  {
    constexpr int QE = QB;
    using AQ = Attn<D, QE, KVI8>;
#include "attn_prefill_item.inc"
  }
}

// Same, for GQA groups whose last head chunk is partial (the chunk size does
// not divide G): each item runs the body for its own head count, so a partial
// chunk's missing q-blocks are not computed on zeros.
template <int D, int QB, bool KVI8, int OTFM, bool DBG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd<D, QB, KVI8, OTFM>(),
                                                                     attn_waves_per_simd<D, QB, KVI8, OTFM>())))
void attn_prefill_mixed_kernel(const AttnArgs a) {
  constexpr bool OTF = OTFM == kOtfQK;
  constexpr bool QOTF = OTFM != kOtfNone;
  static_assert(!(KVI8 && OTF), "on-the-fly quantisation applies to an fp16 K");
  static_assert(QB > 1, "a one-head chunk is never partial");
  using A = Attn<D, QB, KVI8>;
  constexpr int NDS = A::NDS, NDS8 = A::NDS8, NDB = A::NDB;
  constexpr bool RAWST = KVI8 && QB == 3;
  constexpr bool VS1 = attn_single_v<D, QB, KVI8, OTFM>();
  const AttnLds lds = attn_lds<D, QB, KVI8, OTFM>();
  char* const stA = lds.stA;
  char* const stB = lds.stB;
  char* const raw = lds.raw;
  char* const k8s = lds.k8s;
  uint32_t* const qam = lds.qam;
  const WorkItem item = a.items[blockIdx.x];
  const int b = uniform(item.b);
  const int hk = uniform(item.hk);
  const int m = uniform(item.m);
  const int chunk = uniform(item.chunk);
  if (b < 0 || b >= a.batch || hk < 0 || hk >= a.Hk || m < 0 || m >= a.T || chunk < 0 || chunk >= a.nch) return;
  const int heads = min(a.hc, a.G - chunk * a.hc);
  if (heads >= QB) {
    constexpr int QE = QB;
    using AQ = Attn<D, QE, KVI8>;
#include "attn_prefill_item.inc"
  } else if (QB == 3 && heads == 2) {   // (dead code at QB = 2, which the QE below keeps compilable)
    constexpr int QE = QB == 3 ? 2 : 1;
    using AQ = Attn<D, QE, KVI8>;
#include "attn_prefill_item.inc"
  } else {
    constexpr int QE = 1;
    using AQ = Attn<D, QE, KVI8>;
#include "attn_prefill_item.inc"
  }
}

template <int D, int QB, bool KVI8, int OTFM, bool DBG>
hipError_t launch_attn_inst(const AttnArgs& a, int64_t nslots, hipStream_t s) {
  if constexpr (QB > 1) {
    if (a.G % a.hc != 0) {
      hipLaunchKernelGGL((attn_prefill_mixed_kernel<D, QB, KVI8, OTFM, DBG>), dim3((unsigned)nslots), dim3(256), 0,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_prefill_kernel<D, QB, KVI8, OTFM, DBG>), dim3((unsigned)nslots), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tilemix
