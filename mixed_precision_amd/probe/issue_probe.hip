// Microbenchmarks of one gfx950 compute unit: what an instruction costs the
// SIMD's issue port, and what the LDS delivers.  They back the cost model of
// the attention kernel (its softmax VALU work and its MFMAs share each SIMD's
// issue port; its operands come from LDS).  Not part of the attention path.
//
// One 8-wave workgroup per CU (512 threads, 80 KB of LDS so no second one
// fits): waves w and w + 4 share SIMD w.  Waves 0-3 run stream A, waves 4-7
// stream B, each for its own iteration count, after a common barrier; each
// wave stamps the shader clock (s_memtime) before and after its loop.
// Streams (instructions per iteration):
//   FMA       32 v_fma_f32 in 8 independent chains
//   EXP       32 v_exp_f32 in 8 independent chains (x <- 2^-x stays in (0.5, 1))
//   MFMA_F16  16 v_mfma_f32_16x16x32_f16 into 4 independent accumulators
//   MFMA_I8   16 v_mfma_i32_16x16x64_i8, 4 accumulators
//   MFMA32    16 v_mfma_f32_32x32x16_f16, 4 accumulators
//   MIX       16 v_mfma_f32_16x16x32_f16 and 32 v_fma_f32 of one wave, one MFMA
//             then two FMAs
//   LDS128 / LDSTR16: 8 ds_read_b128 / ds_read_b64_tr_b16, each lane's
//   address inside the 64 KB probe area (a contiguous 16-byte slot per lane;
//   the transposed reads use the attention kernel's V^T addressing over
//   1056-byte blocks).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tilemix_probe.h"

namespace tmprobe {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kLdsAlloc = 80 * 1024;   // more than half the CU's LDS: one workgroup per CU
constexpr int kArea = 64 * 1024;       // the part the LDS streams read (a power of two)

template <int OP>
__device__ __forceinline__ float stream(int iters, const char* lds, int lane, int wave) {
  float r = 0.0f;
  if constexpr (OP == TILEMIX_PROBE_FMA) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)lane * 1e-3f + (float)k;
    // lane-dependent operands stay in VGPRs (no literal forms), as in the
    // attention kernel's score FMAs
    const float a = 0.999f - (float)lane * 1e-7f, b = 1e-3f + (float)lane * 1e-7f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], a, b);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) r += x[k];
  } else if constexpr (OP == TILEMIX_PROBE_EXP) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = 0.5f + (float)k * 0.01f + (float)lane * 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) r += x[k];
  } else if constexpr (OP == TILEMIX_PROBE_MFMA_F16) {
    const f16x8 a = {(f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f, (f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f};
    const f16x8 b = {(f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f};
    f32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) r += acc[k][0] + acc[k][3];
  } else if constexpr (OP == TILEMIX_PROBE_MFMA_I8) {
    const i32x4 a = {0x01020304, 0x05060708, 0x01020304, 0x05060708};
    const i32x4 b = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    i32x4 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) r += (float)(acc[k][0] + acc[k][3]);
  } else if constexpr (OP == TILEMIX_PROBE_MFMA32_F16) {
    const f16x8 a = {(f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f, (f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f};
    const f16x8 b = {(f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f};
    f32x16 acc[4] = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) r += acc[k][0] + acc[k][15];
  } else if constexpr (OP == TILEMIX_PROBE_MIX) {
    // one wave's own MFMAs and FMAs, interleaved one MFMA to two FMAs
    const f16x8 a = {(f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f, (f16)1.0f, (f16)0.5f, (f16)0.25f, (f16)0.125f};
    const f16x8 b = {(f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f, (f16)1e-3f};
    const float fa = 0.999f - (float)lane * 1e-7f, fb = 1e-3f + (float)lane * 1e-7f;
    f32x4 acc[4] = {};
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)lane * 1e-3f + (float)k;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
          x[2 * k] = __builtin_fmaf(x[2 * k], fa, fb);
          x[2 * k + 1] = __builtin_fmaf(x[2 * k + 1], fa, fb);
        }
      }
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) r += acc[k][0] + acc[k][3];
#pragma unroll
    for (int k = 0; k < 8; ++k) r += x[k];
  } else if constexpr (OP == TILEMIX_PROBE_LDS128) {
    u32x4 acc = {0, 0, 0, 0};
    const int base = wave * 8192 + lane * 16;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        acc ^= *reinterpret_cast<const u32x4*>(lds + ((base + (i * 8 + u) * 1024) & (kArea - 1)));
    }
    r = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  } else if constexpr (OP == TILEMIX_PROBE_LDS_TR16) {
    // the attention kernel's V^T read: 16-lane group gq reads keys 4gq .. 4gq+3
    // (one 1056-byte block each), 32 bytes of channels per key
    // (the 8 addresses are loop-invariant: the LDS has no cache, so reading
    // them again costs the same, and no address arithmetic enters the loop)
    const int gq = lane >> 4, jl = lane & 15;
    const int base = (4 * gq + (jl >> 2)) * 1056 + 8 * (jl & 3) + (wave & 1) * 16 * 1056;
    s16x4 acc = {0, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int off = base + u * 64;   // channel blocks of one key group, as P.V reads them
        acc ^= __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off));
      }
    }
    r = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  }
  return r;
}

template <int OPA, int OPB>
__global__ __launch_bounds__(512) void probe_kernel(int iters_a, int iters_b, unsigned long long* stamps,
                                                    float* sink) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsAlloc];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // fill the area once (16 bytes per thread per step)
  for (int o = tid * 16; o < kLdsAlloc; o += 512 * 16)
    *reinterpret_cast<u32x4*>(lds + o) = u32x4{(unsigned)o, (unsigned)o ^ 0x5a5a5a5au, (unsigned)tid, 7u};
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const float r = wave < 4 ? stream<OPA>(iters_a, lds, lane, wave) : stream<OPB>(iters_b, lds, lane, wave);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const int w = blockIdx.x * 8 + wave;
  if (lane == 0) {
    stamps[2 * w] = t0;
    stamps[2 * w + 1] = t1;
  }
  sink[w * 64 + lane] = r;
}

template <int OPA, int OPB>
hipError_t launch(int iters_a, int iters_b, int nwg, unsigned long long* stamps, float* sink, hipStream_t s) {
  hipLaunchKernelGGL((probe_kernel<OPA, OPB>), dim3((unsigned)nwg), dim3(512), 0, s, iters_a, iters_b, stamps, sink);
  return hipGetLastError();
}

}  // namespace tmprobe

extern "C" int tilemix_probe_run(int op_a, int op_b, int iters_a, int iters_b, int num_workgroups,
                                 unsigned long long* stamps, float* sink, void* stream) {
  using namespace tmprobe;
  if (iters_a < 0 || iters_b < 0 || num_workgroups < 1 || num_workgroups > 65536 || !stamps || !sink) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
#define TM_PROBE_CASE(A, B) \
  if (op_a == (A) && op_b == (B)) e = launch<(A), (B)>(iters_a, iters_b, num_workgroups, stamps, sink, s);
  TM_PROBE_CASE(TILEMIX_PROBE_FMA, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_FMA, TILEMIX_PROBE_FMA)
  TM_PROBE_CASE(TILEMIX_PROBE_EXP, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_EXP, TILEMIX_PROBE_EXP)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA_F16, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA_F16, TILEMIX_PROBE_MFMA_F16)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA_I8, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA32_F16, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA_F16, TILEMIX_PROBE_FMA)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA_I8, TILEMIX_PROBE_FMA)
  TM_PROBE_CASE(TILEMIX_PROBE_MFMA32_F16, TILEMIX_PROBE_FMA)
  TM_PROBE_CASE(TILEMIX_PROBE_MIX, TILEMIX_PROBE_IDLE)
  TM_PROBE_CASE(TILEMIX_PROBE_MIX, TILEMIX_PROBE_MIX)
  TM_PROBE_CASE(TILEMIX_PROBE_LDS128, TILEMIX_PROBE_LDS128)
  TM_PROBE_CASE(TILEMIX_PROBE_LDS_TR16, TILEMIX_PROBE_LDS_TR16)
#undef TM_PROBE_CASE
  return e == hipSuccess ? 0 : 2;
}
