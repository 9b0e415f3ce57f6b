/* Microbenchmarks of one gfx950 compute unit, in their own library
 * (libtilemix_probe.so), not part of the attention path.
 *
 * They measure what the attention kernel's cost model rests on: how many
 * issue cycles of a SIMD an instruction takes (VALU FMA and exp2, the
 * 16x16x32 f16, 16x16x64 i8 and 32x32x16 f16 MFMAs, alone and beside another
 * wave's FMA stream) and how many bytes per cycle the LDS delivers to
 * ds_read_b128 and ds_read_b64_tr_b16.  The Python runner
 * (python -m mixed_precision_amd.probe) turns the stamps into those figures.
 */
#ifndef TILEMIX_PROBE_H
#define TILEMIX_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

/* instruction streams a wave can run */
enum {
  TILEMIX_PROBE_IDLE = 0,        /* nothing: the wave ends at once */
  TILEMIX_PROBE_FMA = 1,         /* 32 v_fma_f32 per iteration, 8 independent chains */
  TILEMIX_PROBE_EXP = 2,         /* 32 v_exp_f32 per iteration, 8 independent chains */
  TILEMIX_PROBE_MFMA_F16 = 3,    /* 16 v_mfma_f32_16x16x32_f16 per iteration, 4 accumulators */
  TILEMIX_PROBE_MFMA_I8 = 4,     /* 16 v_mfma_i32_16x16x64_i8 per iteration, 4 accumulators */
  TILEMIX_PROBE_MFMA32_F16 = 5,  /* 16 v_mfma_f32_32x32x16_f16 per iteration, 4 accumulators */
  TILEMIX_PROBE_LDS128 = 6,      /* 8 ds_read_b128 per iteration, 16 contiguous bytes per lane */
  TILEMIX_PROBE_LDS_TR16 = 7,    /* 8 ds_read_b64_tr_b16 per iteration, the attention kernel's V^T addressing */
  TILEMIX_PROBE_MIX = 8          /* 16 v_mfma_f32_16x16x32_f16 and 32 v_fma_f32 per iteration, one wave,
                                    each MFMA followed by two independent FMAs */
};

/* Launches num_workgroups (1..65536) workgroups of 8 waves, one per CU (80 KB
 * of LDS each): waves 0-3 run stream op_a for iters_a iterations, waves 4-7
 * (wave w + 4 on the SIMD of wave w) run op_b for iters_b, after a common
 * barrier.  Supported pairs: (FMA, IDLE), (FMA, FMA), (EXP, IDLE), (EXP, EXP),
 * (MFMA_F16, IDLE), (MFMA_F16, MFMA_F16), (MFMA_I8, IDLE), (MFMA32_F16, IDLE),
 * (MFMA_F16, FMA), (MFMA_I8, FMA), (MFMA32_F16, FMA), (MIX, IDLE), (MIX, MIX)
 * and each LDS stream with
 * itself.
 *   stamps: device, uint64 [num_workgroups * 8][2], caller-owned: each wave's
 *           shader-clock stamps (s_memtime) before and after its loop;
 *   sink:   device, float [num_workgroups * 8 * 64], caller-owned: each lane's
 *           result, so that no stream is optimised away;
 *   stream: a hipStream_t; the call is asynchronous on it.
 * Returns 0 when launched, 1 for an invalid argument, 2 for an unsupported
 * pair or a launch failure. */
int tilemix_probe_run(int op_a, int op_b, int iters_a, int iters_b, int num_workgroups,
                      unsigned long long* stamps, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEMIX_PROBE_H */
