"""Runner of the compute-unit microbenchmarks in ``libtilemix_probe.so``
(``include/tilemix_probe.h``): ``python -m mixed_precision_amd.probe``.

Prints one JSON object with, per stream, the shader-clock cycles each
instruction takes a wave alone on its SIMD and the SIMD's cycles per
instruction when two waves stream it, the issue cycles an MFMA takes from a
co-running wave's FMA stream, and the LDS bytes a CU reads per cycle.  Cycles
are those of the s_memtime counter; the run also reports that counter's rate
against host time.

The mixed stream: one wave issues 16 MFMAs and 32 independent FMAs per
iteration, one MFMA then two FMAs; compared with the MFMA-only and FMA-only
times of the same counts it shows how much VALU work hides under a wave's own
MFMAs.

The MFMA cost to the port: waves 0-3 stream MFMAs while waves 4-7 (one per
SIMD beside them) stream F FMAs.  The MFMA stream is sized to outlast the FMA
stream; the MFMAs issued inside the FMA window are its count minus those
issued after it, at the MFMA-alone rate.  Then
    cost = (T_fma_beside_mfma - F * c_fma_alone) / MFMAs_in_window.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtilemix_probe.so")

IDLE, FMA, EXP, MFMA_F16, MFMA_I8, MFMA32_F16, LDS128, LDS_TR16, MIX = range(9)
PER_ITER = {FMA: 32, EXP: 32, MFMA_F16: 16, MFMA_I8: 16, MFMA32_F16: 16, LDS128: 8, LDS_TR16: 8}
LDS_BYTES_PER_LANE = {LDS128: 16, LDS_TR16: 8}


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: build with __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.tilemix_probe_run.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 3
    lib.tilemix_probe_run.restype = ctypes.c_int
    return lib


class Probe:
    def __init__(self, nwg: int | None = None, dev: str = "cuda:0"):
        if not torch.cuda.is_available():
            raise RuntimeError("the probes need a GPU")
        self.lib = _lib()
        self.dev = torch.device(dev)
        self.nwg = nwg or torch.cuda.get_device_properties(self.dev).multi_processor_count
        self.stamps = torch.zeros((self.nwg * 8, 2), dtype=torch.int64, device=self.dev)
        self.sink = torch.zeros(self.nwg * 8 * 64, dtype=torch.float32, device=self.dev)

    def run(self, op_a: int, op_b: int, it_a: int, it_b: int, reps: int = 3):
        """Median over `reps` launches of the per-wave cycles (mean over the
        workgroups) of waves 0-3 and 4-7, the per-workgroup span, and the host
        time of the launch (ms)."""
        stream = torch.cuda.current_stream(self.dev)
        res = []
        for _ in range(reps + 1):                      # the first launch warms up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = self.lib.tilemix_probe_run(op_a, op_b, it_a, it_b, self.nwg, self.stamps.data_ptr(),
                                            self.sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"tilemix_probe_run({op_a}, {op_b}) returned {rc}")
            e1.record(stream)
            torch.cuda.synchronize(self.dev)
            st = self.stamps.cpu().view(self.nwg, 8, 2).to(torch.float64)
            dur = st[:, :, 1] - st[:, :, 0]
            span = st[:, :, 1].max(dim=1).values - st[:, :, 0].min(dim=1).values
            res.append((float(dur[:, :4].mean()), float(dur[:, 4:].mean()), float(span.mean()), e0.elapsed_time(e1)))
        res = sorted(res[1:], key=lambda r: r[2])
        return res[len(res) // 2]


def measure(p: Probe, iters: int = 2048) -> dict:
    out = {"workgroups": p.nwg}
    # one wave per SIMD, then two
    for name, op in (("fma", FMA), ("exp", EXP), ("mfma_f16_16x16x32", MFMA_F16), ("mfma_i8_16x16x64", MFMA_I8),
                     ("mfma_f16_32x32x16", MFMA32_F16)):
        a, _, _, ms = p.run(op, IDLE, iters, 0)
        out[name] = {"cycles_alone": a / (iters * PER_ITER[op])}
        if op in (FMA, EXP, MFMA_F16):
            # two waves per SIMD: the SIMD's rate over the workgroup's span
            # (one wave may finish first, so the waves' own times would overstate it)
            _, _, span, _ = p.run(op, op, iters, iters)
            out[name]["simd_cycles_two_waves"] = span / (2 * iters * PER_ITER[op])
        if op == MFMA_F16:
            out["counter_per_ns"] = a / (ms * 1e6)       # s_memtime ticks per ns of host time
    c_fma = out["fma"]["cycles_alone"]
    # one wave's own MFMAs and FMAs interleaved (16 + 32 per iteration): how much
    # of the FMA time hides under the MFMAs, alone and with two such waves per SIMD
    t_m, t_f = 16 * out["mfma_f16_16x16x32"]["cycles_alone"], 32 * c_fma
    a, _, _, _ = p.run(MIX, IDLE, iters, 0)
    _, _, span, _ = p.run(MIX, MIX, iters, iters)
    out["mix_mfma_fma"] = {"cycles_per_iteration_alone": a / iters, "mfma_only": t_m, "fma_only": t_f,
                           "fma_hidden_fraction": (t_m + t_f - a / iters) / t_f,
                           "simd_cycles_per_iteration_two_waves": span / (2 * iters)}
    # MFMA cost to a co-running wave's FMA issue
    f_iters = iters
    for name, op in (("mfma_f16_16x16x32", MFMA_F16), ("mfma_i8_16x16x64", MFMA_I8),
                     ("mfma_f16_32x32x16", MFMA32_F16)):
        c_m = out[name]["cycles_alone"]
        t_f_guess = f_iters * 32 * c_fma * 2.0
        m_iters = max(1, int(1.15 * t_f_guess / (16 * c_m)))
        for _ in range(4):
            t_m, t_f, _, _ = p.run(op, FMA, m_iters, f_iters)
            if 1.02 * t_f <= t_m <= 1.4 * t_f:
                break
            m_iters = max(1, int(m_iters * 1.2 * t_f / t_m))
        in_window = 16 * m_iters - max(t_m - t_f, 0.0) / c_m
        out[name]["fma_cycles_beside"] = t_f / (f_iters * 32)
        out[name]["port_cycles_per_mfma"] = (t_f - f_iters * 32 * c_fma) / in_window
        out[name]["mfma_stream_outlasted_fma_by"] = t_m / t_f
    # LDS: all eight waves read; bytes per CU per counter cycle over the workgroup's span
    for name, op in (("lds_read_b128", LDS128), ("lds_read_b64_tr_b16", LDS_TR16)):
        _, _, span, _ = p.run(op, op, iters, iters)
        nbytes = 8 * 64 * LDS_BYTES_PER_LANE[op] * PER_ITER[op] * iters
        out[name] = {"bytes_per_cu_cycle": nbytes / span}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--iters", type=int, default=2048)
    ap.add_argument("--workgroups", type=int, default=None, help="default: one per CU")
    args = ap.parse_args(argv)
    res = measure(Probe(args.workgroups), args.iters)
    res["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
