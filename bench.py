"""Benchmark: routed FP16/INT8 causal prefill attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: blockwise INT8 quantisation of Q and K (and V for the
INT8 KV cache), route-word packing, the varlen/GQA work list and the fused
attention kernel (packing and the work list run on a second stream beside the
quantiser).  For an fp16 K/V the attention kernel makes Q's INT8 operands
on chip by default, so the step's quantiser call covers K only; --once
quantises Q beforehand as well, --otf makes K's on chip too.  All three give
the same output bits.  The step is captured once as a HIP graph and replayed
(--eager: launched directly); the attention kernel's own time comes from HIP
events around it in the eager steps that precede the capture.  Before the
warm-up steps of each phase the step runs untimed for --settle-ms of wall time
(default 300 ms, reported in the line): the GPU raises its clocks over tens of
milliseconds of sustained work, and a short timed window would otherwise time
that ramp.  Default workload: the LLaMA-3.2-3B-shaped attention layer
(batch 8, L = 4096, 24 query / 8 KV heads, d = 128, causal, FP16, 4 outlier
channels, 64x64 tiles, g = 1, 75 % of the legal tile groups INT8).

Prints one JSON line (rank 0).  Extra fields: the attention kernel's own time
and blended-MFMA roofline, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks
P_FP16 = 2516.6e12        # FLOP/s
P_INT8 = 5033.2e12        # OP/s
HBM_PEAK = 8.0e12         # B/s


# what decides the attention kernel's code on this workload: its headers and
# item body, the file that instantiates it at 3 heads per work item, and the
# build flags
KERNEL_SOURCES = ("mixed_precision_amd/csrc/attn_kernel.hpp", "mixed_precision_amd/csrc/attn_prefill_item.inc",
                  "mixed_precision_amd/csrc/device_common.hpp", "mixed_precision_amd/csrc/internal.hpp",
                  "mixed_precision_amd/csrc/attn_d128_qb3.hip", "mixed_precision_amd/build.py")


def kernel_source_digest():
    return source_digest(KERNEL_SOURCES)


def build_flags_text():
    """What the build script decides about the kernels' code: the target, the
    compile flags (without the absolute include paths, which differ between
    checkouts) and the per-source flags."""
    from mixed_precision_amd import build as b
    flags = [f for f in b.CXXFLAGS if not os.path.isabs(f)]
    return json.dumps({"arch": b.ARCH, "flags": flags, "source_flags": b.SOURCE_FLAGS}, sort_keys=True).encode()


def source_digest(files):
    """sha256 over sources: C++ files without their // comments and blank lines
    (an edit of a comment leaves the code, and so the counters taken on it,
    valid), the build script by its compile flags alone, other Python files as
    they are."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in files:
        if rel.endswith("build.py"):
            h.update(build_flags_text())
            continue
        with open(os.path.join(ROOT, rel), "rb") as f:
            data = f.read()
        if not rel.endswith(".py"):
            lines = (re.sub(rb"\s*//.*$", b"", ln).rstrip() for ln in data.split(b"\n"))
            data = b"\n".join(ln for ln in lines if ln)
        h.update(data)
    return h.hexdigest()


def measured_traffic(workload_name):
    """HBM bytes per attention launch from the committed counter summary, if it was taken on this
    workload with the attention kernel sources as they are now (else None)."""
    import re
    prof = os.path.join(ROOT, "profiles", "attn_prefill_kernel_llama3b_B8_L4096_hbm_bytes.md")
    if workload_name != "llama3.2-3b_attn_B8_L4096_h24kv8_d128_int8p75" or not os.path.exists(prof):
        return None
    text = open(prof).read()
    h = re.search(r"sources sha256[^:]*: `([0-9a-f]{64})`", text)
    t = re.search(r"roofline.traffic` = (\d+) bytes", text)
    if not h or not t or h.group(1) != kernel_source_digest():
        return None
    return int(t.group(1))


def attn_kernel_name(G, kv_int8):
    """The prefill kernel the library launches for a GQA ratio: query heads go to
    work items in chunks of up to 3 (INT8 cache: 2 when G is 4 or less and not a
    multiple of 3), and a partial last chunk selects the mixed-chunk kernel."""
    cap = 3 if (not kv_int8 or G % 3 == 0 or G > 4) else 2
    nch = -(-G // cap)
    hc = -(-G // nch)
    return "attn_prefill_mixed_kernel" if hc > 1 and G % hc else "attn_prefill_kernel"


def legal_pairs(lengths):
    return sum(L * (L + 1) // 2 for L in lengths)


def work_model(w, words):
    """Algorithmic work of one attention call, split by route.

    Per legal (query, key) pair: QK 2d ops on its tile's path, PV 2d fp16 flops.
    Pairs are counted exactly per tile: full off-diagonal tiles, lower triangles
    (clipped to the sequence) on the diagonal.  `words` are the packed route
    words (uint64 [Hk][B][T]) the library built for this call."""
    d = w.head_dim
    G = w.num_q_heads // w.num_kv_heads
    pairs16 = pairs8 = 0
    visits8 = 0            # (query tile, KV head, INT8 key tile) visits
    tiles8 = set()         # distinct INT8 key tiles (sequence, KV head, key tile)
    for b, L in enumerate(w.lengths):
        L = int(L)
        Tb = (L + 63) // 64
        for m in range(Tb):
            rows = min(64, L - 64 * m)
            for hk in range(w.num_kv_heads):
                word = int(words[hk, b, m])
                n_full = m                                   # key tiles 0..m-1 are fully legal
                bits = [(word >> (n // w.g)) & 1 for n in range(m + 1)]
                full8 = sum(bits[:n_full])
                diag = rows * (rows + 1) // 2
                dbit = bits[m]
                visits8 += full8 + dbit
                tiles8.update((b, hk, n) for n in range(m + 1) if bits[n])
                p8 = full8 * 64 * rows + (diag if dbit else 0)
                p16 = (n_full - full8) * 64 * rows + (0 if dbit else diag)
                pairs8 += G * p8
                pairs16 += G * p16
    f_qk16 = 2 * d * pairs16
    f_qk8 = 2 * d * pairs8
    f_pv = 2 * d * (pairs16 + pairs8)
    t_star = f_qk16 / P_FP16 + f_qk8 / P_INT8 + f_pv / P_FP16
    return dict(pairs=pairs16 + pairs8, pairs_int8=pairs8, f_qk16=f_qk16, f_qk8=f_qk8, f_pv=f_pv,
                ops=f_qk16 + f_qk8 + f_pv, t_star=t_star, visits8=visits8, tiles8=len(tiles8))


def _sampled_rows(inp, total_work, budget_s, seed=0):
    """Time the oracle on random (sequence, head, query-tile) rows in this
    process for about budget_s; returns (seconds per unit of legal-tile work, rows, work)."""
    import oracle as orc
    spans = orc.seq_spans(inp.cu)
    rng = np.random.default_rng(seed)
    done_work, t_attn, rows = 0, 0.0, 0
    while t_attn < budget_s:
        b = int(rng.integers(len(spans)))
        Tb = orc.num_tiles(spans[b][1])
        m = int(rng.integers(Tb))
        hq = int(rng.integers(inp.Hq))
        t1 = time.perf_counter()
        orc.attn_tile_row(inp, b, hq, m)
        t_attn += time.perf_counter() - t1
        done_work += m + 1
        rows += 1
    return t_attn / done_work, rows, done_work, t_attn


# whole-workload oracle timing up to this much legal-tile work (the 3B layer has 399,360 units)
FULL_ORACLE_WORK = 500_000


def cpu_baseline(w, budget_s=15.0, budget_1t=5.0):
    """The oracle, as it stands, timed on this host's cores.  The oracle inputs
    (its own quantiser and packer) are made in full.  The attention is timed
    on the whole workload when its legal-tile work is at most FULL_ORACLE_WORK
    units: rows go to worker processes, one BLAS thread each.  Larger
    workloads use a bounded random sample of rows, extrapolated by legal-tile
    work.  A one-thread figure (one process, BLAS limited to one thread, a
    sample of rows) is reported beside it."""
    import oracle as orc
    from tests.oracle_inputs import oracle_inputs
    from tests import oracle_pool
    t0 = time.perf_counter()
    inp = oracle_inputs(w)          # quantise Q/K(/V) and pack the route words, in full
    t_prep = time.perf_counter() - t0
    spans = orc.seq_spans(w.cu_seqlens)
    total_work = sum(w.num_q_heads * t * (t + 1) // 2 for t in (orc.num_tiles(L) for _, L in spans))
    host = len(os.sched_getaffinity(0))
    if total_work <= FULL_ORACLE_WORK:
        procs = oracle_pool.workers()
        t1 = time.perf_counter()
        oracle_pool.full_output(inp, procs=procs)
        t_attn = time.perf_counter() - t1
        t_full = t_prep + t_attn
        sample = (f"whole workload: quantise+pack {t_prep:.2f} s (one process), attention over all "
                  f"{total_work} legal (sequence, head, query tile, key tile) units {t_attn:.1f} s "
                  f"({procs} worker processes, one BLAS thread each)")
        cores = procs
    else:
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = 1
        per_work, rows, done, t_attn = _sampled_rows(inp, total_work, budget_s)
        t_full = t_prep + per_work * total_work
        sample = (f"quantise+pack in full ({t_prep:.2f} s); attention on {rows} random (seq, head, query-tile) "
                  f"rows ({done} of {total_work} legal tile visits, {t_attn:.1f} s), extrapolated by "
                  f"legal-tile work")
    res = {"value": w.num_tokens / t_full, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "host_cpus": host, "sample": sample}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            per_work, rows, done, t_attn = _sampled_rows(inp, total_work, budget_1t, seed=1)
        t1t = t_prep + per_work * total_work
        res["one_thread"] = {"value": w.num_tokens / t1t, "unit": "tokens/s", "cores": 1,
                             "sample": f"{rows} random rows ({done} tile visits, {t_attn:.1f} s) in one process "
                                       f"with one BLAS thread, extrapolated by legal-tile work; "
                                       f"quantise+pack as above"}
    except ImportError:  # pragma: no cover
        pass
    return res


def settle_clocks(step, settle_ms):
    """Run the step untimed until the GPU has been busy for settle_ms of wall
    time, before the warm-up steps.  The part raises its clocks over tens of
    milliseconds of sustained work: without this, a short run (a few warm-up
    steps, 20 timed ones) times the ramp rather than the steady state a
    stream of layers runs at.  Returns what was run, for the JSON line."""
    import torch
    if settle_ms <= 0:
        return {"ms": 0.0, "steps": 0}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()      # keep the host within a few steps of the GPU
    torch.cuda.synchronize()
    return {"ms": (time.perf_counter() - t0) * 1e3, "steps": n}


def deviation_sweep(args, w, plan, q, k, v, cu, q_q, q_s, k_q, k_s, v_q, v_s, words, stream):
    """Coverage -> deviation: the same inputs routed at each INT8 coverage p; MaxDiff and MeanDiff
    (largest and mean absolute elementwise difference, all tokens/heads/channels) of the fp32 output
    against the 0 % output, which takes the FP16 path on every tile."""
    import torch
    from mixed_precision_amd import tilemix as tm
    from workloads import route_bernoulli_groups
    if args.config == 3 and not args.template:
        raise SystemExit("--deviation-sweep needs a Bernoulli-routed workload (configs 1, 2, 4, 5) or --template")
    dev = q.device
    ps = [float(x) for x in args.deviation_sweep.split(",")]
    if 0.0 not in ps:
        ps = [0.0] + ps
    N, Hq, d = w.q.shape
    plan32 = tm.AttnPlan(tm.AttnProblem(w.batch, w.max_seqlen, Hq, w.num_kv_heads, d, w.g, w.blk_q, w.sm_scale,
                                        w.kv_int8, True), dev)
    tm.tilemix_quantize_blockwise(q, cu, w.max_seqlen, w.blk_q, q_q, q_s, stream=stream)
    if w.kv_int8:
        tm.tilemix_quantize_blockwise(k, cu, w.max_seqlen, 64, k_q, k_s, stream=stream)
        tm.tilemix_quantize_blockwise(v, cu, w.max_seqlen, 64, v_q, v_s, stream=stream)
    else:
        tm.tilemix_quantize_blockwise(k, cu, w.max_seqlen, 64, k_q, k_s, stream=stream)
    plan32.schedule(cu, stream=stream)
    ref = None
    outs = {}
    for p in sorted(set(ps)):
        if args.template:
            tm.tilemix_template_route_words(args.template, int(round(p * 1000)), 2026, cu, w.max_seqlen,
                                            w.num_kv_heads, w.g, route_words=words, stream=stream)
        else:
            tr = torch.from_numpy(route_bernoulli_groups(w.cfg_id, w.num_kv_heads, [int(x) for x in w.lengths],
                                                         w.T, w.g, p)).to(dev)
            tm.tilemix_build_route_mask(tr, cu, w.max_seqlen, w.g, words, stream=stream)
        work = work_model(w, words.cpu().numpy().view(np.uint64))
        out = torch.empty((N, Hq, d), dtype=torch.float32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if w.kv_int8:
            plan32.run_planned(q, k_q, v_q, q_q, q_s, None, k_s, cu, words, out, v_scale=v_s, stream=stream)
        else:
            plan32.run_planned(q, k, v, q_q, q_s, k_q, k_s, cu, words, out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        if ref is None:
            ref = out
        diff = (out - ref).abs()
        res = {"deviation_sweep": w.name, "routing": args.template or "bernoulli", "p": p, "int8_pair_fraction": work["pairs_int8"] / work["pairs"],
               "max_diff": float(diff.max()), "mean_diff": float(diff.double().mean()),
               "reference": "same inputs at 0 % INT8 (all tiles FP16)", "attn_ms_fp32_out": e0.elapsed_time(e1)}
        del diff
        print(json.dumps(res), flush=True)


def chunked_work(w, words):
    """Legal (query, key) pairs of a chunked-prefill / decode call per route: the
    queries are the last Lq of Lk positions (key j legal for query i iff
    j <= Lk - Lq + i), counted exactly per score tile from the route words."""
    G = w.num_q_heads // w.num_kv_heads
    pairs16 = pairs8 = 0
    for b, (Lq, Lk) in enumerate(zip(w.lengths, w.lengths_k)):
        Lq, Lk, off = int(Lq), int(Lk), int(Lk) - int(Lq)
        for m in range((Lq + 63) // 64):
            i = np.arange(64 * m, min(64 * m + 64, Lq))
            last = off + i                                   # last legal key of each row
            for n in range((int(last.max())) // 64 + 1):
                cnt = int(np.clip(np.minimum(last, min(64 * n + 63, Lk - 1)) - 64 * n + 1, 0, None).sum())
                for hk in range(w.num_kv_heads):
                    if (int(words[hk, b, m]) >> (n // w.g)) & 1:
                        pairs8 += G * cnt
                    else:
                        pairs16 += G * cnt
    d = w.head_dim
    f_qk16, f_qk8, f_pv = 2 * d * pairs16, 2 * d * pairs8, 2 * d * (pairs16 + pairs8)
    return dict(pairs=pairs16 + pairs8, pairs_int8=pairs8, ops=f_qk16 + f_qk8 + f_pv,
                t_star=f_qk16 / P_FP16 + f_qk8 / P_INT8 + f_pv / P_FP16)


def chunked_bench(args):
    """Chunked prefill or decode over a resident INT8 KV cache (the cache is
    quantised once, when written; a step quantises the new queries, packs their
    route words, plans and runs the attention)."""
    import torch
    from mixed_precision_amd import tilemix as tm
    from workloads import make_chunked_workload
    dev = torch.device("cuda:0")
    p = 0.75 if args.p is None else args.p
    if args.chunked == "prefill":
        w = make_chunked_workload(6, lengths_q=[512] * 8, lengths_k=[4096] * 8, num_q_heads=24, num_kv_heads=8,
                                  head_dim=128, g=1, p=p, outliers=True, kv_int8=True,
                                  name="chunk512_over_kv4096_B8_h24kv8_d128_int8kv")
    else:
        w = make_chunked_workload(7, lengths_q=[1] * 64, lengths_k=[4096] * 64, num_q_heads=24, num_kv_heads=8,
                                  head_dim=128, g=1, p=p, outliers=True, kv_int8=True,
                                  name="decode_B64_kv4096_h24kv8_d128_int8kv")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    cu_k = torch.from_numpy(w.cu_seqlens_k).to(dev)
    tr = torch.from_numpy(w.tile_route).to(dev)
    N, Hq, d = w.q.shape
    Hk, B = w.num_kv_heads, w.batch
    k8, k_s = tm.tilemix_quantize_blockwise(k, cu_k, w.max_seqlen_k, 64)      # the resident INT8 cache
    v8, v_s = tm.tilemix_quantize_blockwise(v, cu_k, w.max_seqlen_k, 64)
    if args.kv_layout == "head":
        # head-major storage ([Hk][N][d], viewed as [N][Hk][d] through strides): a KV head's rows are contiguous,
        # as in paged caches that keep each head's block of tokens together
        k8 = k8.transpose(0, 1).contiguous().transpose(0, 1)
        v8 = v8.transpose(0, 1).contiguous().transpose(0, 1)
    nbq = (w.max_seqlen + w.blk_q - 1) // w.blk_q
    q_q = torch.empty((N, Hq, d), dtype=torch.int8, device=dev)
    q_s = torch.empty((Hq, B, nbq), dtype=torch.float32, device=dev)
    words = torch.empty((Hk, B, w.T), dtype=torch.int64, device=dev)
    out = torch.empty((N, Hq, d), dtype=torch.float16, device=dev)
    plan = tm.AttnPlan(tm.AttnProblem(B, w.max_seqlen, Hq, Hk, d, w.g, w.blk_q, w.sm_scale, True, False, False,
                                      w.max_seqlen_k), dev)
    stream = torch.cuda.current_stream()
    kw = dict(cu_seqlens_k=cu_k, max_seqlen_k=w.max_seqlen_k)
    tm.tilemix_build_route_mask(tr, cu, w.max_seqlen, w.g, words, stream=stream, **kw)
    work = chunked_work(w, words.cpu().numpy().view(np.uint64))

    side = torch.cuda.Stream(device=dev)

    def step(ev=None, stream=stream):
        if args.chunked == "prefill":            # the work list on a second stream, beside Q and the routes
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                plan.schedule(cu, stream=side, cu_seqlens_k=cu_k)
        tm.tilemix_quantize_blockwise(q, cu, w.max_seqlen, w.blk_q, q_q, q_s, stream=stream)
        tm.tilemix_build_route_mask(tr, cu, w.max_seqlen, w.g, words, stream=stream, **kw)
        if args.chunked == "prefill":
            stream.wait_stream(side)
        if ev is not None:
            ev[0].record(stream)
        if args.chunked == "prefill":
            plan.run_planned(q, k8, v8, q_q, q_s, None, k_s, cu, words, out, v_scale=v_s, stream=stream,
                             cu_seqlens_k=cu_k)
        else:   # one call: decode needs no work list, and the library skips building it
            plan.run(q, k8, v8, q_q, q_s, None, k_s, cu, words, out, v_scale=v_s, stream=stream, cu_seqlens_k=cu_k)
        if ev is not None:
            ev[1].record(stream)

    settle = settle_clocks(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    eager_ms = ms_per_step
    if args.graph:
        # the step's launches captured once in a HIP graph and replayed: no per-launch host work
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(stream=torch.cuda.current_stream())
        settle_graph = settle_clocks(lambda: g.replay(), args.settle_ms)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        settle = {"eager": settle, "graph": settle_graph}
    t_attn = float(np.mean(attn_ms)) * 1e-3
    # bytes every operand once: the INT8 cache (K8, V8 and their scales), fp16 Q, its int8 copy and scales,
    # route words, fp16 output
    kv_bytes = 2 * int(w.cu_seqlens_k[-1]) * Hk * d + 2 * 4 * Hk * B * w.T_k
    q_bytes = N * Hq * d * (2 + 1) + 4 * Hq * B * nbq + 8 * Hk * B * w.T
    bytes_ = kv_bytes + q_bytes + 2 * N * Hq * d
    res = {"metric": f"chunked {args.chunked} over an INT8 KV cache: new tokens/s", "value": N / (ms_per_step * 1e-3),
           "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
           "higher_is_better": True, "data": "synthetic", "hip_graph": bool(args.graph), "ms_per_step_eager": eager_ms,
           "config": {"workload": w.name, "batch": B, "query_tokens": N, "kv_layout": args.kv_layout, "keys_per_sequence": int(w.lengths_k[0]),
                      "num_q_heads": Hq, "num_kv_heads": Hk, "head_dim": d, "int8_pair_fraction":
                      work["pairs_int8"] / work["pairs"]},
           "attn_ms": float(np.mean(attn_ms)), "attn_ms_min": float(np.min(attn_ms)), "settle": settle,
           "roofline_mfma": {"achieved": work["ops"] / t_attn / 1e12, "peak": work["ops"] / work["t_star"] / 1e12,
                             "unit": "TFLOP/s", "frac": work["t_star"] / t_attn},
           "roofline_hbm": {"achieved": bytes_ / t_attn / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": bytes_ / t_attn / HBM_PEAK, "algorithmic_bytes": bytes_}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--p", type=float, default=None, help="INT8 coverage override (configs 2, 4, 5)")
    ap.add_argument("--head-dim", type=int, default=None, choices=[64, 128],
                    help="re-shape configs 2-5 to this head dimension (same lengths, heads, routes, seeds)")
    ap.add_argument("--otf", action="store_true",
                    help="on-the-fly quantisation: Q/K INT8 operands made inside the attention kernel "
                         "(no quantiser calls in the step)")
    ap.add_argument("--once", action="store_true",
                    help="quantise-once operands: the step quantises Q and K before the attention kernel "
                         "(default for an fp16 K/V: Q's operands made inside the kernel, K quantised once)")
    ap.add_argument("--deviation-sweep", type=str, default=None, metavar="P,P,...",
                    help="instead of the bench line: MaxDiff / MeanDiff of the routed output against the "
                         "0 %% INT8 output at each INT8 coverage (Bernoulli-routed workloads), one JSON line each")
    ap.add_argument("--template", type=str, default=None,
                    help="with --deviation-sweep: route by a static template (band, global, row_random, "
                         "aligned_sparse, bigbird, sptrans) instead of Bernoulli tile groups")
    ap.add_argument("--chunked", choices=["prefill", "decode"], default=None,
                    help="instead of the bench line: chunked prefill (512 new tokens over 4096 cached, batch 8) "
                         "or decode (1 new token over 4096 cached, batch 64) on an INT8 KV cache")
    ap.add_argument("--kv-layout", choices=["token", "head"], default="token",
                    help="with --chunked: INT8 cache stored token-major [N][Hk][d] or head-major [Hk][N][d]")
    ap.add_argument("--eager", action="store_true",
                    help="launch the step directly instead of replaying it as a captured HIP graph")
    ap.add_argument("--graph", action="store_true", help="(the default) replay the step as a captured HIP graph")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="before the warm-up steps, run the step untimed for this many ms of wall time so the GPU "
                         "clocks reach their sustained level (0: off); reported in the JSON line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device a few times (calibrates HBM byte counters) and exit")
    args = ap.parse_args()
    args.graph = not args.eager
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the path has no multi-GPU mode (it would "
              "shard by KV head, each GPU taking its heads' K/V, route words and query heads, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return
    if args.chunked:
        chunked_bench(args)
        return
    from mixed_precision_amd import tilemix as tm
    from workloads import config

    dev = torch.device("cuda:0")
    w = config(args.config, p=args.p, head_dim=args.head_dim)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    cu = torch.from_numpy(w.cu_seqlens).to(dev)
    tr = torch.from_numpy(w.tile_route).to(dev)
    N, Hq, d = w.q.shape
    Hk = w.num_kv_heads
    B = w.batch
    if args.otf and w.kv_int8:
        print("--otf applies to an fp16 K/V workload", file=sys.stderr)
        sys.exit(2)
    if args.otf and args.once:
        print("--otf and --once are exclusive", file=sys.stderr)
        sys.exit(2)
    # operand preparation (otf_quant): 0 quantise-once, 1 Q and K on chip, 2 Q on chip
    mode = 1 if args.otf else (0 if (args.once or w.kv_int8) else 2)
    plan = tm.AttnPlan(tm.AttnProblem(B, w.max_seqlen, Hq, Hk, d, w.g, w.blk_q, w.sm_scale, w.kv_int8, False,
                                      mode), dev)
    nbq = (w.max_seqlen + w.blk_q - 1) // w.blk_q
    T = w.T
    q_q = torch.empty((N, Hq, d), dtype=torch.int8, device=dev)
    q_s = torch.empty((Hq, B, nbq), dtype=torch.float32, device=dev)
    k_q = torch.empty((N, Hk, d), dtype=torch.int8, device=dev)
    k_s = torch.empty((Hk, B, T), dtype=torch.float32, device=dev)
    v_q = torch.empty((N, Hk, d), dtype=torch.int8, device=dev) if w.kv_int8 else None
    v_s = torch.empty((Hk, B, T), dtype=torch.float32, device=dev) if w.kv_int8 else None
    words = torch.empty((Hk, B, T), dtype=torch.int64, device=dev)
    out = torch.empty((N, Hq, d), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    if args.deviation_sweep:
        deviation_sweep(args, w, plan, q, k, v, cu, q_q, q_s, k_q, k_s, v_q, v_s, words, stream)
        return
    tm.tilemix_build_route_mask(tr, cu, w.max_seqlen, w.g, words, stream=stream)
    work = work_model(w, words.cpu().numpy().view(np.uint64))

    # The route words and the work list depend only on the routing template and
    # cu_seqlens: they are built on a second stream (default priority) beside the
    # quantiser, and the attention waits for both.  (Quantising K on a third
    # stream beside Q measured no faster: both are HBM-bound, and each
    # cross-stream wait costs several microseconds.)
    side = torch.cuda.Stream(device=dev)

    def step(ev=None, stream=stream):
        side.wait_stream(stream)                 # the previous step's attention has read words / work list
        with torch.cuda.stream(side):
            tm.tilemix_build_route_mask(tr, cu, w.max_seqlen, w.g, words, stream=side)
            plan.schedule(cu, stream=side)
        if mode == 0:
            tm.tilemix_quantize_blockwise(q, cu, w.max_seqlen, w.blk_q, q_q, q_s, stream=stream)
        if mode != 1:
            tm.tilemix_quantize_blockwise(k, cu, w.max_seqlen, 64, k_q, k_s, stream=stream)
        if w.kv_int8:
            tm.tilemix_quantize_blockwise(v, cu, w.max_seqlen, 64, v_q, v_s, stream=stream)
        stream.wait_stream(side)
        if ev is not None:
            ev[0].record(stream)
        if w.kv_int8:
            plan.run_planned(q, k_q, v_q, q_q, q_s, None, k_s, cu, words, out, v_scale=v_s, stream=stream)
        elif mode == 1:
            plan.run_planned(q, k, v, None, None, None, None, cu, words, out, stream=stream)
        elif mode == 2:
            plan.run_planned(q, k, v, None, None, k_q, k_s, cu, words, out, stream=stream)
        else:
            plan.run_planned(q, k, v, q_q, q_s, k_q, k_s, cu, words, out, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    settle = settle_clocks(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    ms_per_step = wall * 1e3 / args.steps
    eager_ms = ms_per_step
    if args.graph:
        # the same step captured once in a HIP graph (the side stream forked
        # from and joined to the capture stream) and replayed
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(stream=torch.cuda.current_stream())
        # capture and instantiation leave the GPU idle: settle again before the replays
        settle_graph = settle_clocks(lambda: g.replay(), args.settle_ms)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        settle = {"eager": settle, "graph": settle_graph}
    t_attn = float(np.mean(attn_ms)) * 1e-3
    achieved = work["ops"] / t_attn
    blended_peak = work["ops"] / work["t_star"]
    tokens_per_s = N / (ms_per_step * 1e-3)

    res = {
        "metric": "prefill tokens/s & % blended MFMA peak, 3B-shaped GQA attn L=4K b=8 75% INT8",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16+int8 (fp32 accumulation / int32 accumulation)", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": w.max_seqlen, "num_q_heads": Hq, "num_kv_heads": Hk,
                   "head_dim": d, "g": w.g, "blk_q": w.blk_q, "kv_int8": w.kv_int8,
                   "operands": ("quantize-once", "on-the-fly", "on-the-fly Q")[mode],
                   "int8_pair_fraction": work["pairs_int8"] / work["pairs"], "tokens": N},
        "roofline": {"bound": "mfma", "achieved": achieved / 1e12, "peak": blended_peak / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / blended_peak,
                     "traffic": measured_traffic(w.name) if mode == 2 else None,
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE x2 + WRITE_SIZE x1, copy-calibrated), read from "
                                     "the committed rocprofv3 counter summary profiles/attn_prefill_kernel_llama3b_B8_"
                                     "L4096_hbm_bytes.md while its kernel-source digest matches the sources (else null)",
                     "kernel": attn_kernel_name(Hq // Hk, w.kv_int8),
                     "note": "peak = blended MFMA peak of this launch's mix: ops / (F_qk16/P16 + F_qk8/P8 + F_pv/P16)"},
        "attn_ms": float(np.mean(attn_ms)), "attn_ms_min": float(np.min(attn_ms)),
        "attn_tokens_per_s": N / t_attn, "t_star_ms": work["t_star"] * 1e3,
        "hip_graph": bool(args.graph), "ms_per_step_eager": eager_ms,
        "settle": settle,
    }
    if mode == 1:
        res["config"]["k_quant_on_chip"] = k_quant_cost(args, w, tm, dev, q, k, v, cu, words, work,
                                                        float(np.mean(attn_ms)))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)


def k_quant_cost(args, w, tm, dev, q, k, v, cu, words, work, attn_ms_otf):
    """Where on-the-fly K goes: the same attention with K quantised once
    beforehand (Q's operands still made in the kernel), timed in this process,
    and the extra time per on-chip quantisation of an INT8 key tile.  Each
    work item (query tile, KV head, chunk of up to three query heads) quantises
    every INT8 key tile it visits, between two barriers of its workgroup."""
    import torch
    B, Hq, Hk, d = len(w.lengths), w.num_q_heads, w.num_kv_heads, w.head_dim
    N = q.shape[0]
    plan = tm.AttnPlan(tm.AttnProblem(B, w.max_seqlen, Hq, Hk, d, w.g, w.blk_q, w.sm_scale, w.kv_int8, False, 2),
                       dev)
    k_q = torch.empty((N, Hk, d), dtype=torch.int8, device=dev)
    k_s = torch.empty((Hk, B, w.T), dtype=torch.float32, device=dev)
    out = torch.empty((N, Hq, d), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream()
    plan.schedule(cu, stream=stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tm.tilemix_quantize_blockwise(k, cu, w.max_seqlen, 64, k_q, k_s, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        plan.run_planned(q, k, v, None, None, k_q, k_s, cu, words, out, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    settle_clocks(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    kq_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    once_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    G = Hq // Hk
    chunks = -(-G // 3)                               # fp16 K/V: up to three query heads per item
    heads = -(-G // chunks)
    quants = work["visits8"] * chunks
    # resident workgroups (four waves each): the kernel's waves per SIMD times the CUs
    waves = 2 if d == 128 else (3 if heads == 3 else 4)
    slots = waves * torch.cuda.get_device_properties(dev).multi_processor_count
    extra = attn_ms_otf - once_ms
    return {"int8_tile_quantisations": quants, "distinct_int8_tiles": work["tiles8"],
            "repeats_per_tile": quants / max(work["tiles8"], 1),
            "attn_ms_k_quantised_once": once_ms, "k_quantiser_pass_ms": kq_ms,
            "attn_ms_extra": extra,
            "us_per_tile_quantisation_per_workgroup": extra * 1e3 * slots / max(quants, 1),
            "concurrent_workgroups": slots,
            "note": "attention with K quantised once (and its quantiser pass) timed in the same process; "
                    "extra time spread over the concurrent workgroups"}


if __name__ == "__main__":
    main()
