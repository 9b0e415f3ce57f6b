"""The oracle over many query-tile rows at once, in worker processes (test
infrastructure).

The oracle is plain single-threaded NumPy.  Comparing a full-size workload with
it, every row or thousands of sampled rows, takes minutes on one core, so the
rows are spread over worker processes.  Workers are started with "spawn": they
never inherit the parent's GPU state (and import no GPU library).  They read the
oracle inputs from .npy files, memory-mapped from a temporary directory the
parent writes once.
"""
from __future__ import annotations

import json
import multiprocessing as mp
import os
import shutil
import tempfile
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

import oracle as orc

_ARRAYS = ("q", "k", "v", "q_q", "q_scale", "k_q", "k_scale", "v_q", "v_scale", "words", "cu", "cu_k")
_INP: Optional[orc.AttnInputs] = None


def _save(inp: orc.AttnInputs, d: str) -> None:
    arrays = dict(q=inp.q, k=inp.k, v=inp.v, q_q=inp.q_q, q_scale=inp.q_scale, k_q=inp.k_q, k_scale=inp.k_scale,
                  v_q=inp.v_q, v_scale=inp.v_scale, words=inp.words, cu=inp.cu, cu_k=inp.cu_k)
    for name, a in arrays.items():
        if a is not None:
            np.save(os.path.join(d, name + ".npy"), np.ascontiguousarray(a))
    meta = dict(max_seqlen=inp.max_seqlen, max_seqlen_k=inp.max_seqlen_k, Hk=inp.Hk, g=inp.g, sm=inp.sm,
                blk_q=inp.blk_q, kv_int8=inp.kv_int8, chunked=bool(inp.pairs != [(L, L) for _, L in inp.spans]))
    with open(os.path.join(d, "meta.json"), "w") as f:
        json.dump(meta, f)


def _load(d: str) -> orc.AttnInputs:
    a = {}
    for name in _ARRAYS:
        p = os.path.join(d, name + ".npy")
        a[name] = np.load(p, mmap_mode="r") if os.path.exists(p) else None
    meta = json.load(open(os.path.join(d, "meta.json")))
    chunk = {}
    if meta["chunked"]:
        chunk = dict(cu_seqlens_k=np.asarray(a["cu_k"]), max_seqlen_k=meta["max_seqlen_k"])
    common = dict(q=a["q"], cu_seqlens=np.asarray(a["cu"]), max_seqlen=meta["max_seqlen"], num_kv_heads=meta["Hk"],
                  route_words=np.asarray(a["words"]), g=meta["g"], sm_scale=meta["sm"], q_q=a["q_q"],
                  q_scale=a["q_scale"], blk_q=meta["blk_q"], k_q=a["k_q"], k_scale=a["k_scale"], **chunk)
    if meta["kv_int8"]:
        return orc.AttnInputs(v_q=a["v_q"], v_scale=a["v_scale"], kv_int8=True, **common)
    return orc.AttnInputs(k=a["k"], v=a["v"], kv_int8=False, **common)


def _init(d: str) -> None:
    global _INP
    _INP = _load(d)


def _task(task: Tuple[int, int, Tuple[int, ...], bool]):
    b, hq, ms, with_lse = task
    if len(_INP._kv_cache) > 4:            # bound the per-worker float64 K/V copies
        _INP._kv_cache.clear()
    out = []
    for m in ms:
        r = orc.attn_tile_row(_INP, b, hq, m, with_lse=with_lse)
        out.append((b, hq, m, r))
    return out


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run(inp: orc.AttnInputs, tasks: List[Tuple[int, int, Tuple[int, ...], bool]], procs: Optional[int]):
    d = tempfile.mkdtemp(prefix="oracle_pool_")
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        _save(inp, d)
        for k in saved:                      # one BLAS thread per worker
            os.environ[k] = "1"
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs or workers(), initializer=_init, initargs=(d,)) as pool:
            res = []
            for part in pool.imap_unordered(_task, tasks):
                res.extend(part)
        return res
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        shutil.rmtree(d, ignore_errors=True)


def tile_rows(inp: orc.AttnInputs, samples: Iterable[Tuple[int, int, int]], with_lse: bool = False,
              procs: Optional[int] = None) -> Dict[Tuple[int, int, int], object]:
    """{(b, hq, m): oracle output rows of query tile m} for every sample
    (with_lse: (rows, lse) pairs), computed in worker processes."""
    by_head: Dict[Tuple[int, int], List[int]] = {}
    for b, hq, m in samples:
        by_head.setdefault((b, hq), []).append(m)
    tasks = []
    for (b, hq), ms in sorted(by_head.items()):
        ms = sorted(set(ms))
        for i in range(0, len(ms), 8):
            tasks.append((b, hq, tuple(ms[i:i + 8]), with_lse))
    return {(b, hq, m): r for b, hq, m, r in _run(inp, tasks, procs)}


def full_output(inp: orc.AttnInputs, procs: Optional[int] = None) -> np.ndarray:
    """The oracle's whole output, float64 [N][Hq][d] (attn_prefill, in worker processes)."""
    samples = [(b, hq, m) for b, (_, Lq) in enumerate(inp.spans) for hq in range(inp.Hq)
               for m in range(orc.num_tiles(Lq))]
    rows = tile_rows(inp, samples, procs=procs)
    N = int(inp.cu[-1])
    out = np.zeros((N, inp.Hq, inp.d))
    for (b, hq, m), r in rows.items():
        s0, Lq = inp.spans[b]
        out[s0 + m * orc.BLOCK_M:s0 + min(m * orc.BLOCK_M + orc.BLOCK_M, Lq), hq] = r
    return out
