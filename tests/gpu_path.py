"""Run a synthetic workload through the HIP library (via the binding) on cuda:0.

Every operand the attention call consumes is produced by the library itself
(quantiser, route packer); the oracle side builds its own from the same host
arrays, so the two share only the seeded inputs."""
from __future__ import annotations

import os

import numpy as np
import torch

from mixed_precision_amd import tilemix as tm
from workloads import Workload

DEV = "cuda:0"


def upload(w: Workload, dev=DEV):
    t = dict(q=torch.from_numpy(w.q).to(dev), k=torch.from_numpy(w.k).to(dev), v=torch.from_numpy(w.v).to(dev),
             cu=torch.from_numpy(w.cu_seqlens).to(dev), tile_route=torch.from_numpy(w.tile_route).to(dev))
    t["cu_k"] = None if w.cu_seqlens_k is None else torch.from_numpy(w.cu_seqlens_k).to(dev)
    return t


def _keys(w: Workload, t):
    """(key prefix sums, bound) for the quantiser: the keys' own in chunked prefill."""
    return (t["cu"], w.max_seqlen) if t.get("cu_k") is None else (t["cu_k"], w.max_seqlen_k)


def _chunk_kw(w: Workload, t):
    return {} if t.get("cu_k") is None else dict(cu_seqlens_k=t["cu_k"], max_seqlen_k=w.max_seqlen_k)


def prepare(w: Workload, dev=DEV, t=None):
    """Device tensors for one attention call, operands made by the library."""
    t = t or upload(w, dev)
    t.setdefault("cu_k", None)
    cu_k, max_k = _keys(w, t)
    t["q_q"], t["q_s"] = tm.tilemix_quantize_blockwise(t["q"], t["cu"], w.max_seqlen, w.blk_q)
    if w.kv_int8:
        t["k8"], t["k_s"] = tm.tilemix_quantize_blockwise(t["k"], cu_k, max_k, 64)
        t["v8"], t["v_s"] = tm.tilemix_quantize_blockwise(t["v"], cu_k, max_k, 64)
        t["k_q"] = None
    else:
        t["k_q"], t["k_s"] = tm.tilemix_quantize_blockwise(t["k"], cu_k, max_k, 64)
    t["words"] = tm.tilemix_build_route_mask(t["tile_route"], t["cu"], w.max_seqlen, w.g, **_chunk_kw(w, t))
    return t


def attn(w: Workload, t, out_fp32=True, plan=None, out=None, otf=False, lse=None):
    ck = _chunk_kw(w, t)
    if otf == 2:   # on-the-fly Q: fp16 q, K quantised once
        return tm.tilemix_attn_prefill(t["q"], t["k"], t["v"], k_q=t["k_q"], k_scale=t["k_s"], cu_seqlens=t["cu"],
                                       route_words=t["words"], max_seqlen=w.max_seqlen, g=w.g, blk_q=w.blk_q,
                                       sm_scale=w.sm_scale, out_fp32=out_fp32, otf_quant=2, plan=plan, out=out,
                                       lse=lse, **ck)
    if otf:   # on-the-fly quantisation: only fp16 q, k, v, the route words and cu_seqlens
        return tm.tilemix_attn_prefill(t["q"], t["k"], t["v"], cu_seqlens=t["cu"], route_words=t["words"],
                                       max_seqlen=w.max_seqlen, g=w.g, blk_q=w.blk_q, sm_scale=w.sm_scale,
                                       out_fp32=out_fp32, otf_quant=True, plan=plan, out=out, lse=lse, **ck)
    if w.kv_int8:
        return tm.tilemix_attn_prefill(t["q"], t["k8"], t["v8"], q_q=t["q_q"], q_scale=t["q_s"], k_q=None,
                                       k_scale=t["k_s"], v_scale=t["v_s"], kv_int8=True, cu_seqlens=t["cu"],
                                       route_words=t["words"], max_seqlen=w.max_seqlen, g=w.g, blk_q=w.blk_q,
                                       sm_scale=w.sm_scale, out_fp32=out_fp32, plan=plan, out=out, lse=lse, **ck)
    return tm.tilemix_attn_prefill(t["q"], t["k"], t["v"], q_q=t["q_q"], q_scale=t["q_s"], k_q=t["k_q"],
                                   k_scale=t["k_s"], cu_seqlens=t["cu"], route_words=t["words"],
                                   max_seqlen=w.max_seqlen, g=w.g, blk_q=w.blk_q, sm_scale=w.sm_scale,
                                   out_fp32=out_fp32, plan=plan, out=out, lse=lse, **ck)


def attn_debug(w: Workload, t, seq=0, q_head=0, m_begin=0, m_end=None, otf=False):
    kw = dict(q_q=t["q_q"], q_scale=t["q_s"], k_scale=t["k_s"], cu_seqlens=t["cu"], route_words=t["words"],
              max_seqlen=w.max_seqlen, g=w.g, blk_q=w.blk_q, sm_scale=w.sm_scale, seq=seq, q_head=q_head,
              m_begin=m_begin, m_end=m_end, **_chunk_kw(w, t))
    if otf == 2:
        kw.update(q_q=None, q_scale=None, otf_quant=2)
        return tm.tilemix_attn_prefill_debug(t["q"], t["k"], t["v"], k_q=t["k_q"], **kw)
    if otf:
        kw.update(q_q=None, q_scale=None, k_scale=None, otf_quant=True)
        return tm.tilemix_attn_prefill_debug(t["q"], t["k"], t["v"], **kw)
    if w.kv_int8:
        return tm.tilemix_attn_prefill_debug(t["q"], t["k8"], t["v8"], k_q=None, v_scale=t["v_s"], kv_int8=True, **kw)
    return tm.tilemix_attn_prefill_debug(t["q"], t["k"], t["v"], k_q=t["k_q"], **kw)


def words_u64(words: torch.Tensor) -> np.ndarray:
    return words.cpu().numpy().view(np.uint64)


# (test id, max-abs error, relative Frobenius error) of every comparison made
# through errors(); the session prints them as a margin table at the end
MARGINS = []


def record(ma: float, rf: float, label: str = "") -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::")[-1]
    MARGINS.append((test + (f" [{label}]" if label else ""), ma, rf))


def errors(got: np.ndarray, ref: np.ndarray, label: str = ""):
    got = got.astype(np.float64)
    diff = got - ref
    ma, rf = float(np.max(np.abs(diff))), float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    record(ma, rf, label)
    return ma, rf
