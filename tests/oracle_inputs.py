"""Build oracle inputs for a synthetic workload using only the oracle's own
quantiser and mask packer (no value ever comes from the GPU path)."""
from __future__ import annotations

import numpy as np

import oracle as orc
from workloads import Workload


def oracle_inputs(w: Workload, route_words=None, with_int8: bool = True) -> orc.AttnInputs:
    cu_k = w.cu_seqlens if w.cu_seqlens_k is None else w.cu_seqlens_k
    max_k = w.max_seqlen if w.max_seqlen_k is None else w.max_seqlen_k
    chunk = dict(cu_seqlens_k=w.cu_seqlens_k, max_seqlen_k=w.max_seqlen_k)
    if route_words is None:
        route_words = orc.build_route_mask(w.tile_route, w.cu_seqlens, w.max_seqlen, w.g, **chunk)
    q_q = q_scale = k_q = k_scale = v_q = v_scale = None
    if with_int8 or w.kv_int8:
        q_q, q_scale = orc.quantize_blockwise(w.q, w.cu_seqlens, w.max_seqlen, w.blk_q)
        k_q, k_scale = orc.quantize_blockwise(w.k, cu_k, max_k, 64)
    if w.kv_int8:
        v_q, v_scale = orc.quantize_blockwise(w.v, cu_k, max_k, 64)
        return orc.AttnInputs(q=w.q, cu_seqlens=w.cu_seqlens, max_seqlen=w.max_seqlen,
                              num_kv_heads=w.num_kv_heads, route_words=route_words, g=w.g,
                              sm_scale=w.sm_scale, q_q=q_q, q_scale=q_scale, blk_q=w.blk_q,
                              k_q=k_q, k_scale=k_scale, v_q=v_q, v_scale=v_scale, kv_int8=True, **chunk)
    return orc.AttnInputs(q=w.q, cu_seqlens=w.cu_seqlens, max_seqlen=w.max_seqlen,
                          num_kv_heads=w.num_kv_heads, route_words=route_words, g=w.g,
                          sm_scale=w.sm_scale, q_q=q_q, q_scale=q_scale, blk_q=w.blk_q,
                          k=w.k, v=w.v, k_q=k_q, k_scale=k_scale, kv_int8=False, **chunk)


def words_from_group_bits(bits_fn, num_kv_heads, cu_seqlens, max_seqlen, g):
    """uint64 words straight from a per-(hk, b, m, j) bit function (test helper)."""
    T = orc.num_tiles(max_seqlen)
    spans = orc.seq_spans(cu_seqlens)
    words = np.zeros((num_kv_heads, len(spans), T), dtype=np.uint64)
    for hk in range(num_kv_heads):
        for b, (_, L) in enumerate(spans):
            for m in range(orc.num_tiles(L)):
                w = 0
                for j in range(m // g + 1):
                    if bits_fn(hk, b, m, j):
                        w |= 1 << j
                words[hk, b, m] = np.uint64(w)
    return words
