"""CPU checks of the benchmark's work models: the legal (query, key) pairs per
path that set the blended MFMA roofline (prefill, and chunked prefill / decode),
and the INT8 tile visits that the on-the-fly line reports, against brute force
over every pair of small ragged GQA batches with route words from the oracle's
packer."""
import numpy as np
import pytest

import bench
from oracle.tilemix_oracle import build_route_mask, route_bit
from workloads.synth import make_workload


@pytest.mark.parametrize("g,p", [(1, 0.5), (2, 0.7), (3, 0.0), (1, 1.0)])
def test_work_model_matches_brute_force(g, p):
    w = make_workload(611 + g, lengths=[130, 64, 1, 200], num_q_heads=6, num_kv_heads=2, head_dim=64, g=g, p=p)
    words = build_route_mask(w.tile_route, w.cu_seqlens, w.max_seqlen, g)
    G = w.num_q_heads // w.num_kv_heads
    pairs8 = pairs16 = 0
    visits8, tiles8 = 0, set()
    for b, L in enumerate(w.lengths):
        for hk in range(w.num_kv_heads):
            for m in range((L + 63) // 64):
                # a work item per (sequence, KV head, query tile): each INT8 key tile it visits
                for n in range(m + 1):
                    if route_bit(words[hk, b, m], n, g):
                        visits8 += 1
                        tiles8.add((b, hk, n))
            for i in range(L):
                m = i // 64
                bits = np.array([route_bit(words[hk, b, m], j // 64, g) for j in range(i + 1)])
                pairs8 += G * int(bits.sum())
                pairs16 += G * int((1 - bits).sum())
    got = bench.work_model(w, words)
    assert got["pairs"] == pairs8 + pairs16 == w.num_q_heads * bench.legal_pairs(w.lengths)
    assert got["pairs_int8"] == pairs8
    assert got["visits8"] == visits8 and got["tiles8"] == len(tiles8)
    d = w.head_dim
    assert got["f_qk8"] == 2 * d * pairs8 and got["f_qk16"] == 2 * d * pairs16
    assert got["f_pv"] == 2 * d * (pairs8 + pairs16)
    t_star = (2 * d * pairs16 / bench.P_FP16 + 2 * d * pairs8 / bench.P_INT8 +
              2 * d * (pairs8 + pairs16) / bench.P_FP16)
    assert got["t_star"] == pytest.approx(t_star, rel=1e-12)
    if p == 0.0:
        assert pairs8 == 0 and visits8 == 0
    if p == 1.0:
        assert pairs16 == 0


@pytest.mark.parametrize("g", [1, 2])
def test_chunked_work_model_matches_brute_force(g):
    """Chunked prefill and decode: the queries are the last Lq of Lk positions
    (key j legal for query i iff j <= Lk - Lq + i); pairs per path against
    every pair, including one-query rows and chunks that start inside a tile."""
    from workloads.synth import make_chunked_workload
    w = make_chunked_workload(620 + g, lengths_q=[130, 1, 64, 7], lengths_k=[300, 200, 64, 70], num_q_heads=4,
                              num_kv_heads=2, head_dim=64, g=g, p=0.6)
    words = build_route_mask(w.tile_route, w.cu_seqlens, w.max_seqlen, g, w.cu_seqlens_k, w.max_seqlen_k)
    G = w.num_q_heads // w.num_kv_heads
    pairs8 = pairs16 = 0
    for b, (Lq, Lk) in enumerate(zip(w.lengths, w.lengths_k)):
        for hk in range(w.num_kv_heads):
            for i in range(Lq):
                for j in range(Lk - Lq + i + 1):
                    if route_bit(words[hk, b, i // 64], j // 64, g):
                        pairs8 += G
                    else:
                        pairs16 += G
    got = bench.chunked_work(w, words)
    assert got["pairs_int8"] == pairs8 and got["pairs"] == pairs8 + pairs16
    d = w.head_dim
    assert got["t_star"] == pytest.approx(2 * d * pairs16 / bench.P_FP16 + 2 * d * pairs8 / bench.P_INT8 +
                                          2 * d * (pairs8 + pairs16) / bench.P_FP16, rel=1e-12)
