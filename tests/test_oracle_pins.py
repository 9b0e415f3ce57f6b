"""Pins of the CPU oracle against things other than itself: a library routine,
closed forms, invariants, exact rational arithmetic, brute force on tiny inputs
and figures printed on the pages.  CPU only."""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as orc
from workloads import config, make_workload, make_chunked_workload, cu_from_lengths, legal_tile_matrix
from tests.oracle_inputs import oracle_inputs, words_from_group_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small(lengths, hq=2, hk=1, d=64, g=1, p=0.5, route="bernoulli", cfg=101, outliers=False,
           kv_int8=False, blk_q=64):
    return make_workload(cfg, lengths=lengths, num_q_heads=hq, num_kv_heads=hk, head_dim=d, g=g,
                         route=route, p=p, outliers=outliers, kv_int8=kv_int8, blk_q=blk_q)


# ---------------------------------------------------------------- pin A
@pytest.mark.parametrize("lengths,hq,hk,d", [([200], 2, 1, 64), ([70, 130, 1], 3, 1, 128), ([129, 64], 4, 2, 64)])
def test_pin_A_zero_mask_equals_torch_sdpa(lengths, hq, hk, d):
    """All-FP16 routing reduces to textbook causal attention: compare with
    torch's scaled_dot_product_attention in float64 (an independent routine,
    including its own GQA head mapping)."""
    w = _small(lengths, hq=hq, hk=hk, d=d, route="zeros")
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
        q = torch.from_numpy(w.q[s0:s0 + L].astype(np.float64)).permute(1, 0, 2)[None]
        k = torch.from_numpy(w.k[s0:s0 + L].astype(np.float64)).permute(1, 0, 2)[None]
        v = torch.from_numpy(w.v[s0:s0 + L].astype(np.float64)).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, is_causal=True, scale=float(np.float32(w.sm_scale)), enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        got = out[s0:s0 + L]
        assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


# ---------------------------------------------------------------- pin B
@pytest.mark.parametrize("seed,lengths,g", [(102, [300], 1), (103, [257, 64, 5], 2), (104, [640], 4)])
def test_pin_B_streaming_equals_two_pass(seed, lengths, g):
    """Streaming online softmax over routed scores equals a materialised two-pass
    softmax over the same routed scores."""
    w = _small(lengths, hq=2, hk=1, d=64, g=g, p=0.5, cfg=seed, outliers=True)
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for hq in range(w.num_q_heads):
            ref = orc.attn_dense_two_pass(inp, b, hq)
            got = out[s0:s0 + L, hq]
            rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
            assert rel <= 1e-12, rel


# ---------------------------------------------------------------- pin C
def test_pin_C_visit_matrix_is_legality():
    lengths = [1, 64, 65, 300]
    cu = cu_from_lengths(lengths)
    vis = orc.visit_matrix(cu, 300, 3)
    T = orc.num_tiles(300)
    for b, L in enumerate(lengths):
        Tb = -(-L // 64)
        assert int(vis[b, 0].sum()) == Tb * (Tb + 1) // 2       # closed form
        for m in range(T):
            for n in range(T):
                assert vis[b, 1, m, n] == (1 if (n <= m and m < Tb) else 0)


# ---------------------------------------------------------------- pin D
@pytest.mark.parametrize("g", [2, 4, 16])
def test_pin_D_grouping_equivalence(g):
    """Tile routes constant within groups: words packed at g = 1 and at g > 1
    decode to the same tile routes and give a bit-identical output."""
    L = 64 * 37 + 11 if g == 16 else 64 * 9 + 3
    w = _small([L], hq=2, hk=1, d=64, g=g, p=0.5, cfg=110 + g)   # group-constant by construction
    tr = w.tile_route
    w1 = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, 1)
    wg = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, g)
    d1 = orc.decode_route_mask(w1, w.cu_seqlens, w.max_seqlen, 1)
    dg = orc.decode_route_mask(wg, w.cu_seqlens, w.max_seqlen, g)
    assert np.array_equal(d1, dg)
    w.g = 1
    o1 = orc.attn_prefill(oracle_inputs(w, route_words=w1))
    w.g = g
    og = orc.attn_prefill(oracle_inputs(w, route_words=wg))
    assert np.array_equal(o1, og)


# ---------------------------------------------------------------- pin E
@pytest.mark.parametrize("L,d", [(1, 64), (2, 64), (63, 64), (64, 64), (65, 64), (127, 64), (128, 64),
                                 (129, 64), (130, 64), (65, 128), (130, 128)])
def test_pin_E_brute_force_tiny(L, d):
    w = _small([L], hq=1, hk=1, d=d, p=0.5, cfg=200 + L + d, outliers=True)
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    bf = np.array(orc.attn_brute_force(inp, 0, 0))
    assert np.max(np.abs(out[:, 0] - bf)) <= 1e-12


def test_pin_E_brute_force_mixed_batch_gqa():
    w = _small([1, 65, 130, 64], hq=4, hk=2, d=64, p=0.5, cfg=230, outliers=True)
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for hq in (0, 3):
            bf = np.array(orc.attn_brute_force(inp, b, hq))
            assert np.max(np.abs(out[s0:s0 + L, hq] - bf)) <= 1e-12


def test_pin_E_all_masks_T3():
    """T = 3 has 6 legal tiles: every one of the 2^6 tile masks, streaming vs
    materialised two-pass; four of them also against plain-Python brute force."""
    L = 130
    w = _small([L], hq=1, hk=1, d=64, cfg=240, outliers=True)
    legal = [(m, n) for m in range(3) for n in range(m + 1)]
    for idx, bits in enumerate(itertools.product([0, 1], repeat=len(legal))):
        tr = np.zeros_like(w.tile_route)
        for (m, n), bit in zip(legal, bits):
            tr[0, 0, m, n] = bit
        words = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, 1)
        inp = oracle_inputs(w, route_words=words)
        out = orc.attn_prefill(inp)[:, 0]
        ref = orc.attn_dense_two_pass(inp, 0, 0)
        assert np.max(np.abs(out - ref)) <= 1e-12
        if idx in (0, 21, 42, 63):
            bf = np.array(orc.attn_brute_force(inp, 0, 0))
            assert np.max(np.abs(out - bf)) <= 1e-12


# ---------------------------------------------------------------- pin F
def _lossless_operand(rng, shape, blk, cu):
    """Values j * 2^-6 with integer |j| <= 127 and a 127 in every (sequence,
    block, head): INT8 quantisation is then exact (scale = 2^-6, q = j)."""
    j = rng.integers(-127, 128, size=shape)
    for s0, L in orc.seq_spans(cu):
        for b0 in range(0, L, blk):
            j[s0 + b0, :, 0] = 127 * (1 if rng.random() < 0.5 else -1)
    return (j.astype(np.float64) * 2.0 ** -6).astype(np.float16), j


def test_pin_F_lossless_int8_mask_independent():
    rng = np.random.default_rng(7)
    w = _small([200, 77], hq=2, hk=1, d=64, cfg=250)
    q, jq = _lossless_operand(rng, w.q.shape, 64, w.cu_seqlens)
    k, jk = _lossless_operand(rng, w.k.shape, 64, w.cu_seqlens)
    w.q, w.k = q, k
    qq, qs = orc.quantize_blockwise(q, w.cu_seqlens, w.max_seqlen, 64)
    kq, ks = orc.quantize_blockwise(k, w.cu_seqlens, w.max_seqlen, 64)
    assert np.array_equal(qq.astype(np.int64), jq) and np.array_equal(kq.astype(np.int64), jk)
    used = [orc.num_tiles(L) for _, L in orc.seq_spans(w.cu_seqlens)]
    for h in range(2):
        for b, nb in enumerate(used):
            assert np.all(qs[h, b, :nb] == np.float32(2.0 ** -6))
    outs = []
    for p in (0.0, 0.3, 1.0):
        tr = _small([200, 77], hq=2, hk=1, d=64, cfg=251 + int(10 * p), p=p).tile_route
        words = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, 1)
        outs.append(orc.attn_prefill(oracle_inputs(w, route_words=words)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ---------------------------------------------------------------- pin G
def test_pin_G_closed_forms():
    w = _small([1, 150, 64], hq=2, hk=1, d=64, p=0.6, cfg=260, outliers=True)
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    for s0, L in orc.seq_spans(w.cu_seqlens):
        # the first query of a sequence sees only its own key: O = V[0]
        assert np.array_equal(out[s0, 0], w.v[s0, 0].astype(np.float64))
    # Q == 0: every score is 0 on both paths, O_i = mean of V[0..i]
    w0 = _small([150], hq=1, hk=1, d=64, p=0.5, cfg=261)
    w0.q[:] = 0
    out0 = orc.attn_prefill(oracle_inputs(w0))
    vf = w0.v[:, 0].astype(np.float64)
    ref = np.cumsum(vf, axis=0) / np.arange(1, 151)[:, None]
    assert np.max(np.abs(out0[:, 0] - ref)) <= 1e-13
    # V constant per channel: O = V
    wc = _small([150], hq=1, hk=1, d=64, p=0.5, cfg=262, outliers=True)
    wc.v[:] = wc.v[0:1]
    outc = orc.attn_prefill(oracle_inputs(wc))
    assert np.max(np.abs(outc[:, 0] - wc.v[0, 0].astype(np.float64))) <= 1e-13


def test_pin_G_kv_int8_row0_is_dequantised_v():
    w = _small([100], hq=2, hk=1, d=64, p=0.5, cfg=263, kv_int8=True)
    inp = oracle_inputs(w)
    out = orc.attn_prefill(inp)
    ref = inp.v_q[0, 0].astype(np.float64) * float(inp.v_scale[0, 0, 0])
    assert np.array_equal(out[0, 0], ref)


# ---------------------------------------------------------------- pin E, INT8 KV cache
def _kv_blocks_scaled(w, rng):
    """Scale K and V of every (sequence, 64-key block, KV head) by its own factor
    e^u, u ~ U(-4, 4), before quantisation, so the per-block scales of one
    sequence spread over more than three orders of magnitude: a scale looked up
    in the wrong block then moves the result far outside the tolerance."""
    cu_k = w.cu_seqlens if w.cu_seqlens_k is None else w.cu_seqlens_k
    for s0, L in orc.seq_spans(cu_k):
        for b0 in range(0, L, 64):
            r0, r1 = s0 + b0, s0 + min(b0 + 64, L)
            for arr in (w.k, w.v):
                f = np.exp(rng.uniform(-4.0, 4.0, size=(1, arr.shape[1], 1)))
                arr[r0:r1] = (arr[r0:r1].astype(np.float64) * f).astype(np.float16)


def _check_kv_int8_brute_force(w, inp):
    out, lse = orc.attn_prefill(inp, with_lse=True)
    routes = set()
    for b, (s0, Lq) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for hq in range(w.num_q_heads):
            bf, bl = orc.attn_brute_force(inp, b, hq, with_lse=True)
            bf, bl = np.array(bf), np.array(bl)
            tol = 1e-12 * max(1.0, float(np.max(np.abs(bf))))
            assert np.max(np.abs(out[s0:s0 + Lq, hq] - bf)) <= tol
            assert np.max(np.abs(lse[s0:s0 + Lq, hq] - bl)) <= 1e-12 * max(1.0, float(np.max(np.abs(bl))))
            hk = inp.kv_head(hq)
            for m in range(orc.num_tiles(Lq)):
                for n in range(orc.last_key_tile(m, *inp.pairs[b]) + 1):
                    routes.add(orc.route_bit(int(inp.words[hk, b, m]), n, w.g))
    assert routes == {0, 1}                       # both score paths were exercised


@pytest.mark.parametrize("g", [1, 2])
def test_pin_E_brute_force_kv_int8(g):
    """INT8 KV cache (K_eff = k8 s_k, V_eff = v8 s_v, one scale per 64-key block,
    [PL App. C]): the streaming oracle's rows and log-sum-exp against the
    element-by-element brute force, which dequantises every key and value
    element with the scale of its own block.  Two sequences of 3 and 2 key
    blocks (the last ones partial), GQA 2:1 over two KV heads, both routes,
    block scales spread over e^+-4 per block and head."""
    w = _small([150, 70], hq=4, hk=2, d=64, g=g, p=0.5, cfg=232 + g, outliers=True, kv_int8=True)
    _kv_blocks_scaled(w, np.random.default_rng(33 + g))
    inp = oracle_inputs(w)
    for sc in (inp.k_scale, inp.v_scale):       # the spread the pin relies on
        assert sc[:, 0, :3].max() / sc[:, 0, :3].min() > 20
    _check_kv_int8_brute_force(w, inp)


def test_pin_M_chunked_brute_force_kv_int8():
    """Chunked prefill and decode over an INT8 KV cache against the brute force:
    queries are the last Lq of Lk keys, so their keys span every block of the
    cache (block scales spread as above)."""
    w = make_chunked_workload(292, lengths_q=[70, 1, 5], lengths_k=[200, 130, 5], num_q_heads=4, num_kv_heads=2,
                              head_dim=64, g=1, p=0.5, outliers=True, kv_int8=True)
    _kv_blocks_scaled(w, np.random.default_rng(34))
    inp = oracle_inputs(w)
    assert inp.k_scale[:, 0, :4].max() / inp.k_scale[:, 0, :4].min() > 20
    _check_kv_int8_brute_force(w, inp)


# ---------------------------------------------------------------- pin H
def test_pin_H_quantizer_invariants_and_exact_rounding():
    rng = np.random.default_rng(11)
    lengths = [1, 63, 64, 65, 200]
    cu = cu_from_lengths(lengths)
    N = int(cu[-1])
    x = (rng.standard_normal((N, 3, 64)) * np.exp(rng.uniform(-6, 6, size=(N, 3, 1)))).astype(np.float16)
    x[cu[2]:cu[2] + 64, 1] = 0                                   # an all-zero block
    for blk in (64, 128):
        q, s = orc.quantize_blockwise(x, cu, 200, blk)
        assert s.shape == (3, 5, -(-200 // blk))
        for b, (s0, L) in enumerate(orc.seq_spans(cu)):
            nb = -(-L // blk)
            assert np.all(s[:, b, nb:] == 0)
            for kb in range(nb):
                r0, r1 = s0 + kb * blk, s0 + min((kb + 1) * blk, L)
                for h in range(3):
                    xb = x[r0:r1, h].astype(np.float32)
                    qb = q[r0:r1, h].astype(np.int64)
                    sc = s[h, b, kb]
                    a = np.max(np.abs(xb))
                    if a == 0:
                        assert sc == 1.0 and np.all(qb == 0)
                        continue
                    assert np.all(np.abs(qb) <= 127) and np.max(np.abs(qb)) == 127
                    assert np.all((np.sign(qb) == np.sign(xb)) | (qb == 0))
                    # scale = float32 nearest to a/127, checked with exact rationals
                    assert sc == orc.nearest_fp32(Fraction(float(a)) / 127)
                    # |x - q*scale| <= scale*(1/2 + 127*2^-24)
                    err = np.abs(xb.astype(np.float64) - qb * float(sc))
                    assert np.all(err <= float(sc) * (0.5 + 127 * 2.0 ** -24))
                    # q = round-half-even of the correctly rounded fp32 quotient (sampled)
                    for t in rng.choice(xb.size, size=min(40, xb.size), replace=False):
                        xv = float(xb.flat[t])
                        quo = orc.nearest_fp32(Fraction(xv) / Fraction(float(sc)))
                        ref = int(np.rint(np.float64(quo)))
                        assert int(qb.flat[t]) == max(-127, min(127, ref))


def test_pin_H_int8_scores_within_quantisation_bound():
    """INT8 scores approximate the FP16 scores within the bound implied by
    per-block rounding; blocks have very different magnitudes, so a wrong block
    or head index for a scale breaks the bound."""
    rng = np.random.default_rng(12)
    w = _small([256, 130], hq=2, hk=1, d=64, cfg=270, blk_q=64)
    for arr in (w.q, w.k):
        f = np.exp(rng.uniform(-3, 3, size=(arr.shape[0] // 64 + 1, arr.shape[1])))
        arr[:] = (arr.astype(np.float32) * np.repeat(f, 64, axis=0)[: arr.shape[0], :, None]).astype(np.float16)
    inp = oracle_inputs(w)
    for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for hq in range(2):
            s16 = inp.routed_scores(b, hq, 0, L, 0, L, 0)
            s8 = inp.routed_scores(b, hq, 0, L, 0, L, 1)
            qf = w.q[s0:s0 + L, hq].astype(np.float64)
            kf = w.k[s0:s0 + L, 0].astype(np.float64)
            dq = 0.5 * (1 + 1e-6) * inp.q_scale[hq, b, np.arange(L) // 64].astype(np.float64)
            dk = 0.5 * (1 + 1e-6) * inp.k_scale[0, b, np.arange(L) // 64].astype(np.float64)
            bound = inp.sm * (np.abs(qf).sum(1)[:, None] * dk[None, :] + dq[:, None] * np.abs(kf).sum(1)[None, :]
                              + 64 * dq[:, None] * dk[None, :])
            assert np.all(np.abs(s8 - s16) <= bound * (1 + 1e-9) + 1e-12)


# ---------------------------------------------------------------- pin L
def test_pin_L_output_deviation():
    """MaxDiff / MeanDiff ([PL §5 Numerical Behavior], [PL App. G]): closed form
    on a hand-worked pair; zero at 0 % INT8 coverage (the routed output is the
    FP16 output); and at p > 0 bounded by the score perturbation: a softmax whose
    scores move by at most e changes each weight by a factor within
    [exp(-2e), exp(2e)], so |dO| <= (exp(2e) - 1) max|V|."""
    mx, mn = orc.output_deviation(np.array([[1.0, 2.0], [3.0, 4.0]]), np.array([[1.0, 2.5], [2.0, 4.0]]))
    assert mx == 1.0 and mn == 0.375
    assert orc.output_deviation(np.zeros((0, 3)), np.zeros((0, 3))) == (0.0, 0.0)
    lengths, hq, hk, d = [300, 130], 2, 1, 64
    ref = orc.attn_prefill(oracle_inputs(_small(lengths, hq=hq, hk=hk, d=d, p=0.0, cfg=280, outliers=True)))
    assert orc.output_deviation(ref, ref) == (0.0, 0.0)
    for p in (0.3, 1.0):
        w = _small(lengths, hq=hq, hk=hk, d=d, p=p, cfg=280, outliers=True)
        inp = oracle_inputs(w)
        out = orc.attn_prefill(inp)
        mx, mn = orc.output_deviation(out, ref)
        assert mx > 0 and 0 < mn <= mx
        eps = 0.0
        for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
            for h in range(hq):
                eps = max(eps, float(np.max(np.abs(inp.routed_scores(b, h, 0, L, 0, L, 1) -
                                                   inp.routed_scores(b, h, 0, L, 0, L, 0)))))
        vmax = float(np.max(np.abs(w.v.astype(np.float64))))
        assert mx <= (math.exp(2 * eps) - 1) * vmax


# ---------------------------------------------------------------- pin M
@pytest.mark.parametrize("kv_int8,blk_q", [(False, 64), (False, 128), (True, 64)])
def test_pin_M_chunk_rows_equal_prefill_rows(kv_int8, blk_q):
    """Chunked prefill with bottom-right alignment: when each chunk starts on a Q
    block boundary, its queries see exactly the keys, scales and routes the same
    positions see in a full prefill, so its rows equal the prefill's rows bit for
    bit (the streaming order is the same)."""
    lengths_k = [640, 300, 256]
    lengths_q = [200, 44, 256]          # offsets 440 -> rounded below to blocks
    lengths_q = [L - ((L - q + 127) // 128) * 128 for L, q in zip(lengths_k, lengths_q)]
    full = make_workload(290, lengths=lengths_k, num_q_heads=4, num_kv_heads=2, head_dim=64, g=2, p=0.5,
                         outliers=True, kv_int8=kv_int8, blk_q=blk_q)
    chunk = make_chunked_workload(290, lengths_q=lengths_q, lengths_k=lengths_k, num_q_heads=4, num_kv_heads=2,
                                  head_dim=64, g=2, p=0.5, outliers=True, kv_int8=kv_int8, blk_q=blk_q)
    fin = oracle_inputs(full)
    ref = orc.attn_prefill(fin)
    # the chunk's route words: the full words of the same query-tile rows
    words = np.zeros((2, 3, chunk.T), dtype=np.uint64)
    for b, (Lq, Lk) in enumerate(zip(lengths_q, lengths_k)):
        off = (Lk - Lq) // 64
        words[:, b, : (Lq + 63) // 64] = fin.words[:, b, off: off + (Lq + 63) // 64]
    out = orc.attn_prefill(oracle_inputs(chunk, route_words=words))
    for b, (Lq, Lk) in enumerate(zip(lengths_q, lengths_k)):
        s0q, s0k = int(chunk.cu_seqlens[b]), int(full.cu_seqlens[b])
        assert np.array_equal(out[s0q:s0q + Lq], ref[s0k + Lk - Lq:s0k + Lk])


def test_pin_M_chunked_dense_brute_force_and_lse():
    """Chunked prefill and decode (Lq = 1) against the materialised two-pass
    formulation and the element-by-element brute force; the log-sum-exp against
    the two-pass one and, for the very first query of a prefill, the closed form
    LSE = s_00 (its only key)."""
    w = make_chunked_workload(291, lengths_q=[70, 1, 5], lengths_k=[200, 77, 5], num_q_heads=2, num_kv_heads=1,
                              head_dim=64, g=1, p=0.5, outliers=True)
    inp = oracle_inputs(w)
    out, lse = orc.attn_prefill(inp, with_lse=True)
    for b, (s0, Lq) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for h in range(2):
            o2, l2 = orc.attn_dense_two_pass(inp, b, h, with_lse=True)
            assert np.allclose(out[s0:s0 + Lq, h], o2, rtol=0, atol=1e-12)
            assert np.allclose(lse[s0:s0 + Lq, h], l2, rtol=0, atol=1e-12)
    bf = np.array(orc.attn_brute_force(inp, 1, 1))          # decode: one query over 77 keys
    assert np.allclose(out[70:71, 1], bf, rtol=0, atol=1e-12)
    bf = np.array(orc.attn_brute_force(inp, 2, 0))          # Lq = Lk: plain prefill rows
    assert np.allclose(out[71:76, 0], bf, rtol=0, atol=1e-12)
    # sequence 2 has Lq = Lk: query 0 sees only key 0, so LSE = its score
    s00 = inp.routed_scores(2, 0, 0, 1, 0, 1, orc.route_bit(int(inp.words[0, 2, 0]), 0, 1))[0, 0]
    assert lse[71, 0] == s00


def test_pin_M_chunked_legality_and_packer():
    """Visit matrix = brute-force legality (tile (m, n) holds a pair j <= off + i);
    the packer ANDs exactly the legal tiles of each group."""
    Lq, Lk = [100, 1, 64], [300, 129, 64]
    cu_q, cu_k = cu_from_lengths(Lq), cu_from_lengths(Lk)
    vis = orc.visit_matrix(cu_q, max(Lq), 1, cu_k, max(Lk))
    for b in range(3):
        for m in range(vis.shape[2]):
            for n in range(vis.shape[3]):
                legal = any(j <= Lk[b] - Lq[b] + i for i in range(m * 64, min(m * 64 + 64, Lq[b]))
                            for j in range(n * 64, min(n * 64 + 64, Lk[b])))
                assert vis[b, 0, m, n] == int(legal)
    rng = np.random.default_rng(5)
    tr = rng.integers(0, 2, size=(1, 3, vis.shape[2], vis.shape[3])).astype(np.uint8)
    for g in (1, 2, 3):
        words = orc.build_route_mask(tr, cu_q, max(Lq), g, cu_k, max(Lk))
        for b in range(3):
            for m in range(vis.shape[2]):
                want = 0
                for j in range((vis.shape[3] + g - 1) // g):
                    tiles = [n for n in range(j * g, min(j * g + g, vis.shape[3])) if vis[b, 0, m, n]]
                    if tiles and all(tr[0, b, m, n] for n in tiles):
                        want |= 1 << j
                assert int(words[0, b, m]) == want


# ---------------------------------------------------------------- pin N
def test_pin_N_splitmix64_reference_outputs():
    """The templates' counter-based generator against SplitMix64's published outputs."""
    ref = json.load(open(os.path.join(GOLDEN, "splitmix64_seed0.json")))["outputs_hex"]
    golden = 0x9E3779B97F4A7C15
    got = [orc.splitmix64((k * golden) & ((1 << 64) - 1)) for k in range(3)]
    assert got == [int(x, 16) for x in ref]


@pytest.mark.parametrize("chunked", [False, True])
def test_pin_N_template_coverage_and_structure(chunked):
    """Static templates ([PL App. B]): in every row exactly F = round((1-p) n)
    legal groups are FP16 (the rest INT8, nothing past the row's last legal
    group), so the INT8 coverage of legal groups is within rounding of p; band
    is the diagonal suffix, global the prefix, aligned-sparse evenly spaced,
    SpTrans and BigBird contain their band (and BigBird its global) part; the
    words survive a decode and re-pack unchanged."""
    if chunked:
        Lq, Lk, mq, mk = [300, 1, 64], [3000, 700, 64], 300, 3000
        cu, cu_k = cu_from_lengths(Lq), cu_from_lengths(Lk)
    else:
        Lq = Lk = [3000, 700, 64]
        mq = mk = 3000
        cu, cu_k = cu_from_lengths(Lq), None
    g = 1
    for permille in (0, 250, 500, 750, 1000, 333):
        for kind in orc.TEMPLATES:
            w = orc.template_route_words(kind, permille, 11, cu, mq, 2, g, cu_k, None if cu_k is None else mk)
            int8 = legal = 0
            for hk in range(2):
                for b in range(3):
                    for m in range(orc.num_tiles(Lq[b])):
                        n = orc.last_key_tile(m, Lq[b], Lk[b]) // g + 1
                        word = int(w[hk, b, m])
                        assert word >> n == 0
                        fp = {j for j in range(n) if not (word >> j) & 1}
                        F = ((1000 - permille) * n + 500) // 1000
                        if kind == "all_fp16":
                            assert len(fp) == n
                        elif kind == "all_int8":
                            assert not fp
                        else:
                            assert len(fp) == F, (kind, permille, n)
                        if kind == "band":
                            assert fp == set(range(n - F, n))
                        if kind == "global":
                            assert fp == set(range(F))
                        if kind == "aligned_sparse" and F > 1:
                            gaps = np.diff(sorted(fp))
                            assert gaps.max() - gaps.min() <= 1
                        if kind == "sptrans":
                            assert set(range(n - (F + 1) // 2, n)) <= fp
                        if kind == "bigbird":
                            wb = (F + 2) // 3
                            assert set(range(n - wb, n)) | set(range((F - wb + 1) // 2)) <= fp
                        int8 += n - len(fp)
                        legal += n
            if kind not in ("all_fp16", "all_int8") and not chunked:
                assert abs(int8 / legal - permille / 1000) < 0.02
            # decode + AND re-pack gives the same words (the packer's legality agrees)
            Tq, Tk = orc.num_tiles(mq), orc.num_tiles(mk)
            dec = orc.decode_route_mask(w, cu, mq, g, cu_k, None if cu_k is None else mk)
            tr = np.where(dec == 0xFF, 0, dec).astype(np.uint8)
            assert np.array_equal(orc.build_route_mask(tr, cu, mq, g, cu_k, None if cu_k is None else mk), w)


def test_pin_N_row_random_is_seeded_and_spread():
    """Row-Random: deterministic per seed, different across seeds, and every
    group position about equally likely to stay FP16."""
    cu = cu_from_lengths([64 * 64])
    a = orc.template_route_words("row_random", 500, 1, cu, 64 * 64, 4, 1)
    assert np.array_equal(a, orc.template_route_words("row_random", 500, 1, cu, 64 * 64, 4, 1))
    assert not np.array_equal(a, orc.template_route_words("row_random", 500, 2, cu, 64 * 64, 4, 1))
    # over the 4 x 64 rows of 64 groups (last row: all 64 legal), FP16 frequency per position
    counts = np.zeros(64)
    for hk in range(4):
        for m in range(48, 64):
            word = int(a[hk, 0, m])
            for j in range(m + 1):
                counts[j] += 0 if (word >> j) & 1 else 1
    frac = counts[:49] / 64.0
    assert frac.min() > 0.25 and frac.max() < 0.75


# ---------------------------------------------------------------- pin I
@pytest.mark.parametrize("g", [1, 2, 3, 16])
def test_pin_I_packer_decoder(g):
    lengths = [1, 64, 65, 64 * 40 + 7]
    cu = cu_from_lengths(lengths)
    T = orc.num_tiles(max(lengths))
    rng = np.random.default_rng(20 + g)
    tr = rng.integers(0, 2, size=(2, len(lengths), T, T)).astype(np.uint8)
    tr[:, :, ::3] *= 2                                            # other nonzero values count as INT8
    words = orc.build_route_mask(tr, cu, max(lengths), g)
    dec = orc.decode_route_mask(words, cu, max(lengths), g)
    for hk in range(2):
        for b, L in enumerate(lengths):
            Tb = -(-L // 64)
            for m in range(T):
                w = int(words[hk, b, m])
                if m >= Tb:
                    assert w == 0 and np.all(dec[hk, b, m] == 0xFF)
                    continue
                assert w >> (m // g + 1) == 0                     # no bits past the last legal group
                expect_pop = 0
                for j in range(m // g + 1):
                    grp = [tr[hk, b, m, n] != 0 for n in range(j * g, min(j * g + g, m + 1))]
                    expect_pop += int(all(grp))
                    for n in range(j * g, min(j * g + g, m + 1)):
                        assert dec[hk, b, m, n] == int(all(grp))
                assert bin(w).count("1") == expect_pop
                assert np.all(dec[hk, b, m, m + 1:] == 0xFF)
                if g == 1:
                    assert w == sum(int(tr[hk, b, m, n] != 0) << n for n in range(m + 1))


def test_pin_I_too_many_groups():
    cu = cu_from_lengths([64 * 65])
    tr = np.zeros((1, 1, 65, 65), dtype=np.uint8)
    with pytest.raises(ValueError):
        orc.build_route_mask(tr, cu, 64 * 65, 1)
    orc.build_route_mask(tr, cu, 64 * 65, 2)


# ---------------------------------------------------------------- pin J
def test_pin_J_s32_triple_loop():
    w = _small([150], hq=2, hk=1, d=64, p=1.0, cfg=280, outliers=True)
    inp = oracle_inputs(w)
    tiles = orc.s32_tiles(inp, 0, 1, 0, 3)
    assert tiles.shape == (3, 3, 64, 64)
    q8, k8 = inp.q_q[:, 1].astype(np.int64), inp.k_q[:, 0].astype(np.int64)
    for m in range(3):
        for n in range(3):
            if n > m:
                assert np.all(tiles[m, n] == orc.INT32_MIN)
                continue
            for r in range(0, 64, 7):
                for c in range(0, 64, 5):
                    i, j = 64 * m + r, 64 * n + c
                    ref = 0
                    if i < 150 and j < 150:
                        for ch in range(64):
                            ref += int(q8[i, ch]) * int(k8[j, ch])
                    assert tiles[m, n, r, c] == ref
    assert np.max(np.abs(tiles[tiles != orc.INT32_MIN])) <= 127 * 127 * 64


# ---------------------------------------------------------------- pin K
def test_pin_K_footprint_matches_printed_figures():
    with open(os.path.join(GOLDEN, "footprint_app_d.json")) as f:
        gold = json.load(f)
    sh = gold["shape_reading"]
    pr = gold["printed"]
    fp = orc.footprint_bytes(tokens=sh["tokens"], num_q_heads=sh["num_q_heads"], num_kv_heads=sh["num_kv_heads"],
                             head_dim=sh["head_dim"], blk_q=sh["blk_q"], blk_k=sh["blk_k"])
    assert fp["dense_fp16_qkv"] == pr["fused_on_the_fly_resident_MB"] * 2 ** 20
    assert round(fp["total"] / 2 ** 20, 2) == pr["quantize_once_resident_MiB"]
    # BLKQ = 64 would print 136.02: the printed figure pins per-block (not per-token) scales at 128
    fp64 = orc.footprint_bytes(tokens=sh["tokens"], num_q_heads=sh["num_q_heads"], num_kv_heads=sh["num_kv_heads"],
                               head_dim=sh["head_dim"], blk_q=64, blk_k=64)
    assert round(fp64["total"] / 2 ** 20, 2) != pr["quantize_once_resident_MiB"]
    assert orc.qk_tile_operand_bytes(sh["block_m"], sh["block_n"], sh["head_dim"], False) == pr["fp16_qk_tile_operand_KB"] * 1024
    i8 = orc.qk_tile_operand_bytes(sh["block_m"], sh["block_n"], sh["head_dim"], True)
    assert i8 <= pr["int8_qk_tile_operand_KB"] * 1024 < i8 + 512


# ---------------------------------------------------------------- standard configs
def test_standard_config_shapes():
    w1 = config(1)
    assert w1.q.shape == (512, 1, 64) and w1.T == 8
    legal = legal_tile_matrix(8, 8)
    assert int(legal.sum()) == 36
    w3 = config(3, scale_down=8)
    assert w3.batch == 16 and w3.g == 2
