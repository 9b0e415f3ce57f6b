"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bars: bit-exact for the quantiser (int8 values and fp32 scales), the route
words and their decode, the INT32 score tiles and the tile-visit counts;
outputs (fp32 output option) within max-abs 2e-3 and relative Frobenius 1e-3;
row log-sum-exp within 1e-3.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from workloads import config, make_workload, make_chunked_workload, cu_from_lengths
from tests.oracle_inputs import oracle_inputs

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-3
REL_FRO = 1e-3
# log-sum-exp: the normaliser sums fp16-rounded probabilities (relative error
# below 2^-11 for the sum) and v_log_f32 adds about 1 ulp, so |dLSE| < 1e-3
LSE_ABS = 1e-3


@pytest.fixture(scope="module")
def gp():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_path
    return gpu_path


def _announce(msg):
    print(f"[case] {msg}", flush=True)


# ------------------------------------------------------------------ quantiser
QUANT_CASES = [
    ("tiny_d64_blk64", dict(lengths=[512], hq=1, hk=1, d=64), 64),
    ("varlen_d128_blk64", dict(lengths=[1, 63, 64, 65, 200, 129], hq=3, hk=1, d=128), 64),
    ("varlen_d128_blk128", dict(lengths=[1, 127, 128, 129, 300], hq=2, hk=2, d=128), 128),
    ("varlen_d64_blk128", dict(lengths=[5, 190, 256], hq=5, hk=1, d=64), 128),
]


@pytest.mark.parametrize("name,shape,blk", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantize_bitexact(gp, name, shape, blk):
    import torch
    _announce(f"quantize {name}")
    w = make_workload(300, lengths=shape["lengths"], num_q_heads=shape["hq"], num_kv_heads=shape["hk"],
                      head_dim=shape["d"], g=1, outliers=True)
    w.q[: min(64, w.q.shape[0]), 0] = 0          # an all-zero block
    t = gp.upload(w)
    qq, qs = gp.tm.tilemix_quantize_blockwise(t["q"], t["cu"], w.max_seqlen, blk)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_blockwise(w.q, w.cu_seqlens, w.max_seqlen, blk)
    assert np.array_equal(qq.cpu().numpy(), rq)
    assert np.array_equal(qs.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def _edge_blocks(rng):
    """64 x 128 fp16 blocks that stress the quantiser's rounding: exact half-way
    quotients (ties to even) at several power-of-two scales, subnormal-only
    blocks, the largest fp16 magnitude, an all-zero block, all-ones mantissas."""
    blocks = []
    for e in (-14, -10, -3, 0, 2, 8):
        k = rng.integers(-127, 127, size=(64, 128))
        b = ((k + 0.5) * 2.0 ** e).astype(np.float64)
        b[0, 0] = 127 * 2.0 ** e                        # amax = 127 * 2^e -> scale 2^e exactly
        blocks.append(b)
    sub = rng.integers(-1023, 1024, size=(64, 128)) * 2.0 ** -24   # fp16 subnormals
    blocks.append(sub)
    big = rng.standard_normal((64, 128)) * 1000.0
    big[5, 7] = -65504.0
    blocks.append(big)
    blocks.append(np.zeros((64, 128)))
    ones = rng.uniform(-1, 1, size=(64, 128)) * (2047 / 1024) * 2.0 ** 5
    ones[3, 3] = (2047 / 1024) * 2.0 ** 5
    blocks.append(ones)
    for _ in range(6):
        m = rng.integers(-14, 15)
        blocks.append(rng.standard_normal((64, 128)) * 2.0 ** m)
    return np.concatenate(blocks).astype(np.float16)[:, None, :]


def test_quantize_edge_cases_bitexact(gp):
    import torch
    _announce("quantize edge cases")
    rng = np.random.default_rng(77)
    x = _edge_blocks(rng)
    N = x.shape[0]
    cu = np.array([0, N], dtype=np.int32)
    xd = torch.from_numpy(x).cuda()
    qq, qs = gp.tm.tilemix_quantize_blockwise(xd, torch.from_numpy(cu).cuda(), N, 64)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_blockwise(x, cu, N, 64)
    assert np.array_equal(qs.cpu().numpy(), rs)
    assert np.array_equal(qq.cpu().numpy(), rq)


def test_quantize_strided_input(gp):
    """Q as a view into a packed QKV buffer (token stride > heads*d)."""
    import torch
    _announce("quantize strided")
    w = make_workload(301, lengths=[70, 130], num_q_heads=4, num_kv_heads=2, head_dim=128, g=1, outliers=True)
    N = w.q.shape[0]
    qkv = torch.zeros((N, 8, 128), dtype=torch.float16, device="cuda:0")
    qkv[:, :4] = torch.from_numpy(w.q).cuda()
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    qq, qs = gp.tm.tilemix_quantize_blockwise(qkv[:, :4], cu, w.max_seqlen, 64)
    torch.cuda.synchronize()
    rq, rs = orc.quantize_blockwise(w.q, w.cu_seqlens, w.max_seqlen, 64)
    assert np.array_equal(qq.cpu().numpy(), rq)
    assert np.array_equal(qs.cpu().numpy(), rs)


# ------------------------------------------------------------------ route words
@pytest.mark.parametrize("g", [1, 2, 3, 16])
def test_route_mask_bitexact(gp, g):
    import torch
    _announce(f"route mask g={g}")
    lengths = [1, 64, 65, 64 * 40 + 7]
    w = make_workload(310 + g, lengths=lengths, num_q_heads=2, num_kv_heads=2, head_dim=64, g=1)
    rng = np.random.default_rng(g)
    T = w.T
    tr = rng.integers(0, 3, size=(2, len(lengths), T, T)).astype(np.uint8)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    words = gp.tm.tilemix_build_route_mask(torch.from_numpy(tr).cuda(), cu, w.max_seqlen, g)
    dec = gp.tm.tilemix_decode_route_mask(words, cu, w.max_seqlen, g)
    torch.cuda.synchronize()
    ref = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, g)
    assert np.array_equal(gp.words_u64(words), ref)
    assert np.array_equal(dec.cpu().numpy(), orc.decode_route_mask(ref, w.cu_seqlens, w.max_seqlen, g))


@pytest.mark.parametrize("g", [1, 3])
def test_route_mask_chunked_bitexact(gp, g):
    """Packer and decoder with key prefix sums (chunked prefill / decode): the
    legal tiles of a row run to the key tile of its last query."""
    import torch
    _announce(f"route mask chunked g={g}")
    Lq, Lk = [1, 70, 64, 200, 5], [1, 300, 64, 2600, 900]
    w = make_chunked_workload(320 + g, lengths_q=Lq, lengths_k=Lk, num_q_heads=2, num_kv_heads=2, head_dim=64, g=1)
    rng = np.random.default_rng(g)
    tr = rng.integers(0, 3, size=(2, len(Lq), w.T, w.T_k)).astype(np.uint8)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    cu_k = torch.from_numpy(w.cu_seqlens_k).cuda()
    kw = dict(cu_seqlens_k=cu_k, max_seqlen_k=w.max_seqlen_k)
    words = gp.tm.tilemix_build_route_mask(torch.from_numpy(tr).cuda(), cu, w.max_seqlen, g, **kw)
    dec = gp.tm.tilemix_decode_route_mask(words, cu, w.max_seqlen, g, **kw)
    torch.cuda.synchronize()
    ref = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, g, w.cu_seqlens_k, w.max_seqlen_k)
    assert np.array_equal(gp.words_u64(words), ref)
    assert np.array_equal(dec.cpu().numpy(),
                          orc.decode_route_mask(ref, w.cu_seqlens, w.max_seqlen, g, w.cu_seqlens_k, w.max_seqlen_k))


@pytest.mark.parametrize("chunked", [False, True])
def test_template_route_words_bitexact(gp, chunked):
    """Static routing templates: every template, several coverages and group
    sizes, prefill and chunked, bit-exact against the oracle's words."""
    import torch
    _announce(f"templates chunked={chunked}")
    if chunked:
        Lq, Lk = [300, 1, 64, 2000], [3000, 700, 64, 2000]
    else:
        Lq = Lk = [3000, 700, 64, 1, 4096]
    cu_h, cuk_h = cu_from_lengths(Lq), cu_from_lengths(Lk)
    cu = torch.from_numpy(cu_h).cuda()
    cu_k = torch.from_numpy(cuk_h).cuda() if chunked else None
    mq, mk = max(Lq), max(Lk)
    for g in (1, 2):
        for permille in (0, 50, 250, 500, 750, 1000, 333):
            for kind in orc.TEMPLATES:
                seed = 1234 + permille
                got = gp.tm.tilemix_template_route_words(kind, permille, seed, cu, mq, 3, g, cu_seqlens_k=cu_k,
                                                         max_seqlen_k=mk if chunked else 0)
                ref = orc.template_route_words(kind, permille, seed, cu_h, mq, 3, g, cuk_h if chunked else None,
                                               mk if chunked else None)
                assert np.array_equal(gp.words_u64(got), ref), (kind, permille, g)


def test_route_mask_too_many_groups(gp):
    import torch
    from mixed_precision_amd.tilemix import TilemixError
    cu = torch.tensor([0, 64 * 65], dtype=torch.int32, device="cuda:0")
    tr = torch.zeros((1, 1, 65, 65), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(TilemixError) as e:
        gp.tm.tilemix_build_route_mask(tr, cu, 64 * 65, 1)
    assert e.value.status == 3


# ------------------------------------------------------------------ attention, small, compared in full
SMALL = [
    # name, lengths, Hq, Hk, d, g, route, p, kv_int8, blk_q, outliers
    ("tiny_L512_d64", [512], 1, 1, 64, 1, "bernoulli", 0.5, False, 64, False),
    ("len1", [1], 2, 1, 64, 1, "bernoulli", 0.5, False, 64, False),
    ("ragged_gqa3_d128", [1, 65, 200, 130], 3, 1, 128, 1, "bernoulli", 0.75, False, 64, True),
    ("gqa4_varlen_g2", [300, 64, 127], 8, 2, 128, 2, "bernoulli", 0.5, False, 64, True),
    ("gqa2_d64", [257, 129], 4, 2, 64, 1, "bernoulli", 0.5, False, 128, True),
    ("gqa7_two_chunks", [190], 7, 1, 128, 1, "bernoulli", 0.5, False, 64, False),
    ("all_fp16", [333], 3, 1, 128, 1, "zeros", 0.0, False, 64, True),
    ("all_int8", [333], 3, 1, 128, 1, "ones", 1.0, False, 64, True),
    ("blkq128", [400, 77], 6, 2, 128, 1, "bernoulli", 0.5, False, 128, True),
    ("kv_int8_gqa7_g4", [520, 100], 7, 1, 128, 4, "bernoulli", 0.5, True, 64, False),
    ("kv_int8_d64", [300], 2, 1, 64, 1, "bernoulli", 0.5, True, 64, False),
    ("band_sink_g2", [700, 450], 4, 1, 128, 2, "band_sink", 0.0, False, 64, True),
    # mild logits (K outliers only): the running max rarely moves
    ("mild_gqa3", [777, 300], 6, 2, 128, 1, "bernoulli", 0.5, False, 64, "mild"),
    ("mild_kv_int8", [500], 7, 1, 128, 2, "bernoulli", 0.5, True, 64, "mild"),
    # more sequences than the work-list planner keeps in LDS (global-scratch path)
    ("many_seqs_4100", [1 + (i * 37) % 70 for i in range(4100)], 2, 1, 64, 1, "bernoulli", 0.5, False, 64, False),
    # INT8 KV cache with a GQA ratio of 3: three heads per item, tiles staged through LDS
    ("kv_int8_gqa3_lds", [300, 64, 130, 1], 6, 2, 128, 2, "bernoulli", 0.5, True, 64, True),
    ("kv_int8_gqa3_d64", [200, 77], 3, 1, 64, 1, "bernoulli", 0.6, True, 128, False),
    # partial head chunks (the chunk size does not divide G): 3 + 2 and 3 + 3 + 2 heads,
    # and 3 + 2 with the INT8 cache (tiles staged through LDS)
    ("gqa5_chunks_3_2", [300, 129, 1], 5, 1, 128, 1, "bernoulli", 0.5, False, 64, True),
    ("gqa8_d64_chunks_3_3_2", [260, 70], 16, 2, 64, 2, "bernoulli", 0.6, False, 128, True),
    ("kv_int8_gqa5_chunks_3_2", [400, 65], 5, 1, 128, 2, "bernoulli", 0.5, True, 64, True),
    # one and two heads per item at d = 128: with Q on the fly, V through a single LDS stage
    ("mha_d128_single_v", [200, 65, 1], 2, 2, 128, 2, "bernoulli", 0.5, False, 64, True),
    ("gqa2_d128_blkq128_single_v", [300, 129], 4, 2, 128, 1, "bernoulli", 0.6, False, 128, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_attn_small_full(gp, case):
    import torch
    name, lengths, hq, hk, d, g, route, p, kv8, blk_q, outl = case
    _announce(f"attn small {name}")
    extra = dict(q_outlier_scale=1.0, k_outlier_scale=10.0) if outl == "mild" else {}
    w = make_workload(400 + SMALL.index(case), lengths=lengths, num_q_heads=hq, num_kv_heads=hk, head_dim=d, g=g,
                      route=route, p=p, kv_int8=kv8, blk_q=blk_q, outliers=bool(outl), **extra)
    t = gp.prepare(w)
    out = gp.attn(w, t, out_fp32=True)
    out16 = gp.attn(w, t, out_fp32=False)
    torch.cuda.synchronize()
    ref = orc.attn_prefill(oracle_inputs(w))
    ma, rf = gp.errors(out.cpu().numpy(), ref)
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO
    # fp16 output: within half an fp16 ulp of the reference plus the same budget
    o16 = out16.cpu().numpy().astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(o16 - ref) <= 0.5 * ulp + MAX_ABS)
    # the first query of each sequence sees only its own key: O = V_eff[0]
    inp = oracle_inputs(w)
    got = out.cpu().numpy()
    for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
        for h in range(hq):
            v0 = inp._kv(b, inp.kv_head(h))[1][0]
            assert np.max(np.abs(got[s0, h] - v0)) <= 1e-3 * max(1.0, np.max(np.abs(v0)))


@pytest.mark.parametrize("case", ["tiny", "gqa3_varlen", "kv_int8", "kv_int8_last_chunk", "kv_int8_gqa3"])
def test_attn_debug_bitexact(gp, case):
    """INT32 score tiles bit-exact; every legal tile visited once, nothing else;
    the decoded route per visited tile equals the oracle's."""
    import torch
    _announce(f"attn debug {case}")
    if case == "tiny":
        w = config(1)
        seq, head = 0, 0
    elif case == "gqa3_varlen":
        w = make_workload(450, lengths=[130, 300, 64], num_q_heads=6, num_kv_heads=2, head_dim=128, g=2,
                          p=0.6, outliers=True)
        seq, head = 1, 4
    elif case in ("kv_int8", "kv_int8_last_chunk"):
        # GQA 7 in chunks of 3 + 3 + 1 heads; head 6 is the partial chunk's
        w = make_workload(451, lengths=[260, 90], num_q_heads=7, num_kv_heads=1, head_dim=128, g=1, p=0.5,
                          kv_int8=True)
        seq, head = (0, 5) if case == "kv_int8" else (1, 6)
    else:   # three heads per item: the INT8 tiles are staged through LDS
        w = make_workload(452, lengths=[200, 70], num_q_heads=3, num_kv_heads=1, head_dim=128, g=1, p=0.5,
                          kv_int8=True, outliers=True)
        seq, head = 0, 2
    t = gp.prepare(w)
    out, s32, visits, used = gp.attn_debug(w, t, seq=seq, q_head=head)
    torch.cuda.synchronize()
    inp = oracle_inputs(w)
    ref_s32 = orc.s32_tiles(inp, seq, head, 0, w.T)
    assert np.array_equal(s32.cpu().numpy(), ref_s32)
    vis = orc.visit_matrix(w.cu_seqlens, w.max_seqlen, w.num_q_heads)
    assert np.array_equal(visits.cpu().numpy().astype(np.uint32), vis)
    assert np.array_equal(used.cpu().numpy(), orc.route_used(inp))
    ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(inp))
    assert ma <= MAX_ABS and rf <= REL_FRO


OTF_SMALL = [c for c in SMALL if not c[8]]


@pytest.mark.parametrize("case", OTF_SMALL, ids=[c[0] for c in OTF_SMALL])
def test_attn_on_the_fly_equals_quantize_once(gp, case):
    """On-the-fly quantisation (Q/K INT8 fragments and block scales made inside
    the kernel, or Q's alone) follows the same blockwise definition as the
    quantiser, so its output equals the quantise-once output bit for bit (fp32
    and fp16 outputs), and therefore meets the oracle bar too."""
    import torch
    name, lengths, hq, hk, d, g, route, p, kv8, blk_q, outl = case
    _announce(f"attn on-the-fly {name}")
    extra = dict(q_outlier_scale=1.0, k_outlier_scale=10.0) if outl == "mild" else {}
    w = make_workload(400 + SMALL.index(case), lengths=lengths, num_q_heads=hq, num_kv_heads=hk, head_dim=d, g=g,
                      route=route, p=p, kv_int8=kv8, blk_q=blk_q, outliers=bool(outl), **extra)
    t = gp.prepare(w)
    once32 = gp.attn(w, t, out_fp32=True)
    otf32 = gp.attn(w, t, out_fp32=True, otf=True)
    once16 = gp.attn(w, t, out_fp32=False)
    otf16 = gp.attn(w, t, out_fp32=False, otf=True)
    qotf32 = gp.attn(w, t, out_fp32=True, otf=2)
    qotf16 = gp.attn(w, t, out_fp32=False, otf=2)
    torch.cuda.synchronize()
    assert torch.equal(otf32, once32)
    assert torch.equal(otf16, once16)
    assert torch.equal(qotf32, once32)
    assert torch.equal(qotf16, once16)
    ma, rf = gp.errors(otf32.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO


@pytest.mark.parametrize("mode", [1, 2], ids=["qk", "q"])
@pytest.mark.parametrize("case", ["tiny", "gqa3_varlen_blkq128"])
def test_attn_on_the_fly_debug_bitexact(gp, case, mode):
    """On-the-fly modes (Q and K, or Q alone): INT32 score tiles bit-exact against
    the oracle's (so the on-chip quantisation and block layout are exact),
    visits and routes too."""
    import torch
    _announce(f"attn on-the-fly debug {case} mode {mode}")
    if case == "tiny":
        w = config(1)
        seq, head = 0, 0
    else:
        w = make_workload(452, lengths=[130, 300, 64], num_q_heads=6, num_kv_heads=2, head_dim=128, g=2,
                          p=0.6, outliers=True, blk_q=128)
        seq, head = 1, 4
    t = gp.prepare(w)
    out, s32, visits, used = gp.attn_debug(w, t, seq=seq, q_head=head, otf=mode)
    torch.cuda.synchronize()
    inp = oracle_inputs(w)
    assert np.array_equal(s32.cpu().numpy(), orc.s32_tiles(inp, seq, head, 0, w.T))
    vis = orc.visit_matrix(w.cu_seqlens, w.max_seqlen, w.num_q_heads)
    assert np.array_equal(visits.cpu().numpy().astype(np.uint32), vis)
    assert np.array_equal(used.cpu().numpy(), orc.route_used(inp))
    ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(inp))
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_attn_on_the_fly_zero_blocks(gp):
    """On-the-fly mode with an all-zero Q block and an all-zero K tile (scale 1,
    int8 zeros by definition): same output as quantise-once and the oracle."""
    import torch
    _announce("attn on-the-fly zero blocks")
    w = make_workload(471, lengths=[200, 150], num_q_heads=3, num_kv_heads=1, head_dim=128, g=1, route="ones",
                      p=1.0, outliers=True)
    s1 = int(w.cu_seqlens[1])
    w.q[64:128, 1, :] = 0
    w.k[s1 + 64:s1 + 128, 0, :] = 0
    t = gp.prepare(w)
    once = gp.attn(w, t)
    otf = gp.attn(w, t, otf=True)
    torch.cuda.synchronize()
    assert torch.equal(otf, once)
    ma, rf = gp.errors(otf.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_attn_zero_scale_blocks(gp):
    """A caller may pass scale 0 for an all-zero INT8 block (the library's own
    quantiser writes 1.0 there).  The INT32 scores of such a block are 0 either
    way, so the output must equal the oracle's, masked keys included."""
    import torch
    _announce("attn zero-scale blocks")
    w = make_workload(470, lengths=[200, 150], num_q_heads=3, num_kv_heads=1, head_dim=128, g=1, route="ones",
                      p=1.0, outliers=True)
    s1 = int(w.cu_seqlens[1])
    w.q[64:128, 1, :] = 0            # seq 0, query tile 1 of head 1 (diagonal tile is INT8)
    w.k[s1 + 64:s1 + 128, 0, :] = 0  # seq 1, key tile 1
    t = gp.prepare(w)
    t["q_s"][1, 0, 1] = 0.0
    t["k_s"][0, 1, 1] = 0.0
    out = gp.attn(w, t)
    torch.cuda.synchronize()
    ref = orc.attn_prefill(oracle_inputs(w))
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    ma, rf = gp.errors(got, ref)
    assert ma <= MAX_ABS and rf <= REL_FRO


@pytest.mark.parametrize("case", ["large_scales", "tiny_key_tiles"])
def test_attn_int8_score_scale_extremes(gp, case):
    """INT8 score factors at both ends.  large_scales: Q and K scaled so that
    s_q s_k sm log2(e) >= 1/2 on every tile (near one-hot rows, scores of
    thousands of log2 units).  tiny_key_tiles: every other key tile scaled by
    1e-4, so rows reach those tiles with a reference maximum far above their
    scores.  Output against the oracle, quantise-once and on-the-fly."""
    import torch
    _announce(f"attn INT8 score scales {case}")
    if case == "large_scales":
        w = make_workload(475, lengths=[300, 150], num_q_heads=3, num_kv_heads=1, head_dim=128, g=1,
                          route="ones", p=1.0)
        w.q *= np.float16(100.0)
        w.k *= np.float16(100.0)
    else:
        w = make_workload(476, lengths=[400, 200], num_q_heads=6, num_kv_heads=2, head_dim=128, g=1, p=0.5,
                          outliers=True)
        for b, (s0, L) in enumerate(orc.seq_spans(w.cu_seqlens)):
            for n in range(1, (L + 63) // 64, 2):
                w.k[s0 + 64 * n:s0 + min(64 * n + 64, L)] *= np.float16(1e-4)
    t = gp.prepare(w)
    if case == "large_scales":
        inp = oracle_inputs(w)
        qs, ks = inp.q_scale.astype(np.float64), inp.k_scale.astype(np.float64)   # (unused blocks hold 0)
        c = (qs[qs > 0].min() * ks[ks > 0].min()
             * float(w.sm_scale) * 1.4426950408889634)
        assert c >= 0.5
    ref = orc.attn_prefill(oracle_inputs(w))
    for otf in (False, True):
        out = gp.attn(w, t, out_fp32=True, otf=otf)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        ma, rf = gp.errors(got, ref)
        print(f"  otf={otf} max_abs={ma:.3e} rel_fro={rf:.3e}")
        assert ma <= MAX_ABS and rf <= REL_FRO


def _greedy_plan(cu, T, Hk, nch, cu_k=None):
    """Work list of the XCD planner, placing one (sequence, KV head) group at a
    time: groups in decreasing tile count, each whole on the XCD with the least
    load (lowest index on ties) that has room, else split over the XCDs with
    the most free slots; slot i takes entry i // 8 of XCD i % 8's list."""
    xcd = 8
    lens = np.diff(cu).astype(np.int64)
    tiles = (lens + 63) // 64
    B = len(lens)
    items_n = B * T * Hk * nch
    nslots = max(-(-items_n // xcd) * xcd, xcd)
    cap = nslots // xcd
    Tk = T if cu_k is None else int(-(-int(np.diff(cu_k).max()) // 64))
    rows = B * Hk * nch * T
    total = rows * (T + 1) // 2 + (rows * Tk if cu_k is not None else 0)
    shift = 0
    while (total >> shift) >= (1 << 28):
        shift += 1
    order = sorted(range(B), key=lambda b: (-tiles[b], b))
    used, load = [0] * xcd, [0] * xcd
    items = np.zeros((nslots, 4), np.int32)
    items[:, 0] = -1
    for b in order:
        tb = int(tiles[b])
        if tb == 0:
            break
        cnt = tb * nch
        tb_cost = tb * (tb + 1) // 2
        if cu_k is not None:
            lead = int(cu_k[b + 1] - cu_k[b]) - int(lens[b])
            tb_cost += tb * max(lead, 0) // 64
        cost = (nch * tb_cost) >> shift
        for hk in range(Hk):
            remaining, ib = cnt, 0
            while remaining > 0:
                fits = [x for x in range(xcd) if cap - used[x] >= remaining]
                if fits:
                    best = min(fits, key=lambda x: (load[x], x))
                    take = remaining
                else:
                    best = max(range(xcd), key=lambda x: (cap - used[x], -x))
                    take = cap - used[best]
                for i in range(take):
                    t = ib + i
                    items[(used[best] + i) * xcd + best] = (b, hk, tb - 1 - t // nch, t % nch)
                load[best] += cost if take == cnt else cost * take // cnt
                used[best] += take
                ib += take
                remaining -= take
    return items


@pytest.mark.parametrize("case", ["equal_B8_hk8", "varlen_hk16", "varlen_hk5_chunks", "many_short"])
def test_plan_matches_greedy_placement(gp, case):
    """The work list equals the one-group-at-a-time greedy placement (the plan
    kernel places a sequence's identical KV-head groups in one step where that
    gives the same result)."""
    import torch
    _announce(f"plan vs greedy {case}")
    rng = np.random.default_rng(5)
    if case == "equal_B8_hk8":
        lens, hq, hk = [4096] * 8, 24, 8
    elif case == "varlen_hk16":
        lens, hq, hk = [int(x) for x in rng.integers(1, 3000, 11)], 32, 16
    elif case == "varlen_hk5_chunks":
        lens, hq, hk = [int(x) for x in rng.integers(1, 2000, 9)], 35, 5
    else:
        lens, hq, hk = [int(x) for x in rng.integers(1, 200, 300)], 8, 8
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    L = max(lens)
    prob = gp.tm.AttnProblem(len(lens), L, hq, hk, 128, 1, 64, 0.088, False, True)
    plan = gp.tm.AttnPlan(prob, "cuda:0")
    plan.schedule(torch.from_numpy(cu).to("cuda:0"))
    torch.cuda.synchronize()
    T = -(-L // 64)
    nch = -(-(hq // hk) // 3)
    ref = _greedy_plan(cu, T, hk, nch)
    got = plan.workspace[:ref.size * 4].cpu().view(torch.int32).numpy().reshape(-1, 4)
    live = ref[:, 0] >= 0
    assert np.array_equal(got[live], ref[live])
    assert np.all(got[~live, 0] == -1)


def test_attn_plan_then_run_equals_prefill(gp):
    """tilemix_attn_plan + tilemix_attn_run give the same bits as tilemix_attn_prefill,
    and one plan serves repeated runs."""
    import torch
    _announce("attn plan + run")
    w = make_workload(480, lengths=[300, 64, 1000], num_q_heads=6, num_kv_heads=2, head_dim=128, g=2, p=0.6,
                      outliers=True)
    t = gp.prepare(w)
    ref = gp.attn(w, t).clone()
    plan = gp.tm.AttnPlan(gp.tm.AttnProblem(w.batch, w.max_seqlen, w.num_q_heads, w.num_kv_heads, w.head_dim, w.g,
                                            w.blk_q, w.sm_scale, False, True), "cuda:0")
    plan.schedule(t["cu"])
    outs = []
    for _ in range(2):
        o = torch.empty_like(ref)
        plan.run_planned(t["q"], t["k"], t["v"], t["q_q"], t["q_s"], t["k_q"], t["k_s"], t["cu"], t["words"], o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref) and torch.equal(outs[1], ref)


def test_attn_g1_equals_g4_when_groups_constant(gp):
    """Same per-tile routes packed at g = 1 and g = 4 give identical outputs."""
    import torch
    _announce("attn g1 vs g4")
    w4 = make_workload(460, lengths=[64 * 12 + 5], num_q_heads=3, num_kv_heads=1, head_dim=128, g=4, p=0.5,
                       outliers=True)
    t = gp.prepare(w4)
    o4 = gp.attn(w4, t).clone()
    w1 = make_workload(460, lengths=[64 * 12 + 5], num_q_heads=3, num_kv_heads=1, head_dim=128, g=4, p=0.5,
                       outliers=True)
    w1.g = 1
    t1 = gp.prepare(w1, t={k: v for k, v in t.items() if k in ("q", "k", "v", "cu", "tile_route")})
    o1 = gp.attn(w1, t1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o4)


# ------------------------------------------------------------------ standard workloads
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_standard_config_scaled_full(gp, cfg):
    """Each standard workload's structure at 1/8 of its lengths (1/16 for the
    long one), compared in full."""
    import torch
    _announce(f"config {cfg} scaled")
    w = config(cfg, scale_down=1 if cfg == 1 else (16 if cfg == 5 else 8))
    t = gp.prepare(w)
    out = gp.attn(w, t)
    otf = None if w.kv_int8 else gp.attn(w, t, otf=True)
    torch.cuda.synchronize()
    ref = orc.attn_prefill(oracle_inputs(w))
    ma, rf = gp.errors(out.cpu().numpy(), ref)
    print(f"  {w.name}: max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO
    if otf is not None:   # on-the-fly quantisation: the same bits
        assert torch.equal(otf, out)


@pytest.mark.parametrize("p", [0.0, 0.25, 0.75, 1.0])
def test_long_context_coverage_sweep_scaled(gp, p):
    """The long-context workload's INT8 coverage sweep (0/25/50/75/100 % of the
    tile groups; 50 % is the standard case above) at 1/16 of its length."""
    import torch
    _announce(f"config 5 scaled, coverage {p}")
    w = config(5, p=p, scale_down=16)
    t = gp.prepare(w)
    out = gp.attn(w, t)
    torch.cuda.synchronize()
    ref = orc.attn_prefill(oracle_inputs(w))
    ma, rf = gp.errors(out.cpu().numpy(), ref)
    print(f"  {w.name}: max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_3b_workload_blkq128_scaled(gp):
    """The 3B-shaped layer with Q quantised in blocks of 128 tokens (the pages'
    BLKQ; the default is 64), at 1/8 of its length, compared in full."""
    import torch
    _announce("config 2 scaled, blk_q 128")
    w = config(2, scale_down=8)
    w.blk_q = 128
    t = gp.prepare(w)
    out = gp.attn(w, t)
    torch.cuda.synchronize()
    inp = oracle_inputs(w)
    assert np.array_equal(t["q_s"].cpu().numpy(), inp.q_scale)
    ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(inp))
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_deviation_sweep_matches_oracle(gp):
    """Coverage -> deviation ([PL §5 Numerical Behavior], [PL App. G]) on a
    long-context-shaped head group: MaxDiff / MeanDiff of the routed output
    against the 0 % output agree with the oracle's; 0 % is exactly zero; the
    mean deviation at 100 % exceeds that at 10 %."""
    import torch
    _announce("deviation sweep")
    ps = [0.0, 0.1, 0.5, 1.0]
    got, ref = {}, {}
    for p in ps:
        w = make_workload(490, lengths=[1536], num_q_heads=4, num_kv_heads=1, head_dim=128, g=4, p=p,
                          outliers=True)
        t = gp.prepare(w)
        o = gp.attn(w, t)
        torch.cuda.synchronize()
        got[p] = o.cpu().numpy()
        ref[p] = orc.attn_prefill(oracle_inputs(w))
    means = {}
    for p in ps:
        mh, nh = orc.output_deviation(got[p], got[0.0])
        mo, no = orc.output_deviation(ref[p], ref[0.0])
        print(f"  p={p}: hip max={mh:.3e} mean={nh:.3e}   oracle max={mo:.3e} mean={no:.3e}")
        if p == 0.0:
            assert mh == 0.0 and nh == 0.0
        assert abs(mh - mo) <= 2 * MAX_ABS
        assert abs(nh - no) <= 0.05 * no + 1e-5
        means[p] = nh
    assert means[1.0] > means[0.1] > 0


# ------------------------------------------------------------------ chunked prefill / decode
CHUNKED = [
    # name, lengths_q, lengths_k, Hq, Hk, d, g, p, kv_int8, blk_q
    ("chunk_gqa3_fp16kv", [200, 64, 1, 130], [1000, 64, 300, 1500], 6, 2, 128, 2, 0.5, False, 64),
    ("chunk_int8kv_gqa7", [333, 50], [2000, 50], 7, 1, 128, 4, 0.6, True, 64),
    ("chunk_d64_blkq128", [257, 100], [900, 700], 4, 2, 64, 1, 0.5, False, 128),
    ("decode_int8kv", [1] * 37, [64 * 30 + 5 + 13 * i for i in range(37)], 4, 1, 128, 2, 0.5, True, 64),
    ("decode_fp16kv_gqa4", [1] * 9, [1, 2, 63, 64, 65, 500, 1000, 2049, 4096], 8, 2, 128, 1, 0.7, False, 64),
    # decode kernel (one query per sequence): GQA 1, 7 and 16 rows, d = 64, keys
    # shorter than one wave's 16-key slice, long caches, groups of 4 tiles
    ("decode_mha_d64_short", [1] * 6, [1, 3, 16, 17, 40, 64], 5, 5, 64, 1, 0.5, False, 64),
    ("decode_gqa7_int8kv", [1] * 5, [1, 15, 129, 3000, 8191], 14, 2, 128, 4, 0.6, True, 64),
    ("decode_gqa16_fp16kv", [1] * 4, [7, 700, 2048, 5000], 16, 1, 128, 2, 0.4, False, 64),
    ("decode_gqa3_d64_int8kv", [1] * 3, [2, 333, 4097], 6, 2, 64, 2, 0.5, True, 64),
    # chunked prefill, INT8 cache, GQA 3 (three heads per item, LDS staging)
    ("chunk_int8kv_gqa3", [190, 64, 5], [900, 64, 700], 6, 2, 128, 1, 0.5, True, 64),
    # decode with more query heads per KV head than one 16-row block: the fused
    # prefill kernel takes it (7 items of 3 heads, one query row each)
    ("decode_gqa20_int8kv", [1] * 3, [5, 640, 2500], 20, 1, 128, 2, 0.5, True, 64),
    # chunked prefill with a partial head chunk (GQA 5 in chunks of 3 + 2), also on the fly
    ("chunk_gqa5_fp16kv_chunks_3_2", [150, 70, 1], [700, 70, 300], 5, 1, 128, 2, 0.5, False, 64),
    # two heads per item at d = 128: with Q on the fly, V through a single LDS stage
    ("chunk_gqa2_fp16kv_single_v", [190, 64, 1, 129], [900, 64, 300, 1500], 4, 2, 128, 2, 0.5, False, 64),
]


@pytest.mark.parametrize("case", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_attn_chunked_full(gp, case):
    """Chunked prefill and decode over a KV cache (bottom-right causal
    alignment): output and log-sum-exp of every query against the oracle;
    fp16-KV cases also through the on-the-fly mode (same bits)."""
    import torch
    name, Lq, Lk, hq, hk, d, g, p, kv8, blk_q = case
    _announce(f"attn chunked {name}")
    w = make_chunked_workload(500 + CHUNKED.index(case), lengths_q=Lq, lengths_k=Lk, num_q_heads=hq,
                              num_kv_heads=hk, head_dim=d, g=g, p=p, outliers=True, kv_int8=kv8, blk_q=blk_q)
    t = gp.prepare(w)
    lse = torch.empty((w.q.shape[0], hq), dtype=torch.float32, device="cuda:0")
    out = gp.attn(w, t, lse=lse)
    otf = None if kv8 else gp.attn(w, t, otf=True)
    qotf = None if kv8 else gp.attn(w, t, otf=2)
    torch.cuda.synchronize()
    ref, ref_lse = orc.attn_prefill(oracle_inputs(w), with_lse=True)
    ma, rf = gp.errors(out.cpu().numpy(), ref)
    le = float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)))
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e} lse_err={le:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO
    assert le <= LSE_ABS
    for o in (otf, qotf):   # operands made in the kernel (Q and K, or Q alone)
        if o is None:
            continue
        if max(Lq) > 1:
            assert torch.equal(o, out)
        else:   # decode goes to the decode kernel, on-the-fly to the prefill kernel: other order
            mo, ro = gp.errors(o.cpu().numpy(), ref)
            assert mo <= MAX_ABS and ro <= REL_FRO



def _random_case(seed):
    """A seeded random configuration inside the supported range: 1-4 sequences
    with lengths at tile edges or random (1..400), prefill or chunked prefill /
    decode, d 64 or 128, 1-3 KV heads and 1-8 or 16 query heads per KV head,
    g 1-4, INT8 coverage 0-100 %, fp16 or INT8 cache, blk_q 64 or 128, with
    or without outlier channels."""
    import random
    rng = random.Random(seed)
    d = rng.choice([64, 128])
    hk = rng.choice([1, 2, 3])
    hq = hk * rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 16])
    kv8 = rng.random() < 0.35
    blk_q = rng.choice([64, 64, 128])
    p = rng.choice([0.0, 0.3, 0.5, 0.8, 1.0])
    outl = rng.random() < 0.6
    chunked = rng.random() < 0.3
    nseq = rng.randint(1, 4)

    def pick():
        return rng.choice([1, 2, 63, 64, 65, 127, 128, 129, rng.randint(1, 400)])

    if chunked:
        lk = [pick() + rng.choice([0, 64, 200]) for _ in range(nseq)]
        lq = [rng.choice([1, min(k, rng.randint(1, k))]) for k in lk]
        g = rng.choice([1, 2, 3])
        w = make_chunked_workload(seed, lengths_q=lq, lengths_k=lk, num_q_heads=hq, num_kv_heads=hk, head_dim=d,
                                  g=g, p=p, outliers=outl, kv_int8=kv8, blk_q=blk_q)
        desc = f"chunked lq={lq} lk={lk}"
    else:
        lens = [pick() for _ in range(nseq)]
        g = rng.choice([1, 2, 3, 4])
        w = make_workload(seed, lengths=lens, num_q_heads=hq, num_kv_heads=hk, head_dim=d, g=g, p=p,
                          outliers=outl, kv_int8=kv8, blk_q=blk_q)
        desc = f"prefill lengths={lens}"
    return w, f"{desc} heads {hq}/{hk} d={d} g={g} p={p} kv_int8={kv8} blk_q={blk_q} outliers={outl}"


@pytest.mark.parametrize("seed", list(range(9000, 9024)))
def test_attn_random_configs(gp, seed):
    """Seeded random configurations (`_random_case`) against the oracle, every
    element; for an fp16 cache also with the operands made in the kernel (the
    same bits, or within the bar where decode goes to the decode kernel)."""
    import torch
    w, desc = _random_case(seed)
    _announce(f"attn random {seed}: {desc}")
    t = gp.prepare(w)
    out = gp.attn(w, t)
    modes = [] if w.kv_int8 else [gp.attn(w, t, otf=True), gp.attn(w, t, otf=2)]
    torch.cuda.synchronize()
    ref = orc.attn_prefill(oracle_inputs(w))
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    ma, rf = gp.errors(got, ref)
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO
    decode = w.cu_seqlens_k is not None and max(w.lengths) == 1
    for o in modes:
        if decode:   # decode kernel against the prefill kernel: another order
            mo, ro = gp.errors(o.cpu().numpy(), ref)
            assert mo <= MAX_ABS and ro <= REL_FRO
        else:
            assert torch.equal(o, out)

def test_attn_chunk_rows_equal_prefill_rows(gp):
    """A chunk that starts on a Q block sees the same keys, scales and routes in
    the same order as the same rows of the full prefill, so the HIP path gives
    the same bits for them (and the same log-sum-exp)."""
    import torch
    _announce("attn chunk rows == prefill rows")
    Lk = [1280, 700, 333]
    Lq = [1280 - 1024, 700 - 512, 333]
    full = make_workload(520, lengths=Lk, num_q_heads=6, num_kv_heads=2, head_dim=128, g=2, p=0.5, outliers=True)
    chunk = make_chunked_workload(520, lengths_q=Lq, lengths_k=Lk, num_q_heads=6, num_kv_heads=2, head_dim=128,
                                  g=2, p=0.5, outliers=True)
    tf = gp.prepare(full)
    lse_f = torch.empty((full.q.shape[0], 6), dtype=torch.float32, device="cuda:0")
    of = gp.attn(full, tf, lse=lse_f)
    tc = gp.prepare(chunk)
    words = torch.zeros_like(tc["words"])
    for b, (q_, k_) in enumerate(zip(Lq, Lk)):          # the chunk's rows of the full words
        off = (k_ - q_) // 64
        words[:, b, : (q_ + 63) // 64] = tf["words"][:, b, off: off + (q_ + 63) // 64]
    tc["words"] = words
    lse_c = torch.empty((chunk.q.shape[0], 6), dtype=torch.float32, device="cuda:0")
    oc = gp.attn(chunk, tc, lse=lse_c)
    torch.cuda.synchronize()
    for b, (q_, k_) in enumerate(zip(Lq, Lk)):
        s0q, s0k = int(chunk.cu_seqlens[b]), int(full.cu_seqlens[b])
        assert torch.equal(oc[s0q:s0q + q_], of[s0k + k_ - q_:s0k + k_])
        assert torch.equal(lse_c[s0q:s0q + q_], lse_f[s0k + k_ - q_:s0k + k_])


def test_attn_decode_kernel_matches_prefill_kernel(gp):
    """Decode calls run on the decode kernel (heads as rows, waves splitting the
    keys); the debug entry point runs the same call on the fused prefill kernel.
    Both meet the oracle bar and agree with each other within it, and the
    decode kernel's row log-sum-exp matches the oracle's."""
    import torch
    _announce("decode kernel vs prefill kernel")
    w = make_chunked_workload(535, lengths_q=[1] * 24, lengths_k=[1 + 97 * i for i in range(24)], num_q_heads=12,
                              num_kv_heads=4, head_dim=128, g=2, p=0.5, outliers=True, kv_int8=True)
    t = gp.prepare(w)
    lse = torch.empty((24, 12), dtype=torch.float32, device="cuda:0")
    dec = gp.attn(w, t, lse=lse)
    gen, _, _, _ = gp.attn_debug(w, t, seq=0, q_head=0)
    torch.cuda.synchronize()
    ref, ref_lse = orc.attn_prefill(oracle_inputs(w), with_lse=True)
    for o in (dec, gen):
        ma, rf = gp.errors(o.cpu().numpy(), ref)
        assert ma <= MAX_ABS and rf <= REL_FRO
    ma, _ = gp.errors(dec.cpu().numpy(), gen.cpu().numpy().astype(np.float64))
    assert ma <= MAX_ABS
    assert float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse))) <= LSE_ABS


def test_decode_step_graph_replay(gp):
    """A decode step (quantise the new queries, pack routes, attention) captured
    in a HIP graph: every replay, with eager calls and synchronisations between
    replays, gives the eager step's bits."""
    import torch
    _announce("decode step graph replay")
    w = make_chunked_workload(536, lengths_q=[1] * 16, lengths_k=[100 + 61 * i for i in range(16)], num_q_heads=8,
                              num_kv_heads=2, head_dim=128, g=1, p=0.5, outliers=True, kv_int8=True)
    t = gp.prepare(w)
    tm = gp.tm
    plan = tm.AttnPlan(tm.AttnProblem(w.batch, w.max_seqlen, 8, 2, 128, 1, w.blk_q, w.sm_scale, True, True, False,
                                      w.max_seqlen_k), "cuda:0")
    out = torch.empty((16, 8, 128), dtype=torch.float32, device="cuda:0")
    kw = dict(cu_seqlens_k=t["cu_k"], max_seqlen_k=w.max_seqlen_k)

    def step(stream):
        tm.tilemix_quantize_blockwise(t["q"], t["cu"], w.max_seqlen, w.blk_q, t["q_q"], t["q_s"], stream=stream)
        tm.tilemix_build_route_mask(t["tile_route"], t["cu"], w.max_seqlen, w.g, t["words"], stream=stream, **kw)
        plan.run(t["q"], t["k8"], t["v8"], t["q_q"], t["q_s"], None, t["k_s"], t["cu"], t["words"], out,
                 v_scale=t["v_s"], stream=stream, cu_seqlens_k=t["cu_k"])

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for _ in range(3):
        out.zero_()
        step(torch.cuda.current_stream())          # eager work between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    ma, rf = gp.errors(eager.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_prefill_step_three_streams_graph_replay(gp):
    """A prefill step as the benchmark runs it: route packing and the work list
    on one stream, K quantised on a second, Q on the capture stream, then the
    planned attention after joining all three.  Captured in a HIP graph: every
    replay, with eager steps and synchronisations between replays, gives the
    eager step's bits, and the eager step matches the oracle."""
    import torch
    _announce("prefill step three streams graph replay")
    w = make_workload(537, lengths=[64 * 5 + 17, 64 * 3, 29], num_q_heads=6, num_kv_heads=2, head_dim=128, g=1,
                      p=0.75, outliers=True)
    t = gp.prepare(w)
    tm = gp.tm
    plan = tm.AttnPlan(tm.AttnProblem(w.batch, w.max_seqlen, 6, 2, 128, 1, w.blk_q, w.sm_scale, False, True, False),
                       "cuda:0")
    out = torch.empty((int(w.cu_seqlens[-1]), 6, 128), dtype=torch.float32, device="cuda:0")
    side, kvs = torch.cuda.Stream(), torch.cuda.Stream()

    def step(stream):
        side.wait_stream(stream)
        kvs.wait_stream(stream)
        with torch.cuda.stream(side):
            tm.tilemix_build_route_mask(t["tile_route"], t["cu"], w.max_seqlen, w.g, t["words"], stream=side)
            plan.schedule(t["cu"], stream=side)
        with torch.cuda.stream(kvs):
            tm.tilemix_quantize_blockwise(t["k"], t["cu"], w.max_seqlen, 64, t["k_q"], t["k_s"], stream=kvs)
        tm.tilemix_quantize_blockwise(t["q"], t["cu"], w.max_seqlen, w.blk_q, t["q_q"], t["q_s"], stream=stream)
        stream.wait_stream(side)
        stream.wait_stream(kvs)
        plan.run_planned(t["q"], t["k"], t["v"], t["q_q"], t["q_s"], t["k_q"], t["k_s"], t["cu"], t["words"], out,
                         stream=stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for _ in range(3):
        out.zero_()
        t["words"].zero_()
        step(torch.cuda.current_stream())          # eager work between replays
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        t["words"].fill_(-1)                       # the replay must rebuild them
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    ma, rf = gp.errors(eager.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_attn_chunked_debug_bitexact(gp):
    """Chunked prefill: INT32 score tiles, visits and decoded routes bit-exact
    (the causal edge cuts two key tiles for some query tiles)."""
    import torch
    _announce("attn chunked debug")
    w = make_chunked_workload(530, lengths_q=[150, 40], lengths_k=[500, 40], num_q_heads=3, num_kv_heads=1,
                              head_dim=128, g=1, p=0.6, outliers=True)
    t = gp.prepare(w)
    out, s32, visits, used = gp.attn_debug(w, t, seq=0, q_head=2)
    torch.cuda.synchronize()
    inp = oracle_inputs(w)
    assert np.array_equal(s32.cpu().numpy(), orc.s32_tiles(inp, 0, 2, 0, w.T))
    vis = orc.visit_matrix(w.cu_seqlens, w.max_seqlen, w.num_q_heads, w.cu_seqlens_k, w.max_seqlen_k)
    assert np.array_equal(visits.cpu().numpy().astype(np.uint32), vis)
    assert np.array_equal(used.cpu().numpy(), orc.route_used(inp))
    ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(inp))
    assert ma <= MAX_ABS and rf <= REL_FRO


def test_attn_prefill_lse(gp):
    """Prefill log-sum-exp of every query row against the oracle's."""
    import torch
    _announce("attn prefill lse")
    w = make_workload(540, lengths=[300, 1, 129], num_q_heads=6, num_kv_heads=2, head_dim=128, g=1, p=0.5,
                      outliers=True)
    t = gp.prepare(w)
    lse = torch.empty((w.q.shape[0], 6), dtype=torch.float32, device="cuda:0")
    gp.attn(w, t, lse=lse)
    torch.cuda.synchronize()
    _, ref_lse = orc.attn_prefill(oracle_inputs(w), with_lse=True)
    assert float(np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse))) <= LSE_ABS


def _sample_rows(w, rng, n):
    """(sequence, query-tile row) samples of a full-size workload: tiles 0, 1,
    T-1 and T-2 of the longest, the shortest and the first sequence, the first
    and last tile of route groups (g boundaries), then random rows up to n."""
    spans = orc.seq_spans(w.cu_seqlens)
    lens = [L for _, L in spans]
    out = set()
    b_long, b_short = int(np.argmax(lens)), int(np.argmin(lens))
    for b in sorted({b_long, b_short, 0}):
        Tb = orc.num_tiles(lens[b])
        for m in (0, 1, Tb - 1, Tb - 2):
            if 0 <= m < Tb:
                out.add((b, m))
        for j in range(1, min(64, (Tb + w.g - 1) // w.g)):   # group boundaries
            for m in (j * w.g - 1, j * w.g):
                if m < Tb and len(out) < n // 2:
                    out.add((b, m))
    while len(out) < n:
        b = int(rng.integers(len(lens)))
        out.add((b, int(rng.integers(orc.num_tiles(lens[b])))))
    return sorted(out)


def _nan_out(w, dev="cuda:0"):
    import torch
    return torch.full((int(w.cu_seqlens[-1]), w.num_q_heads, w.head_dim), float("nan"), dtype=torch.float32,
                      device=dev)


def _compare_rows(gp, inp, got_all, rows, label=""):
    """Max-abs and relative Frobenius error of the sampled tile rows {(b, hq, m): ref}."""
    num = den = 0.0
    ma = 0.0
    for (b, hq, m), ref in rows.items():
        s0, L = inp.spans[b]
        got = got_all[s0 + m * 64:s0 + min(m * 64 + 64, L), hq].astype(np.float64)
        ma = max(ma, float(np.max(np.abs(got - ref))))
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    rf = (num / den) ** 0.5
    gp.record(ma, rf, label)
    return ma, rf


def _operands_bitexact(gp, w, t, inp):
    """Route words, Q8 and its scales, and K8 / K scales (INT8 cache: K8, V8 and
    both scales) of the library equal the oracle's, in full."""
    assert np.array_equal(gp.words_u64(t["words"]), inp.words)
    assert np.array_equal(t["q_q"].cpu().numpy(), inp.q_q)
    assert np.array_equal(t["q_s"].cpu().numpy().view(np.uint32), inp.q_scale.view(np.uint32))
    kq = t["k8"] if w.kv_int8 else t["k_q"]
    assert np.array_equal(kq.cpu().numpy(), inp.k_q)
    assert np.array_equal(t["k_s"].cpu().numpy().view(np.uint32), inp.k_scale.view(np.uint32))
    if w.kv_int8:
        assert np.array_equal(t["v8"].cpu().numpy(), inp.v_q)
        assert np.array_equal(t["v_s"].cpu().numpy().view(np.uint32), inp.v_scale.view(np.uint32))


@pytest.mark.parametrize("cfg,nsamp", [(2, 0), (3, 16), (4, 12), (5, 12)])
def test_standard_config_full_size(gp, cfg, nsamp):
    """Full-size workloads in the launch configuration the bench times.  The
    output buffers start as NaN and every element must come back finite (a
    work item dropped or never written would show).  All INT8 operands, their
    scales and the route words are bit-exact in full.  The 3B-shaped layer
    (config 2) is compared with the oracle in full, every row of every head;
    configs 3-5 on sampled query-tile rows, every query head of each.  For an
    fp16 K/V the bench's operand mode (Q's INT8 operands made in the kernel)
    gives the same bits."""
    import torch
    from tests import oracle_pool
    _announce(f"config {cfg} full size" + (f", {nsamp} sampled rows x all heads" if nsamp else ", compared in full"))
    w = config(cfg)
    t = gp.prepare(w)
    out = gp.attn(w, t, out=_nan_out(w))
    # the bench's operand mode for an fp16 K/V: Q's INT8 operands made in the kernel
    qotf = None if w.kv_int8 else gp.attn(w, t, otf=2, out=_nan_out(w))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    if qotf is not None:
        assert torch.equal(qotf, out)
        del qotf
    inp = oracle_inputs(w)
    _operands_bitexact(gp, w, t, inp)
    got_all = out.cpu().numpy()
    if nsamp == 0:
        ref = oracle_pool.full_output(inp)
        ma, rf = gp.errors(got_all, ref)
        print(f"  {w.name}: max_abs={ma:.3e} rel_fro={rf:.3e} over all {got_all.shape[0]} x {w.num_q_heads} rows")
    else:
        bm = _sample_rows(w, np.random.default_rng(cfg), nsamp)
        rows = oracle_pool.tile_rows(inp, [(b, hq, m) for b, m in bm for hq in range(w.num_q_heads)])
        ma, rf = _compare_rows(gp, inp, got_all, rows)
        print(f"  {w.name}: max_abs={ma:.3e} rel_fro={rf:.3e} over {len(bm)} tile rows x {w.num_q_heads} heads")
    assert ma <= MAX_ABS and rf <= REL_FRO


@pytest.fixture(scope="module")
def long_context(gp):
    """The long-context workload's inputs, uploaded once for the coverage sweep."""
    w = config(5)
    t = gp.upload(w)
    inp = oracle_inputs(w)
    return w, t, inp


@pytest.mark.parametrize("p", [0.0, 0.25, 0.75, 1.0])
def test_long_context_coverage_sweep_full_length(gp, long_context, p):
    """The long-context workload (L = 65536, 32/8 heads, g = 16: 64 route groups
    per row at full length) at INT8 coverage 0/25/75/100 % of the tile groups
    (50 % is the standard case): NaN-initialised output finite everywhere; rows
    0, 1, 1022, 1023, both sides of two group boundaries and a middle row, every
    query head, against the oracle."""
    import torch
    from tests import oracle_pool
    from workloads import route_bernoulli_groups
    _announce(f"config 5 full length, coverage {p}")
    w, t0, inp = long_context
    tr = route_bernoulli_groups(5, w.num_kv_heads, [int(x) for x in w.lengths], w.T, w.g, p)
    t = dict(t0, tile_route=torch.from_numpy(tr).to("cuda:0"))
    t = gp.prepare(w, t=t)
    out = gp.attn(w, t, out=_nan_out(w))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    inp.words = orc.build_route_mask(tr, w.cu_seqlens, w.max_seqlen, w.g)
    assert np.array_equal(gp.words_u64(t["words"]), inp.words)
    if p in (0.0, 1.0):
        legal_groups = [(int(inp.words[hk, 0, m]), m // w.g + 1) for hk in range(w.num_kv_heads) for m in (1023,)]
        assert all(wd == (0 if p == 0.0 else (1 << n) - 1) for wd, n in legal_groups)
    ms = (0, 1, 255, 256, 511, 512, 700, 1022, 1023)
    rows = oracle_pool.tile_rows(inp, [(0, hq, m) for m in ms for hq in range(w.num_q_heads)])
    ma, rf = _compare_rows(gp, inp, out.cpu().numpy(), rows, label=f"p={p}")
    print(f"  p={p}: max_abs={ma:.3e} rel_fro={rf:.3e} over {len(rows)} tile rows")
    assert ma <= MAX_ABS and rf <= REL_FRO


@pytest.mark.parametrize("mode,nsamp", [("prefill", 24), ("decode", 64)])
def test_chunked_bench_workloads_sampled(gp, mode, nsamp):
    """The chunked-prefill and decode benchmark workloads at full size (512 new
    tokens over 4096 cached keys, batch 8; one token over 4096 cached keys,
    batch 64; 24/8 heads, d 128, INT8 cache, 75 % INT8), run as one call:
    sampled query-tile rows and their log-sum-exp against the oracle."""
    import torch
    _announce(f"chunked bench workload {mode} sampled ({nsamp})")
    if mode == "prefill":
        w = make_chunked_workload(6, lengths_q=[512] * 8, lengths_k=[4096] * 8, num_q_heads=24, num_kv_heads=8,
                                  head_dim=128, g=1, p=0.75, outliers=True, kv_int8=True)
    else:
        w = make_chunked_workload(7, lengths_q=[1] * 64, lengths_k=[4096] * 64, num_q_heads=24, num_kv_heads=8,
                                  head_dim=128, g=1, p=0.75, outliers=True, kv_int8=True)
    t = gp.prepare(w)
    lse = torch.empty((w.q.shape[0], 24), dtype=torch.float32, device="cuda:0")
    out = gp.attn(w, t, lse=lse)
    torch.cuda.synchronize()
    inp = oracle_inputs(w)
    assert np.array_equal(gp.words_u64(t["words"]), inp.words)
    got_all, lse_all = out.cpu().numpy(), lse.cpu().numpy()
    rng = np.random.default_rng(61 if mode == "prefill" else 62)
    errs, lerrs, num, den = [], [], 0.0, 0.0
    for _ in range(nsamp):
        b, hq = int(rng.integers(w.batch)), int(rng.integers(24))
        s0, L = inp.spans[b]
        m = int(rng.integers(orc.num_tiles(L)))
        i0, i1 = m * 64, min(m * 64 + 64, L)
        ref, ref_lse = orc.attn_tile_row(inp, b, hq, m, with_lse=True)
        got = got_all[s0 + i0:s0 + i1, hq].astype(np.float64)
        errs.append(np.max(np.abs(got - ref)))
        lerrs.append(np.max(np.abs(lse_all[s0 + i0:s0 + i1, hq].astype(np.float64) - ref_lse)))
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    ma, rf = max(errs), (num / den) ** 0.5
    gp.record(ma, rf)
    print(f"  {mode}: max_abs={ma:.3e} rel_fro={rf:.3e} lse={max(lerrs):.3e} over {nsamp} rows")
    assert ma <= MAX_ABS and rf <= REL_FRO and max(lerrs) <= LSE_ABS


def test_attn_strided_layouts_bitexact(gp):
    """Addressing only: the same operands in other memory layouts give the same
    bits.  Q, K and V as views into one packed QKV buffer (token stride
    (Hq + 2 Hk) d); an INT8 KV cache stored head-major ([Hk][N][d] viewed as
    [N][Hk][d]) for chunked prefill and for decode."""
    import torch
    _announce("attn strided layouts")
    w = make_workload(538, lengths=[200, 64, 130, 1], num_q_heads=6, num_kv_heads=2, head_dim=128, g=1, p=0.6,
                      outliers=True)
    t = gp.prepare(w)
    ref = gp.attn(w, t).clone()
    N = int(w.cu_seqlens[-1])
    qkv = torch.empty((N, 10, 128), dtype=torch.float16, device="cuda:0")
    qkv[:, :6], qkv[:, 6:8], qkv[:, 8:] = t["q"], t["k"], t["v"]
    t2 = dict(t, q=qkv[:, :6], k=qkv[:, 6:8], v=qkv[:, 8:])
    assert torch.equal(gp.attn(w, t2), ref)
    for seed, lq, lk in ((539, [130, 64, 7], [900, 64, 300]), (540, [1] * 9, [1, 63, 64, 65, 200, 511, 1000, 2049, 3000])):
        w = make_chunked_workload(seed, lengths_q=lq, lengths_k=lk, num_q_heads=6, num_kv_heads=2, head_dim=128, g=1,
                                  p=0.6, outliers=True, kv_int8=True)
        t = gp.prepare(w)
        ref = gp.attn(w, t).clone()
        head_major = lambda x: x.transpose(0, 1).contiguous().transpose(0, 1)
        t2 = dict(t, k8=head_major(t["k8"]), v8=head_major(t["v8"]))
        assert t2["k8"].stride(0) == 128 and t2["k8"].stride(1) == int(w.cu_seqlens_k[-1]) * 128
        assert torch.equal(gp.attn(w, t2), ref)


def _big_stride_views(k, v, stride):
    """K and V of one KV head ([N][1][d] host arrays) placed in one device buffer
    of `stride` elements per token (K in channels 0..d-1, V in d..2d-1): views
    [N][1][d] whose token stride is `stride`."""
    import torch
    N, _, d = k.shape
    dtype = torch.float16 if k.dtype == np.float16 else torch.int8
    buf = torch.zeros((N, stride), dtype=dtype, device="cuda:0")
    buf[:, :d] = torch.from_numpy(np.ascontiguousarray(k[:, 0])).to("cuda:0")
    buf[:, d:2 * d] = torch.from_numpy(np.ascontiguousarray(v[:, 0])).to("cuda:0")
    return buf, buf[:, None, :d], buf[:, None, d:2 * d]


@pytest.mark.parametrize("case", ["prefill_fp16", "decode_fp16", "prefill_int8kv_gqa3"])
def test_attn_kv_stride_beyond_4gib(gp, case):
    """K/V tiles are read through 32-bit buffer ranges.  Here K and V are views
    with a token stride of 4 MiB over 2100 keys, so a sequence's keys span about
    8.8 GB while each 64-row tile spans 256 MiB: the fused prefill kernel (fp16
    K/V, and an INT8 cache with three heads per item) and the decode kernel
    against the oracle."""
    import torch
    _announce(f"attn k/v stride beyond 4 GiB: {case}")
    L = 2100
    if case == "decode_fp16":
        w = make_chunked_workload(542, lengths_q=[1], lengths_k=[L], num_q_heads=3, num_kv_heads=1, head_dim=128,
                                  g=1, p=0.5, outliers=True)
    else:
        w = make_workload(541, lengths=[L], num_q_heads=3, num_kv_heads=1, head_dim=128, g=1, p=0.5,
                          outliers=True, kv_int8=case.endswith("gqa3"))
    t = gp.prepare(w)
    ref_out = gp.attn(w, t).clone()          # compact K/V, for the bits
    if w.kv_int8:
        stride = 1 << 22                       # int8 elements = bytes
        buf, k8v, v8v = _big_stride_views(t["k8"].cpu().numpy(), t["v8"].cpu().numpy(), stride)
        t = dict(t, k8=k8v, v8=v8v)
        span = (L - 1) * stride + 256
    else:
        stride = 1 << 21                       # fp16 elements: 4 MiB per token
        buf, kv, vv = _big_stride_views(w.k, w.v, stride)
        t = dict(t, k=kv, v=vv)
        span = ((L - 1) * stride + 256) * 2
    assert span > (1 << 32) and 64 * stride * buf.element_size() < (1 << 32)
    out = gp.attn(w, t, out=_nan_out(w))
    torch.cuda.synchronize()
    del buf
    assert torch.equal(out, ref_out)         # addressing only: the same bits as the compact layout
    ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
    print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
    assert ma <= MAX_ABS and rf <= REL_FRO


@pytest.mark.parametrize("case", ["gqa3_lds_staging", "gqa2_register_staging", "decode"])
def test_attn_kv_int8_tiny_and_zero_v_scales(gp, case):
    """INT8 KV cache with v scales below 2^-24 and a caller-stored zero v scale.
    The second sequence's V is ~1e-6 (its scales ~3e-8), so its output is ~1e-6
    and only its own relative error would see a misapplied scale; one V block
    of the first sequence has its scale set to 0 on both sides (its values then
    count as zero, its probabilities still in the row sums)."""
    import torch
    _announce(f"attn INT8 cache tiny / zero v scales: {case}")
    hq = {"gqa3_lds_staging": 6, "gqa2_register_staging": 4, "decode": 6}[case]
    if case == "decode":
        w = make_chunked_workload(544, lengths_q=[1, 1], lengths_k=[300, 200], num_q_heads=hq, num_kv_heads=2,
                                  head_dim=128, g=1, p=0.5, outliers=True, kv_int8=True)
    else:
        w = make_workload(543, lengths=[300, 200], num_q_heads=hq, num_kv_heads=2, head_dim=128, g=1, p=0.5,
                          outliers=True, kv_int8=True)
    cu_k = w.cu_seqlens if w.cu_seqlens_k is None else w.cu_seqlens_k
    s1 = int(cu_k[1])
    w.v[s1:] = (w.v[s1:].astype(np.float32) * np.float32(1e-6)).astype(np.float16)
    t = gp.prepare(w)
    inp = oracle_inputs(w)
    assert np.all(inp.v_scale[:, 1, :4] < 2.0 ** -24) and np.all(inp.v_scale[:, 1, :4] > 0)
    t["v_s"][0, 0, 2] = 0.0
    inp.v_scale[0, 0, 2] = 0.0
    inp._kv_cache.clear()
    out = gp.attn(w, t, out=_nan_out(w))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    ref = orc.attn_prefill(inp)
    q1 = int(w.cu_seqlens[1])
    for label, sl in (("seq0", slice(0, q1)), ("seq1 tiny v", slice(q1, None))):
        ma, rf = gp.errors(got[sl], ref[sl], label=label)
        print(f"  {label}: max_abs={ma:.3e} rel_fro={rf:.3e} (|ref| max {np.max(np.abs(ref[sl])):.2e})")
        assert ma <= MAX_ABS and rf <= REL_FRO
