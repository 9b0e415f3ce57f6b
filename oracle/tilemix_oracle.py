"""CPU oracle for routed FP16/INT8 causal prefill attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``.
The product path (the HIP library and its Python binding) never does, and this
module imports nothing from the product.

It is a plain, slow, step-by-step NumPy implementation in float64 (INT8 dot
products in exact int64) of what the method computes, written from the pages:

  [PL §n]  paperlayer.ai summary of arXiv 2608.17336, "TileMix: Tile-Centric
           Mixed-Precision Attention for LLM Inference Acceleration", section n
           (App. B/C/D are its appendix bullets).
  [AN]     ainews.surl.tw, "TileMix Mixes FP16 and INT8 Within the Attention
           Matrix, Reaching 2.22x FlashAttention Throughput for 4K Prefill on A100".
  [GS]     gist.science technical summary (Spanish), "Resumen Tecnico", subsection
           "Enrutamiento por Mascara de Bits Compacta".

Readings taken where the pages leave a step open are restated at each
function that takes them.

Conventions (all readings):
  * score tiles are 64 x 64 (BLOCK_M = BLOCK_N = 64);
  * route bit 1 = INT8 path, 0 = FP16 path; bit j of a row's word covers key
    tiles [j*g, j*g+g); LSB = group 0;
  * tokens are packed ``[N][H][d]`` with int32 prefix sums ``cu_seqlens``;
    per-block scales are ``float32 [H][B][ceil(max_seqlen/blk)]``; route words
    are ``uint64 [Hk][B][T]`` with ``T = ceil(max_seqlen/64)``;
  * GQA: query head hq reads KV head ``hq // (Hq // Hk)``;
  * causal alignment: a sequence's Lq queries are its last Lq positions of Lk
    keys (bottom-right alignment; prefill is Lq = Lk): key j is legal for query
    i iff j <= (Lk - Lq) + i and i < Lq.  Query tiles m count from the first
    query, key tiles n from the first key; route words are ``[Hk][B][Tq]`` with
    bits over key tiles.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK_M = 64
BLOCK_N = 64
QMAX = 127
INT32_MIN = -(2 ** 31)


def _cdiv(a: int, b: int) -> int:
    return (a + b - 1) // b


def seq_spans(cu_seqlens) -> List[Tuple[int, int]]:
    cu = [int(x) for x in np.asarray(cu_seqlens)]
    return [(cu[b], cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]


# ---------------------------------------------------------------------------
# O1. Blockwise symmetric INT8 quantisation [PL §3 Preliminaries; PL App. C]
# ---------------------------------------------------------------------------

def quantize_blockwise(x: np.ndarray, cu_seqlens, max_seqlen: int, blk: int):
    """Blockwise symmetric INT8 quantisation of a packed ``[N][H][d]`` tensor.

    The pages quantise Q and K block by block with one scale per block
    ([PL §3 Preliminaries], [PL App. C], BLKQ = 128 and BLKK = 64 in the paper).
    Reading taken: a block is ``blk`` consecutive tokens of one sequence and one
    head, over all d channels; blocks restart at each sequence start; the range
    is symmetric [-127, 127] with divisor 127.  For each block:

        a     = max |x|                       (exact; fp16 -> fp32)
        scale = fl32(a / 127)                 (one correctly rounded fp32 division)
        q     = clamp(rint_half_even(fl32(x / scale)), -127, 127)

    and an all-zero block gets scale 1.0 and q = 0.  Scale entries for blocks
    past a sequence's end are 0.

    Returns ``(q int8 [N][H][d], scales float32 [H][B][ceil(max_seqlen/blk)])``.
    """
    if x.dtype != np.float16:
        raise TypeError("x must be float16")
    N, H, d = x.shape
    spans = seq_spans(cu_seqlens)
    nb = _cdiv(int(max_seqlen), blk)
    xq = np.zeros((N, H, d), dtype=np.int8)
    scales = np.zeros((H, len(spans), nb), dtype=np.float32)
    for b, (s0, L) in enumerate(spans):
        for kb in range(_cdiv(L, blk)):
            r0, r1 = s0 + kb * blk, s0 + min((kb + 1) * blk, L)
            block = x[r0:r1].astype(np.float32)            # [rows][H][d], exact
            for h in range(H):
                xb = block[:, h, :]
                a = np.float32(np.max(np.abs(xb)))
                if a == np.float32(0.0):
                    scale = np.float32(1.0)
                    q = np.zeros_like(xb, dtype=np.int8)
                else:
                    scale = np.float32(a / np.float32(QMAX))  # fp32 / fp32 -> fp32, IEEE rounded
                    r = (xb / scale).astype(np.float32)       # fp32 elementwise division
                    q = np.clip(np.rint(r), -QMAX, QMAX).astype(np.int8)
                xq[r0:r1, h, :] = q
                scales[h, b, kb] = scale
    return xq, scales


# ---------------------------------------------------------------------------
# O2. Legality [PL §3 Preliminaries; PL App. B]
# ---------------------------------------------------------------------------

def num_tiles(L: int) -> int:
    return _cdiv(int(L), BLOCK_M)


def tile_is_legal(m: int, n: int, Tb: int) -> bool:
    """Causal and sequence-boundary legality of score tile (m, n), independent of
    routing ([PL §3 Preliminaries], [PL App. B]); prefill (Lq = Lk)."""
    return 0 <= n <= m < Tb


def last_key_tile(m: int, Lq: int, Lk: int) -> int:
    """Last key tile a query tile m may touch when the Lq queries are the last
    Lq of Lk positions: the tile of key (Lk - Lq) + min(64 m + 63, Lq - 1).
    Prefill (Lq = Lk) gives m."""
    return ((Lk - Lq) + min(m * BLOCK_M + BLOCK_M - 1, Lq - 1)) // BLOCK_N


def _pairs(cu_seqlens, cu_seqlens_k):
    """Per sequence (Lq, Lk); cu_seqlens_k None means Lk = Lq."""
    sq = seq_spans(cu_seqlens)
    sk = sq if cu_seqlens_k is None else seq_spans(cu_seqlens_k)
    if len(sk) != len(sq):
        raise ValueError("cu_seqlens and cu_seqlens_k differ in batch")
    out = []
    for (_, Lq), (_, Lk) in zip(sq, sk):
        if Lk < Lq:
            raise ValueError("a sequence has more queries than keys")
        out.append((Lq, Lk))
    return out


def visit_matrix(cu_seqlens, max_seqlen: int, num_q_heads: int, cu_seqlens_k=None,
                 max_seqlen_k: Optional[int] = None) -> np.ndarray:
    """uint32 [B][Hq][Tq][Tk]: how often a correct kernel visits each score tile.

    Every legal tile group is executed ([PL §3 Preliminaries]) and nothing else:
    1 on legal tiles, 0 elsewhere.
    """
    pairs = _pairs(cu_seqlens, cu_seqlens_k)
    Tq = num_tiles(max_seqlen)
    Tk = num_tiles(max_seqlen if max_seqlen_k is None else max_seqlen_k)
    out = np.zeros((len(pairs), num_q_heads, Tq, Tk), dtype=np.uint32)
    for b, (Lq, Lk) in enumerate(pairs):
        for m in range(num_tiles(Lq)):
            out[b, :, m, : last_key_tile(m, Lq, Lk) + 1] = 1
    return out


# ---------------------------------------------------------------------------
# O3. Packed 64-bit route words and their decode
#     [PL §3 Preliminaries; PL §4; PL App. D; AN; GS]
# ---------------------------------------------------------------------------

def build_route_mask(tile_route: np.ndarray, cu_seqlens, max_seqlen: int, g: int, cu_seqlens_k=None,
                     max_seqlen_k: Optional[int] = None) -> np.ndarray:
    """Pack per-tile decisions into one uint64 per (KV head, sequence, query-tile row).

    One bit governs a group of g adjacent key tiles and bit floor(n/g) selects
    the path of key tile n ([PL §3 Preliminaries], [PL §4]); one 64-bit word per
    (KV head, query-tile row) ([PL App. D], [AN]).  Readings: bit value 1 = INT8;
    a group's bit is the AND of its *legal* tiles' decisions (FP16 wins when they
    disagree); bits of groups with no legal tile, and whole rows past the
    sequence end, are 0.  More than 64 groups per row is an error.

    tile_route: uint8 [Hk][B][Tq][Tk] (nonzero = INT8).  Returns uint64 [Hk][B][Tq].
    With cu_seqlens_k (chunked prefill) the legal tiles of row m are
    n <= last_key_tile(m, Lq, Lk).
    """
    Hk, B, Tq, Tk = tile_route.shape
    Tk_want = num_tiles(max_seqlen if max_seqlen_k is None else max_seqlen_k)
    if Tq != num_tiles(max_seqlen) or Tk != Tk_want:
        raise ValueError("tile_route must be [Hk][B][Tq][Tk] with Tq, Tk = ceil(max_seqlen(_k)/64)")
    if g < 1 or _cdiv(Tk, g) > 64:
        raise ValueError("more than 64 route groups per row")
    pairs = _pairs(cu_seqlens, cu_seqlens_k)
    words = np.zeros((Hk, B, Tq), dtype=np.uint64)
    for hk in range(Hk):
        for b, (Lq, Lk) in enumerate(pairs):
            for m in range(num_tiles(Lq)):
                nl = last_key_tile(m, Lq, Lk)
                w = 0
                for j in range(nl // g + 1):
                    n0, n1 = j * g, min(j * g + g, nl + 1)   # legal tiles of group j
                    if all(int(tile_route[hk, b, m, n]) != 0 for n in range(n0, n1)):
                        w |= 1 << j
                words[hk, b, m] = np.uint64(w)
    return words


def route_bit(word: int, n: int, g: int) -> int:
    """R = (b >> floor(n/g)) & 1: constant-time decode of key tile n's path
    ([GS], [PL §3 Preliminaries])."""
    return (int(word) >> (n // g)) & 1


def decode_route_mask(words: np.ndarray, cu_seqlens, max_seqlen: int, g: int, cu_seqlens_k=None,
                      max_seqlen_k: Optional[int] = None) -> np.ndarray:
    """uint8 [Hk][B][Tq][Tk]: the decoded path of every legal tile, 0xFF on illegal tiles."""
    Hk, B, Tq = words.shape
    if Tq != num_tiles(max_seqlen):
        raise ValueError("words must be [Hk][B][Tq]")
    Tk = num_tiles(max_seqlen if max_seqlen_k is None else max_seqlen_k)
    pairs = _pairs(cu_seqlens, cu_seqlens_k)
    out = np.full((Hk, B, Tq, Tk), 0xFF, dtype=np.uint8)
    for hk in range(Hk):
        for b, (Lq, Lk) in enumerate(pairs):
            for m in range(num_tiles(Lq)):
                w = int(words[hk, b, m])
                for n in range(last_key_tile(m, Lq, Lk) + 1):
                    out[hk, b, m, n] = route_bit(w, n, g)
    return out


# ---------------------------------------------------------------------------
# Static routing templates [PL App. B], [PL Limitations], [GS]
# ---------------------------------------------------------------------------
# The pages list All-FP16, All-INT8, Band, Global, Row-Random, Aligned-Sparse,
# BigBird and SpTrans layouts, built statically and data-free, at a target INT8
# coverage of the legal tile groups, but print no definitions.  Readings taken
# (all per query-tile row, over its legal groups j = 0 .. n-1 where n =
# last_key_tile(m) // g + 1; F FP16 groups, F = round((1 - p) n) in exact
# integer arithmetic with p in per mille; every other legal group is INT8):
#   band:           the F groups nearest the diagonal (j >= n - F);
#   global:         the first F groups (j < F);
#   row_random:     the F groups with the smallest splitmix64 keys;
#   aligned_sparse: F evenly spaced groups j = floor(k n / F), k = 0 .. F-1;
#   bigbird:        ceil(F/3) band groups, then ceil((F - that)/2) first
#                   groups, then random groups (key order) up to F in total;
#   sptrans:        ceil(F/2) band groups, then the rest evenly spaced over
#                   the groups before the band (local + strided).
# BigBird and SpTrans are approximations of those papers' patterns at this
# granularity.

TEMPLATES = ("all_fp16", "all_int8", "band", "global", "row_random", "aligned_sparse", "bigbird", "sptrans")
_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 output function (Steele, Lea and Flood, 2014) of a 64-bit value."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def template_key(seed: int, hk: int, b: int, m: int, j: int, batch: int, Tq: int) -> int:
    """Random key of group j of row (hk, b, m): splitmix64 of seed XOR a unique counter."""
    return splitmix64((int(seed) ^ ((((hk * batch + b) * Tq + m) * 64) + j)) & _M64)


def fp16_groups(kind: str, n: int, permille: int, keys) -> set:
    """The FP16 groups of one row with n legal groups (readings above)."""
    if kind == "all_fp16":
        return set(range(n))
    if kind == "all_int8":
        return set()
    F = ((1000 - permille) * n + 500) // 1000
    by_key = sorted(range(n), key=lambda j: (keys[j], j))
    if kind == "band":
        return set(range(n - F, n))
    if kind == "global":
        return set(range(F))
    if kind == "row_random":
        return set(by_key[:F])
    if kind == "aligned_sparse":
        return {k * n // F for k in range(F)}
    if kind == "bigbird":
        w = (F + 2) // 3
        s = set(range(n - w, n))
        s |= set(range((F - w + 1) // 2))
        for j in by_key:
            if len(s) >= F:
                break
            s.add(j)
        return s
    if kind == "sptrans":
        w = (F + 1) // 2
        k = F - w
        s = set(range(n - w, n))
        s |= {i * (n - w) // k for i in range(k)} if k else set()
        return s
    raise ValueError(kind)


def template_route_words(kind: str, permille: int, seed: int, cu_seqlens, max_seqlen: int, num_kv_heads: int,
                         g: int, cu_seqlens_k=None, max_seqlen_k: Optional[int] = None) -> np.ndarray:
    """uint64 [Hk][B][Tq]: route words of a static template (bit j = 1: group j INT8)."""
    if kind not in TEMPLATES or not 0 <= permille <= 1000:
        raise ValueError("template")
    pairs = _pairs(cu_seqlens, cu_seqlens_k)
    Tq = num_tiles(max_seqlen)
    Tk = num_tiles(max_seqlen if max_seqlen_k is None else max_seqlen_k)
    if g < 1 or _cdiv(Tk, g) > 64:
        raise ValueError("more than 64 route groups per row")
    B = len(pairs)
    words = np.zeros((num_kv_heads, B, Tq), dtype=np.uint64)
    for hk in range(num_kv_heads):
        for b, (Lq, Lk) in enumerate(pairs):
            for m in range(num_tiles(Lq)):
                n = last_key_tile(m, Lq, Lk) // g + 1
                keys = [template_key(seed, hk, b, m, j, B, Tq) for j in range(n)]
                f = fp16_groups(kind, n, permille, keys)
                w = 0
                for j in range(n):
                    if j not in f:
                        w |= 1 << j
                words[hk, b, m] = np.uint64(w)
    return words


# ---------------------------------------------------------------------------
# O4-O6. Routed scores, streaming online softmax, normalisation
#        [PL §1; PL §3 Preliminaries; PL App. C; AN; GS]
# ---------------------------------------------------------------------------

class AttnInputs:
    """Host arrays of one attention call.

    kv_int8 = False: ``k``, ``v`` fp16 [N][Hk][d]; ``k_q`` int8 [N][Hk][d] and
        ``k_scale`` float32 [Hk][B][nb64] (64-token blocks) for INT8-routed tiles.
    kv_int8 = True: ``k_q``, ``v_q`` int8 [N][Hk][d] with ``k_scale``, ``v_scale``
        float32 [Hk][B][nb64]; the effective key/value is ``int8 * scale``.
    Always: ``q`` fp16 [N][Hq][d]; ``q_q`` int8 and ``q_scale`` float32
    [Hq][B][ceil(max_seqlen/blk_q)]; ``route_words`` uint64 [Hk][B][Tq].
    Chunked prefill: ``cu_seqlens_k`` / ``max_seqlen_k`` describe the keys (K, V
    and their scales are packed by them, Tk = ceil(max_seqlen_k/64) tiles);
    None means the keys are the queries' own positions (prefill).
    """

    def __init__(self, *, q, cu_seqlens, max_seqlen, num_kv_heads, route_words, g, sm_scale,
                 q_q=None, q_scale=None, blk_q=64, k=None, v=None, k_q=None, k_scale=None,
                 v_q=None, v_scale=None, kv_int8=False, cu_seqlens_k=None, max_seqlen_k=None):
        self.q, self.k, self.v = q, k, v
        self.q_q, self.q_scale, self.k_q, self.k_scale = q_q, q_scale, k_q, k_scale
        self.v_q, self.v_scale = v_q, v_scale
        self.cu = np.asarray(cu_seqlens).astype(np.int64)
        self.spans = seq_spans(self.cu)
        self.cu_k = self.cu if cu_seqlens_k is None else np.asarray(cu_seqlens_k).astype(np.int64)
        self.spans_k = seq_spans(self.cu_k)
        self.pairs = _pairs(self.cu, self.cu_k)
        self.max_seqlen = int(max_seqlen)
        self.max_seqlen_k = int(max_seqlen if max_seqlen_k is None else max_seqlen_k)
        self.Hq = int(q.shape[1])
        self.Hk = int(num_kv_heads)
        self.d = int(q.shape[2])
        self.words = route_words
        self.g = int(g)
        self.sm = float(np.float32(sm_scale))
        self.blk_q = int(blk_q)
        self.kv_int8 = bool(kv_int8)
        if self.Hq % self.Hk:
            raise ValueError("num_q_heads must be a multiple of num_kv_heads")
        self._kv_cache: Dict[Tuple[int, int], tuple] = {}

    def kv_head(self, hq: int) -> int:
        """GQA: contiguous groups of Hq/Hk query heads share one KV head ([PL §4])."""
        return hq // (self.Hq // self.Hk)

    def offset(self, b: int) -> int:
        """Position of query 0 of sequence b among its keys: Lk - Lq."""
        Lq, Lk = self.pairs[b]
        return Lk - Lq

    def _kv(self, b: int, hk: int):
        key = (b, hk)
        if key not in self._kv_cache:
            s0, L = self.spans_k[b]
            nblk = num_tiles(L)
            if self.kv_int8:
                ks = np.repeat(self.k_scale[hk, b, :nblk].astype(np.float64), BLOCK_N)[:L]
                vs = np.repeat(self.v_scale[hk, b, :nblk].astype(np.float64), BLOCK_N)[:L]
                kf = self.k_q[s0:s0 + L, hk].astype(np.float64) * ks[:, None]
                vf = self.v_q[s0:s0 + L, hk].astype(np.float64) * vs[:, None]
                k8 = self.k_q[s0:s0 + L, hk].astype(np.int64)
                sk = ks
            else:
                kf = self.k[s0:s0 + L, hk].astype(np.float64)
                vf = self.v[s0:s0 + L, hk].astype(np.float64)
                if self.k_q is not None:
                    k8 = self.k_q[s0:s0 + L, hk].astype(np.int64)
                    sk = np.repeat(self.k_scale[hk, b, :nblk].astype(np.float64), BLOCK_N)[:L]
                else:
                    k8 = sk = None
            self._kv_cache[key] = (kf, vf, k8, sk)
        return self._kv_cache[key]

    def routed_scores(self, b: int, hq: int, i0: int, i1: int, j0: int, j1: int, bit: int) -> np.ndarray:
        """Scores s_ij for query rows [i0, i1) and key rows [j0, j1) of sequence b,
        on the path the route bit selects, before masking (float64).

        FP16 path: s = sm * sum_c Q[i,c] * K_eff[j,c]  ([PL §3 Preliminaries]).
        INT8 path: s = sm * s_q(i) * s_k(j) * S32_ij with S32 the exact integer dot
        product of the INT8 operands, i.e. INT32 accumulation followed by the block
        scales that bring the tile into the common floating-point domain
        ([PL §3 Preliminaries], [AN], [GS]).  Reading: sm_scale is applied after
        dequantisation; Q is not pre-scaled before quantising.
        """
        s0, _ = self.spans[b]              # query rows i are counted from the chunk start
        hk = self.kv_head(hq)
        kf, _, k8, sk = self._kv(b, hk)    # key rows j from the sequence's first key
        if bit == 0:
            qf = self.q[s0 + i0:s0 + i1, hq].astype(np.float64)
            return self.sm * (qf @ kf[j0:j1].T)
        q8 = self.q_q[s0 + i0:s0 + i1, hq].astype(np.int64)
        s32 = q8 @ k8[j0:j1].T                                   # exact integers
        sq = self.q_scale[hq, b, np.arange(i0, i1) // self.blk_q].astype(np.float64)
        return self.sm * sq[:, None] * sk[None, j0:j1] * s32.astype(np.float64)


def attn_tile_row(inp: AttnInputs, b: int, hq: int, m: int, with_lse: bool = False):
    """Output rows of query tile m of (sequence b, query head hq), float64 [rows][d]
    (with_lse: also the rows' log-sum-exp of the scores, natural log, [rows]).

    Streams the legal key tiles n = 0..last_key_tile(m) in increasing order
    ([PL §3 Preliminaries]: the FlashAttention-style kernel iterates key tiles for
    each query tile and divides by the final normaliser).  For each tile the route
    bit picks the score path (O3/O4), then both paths update one shared state
    ([PL §1], [PL §3 Preliminaries], [AN]):

        m' = max(m, rowmax s);  alpha = exp(m - m');  p = exp(s - m')
        l  <- alpha * l + rowsum p;  acc <- alpha * acc + p @ V_eff
    and finally O = acc / l, LSE = m + log l.  Initial m = -inf, l = 0, acc = 0.
    Query i sits at key position (Lk - Lq) + i (bottom-right alignment; 0 offset
    in prefill).
    """
    Lq, Lk = inp.pairs[b]
    off = Lk - Lq
    i0, i1 = m * BLOCK_M, min((m + 1) * BLOCK_M, Lq)
    if i0 >= i1:
        raise ValueError("query tile past sequence end")
    hk = inp.kv_head(hq)
    _, vf, _, _ = inp._kv(b, hk)
    word = int(inp.words[hk, b, m])
    rows = i1 - i0
    run_max = np.full(rows, -np.inf)
    run_sum = np.zeros(rows)
    acc = np.zeros((rows, inp.d))
    qpos = off + np.arange(i0, i1)[:, None]
    for n in range(last_key_tile(m, Lq, Lk) + 1):
        j0, j1 = n * BLOCK_N, min((n + 1) * BLOCK_N, Lk)
        bit = route_bit(word, n, inp.g)
        s = inp.routed_scores(b, hq, i0, i1, j0, j1, bit)
        kj = np.arange(j0, j1)[None, :]
        s = np.where(kj <= qpos, s, -np.inf)                    # causal legality
        new_max = np.maximum(run_max, s.max(axis=1))
        alpha = np.exp(run_max - new_max)
        p = np.exp(s - new_max[:, None])
        run_sum = alpha * run_sum + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ vf[j0:j1]
        run_max = new_max
    out = acc / run_sum[:, None]
    if with_lse:
        return out, run_max + np.log(run_sum)
    return out


def attn_prefill(inp: AttnInputs, with_lse: bool = False):
    """Full routed causal attention of every query, float64 [N][Hq][d]
    (with_lse: also the log-sum-exp of every query row's scores, [N][Hq])."""
    N = int(inp.cu[-1])
    out = np.zeros((N, inp.Hq, inp.d))
    lse = np.zeros((N, inp.Hq))
    for b, (s0, L) in enumerate(inp.spans):
        for hq in range(inp.Hq):
            for m in range(num_tiles(L)):
                i0, i1 = m * BLOCK_M, min((m + 1) * BLOCK_M, L)
                o, e = attn_tile_row(inp, b, hq, m, with_lse=True)
                out[s0 + i0:s0 + i1, hq] = o
                lse[s0 + i0:s0 + i1, hq] = e
        inp._kv_cache.clear()
    return (out, lse) if with_lse else out


def attn_rows(inp: AttnInputs, samples: Sequence[Tuple[int, int, int]]) -> Dict[Tuple[int, int, int], np.ndarray]:
    """Output tiles for a list of (sequence, query head, query-tile row) samples."""
    return {(b, hq, m): attn_tile_row(inp, b, hq, m) for (b, hq, m) in samples}


def s32_tiles(inp: AttnInputs, b: int, hq: int, m_begin: int, m_end: int) -> np.ndarray:
    """int32 [m_end-m_begin][Tk][64][64]: the INT32 score tile of every INT8-routed
    legal tile of (b, hq), rows = query offset, cols = key offset within the tile.

    Entries for query or key positions past the sequence end are 0 (their
    operands are zero); tiles that are illegal or FP16-routed hold INT32_MIN.
    """
    s0, _ = inp.spans[b]
    Lq, Lk = inp.pairs[b]
    Tk = num_tiles(inp.max_seqlen_k)
    hk = inp.kv_head(hq)
    out = np.full((m_end - m_begin, Tk, BLOCK_M, BLOCK_N), INT32_MIN, dtype=np.int64)
    _, _, k8, _ = inp._kv(b, hk)
    for m in range(m_begin, min(m_end, num_tiles(Lq))):
        word = int(inp.words[hk, b, m])
        i0, i1 = m * BLOCK_M, min((m + 1) * BLOCK_M, Lq)
        q8 = inp.q_q[s0 + i0:s0 + i1, hq].astype(np.int64)
        for n in range(last_key_tile(m, Lq, Lk) + 1):
            if route_bit(word, n, inp.g) != 1:
                continue
            j0, j1 = n * BLOCK_N, min((n + 1) * BLOCK_N, Lk)
            tile = np.zeros((BLOCK_M, BLOCK_N), dtype=np.int64)
            tile[: i1 - i0, : j1 - j0] = q8 @ k8[j0:j1].T
            out[m - m_begin, n] = tile
    return out.astype(np.int32)


def route_used(inp: AttnInputs) -> np.ndarray:
    """uint8 [B][Hq][Tq][Tk]: path taken per visited tile, 0xFF where not visited."""
    Tq, Tk = num_tiles(inp.max_seqlen), num_tiles(inp.max_seqlen_k)
    out = np.full((len(inp.spans), inp.Hq, Tq, Tk), 0xFF, dtype=np.uint8)
    for b, (Lq, Lk) in enumerate(inp.pairs):
        for hq in range(inp.Hq):
            hk = inp.kv_head(hq)
            for m in range(num_tiles(Lq)):
                w = int(inp.words[hk, b, m])
                for n in range(last_key_tile(m, Lq, Lk) + 1):
                    out[b, hq, m, n] = route_bit(w, n, inp.g)
    return out


# ---------------------------------------------------------------------------
# Independent formulations used to pin the streaming oracle
# ---------------------------------------------------------------------------

def attn_dense_two_pass(inp: AttnInputs, b: int, hq: int, with_lse: bool = False):
    """The same routed attention, materialised: the full L x L score matrix with each
    element taken from its tile's path, then a two-pass softmax (max, then
    normalised exponentials) and O = P V ([PL §3 Preliminaries]: S = QK^T,
    P = softmax(S), O = PV).  float64 [Lq][d] (with_lse: and log sum exp S, [Lq])."""
    s0, _ = inp.spans[b]
    Lq, Lk = inp.pairs[b]
    hk = inp.kv_head(hq)
    kf, vf, k8, sk = inp._kv(b, hk)
    qf = inp.q[s0:s0 + Lq, hq].astype(np.float64)
    S_fp = inp.sm * (qf @ kf.T)
    if inp.q_q is not None and k8 is not None:
        q8 = inp.q_q[s0:s0 + Lq, hq].astype(np.int64)
        sq = inp.q_scale[hq, b, np.arange(Lq) // inp.blk_q].astype(np.float64)
        S_i8 = inp.sm * np.outer(sq, sk) * (q8 @ k8.T).astype(np.float64)
    else:
        S_i8 = np.full((Lq, Lk), np.nan)
    tile_i = np.arange(Lq) // BLOCK_M
    tile_j = np.arange(Lk) // BLOCK_N
    words = np.array([int(w) for w in inp.words[hk, b]], dtype=object)
    # element (i, j) follows bit floor(tile_j / g) of word[tile_i]
    bits = np.array([[(int(words[ti]) >> (tj // inp.g)) & 1 for tj in tile_j] for ti in range(num_tiles(Lq))])
    R = bits[tile_i]                                      # [Lq][Lk]
    S = np.where(R == 1, S_i8, S_fp)
    legal = np.arange(Lk)[None, :] <= (Lk - Lq) + np.arange(Lq)[:, None]
    S = np.where(legal, S, -np.inf)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    P = E / E.sum(axis=1, keepdims=True)
    if with_lse:
        return P @ vf, mx[:, 0] + np.log(E.sum(axis=1))
    return P @ vf


def attn_brute_force(inp: AttnInputs, b: int, hq: int, with_lse: bool = False):
    """Element-by-element evaluation in plain Python for tiny L: each score from
    its own definition (route bit decoded per element, INT8 dot product summed
    as Python integers; with an INT8 KV cache each key and value element is
    dequantised with the scale of its own 64-key block, looked up per element),
    then softmax of each row and the weighted sum of values.  Returns the rows
    ([Lq][d] lists); with_lse: also each row's log-sum-exp of its scores."""
    s0, _ = inp.spans[b]
    k0, _ = inp.spans_k[b]
    Lq, Lk = inp.pairs[b]
    d = inp.d
    hk = inp.kv_head(hq)
    sm = inp.sm
    out, lses = [], []
    for i in range(Lq):
        word = int(inp.words[hk, b, i // BLOCK_M])
        scores = []
        for j in range(Lk - Lq + i + 1):
            bit = (word >> ((j // BLOCK_N) // inp.g)) & 1
            if bit == 0:
                if inp.kv_int8:
                    ks = float(inp.k_scale[hk, b, j // BLOCK_N])
                    kvec = [float(inp.k_q[k0 + j, hk, c]) * ks for c in range(d)]
                else:
                    kvec = [float(inp.k[k0 + j, hk, c]) for c in range(d)]
                s = sm * sum(float(inp.q[s0 + i, hq, c]) * kvec[c] for c in range(d))
            else:
                dot = sum(int(inp.q_q[s0 + i, hq, c]) * int(inp.k_q[k0 + j, hk, c]) for c in range(d))
                s = sm * float(inp.q_scale[hq, b, i // inp.blk_q]) * float(inp.k_scale[hk, b, j // BLOCK_N]) * dot
            scores.append(s)
        mx = max(scores)
        e = [math.exp(s - mx) for s in scores]
        z = sum(e)
        lses.append(mx + math.log(z))
        row = []
        for c in range(d):
            acc = 0.0
            for j in range(len(scores)):
                if inp.kv_int8:
                    vv = float(inp.v_q[k0 + j, hk, c]) * float(inp.v_scale[hk, b, j // BLOCK_N])
                else:
                    vv = float(inp.v[k0 + j, hk, c])
                acc += e[j] * vv
            row.append(acc / z)
        out.append(row)
    return (out, lses) if with_lse else out


# ---------------------------------------------------------------------------
# Numerical deviation [PL §5 Numerical Behavior], [PL App. G, G.1, G.2]
# ---------------------------------------------------------------------------

def output_deviation(o: np.ndarray, o_ref: np.ndarray) -> Tuple[float, float]:
    """(MaxDiff, MeanDiff) of an attention output against a reference output.

    The pages measure routed outputs against a fixed FP16 reference with the
    maximum and the mean elementwise difference.  Reading taken: both are
    absolute differences over every output element (all tokens, heads and
    channels), computed in float64."""
    if o.shape != o_ref.shape:
        raise ValueError("shape mismatch")
    diff = np.abs(o.astype(np.float64) - o_ref.astype(np.float64))
    if diff.size == 0:
        return 0.0, 0.0
    return float(diff.max()), float(diff.mean())


# ---------------------------------------------------------------------------
# Resident-footprint calculator [PL App. D]
# ---------------------------------------------------------------------------

def footprint_bytes(*, tokens: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    blk_q: int = 128, blk_k: int = 64, quantize_once: bool = True) -> Dict[str, float]:
    """Resident HBM bytes of one attention call: dense fp16 Q/K/V, plus (quantize-once)
    Q8/K8 and one fp32 scale per (head, token block) ([PL App. C], [PL App. D])."""
    dense = 2 * tokens * head_dim * (num_q_heads + 2 * num_kv_heads)
    res = {"dense_fp16_qkv": dense}
    if quantize_once:
        res["q8_k8"] = tokens * head_dim * (num_q_heads + num_kv_heads)
        res["scales"] = 4 * (num_q_heads * _cdiv(tokens, blk_q) + num_kv_heads * _cdiv(tokens, blk_k))
    res["total"] = sum(res.values())
    return res


def qk_tile_operand_bytes(block_m: int, block_n: int, head_dim: int, int8: bool) -> int:
    """Bytes of the Q and K operand tiles one score tile reads ([PL App. D])."""
    per = 1 if int8 else 2
    return (block_m + block_n) * head_dim * per


# Exact-arithmetic helpers for the quantiser pins --------------------------

def nearest_fp32(fr: Fraction) -> np.float32:
    """The float32 nearest to an exact rational (ties to even), by exhaustive
    comparison of the two float32 neighbours of the float64 estimate."""
    est = np.float32(float(fr))
    cands = {est, np.nextafter(est, np.float32(np.inf)), np.nextafter(est, np.float32(-np.inf))}
    best = None
    for c in cands:
        err = abs(Fraction(float(c)) - fr)
        key = (err, int(np.array(c, dtype=np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])
