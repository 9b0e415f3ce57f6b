"""Seeded synthetic inputs for routed FP16/INT8 prefill attention.

This module is the only code shared by the CPU oracle side and the GPU side.
It draws random tensors, sequence lengths and per-tile route decisions; it
holds none of the method's arithmetic (no quantisation, no mask packing, no
attention).  Every array is produced with NumPy from
``numpy.random.default_rng(SeedSequence([cfg_id, stream]))`` so both sides see
the same bits.

Streams: Q=0, K=1, V=2, route=3, lengths=4, outlier channels=5.

Shapes follow the workloads described on the pages: LLaMA-3.2-3B-shaped GQA
attention at 4K tokens and batch 8 with 75 % of the legal tile groups routed to
INT8 (the efficiency section of the paperlayer.ai summary of arXiv 2608.17336,
"TileMix: Tile-Centric Mixed-Precision Attention for LLM Inference
Acceleration", §5 Prefill Efficiency), plus varlen, INT8-KV-cache and long
context variants exercising the features the summary lists in §4.  The
benchmarks the pages ran on (LongEval, LV-Eval, model weights) are not
available; these synthetic tensors stand in for the attention shapes only.

Layout: tokens of all sequences are packed without padding, ``[N][H][d]``
(token-major, heads, channels) with ``cu_seqlens`` int32 ``[B+1]`` prefix sums.
Tile route decisions are ``uint8 [Hk][B][T][T]`` with ``T = ceil(max_seqlen/64)``,
1 = INT8, 0 = FP16; entries of illegal tiles (key tile after query tile, or
past the sequence end) are 0 and ignored by the packer.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

TILE = 64

S_Q, S_K, S_V, S_ROUTE, S_LEN, S_OUTLIER = 0, 1, 2, 3, 4, 5


def rng_for(cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(stream)]))


@dataclasses.dataclass
class Workload:
    """One synthetic attention call (host arrays)."""

    name: str
    cfg_id: int
    q: np.ndarray            # fp16 [N][Hq][d]
    k: np.ndarray            # fp16 [N][Hk][d]
    v: np.ndarray            # fp16 [N][Hk][d]
    cu_seqlens: np.ndarray   # int32 [B+1]
    max_seqlen: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    g: int                   # key tiles per route bit
    blk_q: int               # Q quantisation block (tokens)
    tile_route: np.ndarray   # uint8 [Hk][B][T][T], 1 = INT8
    kv_int8: bool = False    # K/V consumed as an INT8 cache
    sm_scale: float = 0.0    # fp32 value of 1/sqrt(d)
    notes: str = ""
    # chunked prefill: the keys (K, V rows) per sequence; None = the queries' own
    # positions.  The queries are then the last Lq of each sequence's Lk positions.
    cu_seqlens_k: Optional[np.ndarray] = None
    max_seqlen_k: Optional[int] = None

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def T(self) -> int:
        return (self.max_seqlen + TILE - 1) // TILE

    @property
    def T_k(self) -> int:
        return ((self.max_seqlen_k or self.max_seqlen) + TILE - 1) // TILE

    @property
    def lengths_k(self) -> np.ndarray:
        return self.lengths if self.cu_seqlens_k is None else np.diff(self.cu_seqlens_k.astype(np.int64))


def fp32_inv_sqrt(d: int) -> float:
    """The fp32 value nearest 1/sqrt(d), used exactly by both sides."""
    return float(np.float32(1.0 / math.sqrt(d)))


# Channel outliers: the same 4 channels of Q and K are scaled x10, the pattern
# that makes per-block INT8 scales matter.  At d = 128 the scaled logits then
# spread with a standard deviation of ~18 nats (rows close to one-hot), so the
# online softmax's running max keeps moving.
Q_OUTLIER_SCALE, K_OUTLIER_SCALE = 10.0, 10.0


def _normal_fp16(rng: np.random.Generator, shape, outlier_channels=None, outlier_scale=10.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_channels is not None and len(outlier_channels):
        x[..., outlier_channels] *= np.float32(outlier_scale)
    return x.astype(np.float16)  # IEEE round-to-nearest-even


def outlier_channels(cfg_id: int, head_dim: int, count: int = 4) -> np.ndarray:
    rng = rng_for(cfg_id, S_OUTLIER)
    return np.sort(rng.choice(head_dim, size=count, replace=False)).astype(np.int64)


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def legal_tile_matrix(Tb: int, T: int) -> np.ndarray:
    """bool [T][T]: tile (m, n) is legal iff n <= m < Tb (causal, in-sequence)."""
    m = np.arange(T)[:, None]
    n = np.arange(T)[None, :]
    return (n <= m) & (m < Tb)


def route_bernoulli_groups(cfg_id: int, num_kv_heads: int, lengths, T: int, g: int, p: float) -> np.ndarray:
    """Each legal tile group (row m, group j) is INT8 with probability p.

    All tiles of a group get the group's decision, so packing is lossless.
    """
    rng = rng_for(cfg_id, S_ROUTE)
    B = len(lengths)
    ngroups = (T + g - 1) // g
    u = rng.random(size=(num_kv_heads, B, T, ngroups))
    group_bits = (u < p).astype(np.uint8)
    tiles = np.repeat(group_bits, g, axis=3)[..., :T]
    out = np.zeros((num_kv_heads, B, T, T), dtype=np.uint8)
    for b, L in enumerate(lengths):
        Tb = (int(L) + TILE - 1) // TILE
        legal = legal_tile_matrix(Tb, T)
        out[:, b] = np.where(legal[None], tiles[:, b], 0)
    return out


def route_band_sink(num_kv_heads: int, lengths, T: int, band: int = 2, sink: int = 2) -> np.ndarray:
    """FP16 on the diagonal band |m-n| <= band and the first `sink` key tiles, INT8 elsewhere."""
    B = len(lengths)
    m = np.arange(T)[:, None]
    n = np.arange(T)[None, :]
    fp16 = (np.abs(m - n) <= band) | (n < sink)
    out = np.zeros((num_kv_heads, B, T, T), dtype=np.uint8)
    for b, L in enumerate(lengths):
        Tb = (int(L) + TILE - 1) // TILE
        legal = legal_tile_matrix(Tb, T)
        out[:, b] = np.where(legal & ~fp16, 1, 0).astype(np.uint8)[None]
    return out


def route_bernoulli_tiles(cfg_id: int, num_kv_heads: int, lengths, T: int, p: float) -> np.ndarray:
    return route_bernoulli_groups(cfg_id, num_kv_heads, lengths, T, 1, p)


def make_workload(cfg_id: int, *, lengths, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  g: int, blk_q: int = 64, route: str = "bernoulli", p: float = 0.5,
                  outliers: bool = False, kv_int8: bool = False, max_seqlen: Optional[int] = None,
                  q_outlier_scale: float = Q_OUTLIER_SCALE, k_outlier_scale: float = K_OUTLIER_SCALE,
                  name: str = "", notes: str = "") -> Workload:
    lengths = [int(x) for x in lengths]
    cu = cu_from_lengths(lengths)
    N = int(cu[-1])
    max_seqlen = int(max_seqlen if max_seqlen is not None else max(lengths) if lengths else 1)
    T = (max_seqlen + TILE - 1) // TILE
    oc = outlier_channels(cfg_id, head_dim) if outliers else None
    q = _normal_fp16(rng_for(cfg_id, S_Q), (N, num_q_heads, head_dim), oc, q_outlier_scale)
    k = _normal_fp16(rng_for(cfg_id, S_K), (N, num_kv_heads, head_dim), oc, k_outlier_scale)
    v = _normal_fp16(rng_for(cfg_id, S_V), (N, num_kv_heads, head_dim), None)
    if route == "bernoulli":
        tr = route_bernoulli_groups(cfg_id, num_kv_heads, lengths, T, g, p)
    elif route == "band_sink":
        tr = route_band_sink(num_kv_heads, lengths, T)
    elif route == "zeros":
        tr = np.zeros((num_kv_heads, len(lengths), T, T), dtype=np.uint8)
    elif route == "ones":
        tr = np.ones((num_kv_heads, len(lengths), T, T), dtype=np.uint8)
        for b, L in enumerate(lengths):
            tr[:, b] &= legal_tile_matrix((L + TILE - 1) // TILE, T)[None].astype(np.uint8)
    else:
        raise ValueError(route)
    return Workload(name=name or f"cfg{cfg_id}", cfg_id=cfg_id, q=q, k=k, v=v, cu_seqlens=cu,
                    max_seqlen=max_seqlen, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, g=g, blk_q=blk_q, tile_route=tr, kv_int8=kv_int8,
                    sm_scale=fp32_inv_sqrt(head_dim), notes=notes)


def chunk_legal_tiles(Lq: int, Lk: int, Tq: int, Tk: int) -> np.ndarray:
    """bool [Tq][Tk]: tiles a query tile touches when the Lq queries are the last
    Lq of Lk positions (key j allowed for query i iff j <= Lk - Lq + i)."""
    out = np.zeros((Tq, Tk), dtype=bool)
    for m in range((Lq + TILE - 1) // TILE):
        last_q = min(m * TILE + TILE - 1, Lq - 1)
        out[m, : (Lk - Lq + last_q) // TILE + 1] = True
    return out


def make_chunked_workload(cfg_id: int, *, lengths_q, lengths_k, num_q_heads: int, num_kv_heads: int,
                          head_dim: int, g: int, blk_q: int = 64, p: float = 0.5, outliers: bool = False,
                          kv_int8: bool = False, name: str = "") -> Workload:
    """Chunked prefill / decode: sequence b has Lk_b keys and its last Lq_b
    positions are the queries.  Q rows are those positions' rows of the Q that
    make_workload(cfg_id, lengths=lengths_k, ...) draws, so a chunk's inputs
    equal the matching rows of the full prefill's.  Routes: Bernoulli(p) per
    legal tile group of [Hk][B][Tq][Tk], drawn from the route stream."""
    lengths_q = [int(x) for x in lengths_q]
    lengths_k = [int(x) for x in lengths_k]
    assert len(lengths_q) == len(lengths_k) and all(0 < a <= b for a, b in zip(lengths_q, lengths_k))
    cu_k = cu_from_lengths(lengths_k)
    cu_q = cu_from_lengths(lengths_q)
    Nk = int(cu_k[-1])
    oc = outlier_channels(cfg_id, head_dim) if outliers else None
    q_full = _normal_fp16(rng_for(cfg_id, S_Q), (Nk, num_q_heads, head_dim), oc, Q_OUTLIER_SCALE)
    k = _normal_fp16(rng_for(cfg_id, S_K), (Nk, num_kv_heads, head_dim), oc, K_OUTLIER_SCALE)
    v = _normal_fp16(rng_for(cfg_id, S_V), (Nk, num_kv_heads, head_dim), None)
    q = np.concatenate([q_full[int(cu_k[b + 1]) - Lq:int(cu_k[b + 1])] for b, Lq in enumerate(lengths_q)], axis=0)
    max_q, max_k = max(lengths_q), max(lengths_k)
    Tq, Tk = (max_q + TILE - 1) // TILE, (max_k + TILE - 1) // TILE
    rng = rng_for(cfg_id, S_ROUTE)
    ngroups = (Tk + g - 1) // g
    u = rng.random(size=(num_kv_heads, len(lengths_q), Tq, ngroups))
    tiles = np.repeat((u < p).astype(np.uint8), g, axis=3)[..., :Tk]
    tr = np.zeros((num_kv_heads, len(lengths_q), Tq, Tk), dtype=np.uint8)
    for b, (Lq, Lk) in enumerate(zip(lengths_q, lengths_k)):
        tr[:, b] = np.where(chunk_legal_tiles(Lq, Lk, Tq, Tk)[None], tiles[:, b], 0)
    return Workload(name=name or f"chunk{cfg_id}", cfg_id=cfg_id, q=q, k=k, v=v, cu_seqlens=cu_q,
                    max_seqlen=max_q, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    g=g, blk_q=blk_q, tile_route=tr, kv_int8=kv_int8, sm_scale=fp32_inv_sqrt(head_dim),
                    cu_seqlens_k=cu_k, max_seqlen_k=max_k)


def varlen_lengths(cfg_id: int, count: int = 16, lo: int = 512, hi: int = 8192):
    rng = rng_for(cfg_id, S_LEN)
    return [int(x) for x in rng.integers(lo, hi + 1, size=count)]


# The five standard workloads.  Sizes are those of the pages' prefill runs
# (LLaMA-3.2-3B-shaped layer at 4K, batch 8) and of the features the pages list
# (GQA, unpadded varlen, INT8 KV cache, long context).

def config(cfg_id: int, *, p: Optional[float] = None, scale_down: int = 1, head_dim: Optional[int] = None) -> Workload:
    """Standard workload `cfg_id` in 1..5.  `scale_down` > 1 shrinks lengths (tests only).
    `head_dim` re-shapes configs 2-5 to another head dimension (same lengths, heads,
    routes and seeds; the name's d128 becomes d<head_dim>)."""
    if head_dim is not None and head_dim != 128 and cfg_id != 1:
        w = config(cfg_id, p=p, scale_down=scale_down)
        kw = dict(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=head_dim, g=w.g,
                  outliers=cfg_id != 4, kv_int8=w.kv_int8, name=w.name.replace("_d128_", f"_d{head_dim}_"))
        if cfg_id == 3:
            lens = [int(x) for x in np.diff(w.cu_seqlens)]
            return make_workload(3, lengths=lens, route="band_sink", **kw)
        return make_workload(cfg_id, lengths=[int(x) for x in np.diff(w.cu_seqlens)], route="bernoulli",
                             p=(0.75 if cfg_id == 2 else 0.5) if p is None else p, **kw)
    if cfg_id == 1:
        return make_workload(1, lengths=[512 // scale_down], num_q_heads=1, num_kv_heads=1, head_dim=64,
                             g=1, route="bernoulli", p=0.5 if p is None else p,
                             name="tiny_L512_h1_d64_g1_p50")
    if cfg_id == 2:
        L = 4096 // scale_down
        return make_workload(2, lengths=[L] * 8, num_q_heads=24, num_kv_heads=8, head_dim=128,
                             g=1, route="bernoulli", p=0.75 if p is None else p, outliers=True,
                             name="llama3.2-3b_attn_B8_L4096_h24kv8_d128_int8p75")
    if cfg_id == 3:
        lens = varlen_lengths(3)
        if scale_down > 1:
            lens = [max(1, x // scale_down) for x in lens]
        return make_workload(3, lengths=lens, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             g=2, route="band_sink", outliers=True,
                             name="varlen16_U512-8192_h32kv8_d128_band2sink2_g2")
    if cfg_id == 4:
        L = 16384 // scale_down
        return make_workload(4, lengths=[L] * 2, num_q_heads=28, num_kv_heads=4, head_dim=128,
                             g=4, route="bernoulli", p=0.5 if p is None else p, kv_int8=True,
                             name="int8kv_B2_L16384_h28kv4_d128_g4_p50")
    if cfg_id == 5:
        L = 65536 // scale_down
        return make_workload(5, lengths=[L], num_q_heads=32, num_kv_heads=8, head_dim=128,
                             g=16, route="bernoulli", p=0.5 if p is None else p, outliers=True,
                             name=f"long_L65536_h32kv8_d128_g16_p{int(round(100 * (0.5 if p is None else p)))}")
    raise ValueError(cfg_id)
