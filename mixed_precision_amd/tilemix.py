"""Python binding of libtilemix.so (routed FP16/INT8 prefill attention on gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/tilemix.h``.  PyTorch provides
device memory (tensors) and the current HIP stream; nothing here computes.
The library must be built (``__graft_entry__.build()``); importing this module
without it raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtilemix.so")

TILE = 64

TILEMIX_OK = 0
STATUS_NAMES = {0: "TILEMIX_OK", 1: "TILEMIX_ERR_INVALID_ARG", 2: "TILEMIX_ERR_UNSUPPORTED",
                3: "TILEMIX_ERR_TOO_MANY_GROUPS", 4: "TILEMIX_ERR_WORKSPACE", 5: "TILEMIX_ERR_HIP"}

# Every symbol include/tilemix.h declares.
EXPORTED = ("tilemix_status_string", "tilemix_last_error", "tilemix_version", "tilemix_quantize_blockwise",
            "tilemix_build_route_mask", "tilemix_decode_route_mask", "tilemix_attn_workspace_size",
            "tilemix_attn_prefill", "tilemix_attn_plan", "tilemix_attn_run", "tilemix_attn_prefill_debug",
            "tilemix_template_route_words", "tilemix_attn_prefill_noalloc")

# Static routing templates (tilemix_template enum of include/tilemix.h).
TEMPLATES = {"all_fp16": 0, "all_int8": 1, "band": 2, "global": 3, "row_random": 4, "aligned_sparse": 5,
             "bigbird": 6, "sptrans": 7}


class TilemixError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class AttnParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_seqlen", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("g", ctypes.c_int32),
                ("blk_q", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("kv_int8", ctypes.c_int32), ("out_fp32", ctypes.c_int32), ("otf_quant", ctypes.c_int32),
                ("max_seqlen_k", ctypes.c_int32)]


class AttnTensors(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
                ("kv_stride_tok", ctypes.c_int64), ("kv_stride_head", ctypes.c_int64),
                ("q_q", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("k_q", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("route_words", ctypes.c_void_p), ("out", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("lse", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("q_head", ctypes.c_int32), ("m_begin", ctypes.c_int32),
                ("m_end", ctypes.c_int32), ("s32_tiles", ctypes.c_void_p), ("visit_count", ctypes.c_void_p),
                ("route_used", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.tilemix_status_string.restype = ctypes.c_char_p
    lib.tilemix_status_string.argtypes = [i32]
    lib.tilemix_last_error.restype = ctypes.c_char_p
    lib.tilemix_last_error.argtypes = []
    lib.tilemix_version.restype = ctypes.c_char_p
    lib.tilemix_version.argtypes = []
    lib.tilemix_quantize_blockwise.restype = i32
    lib.tilemix_quantize_blockwise.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.tilemix_build_route_mask.restype = i32
    lib.tilemix_build_route_mask.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.tilemix_decode_route_mask.restype = i32
    lib.tilemix_decode_route_mask.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.tilemix_template_route_words.restype = i32
    lib.tilemix_template_route_words.argtypes = [i32, i32, ctypes.c_uint64, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    lib.tilemix_attn_workspace_size.restype = i32
    lib.tilemix_attn_workspace_size.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(sz)]
    lib.tilemix_attn_prefill.restype = i32
    lib.tilemix_attn_prefill.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(AttnTensors), vp, sz, vp]
    lib.tilemix_attn_plan.restype = i32
    lib.tilemix_attn_plan.argtypes = [ctypes.POINTER(AttnParams), vp, vp, vp, sz, vp]
    lib.tilemix_attn_run.restype = i32
    lib.tilemix_attn_run.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(AttnTensors), vp, sz, vp]
    lib.tilemix_attn_prefill_noalloc.restype = i32
    lib.tilemix_attn_prefill_noalloc.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(AttnTensors), vp]
    lib.tilemix_attn_prefill_debug.restype = i32
    lib.tilemix_attn_prefill_debug.argtypes = [ctypes.POINTER(AttnParams), ctypes.POINTER(AttnTensors), vp, sz,
                                               ctypes.POINTER(Debug), vp]
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def last_error() -> str:
    return _lib.tilemix_last_error().decode()


def _check(status: int):
    if status != TILEMIX_OK:
        raise TilemixError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def num_tiles(max_seqlen: int) -> int:
    return (int(max_seqlen) + TILE - 1) // TILE


def _expect(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")


# ----------------------------------------------------------------------------- quantiser

def tilemix_quantize_blockwise(x: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, blk: int,
                               x_q: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """x: fp16 [N][H][d] (channels contiguous).  Returns (x_q int8 [N][H][d], scales f32 [H][B][ceil(max_seqlen/blk)])."""
    _expect(x, torch.float16, "x")
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    N, H, d = x.shape
    if x.stride(2) != 1:
        raise ValueError("x channels must be contiguous")
    B = cu_seqlens.numel() - 1
    nb = (int(max_seqlen) + blk - 1) // blk
    if x_q is None:
        x_q = torch.empty((N, H, d), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((H, B, nb), dtype=torch.float32, device=x.device)
    # the stride of a size-1 dimension never addresses anything (it can be 0 on views)
    st_tok = x.stride(0) if N > 1 else H * d
    st_head = x.stride(1) if H > 1 else d
    _check(_lib.tilemix_quantize_blockwise(_ptr(x), st_tok, st_head, _ptr(cu_seqlens), B, int(max_seqlen),
                                           H, d, int(blk), _ptr(x_q), _ptr(scales), _stream(stream)))
    return x_q, scales


# ----------------------------------------------------------------------------- route words

def tilemix_build_route_mask(tile_route: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, g: int,
                             route_words: Optional[torch.Tensor] = None, stream=None,
                             cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_k: int = 0) -> torch.Tensor:
    """tile_route: uint8 [Hk][B][T][Tk].  Returns route words as int64 [Hk][B][T] (uint64 bit patterns).
    cu_seqlens_k / max_seqlen_k: key prefix sums and bound for chunked prefill (None / 0: prefill)."""
    _expect(tile_route, torch.uint8, "tile_route")
    Hk, B, T, _ = tile_route.shape
    if route_words is None:
        route_words = torch.empty((Hk, B, T), dtype=torch.int64, device=tile_route.device)
    _check(_lib.tilemix_build_route_mask(_ptr(tile_route.contiguous()), _ptr(cu_seqlens), _ptr(cu_seqlens_k), B,
                                         int(max_seqlen), int(max_seqlen_k), Hk, int(g), _ptr(route_words),
                                         _stream(stream)))
    return route_words


def tilemix_decode_route_mask(route_words: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, g: int,
                              stream=None, cu_seqlens_k: Optional[torch.Tensor] = None,
                              max_seqlen_k: int = 0) -> torch.Tensor:
    """Returns uint8 [Hk][B][T][Tk]: the decoded bit of every legal tile, 0xFF elsewhere."""
    Hk, B, T = route_words.shape
    Tk = num_tiles(max_seqlen_k if max_seqlen_k else max_seqlen)
    out = torch.empty((Hk, B, T, Tk), dtype=torch.uint8, device=route_words.device)
    _check(_lib.tilemix_decode_route_mask(_ptr(route_words), _ptr(cu_seqlens), _ptr(cu_seqlens_k), B,
                                          int(max_seqlen), int(max_seqlen_k), Hk, int(g), _ptr(out),
                                          _stream(stream)))
    return out


def tilemix_template_route_words(kind: str, int8_permille: int, seed: int, cu_seqlens: torch.Tensor, max_seqlen: int,
                                 num_kv_heads: int, g: int, cu_seqlens_k: Optional[torch.Tensor] = None,
                                 max_seqlen_k: int = 0, route_words: Optional[torch.Tensor] = None,
                                 stream=None) -> torch.Tensor:
    """Route words int64 [Hk][B][T] of a static template ('band', 'global', 'row_random', 'aligned_sparse',
    'bigbird', 'sptrans', 'all_fp16', 'all_int8') at int8_permille / 1000 INT8 coverage of the legal groups."""
    _expect(cu_seqlens, torch.int32, "cu_seqlens")
    B = cu_seqlens.numel() - 1
    T = num_tiles(max_seqlen)
    if route_words is None:
        route_words = torch.empty((num_kv_heads, B, T), dtype=torch.int64, device=cu_seqlens.device)
    _check(_lib.tilemix_template_route_words(TEMPLATES[kind], int(int8_permille), int(seed) & ((1 << 64) - 1),
                                             _ptr(cu_seqlens), _ptr(cu_seqlens_k), B, int(max_seqlen),
                                             int(max_seqlen_k), int(num_kv_heads), int(g), _ptr(route_words),
                                             _stream(stream)))
    return route_words


# ----------------------------------------------------------------------------- attention

@dataclass
class AttnProblem:
    batch: int
    max_seqlen: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    g: int
    blk_q: int
    sm_scale: float
    kv_int8: bool = False
    out_fp32: bool = False
    otf_quant: int = 0        # 1 (or True): Q/K INT8 operands made inside the kernel (q_q, q_scale, k_q, k_scale
                              # unused); 2: Q's alone (q_q, q_scale unused)
    max_seqlen_k: int = 0     # chunked prefill: bound of the key counts (0: prefill)

    def params(self) -> AttnParams:
        return AttnParams(self.batch, self.max_seqlen, self.num_q_heads, self.num_kv_heads, self.head_dim, self.g,
                          self.blk_q, float(self.sm_scale), 1, int(self.kv_int8), int(self.out_fp32),
                          int(self.otf_quant), int(self.max_seqlen_k))


def tilemix_attn_workspace_size(problem: AttnProblem) -> int:
    n = ctypes.c_size_t(0)
    p = problem.params()
    _check(_lib.tilemix_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def _tensors(q, k, v, q_q, q_scale, k_q, k_scale, v_scale, cu_seqlens, route_words, out, cu_seqlens_k=None,
             lse=None) -> AttnTensors:
    if q.stride(2) != 1 or k.stride(2) != 1 or v.stride(2) != 1 or k.stride() != v.stride():
        raise ValueError("q/k/v channels must be contiguous and k, v must share strides")
    def st(t, dim):   # the stride of a size-1 dimension never addresses anything (it can be 0 on views)
        if t.shape[dim] > 1:
            return t.stride(dim)
        return t.shape[2] * (t.shape[1] if dim == 0 else 1)
    def p(t):
        return None if t is None else t.data_ptr()
    return AttnTensors(q.data_ptr(), k.data_ptr(), v.data_ptr(), st(q, 0), st(q, 1), st(k, 0), st(k, 1),
                       p(q_q), p(q_scale), p(k_q), p(k_scale), p(v_scale), cu_seqlens.data_ptr(),
                       route_words.data_ptr(), out.data_ptr(), p(cu_seqlens_k), p(lse))


class AttnPlan:
    """Problem description plus a reusable workspace and C structs for repeated calls."""

    def __init__(self, problem: AttnProblem, device="cuda"):
        self.problem = problem
        self.params = problem.params()
        self.ws_bytes = tilemix_attn_workspace_size(problem)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)

    def schedule(self, cu_seqlens, stream=None, cu_seqlens_k=None):
        """tilemix_attn_plan: build the work list for `cu_seqlens` (and `cu_seqlens_k`) into the workspace."""
        _check(_lib.tilemix_attn_plan(ctypes.byref(self.params), _ptr(cu_seqlens), _ptr(cu_seqlens_k),
                                      _ptr(self.workspace), self.ws_bytes, _stream(stream)))

    def run_planned(self, q, k, v, q_q, q_scale, k_q, k_scale, cu_seqlens, route_words, out, v_scale=None,
                    stream=None, cu_seqlens_k=None, lse=None):
        """tilemix_attn_run: attention over the work list a previous schedule() built."""
        t = _tensors(q, k, v, q_q, q_scale, k_q, k_scale, v_scale, cu_seqlens, route_words, out, cu_seqlens_k, lse)
        _check(_lib.tilemix_attn_run(ctypes.byref(self.params), ctypes.byref(t), _ptr(self.workspace),
                                     self.ws_bytes, _stream(stream)))
        return out

    def run(self, q, k, v, q_q, q_scale, k_q, k_scale, cu_seqlens, route_words, out, v_scale=None,
            debug: Optional[Debug] = None, stream=None, cu_seqlens_k=None, lse=None):
        """tilemix_attn_prefill (work list + attention), or its debug variant."""
        t = _tensors(q, k, v, q_q, q_scale, k_q, k_scale, v_scale, cu_seqlens, route_words, out, cu_seqlens_k, lse)
        if debug is None:
            st = _lib.tilemix_attn_prefill(ctypes.byref(self.params), ctypes.byref(t), _ptr(self.workspace),
                                           self.ws_bytes, _stream(stream))
        else:
            st = _lib.tilemix_attn_prefill_debug(ctypes.byref(self.params), ctypes.byref(t), _ptr(self.workspace),
                                                 self.ws_bytes, ctypes.byref(debug), _stream(stream))
        _check(st)
        return out


def tilemix_attn_prefill(q, k, v, *, cu_seqlens, route_words, max_seqlen: int, g: int, q_q=None, q_scale=None,
                         k_q=None, k_scale=None, blk_q: int = 64, sm_scale: Optional[float] = None,
                         kv_int8: bool = False, v_scale=None, out_fp32: bool = False, otf_quant: int = 0,
                         cu_seqlens_k=None, max_seqlen_k: int = 0, lse=None, out=None,
                         plan: Optional[AttnPlan] = None, stream=None) -> torch.Tensor:
    """Fused routed causal attention; returns out [N][Hq][d] (fp16, or fp32 if out_fp32).

    otf_quant=0 takes the quantise-once operands q_q, q_scale, k_q, k_scale (k_q unused with kv_int8);
    otf_quant=1 (True) makes them inside the kernel and ignores those arguments; otf_quant=2 makes Q's
    (q_q, q_scale ignored) and takes k_q, k_scale.  cu_seqlens_k / max_seqlen_k:
    chunked prefill or decode (the queries are the last positions of each sequence's keys).  lse: optional
    float32 [N][Hq] output of each row's log-sum-exp."""
    N, Hq, d = q.shape
    Hk = k.shape[1]
    B = cu_seqlens.numel() - 1
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    if plan is None:
        plan = AttnPlan(AttnProblem(B, int(max_seqlen), Hq, Hk, d, int(g), int(blk_q), float(sm_scale),
                                    bool(kv_int8), bool(out_fp32), int(otf_quant), int(max_seqlen_k)),
                        device=q.device)
    if out is None:
        out = torch.empty((N, Hq, d), dtype=torch.float32 if out_fp32 else torch.float16, device=q.device)
    return plan.run(q, k, v, q_q, q_scale, k_q, k_scale, cu_seqlens, route_words, out, v_scale=v_scale,
                    stream=stream, cu_seqlens_k=cu_seqlens_k, lse=lse)


def tilemix_attn_prefill_noalloc(q, k, v, *, cu_seqlens, route_words, max_seqlen: int, g: int, q_q=None,
                                 q_scale=None, k_q=None, k_scale=None, blk_q: int = 64,
                                 sm_scale: Optional[float] = None, kv_int8: bool = False, v_scale=None,
                                 otf_quant: int = 0, cu_seqlens_k=None, max_seqlen_k: int = 0, lse=None,
                                 out: torch.Tensor, stream=None) -> torch.Tensor:
    """tilemix_attn_prefill_noalloc: the same call as tilemix_attn_prefill with no workspace (the library
    keeps the work list in a fixed device array).  `out` (fp16 or float32 [N][Hq][d]) is the caller's; this
    wrapper allocates nothing on the device."""
    N, Hq, d = q.shape
    Hk = k.shape[1]
    B = cu_seqlens.numel() - 1
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    params = AttnProblem(B, int(max_seqlen), Hq, Hk, d, int(g), int(blk_q), float(sm_scale), bool(kv_int8),
                         out.dtype == torch.float32, int(otf_quant), int(max_seqlen_k)).params()
    t = _tensors(q, k, v, q_q, q_scale, k_q, k_scale, v_scale, cu_seqlens, route_words, out, cu_seqlens_k, lse)
    _check(_lib.tilemix_attn_prefill_noalloc(ctypes.byref(params), ctypes.byref(t), _stream(stream)))
    return out


def tilemix_attn_prefill_debug(q, k, v, *, cu_seqlens, route_words, max_seqlen: int, g: int, q_q=None,
                               q_scale=None, k_q=None, k_scale=None, blk_q: int = 64,
                               sm_scale: Optional[float] = None, kv_int8: bool = False, v_scale=None,
                               out_fp32: bool = True, otf_quant: int = 0, cu_seqlens_k=None,
                               max_seqlen_k: int = 0, seq: int = 0, q_head: int = 0, m_begin: int = 0,
                               m_end: Optional[int] = None, stream=None):
    """As tilemix_attn_prefill, plus (s32_tiles, visit_count, route_used) debug products."""
    N, Hq, d = q.shape
    Hk = k.shape[1]
    B = cu_seqlens.numel() - 1
    T = num_tiles(max_seqlen)
    Tk = num_tiles(max_seqlen_k if max_seqlen_k else max_seqlen)
    if m_end is None:
        m_end = T
    if sm_scale is None:
        sm_scale = float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32))
    plan = AttnPlan(AttnProblem(B, int(max_seqlen), Hq, Hk, d, int(g), int(blk_q), float(sm_scale), bool(kv_int8),
                                bool(out_fp32), int(otf_quant), int(max_seqlen_k)), device=q.device)
    out = torch.empty((N, Hq, d), dtype=torch.float32 if out_fp32 else torch.float16, device=q.device)
    s32 = torch.empty((m_end - m_begin, Tk, TILE, TILE), dtype=torch.int32, device=q.device)
    visits = torch.empty((B, Hq, T, Tk), dtype=torch.int32, device=q.device)
    used = torch.empty((B, Hq, T, Tk), dtype=torch.uint8, device=q.device)
    dbg = Debug(seq, q_head, m_begin, m_end, s32.data_ptr(), visits.data_ptr(), used.data_ptr())
    plan.run(q, k, v, q_q, q_scale, k_q, k_scale, cu_seqlens, route_words, out, v_scale=v_scale, debug=dbg,
             stream=stream, cu_seqlens_k=cu_seqlens_k)
    return out, s32, visits, used
