"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects invalid arguments on the host before any launch (no
compute call is made here)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilemix.h")
LIB = os.path.join(ROOT, "mixed_precision_amd", "libtilemix.so")


@pytest.fixture(scope="module")
def tm():
    if not os.path.exists(LIB):
        from mixed_precision_amd import build as b
        b.build(verbose=False)
    from mixed_precision_amd import tilemix
    return tilemix


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tilemix_\w+)\s*\(", src)))


def test_header_declares_expected_calls():
    names = header_functions()
    for n in ("tilemix_quantize_blockwise", "tilemix_build_route_mask", "tilemix_decode_route_mask",
              "tilemix_attn_workspace_size", "tilemix_attn_prefill", "tilemix_attn_plan", "tilemix_attn_run",
              "tilemix_attn_prefill_debug", "tilemix_status_string", "tilemix_last_error",
              "tilemix_template_route_words"):
        assert n in names


def test_library_exports_every_declared_symbol(tm):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tilemix_\w+)", out))
    declared = set(header_functions())
    assert declared <= exported, declared - exported
    assert set(tm.EXPORTED) == declared
    for n in declared:
        getattr(tm.lib(), n)


def test_probe_library_exports_its_header():
    """The microbenchmark library (not part of the attention path) exports
    what include/tilemix_probe.h declares."""
    probe_lib = os.path.join(ROOT, "mixed_precision_amd", "libtilemix_probe.so")
    if not os.path.exists(probe_lib):
        from mixed_precision_amd import build as b
        b.build(verbose=False)
    src = open(os.path.join(ROOT, "include", "tilemix_probe.h")).read()
    declared = set(re.findall(r"\b(tilemix_\w+)\s*\(", src))
    out = subprocess.run(["nm", "-D", "--defined-only", probe_lib], capture_output=True, text=True, check=True).stdout
    assert declared and declared <= set(re.findall(r"\bT (tilemix_\w+)", out))


def test_status_strings(tm):
    for code, name in tm.STATUS_NAMES.items():
        assert tm.lib().tilemix_status_string(code).decode() == name
    assert tm.lib().tilemix_version().decode().startswith("tilemix")


def _params(tm, **kw):
    base = dict(batch=8, max_seqlen=4096, num_q_heads=24, num_kv_heads=8, head_dim=128, g=1, blk_q=64,
                sm_scale=0.088388, kv_int8=False, out_fp32=False)
    base.update(kw)
    return tm.AttnProblem(**base)


def test_workspace_size_and_param_validation(tm):
    n = tm.tilemix_attn_workspace_size(_params(tm))
    # work list: 8 x 64 x 8 items of 16 bytes, plus the segment table
    assert n >= 8 * 64 * 8 * 16 and n % 256 == 0
    bad = [
        (dict(head_dim=96), 2), (dict(blk_q=32), 2), (dict(num_q_heads=20), 1), (dict(num_kv_heads=0), 1),
        (dict(batch=0), 1), (dict(max_seqlen=0), 1), (dict(g=0), 1), (dict(max_seqlen=64 * 65, g=1), 3),
        (dict(sm_scale=0.0), 1), (dict(sm_scale=float("nan")), 1),
    ]
    for kw, status in bad:
        with pytest.raises(tm.TilemixError) as e:
            tm.tilemix_attn_workspace_size(_params(tm, **kw))
        assert e.value.status == status, (kw, e.value)
    assert tm.tilemix_attn_workspace_size(_params(tm, max_seqlen=64 * 65, g=2)) > 0


def test_null_pointer_and_workspace_errors(tm):
    lib = tm.lib()
    p = _params(tm).params()
    t = tm.AttnTensors()
    st = lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None)
    assert st == 1 and "non-NULL" in tm.last_error()
    # well-formed (fake, 256-aligned) addresses but no workspace: rejected before any launch
    a = 1 << 20
    t = tm.AttnTensors(a, a, a, 24 * 128, 128, 8 * 128, 128, a, a, a, a, None, a, a, a)
    st = lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None)
    assert st == 4 and "workspace" in tm.last_error()
    t.q_stride_tok = 24 * 128 + 3
    st = lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None)
    assert st == 1 and "stride" in tm.last_error()
    pc = _params(tm).params()
    pc.causal = 0
    t.q_stride_tok = 24 * 128
    assert lib.tilemix_attn_prefill(ctypes.byref(pc), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 2
    assert lib.tilemix_attn_prefill_debug(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None,
                                          None) == 1
    # plan / run split: same validation, before any launch
    assert lib.tilemix_attn_plan(ctypes.byref(p), None, None, ctypes.c_void_p(a), 1 << 30, None) == 1
    assert lib.tilemix_attn_plan(ctypes.byref(p), ctypes.c_void_p(a), None, None, 0, None) == 4
    assert lib.tilemix_attn_plan(ctypes.byref(pc), ctypes.c_void_p(a), None, ctypes.c_void_p(a), 1 << 30, None) == 2
    # a plan with key prefix sums needs max_seqlen_k > 0, and the other way round
    assert lib.tilemix_attn_plan(ctypes.byref(p), ctypes.c_void_p(a), ctypes.c_void_p(a), ctypes.c_void_p(a),
                                 1 << 30, None) == 1
    assert lib.tilemix_attn_run(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 4
    t.q_stride_tok = 24 * 128 + 3
    assert lib.tilemix_attn_run(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 1


def test_on_the_fly_mode_validation(tm):
    """otf_quant: 0, 1 or 2, not with an INT8 KV cache.  With 1 the quantise-once
    operands may be NULL, with 2 those of Q (the call then fails only on the
    missing workspace); 2 still needs k_q and k_scale."""
    lib = tm.lib()
    a = 1 << 20
    t = tm.AttnTensors(a, a, a, 24 * 128, 128, 8 * 128, 128, None, None, None, None, None, a, a, a)
    p = _params(tm, otf_quant=True).params()
    assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 4
    assert lib.tilemix_attn_run(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 4
    p0 = _params(tm).params()
    assert lib.tilemix_attn_prefill(ctypes.byref(p0), ctypes.byref(t), None, 0, None) == 1
    assert "q_q" in tm.last_error()
    p.otf_quant = 3
    assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 1
    p.otf_quant = 2
    assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 1
    assert "k_scale" in tm.last_error()
    t.k_q, t.k_scale = a, a
    assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 4
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_workspace_size(_params(tm, otf_quant=2, kv_int8=True))
    assert e.value.status == 2
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_workspace_size(_params(tm, otf_quant=True, kv_int8=True))
    assert e.value.status == 2 and "kv_int8" in str(e.value)


def test_chunked_prefill_validation(tm):
    """max_seqlen_k: >= 0, >= max_seqlen when set, its groups within one word;
    cu_seqlens_k exactly when max_seqlen_k > 0; the workspace follows the query tiles."""
    lib = tm.lib()
    a = 1 << 20
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_workspace_size(_params(tm, max_seqlen_k=-1))
    assert e.value.status == 1
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_workspace_size(_params(tm, max_seqlen=4096, max_seqlen_k=2048))
    assert e.value.status == 1
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_workspace_size(_params(tm, max_seqlen=64, max_seqlen_k=64 * 65, g=1))
    assert e.value.status == 3
    n = tm.tilemix_attn_workspace_size(_params(tm, max_seqlen=64, max_seqlen_k=64 * 64, g=1))
    assert n == tm.tilemix_attn_workspace_size(_params(tm, max_seqlen=64, g=1))
    t = tm.AttnTensors(a, a, a, 24 * 128, 128, 8 * 128, 128, a, a, a, a, None, a, a, a)
    pk = _params(tm, max_seqlen=64, max_seqlen_k=4096).params()
    assert lib.tilemix_attn_prefill(ctypes.byref(pk), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 1
    assert "cu_seqlens_k" in tm.last_error()
    t.cu_seqlens_k = a
    assert lib.tilemix_attn_prefill(ctypes.byref(pk), ctypes.byref(t), None, 0, None) == 4
    p0 = _params(tm).params()
    assert lib.tilemix_attn_prefill(ctypes.byref(p0), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 1
    t.cu_seqlens_k = None
    t.lse = a + 2
    assert lib.tilemix_attn_prefill(ctypes.byref(p0), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 1


def test_template_validation(tm):
    lib = tm.lib()
    a = ctypes.c_void_p(1 << 20)
    assert lib.tilemix_template_route_words(8, 500, 1, a, None, 1, 64, 0, 1, 1, a, None) == 1
    assert lib.tilemix_template_route_words(-1, 500, 1, a, None, 1, 64, 0, 1, 1, a, None) == 1
    assert lib.tilemix_template_route_words(2, 1001, 1, a, None, 1, 64, 0, 1, 1, a, None) == 1
    assert lib.tilemix_template_route_words(2, 500, 1, a, None, 1, 64 * 65, 0, 1, 1, a, None) == 3
    assert lib.tilemix_template_route_words(2, 500, 1, a, None, 1, 64, 0, 1, 1, None, None) == 1
    assert lib.tilemix_template_route_words(2, 500, 1, a, a, 1, 64, 0, 1, 1, a, None) == 1
    assert tm.TEMPLATES["sptrans"] == 7


def test_quantize_and_route_validation(tm):
    lib = tm.lib()
    a = ctypes.c_void_p(1 << 20)
    assert lib.tilemix_quantize_blockwise(None, 128, 128, a, 1, 64, 1, 128, 64, a, a, None) == 1
    assert lib.tilemix_quantize_blockwise(a, 128, 128, a, 1, 64, 1, 96, 64, a, a, None) == 2
    assert lib.tilemix_quantize_blockwise(a, 128, 128, a, 1, 64, 1, 128, 32, a, a, None) == 2
    assert lib.tilemix_quantize_blockwise(a, 129, 128, a, 1, 64, 1, 128, 64, a, a, None) == 1
    assert lib.tilemix_quantize_blockwise(a, 128, 128, None, 1, 64, 1, 128, 64, a, a, None) == 1
    assert lib.tilemix_build_route_mask(a, a, None, 1, 64 * 65, 0, 1, 1, a, None) == 3
    assert lib.tilemix_build_route_mask(a, a, None, 1, 64 * 65, 0, 1, 0, a, None) == 1
    assert lib.tilemix_build_route_mask(None, a, None, 1, 64, 0, 1, 1, a, None) == 1
    assert lib.tilemix_decode_route_mask(a, a, None, 1, 64 * 129, 0, 1, 2, a, None) == 3
    assert "64-bit" in tm.last_error()
    # chunked: the groups count key tiles (max_seqlen_k), and cu_seqlens_k goes with max_seqlen_k > 0
    assert lib.tilemix_build_route_mask(a, a, a, 1, 64, 64 * 65, 1, 1, a, None) == 3
    assert lib.tilemix_build_route_mask(a, a, a, 1, 64, 0, 1, 1, a, None) == 1
    assert lib.tilemix_build_route_mask(a, a, None, 1, 64, 128, 1, 1, a, None) == 1
    assert lib.tilemix_build_route_mask(a, a, a, 1, 128, 64, 1, 1, a, None) == 1


def test_kv_stride_tile_span_limit(tm):
    """A K/V tile is read through one 32-bit buffer range: a token stride whose
    64 rows span 4 GiB or more is rejected on the host (fp16: stride >= 2^25
    elements; INT8 cache: >= 2^26), one element of stride less is accepted (the
    call then fails only on the missing workspace)."""
    lib = tm.lib()
    a = 1 << 20
    p16 = _params(tm).params()
    p8 = _params(tm, kv_int8=True).params()
    for p, limit in ((p16, 1 << 25), (p8, 1 << 26)):
        t = tm.AttnTensors(a, a, a, 24 * 128, 128, limit, 128, a, a, a, a, a, a, a, a)
        assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 2
        assert "4 GiB" in tm.last_error()
        assert lib.tilemix_attn_run(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(a), 1 << 30, None) == 2
        t.kv_stride_tok = limit - 16
        assert lib.tilemix_attn_prefill(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 4


def test_noalloc_entry_point_host_checks(tm):
    """tilemix_attn_prefill_noalloc validates like tilemix_attn_prefill and
    rejects, before any HIP call, a call whose work list exceeds its fixed
    device array of 4 MiB (a batch of 480 sequences of 4096 tokens at 8 KV
    heads, 245,760 items of 16 bytes plus the segment table, still fits)."""
    lib = tm.lib()
    a = 1 << 20
    t = tm.AttnTensors(a, a, a, 24 * 128, 128, 8 * 128, 128, a, a, a, a, None, a, a, a)
    p = _params(tm).params()
    p.causal = 0
    assert lib.tilemix_attn_prefill_noalloc(ctypes.byref(p), ctypes.byref(t), None) == 2
    p = _params(tm).params()
    t0 = tm.AttnTensors()
    assert lib.tilemix_attn_prefill_noalloc(ctypes.byref(p), ctypes.byref(t0), None) == 1
    # 1024 sequences x 64 query tiles x 8 KV heads x 1 chunk of 3 heads = 524,288 items: 8 MiB of work list
    big = _params(tm, batch=1024).params()
    need = tm.tilemix_attn_workspace_size(_params(tm, batch=1024))
    assert need > 4 << 20
    assert lib.tilemix_attn_prefill_noalloc(ctypes.byref(big), ctypes.byref(t), None) == 4
    assert "no-allocation" in tm.last_error() and str(need) in tm.last_error()
    assert tm.tilemix_attn_workspace_size(_params(tm, batch=480)) <= 4 << 20 < need


# Known spills of non-debug kernels (VGPRs), at their current counts: the full
# on-the-fly mode with 3 heads per item keeps K's quantisation between two
# barriers beside three q-blocks, in the kernels for partial head chunks at
# d = 128 and at d = 64 (whose three item bodies share the 168 VGPRs of three
# waves per SIMD).  And the d = 128 two-head kernels with a single V stage,
# built for three waves per SIMD (measured faster with their spills).
SPILL_ALLOWANCE = {"_ZN7tilemix25attn_prefill_mixed_kernelILi128ELi3ELb0ELi1ELb0EEEvNS_8AttnArgsE": 1,
                   "_ZN7tilemix25attn_prefill_mixed_kernelILi64ELi3ELb0ELi1ELb0EEEvNS_8AttnArgsE": 8,
                   # two q-blocks at d = 128 with a single V stage, at 3 waves per SIMD (168 VGPRs)
                   "_ZN7tilemix19attn_prefill_kernelILi128ELi2ELb0ELi0ELb0EEEvNS_8AttnArgsE": 7,
                   "_ZN7tilemix25attn_prefill_mixed_kernelILi128ELi2ELb0ELi0ELb0EEEvNS_8AttnArgsE": 5,
                   "_ZN7tilemix25attn_prefill_mixed_kernelILi128ELi2ELb0ELi2ELb0EEEvNS_8AttnArgsE": 2}


def test_kernel_resources_no_new_spills(tm):
    """The compiler's resource figures of the built library (kernel_resources.json,
    written by the build): every attention kernel keeps two waves per SIMD, and no
    non-debug kernel spills registers beyond the known case above."""
    import json
    path = os.path.join(ROOT, "mixed_precision_amd", "kernel_resources.json")
    if not os.path.exists(path):
        from mixed_precision_amd import build as b
        b.build(verbose=False)
    res = json.load(open(path))
    attn = {k: v for k, v in res.items()
            if "attn_prefill_kernel" in k or "attn_prefill_mixed_kernel" in k or "attn_decode_kernel" in k}
    assert len(attn) >= 80
    for name, r in attn.items():
        assert r["Occupancy"] >= 2, (name, r)
        if "prefill" in name and "Li64E" in name:   # d = 64: 3 or 4 waves per SIMD
            assert r["Occupancy"] >= 3, (name, r)
        debug = name.endswith("ELb1EEEvNS_8AttnArgsE") and "prefill" in name
        if not debug:
            assert r["VGPRs Spill"] <= SPILL_ALLOWANCE.get(name, 0), (name, r)
    headline = attn["_ZN7tilemix19attn_prefill_kernelILi128ELi3ELb0ELi2ELb0EEEvNS_8AttnArgsE"]
    assert headline["VGPRs Spill"] == 0 and headline["ScratchSize"] == 0
    # the INT8-cache kernel of three heads per item (chunked prefill) sits at the limit
    kv8 = attn["_ZN7tilemix19attn_prefill_kernelILi128ELi3ELb1ELi0ELb0EEEvNS_8AttnArgsE"]
    assert kv8["VGPRs Spill"] == 0 and kv8["ScratchSize"] == 0
