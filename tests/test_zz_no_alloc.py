"""The attention entry point that allocates nothing (tilemix_attn_prefill_noalloc:
work list in the library's fixed device array) against tilemix_attn_prefill with a
caller workspace: the same output bits on consecutive calls, each later one with a
smaller input than the one before (the array still holds the earlier, longer work
list, which each call rewrites), and within the oracle bars."""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from workloads import make_chunked_workload, make_workload
from tests.oracle_inputs import oracle_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gp():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_path
    return gpu_path


def _noalloc(gp, w, t, out):
    tm = gp.tm
    ck = {} if t.get("cu_k") is None else dict(cu_seqlens_k=t["cu_k"], max_seqlen_k=w.max_seqlen_k)
    if w.kv_int8:
        return tm.tilemix_attn_prefill_noalloc(t["q"], t["k8"], t["v8"], q_q=t["q_q"], q_scale=t["q_s"],
                                               k_scale=t["k_s"], v_scale=t["v_s"], kv_int8=True,
                                               cu_seqlens=t["cu"], route_words=t["words"], max_seqlen=w.max_seqlen,
                                               g=w.g, blk_q=w.blk_q, sm_scale=w.sm_scale, out=out, **ck)
    return tm.tilemix_attn_prefill_noalloc(t["q"], t["k"], t["v"], k_q=t["k_q"], k_scale=t["k_s"], otf_quant=2,
                                           cu_seqlens=t["cu"], route_words=t["words"], max_seqlen=w.max_seqlen,
                                           g=w.g, blk_q=w.blk_q, sm_scale=w.sm_scale, out=out, **ck)


def test_noalloc_matches_workspace_entry_point(gp):
    import torch
    calls = [
        make_workload(560, lengths=[1500, 700, 300, 64, 1], num_q_heads=6, num_kv_heads=2, head_dim=128, g=1,
                      p=0.75, outliers=True),
        make_workload(561, lengths=[200, 77], num_q_heads=3, num_kv_heads=1, head_dim=128, g=2, p=0.5,
                      outliers=True),
        make_chunked_workload(562, lengths_q=[40, 1], lengths_k=[150, 90], num_q_heads=2, num_kv_heads=1,
                              head_dim=64, g=1, p=0.5, outliers=True, kv_int8=True),
    ]
    for i, w in enumerate(calls):
        print(f"[case] noalloc call {i}: lengths {list(map(int, w.lengths))}", flush=True)
        t = gp.prepare(w)
        ref = gp.attn(w, t, otf=0 if w.kv_int8 else 2).clone()      # caller workspace
        out = torch.full_like(ref, float("nan"))
        _noalloc(gp, w, t, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        ma, rf = gp.errors(out.cpu().numpy(), orc.attn_prefill(oracle_inputs(w)))
        print(f"  max_abs={ma:.3e} rel_fro={rf:.3e}")
        assert ma <= 2e-3 and rf <= 1e-3


def test_noalloc_rejects_oversized_work_list(gp):
    """A work list above the fixed array is refused (TILEMIX_ERR_WORKSPACE), nothing launched."""
    import torch
    tm = gp.tm
    B, L = 1024, 4096
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda:0")
    q = torch.zeros((8, 24, 128), dtype=torch.float16, device="cuda:0")      # never read: rejected first
    k = torch.zeros((8, 8, 128), dtype=torch.float16, device="cuda:0")
    words = torch.zeros((8, B, 64), dtype=torch.int64, device="cuda:0")
    out = torch.empty((8, 24, 128), dtype=torch.float16, device="cuda:0")
    with pytest.raises(tm.TilemixError) as e:
        tm.tilemix_attn_prefill_noalloc(q, k, k, k_q=k.to(torch.int8), k_scale=out.float(), otf_quant=2,
                                        cu_seqlens=cu, route_words=words, max_seqlen=L, g=1, out=out)
    assert e.value.status == 4 and "no-allocation" in str(e.value)
