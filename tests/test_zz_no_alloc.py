"""The no-allocation decode entry point (nvfp4_paged_decode_attn_noalloc, library-held partials)
against the workspace entry point on the same inputs, through the C ABI: two calls in a row, the
second smaller than the first (the library's array keeps the first call's partials), each
bit-identical to the workspace call and within the oracle's tolerance."""
import numpy as np
import pytest
import torch

import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(nv, wl, fused):
    ks, vs = H.oracle_inputs(wl, with_new=fused)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool_a, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0xFF)
    pool_b = {k: t.clone() for k, t in pool_a.items()}
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()), 4)
    assert plan[1] > 1, plan                                   # several splits: partials are used
    q = wl.q().to(DEV)
    nk = wl.new_token("k").to(DEV) if fused else None
    nvv = wl.new_token("v").to(DEV) if fused else None
    ref = nv.nvfp4_decode(q, pool_a, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv, new_k=nk, new_v=nvv)
    got = nv.nvfp4_decode_noalloc(q, pool_b, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv, new_k=nk,
                                  new_v=nvv)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "no-allocation output differs from the workspace call"
    for k in pool_a:
        assert torch.equal(pool_a[k], pool_b[k]), k
    H.assert_attention_close(got.cpu().numpy(), want, f"noalloc {wl.name} plan={plan}")
    return nv.decode_workspace_size(wl.batch, wl.h_q, wl.h_kv, plan[1])


def test_noalloc_matches_workspace_call_twice_smaller_second():
    import bit_paged_kv_amd as nv
    big = workloads.Workload(name="noalloc-big", seed=41, batch=6, h_kv=4, h_q=32,
                             seq_lens=[3000, 1, 777, 4096, 16, 2500], extra_pages=3)
    small = workloads.Workload(name="noalloc-small", seed=42, batch=2, h_kv=2, h_q=8, seq_lens=[700, 45],
                               append=True)
    n_big = _case(nv, big, fused=False)
    n_small = _case(nv, small, fused=True)
    assert 0 < n_small < n_big <= nv.decode_noalloc_max_bytes()


def test_noalloc_rejects_partials_beyond_the_array():
    import bit_paged_kv_amd as nv
    q = torch.zeros((64, 64, 128), dtype=torch.bfloat16, device=DEV)
    pool = nv.alloc_nvfp4_pool(1, 8, DEV)
    pt = torch.zeros((64, 1), dtype=torch.int32, device=DEV)
    sl = torch.ones(64, dtype=torch.int32, device=DEV)
    # (7553 pieces + 512 streams) x 8 heads x 520 B of partials and 512 arrival words: just past 32 MiB
    assert nv.decode_workspace_size(64, 64, 8, 7552) <= nv.decode_noalloc_max_bytes()
    with pytest.raises(RuntimeError, match="status -5"):
        nv.nvfp4_decode_noalloc(q, pool, 1.0, 1.0, pt, sl, 0.1, (2, 7553), 8)
