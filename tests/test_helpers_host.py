"""The whole-cache byte comparison the full-size GPU tests use, checked on the host: digests that
spawned workers compute from the seeded inputs equal the digests of the oracle's own pool as the
layout reader sees it, and one changed byte changes its stream's digest."""
import multiprocessing as mp

import numpy as np

import workloads
from tests import helpers as H


def test_stream_digests_match_the_oracle_pool():
    wl = workloads.Workload(name="digest", seed=52, batch=3, h_kv=2, h_q=4, seq_lens=[20, 33, 7],
                            append=True, extra_pages=3)
    ks, vs = H.oracle_inputs(wl)                 # cache + appended token
    gk, gv = H.oracle_nvfp4_scales(wl)           # from the cache only, as the cache build sets them
    pool = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0x3C)
    tasks = [(wl, b, list(range(wl.h_kv)), gk, gv) for b in range(wl.batch)]
    want = {}
    with mp.get_context("spawn").Pool(2) as workers:
        for d in workers.map(H.oracle_stream_digests, tasks):
            want.update(d)
    assert sorted(want) == [(b, hk) for b in range(wl.batch) for hk in range(wl.h_kv)]

    def got(b, hk):
        n = int(wl.total_lens[b])
        pages = wl.page_table[b, :(n + 15) // 16]
        return H.pool_stream_digest({key: a[pages, hk:hk + 1] for key, a in pool.items()}, n)

    for b in range(wl.batch):
        for hk in range(wl.h_kv):
            assert got(b, hk) == want[(b, hk)], (b, hk)
    page = int(wl.page_table[1, 0])
    pool["v_scale"][page, 1, 0] ^= np.uint8(1)
    assert got(1, 1) != want[(1, 1)]
    assert got(1, 0) == want[(1, 0)]


def test_fp8_stream_digests_match_the_oracle_pool():
    from oracle import fp8 as o_fp8
    from oracle import layout as o_layout
    wl = workloads.Workload(name="digest-fp8", seed=53, batch=2, h_kv=2, h_q=4, seq_lens=[40, 17],
                            extra_pages=2)
    ks, vs = H.oracle_inputs(wl)
    s_k = o_fp8.fp8_scale(np.array([max(float(np.abs(k).max()) for k in ks)], np.float32))
    s_v = o_fp8.fp8_scale(np.array([max(float(np.abs(v).max()) for v in vs)], np.float32))
    pool = {key: np.zeros(o_layout.fp8_pool_shape(wl.num_pages, wl.h_kv), np.uint8) for key in ("k", "v")}
    for b in range(wl.batch):
        slots = wl.slots(b, 0, ks[b].shape[0])
        o_layout.write_fp8_tokens(pool["k"], "k", slots, o_fp8.fp8_quantize(ks[b], s_k))
        o_layout.write_fp8_tokens(pool["v"], "v", slots, o_fp8.fp8_quantize(vs[b], s_v))
    want = {}
    for task in H.digest_tasks(wl, wl, s_k, s_v, 0, True):
        want.update(H.oracle_stream_digests(task))
    for b in range(wl.batch):
        n = int(wl.total_lens[b])
        pages = wl.page_table[b, :(n + 15) // 16]
        for hk in range(wl.h_kv):
            rows = {key: a[pages, hk:hk + 1] for key, a in pool.items()}
            assert H.pool_stream_digest(rows, n, fp8=True) == want[(b, hk)], (b, hk)
