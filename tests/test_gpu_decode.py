"""GPU parity of decode attention through the C ABI against the fp64 oracle on the oracle's own
dequantized cache: max-abs <= 2e-3 and rel-L2 <= 1e-3 over the whole output (tests/helpers.py)."""
import multiprocessing as mp

import numpy as np
import pytest
import torch

import workloads
from oracle import attention as o_att
from oracle import fp8 as o_fp8
from oracle import layout as o_layout
from oracle import nvfp4 as o_nv
from tests import helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def nv():
    import bit_paged_kv_amd as nv
    return nv


def _run_nvfp4(nv, wl, pool, gk, gv, force_pps=0, layer=0, fused=False):
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()), force_pps)
    q = wl.q(layer).to(DEV)
    nk = wl.new_token("k", layer).to(DEV) if fused else None
    nvv = wl.new_token("v", layer).to(DEV) if fused else None
    out = nv.nvfp4_decode(q, pool, gk, gv, pt, sl, wl.sm_scale, plan, wl.h_kv, new_k=nk, new_v=nvv)
    torch.cuda.synchronize()
    return out.cpu().numpy(), plan


def test_decode_tiny(nv):
    wl = workloads.config(0)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool, g_k, g_v = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0xFF)   # unused bytes hold NaN scale patterns
    assert (np.float32(g_k), np.float32(g_v)) == (gk, gv), "GPU global scales differ from the oracle's"
    for pps in (0, 2, 4, 16):
        got, plan = _run_nvfp4(nv, wl, pool, gk, gv, force_pps=pps)
        H.assert_attention_close(got, want, f"tiny plan={plan}")


@pytest.fixture(scope="module")
def ragged(nv):
    wl = workloads.Workload(name="ragged-small", seed=21, batch=7, h_kv=2, h_q=16,
                            seq_lens=[1, 15, 16, 17, 33, 700, 1283], extra_pages=5)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0xFF)
    return wl, pool, gk, gv, want


@pytest.mark.parametrize("pps", [0, 2, 4, 6, 32, 1000])
def test_decode_ragged_split_sizes(nv, ragged, pps):
    wl, pool, gk, gv, want = ragged
    got, plan = _run_nvfp4(nv, wl, pool, float(gk), float(gv), force_pps=pps)
    H.assert_attention_close(got, want, f"ragged plan={plan}")


def test_decode_split_count_invariance(nv, ragged):
    wl, pool, gk, gv, _ = ragged
    outs = [_run_nvfp4(nv, wl, pool, float(gk), float(gv), force_pps=p)[0] for p in (2, 8, 1000)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-5


@pytest.mark.parametrize("plan", [(2, 3), (3, 2), (5, 1), (7, 4)])
def test_decode_plan_shorter_than_sequences(nv, ragged, plan):
    """Plans whose num_splits x pages_per_split units do not cover the step (and odd minimum piece
    sizes): the pieces grow to the even ceiling of the step's cost over num_splits."""
    wl, pool, gk, gv, want = ragged
    pt, sl = H.gpu_tables(wl, DEV)
    got = nv.nvfp4_decode(wl.q().to(DEV), pool, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv)
    torch.cuda.synchronize()
    H.assert_attention_close(got.cpu().numpy(), want, f"plan {plan}")


@pytest.mark.parametrize("group", [1, 2, 8, 16])
def test_decode_gqa_groups(nv, group):
    wl = workloads.Workload(name=f"gqa{group}", seed=30 + group, batch=2, h_kv=2, h_q=2 * group,
                            seq_lens=[257, 100])
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV)
    got, plan = _run_nvfp4(nv, wl, pool, float(gk), float(gv))
    H.assert_attention_close(got, want, f"group {group}")


def test_decode_page_permutation_invariance(nv):
    a = workloads.Workload(name="perm", seed=40, batch=2, h_kv=2, h_q=8, seq_lens=[500, 231], page_mode="identity")
    b = workloads.Workload(name="perm", seed=40, batch=2, h_kv=2, h_q=8, seq_lens=[500, 231], extra_pages=11)
    assert not np.array_equal(a.page_table, b.page_table[:, :a.page_table.shape[1]])
    outs = []
    for wl in (a, b):
        pool, gk, gv = H.gpu_nvfp4_layer(wl, 0, DEV)
        outs.append(_run_nvfp4(nv, wl, pool, gk, gv, force_pps=4)[0])
    # the same pages in the same order: the result must not depend on where they sit in the pool
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("lens_kind", ["ragged", "equal"])
def test_decode_batch_over_64(nv, lens_kind):
    """More than 64 sequences: every workgroup finds its first stream, and the merging piece its
    stream's pieces, from the lengths 64 at a time.  Ragged lengths (pieces of equal cost, several
    streams per piece) and equal ones (paired pieces), under the automatic plan and forced ones."""
    rng = np.random.default_rng(130)
    lens = rng.integers(1, 200, size=130) if lens_kind == "ragged" else np.full(130, 70)
    wl = workloads.Workload(name=f"b130-{lens_kind}", seed=131, batch=130, h_kv=2, h_q=8,
                            seq_lens=[int(x) for x in lens], extra_pages=9)
    ks, vs = H.oracle_inputs(wl)
    gk, gv = H.oracle_nvfp4_scales(wl)
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0xFF)
    outs = []
    for pps in (0, 2, 6, 1000):
        got, plan = _run_nvfp4(nv, wl, pool, float(gk), float(gv), force_pps=pps)
        H.assert_attention_close(got, want, f"{lens_kind} plan={plan}")
        outs.append(got)
    for o in outs[1:]:   # plans differ only in the order of fp32 sums
        np.testing.assert_allclose(o, outs[0], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("fill", ["random", 0x00, 0xFF])
def test_decode_workspace_reuse_across_plans(nv, ragged, fill):
    """One workspace, never cleared, starting from arbitrary bytes, shared by calls with different
    plans (so each call's partials and arrival words sit where other calls left other data) and by
    an FP8 decode: every result matches the oracle and repeats bit for bit."""
    wl, pool, gk, gv, want = ragged
    pt, sl = H.gpu_tables(wl, DEV)
    q = wl.q().to(DEV)
    plans = [nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, p) for p in (2, 6, 4, 2)]
    plans.append((2, 3))
    size = max(nv.decode_workspace_size(wl.batch, wl.h_q, wl.h_kv, ns) for _, ns in plans)
    g = torch.Generator(device="cpu").manual_seed(77)
    if fill == "random":
        ws = torch.randint(0, 256, (size,), dtype=torch.uint8, generator=g).to(DEV)
    else:
        ws = torch.full((size,), fill, dtype=torch.uint8, device=DEV)
    first = {}
    for rep in range(2):
        for plan in plans:
            got = nv.nvfp4_decode(q, pool, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv,
                                  workspace=ws).cpu().numpy()
            H.assert_attention_close(got, want, f"plan {plan} fill {fill}")
            if plan in first:
                assert np.array_equal(got, first[plan])
            first.setdefault(plan, got)
        # an FP8 decode of other data through the same workspace in between
        fp8_pool = nv.alloc_fp8_pool(wl.num_pages, wl.h_kv, DEV, fill=0)
        nv.fp8_decode(q, fp8_pool, 1.0, 1.0, pt, sl, wl.sm_scale, plans[0], wl.h_kv, workspace=ws)
    torch.cuda.synchronize()


def test_decode_repeat_calls_agree_to_rounding(nv, ragged):
    """Run-to-run: a shared workspace reused by several calls gives the same result each time."""
    wl, pool, gk, gv, want = ragged
    pt, sl = H.gpu_tables(wl, DEV)
    q = wl.q().to(DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, 2)
    ws = nv.alloc_decode_workspace(wl.batch, wl.h_q, wl.h_kv, plan[1], DEV)
    outs = []
    for _ in range(4):
        outs.append(nv.nvfp4_decode(q, pool, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv,
                                    workspace=ws).cpu().numpy())
    for o in outs:
        H.assert_attention_close(o, want, "repeat")
        assert np.array_equal(o, outs[0])


def test_decode_fused_append(nv):
    wl = workloads.Workload(name="append", seed=50, batch=6, h_kv=2, h_q=16,
                            seq_lens=[15, 16, 31, 1, 200, 513], append=True, extra_pages=3)
    ks, vs = H.oracle_inputs(wl)                        # cache + new token
    gk, gv = H.oracle_nvfp4_scales(wl)                  # from the cache only
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    want_pool = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0x3C)
    for pps in (0, 2, 1000):
        pool, g_k, g_v = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0x3C)   # cache without the new tokens
        assert (np.float32(g_k), np.float32(g_v)) == (gk, gv)
        got, plan = _run_nvfp4(nv, wl, pool, g_k, g_v, force_pps=pps, fused=True)
        H.assert_attention_close(got, want, f"fused append plan={plan}")
        for key in ("k_data", "k_scale", "v_data", "v_scale"):
            assert np.array_equal(pool[key].cpu().numpy(), want_pool[key]), key


def test_fused_append_infinities_match_standalone_writer(nv):
    """New tokens holding +-inf and values far past the calibrated range: the decode kernel's fused
    append (built without NaN semantics) writes the same bytes as nvfp4_kv_quantize_append and as
    the oracle -- infinities saturate to a 448 block scale and code +-6, no NaN arises."""
    wl = workloads.Workload(name="append-inf", seed=51, batch=3, h_kv=2, h_q=8, seq_lens=[20, 33, 7],
                            append=True, extra_pages=1)
    gk, gv = H.oracle_nvfp4_scales(wl)
    nk = wl.new_token("k").clone()
    nvv = wl.new_token("v").clone()
    nk[0, 0, 5] = float("inf")
    nk[1, 1, 64:80] = float("-inf")
    nk[2, 0, :16] = 1e30
    nvv[0, 1, 127] = float("-inf")
    nvv[2, 1, 40] = float("inf")
    # oracle bytes of the whole cache + the new tokens
    ks, vs = H.oracle_inputs(wl, with_new=False)
    ks = [np.concatenate([k, nk[b:b + 1].float().numpy()]) for b, k in enumerate(ks)]
    vs = [np.concatenate([v, nvv[b:b + 1].float().numpy()]) for b, v in enumerate(vs)]
    want_pool = H.oracle_nvfp4_pool(wl, ks, vs, gk, gv, fill=0x11)
    # fused: decode with new_k / new_v
    pool_f, g_k, g_v = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0x11)
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, 2)
    nv.nvfp4_decode(wl.q().to(DEV), pool_f, g_k, g_v, pt, sl, wl.sm_scale, plan, wl.h_kv, new_k=nk.to(DEV),
                    new_v=nvv.to(DEV))
    # standalone writer of the same tokens
    pool_s, _, _ = H.gpu_nvfp4_layer(wl, 0, DEV, fill=0x11)
    slots = np.array([wl.page_table[b, int(wl.seq_lens[b]) // 16] * 16 + int(wl.seq_lens[b]) % 16
                      for b in range(wl.batch)], dtype=np.int32)
    nv.nvfp4_quantize_append(nk.to(DEV), nvv.to(DEV), torch.from_numpy(slots).to(DEV), g_k, g_v, pool_s)
    torch.cuda.synchronize()
    for key in ("k_data", "k_scale", "v_data", "v_scale"):
        f, st = pool_f[key].cpu().numpy(), pool_s[key].cpu().numpy()
        assert np.array_equal(f, st), f"{key}: fused append differs from the standalone writer"
        assert np.array_equal(f, want_pool[key]), f"{key}: differs from the oracle"


def _fp8_case(wl, layer=0):
    ks, vs = H.oracle_inputs(wl, layer)
    sk = o_fp8.fp8_scale(np.concatenate(ks))
    sv = o_fp8.fp8_scale(np.concatenate(vs))
    want = H.oracle_fp8_decode(wl, wl.q(layer).float().numpy(), ks, vs, sk, sv)
    return want, sk, sv


@pytest.mark.parametrize("group", [1, 2, 4, 8, 16])
def test_fp8_decode(nv, group):
    """FP8 layers across GQA groups: 1..8 use the packed hi/lo kernel, 16 the two-product one."""
    from bit_paged_kv_amd import paged
    wl = workloads.Workload(name=f"fp8-g{group}", seed=60 + group, batch=4, h_kv=2, h_q=2 * group,
                            seq_lens=[1, 17, 300, 1029], chan="outlier2", extra_pages=2)
    want, sk, sv = _fp8_case(wl)
    k, v, slots = H.gpu_all_tokens(wl, 0, DEV)
    pool, g_sk, g_sv = paged.build_fp8_cache(k, v, slots, wl.num_pages, fill=0xFF)
    pt, sl = H.gpu_tables(wl, DEV)
    for pps in (0, 2, 64):
        plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, pps)
        got = nv.fp8_decode(wl.q().to(DEV), pool, g_sk, g_sv, pt, sl, wl.sm_scale, plan, wl.h_kv)
        H.assert_attention_close(got.cpu().numpy(), want, f"fp8 plan={plan}")


@pytest.mark.parametrize("i", range(8))
def test_fp8_decode_random_shapes(nv, i):
    """FP8 layers on seeded random shapes (as the NVFP4 ones, without the append, which FP8 caches
    do not have), automatic and forced plans."""
    import dataclasses
    from bit_paged_kv_amd import paged
    wl, pps = _random_case(50 + i)
    wl = dataclasses.replace(wl, name=f"fp8-random-{i}", append=False)
    want, sk, sv = _fp8_case(wl)
    k, v, slots = H.gpu_all_tokens(wl, 0, DEV)
    pool, g_sk, g_sv = paged.build_fp8_cache(k, v, slots, wl.num_pages, fill=0xFF)
    assert (np.float32(g_sk), np.float32(g_sv)) == (sk, sv)
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()), pps)
    got = nv.fp8_decode(wl.q().to(DEV), pool, g_sk, g_sv, pt, sl, wl.sm_scale, plan, wl.h_kv)
    tag = f"fp8 random case {i}: batch {wl.batch}, Hkv {wl.h_kv}, G {wl.h_q // wl.h_kv}, plan {plan}"
    err = H.assert_attention_close(got.cpu().numpy(), want, tag)
    print(f"{tag}: max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}", flush=True)


def test_decode_layers_mixed_stack(nv):
    from bit_paged_kv_amd import paged
    wl = workloads.Workload(name="mixed-small", seed=70, batch=3, h_kv=2, h_q=8, seq_lens=[64, 300, 17],
                            chan="outlier2", layers=4, fp8_layers=(0, 3))
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()))
    layers, wants = [], []
    for layer in range(wl.layers):
        k, v, slots = H.gpu_all_tokens(wl, layer, DEV)
        if wl.is_fp8(layer):
            pool, s1, s2 = paged.build_fp8_cache(k, v, slots, wl.num_pages)
            want, _, _ = _fp8_case(wl, layer)
            prec = nv.PREC_FP8
        else:
            pool, s1, s2 = paged.build_nvfp4_cache(k, v, slots, wl.num_pages)
            ks, vs = H.oracle_inputs(wl, layer)
            gk, gv = H.oracle_nvfp4_scales(wl, layer)
            want = H.oracle_nvfp4_decode(wl, wl.q(layer).float().numpy(), ks, vs, gk, gv)
            prec = nv.PREC_NVFP4
        layers.append(dict(precision=prec, q=wl.q(layer).to(DEV), pool=pool, k_gscale=s1, v_gscale=s2,
                           out=torch.empty((wl.batch, wl.h_q, 128), dtype=torch.float32, device=DEV)))
        wants.append(want)
    outs = nv.decode_layers(layers, pt, sl, wl.sm_scale, plan, wl.h_kv)
    torch.cuda.synchronize()
    for i, (o, w) in enumerate(zip(outs, wants)):
        H.assert_attention_close(o.cpu().numpy(), w, f"layer {i}")
    # the prepared form issues the same launches: bitwise equal results, call after call
    first = [o.clone() for o in outs]
    for L in layers:
        L["out"] = torch.full_like(L["out"], float("nan"))
    call = nv.prepare_decode_layers(layers, pt, sl, wl.sm_scale, plan, wl.h_kv)
    for _ in range(2):
        call.run()
        torch.cuda.synchronize()
        for i, L in enumerate(layers):
            assert torch.equal(L["out"], first[i]), f"prepared layer {i}"


def _random_case(i):
    """A seeded random decode shape: batch, kv heads, group size (1..16, not only powers of two),
    equal, ragged or mostly one-token lengths, fused append or not, and an automatic or forced plan.
    The whole cache stays under ~80k token-heads so the oracle finishes in about a second."""
    rng = np.random.default_rng(9000 + i)
    batch = int(rng.choice([1, 2, 3, 7, 31, 64, 65, 100, 140]))
    h_kv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    kind = int(rng.integers(0, 3))
    budget = 80_000 // h_kv
    if kind == 0:
        lens = [int(rng.integers(1, max(2, budget // batch)))] * batch
    else:
        lens = rng.integers(1, max(2, min(4000, 2 * budget // batch)), size=batch)
        if kind == 2:
            lens[rng.random(batch) < 0.3] = 1
    wl = workloads.Workload(name=f"random-{i}", seed=9100 + i, batch=batch, h_kv=h_kv, h_q=h_kv * group,
                            seq_lens=lens, append=bool(rng.integers(0, 2)), extra_pages=int(rng.integers(0, 5)))
    return wl, int(rng.choice([0, 0, 2, 4, 6, 16, 64, 1000]))


@pytest.mark.parametrize("i", range(24))
def test_decode_random_shapes(nv, i):
    wl, pps = _random_case(i)
    ks, vs = H.oracle_inputs(wl)                        # cache (+ the appended token)
    gk, gv = H.oracle_nvfp4_scales(wl)                  # from the cache only
    want = H.oracle_nvfp4_decode(wl, wl.q().float().numpy(), ks, vs, gk, gv)
    pool, g_k, g_v = H.gpu_nvfp4_layer(wl, 0, DEV)
    assert (np.float32(g_k), np.float32(g_v)) == (gk, gv)
    got, plan = _run_nvfp4(nv, wl, pool, g_k, g_v, force_pps=pps, fused=wl.append)
    tag = (f"random case {i}: batch {wl.batch}, Hkv {wl.h_kv}, G {wl.h_q // wl.h_kv}, tokens {int(wl.total_lens.sum())}, "
           f"append {wl.append}, plan {plan}")
    err = H.assert_attention_close(got, want, tag)
    print(f"{tag}: max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}", flush=True)


def _pool_rows(pool, wl, b, hk, n_tok):
    """The pages of stream (b, hk) that hold its first n_tok tokens, copied to the host in sequence
    order: {key: [pages][1][bytes]}, so that token t sits at local slot t."""
    pages = torch.from_numpy(wl.page_table[b, :(n_tok + 15) // 16].astype(np.int64)).to(DEV)
    return {key: t[pages, hk:hk + 1].cpu().numpy() for key, t in pool.items()}


def _assert_nvfp4_rows(rows, ck, sk, cv, sv, tag):
    """Every code and scale byte of one stream's tokens equals the oracle's."""
    n = ck.shape[0]
    local = np.arange(n)
    gck, gsk = o_layout.read_nvfp4_tokens(rows["k_data"], rows["k_scale"], "k", local)
    gcv, gsv = o_layout.read_nvfp4_tokens(rows["v_data"], rows["v_scale"], "v", local)
    for name, got, want in (("K codes", gck[:, 0], ck), ("K scales", gsk[:, 0], sk), ("V codes", gcv[:, 0], cv),
                            ("V scales", gsv[:, 0], sv)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{tag}: {name} differ at {len(bad)} places, first (token, index) {bad[0].tolist()}"
    print(f"{tag}: {n} tokens' codes and scales bit-exact", flush=True)


def _sampled_full_size(nv, index, samples):
    """Full-size workload in the bench's launch configuration.  Every (sequence, kv head) stream's
    code and scale bytes, as the step left them, are compared with the oracle's (digests that a
    pool of host workers computes from the seeded inputs); the oracle recomputes the sampled
    streams' attention rows from the same inputs.  Nothing the GPU produced is fed to the oracle."""
    wl = workloads.config(index)
    ks = [wl.kv("k", b) for b in range(wl.batch)]
    vs = [wl.kv("v", b) for b in range(wl.batch)]
    print(f"cfg{index}: inputs generated", flush=True)
    from bit_paged_kv_amd import paged
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(DEV)
    k_all = torch.cat(ks).to(DEV)
    v_all = torch.cat(vs).to(DEV)
    pool, gk, gv = paged.build_nvfp4_cache(k_all, v_all, slots, wl.num_pages)
    del k_all, v_all
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()))
    q = wl.q()
    fused = wl.append
    nk = wl.new_token("k") if fused else None
    nvv = wl.new_token("v") if fused else None
    out = nv.nvfp4_decode(q.to(DEV), pool, gk, gv, pt, sl, wl.sm_scale, plan, wl.h_kv,
                          new_k=nk.to(DEV) if fused else None, new_v=nvv.to(DEV) if fused else None).cpu().numpy()
    print(f"cfg{index}: GPU step done, plan {plan}", flush=True)
    # the oracle's own global scales, over the whole cached tensors
    ogk = o_nv.global_scale(np.array([max(float(t.float().abs().max()) for t in ks)], np.float32))
    ogv = o_nv.global_scale(np.array([max(float(t.float().abs().max()) for t in vs)], np.float32))
    assert (np.float32(gk), np.float32(gv)) == (ogk, ogv)
    # every stream's pages as the step left them (the appended token included), digested here
    # while host workers digest the oracle's bytes of the same streams
    rows, got = {}, {}
    with mp.get_context("spawn").Pool(H.host_workers()) as workers:
        pending = workers.map_async(H.oracle_stream_digests, H.digest_tasks(wl, index, ogk, ogv))
        for b in range(wl.batch):
            n_tok = int(wl.total_lens[b])
            for hk in range(wl.h_kv):
                r = _pool_rows(pool, wl, b, hk, n_tok)
                got[(b, hk)] = H.pool_stream_digest(r, n_tok)
                if (b, hk) in samples:
                    rows[(b, hk)] = r
        want = {}
        for d in pending.get(timeout=600):
            want.update(d)
    del pool
    torch.cuda.empty_cache()
    bad = sorted(s for s in got if got[s] != want.get(s))
    assert not bad and len(want) == len(got), \
        f"cfg{index}: {len(bad)} of {len(got)} streams' bytes differ from the oracle's, first (b, hk) {bad[:4]}"
    print(f"cfg{index}: every code and scale byte of all {len(got)} streams bit-exact", flush=True)
    qf = q.float().numpy()
    G = wl.group
    for b, hk in samples:
        k = ks[b][:, hk].float().numpy()
        v = vs[b][:, hk].float().numpy()
        if fused:
            k = np.concatenate([k, nk[b, hk][None].float().numpy()])
            v = np.concatenate([v, nvv[b, hk][None].float().numpy()])
        ck, sk = o_nv.quantize_blocks(k, ogk)
        cv, sv = o_nv.quantize_blocks(v, ogv)
        _assert_nvfp4_rows(rows[(b, hk)], ck, sk, cv, sv, f"cfg{index} b={b} hk={hk}")
        kh = o_nv.dequantize_blocks(ck, sk, ogk)[:, None]
        vh = o_nv.dequantize_blocks(cv, sv, ogv)[:, None]
        want = o_att.decode_attention_one(qf[b, hk * G:(hk + 1) * G], kh, vh, wl.sm_scale)
        err = H.assert_attention_close(out[b, hk * G:(hk + 1) * G], want, f"cfg{index} b={b} hk={hk} plan={plan}")
        print(f"cfg{index}: sample b={b} hk={hk} max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}", flush=True)


@pytest.mark.timeout(900)
def test_full_size_long_sampled(nv):
    _sampled_full_size(nv, 2, [(0, 0), (3, 7)])


@pytest.mark.timeout(600)
def test_full_size_batch32_sampled(nv):
    _sampled_full_size(nv, 1, [(0, 0), (17, 3), (31, 7)])


@pytest.mark.timeout(600)
def test_full_size_ragged_fused_sampled(nv):
    wl = workloads.config(3)
    longest = int(np.argmax(wl.seq_lens))
    shortest = int(np.argmin(wl.seq_lens))
    _sampled_full_size(nv, 3, [(longest, 2), (shortest, 5)])


@pytest.mark.timeout(900)
def test_full_size_mixed_stack_sampled(nv):
    """The 28-layer stack's shape (44 x 8192 tokens, 8 KV / 32 query heads) in the bench's plan, one
    FP8 layer and one NVFP4 layer dispatched together by nvkv_decode_layers; sampled (sequence, kv
    head) rows against the oracle, which derives every scale from the seeded inputs itself."""
    from bit_paged_kv_amd import paged
    wl = workloads.config(4)
    fp8_layer = int(wl.fp8_layers[0])
    nv4_layer = next(l for l in range(wl.layers) if not wl.is_fp8(l))
    pt, sl = H.gpu_tables(wl, DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), int(wl.total_lens.sum()))
    slots = torch.from_numpy(np.concatenate([wl.slots(b) for b in range(wl.batch)])).to(DEV)
    layers, host = [], {}
    for layer in (fp8_layer, nv4_layer):
        ks = [wl.kv("k", b, layer) for b in range(wl.batch)]
        vs = [wl.kv("v", b, layer) for b in range(wl.batch)]
        k_all, v_all = torch.cat(ks).to(DEV), torch.cat(vs).to(DEV)
        if wl.is_fp8(layer):
            pool, s1, s2 = paged.build_fp8_cache(k_all, v_all, slots, wl.num_pages)
            prec = nv.PREC_FP8
        else:
            pool, s1, s2 = paged.build_nvfp4_cache(k_all, v_all, slots, wl.num_pages)
            prec = nv.PREC_NVFP4
        del k_all, v_all
        layers.append(dict(precision=prec, q=wl.q(layer).to(DEV), pool=pool, k_gscale=s1, v_gscale=s2,
                           out=torch.empty((wl.batch, wl.h_q, 128), dtype=torch.float32, device=DEV)))
        amax_k = np.array([max(float(t.float().abs().max()) for t in ks)], np.float32)
        amax_v = np.array([max(float(t.float().abs().max()) for t in vs)], np.float32)
        host[layer] = (ks, vs, amax_k, amax_v, s1, s2)
        print(f"mixed full size: layer {layer} cache built", flush=True)
    outs = [o.cpu().numpy() for o in nv.decode_layers(layers, pt, sl, wl.sm_scale, plan, wl.h_kv)]
    print(f"mixed full size: GPU step done, plan {plan}", flush=True)
    samples = [(0, 0), (21, 5), (43, 7)]
    # the oracle's scales from the seeded inputs; then every stream's bytes of both layers against
    # the oracle's (digests from host workers), keeping the sampled streams' pages
    scales = {}
    for layer in (fp8_layer, nv4_layer):
        ks, vs, amax_k, amax_v, s1, s2 = host[layer]
        if wl.is_fp8(layer):
            scales[layer] = (o_fp8.fp8_scale(amax_k), o_fp8.fp8_scale(amax_v))
        else:
            scales[layer] = (o_nv.global_scale(amax_k), o_nv.global_scale(amax_v))
        assert (np.float32(s1), np.float32(s2)) == scales[layer], f"layer {layer} scales"
    rows = {}
    with mp.get_context("spawn").Pool(H.host_workers()) as workers:
        pending = {layer: workers.map_async(H.oracle_stream_digests,
                                            H.digest_tasks(wl, 4, *scales[layer], layer, wl.is_fp8(layer)))
                   for layer in (fp8_layer, nv4_layer)}
        for i, layer in enumerate((fp8_layer, nv4_layer)):
            got = {}
            for b in range(wl.batch):
                n_tok = int(wl.total_lens[b])
                for hk in range(wl.h_kv):
                    r = _pool_rows(layers[i]["pool"], wl, b, hk, n_tok)
                    got[(b, hk)] = H.pool_stream_digest(r, n_tok, wl.is_fp8(layer))
                    if (b, hk) in samples:
                        rows[(i, b, hk)] = r
            want = {}
            for d in pending[layer].get(timeout=600):
                want.update(d)
            bad = sorted(s for s in got if got[s] != want.get(s))
            assert not bad and len(want) == len(got), \
                f"mixed layer {layer}: {len(bad)} of {len(got)} streams' bytes differ, first (b, hk) {bad[:4]}"
            print(f"mixed full size: layer {layer}: every cache byte of all {len(got)} streams bit-exact", flush=True)
    del layers
    torch.cuda.empty_cache()
    G = wl.group
    for i, layer in enumerate((fp8_layer, nv4_layer)):
        ks, vs, amax_k, amax_v, s1, s2 = host[layer]
        qf = wl.q(layer).float().numpy()
        fp8 = wl.is_fp8(layer)
        ok, ov = scales[layer]
        for b, hk in samples:
            k = ks[b][:, hk].float().numpy()
            v = vs[b][:, hk].float().numpy()
            r = rows[(i, b, hk)]
            tag = f"mixed layer {layer} b={b} hk={hk}"
            if fp8:
                bk, bv = o_fp8.fp8_quantize(k, ok), o_fp8.fp8_quantize(v, ov)
                local = np.arange(k.shape[0])
                assert np.array_equal(o_layout.read_fp8_tokens(r["k"], "k", local)[:, 0], bk), f"{tag}: K bytes"
                assert np.array_equal(o_layout.read_fp8_tokens(r["v"], "v", local)[:, 0], bv), f"{tag}: V bytes"
                print(f"{tag}: {k.shape[0]} tokens' FP8 bytes bit-exact", flush=True)
                kh = o_fp8.fp8_dequantize(bk, ok)[:, None]
                vh = o_fp8.fp8_dequantize(bv, ov)[:, None]
            else:
                ck, sk = o_nv.quantize_blocks(k, ok)
                cv, sv = o_nv.quantize_blocks(v, ov)
                _assert_nvfp4_rows(r, ck, sk, cv, sv, tag)
                kh = o_nv.dequantize_blocks(ck, sk, ok)[:, None]
                vh = o_nv.dequantize_blocks(cv, sv, ov)[:, None]
            want = o_att.decode_attention_one(qf[b, hk * G:(hk + 1) * G], kh, vh, wl.sm_scale)
            err = H.assert_attention_close(outs[i][b, hk * G:(hk + 1) * G], want,
                                           f"mixed layer {layer} b={b} hk={hk} plan={plan}")
            print(f"mixed full size: layer {layer} b={b} hk={hk} max-abs {err[0]:.2e} rel-L2 {err[1]:.2e}",
                  flush=True)


def test_workspace_reused_across_plans(nv, ragged):
    wl, pool, gk, gv, want = ragged
    pt, sl = H.gpu_tables(wl, DEV)
    q = wl.q().to(DEV)
    plans = [nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, p) for p in (2, 8, 4, 2)]
    most = max(p[1] for p in plans)
    ws = nv.alloc_decode_workspace(wl.batch, wl.h_q, wl.h_kv, most, DEV)
    for plan in plans:
        got = nv.nvfp4_decode(q, pool, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv, workspace=ws)
        torch.cuda.synchronize()
        H.assert_attention_close(got.cpu().numpy(), want, f"reused workspace plan={plan}")


def test_timed_entry_matches_and_records_the_split_kernel(nv, ragged):
    """nvfp4_paged_decode_attn_timed computes what the plain call does, and the event pair its
    split-kernel dispatch records spans a positive time."""
    import ctypes
    wl, pool, gk, gv, want = ragged
    pt, sl = H.gpu_tables(wl, DEV)
    q = wl.q().to(DEV)
    plan = nv.plan_decode(wl.batch, wl.h_kv, int(wl.total_lens.max()), 0, 4)
    call, out = nv.prepare_nvfp4_decode(q, pool, float(gk), float(gv), pt, sl, wl.sm_scale, plan, wl.h_kv)
    call.run()
    torch.cuda.synchronize()
    plain = out.clone()
    hip = ctypes.CDLL("libamdhip64.so.7")
    ev = [ctypes.c_void_p() for _ in range(2)]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    try:
        out.fill_(float("nan"))
        call.run_timed(ev[0], ev[1])
        torch.cuda.synchronize()
        assert torch.equal(out, plain)
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert 0.0 < ms.value < 1000.0
    finally:
        for e in ev:
            hip.hipEventDestroy(e)
    H.assert_attention_close(plain.cpu().numpy(), want, f"timed plan={plan}")
