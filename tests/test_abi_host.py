"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function that
include/nvkv.h declares, plans splits consistently, and rejects bad arguments before any launch.

Every call below is invalid on purpose and must fail validation; no kernel is ever launched with
the fake pointers used here.
"""
import ctypes
import math
import os
import re

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvkv.h")

OK, INVAL, UNSUP, LAUNCH, WS, SCRATCH = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    from bit_paged_kv_amd import _lib
    return _lib


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"NVKV_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))


def test_every_declared_function_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(lib._lib, n), f"{n} not exported by libnvkv.so"
        assert n in lib.EXPORTED, f"{n} has no binding"
    assert set(lib.EXPORTED) == names


def test_header_is_plain_c():
    text = open(HEADER).read()
    assert 'extern "C"' in text and "torch" not in text.lower().replace("torch types", "")


def test_status_strings(lib):
    for st in (OK, INVAL, UNSUP, LAUNCH, WS, SCRATCH, 12345):
        assert isinstance(lib.status_string(st), str) and lib.status_string(st)
    assert lib.version() >= 100


def _units(b, hkv, L, tot):
    pages = b * math.ceil(L / 16)
    if tot > 0:
        pages = min(pages, (tot + b * 15) // 16)
    return pages * hkv


@pytest.mark.parametrize("b,hkv,L,tot", [(4, 8, 131072, 0), (32, 8, 4096, 0), (1, 1, 1, 0), (1, 1, 256, 0),
                                         (64, 8, 32768, 500000), (44, 8, 8192, 0), (3, 2, 17, 40)])
def test_plan_pieces(lib, b, hkv, L, tot):
    """The automatic plan: at most two workgroups per CU (256 CUs assumed without a GPU), pieces of
    at least 16 pages, and a minimum piece size that leaves the balancing to the kernel."""
    pps, ns = lib.plan_decode(b, hkv, L, tot)
    assert pps == 2 and 1 <= ns <= 512
    assert ns == min(512, math.ceil(_units(b, hkv, L, tot) / 16))


def test_plan_shapes(lib):
    """The planner's shapes on a 256-CU device (the count it assumes without a GPU, and MI355X's):
    two pieces of equal cost per CU whenever the step has at least 512 x 16 page-heads; on equal lengths
    whose stream count divides 512 the pieces fall on stream boundaries (the kernel's piece is
    the even ceiling of units / pieces)."""
    for args, pieces_per_stream in (((4, 8, 131072, 4 * 131072), 16), ((32, 8, 4096, 32 * 4096), 2)):
        assert lib.plan_decode(*args) == (2, 512)
        assert _units(*args) // 512 * pieces_per_stream == math.ceil(args[2] / 16)
    assert lib.plan_decode(44, 8, 8192, 44 * 8192) == (2, 512)
    rag = workloads.config(3)
    assert lib.plan_decode(rag.batch, rag.h_kv, int(rag.total_lens.max()), int(rag.total_lens.sum())) == (2, 512)
    assert lib.plan_decode(1, 1, 256, 256) == (2, 1)                    # one piece: no merge, no workspace
    assert lib.plan_decode(3, 2, 100, 300) == (2, 3)                    # 42 page-heads: pieces of >= 16


def test_plan_forced_split(lib):
    assert lib.plan_decode(2, 2, 1000, 0, 6) == (6, math.ceil(252 / 6))      # 2 x 63 pages x 2 heads
    assert lib.plan_decode(2, 2, 1000, 0, 5) == (6, math.ceil(252 / 6))      # rounded up to even
    assert lib.plan_decode(2, 2, 100, 0, 1000) == (28, 1)                    # capped at the step


def test_plan_rejects_bad_hints(lib):
    for args in ((0, 8, 10, 0, 0), (1, 0, 10, 0, 0), (1, 8, 0, 0, 0), (1, 8, 10, -1, 0), (1, 8, 10, 0, -2)):
        with pytest.raises(RuntimeError):
            lib.plan_decode(*args)


def test_workspace_size(lib):
    assert lib.decode_workspace_size(4, 64, 8, 1) == 0                   # one piece: no partials
    n = lib.decode_workspace_size(4, 64, 8, 16)
    assert n == (16 + 4 * 8) * 8 * 130 * 4 + 4 * 8 * 8                   # [pieces + streams][group][128 + 2] fp32,
    assert lib.decode_workspace_size(1, 4, 1, 3) == (3 + 1) * 4 * 130 * 4 + 8   # then a 64-bit word per stream
    assert lib._lib.nvkv_decode_workspace_size(4, 64, 8, 64, 16) == 0      # head_dim other than 128


# ---- validation of the compute entry points, with fake (never dereferenced) pointers ----
A = 1 << 20          # a 16-byte aligned fake address
MIS = A + 4          # misaligned
S = None             # default stream


def _decode(lib, **kw):
    a = dict(q=A, kd=A, ks=A, vd=A, vs=A, gk=1.0, gv=1.0, pt=A, maxp=4, sl=A, b=1, hq=8, hkv=2, d=128, page=16,
             sm=0.1, pps=2, ns=1, nk=None, nv=None, out=A, ws=A, wsb=1 << 20)
    a.update(kw)
    return lib._lib.nvfp4_paged_decode_attn(a["q"], a["kd"], a["ks"], a["vd"], a["vs"], a["gk"], a["gv"], a["pt"],
                                            a["maxp"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"], a["page"], a["sm"],
                                            a["pps"], a["ns"], a["nk"], a["nv"], a["out"], a["ws"], a["wsb"], S)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVAL), (dict(kd=None), INVAL), (dict(out=None), INVAL), (dict(pt=None), INVAL),
    (dict(q=MIS), INVAL), (dict(vs=MIS), INVAL), (dict(out=MIS), INVAL), (dict(sl=A + 2), INVAL),
    (dict(d=64), UNSUP), (dict(page=32), UNSUP), (dict(d=0), INVAL),
    (dict(hq=7), INVAL), (dict(hq=64, hkv=2), UNSUP), (dict(hkv=0), INVAL),
    (dict(gk=float("nan")), INVAL), (dict(gv=0.0), INVAL), (dict(gk=-1.0), INVAL), (dict(gk=float("inf")), INVAL),
    (dict(sm=0.0), INVAL), (dict(sm=float("nan")), INVAL),
    (dict(b=0), INVAL), (dict(maxp=0), INVAL), (dict(pps=0), INVAL), (dict(ns=0), INVAL),
    (dict(maxp=1 << 30), UNSUP), (dict(ns=1 << 28, pps=8), UNSUP),   # page-heads / piece offsets past 32 bits
    (dict(nk=A), INVAL),                                    # new_k without new_v
    (dict(ns=4, ws=None, wsb=0), WS), (dict(ns=4, wsb=100), WS),   # workspace missing / too small
    (dict(ns=4, ws=MIS, wsb=1 << 20), INVAL),                        # misaligned workspace
])
def test_decode_validation(lib, kw, want):
    assert _decode(lib, **kw) == want


@pytest.mark.parametrize("kw,want", [(dict(q=None), INVAL), (dict(d=64), UNSUP), (dict(ns=4), WS)])
def test_timed_decode_validates_like_the_plain_call(lib, kw, want):
    a = dict(q=A, kd=A, ks=A, vd=A, vs=A, gk=1.0, gv=1.0, pt=A, maxp=4, sl=A, b=1, hq=8, hkv=2, d=128, page=16,
             sm=0.1, pps=2, ns=1, nk=None, nv=None, out=A, ws=None, wsb=0)
    a.update(kw)
    st = lib._lib.nvfp4_paged_decode_attn_timed(a["q"], a["kd"], a["ks"], a["vd"], a["vs"], a["gk"], a["gv"],
                                                a["pt"], a["maxp"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"],
                                                a["page"], a["sm"], a["pps"], a["ns"], a["nk"], a["nv"], a["out"],
                                                a["ws"], a["wsb"], S, None, None)
    assert st == want


def _decode_noalloc(lib, **kw):
    a = dict(q=A, kd=A, ks=A, vd=A, vs=A, gk=1.0, gv=1.0, pt=A, maxp=4, sl=A, b=1, hq=8, hkv=2, d=128, page=16,
             sm=0.1, pps=2, ns=4, nk=None, nv=None, out=A)
    a.update(kw)
    return lib._lib.nvfp4_paged_decode_attn_noalloc(a["q"], a["kd"], a["ks"], a["vd"], a["vs"], a["gk"], a["gv"],
                                                    a["pt"], a["maxp"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"],
                                                    a["page"], a["sm"], a["pps"], a["ns"], a["nk"], a["nv"], a["out"],
                                                    S)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INVAL), (dict(kd=None), INVAL), (dict(out=MIS), INVAL), (dict(d=64), UNSUP),
    (dict(hq=64, hkv=2), UNSUP), (dict(gk=float("inf")), INVAL), (dict(sm=0.0), INVAL), (dict(ns=0), INVAL),
    (dict(nk=A), INVAL),
    # partials beyond the library-held array: (7553 pieces + 512 streams) x 8 heads x 520 B + 4 KiB > 32 MiB
    (dict(b=64, hq=64, hkv=8, ns=7553), SCRATCH),
    (dict(b=64, hq=64, hkv=8, ns=7553, q=None), INVAL),     # argument errors are reported first
])
def test_noalloc_decode_validation(lib, kw, want):
    assert lib.decode_noalloc_max_bytes() == 32 << 20
    assert lib.decode_workspace_size(64, 64, 8, 7552) <= 32 << 20 < lib.decode_workspace_size(64, 64, 8, 7553)
    assert _decode_noalloc(lib, **kw) == want


def test_fp8_decode_and_layers_validation(lib):
    f = lib._lib.fp8_paged_decode_attn
    assert f(A, A, A, 1.0, 1.0, A, 4, A, 1, 8, 2, 128, 16, 0.1, 2, 1, None, A, 1 << 20, S) == INVAL   # out null
    assert f(A, A, A, 1.0, 1.0, A, 4, A, 1, 8, 2, 128, 16, 0.1, 2, 4, A, None, 0, S) == WS     # no workspace
    assert f(A, A, None, 1.0, 1.0, A, 4, A, 1, 8, 2, 128, 16, 0.1, 2, 1, A, A, 1 << 20, S) == INVAL
    assert f(A, A, A, 0.0, 1.0, A, 4, A, 1, 8, 2, 128, 16, 0.1, 2, 1, A, A, 1 << 20, S) == INVAL
    assert lib._lib.nvkv_decode_layers(None, 1, A, 4, A, 1, 8, 2, 128, 16, 0.1, 2, 1, A, 1 << 20, S) == INVAL
    layers = (lib.NvkvLayer * 2)()
    layers[0] = lib.NvkvLayer(0, A, A, A, A, A, 1.0, 1.0, A)
    layers[1] = lib.NvkvLayer(7, A, A, A, A, A, 1.0, 1.0, A)          # unknown precision: nothing launches
    assert lib._lib.nvkv_decode_layers(ctypes.cast(layers, ctypes.c_void_p), 2, A, 4, A, 1, 8, 2, 128, 16, 0.1,
                                       2, 1, A, 1 << 20, S) == INVAL
    layers[1] = lib.NvkvLayer(0, A, A, None, A, A, 1.0, 1.0, A)       # NVFP4 layer without K scales
    assert lib._lib.nvkv_decode_layers(ctypes.cast(layers, ctypes.c_void_p), 2, A, 4, A, 1, 8, 2, 128, 16, 0.1,
                                       2, 1, A, 1 << 20, S) == INVAL


def test_quantize_validation(lib):
    q = lib._lib.nvfp4_kv_quantize_append
    base = [A, A, 0, 1.0, 1.0, A, 4, 2, 128, 16, 1.0, 1.0, A, A, A, A, S]

    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return q(*a)
    assert call(a0=None) == INVAL
    assert call(a0=MIS) == INVAL
    assert call(a2=5) == INVAL                           # unknown input dtype
    assert call(a2=1, a3=0.0) == INVAL                   # FP8 input needs its scale
    assert call(a6=-1) == INVAL
    assert call(a6=0) == OK                              # nothing to do: no launch
    assert call(a8=64) == UNSUP
    assert call(a9=8) == UNSUP
    assert call(a10=float("nan")) == INVAL
    assert call(a11=1e-39) == INVAL                      # subnormal global scale
    assert call(a15=MIS) == INVAL
    f = lib._lib.fp8_kv_quantize_append
    assert f(A, A, A, 4, 2, 128, 16, 0.0, 1.0, A, A, S) == INVAL
    assert f(A, None, A, 4, 2, 128, 16, 1.0, 1.0, A, A, S) == INVAL
    assert f(A, A, A, 0, 2, 128, 16, 1.0, 1.0, A, A, S) == OK


def test_global_scale_and_dequant_validation(lib):
    g = lib._lib.nvkv_global_scale
    wsz = lib._lib.nvkv_global_scale_workspace_size()
    assert wsz >= 4
    assert g(A, 0, 1.0, 0, 2688.0, A, A, wsz, S) == INVAL        # empty tensor
    assert g(A, 0, 1.0, 10, 0.0, A, A, wsz, S) == INVAL          # divisor
    assert g(A, 2, 1.0, 10, 2688.0, A, A, wsz, S) == INVAL       # dtype
    assert g(A, 0, 1.0, 10, 2688.0, A, A, wsz - 1, S) == WS
    assert g(MIS, 0, 1.0, 10, 2688.0, A, A, wsz, S) == INVAL
    d = lib._lib.nvfp4_dequant_to_workspace
    args = [A, A, A, A, 1.0, 1.0, A, 4, A, A, 1, 2, 128, 16, 64, 1.0, 1.0, A, A, S]
    bad = list(args); bad[14] = 65                               # prefix longer than the page table
    assert d(*bad) == INVAL
    bad = list(args); bad[15] = 0.0
    assert d(*bad) == INVAL
    bad = list(args); bad[17] = None
    assert d(*bad) == INVAL
    bad = list(args); bad[12] = 256
    assert d(*bad) == UNSUP
    ok0 = list(args); ok0[14] = 0                                 # nothing to gather: no launch
    assert d(*ok0) == OK


def test_extend_validation(lib):
    """The extend calls reject bad arguments; a zero chunk bound is a no-op (no launch)."""
    ap = lib._lib.fp8_workspace_append
    #       k  v  chunk_off ws_off prefix batch hkv D    max_c max_p  sk   sv   k_ws v_ws stream
    base = [A, A, A,        A,     A,     2,    8,  128, 64,   1024,  1.0, 1.0, A,   A,   S]
    assert ap(*base[:8], 0, *base[9:]) == OK
    mis4 = A + 2                                      # not 4-byte aligned (int32 arrays)
    for i, v, want in ((0, None, INVAL), (1, MIS, INVAL), (2, mis4, INVAL), (4, None, INVAL), (5, 0, INVAL),
                       (5, 70000, INVAL), (6, 0, INVAL), (7, 64, UNSUP), (8, -1, INVAL), (9, -1, INVAL),
                       (10, 0.0, INVAL), (11, float("inf"), INVAL), (12, None, INVAL), (13, MIS, INVAL),
                       (9, 1 << 21, INVAL)):                  # (prefix + chunk) * H_kv * 128 >= 2^31 bytes
        a = list(base); a[i] = v
        assert ap(*a) == want, (i, v)
    ex = lib._lib.fp8_extend_attn
    #       q  c_off k_ws v_ws ws_off prefix sk   sv   sm    batch hq  hkv D    max_c max_p out stream
    base = [A, A,    A,   A,   A,     A,     1.0, 1.0, 0.09, 2,    32, 8,  128, 64,   1024, A,  S]
    assert ex(*base[:13], 0, *base[14:]) == OK
    for i, v, want in ((0, None, INVAL), (0, MIS, INVAL), (15, None, INVAL), (15, MIS, INVAL), (8, 0.0, INVAL),
                       (8, float("nan"), INVAL), (10, 30, INVAL), (10, 8 * 17, UNSUP), (12, 96, UNSUP),
                       (9, 0, INVAL), (13, -5, INVAL), (6, -1.0, INVAL), (14, 1 << 21, INVAL), (1, A + 2, INVAL),
                       (4, None, INVAL)):
        a = list(base); a[i] = v
        assert ex(*a) == want, (i, v)


def test_prefill_write_validation(lib):
    pw = lib._lib.nvfp4_prefill_write
    #       k  v  dt  ks   vs   slots n  hkv D    page g_k  g_v  kd ks vd vs  sk_ws sv_ws k_ws v_ws stream
    base = [A, A, 0,  1.0, 1.0, A,    4, 2,  128, 16,  1.0, 1.0, A, A, A, A,  1.0,  1.0,  A,   A,   S]
    ok0 = list(base); ok0[6] = 0
    assert pw(*ok0) == OK                                 # nothing to write: no launch
    for i, v, want in ((0, None, INVAL), (0, MIS, INVAL), (2, 7, INVAL), (5, A + 2, INVAL), (6, -1, INVAL),
                       (7, 0, INVAL), (7, 70000, UNSUP), (8, 64, UNSUP), (9, 32, UNSUP), (10, 0.0, INVAL),
                       (16, 0.0, INVAL), (17, float("nan"), INVAL), (18, None, INVAL), (19, MIS, INVAL),
                       (15, None, INVAL)):
        a = list(base); a[i] = v
        assert pw(*a) == want, (i, v)


def test_read_probe_validation(lib):
    p = lib._lib.nvkv_read_probe
    assert p(None, 32, A, S) == INVAL
    assert p(A, 32, None, S) == INVAL
    assert p(A, 0, A, S) == INVAL
    assert p(A, 15, A, S) == INVAL
    assert p(A, 40, A, S) == INVAL          # not a multiple of 16
    assert p(MIS, 32, A, S) == INVAL
    assert p(A, 32, A + 2, S) == INVAL      # sink not 4-byte aligned


@pytest.mark.parametrize("dtype", ["float16", "float32", "int8"])
def test_quantize_binding_rejects_other_input_dtypes(lib, dtype):
    """Only bf16 values or E4M3 bytes (uint8) may be quantized; other dtypes raise before any call."""
    import torch
    k = torch.zeros((1, 1, 128), dtype=getattr(torch, dtype))
    pool = {n: torch.zeros((1, 1, 8), dtype=torch.uint8) for n in ("k_data", "k_scale", "v_data", "v_scale")}
    slots = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError):
        lib.nvfp4_quantize_append(k, k.clone(), slots, 1.0, 1.0, pool)
    with pytest.raises(TypeError):
        lib.nvfp4_prefill_write(k, k.clone(), slots, 1.0, 1.0, pool, 1.0, 1.0, k, k)


def test_quantize_binding_rejects_mixed_k_v_dtypes(lib):
    import torch
    k = torch.zeros((1, 1, 128), dtype=torch.bfloat16)
    v = torch.zeros((1, 1, 128), dtype=torch.uint8)
    pool = {n: torch.zeros((1, 1, 8), dtype=torch.uint8) for n in ("k_data", "k_scale", "v_data", "v_scale")}
    with pytest.raises(TypeError):
        lib.nvfp4_quantize_append(k, v, torch.zeros(1, dtype=torch.int32), 1.0, 1.0, pool)
