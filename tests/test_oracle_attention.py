"""Pins for the fp64 attention oracle: brute force with Python floats, torch's fp64 SDPA
(a library routine, with GQA), and special cases with closed forms."""
import math

import numpy as np
import torch

from oracle import attention


def _brute(q, k, v, sm):
    """Naive per-element loops (Python floats)."""
    hq, d = q.shape
    length, hkv, _ = k.shape
    g = hq // hkv
    out = np.zeros((hq, d))
    for h in range(hq):
        kh = h // g
        z = [sm * sum(q[h, i] * k[t, kh, i] for i in range(d)) for t in range(length)]
        m = max(z)
        e = [math.exp(zz - m) for zz in z]
        s = sum(e)
        for i in range(d):
            out[h, i] = sum(e[t] * v[t, kh, i] for t in range(length)) / s
    return out


def test_brute_force_tiny():
    rng = np.random.default_rng(9)
    for length, hq, hkv, d in ((1, 2, 1, 4), (5, 4, 2, 8), (17, 6, 3, 5)):
        q = rng.standard_normal((hq, d))
        k = rng.standard_normal((length, hkv, d)) * 3
        v = rng.standard_normal((length, hkv, d))
        sm = 1 / math.sqrt(d)
        np.testing.assert_allclose(attention.decode_attention_one(q, k, v, sm), _brute(q, k, v, sm), rtol=0, atol=1e-12)


def test_torch_sdpa_fp64_gqa():
    rng = np.random.default_rng(10)
    b, hq, hkv, d = 3, 8, 2, 16
    lens = [1, 40, 97]
    q = rng.standard_normal((b, hq, d))
    ks = [rng.standard_normal((n, hkv, d)) * 2 for n in lens]
    vs = [rng.standard_normal((n, hkv, d)) for n in lens]
    sm = 1 / math.sqrt(d)
    ours = attention.decode_attention(q, ks, vs, sm)
    for i, n in enumerate(lens):
        tq = torch.from_numpy(q[i][None, :, None, :])                 # [1, Hq, 1, D]
        tk = torch.from_numpy(ks[i].transpose(1, 0, 2)[None].copy())  # [1, Hkv, L, D]
        tv = torch.from_numpy(vs[i].transpose(1, 0, 2)[None].copy())
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sm, enable_gqa=True)
        np.testing.assert_allclose(ours[i], ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


def test_special_cases():
    rng = np.random.default_rng(11)
    d = 8
    v = rng.standard_normal((6, 1, d))
    # one token: the output is that token's value
    q = rng.standard_normal((4, d))
    np.testing.assert_allclose(attention.decode_attention_one(q, rng.standard_normal((1, 1, d)), v[:1], 0.3)[0], v[0, 0], atol=1e-15)
    # all keys equal, or q = 0: the output is the mean of the values
    k_eq = np.repeat(rng.standard_normal((1, 1, d)), 6, axis=0)
    np.testing.assert_allclose(attention.decode_attention_one(q, k_eq, v, 0.3), np.repeat(v.mean(0), 4, 0), atol=1e-14)
    np.testing.assert_allclose(attention.decode_attention_one(np.zeros((4, d)), rng.standard_normal((6, 1, d)), v, 0.3),
                               np.repeat(v.mean(0), 4, 0), atol=1e-14)


def test_permutation_invariance_and_gqa_mapping():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((30, 2, 16))
    v = rng.standard_normal((30, 2, 16))
    o = attention.decode_attention_one(q, k, v, 0.25)
    perm = rng.permutation(30)
    np.testing.assert_allclose(attention.decode_attention_one(q, k[perm], v[perm], 0.25), o, atol=1e-13)
    # swapping the two KV heads swaps the two contiguous query groups
    o2 = attention.decode_attention_one(np.concatenate([q[4:], q[:4]]), k[:, ::-1], v[:, ::-1], 0.25)
    np.testing.assert_allclose(np.concatenate([o2[4:], o2[:4]]), o, atol=1e-13)


# ---- extend (chunked prefill) attention ----------------------------------------------------------
def _brute_extend(q, k, v, prefix_len, sm):
    c, hq, d = q.shape
    _, hkv, _ = k.shape
    g = hq // hkv
    out = np.zeros((c, hq, d))
    for i in range(c):
        for h in range(hq):
            kh = h // g
            n = prefix_len + i + 1
            z = [sm * sum(q[i, h, x] * k[t, kh, x] for x in range(d)) for t in range(n)]
            m = max(z)
            e = [math.exp(zz - m) for zz in z]
            s = sum(e)
            for x in range(d):
                out[i, h, x] = sum(e[t] * v[t, kh, x] for t in range(n)) / s
    return out


def test_extend_brute_force_tiny():
    rng = np.random.default_rng(21)
    for prefix, c, hq, hkv, d in ((0, 1, 2, 1, 4), (3, 4, 4, 2, 8), (7, 5, 6, 3, 5), (0, 6, 2, 2, 3)):
        q = rng.standard_normal((c, hq, d))
        k = rng.standard_normal((prefix + c, hkv, d)) * 3
        v = rng.standard_normal((prefix + c, hkv, d))
        sm = 1 / math.sqrt(d)
        np.testing.assert_allclose(attention.extend_attention_one(q, k, v, prefix, sm),
                                   _brute_extend(q, k, v, prefix, sm), rtol=0, atol=1e-12)


def test_extend_rows_are_decode_steps():
    """Row i equals a decode step over the first prefix + i + 1 keys (a different routine)."""
    rng = np.random.default_rng(22)
    prefix, c, hq, hkv, d = 40, 9, 8, 2, 16
    q = rng.standard_normal((c, hq, d))
    k = rng.standard_normal((prefix + c, hkv, d))
    v = rng.standard_normal((prefix + c, hkv, d))
    o = attention.extend_attention_one(q, k, v, prefix, 0.25)
    for i in range(c):
        n = prefix + i + 1
        np.testing.assert_allclose(o[i], attention.decode_attention_one(q[i], k[:n], v[:n], 0.25), atol=1e-13)


def test_extend_causal_prefill_matches_torch_sdpa():
    """prefix = 0 is ordinary causal self-attention: torch's fp64 SDPA with is_causal (a library routine)."""
    rng = np.random.default_rng(23)
    c, hq, hkv, d = 33, 8, 2, 16
    q = rng.standard_normal((c, hq, d))
    k = rng.standard_normal((c, hkv, d)) * 2
    v = rng.standard_normal((c, hkv, d))
    ours = attention.extend_attention_one(q, k, v, 0, 0.3)
    tq = torch.from_numpy(q.transpose(1, 0, 2)[None].copy())
    tk = torch.from_numpy(k.transpose(1, 0, 2)[None].copy())
    tv = torch.from_numpy(v.transpose(1, 0, 2)[None].copy())
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3, is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(ours, ref[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_extend_future_keys_do_not_leak():
    rng = np.random.default_rng(24)
    prefix, c, hq, hkv, d = 12, 7, 4, 1, 8
    q = rng.standard_normal((c, hq, d))
    k = rng.standard_normal((prefix + c, hkv, d))
    v = rng.standard_normal((prefix + c, hkv, d))
    o = attention.extend_attention_one(q, k, v, prefix, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[prefix + 3:] += 100.0
    v2[prefix + 3:] -= 50.0
    o2 = attention.extend_attention_one(q, k2, v2, prefix, 0.5)
    np.testing.assert_array_equal(o2[:3], o[:3])
    assert np.abs(o2[3:] - o[3:]).max() > 1.0
