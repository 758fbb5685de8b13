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
