"""fp64 decode and extend attention on the dequantized cache (oracle, test infrastructure).

The decode path of the SGLang x Qwen x NVIDIA story ("Three Paths" paragraph 3)
reads the NVFP4 cache, dequantizes on the fly and runs ordinary attention; the
result it aims at is therefore exactly softmax attention over the dequantized
K/V.  This module is that definition, in fp64:

    z_t = sm_scale * <q, K_hat_t>,  p = softmax(z),  o = sum_t p_t V_hat_t

over the sequence's tokens.  Reading R10: query head hq uses KV head
hq // (H_q / H_kv) (contiguous GQA groups).  The maximum is subtracted before
the exponential (it cancels exactly in the ratio).  Matrix products use numpy's
fp64 routines.
"""

from __future__ import annotations

import numpy as np


def decode_attention_one(q, k_hat, v_hat, sm_scale) -> np.ndarray:
    """One sequence: q [H_q][D], k_hat/v_hat [L][H_kv][D] (fp64) -> out [H_q][D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    h_q, d = q.shape
    length, h_kv, _ = k_hat.shape
    if length < 1:
        raise ValueError("a decode step needs at least one cached token")
    if h_q % h_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    group = h_q // h_kv
    out = np.empty((h_q, d), dtype=np.float64)
    for hk in range(h_kv):
        qg = q[hk * group:(hk + 1) * group]               # [G][D]
        z = float(sm_scale) * (qg @ k_hat[:, hk, :].T)      # [G][L]
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        out[hk * group:(hk + 1) * group] = p @ v_hat[:, hk, :]
    return out


def decode_attention(q, k_hat_seqs, v_hat_seqs, sm_scale) -> np.ndarray:
    """Batch: q [B][H_q][D]; k_hat_seqs[b], v_hat_seqs[b] are [L_b][H_kv][D] -> out [B][H_q][D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    return np.stack([decode_attention_one(q[b], k_hat_seqs[b], v_hat_seqs[b], sm_scale)
                     for b in range(q.shape[0])])


def extend_attention_one(q, k_hat, v_hat, prefix_len: int, sm_scale) -> np.ndarray:
    """Chunked extend of one sequence: the chunk's queries attend over prefix || chunk, causally.

    SGLang x Qwen x NVIDIA story, "Three Paths" paragraph 2 (extend gathers the cached prefix into
    an FP8 workspace and attends over it together with the new chunk) and summary bullet 2 (the
    prefill-side attention takes BF16 Q against FP8 KV).  The chunk's token i sits at position
    prefix_len + i and sees keys 0 .. prefix_len + i (ordinary causal attention over the whole
    sequence, restricted to the chunk's rows).

    q [C][H_q][D]; k_hat, v_hat [prefix_len + C][H_kv][D] (fp64, the dequantized workspace rows)
    -> out [C][H_q][D] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    c, h_q, d = q.shape
    total, h_kv, _ = k_hat.shape
    if total != prefix_len + c or prefix_len < 0:
        raise ValueError("k_hat / v_hat must hold prefix_len + C rows")
    if h_q % h_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    group = h_q // h_kv
    # key j is visible to chunk row i iff j <= prefix_len + i
    visible = np.arange(total)[None, :] <= (prefix_len + np.arange(c))[:, None]      # [C][T]
    out = np.empty((c, h_q, d), dtype=np.float64)
    for hq in range(h_q):
        hk = hq // group
        z = float(sm_scale) * (q[:, hq, :] @ k_hat[:, hk, :].T)                       # [C][T]
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, hq, :] = p @ v_hat[:, hk, :]
    return out
