"""fp64 decode attention on the dequantized cache (oracle, test infrastructure).

The decode path of the SGLang x Qwen x NVIDIA story ("Three Paths" paragraph 3)
reads the NVFP4 cache, dequantizes on the fly and runs ordinary attention; the
result it aims at is therefore exactly softmax attention over the dequantized
K/V.  This module is that definition, in fp64:

    z_t = sm_scale * <q, K_hat_t>,  p = softmax(z),  o = sum_t p_t V_hat_t

over the sequence's tokens.  Reading R11: query head hq uses KV head
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
