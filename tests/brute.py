"""Brute-force numpy attention for tiny inputs (test-only pin of the oracle).

Full score matrix per sequence in matrix form, an explicit -inf mask above the
causal diagonal, np.exp, row normalisation.  Independent of oracle.c: it reads
the logical dense K/V rows, not the pool.
"""
import numpy as np

from workloads import bf16_bits_to_f32


def brute_attend(q_bits, k_dense_bits, v_dense_bits, seq_lens, qsl, scale):
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    kd = bf16_bits_to_f32(k_dense_bits).astype(np.float64)
    vd = bf16_bits_to_f32(v_dense_bits).astype(np.float64)
    T, Hq, D = q.shape
    Hkv = kd.shape[1]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    start = 0
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        t0, t1 = int(qsl[b]), int(qsl[b + 1])
        Q = t1 - t0
        Kb = kd[start:start + L]          # [L][Hkv][D]
        Vb = vd[start:start + L]
        start += L
        if Q == 0:
            continue
        rows = np.arange(Q)[:, None] + (L - Q)
        cols = np.arange(L)[None, :]
        mask = cols > rows                 # keys after the query's position
        for h in range(Hq):
            S = np.float64(np.float32(scale)) * (q[t0:t1, h, :] @ Kb[:, h // G, :].T)
            S[mask] = -np.inf
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P /= P.sum(axis=1, keepdims=True)
            out[t0:t1, h, :] = P @ Vb[:, h // G, :]
    return out
