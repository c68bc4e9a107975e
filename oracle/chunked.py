"""Chunkwise form of the KDA recurrence in fp64 -- TEST INFRASTRUCTURE ONLY.

This module exists to pin the token-by-token oracle (``oracle.recurrent``) by
brute force on tiny inputs: two independently written forms of the same
function must agree to rounding.  It is not used to check the GPU path.

The pages only state the idea: [Walkthrough] 彩蛋 -- groups of tokens pass the
state between groups while the work inside a group becomes matrix products,
with causality kept; [K3-memory] "KDA 谱系速查" -- the delta update rewritten in Householder
form (key-first layout here: S_t = (I - beta k k^T) diag(alpha_t) S_{t-1} + beta k v^T)
so that the steps can run chunk-parallel; [Replication-2] figure 1 -- state transitions compose affinely
into one chunk-level transform.  The algebra below is derived from the
recurrence, not copied from any listing.

Derivation (key-first state S in R^{DK x DV}, one chunk of n tokens entered
with state S0).  Let G_t = sum_{j<=t} g_j (per key channel) and D(t,i) =
exp(G_t - G_i).  Induction on t shows
    S_t = diag(exp G_t) S0 + sum_{i<=t} (k_i * D(t,i)) u_i^T
for pseudo-values u_i.  The corrective write gives
    u_t = beta_t (v_t - [decayed S_{t-1}]^T k_t)
        = beta_t (v_t - S0^T (k_t * exp G_t) - sum_{i<t} A_ti u_i),
    A_ti = sum_c k_tc k_ic D(t,i)_c.
Hence (I + diag(beta) A) U = diag(beta) (V - (K * exp G) S0), i.e.
    U = T diag(beta) V - T diag(beta) (K * exp G) S0,   T = (I + diag(beta) A)^{-1}
and the read-out after the write and the chunk's final state are
    O   = scale [ (Q * exp G) S0 + P U ],   P_ti = sum_c q_tc k_ic D(t,i)_c  (i <= t)
    S_n = diag(exp G_n) S0 + (K * exp(G_n - G))^T U.
Differences of G are exponentiated directly (never exp(-G) alone).
"""
from __future__ import annotations

import numpy as np


def chunk_step(q, k, v, g, beta, S0, scale):
    """One chunk. q,k,g: [n,DK]; v: [n,DV]; beta: [n]; S0: [DK,DV]. Returns (O, S_n)."""
    n = q.shape[0]
    G = np.cumsum(g, axis=0)                               # [n, DK]
    D = np.exp(G[:, None, :] - G[None, :, :])              # [t, i, DK]: exp(G_t - G_i)
    lower_strict = np.tril(np.ones((n, n)), -1)
    lower_incl = np.tril(np.ones((n, n)), 0)
    # The (t, i) entries with i > t are masked; their exponent can be positive, so
    # zero the argument first to keep the arrays finite.
    D = np.where(lower_incl[:, :, None] > 0, D, 0.0)
    A = np.einsum("tc,ic,tic->ti", k, k, D) * lower_strict
    P = np.einsum("tc,ic,tic->ti", q, k, D) * lower_incl
    T = np.linalg.inv(np.eye(n) + beta[:, None] * A)
    Ku = k * np.exp(G)                                     # K * exp(G_t)
    U = T @ (beta[:, None] * v) - T @ (beta[:, None] * Ku) @ S0
    O = scale * ((q * np.exp(G)) @ S0 + P @ U)
    Gn = G[-1]
    Sn = np.exp(Gn)[:, None] * S0 + (k * np.exp(Gn[None, :] - G)).T @ U
    return O, Sn


def chunked_forward(q, k, v, g, beta, cu_seqlens=None, scale=1.0, h0=None, chunk=64):
    """Chunkwise KDA forward over packed sequences (chunks restart at each sequence).

    q, k, g: [T, H, DK]; v: [T, H, DV]; beta: [T, H]; h0: [N, H, DK, DV] or None.
    The last chunk of a sequence may be shorter than ``chunk``.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    T, H, DK = q.shape
    DV = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    o = np.zeros((T, H, DV))
    hT = np.zeros((N, H, DK, DV))
    for n in range(N):
        for h in range(H):
            S = np.zeros((DK, DV)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            for s in range(int(cu[n]), int(cu[n + 1]), chunk):
                e = min(s + chunk, int(cu[n + 1]))
                O, S = chunk_step(q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h], beta[s:e, h], S,
                                  scale)
                o[s:e, h] = O
            hT[n, h] = S
    return o, hT
