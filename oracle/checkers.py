"""Independent fp64 re-derivations of the gated delta rule, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (imported by tests, never by the product path).
Neither routine calls the token-by-token loop in gdn_oracle; they rest on
different algebra, so a mistake in one is not repeated in the other.

* ``closed_form``: the state after t tokens written as an explicit product of
  per-token transition matrices.  From S_t = M_t S_{t-1} + beta_t k_t v_t^T with
  M_t = exp(g_t) (I - beta_t k_t k_t^T):
      S_t = Phi(1..t) S_0 + sum_{j<=t} Phi(j+1..t) beta_j k_j v_j^T,
      Phi(a..b) = M_b M_{b-1} ... M_a   (identity for an empty range),
  and o_t = S_t^T q_t * scale.  Cost O(T^2 d^3): tiny inputs only.

* ``chunked_ut``: the chunked form (the one the pages call "chunked" and
  state to be algebraically identical to the recurrent one -- KerasFormers Qwen
  page, "Verified parity").  Inside a chunk with in-chunk cumulative log-decay
  gamma_i = g_1 + ... + g_i and start state S:
      A_ij = beta_i exp(gamma_i - gamma_j) (k_i . k_j)   for j < i, else 0
      T    = (I + A)^{-1}
      W    = T diag(beta exp(gamma)) K,   U' = T diag(beta) V,   U = U' - W S
      O    = scale (diag(exp(gamma)) Q S + tril(Q K^T * D) U),  D_ij = exp(gamma_i - gamma_j)
      S'   = exp(gamma_L) S + (diag(exp(gamma_L - gamma)) K)^T U
  Derivation: with u_i = beta_i (v_i - exp(g_i) S_{i-1}^T k_i) the recurrence
  is S_i = exp(g_i) S_{i-1} + k_i u_i^T, so S_i = exp(gamma_i) S + sum_{j<=i}
  exp(gamma_i - gamma_j) k_j u_j^T; substituting into u_i gives (I + A) U =
  diag(beta) V - diag(beta exp(gamma)) K S.
"""
from __future__ import annotations

import numpy as np


def closed_form(q, k, v, g, beta, S0, scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    eye = np.eye(dk)
    M = [np.exp(g[t]) * (eye - beta[t] * np.outer(k[t], k[t])) for t in range(L)]

    def phi(a, b):   # product M_b ... M_a over token indices a..b inclusive
        P = eye.copy()
        for s in range(a, b + 1):
            P = M[s] @ P
        return P

    o = np.zeros((L, dv))
    S_t = None
    for t in range(L):
        S_t = phi(0, t) @ S0
        for j in range(t + 1):
            S_t = S_t + phi(j + 1, t) @ (beta[j] * np.outer(k[j], v[j]))
        o[t] = scale * (S_t.T @ q[t])
    if S_t is None:
        S_t = np.array(S0, dtype=np.float64)
    return o, S_t


def chunked_ut(q, k, v, g, beta, S0, scale, chunk=64):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    L = k.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        Q, K, V = q[c0:c1], k[c0:c1], v[c0:c1]
        bt = beta[c0:c1]
        gam = np.cumsum(g[c0:c1])
        n = c1 - c0
        lower = np.tril(np.ones((n, n), dtype=bool))
        diff = np.where(lower, gam[:, None] - gam[None, :], -np.inf)   # mask before exp
        D = np.exp(diff)
        A = np.tril(bt[:, None] * (K @ K.T) * D, -1)
        T = np.linalg.inv(np.eye(n) + A)
        W = T @ ((bt * np.exp(gam))[:, None] * K)
        Up = T @ (bt[:, None] * V)
        U = Up - W @ S
        o[c0:c1] = scale * (np.exp(gam)[:, None] * (Q @ S) + ((Q @ K.T) * D) @ U)
        S = np.exp(gam[-1]) * S + (np.exp(gam[-1] - gam)[:, None] * K).T @ U
    return o, S
