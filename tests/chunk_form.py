"""Dense chunk-form evaluation of the KDA forward in float64 (numpy).

This is a *second, independent* statement of the method, used only to pin the
token-by-token oracle.  It follows the chunkwise forward of "Reading Notes:
Implementation Notes for KDA in FLA" (mzeromiko.github.io, kimi_linear /
kda-fla), forward steps 1-5, with the decay notation read as multiplication by
exp(+Gamma) / exp(-Gamma) of the in-chunk cumulative log decay Gamma:

  step 1  Gamma  = inclusive cumsum of the log decays inside the chunk
  step 2  Aqk    = tril((Q * e^Gamma)(K * e^-Gamma)^T)              (diagonal kept)
          Akk0   = Diag(beta) strict_tril((K * e^Gamma)(K * e^-Gamma)^T)
          A      = (I + Akk0)^-1
  step 3  U = A Diag(beta) V;   W = A (e^Gamma * Diag(beta) K)
          Qg = e^Gamma * Q;     Kg = e^(gamma_C - Gamma) * K    (gamma_C = last row)
  step 4  V_new = U - W S;      S <- Diag(e^gamma_C) S + Kg^T V_new
  step 5  O = Qg S + Aqk V_new                 (S before the step-4 update)

Here ``*`` is the row-wise (per key channel) product.  e^-Gamma overflows for
strong decay over long chunks, so this form is only evaluated on small, mildly
gated inputs.  It receives already-activated gates, normalised q/k and final
beta values: the gate and input transforms are pinned separately.
"""
from __future__ import annotations

import numpy as np


def chunk_form_sequence(q, k, v, g, beta, S0, chunk, starts_out=None):
    """One sequence, one value head.  q, k, g: [T, K]; v: [T, V]; beta: [T];
    S0: [K, V].  Returns (o [T, V], S_T [K, V]); appends the S each chunk starts
    from (the S of step 4 before its update) to starts_out when given."""
    T, K = q.shape
    V = v.shape[1]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, V))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        L = e - s
        Q, Kc, Vc, b = q[s:e], k[s:e], v[s:e], beta[s:e]
        Gam = np.cumsum(g[s:e], axis=0)                       # step 1
        Qf, Kf, Kb = Q * np.exp(Gam), Kc * np.exp(Gam), Kc * np.exp(-Gam)
        Aqk = np.tril(Qf @ Kb.T)                               # step 2
        Akk0 = b[:, None] * np.tril(Kf @ Kb.T, -1)
        A = np.linalg.inv(np.eye(L) + Akk0)
        U = A @ (b[:, None] * Vc)                              # step 3
        W = A @ (np.exp(Gam) * (b[:, None] * Kc))
        Qg = np.exp(Gam) * Q
        gC = Gam[-1]
        Kg = np.exp(gC[None, :] - Gam) * Kc
        if starts_out is not None:
            starts_out.append(S.copy())
        Vn = U - W @ S                                         # step 4
        o[s:e] = Qg @ S + Aqk @ Vn                             # step 5 (old S)
        S = np.exp(gC)[:, None] * S + Kg.T @ Vn
    return o, S


def chunk_form(q, k, v, g, beta, S0, chunk, seq_starts, hv_to_h):
    """Several sequences and heads.  q, k: [Ttot, H, K]; v: [Ttot, HV, V];
    g: [Ttot, HV, K]; beta: [Ttot, HV]; S0: [N, HV, K, V] (or None)."""
    Ttot, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    N = len(seq_starts) - 1
    o = np.zeros((Ttot, HV, V))
    ht = np.zeros((N, HV, K, V))
    for n in range(N):
        a, b_ = seq_starts[n], seq_starts[n + 1]
        for hv in range(HV):
            h = hv_to_h(hv)
            s0 = np.zeros((K, V)) if S0 is None else S0[n, hv]
            if b_ == a:
                ht[n, hv] = s0
                continue
            o[a:b_, hv], ht[n, hv] = chunk_form_sequence(
                q[a:b_, h], k[a:b_, h], v[a:b_, hv], g[a:b_, hv], beta[a:b_, hv], s0, chunk)
    return o, ht
