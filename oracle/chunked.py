"""Chunkwise schedule of the KDA recurrence, float64 numpy.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see ``oracle/__init__.py``).  It exists
to pin the token-by-token oracle with a second, independently written
schedule: the two must agree to float64 rounding for every chunk size,
including sizes that do not divide T and C = T.

Chunk form (derived from the recurrence; the skeleton -- intra-chunk parallel
part plus an inter-chunk state hand-off, with the cumulative decay folded into
the incoming state and the intra-chunk mask -- is the one of the
"Linear/sparse attention tutorial" page, sect. 6.2; the lower-triangular
system that corrects each token's provisional error is the chunk mode of the
"KDA derivation summary" page, sect. 6; the compact WY form is sect. 5.3 of the
tutorial page).  For one chunk of c tokens with incoming state S (dv x dk) and
per-channel cumulative log-decay G_r = sum_{s<=r} log_alpha_s:

    A_rj = beta_r sum_c k_rc k_jc exp(G_rc - G_jc)       j <  r   (else 0)
    P_rj =        sum_c q_rc k_jc exp(G_rc - G_jc)       j <= r   (else 0)
    R    = Diag(beta) (V - (K*exp(G)) S^T)                provisional errors
    (I + A) E = R                                        corrected errors
    O    = (Q*exp(G)) S^T + P E
    S   <- S Diag(exp(G_last)) + E^T (K*exp(G_last - G))

WY variant: T = (I + A)^{-1} Diag(beta), W = T (K*exp(G)), U = T V,
E = U - W S^T.  In the additive write mode A = 0 and R = Diag(beta) V.

The pairwise decays exp(G_rc - G_jc) are formed directly (a c x c x dk array),
so nothing here can overflow for any decay.
"""
from __future__ import annotations

import numpy as np


def _forward_substitution(L_strict, R):
    """Solve (I + L_strict) E = R for unit lower-triangular I + L_strict."""
    c = R.shape[0]
    E = np.zeros_like(R)
    for r in range(c):
        E[r] = R[r] - L_strict[r, :r] @ E[:r]
    return E


def chunk_forward_head(q, k, v, log_alpha, beta, S0, C, write="delta", variant="direct"):
    """One head.  q, k, log_alpha [T, dk]; v [T, dv]; beta [T]; S0 [dv, dk].

    Returns ``(out [T, dv], S_final [dv, dk])``.
    """
    T, dk = q.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64, copy=True)
    out = np.zeros((T, dv), dtype=np.float64)
    for s in range(0, T, C):
        e = min(s + C, T)
        c = e - s
        Q, K, V = q[s:e], k[s:e], v[s:e]
        b = beta[s:e]
        G = np.cumsum(log_alpha[s:e], axis=0)                       # [c, dk]
        decay = np.exp(G[:, None, :] - G[None, :, :])                # [r, j, dk], r >= j used
        strict = np.tril(np.ones((c, c)), -1)
        incl = np.tril(np.ones((c, c)), 0)
        P = np.einsum("rc,jc,rjc->rj", Q, K, decay * incl[:, :, None])
        Kbar = K * np.exp(G)
        Qbar = Q * np.exp(G)
        Ktil = K * np.exp(G[-1][None, :] - G)
        if write == "add":
            E = b[:, None] * V
        elif write == "delta":
            A = b[:, None] * np.einsum("rc,jc,rjc->rj", K, K, decay * strict[:, :, None])
            if variant == "direct":
                R = b[:, None] * (V - Kbar @ S.T)
                E = _forward_substitution(A, R)
            elif variant == "wy":
                Tm = np.linalg.solve(np.eye(c) + A, np.diag(b))
                W = Tm @ Kbar
                U = Tm @ V
                E = U - W @ S.T
            else:
                raise ValueError(variant)
        else:
            raise ValueError(write)
        out[s:e] = Qbar @ S.T + P @ E
        S = S * np.exp(G[-1])[None, :] + E.T @ Ktil
    return out, S


def chunk_forward(q, k, v, log_alpha, beta, S0=None, C=16, write="delta", variant="direct"):
    """Batch version over token-major [B, T, H, d] arrays (float64)."""
    q, k, v, la, be = (np.asarray(x, dtype=np.float64) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((dv, dk)) if S0 is None else S0[b, h]
            o, s = chunk_forward_head(q[b, :, h], k[b, :, h], v[b, :, h], la[b, :, h],
                                      be[b, :, h], s0, C, write=write, variant=variant)
            out[b, :, h] = o
            Sf[b, h] = s
    return out, Sf
