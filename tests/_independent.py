"""Independent formulations used only to pin the sequential oracle.

Neither function shares code with ``oracle/`` or with the HIP path; each is a
different way of writing the same Mamba-2 selective state-space map (the
method listed under "References" on page "Mamb2_8B_FP4_Recall_SQ3.25":
Dao and Gu 2024, structured state-space duality).

* ``dual_form_mp`` materialises the unrolled sum in multiprecision:
      y_t = sum_{s<=t} (C_t . B_s) exp(A (cs_t - cs_s)) dt_s x_s
            + exp(A cs_t) C_t . h0 + D x_t,     cs = inclusive cumsum of dt.
* ``chunked_fp64`` is the block (chunked) decomposition that the GPU path
  uses: a decay-masked C.B^T product inside each chunk, a per-chunk state,
  a chunk-to-chunk state recurrence and an off-diagonal readout.
"""
from __future__ import annotations

import mpmath
import numpy as np


def dual_form_mp(x, dt, A, Bm, Cm, D, h0=None, dps=50):
    """Tiny inputs only (loops in mpmath).  Shapes as the oracle, batch 1 folded:
    x (L,H,P), dt (L,H), Bm, Cm (L,G,N), h0 (H,P,N).  Returns y (L,H,P) as
    float64 and the final state (H,P,N)."""
    mpmath.mp.dps = dps
    L, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    hpg = H // G
    mp = mpmath.mpf
    y = np.zeros((L, H, P))
    hT = np.zeros((H, P, N))
    for h in range(H):
        g = h // hpg
        a = mp(float(A[h]))
        cs = []
        acc = mp(0)
        for t in range(L):
            acc += mp(float(dt[t, h]))
            cs.append(acc)
        for t in range(L):
            for p in range(P):
                tot = mp(0)
                for s in range(t + 1):
                    cb = mpmath.fsum(mp(float(Cm[t, g, n])) * mp(float(Bm[s, g, n])) for n in range(N))
                    tot += cb * mpmath.exp(a * (cs[t] - cs[s])) * mp(float(dt[s, h])) * mp(float(x[s, h, p]))
                if h0 is not None:
                    tot += mpmath.exp(a * cs[t]) * mpmath.fsum(
                        mp(float(Cm[t, g, n])) * mp(float(h0[h, p, n])) for n in range(N))
                tot += mp(float(D[h])) * mp(float(x[t, h, p]))
                y[t, h, p] = float(tot)
        # final state: h_T = exp(A cs_T) h0 + sum_s exp(A (cs_T - cs_s)) dt_s x_s B_s^T
        for p in range(P):
            for n in range(N):
                tot = mp(0)
                for s in range(L):
                    tot += mpmath.exp(a * (cs[L - 1] - cs[s])) * mp(float(dt[s, h])) * \
                        mp(float(x[s, h, p])) * mp(float(Bm[s, g, n]))
                if h0 is not None:
                    tot += mpmath.exp(a * cs[L - 1]) * mp(float(h0[h, p, n]))
                hT[h, p, n] = float(tot)
    return y, hT


def chunked_fp64(x, dt, A, Bm, Cm, D, Q, h0=None):
    """Block decomposition in fp64 with chunk length Q (the last chunk may be
    shorter).  Shapes: x (L,H,P), dt (L,H), Bm, Cm (L,G,N), h0 (H,P,N)."""
    x, dt, Bm, Cm = (np.asarray(a, np.float64) for a in (x, dt, Bm, Cm))
    A = np.asarray(A, np.float64)
    D = np.asarray(D, np.float64)
    L, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    hpg = H // G
    y = np.zeros((L, H, P))
    state = np.zeros((H, P, N)) if h0 is None else np.array(h0, np.float64)
    for c0 in range(0, L, Q):
        c1 = min(L, c0 + Q)
        for h in range(H):
            g = h // hpg
            la = dt[c0:c1, h] * A[h]                       # log decay per token (<= 0)
            cs = np.cumsum(la)                             # inclusive, from the chunk start
            diff = cs[:, None] - cs[None, :]
            mask = np.tril(np.ones((c1 - c0, c1 - c0), bool))
            decay = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
            cb = Cm[c0:c1, g] @ Bm[c0:c1, g].T              # (t, s)
            xdt = x[c0:c1, h] * dt[c0:c1, h][:, None]      # (s, p)
            y_diag = (cb * decay) @ xdt
            y_off = np.exp(cs)[:, None] * (Cm[c0:c1, g] @ state[h].T)
            y[c0:c1, h] = y_diag + y_off + D[h] * x[c0:c1, h]
            w = np.exp(cs[-1] - cs)                        # decay to the chunk end
            chunk_state = (xdt * w[:, None]).T @ Bm[c0:c1, g]   # (p, n)
            state[h] = np.exp(cs[-1]) * state[h] + chunk_state
    return y, state
