"""Independent fp64 formulations of the selective scan, used to pin the oracle.

None of this shares code with ``oracle/ssd_oracle.c``: it is written from the
mathematics in numpy/scipy, in forms other than the token recurrence.

* ``ssd_quadratic``: the "state space duality" form, in which the whole scan
  is one lower-triangular matrix M applied to x ("Hybrid Architectures for
  Language Models" summary, section 2 Background: SSD recasts the state-space
  computation as matrix multiplies; Appendix O draws |M| as Mamba's implicit
  attention).  Unrolling h_t = a_t h_{t-1} + delta_t x_t B_t^T gives
      y_t = sum_{s<=t} (C_t . B_s) * prod_{r=s+1..t} a_r * delta_s * x_s
            + (prod_{r<=t} a_r) * h0 C_t + D x_t.
  The products of decays are evaluated as exp of explicit sums.
* ``ssd_chunked``: the same result computed chunk by chunk (intra-chunk
  matrix product, per-chunk state, state passed between chunks), for any
  chunk length including ragged tails.
* ``conv_correlate``: the causal depthwise conv written with numpy's
  ``np.correlate`` on a left-padded series.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def softplus(v):
    return np.logaddexp(0.0, v)


def silu(u):
    return u * expit(u)


def _delta(dt, dt_bias, dt_softplus):
    v = np.asarray(dt, np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, np.float64)
    return softplus(v) if dt_softplus else v


def ssd_quadratic(x, Bm, Cm, dt, A, *, D=None, z=None, dt_bias=None, dt_softplus=True,
                  h0=None):
    """x [B,L,H,P], Bm/Cm [B,L,G,N], dt [B,L,H] -> y [B,L,H,P] (float64).
    O(L^3) in the decay sums: tiny inputs only."""
    x = np.asarray(x, np.float64)
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    delta = _delta(dt, dt_bias, dt_softplus)
    y = np.zeros((Bt, L, H, P))
    for b in range(Bt):
        for h in range(H):
            g = (h * G) // H
            la = delta[b, :, h] * float(A[h])          # log of each token's decay
            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    decay = np.exp(la[s + 1:t + 1].sum())
                    M[t, s] = Cm[b, t, g] @ Bm[b, s, g] * decay * delta[b, s, h]
            yy = M @ x[b, :, h, :]
            if h0 is not None:
                for t in range(L):
                    yy[t] += np.exp(la[:t + 1].sum()) * (np.asarray(h0[b, h], np.float64) @ Cm[b, t, g])
            if D is not None:
                yy += float(D[h]) * x[b, :, h, :]
            if z is not None:
                yy *= silu(np.asarray(z[b, :, h, :], np.float64))
            y[b, :, h, :] = yy
    return y


def ssd_chunked(x, Bm, Cm, dt, A, chunk, *, D=None, z=None, dt_bias=None, dt_softplus=True,
                h0=None):
    """Chunk-by-chunk fp64 form; returns (y [B,L,H,P], h_final [B,H,P,N])."""
    x = np.asarray(x, np.float64)
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    delta = _delta(dt, dt_bias, dt_softplus)
    y = np.zeros((Bt, L, H, P))
    hT = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = (h * G) // H
            state = np.zeros((P, N)) if h0 is None else np.array(h0[b, h], np.float64)
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                xc, Bc, Cc = x[b, c0:c1, h], Bm[b, c0:c1, g], Cm[b, c0:c1, g]
                dc = delta[b, c0:c1, h]
                lam = np.cumsum(dc * float(A[h]))         # cumulative log decay in the chunk
                q = c1 - c0
                tri = np.tril(np.ones((q, q), bool))
                seg = np.where(tri, lam[:, None] - lam[None, :], -np.inf)
                Mc = (Cc @ Bc.T) * np.exp(seg) * dc[None, :]
                yc = Mc @ xc + np.exp(lam)[:, None] * (Cc @ state.T)
                w = np.exp(lam[-1] - lam) * dc
                state = np.exp(lam[-1]) * state + (xc * w[:, None]).T @ Bc
                if D is not None:
                    yc = yc + float(D[h]) * xc
                y[b, c0:c1, h] = yc
            hT[b, h] = state
            if z is not None:
                y[b, :, h] *= silu(np.asarray(z[b, :, h], np.float64))
    return y, hT


def conv_correlate(xbc, w, bias=None, hist=None, apply_silu=True):
    """xbc [B,L,C], w [C,K], hist [B,K-1,C] or None -> [B,L,C] float64."""
    xbc = np.asarray(xbc, np.float64)
    Bt, L, C = xbc.shape
    K = w.shape[1]
    out = np.zeros((Bt, L, C))
    for b in range(Bt):
        for c in range(C):
            pad = np.zeros(K - 1) if hist is None else np.asarray(hist[b, :, c], np.float64)
            series = np.concatenate([pad, xbc[b, :, c]])
            u = np.correlate(series, np.asarray(w[c], np.float64), mode="valid")
            if bias is not None:
                u = u + float(bias[c])
            out[b, :, c] = silu(u) if apply_silu else u
    return out


def pack_xbc(x, Bm, Cm):
    """[B,L,H,P], [B,L,G,N], [B,L,G,N] -> the x|B|C channel layout [B,L,Cdim]."""
    Bt, L = x.shape[:2]
    return np.concatenate([x.reshape(Bt, L, -1), Bm.reshape(Bt, L, -1),
                           Cm.reshape(Bt, L, -1)], axis=2)
