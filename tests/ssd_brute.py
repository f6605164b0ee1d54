"""Independent float64 checkers used to pin the oracle (test helpers, numpy only).

`semiseparable` materialises the SSD map as a matrix, per (sequence, head):
    M[i, j] = (C_i . B_j) * exp(sum_{k=j+1..i} a_k) * delta_j   for j <= i
    y       = M x + exp(sum_{k=start..i} a_k) * (C_i . h0) + D x
    h_final = exp(sum_all a) h0 + sum_j exp(sum_{k=j+1..end} a_k) delta_j x_j B_j^T
with delta = softplus(dt + dt_bias) and a = delta * A.  This is the
"semiseparable matrix" view of the selective state-space layer (a quadratic,
attention-like form of the same linear recurrence), written independently of
the oracle's token loop: no shared code, and softplus here is numpy's
logaddexp(0, u) rather than log1p(exp(u)).

`chunked` is the chunked decomposition the scan kernels implement (chunk-local
cumulative decay, C.B^T with the segment-sum mask, per-chunk states, state
passing between chunks, inter-chunk output term), in float64.  It must equal
the recurrence to rounding at every chunk size, which pins the decomposition
against the recurrence.
"""
import numpy as np


def _softplus(u):
    return np.where(u > 20.0, u, np.logaddexp(0.0, u))


def _prep(x, dt, dt_bias, A, B, C, D, cu):
    x, dt, B, C = (np.asarray(v, np.float64) for v in (x, dt, B, C))
    H = x.shape[1]
    dt_bias = np.zeros(H) if dt_bias is None else np.asarray(dt_bias, np.float64)
    D = np.zeros(H) if D is None else np.asarray(D, np.float64)
    A = np.asarray(A, np.float64)
    cu = np.asarray(cu, np.int64)
    delta = _softplus(dt + dt_bias[None, :])
    return x, B, C, D, A, cu, delta


def semiseparable(x, dt, dt_bias, A, B, C, D, cu, init=None, has_init=None):
    x, B, C, D, A, cu, delta = _prep(x, dt, dt_bias, A, B, C, D, cu)
    T, H, P = x.shape
    G, N = B.shape[1:]
    S = len(cu) - 1
    y = np.zeros((T, H, P))
    final = np.zeros((S, H, P, N))
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        L = t1 - t0
        for h in range(H):
            g = h // (H // G)
            a = delta[t0:t1, h] * A[h]
            cum = np.concatenate([[0.0], np.cumsum(a)])          # cum[i+1] = sum_{k<=i} a_k
            h0 = np.zeros((P, N))
            if init is not None and (has_init is None or has_init[s]):
                h0 = np.asarray(init[s, h], np.float64)
            Cs, Bs = C[t0:t1, g], B[t0:t1, g]
            if L:
                seg = cum[1:, None] - cum[None, 1:]               # sum_{k=j+1..i} a_k
                mask = np.tril(np.ones((L, L), bool))
                Lmat = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
                M = (Cs @ Bs.T) * Lmat * delta[t0:t1, h][None, :]
                xs = x[t0:t1, h]
                y[t0:t1, h] = M @ xs + np.exp(cum[1:])[:, None] * (Cs @ h0.T) + D[h] * xs
                wdec = np.exp(cum[-1] - cum[1:]) * delta[t0:t1, h]
                final[s, h] = np.exp(cum[-1]) * h0 + (xs * wdec[:, None]).T @ Bs
            else:
                final[s, h] = h0
    return y, final


def chunked(x, dt, dt_bias, A, B, C, D, cu, chunk_size, init=None, has_init=None):
    """float64 chunked SSD: returns (y, final, chunk_states after each chunk)."""
    x, B, C, D, A, cu, delta = _prep(x, dt, dt_bias, A, B, C, D, cu)
    T, H, P = x.shape
    G, N = B.shape[1:]
    S = len(cu) - 1
    y = np.zeros((T, H, P))
    final = np.zeros((S, H, P, N))
    states = []
    for s in range(S):
        t0, t1 = cu[s], cu[s + 1]
        hst = np.zeros((H, P, N))
        if init is not None and (has_init is None or has_init[s]):
            hst = np.asarray(init[s], np.float64).copy()
        for c0 in range(t0, t1, chunk_size):
            c1 = min(c0 + chunk_size, t1)
            Lc = c1 - c0
            out = np.zeros((H, P, N))
            for h in range(H):
                g = h // (H // G)
                dA = delta[c0:c1, h] * A[h]
                dA_cs = np.cumsum(dA)                              # inclusive, chunk-local
                seg = dA_cs[:, None] - dA_cs[None, :]
                mask = np.tril(np.ones((Lc, Lc), bool))
                Lmat = np.where(mask, np.exp(np.where(mask, seg, 0.0)), 0.0)
                CB = C[c0:c1, g] @ B[c0:c1, g].T
                xdt = x[c0:c1, h] * delta[c0:c1, h][:, None]
                y_intra = (CB * Lmat) @ xdt
                y_inter = np.exp(dA_cs)[:, None] * (C[c0:c1, g] @ hst[h].T)
                y[c0:c1, h] = y_intra + y_inter + D[h] * x[c0:c1, h]
                chunk_state = (xdt * np.exp(dA_cs[-1] - dA_cs)[:, None]).T @ B[c0:c1, g]
                out[h] = np.exp(dA_cs[-1]) * hst[h] + chunk_state
            hst = out
            states.append(hst.copy())
        final[s] = hst
    cs = np.stack(states) if states else np.zeros((0, H, P, N))
    return y, final, cs


def gdn_chunked(q, k, v, gate, beta, cu, scale, h0, chunk):
    """Independent float64 chunked (WY) form of the gated delta rule, per sequence
    and value head: within a chunk with entering state H0 and inclusive log-gate
    cumsum G (gamma = e^G),
        (I + A) U = diag(beta) V - diag(beta gamma) K H0,  A_ij = beta_i e^(G_i - G_j) k_i.k_j (j < i)
        O = scale (diag(gamma) Q H0 + (e^(G_i - G_j) q_i.k_j)_{j <= i} U)
        H_next = gamma_last H0 + K^T diag(e^(G_last - G)) U
    (H0 here is key-major, dk x dv; states in and out are value-major like the
    oracle's, dv x dk.) Returns (o, final_states, chunk_states) like the oracle."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    gate, beta = np.asarray(gate, np.float64), np.asarray(beta, np.float64)
    T, G, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    S = len(cu) - 1
    o = np.zeros((T, H, dv))
    fin = np.zeros((S, H, dv, dk))
    cst = []
    for s in range(S):
        a0, a1 = int(cu[s]), int(cu[s + 1])
        per = []
        for h in range(H):
            g = h // (H // G)
            Hs = np.array(h0[s, h], np.float64).T if h0 is not None else np.zeros((dk, dv))
            states = []
            for c0 in range(a0, a1, chunk):
                c1 = min(c0 + chunk, a1)
                K, Q, V = k[c0:c1, g], q[c0:c1, g], v[c0:c1, h]
                Gc = np.cumsum(gate[c0:c1, h])
                bt = beta[c0:c1, h]
                gam = np.exp(Gc)
                D = np.exp(Gc[:, None] - Gc[None, :])
                n = c1 - c0
                A = np.tril(bt[:, None] * D * (K @ K.T), -1)
                U = np.linalg.solve(np.eye(n) + A, bt[:, None] * V - (bt * gam)[:, None] * (K @ Hs))
                Mq = np.tril(D * (Q @ K.T))
                o[c0:c1, h] = scale * (gam[:, None] * (Q @ Hs) + Mq @ U)
                Hs = gam[-1] * Hs + K.T @ (np.exp(Gc[-1] - Gc)[:, None] * U)
                states.append(Hs.T.copy())
            fin[s, h] = Hs.T
            per.append(states)
        for c in range(len(per[0]) if per else 0):
            cst.append(np.stack([per[h][c] for h in range(H)]))
    return o, fin, (np.stack(cst) if cst else np.zeros((0, H, dv, dk)))
