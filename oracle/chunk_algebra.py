"""Oracle O2: the chunked three-part form of the SDM forward, in fp64, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

This is the chunk algebra the pages describe (module docstring of memory_ops.py and
of phase2_kernels.py, sparse-delta-memory 2.0.0 wheel, diffend pages 21 and 23),
written out with explicit loops and no blocking or fusion:

  Phase 1, per chunk (independent of the bank):
    L[i, w]   cumulative log-decay of write entry (i, w): the sum of the gates of all
              writes to the same slot at chunk tokens <= i
    Lr[i, r]  the same sum for the slot read by entry (i, r) (0 if unwritten so far)
    is_only   write entries whose slot occurs once among the chunk's writes
    gw, gr    gather weights k * exp(L), q * exp(Lr)
    A[i, j]   j < i: sum over write pairs (i, w), (j, w') on one slot of
              k[i,w] k[j,w'] exp(L[i,w] - L[j,w'])
    QK[i, j]  j <= i: sum over (read (i, r), write (j, w')) pairs on one slot of
              q[i,r] k[j,w'] exp(Lr[i,r] - L[j,w'])
  Solve (wy_solve.py docstring): X = (I + tril(beta * A, -1))^-1, QX = QK @ X
  Phase 2, per chunk in order (phase2_kernels.py docstring and _sdm_dual_matmul):
    gather       retrieved[i] = sum_w gw[i,w] B0[s], inter[i] = sum_r gr[i,r] B0[q]
    dual matmul  u = beta (v - retrieved); delta_v = X u; readings = QX u + inter
    DW           every written slot s: B[s] = exp(Llast_s) B0[s]
                                              + sum over its writes k exp(Llast_s - L) delta_v[i]
Padding tokens (at or past the stream's valid count) take no part: beta 0, no
entries, zero readings.

Any chunk size C >= 1 is accepted. ``numpy.linalg.inv`` forms X.
"""

from __future__ import annotations

import numpy as np


def phase1(k_idx, k_val, g, q_idx, q_val, beta, n_live):
    """Phase-1 quantities of one chunk. Arrays are the chunk's rows [C, W] etc.; only
    the first ``n_live`` tokens take part. Returns a dict of fp64 intermediates."""
    C, W = k_idx.shape
    R = q_idx.shape[1]
    G = g.shape[1]
    gate = np.zeros((C, W))
    for i in range(n_live):
        for w in range(W):
            gate[i, w] = g[i, 0 if G == 1 else w]
    L = np.zeros((C, W))
    for i in range(n_live):
        for w in range(W):
            s = k_idx[i, w]
            L[i, w] = sum(gate[j, w2] for j in range(i + 1) for w2 in range(W) if k_idx[j, w2] == s)
    Lr = np.zeros((C, R))
    for i in range(n_live):
        for r in range(R):
            s = q_idx[i, r]
            Lr[i, r] = sum(gate[j, w2] for j in range(i + 1) for w2 in range(W) if k_idx[j, w2] == s)
    counts = {}
    for i in range(n_live):
        for w in range(W):
            counts[int(k_idx[i, w])] = counts.get(int(k_idx[i, w]), 0) + 1
    is_only = np.zeros((C, W), dtype=bool)
    for i in range(n_live):
        for w in range(W):
            is_only[i, w] = counts[int(k_idx[i, w])] == 1
    gw = np.zeros((C, W))
    gr = np.zeros((C, R))
    for i in range(n_live):
        for w in range(W):
            gw[i, w] = k_val[i, w] * np.exp(L[i, w])
        for r in range(R):
            gr[i, r] = q_val[i, r] * np.exp(Lr[i, r])
    A = np.zeros((C, C))
    QK = np.zeros((C, C))
    for i in range(n_live):
        for j in range(i + 1):
            for w2 in range(W):
                s = k_idx[j, w2]
                if j < i:
                    for w in range(W):
                        if k_idx[i, w] == s:
                            A[i, j] += k_val[i, w] * k_val[j, w2] * np.exp(L[i, w] - L[j, w2])
                for r in range(R):
                    if q_idx[i, r] == s:
                        QK[i, j] += q_val[i, r] * k_val[j, w2] * np.exp(Lr[i, r] - L[j, w2])
    b = np.zeros(C)
    b[:n_live] = beta[:n_live]
    # the final log-decay of each written slot and its write entries, in token order
    groups = {}
    for i in range(n_live):
        for w in range(W):
            groups.setdefault(int(k_idx[i, w]), []).append((i, w))
    Llast = {s: L[m[-1]] for s, m in groups.items()}
    return dict(gate=gate, L=L, Lr=Lr, is_only=is_only, gw=gw, gr=gr, A=A, QK=QK, beta=b,
                groups=groups, Llast=Llast)


def wy_solve(A, beta, QK):
    """X = (I + tril(beta[:, None] * A, -1))^-1 and QX = QK @ X (lower part of QK)."""
    C = A.shape[0]
    Lm = np.tril(beta[:, None] * A, -1)
    X = np.linalg.inv(np.eye(C) + Lm)
    X = np.tril(X)
    QX = np.tril(QK) @ X
    return X, QX


def phase2_step(B, p1, X, QX, k_idx, q_idx, k_val, v, n_live):
    """One chunk's gather, dual matmul and DW on the stream's bank ``B`` (updated in
    place). Returns (readings [C, hd], retrieved, inter, u, delta_v)."""
    C, W = k_idx.shape
    R = q_idx.shape[1]
    hd = B.shape[1]
    B0 = B.copy()
    retrieved = np.zeros((C, hd))
    inter = np.zeros((C, hd))
    for i in range(n_live):
        for w in range(W):
            retrieved[i] += p1["gw"][i, w] * B0[k_idx[i, w]]
        for r in range(R):
            inter[i] += p1["gr"][i, r] * B0[q_idx[i, r]]
    u = np.zeros((C, hd))
    u[:n_live] = p1["beta"][:n_live, None] * (v[:n_live] - retrieved[:n_live])
    delta_v = X @ u
    readings = QX @ u + inter
    readings[n_live:] = 0.0
    for s, members in p1["groups"].items():
        Llast = p1["Llast"][s]
        row = np.exp(Llast) * B0[s]
        for (i, w) in members:
            row = row + k_val[i, w] * np.exp(Llast - p1["L"][i, w]) * delta_v[i]
        B[s] = row
    return readings, retrieved, inter, u, delta_v


def forward(inputs: dict, C: int, emit: bool = False):
    """Chunked forward over all streams of float64 ``inputs`` (keys as in
    oracle.token_loop). Returns (readings [P, T, hd], bank [P, M, hd], intermediates)
    where intermediates (if ``emit``) is a list per stream of per-chunk dicts."""
    bank = np.array(inputs["bank"], dtype=np.float64, copy=True)
    P, T = inputs["k_idx"].shape[:2]
    hd = bank.shape[2]
    valid = inputs.get("valid")
    out = np.zeros((P, T, hd))
    inter_all = []
    Nt = -(-T // C)
    for p in range(P):
        nvalid = T if valid is None else int(valid[p])
        per = []
        for ti in range(Nt):
            t0 = ti * C
            rows = min(C, T - t0)

            def pad(a, width):
                z = np.zeros((C, width), dtype=a.dtype)
                z[:rows] = a[p, t0:t0 + rows].reshape(rows, width)
                return z
            W = inputs["k_idx"].shape[2]
            R = inputs["q_idx"].shape[2]
            G = inputs["g"].shape[2]
            k_idx = pad(inputs["k_idx"], W)
            q_idx = pad(inputs["q_idx"], R)
            k_val = pad(inputs["k_val"], W)
            q_val = pad(inputs["q_val"], R)
            g = pad(inputs["g"], G)
            beta = pad(inputs["beta"][:, :, None], 1)[:, 0]
            v = pad(inputs["v"], hd)
            n_live = max(0, min(rows, nvalid - t0))
            p1 = phase1(k_idx, k_val, g, q_idx, q_val, beta, n_live)
            X, QX = wy_solve(p1["A"], p1["beta"], p1["QK"])
            readings, retrieved, inter, u, delta_v = phase2_step(
                bank[p], p1, X, QX, k_idx, q_idx, k_val, v, n_live)
            out[p, t0:t0 + rows] = readings[:rows]
            if emit:
                per.append(dict(p1, X=X, QX=QX, retrieved=retrieved, inter=inter, u=u,
                                delta_v=delta_v, n_live=n_live))
        inter_all.append(per)
    return out, bank, inter_all
