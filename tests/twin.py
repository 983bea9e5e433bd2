"""Brute-force NumPy restatement of MALA for tiny inputs (test code only).

A second, independent formulation used to pin the C oracle: it never keeps
the running (m, l) state. The forward test recomputes the retained normaliser
Z_q^(t) as an explicit sum over the keys retained so far (paper Sec. 2.2,
Eq. 1) and compares the ratio of Eq. 2 with tau/L_q directly (no logarithms).
The backward is written as the masked gradient formula: with the tile mask
M of Eq. 4 (P_qk >= tau/L_q for some legal entry of the tile),
dV = (P o M)^T dO, dS = P o M o (dP - rowsum(O o dO)), dQ = s dS K,
dK = s dS^T Q. Decode retains per split with the split's own Z and outputs
softmax over the union of retained keys, which is what the merge computes.

Only for small N (exp of raw scores must not overflow).
"""
from __future__ import annotations

import numpy as np


def _legal(Nq, Nk, causal):
    # causal queries sit at the last Nq key positions: query q is at q + Nk - Nq
    qi = np.arange(Nq)[:, None] + (Nk - Nq)
    kj = np.arange(Nk)[None, :]
    return (kj <= qi) if causal else np.ones((Nq, Nk), dtype=bool)


def _visible(Nq, Nk, causal):
    return (np.arange(Nq) + 1.0 + (Nk - Nq)) if causal else np.full(Nq, float(Nk))


def twin_fwd_head(q, k, v, tau, causal, bq, bk, scale):
    """One head. q [Nq,d], k/v [Nk,d] -> (o, lse, dec [Tr,Tc])."""
    Nq, Nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    leg = _legal(Nq, Nk, causal)
    L = _visible(Nq, Nk, causal)
    Tr, Tc = -(-Nq // bq), -(-Nk // bk)
    dec = np.full((Tr, Tc), -1, dtype=np.int8)
    keep = np.zeros((Nq, Nk), dtype=bool)
    for i in range(Tr):
        rows = np.arange(i * bq, min(Nq, (i + 1) * bq))
        # blocks that hold a legal key for some row, visited last-to-first
        blocks = [j for j in range(Tc) if leg[np.ix_(rows, np.arange(j * bk, min(Nk, (j + 1) * bk)))].any()]
        for j in sorted(blocks, reverse=True):
            cols = np.arange(j * bk, min(Nk, (j + 1) * bk))
            skip = True
            for r in rows:
                lc = cols[leg[r, cols]]
                if lc.size == 0:
                    continue  # no legal key: this row does not constrain the tile
                Z = np.exp(s[r, keep[r]]).sum()
                if Z == 0.0:
                    skip = False  # ratio is +inf before anything is retained
                    break
                ratio = np.exp(s[r, lc].max()) / Z
                if not ratio < tau / L[r]:
                    skip = False
            dec[i, j] = 0 if skip else 1
            if not skip:
                for r in rows:
                    keep[r, cols] |= leg[r, cols]
    w = np.where(keep, np.exp(s), 0.0)
    Z = w.sum(axis=1)
    return (w @ v) / Z[:, None], np.log(Z), dec, keep


def twin_fwd(q, k, v, tau, causal=True, bq=64, bk=64, scale=None):
    B, Hq, Nq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.zeros_like(q, dtype=np.float64)
    lse = np.zeros(q.shape[:3])
    decs = []
    keeps = []
    for b in range(B):
        db, kb = [], []
        for h in range(Hq):
            oh, lh, dh, kh = twin_fwd_head(q[b, h], k[b, h // G], v[b, h // G], tau, causal, bq, bk, scale)
            o[b, h], lse[b, h] = oh, lh
            db.append(dh)
            kb.append(kh)
        decs.append(db)
        keeps.append(kb)
    return o, lse, np.asarray(decs), np.asarray(keeps)


def twin_bwd(q, k, v, o, lse, dout, tau, causal=True, bq=64, bk=64, scale=None, mag=False,
             dsens=False):
    """Masked-gradient form of Algorithm 2 -> (dq, dk, dv, dec). With
    mag=True every product uses absolute values (|dS| |K|, P |dO|, ...);
    with dsens=True dS is replaced by P * sum_d |O||dO| (and dV is 0)."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    leg = _legal(Nq, Nk, causal)
    L = _visible(Nq, Nk, causal)
    Tr, Tc = -(-Nq // bq), -(-Nk // bk)
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    dec = np.full((B, Hq, Tr, Tc), -1, dtype=np.int8)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, h] @ k[b, g].T)
            P = np.where(leg, np.exp(s - lse[b, h][:, None]), 0.0)
            M = np.zeros((Nq, Nk), dtype=bool)
            for i in range(Tr):
                for j in range(Tc):
                    rs = slice(i * bq, min(Nq, (i + 1) * bq))
                    cs = slice(j * bk, min(Nk, (j + 1) * bk))
                    lg = leg[rs, cs]
                    if not lg.any():
                        continue
                    hit = (P[rs, cs] >= tau / L[rs][:, None]) & lg
                    dec[b, h, i, j] = 1 if hit.any() else 0
                    if hit.any():
                        M[rs, cs] = True
            Pm = np.where(M, P, 0.0)
            dP = dout[b, h] @ v[b, g].T
            D = (o[b, h] * dout[b, h]).sum(axis=1)
            dS = Pm * (dP - D[:, None])
            if dsens:
                dS = Pm * np.abs(o[b, h] * dout[b, h]).sum(axis=1)[:, None]
                mag = True
            f = np.abs if mag else (lambda x: x)
            dq[b, h] = scale * f(dS) @ f(k[b, g])
            dk[b, g] += scale * f(dS).T @ f(q[b, h])
            if not dsens:
                dv[b, g] += Pm.T @ f(dout[b, h])
    return dq, dk, dv, dec


def twin_decode(q, k, v, tau, num_splits, bk=64, scale=None):
    """q [B,Hq,d], k/v [B,Hkv,Nk,d] -> (o, lse, dec [B,Hq,Tc])."""
    B, Hq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    Tc = -(-Nk // bk)
    per = -(-Tc // num_splits)
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    dec = np.full((B, Hq, Tc), -1, dtype=np.int8)
    for b in range(B):
        for h in range(Hq):
            s = scale * (k[b, h // G] @ q[b, h])
            keep = np.zeros(Nk, dtype=bool)
            for sp in range(num_splits):
                tiles = range(sp * per, min(Tc, (sp + 1) * per))
                kept_here = np.zeros(Nk, dtype=bool)
                for j in reversed(list(tiles)):
                    cols = np.arange(j * bk, min(Nk, (j + 1) * bk))
                    Z = np.exp(s[kept_here]).sum()
                    retain = Z == 0.0 or not (np.exp(s[cols].max()) / Z < tau / Nk)
                    dec[b, h, j] = 1 if retain else 0
                    if retain:
                        kept_here[cols] = True
                keep |= kept_here
            w = np.where(keep, np.exp(s), 0.0)
            o[b, h] = (w @ v[b, h // G]) / w.sum()
            lse[b, h] = np.log(w.sum())
    return o, lse, dec
