"""Single rows and columns of causal attention and its backward, in float64
numpy, for sequences too long for the whole-problem oracle.

TEST INFRASTRUCTURE ONLY (same rule as the rest of `oracle/`).

Everything here is the definition of the "Let's build GPT" summary page
written out for one (b, h) slice and one query row at a time: the affinity
of query i with key j is their dot product (1:06:16) divided by sqrt(head
size) (1:17:18), keys after the query are masked out (tril with -inf, 48:54,
55:20), the row is softmax-normalised (51:04) and weights the values
(1:10:15).  The backward is the chain rule of that row:

  P[i][j] = exp(s[i][j] - lse[i]) for j <= i,   D[i] = dO[i] . o[i],
  dS[i][j] = P[i][j] (dO[i] . v[j] - D[i]),
  dq[i] = scale sum_j dS[i][j] k[j],
  dk[j] = scale sum_{i >= j} dS[i][j] q[i],   dv[j] = sum_{i >= j} P[i][j] dO[i].

dq of a row needs that row only; dk and dv of key j need every row i >= j,
so the columns are cheap near the end of the sequence.  Pinned in
tests/test_oracle_pins.py against the whole-problem oracle (every row and
column of small problems).
"""
from __future__ import annotations

import numpy as np


def _row(q, k, v, i: int, scale: float):
    """Row i of the causal forward: (scores, weights P, o, lse)."""
    s = (k[: i + 1] @ q[i]) * scale
    m = float(s.max())
    w = np.exp(s - m)
    l = float(w.sum())
    p = w / l
    return s, p, p @ v[: i + 1], m + np.log(l)


def forward_rows(q, k, v, scale: float, rows):
    """o and lse of the listed query rows of one (T, hs) slice."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    out_o, out_l = [], []
    for i in rows:
        _, _, o, lse = _row(q, k, v, int(i), scale)
        out_o.append(o)
        out_l.append(lse)
    return np.array(out_o), np.array(out_l)


def dq_rows(q, k, v, dO, scale: float, rows):
    """dq of the listed query rows of one (T, hs) slice."""
    q, k, v, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dO))
    out = []
    for i in rows:
        i = int(i)
        _, p, o, _ = _row(q, k, v, i, scale)
        dS = p * (v[: i + 1] @ dO[i] - float(dO[i] @ o))
        out.append(scale * (dS @ k[: i + 1]))
    return np.array(out)


def dkdv_columns(q, k, v, dO, scale: float, j0: int, j1: int):
    """dk and dv of keys j0 .. j1-1 of one (T, hs) slice: every row i >= j0
    contributes to the keys j <= i of the range."""
    q, k, v, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dO))
    T, hs = q.shape
    dk = np.zeros((j1 - j0, hs))
    dv = np.zeros((j1 - j0, hs))
    for i in range(j0, T):
        _, p, o, _ = _row(q, k, v, i, scale)
        hi = min(i + 1, j1)  # keys of the range that row i sees
        pj = p[j0:hi]
        dS = pj * (v[j0:hi] @ dO[i] - float(dO[i] @ o))
        dv[: hi - j0] += np.outer(pj, dO[i])
        dk[: hi - j0] += scale * np.outer(dS, q[i])
    return dk, dv


def forward_all_rows(q, k, v, scale: float, block: int = 256):
    """o and lse of every query row of one (T, hs) slice, the rows taken in
    blocks of `block` so that each row's scores, mask, softmax and value sum
    (the definitions above, one row at a time) run as matrix products."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    T, hs = q.shape
    o = np.empty((T, hs))
    lse = np.empty(T)
    for r0 in range(0, T, block):
        r1 = min(T, r0 + block)
        s = q[r0:r1] @ k[:r1].T
        s *= scale
        # keys after row i lie in the block's own columns r0 .. r1-1 only
        diag = s[:, r0:r1]
        diag[np.triu(np.ones((r1 - r0, r1 - r0), dtype=bool), 1)] = -np.inf
        m = s.max(axis=1, keepdims=True)
        s -= m
        np.exp(s, out=s)
        l = s.sum(axis=1, keepdims=True)
        o[r0:r1] = (s @ v[:r1]) / l
        lse[r0:r1] = (m + np.log(l))[:, 0]
    return o, lse


def dkdv_block(q, k, v, dO, scale: float, j0: int, j1: int, o, lse, block: int = 256):
    """dk and dv of keys j0 .. j1-1 from every row i >= j0, given the rows' o
    and lse (from forward_all_rows): P[i][j] = exp(s[i][j] - lse[i]) and
    D[i] = dO[i] . o[i] as in the header; rows taken in blocks."""
    q, k, v, dO, o, lse = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dO, o, lse))
    T, hs = q.shape
    dk = np.zeros((j1 - j0, hs))
    dv = np.zeros((j1 - j0, hs))
    kj, vj = k[j0:j1], v[j0:j1]
    for r0 in range(j0, T, block):
        r1 = min(T, r0 + block)
        s = (q[r0:r1] @ kj.T) * scale
        p = np.exp(s - lse[r0:r1, None])
        p[np.arange(j0, j1)[None, :] > np.arange(r0, r1)[:, None]] = 0.0
        D = np.sum(dO[r0:r1] * o[r0:r1], axis=1)
        dS = p * (dO[r0:r1] @ vj.T - D[:, None])
        dv += p.T @ dO[r0:r1]
        dk += scale * (dS.T @ q[r0:r1])
    return dk, dv
