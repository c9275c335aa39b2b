"""Attention dropout (oracle side, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages train the RobGPT model with dropout 0.1 ("GPT da zero", the
parameter table under "Come funziona") and set it to 0.0 in the GPT-2 124M
configuration ("Model Architecture Nanogpt", Workflow 2).  Neither page shows
where inside attention it acts; the reading taken here is dropout on the
attention weights: after the row softmax and before the weighted sum of the
values, each weight is zeroed with probability p and the kept ones are
multiplied by 1/(1 - p) (inverted dropout, so the expectation of the output
is the output without dropout).

Mask definition (the GPU library draws the same bits with its own
generator code):
  * t = floor(p * 65536 + 0.5), 0 <= t <= 65535 (p is rounded to a multiple
    of 2^-16; the effective probability is t / 65536);
  * for slice (b, h), query i, key j: one Philox-4x32-10 block with counter
    (i, j >> 3, b*H + h, offset) and key (seed mod 2^32, seed >> 32); its
    words x0..x3 hold eight 16-bit values, u(i, j) = the (j & 1)-th half
    (low half first) of word (j & 7) >> 1;
  * keep(i, j) = u(i, j) >= t, and Z(i, j) = keep(i, j) * 65536 / (65536 - t).
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x32


def threshold(p: float) -> int:
    """16-bit drop threshold t of probability p (rounded to nearest)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    t = int(np.floor(p * 65536.0 + 0.5))
    if t > 65535:
        raise ValueError("dropout probability rounds to 1")
    return t


def keep_scale(p: float) -> float:
    """The factor 1/(1 - t/65536) applied to kept weights."""
    t = threshold(p)
    return 65536.0 / (65536.0 - t)


def uniform16_window(bh: int, rows, key0: int, nkeys: int, seed: int, offset: int) -> np.ndarray:
    """u(i, j) for one slice (index bh = b*H + h), i in `rows`, key0 <= j <
    key0 + nkeys, as uint32 (len(rows), nkeys): the decisions of a window
    without the whole T x T mask."""
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(key0, key0 + nkeys)
    g = (j.astype(np.uint64) >> np.uint64(3))[None, :]
    words = philox4x32(i, g, np.uint64(bh), np.uint64(offset & 0xFFFFFFFF),
                       seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(np.broadcast_arrays(*words), axis=0)  # (4, rows, nkeys)
    sel = np.take_along_axis(w, np.broadcast_to(((j & 7) >> 1)[None, None, :],
                                                (1, w.shape[1], nkeys)), axis=0)[0]
    return (sel >> ((j & 1) * 16).astype(np.uint32)) & np.uint32(0xFFFF)


def uniform16(bh: int, Tq: int, Tk: int, seed: int, offset: int) -> np.ndarray:
    """u(i, j) for one slice (index bh = b*H + h), i < Tq, j < Tk, as uint32."""
    return uniform16_window(bh, np.arange(Tq), 0, Tk, seed, offset)


def keep_mask(B: int, H: int, T: int, p: float, seed: int, offset: int, slices=None):
    """keep(i, j) as bool (B, H, T, T) (or only the listed (b, h) slices, as a
    dict {(b, h): (T, T) array})."""
    t = threshold(p)
    if slices is not None:
        return {(b, h): uniform16(b * H + h, T, T, seed, offset) >= t for b, h in slices}
    out = np.empty((B, H, T, T), dtype=bool)
    for b in range(B):
        for h in range(H):
            out[b, h] = uniform16(b * H + h, T, T, seed, offset) >= t
    return out


def keep_window(bh: int, rows, key0: int, nkeys: int, p: float, seed: int,
                offset: int) -> np.ndarray:
    """keep(i, j) as bool for i in `rows`, key0 <= j < key0 + nkeys (slice bh)."""
    return uniform16_window(bh, rows, key0, nkeys, seed, offset) >= threshold(p)


def _slice_fwd(q, k, v, scale, z):
    """One (T, hs) slice: causal softmax attention with the weights multiplied
    by z (T, T) before the value sum.  Returns o, lse and the softmax P."""
    T = q.shape[0]
    s = scale * (q @ k.T)
    s[np.triu_indices(T, 1)] = -np.inf  # a token cannot look ahead
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    return (p * z) @ v, (m + np.log(l))[:, 0], p


def attention_forward_masked(q, k, v, scale: float, z):
    """(o, lse) for (B, H, T, hs) inputs with weight multipliers z (B, H, T, T);
    lse is of the softmax before dropout."""
    q, k, v, z = (np.asarray(a, dtype=np.float64) for a in (q, k, v, z))
    B, H, T, hs = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _ = _slice_fwd(q[b, h], k[b, h], v[b, h], scale, z[b, h])
    return o, lse


def _slice_bwd(q, k, v, do, scale, z):
    o, lse, p = _slice_fwd(q, k, v, scale, z)
    pd = p * z                      # the weights after dropout
    dv = pd.T @ do                  # o = pd v
    dpd = do @ v.T                  # gradient of the dropped weights
    dp = dpd * z                    # through the multiplication by z
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # softmax Jacobian per row
    return scale * (ds @ k), scale * (ds.T @ q), dv, o, lse


def attention_backward_masked(q, k, v, dO, scale: float, z):
    """(dq, dk, dv, o, lse) of L = sum(dO * o) for the forward above."""
    q, k, v, dO, z = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dO, z))
    B, H, T, hs = q.shape
    outs = [np.empty_like(q) for _ in range(4)] + [np.empty((B, H, T))]
    for b in range(B):
        for h in range(H):
            r = _slice_bwd(q[b, h], k[b, h], v[b, h], dO[b, h], scale, z[b, h])
            for dst, val in zip(outs, r):
                dst[b, h] = val
    return tuple(outs)


def _z(B, H, T, p, seed, offset, slices):
    s = keep_scale(p)
    if slices is None:
        return keep_mask(B, H, T, p, seed, offset) * s
    return {bh: m * s for bh, m in keep_mask(B, H, T, p, seed, offset, slices).items()}


def attention_forward_dropout(q, k, v, scale: float, p: float, seed: int, offset: int):
    """(o, lse) with the dropout mask drawn as defined above."""
    B, H, T, _ = np.shape(q)
    return attention_forward_masked(q, k, v, scale, _z(B, H, T, p, seed, offset, None))


def attention_backward_dropout(q, k, v, dO, scale: float, p: float, seed: int, offset: int,
                               slices=None):
    """(dq, dk, dv, o, lse) with the dropout mask drawn as defined above.  With
    `slices` (a list of (b, h)), only those slices are computed and each output
    is (len(slices), T, hs) / (len(slices), T) in that order."""
    B, H, T, _ = np.shape(q)
    if slices is None:
        return attention_backward_masked(q, k, v, dO, scale, _z(B, H, T, p, seed, offset, None))
    zs = _z(B, H, T, p, seed, offset, slices)
    res = [_slice_bwd(*(np.asarray(a[b, h], dtype=np.float64) for a in (q, k, v, dO)), scale,
                      zs[(b, h)]) for b, h in slices]
    return tuple(np.stack([r[n] for r in res]) for n in range(5))
