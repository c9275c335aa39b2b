"""Pins of the oracle's attention dropout (oracle/philox.py, oracle/dropout.py)
to facts fixed outside it.

Generator: the Philox round structure, key schedule and output order are
checked against numpy's own Philox (the 4x64-10 instance of the same family);
the 32-bit constants against the published Philox-4x32-10 known-answer
vectors (tests/golden/philox4x32_10_kat.json).  Mask: the element-to-word
mapping against single scalar blocks, the keep rate and the uniformity of the
16-bit values statistically, and independence from T.  Attention: p = 0
against the C++ oracle, an all-kept mask against a closed form, torch's CPU
float64 autograd, central finite differences, unbiasedness of the output,
causality, and the exact read-out of a mask through a one-hot value matrix.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as od
from oracle.philox import philox4x32, philox_block
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return si.normal_f64(seed, int(np.prod(shape))).reshape(shape)


# ---------------------------------------------------------------- generator

@pytest.mark.parametrize("key", [(0, 0), (0x0123456789ABCDEF, 0xFEDCBA9876543210), (2**64 - 1, 7)])
def test_philox_4x64_matches_numpy(key):
    """numpy's Philox is Philox-4x64-10 and increments its counter before each
    block, so its first blocks are counters 1, 2, 3."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(12)]
    mine = sum((philox_block([c, 0, 0, 0], key, 64) for c in (1, 2, 3)), [])
    assert raw == mine


def test_philox_4x32_known_answers():
    g = json.load(open(os.path.join(GOLDEN, "philox4x32_10_kat.json")))
    for vec in g["vectors"]:
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        exp = [int(x, 16) for x in vec["out"]]
        assert philox_block(ctr, key, 32) == exp
        got = philox4x32(*(np.array([c], dtype=np.uint64) for c in ctr), key[0], key[1])
        assert [int(w[0]) for w in got] == exp


def test_philox_4x32_vectorised_equals_blocks():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    k0, k1 = 0x9ABCDEF0, 0x13572468
    got = philox4x32(ctr[0], ctr[1], ctr[2], ctr[3], k0, k1)
    for n in range(50):
        assert [int(w[n]) for w in got] == philox_block(ctr[:, n], (k0, k1), 32)


# --------------------------------------------------------------------- mask

def test_threshold_and_scale():
    assert od.threshold(0.0) == 0
    assert od.threshold(0.1) == 6554          # 0.1 * 65536 = 6553.6
    assert od.threshold(0.5) == 32768
    assert od.keep_scale(0.0) == 1.0
    assert od.keep_scale(0.5) == 2.0
    assert abs(od.keep_scale(0.1) - 65536 / (65536 - 6554)) == 0.0
    for bad in (-0.1, 1.0, 1.5, 1.0 - 2.0 ** -18):
        with pytest.raises(ValueError):
            od.threshold(bad)


def test_mask_elements_are_halves_of_one_block():
    """u(i, j) is half (j & 1) of word (j & 7) >> 1 of the block for counter
    (i, j >> 3, b*H + h, offset) and key (seed low, seed high)."""
    seed, offset, bh = 0x1234_5678_9ABC_DEF0, 77, 5
    u = od.uniform16(bh, 20, 40, seed, offset)
    for i in (0, 3, 19):
        for j in (0, 1, 6, 7, 8, 13, 39):
            x = philox_block([i, j >> 3, bh, offset], [seed & 0xFFFFFFFF, seed >> 32], 32)
            assert int(u[i, j]) == (x[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFF


def test_window_decisions_equal_the_mask_and_the_blocks():
    """uniform16_window / keep_window (decisions of some rows against a key
    window, for sequences too long for the whole mask) equal the slices of
    the whole mask, and at the positions of the longest sequence the library
    takes (rows up to 131063, keys from 131000) the halves of the single
    blocks of their counters."""
    seed, offset, bh, p = 0x0BAD_CAFE_1234_5678, 9, 3, 0.3
    full = od.uniform16(bh, 60, 70, seed, offset)
    rows = np.array([0, 5, 17, 59])
    for key0, n in ((0, 70), (13, 40), (64, 6)):
        win = od.uniform16_window(bh, rows, key0, n, seed, offset)
        assert np.array_equal(win, full[rows][:, key0:key0 + n])
        assert np.array_equal(od.keep_window(bh, rows, key0, n, p, seed, offset),
                              win >= od.threshold(p))
    big = np.array([131000, 131055, 131063])
    win = od.uniform16_window(bh, big, 131000, 64, seed, offset)
    for a, i in enumerate(big):
        for b_, j in enumerate((131000, 131001, 131007, 131008, 131063)):
            x = philox_block([int(i), j >> 3, bh, offset], [seed & 0xFFFFFFFF, seed >> 32], 32)
            assert int(win[a, j - 131000]) == (x[(j & 7) >> 1] >> (16 * (j & 1))) & 0xFFFF


def test_mask_rate_and_uniformity():
    """Over 4 slices of 512 x 512 values: the keep rate is within 5 standard
    deviations of 1 - t/65536, and the 16 leading-bit bins of the 16-bit values
    pass a chi-square test."""
    p = 0.1
    t = od.threshold(p)
    us = np.concatenate([od.uniform16(bh, 512, 512, 42, 3).ravel() for bh in range(4)])
    n = us.size
    keep = float(np.mean(us >= t))
    q = 1 - t / 65536
    assert abs(keep - q) < 5 * math.sqrt(q * (1 - q) / n)
    counts = np.bincount((us >> 12).astype(np.int64), minlength=16)
    chi2 = float(np.sum((counts - n / 16) ** 2 / (n / 16)))
    assert chi2 < 45.0  # 15 degrees of freedom: P(chi2 > 45) < 1e-4


def test_mask_depends_only_on_position():
    full = od.keep_mask(2, 3, 200, 0.3, 9, 1)
    part = od.keep_mask(2, 3, 50, 0.3, 9, 1)
    assert np.array_equal(full[:, :, :50, :50], part)
    # slice (b, h) uses index b*H + h
    assert np.array_equal(od.keep_mask(1, 1, 30, 0.3, 9, 1)[0, 0],
                          od.uniform16(0, 30, 30, 9, 1) >= od.threshold(0.3))
    assert np.array_equal(full[1, 2, :30, :30], od.uniform16(5, 30, 30, 9, 1) >= od.threshold(0.3))
    # seed and offset each change the mask
    assert not np.array_equal(full, od.keep_mask(2, 3, 200, 0.3, 10, 1))
    assert not np.array_equal(full, od.keep_mask(2, 3, 200, 0.3, 9, 2))
    assert np.array_equal(full, od.keep_mask(2, 3, 200, 0.3, 9, 1))


# ---------------------------------------------------------------- attention

def test_p0_equals_plain_oracle():
    B, H, T, hs = 2, 3, 37, 16
    q, k, v, do = (_rand((B, H, T, hs), 600 + n) for n in range(4))
    s = 1 / math.sqrt(hs)
    got = od.attention_backward_dropout(q, k, v, do, s, 0.0, 1, 0)
    ref = oracle.attention_backward(q, k, v, do, s)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_all_kept_mask_scales_every_output():
    """z = c everywhere: o, dq, dk, dv are c times the plain ones, lse unchanged
    (the weights are scaled after the softmax; dS = P(c dPd - c D))."""
    B, H, T, hs = 1, 2, 29, 8
    q, k, v, do = (_rand((B, H, T, hs), 610 + n) for n in range(4))
    s, c = 0.3, 65536 / (65536 - 6554)
    got = od.attention_backward_masked(q, k, v, do, s, np.full((B, H, T, T), c))
    ref = oracle.attention_backward(q, k, v, do, s)
    for n in range(4):
        np.testing.assert_allclose(got[n], c * ref[n], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[4], ref[4], rtol=0, atol=1e-12)


def test_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, H, T, hs = 2, 2, 33, 8
    q, k, v, do = (_rand((B, H, T, hs), 620 + n) for n in range(4))
    s, p = 1 / math.sqrt(hs), 0.25
    z = od.keep_mask(B, H, T, p, 123, 4) * od.keep_scale(p)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    sc = (tq @ tk.transpose(-1, -2)) * s
    sc = sc.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    o = (torch.softmax(sc, dim=-1) * torch.tensor(z)) @ tv
    lse = torch.logsumexp(sc, dim=-1)
    o.backward(torch.tensor(do))
    got = od.attention_backward_dropout(q, k, v, do, s, p, 123, 4)
    for a, b in zip(got, (tq.grad, tk.grad, tv.grad, o.detach(), lse.detach())):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("T,hs", [(1, 2), (3, 1), (6, 3), (9, 2)])
def test_finite_differences(T, hs):
    q, k, v, do = (_rand((1, 1, T, hs), 630 + 10 * T + n) for n in range(4))
    s, p = 0.7, 0.4
    z = od.keep_mask(1, 1, T, p, 5, T) * od.keep_scale(p)
    dq, dk, dv, _, _ = od.attention_backward_masked(q, k, v, do, s, z)
    L = lambda a, b, c: float(np.sum(do * od.attention_forward_masked(a, b, c, s, z)[0]))
    h = 1e-6
    for grad, idx in ((dq, 0), (dk, 1), (dv, 2)):
        for pos in np.ndindex(grad.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][pos] += h
            up = L(*args)
            args[idx][pos] -= 2 * h
            dn = L(*args)
            assert abs((up - dn) / (2 * h) - grad[pos]) < 1e-7, (idx, pos)


def test_output_is_unbiased():
    """The mean of o over 600 masks (offsets 0..599) approaches the output
    without dropout: every element within 5 standard errors."""
    B, H, T, hs = 1, 1, 12, 4
    q, k, v = (_rand((B, H, T, hs), 640 + n) for n in range(3))
    s, p, N = 0.5, 0.3, 600
    outs = np.stack([od.attention_forward_dropout(q, k, v, s, p, 31, off)[0] for off in range(N)])
    ref, _ = oracle.attention_forward(q, k, v, s)
    se = outs.std(axis=0, ddof=1) / math.sqrt(N)
    assert np.all(np.abs(outs.mean(axis=0) - ref) <= 5 * se + 1e-12)


def test_dropout_forward_is_causal():
    B, H, T, hs = 1, 2, 24, 8
    q, k, v = (_rand((B, H, T, hs), 650 + n) for n in range(3))
    o, lse = od.attention_forward_dropout(q, k, v, 0.4, 0.2, 8, 0)
    for n, a in enumerate((q, k, v)):
        a2 = a.copy()
        a2[:, :, 15:] += _rand((B, H, T - 15, hs), 660 + n)
        args = [q, k, v]
        args[n] = a2
        o2, lse2 = od.attention_forward_dropout(*args, 0.4, 0.2, 8, 0)
        assert np.array_equal(o2[:, :, :15], o[:, :, :15])
        assert np.array_equal(lse2[:, :, :15], lse[:, :, :15])


def test_one_hot_values_read_out_the_mask():
    """q = 0 makes the weights uniform, 1/(i+1) on keys 0..i; with v one-hot on
    a window of keys J..J+hs-1, o[i][d] = z(i, J+d) / (i+1): dropped weights
    give exact zeros.  The GPU tests read the kernels' masks the same way."""
    T, hs, J, p = 80, 16, 40, 0.3
    q = np.zeros((1, 1, T, hs))
    k = _rand((1, 1, T, hs), 670)
    v = np.zeros((1, 1, T, hs))
    v[0, 0, J:J + hs] = np.eye(hs)
    o, _ = od.attention_forward_dropout(q, k, v, 1.0, p, 77, 2)
    z = od.keep_mask(1, 1, T, p, 77, 2)[0, 0] * od.keep_scale(p)
    i = np.arange(T)[:, None]
    exp = np.where(J + np.arange(hs)[None, :] <= i, z[:, J:J + hs] / (i + 1), 0.0)
    np.testing.assert_allclose(o[0, 0], exp, rtol=1e-13, atol=0)
    assert np.array_equal(o[0, 0] == 0, exp == 0)
