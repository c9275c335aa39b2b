"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test names what fixes the expected value: a hand-worked example, a closed
form from the pages' own "running mean with a tril matrix" trick, an invariant
of the definition, a library routine (torch's CPU float64 causal attention and
its autograd), or central finite differences.  None re-types the oracle's loop.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return si.normal_f64(seed, int(np.prod(shape))).reshape(shape)


def _val(x):
    table = {"ln3": math.log(3.0), "ln4": math.log(4.0), "0.75*ln3": 0.75 * math.log(3.0)}
    return table[x] if isinstance(x, str) else float(x)


def test_worked_example_t2():
    """Hand-worked T=2 example (tests/golden/t2_worked_example.json)."""
    g = json.load(open(os.path.join(GOLDEN, "t2_worked_example.json")))
    inp = {k: np.array([_val(x) for x in v]).reshape(1, 1, 2, 1) for k, v in g["inputs"].items()
           if k != "scale"}
    dq, dk, dv, o, lse = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["dO"],
                                                   g["inputs"]["scale"])
    exp = {k: np.array([_val(x) for x in v]) for k, v in g["expected"].items()}
    np.testing.assert_allclose(o.ravel(), exp["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse.ravel(), exp["lse"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dq.ravel(), exp["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), exp["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), exp["dv"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("T,hs", [(1, 3), (7, 4), (33, 8)])
def test_tril_running_mean(T, hs):
    """Q = 0 makes every visible score equal: softmax of the tril-masked row is
    the uniform 1/(i+1) weight of the pages' running-mean trick (47:18-51:04).
    Closed forms: o_i = mean(v_0..v_i), lse_i = ln(i+1),
    dV_j = sum_{i>=j} dO_i/(i+1), dK = 0,
    dQ_i = scale/(i+1) * sum_{j<=i} <dO_i, v_j - o_i> k_j."""
    B, H = 2, 3
    q = np.zeros((B, H, T, hs))
    k, v, dO = _rand((B, H, T, hs), 1), _rand((B, H, T, hs), 2), _rand((B, H, T, hs), 3)
    scale = 0.37
    dq, dk, dv, o, lse = oracle.attention_backward(q, k, v, dO, scale)
    cnt = np.arange(1, T + 1, dtype=np.float64)
    mean = np.cumsum(v, axis=2) / cnt[:, None]
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(cnt), lse.shape), rtol=0, atol=1e-12)
    w = dO / cnt[:, None]
    dv_ref = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    np.testing.assert_allclose(dv, dv_ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(dk, 0.0)
    dq_ref = np.zeros_like(dq)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                for j in range(i + 1):
                    c = np.dot(dO[b, h, i], v[b, h, j] - mean[b, h, i])
                    dq_ref[b, h, i] += scale / (i + 1) * c * k[b, h, j]
    np.testing.assert_allclose(dq, dq_ref, rtol=0, atol=1e-12)


def test_rows_sum_to_one():
    """Rows of the softmax sum to one (51:04): V = 1 gives O = 1; a shared
    constant value row c gives O = c and zero dQ, dK (dP_ij = D_i)."""
    B, H, T, hs = 2, 2, 17, 5
    q, k, dO = _rand((B, H, T, hs), 4), _rand((B, H, T, hs), 5), _rand((B, H, T, hs), 6)
    o, _ = oracle.attention_forward(q, k, np.ones((B, H, T, hs)), 0.5)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
    c = np.array([0.5, -2.0, 3.0, 0.25, 1.5])
    v = np.broadcast_to(c, (B, H, T, hs)).copy()
    dq, dk, dv, o, _ = oracle.attention_backward(q, k, v, dO, 0.5)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dq, 0.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, rtol=0, atol=1e-12)
    # sum_j dV_j = sum_i dO_i (each row of P sums to one)
    np.testing.assert_allclose(dv.sum(axis=2), dO.sum(axis=2), rtol=0, atol=1e-12)


def test_t_equals_one():
    """T = 1: the only visible key is the token itself: o = v, lse = scale q.k,
    dV = dO, dQ = dK = 0."""
    B, H, T, hs = 3, 2, 1, 6
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (7, 8, 9, 10))
    dq, dk, dv, o, lse = oracle.attention_backward(q, k, v, dO, 0.3)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.3 * np.sum(q * k, axis=-1), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(dv, dO)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


def test_causality():
    """Tokens cannot look into the future (55:20): rows <= i of o, lse, dQ do not
    change when rows > i of Q, K, V, dO change; dK_j, dV_j do not change when
    rows < j of Q and dO change.  Exact in the oracle."""
    B, H, T, hs = 1, 2, 12, 4
    base = [_rand((B, H, T, hs), s) for s in (11, 12, 13, 14)]
    i = 6
    pert = [x.copy() for x in base]
    for n, x in enumerate(pert):
        x[:, :, i + 1:] += _rand(x[:, :, i + 1:].shape, 100 + n)
    r0 = oracle.attention_backward(*base, 0.5)
    r1 = oracle.attention_backward(*pert, 0.5)
    for a, b in zip((r0[0], r0[3]), (r1[0], r1[3])):  # dq, o
        np.testing.assert_array_equal(a[:, :, :i + 1], b[:, :, :i + 1])
    np.testing.assert_array_equal(r0[4][:, :, :i + 1], r1[4][:, :, :i + 1])
    j = 5
    pert = [x.copy() for x in base]
    pert[0][:, :, :j] += 1.0  # q rows < j
    pert[3][:, :, :j] -= 2.0  # dO rows < j
    r2 = oracle.attention_backward(*pert, 0.5)
    np.testing.assert_array_equal(r0[1][:, :, j:], r2[1][:, :, j:])  # dk
    np.testing.assert_array_equal(r0[2][:, :, j:], r2[2][:, :, j:])  # dv


def test_key_shift_invariance():
    """Adding one vector c to every key adds scale*q_i.c to every score of row i,
    which the softmax cancels: O and dQ unchanged, lse_i += scale*q_i.c, and
    sum_j dK_j = 0 per (b, h) (each row of dS sums to zero)."""
    B, H, T, hs = 2, 2, 15, 6
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (15, 16, 17, 18))
    c = _rand((hs,), 19)
    s = 0.41
    r0 = oracle.attention_backward(q, k, v, dO, s)
    r1 = oracle.attention_backward(q, k + c, v, dO, s)
    np.testing.assert_allclose(r1[3], r0[3], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r1[0], r0[0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(r1[4], r0[4] + s * (q @ c), rtol=0, atol=1e-12)
    np.testing.assert_allclose(r0[1].sum(axis=2), 0.0, rtol=0, atol=1e-11)


def test_literal_page_form():
    """The pages' own recipe written as matrices: build the full T x T score
    matrix, put -inf above the diagonal, softmax each row, multiply by V."""
    B, H, T, hs = 2, 3, 20, 7
    q, k, v = (_rand((B, H, T, hs), s) for s in (20, 21, 22))
    scale = 1.0 / math.sqrt(hs)
    wei = (q @ np.swapaxes(k, -1, -2)) * scale
    tril = np.tril(np.ones((T, T)))
    wei = np.where(tril == 0, -np.inf, wei)
    wei = np.exp(wei - wei.max(axis=-1, keepdims=True))
    wei = wei / wei.sum(axis=-1, keepdims=True)
    o, _ = oracle.attention_forward(q, k, v, scale)
    np.testing.assert_allclose(o, wei @ v, rtol=0, atol=1e-12)


def test_against_torch_library_float64():
    """Library routine: torch CPU float64 scaled_dot_product_attention with
    is_causal=True, and its autograd gradients, on the same inputs."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    B, H, T, hs = 2, 3, 37, 16
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (23, 24, 25, 26))
    scale = 1.0 / math.sqrt(hs)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    out.backward(torch.tensor(dO))
    dq, dk, dv, o, lse = oracle.attention_backward(q, k, v, dO, scale)
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)
    # lse: torch.logsumexp of the masked, scaled score matrix
    s = torch.tensor(q) @ torch.tensor(k).transpose(-1, -2) * scale
    s = s.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,hs", [(1, 1), (2, 2), (3, 8), (5, 1), (8, 2)])
def test_finite_difference_gradients(T, hs):
    """Central finite differences of L = sum(dO * O) in float64."""
    B, H = 1, 2
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (27 + T, 28 + T, 29 + T, 30 + T))
    scale = 0.8
    dq, dk, dv, _, _ = oracle.attention_backward(q, k, v, dO, scale)

    def loss(qq, kk, vv):
        return float(np.sum(dO * oracle.attention_forward(qq, kk, vv, scale)[0]))

    for idx, (x, g) in enumerate(((q, dq), (k, dk), (v, dv))):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            h = 1e-6 * max(1.0, abs(x[pos]))
            args = [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args[idx] = xp
            lp = loss(*args)
            args[idx] = xm
            lm = loss(*args)
            num[pos] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err <= 1e-6, (idx, err)


def test_heads_independent():
    """Heads run in parallel and independently (1:22:27): 25 heads in one call
    equal 25 single-head calls bit for bit, and permuting (b, h) slices
    permutes the outputs."""
    B, H, T, hs = 1, 25, 9, 4
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (40, 41, 42, 43))
    full = oracle.attention_backward(q, k, v, dO, 0.5)
    for h in range(H):
        one = oracle.attention_backward(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1],
                                        dO[:, h:h + 1], 0.5)
        for a, b in zip(full, one):
            np.testing.assert_array_equal(a[:, h:h + 1], b)
    perm = np.random.default_rng(0).permutation(H)
    pr = oracle.attention_backward(q[:, perm], k[:, perm], v[:, perm], dO[:, perm], 0.5)
    for a, b in zip(full, pr):
        np.testing.assert_array_equal(a[:, perm], b)


def test_scale_gives_unit_variance_scores():
    """Dividing by sqrt(head size) keeps unit variance at init (1:17:18): for
    unit-variance q and k, lse_0 = scale * q_0.k_0 has variance ~1."""
    B, H, T, hs = 64, 64, 1, 64
    q, k, v = (_rand((B, H, T, hs), s) for s in (44, 45, 46))
    _, lse = oracle.attention_forward(q, k, v, 1.0 / math.sqrt(hs))
    var = float(np.var(lse))
    assert 0.9 < var < 1.1, var


def test_threads_do_not_change_results():
    B, H, T, hs = 3, 5, 11, 8
    q, k, v, dO = (_rand((B, H, T, hs), s) for s in (47, 48, 49, 50))
    a = oracle.attention_backward(q, k, v, dO, 0.35, nthreads=1)
    b = oracle.attention_backward(q, k, v, dO, 0.35, nthreads=4)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ------------------------------------------------ newest-Tq-tokens forward (decode)
def test_kv_forward_equal_lengths_is_the_causal_forward():
    """Tq = Tk: every query sees keys j <= i, the forward itself, bit for bit."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 3, 37, 8)) for _ in range(3))
    o, lse = oracle.attention_forward(q, k, v, 0.4)
    o2, lse2 = oracle.attention_forward_kv(q, k, v, 0.4)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("Tq", [1, 2, 7, 30])
def test_kv_forward_is_the_last_rows_of_the_full_forward(Tq):
    """The pages' generate recomputes the whole forward and keeps the last
    positions; the newest-Tq forward must equal those rows exactly."""
    rng = np.random.default_rng(12 + Tq)
    Tk = 30
    q, k, v = (rng.standard_normal((2, 2, Tk, 5)) for _ in range(3))
    o, lse = oracle.attention_forward(q, k, v, 0.7)
    o2, lse2 = oracle.attention_forward_kv(q[:, :, Tk - Tq:], k, v, 0.7)
    assert np.array_equal(o[:, :, Tk - Tq:], o2) and np.array_equal(lse[:, :, Tk - Tq:], lse2)


def test_kv_forward_single_query_is_plain_softmax_attention():
    """Tq = 1: the newest token sees every key, softmax(scale q K^T) V."""
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 2, 1, 6))
    k, v = (rng.standard_normal((1, 2, 19, 6)) for _ in range(2))
    o, lse = oracle.attention_forward_kv(q, k, v, 0.5)
    s = 0.5 * np.einsum("bhd,bhjd->bhj", q[:, :, 0], k)
    w = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("bhj,bhjd->bhd", w / w.sum(-1, keepdims=True), v)
    assert np.allclose(o[:, :, 0], ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse[:, :, 0], np.log(np.exp(s).sum(-1)), rtol=1e-13, atol=1e-13)


# --------------------------------------- single rows and key columns (oracle.rows)
@pytest.mark.parametrize("T,hs,scale", [(37, 16, 0.3), (64, 8, 1.1)])
def test_rows_and_columns_equal_the_whole_problem_oracle(T, hs, scale):
    """oracle.rows evaluates one query row (or one key column) at a time in
    numpy, for sequences too long for the whole-problem oracle.  On small
    problems every row's o, lse and dq and every key's dk and dv equal those of
    the C++ oracle (pinned above) to float64 rounding, and a key range taken
    from the middle equals the same keys of the whole problem."""
    from oracle import rows
    q, k, v, dO = (_rand((T, hs), 60 + i) for i in range(4))
    dq, dk, dv, o, lse = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                                   dO[None, None], scale)
    ro, rl = rows.forward_rows(q, k, v, scale, range(T))
    np.testing.assert_allclose(ro, o[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(rl, lse[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(rows.dq_rows(q, k, v, dO, scale, range(T)), dq[0, 0], rtol=0,
                               atol=1e-12)
    rdk, rdv = rows.dkdv_columns(q, k, v, dO, scale, 0, T)
    np.testing.assert_allclose(rdk, dk[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(rdv, dv[0, 0], rtol=0, atol=1e-12)
    j0, j1 = T // 3, T // 3 + 9
    mdk, mdv = rows.dkdv_columns(q, k, v, dO, scale, j0, j1)
    np.testing.assert_allclose(mdk, dk[0, 0, j0:j1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(mdv, dv[0, 0, j0:j1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,hs,scale,block", [(37, 16, 0.3, 8), (200, 8, 1.1, 64), (64, 4, 0.5, 100)])
def test_blocked_rows_equal_the_whole_problem_oracle(T, hs, scale, block):
    """oracle.rows.forward_all_rows / dkdv_block batch independent rows into
    blocks of matrix products (blocks smaller than, straddling and larger than
    T); every row's o and lse and a key range's dk and dv (from the start, the
    middle and the end, given those rows) equal the C++ oracle to float64
    rounding."""
    from oracle import rows
    q, k, v, dO = (_rand((T, hs), 70 + i) for i in range(4))
    dq, dk, dv, o, lse = oracle.attention_backward(q[None, None], k[None, None], v[None, None],
                                                   dO[None, None], scale)
    bo, bl = rows.forward_all_rows(q, k, v, scale, block=block)
    np.testing.assert_allclose(bo, o[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(bl, lse[0, 0], rtol=0, atol=1e-12)
    for j0, j1 in ((0, min(T, 13)), (T // 2, T // 2 + 5), (T - 3, T)):
        bdk, bdv = rows.dkdv_block(q, k, v, dO, scale, j0, j1, bo, bl, block=block)
        np.testing.assert_allclose(bdk, dk[0, 0, j0:j1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(bdv, dv[0, 0, j0:j1], rtol=0, atol=1e-12)
