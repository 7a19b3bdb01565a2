"""Pins for the fp64 CPU oracle (no GPU).

The pages print no worked numerical example, so every pin here is a closed form,
a library routine the oracle does not use (scipy softmax / logistic, PyTorch's
CPU attention), a brute-force sum over tokens, or an invariant of the method.
Each is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign, a transposed operand, a wrong scale or a mask) fails at least one test.

Sources: gist.science explainer of "Retrofitting Linear Attention into Diffusion
Language Models", Technical Summary, "Methodology: Block-Hybrid Attention" /
"Architecture Design"; pith.science review of the same paper, "The reading",
"What carries the argument".
"""
import numpy as np
import pytest
import scipy.special as sp
import torch

import oracle

SHAPES = [  # (d, FW, B): includes d == F and d != F so a transposed state cannot pass
    (4, 2, 3),
    (8, 4, 1),
    (6, 3, 5),
    (16, 8, 8),
    (8, 8, 4),
]


def _rng(seed):
    return np.random.default_rng(seed)


def _w(rng, fw, d, scale=1.0):
    return rng.standard_normal((fw, d)) * scale / np.sqrt(d)


# ---------------------------------------------------------------- feature map
@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_phi_halves_positive_and_normalised(d, fw, _b):
    rng = _rng(1)
    x = rng.standard_normal((7, d)) * 3
    ph = oracle.phi(x, _w(rng, fw, d, 4.0))
    assert ph.shape == (7, 2 * fw)
    assert np.all(ph > 0)
    np.testing.assert_allclose(ph[:, :fw].sum(1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ph[:, fw:].sum(1), 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_phi_negated_input_swaps_halves(d, fw, _b):
    rng = _rng(2)
    x = rng.standard_normal((5, d))
    w = _w(rng, fw, d, 2.0)
    a, b = oracle.phi(x, w), oracle.phi(-x, w)
    np.testing.assert_allclose(b[:, :fw], a[:, fw:], rtol=1e-13, atol=0)
    np.testing.assert_allclose(b[:, fw:], a[:, :fw], rtol=1e-13, atol=0)


def test_phi_zero_matrix_is_uniform():
    rng = _rng(3)
    x = rng.standard_normal((4, 8))
    ph = oracle.phi(x, np.zeros((5, 8)))
    np.testing.assert_allclose(ph, np.full((4, 10), 0.2), rtol=0, atol=1e-15)


def test_phi_two_column_closed_form():
    # d = 3, FW = 2. W (3 x 2) has columns (0.5, 1, -1) and (2, 0, 1); stored
    # one column per row. For x = (1, -2, 0.5): xW = (-2, 2.5) by hand, and a
    # two-way softmax is the logistic function of the difference, so
    # phi = (L(-4.5), L(4.5), L(4.5), L(-4.5)) with L the logistic function.
    x = np.array([[1.0, -2.0, 0.5]])
    w = np.array([[0.5, 1.0, -1.0], [2.0, 0.0, 1.0]])
    ph = oracle.phi(x, w)[0]
    lo, hi = sp.expit(-4.5), sp.expit(4.5)
    np.testing.assert_allclose(ph, [lo, hi, hi, lo], rtol=1e-14, atol=0)


@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_phi_matches_library_softmax(d, fw, _b):
    rng = _rng(4)
    x = rng.standard_normal((6, d))
    w = _w(rng, fw, d, 3.0)
    ph = oracle.phi(x, w)
    u = x @ w.T
    np.testing.assert_allclose(ph[:, :fw], sp.softmax(u, axis=1), rtol=1e-12, atol=0)
    np.testing.assert_allclose(ph[:, fw:], sp.softmax(-u, axis=1), rtol=1e-12, atol=0)


# ---------------------------------------------------------------- state
@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_normaliser_halves_count_tokens(d, fw, _b):
    rng = _rng(5)
    n = 37
    S, Z = oracle.state_build(rng.standard_normal((n, d)), rng.standard_normal((n, d)),
                              _w(rng, fw, d))
    assert S.shape == (2 * fw, d) and Z.shape == (2 * fw,)
    assert abs(Z[:fw].sum() - n) < n * 1e-14
    assert abs(Z[fw:].sum() - n) < n * 1e-14


@pytest.mark.parametrize("d,fw,b", SHAPES)
def test_incremental_commits_equal_one_shot_build(d, fw, b):
    rng = _rng(6)
    nblk = 6
    k = rng.standard_normal((nblk * b, d))
    v = rng.standard_normal((nblk * b, d))
    w = _w(rng, fw, d)
    S1, Z1 = oracle.state_build(k, v, w)
    S2 = np.zeros_like(S1)
    Z2 = np.zeros_like(Z1)
    for i in range(nblk):
        oracle.state_commit(S2, Z2, k[i * b:(i + 1) * b], v[i * b:(i + 1) * b], w)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Z2, Z1, rtol=1e-12, atol=1e-13)


def test_state_is_order_invariant():
    rng = _rng(7)
    k, v = rng.standard_normal((20, 6)), rng.standard_normal((20, 6))
    w = _w(rng, 3, 6)
    p = rng.permutation(20)
    S1, Z1 = oracle.state_build(k, v, w)
    S2, Z2 = oracle.state_build(k[p], v[p], w)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Z2, Z1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_single_token_state_reads_back_its_value(d, fw, _b):
    # With one committed token, phi(q)^T S / phi(q)^T Z = v_1 for any query.
    rng = _rng(8)
    k1, v1 = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    w = _w(rng, fw, d)
    S, Z = oracle.state_build(k1, v1, w)
    for q in rng.standard_normal((4, d)):
        pq = oracle.phi(q[None], w)[0]
        np.testing.assert_allclose((pq @ S) / (pq @ Z), v1[0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("d,fw,_b", SHAPES)
def test_state_read_equals_bruteforce_over_prior_tokens(d, fw, _b):
    # The state read phi(q)^T S, phi(q)^T Z equals the sums over every prior
    # token of (phi(q) . phi(k_t)) v_t and phi(q) . phi(k_t) (the linear
    # attention kernel trick run in reverse), computed token by token here.
    rng = _rng(9)
    n = 29
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = _w(rng, fw, d, 2.0)
    S, Z = oracle.state_build(k, v, w)
    q = rng.standard_normal((3, d))
    pq = oracle.phi(q, w)
    pk = oracle.phi(k, w)
    for i in range(3):
        num = np.zeros(d)
        den = 0.0
        for t in range(n):
            kap = float(np.dot(pq[i], pk[t]))
            num += kap * v[t]
            den += kap
        np.testing.assert_allclose(pq[i] @ S, num, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(pq[i] @ Z, den, rtol=1e-12, atol=0)


# ---------------------------------------------------------------- forward
def _sdpa(q, k, v, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]  # noqa: E731
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    return out[0, 0].numpy()


def _case(rng, d, fw, b, n):
    q, k, v = (rng.standard_normal((b, d)) for _ in range(3))
    kp, vp = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = _w(rng, fw, d, 2.0)
    S, Z = oracle.state_build(kp, vp, w)
    return q, k, v, kp, vp, w, S, Z


@pytest.mark.parametrize("d,fw,b", SHAPES)
def test_gate_zero_is_block_softmax_attention(d, fw, b):
    rng = _rng(10)
    q, k, v, _, _, w, S, Z = _case(rng, d, fw, b, 16)
    y = oracle.block_forward(q, k, v, w, 0.0, S, Z)
    np.testing.assert_allclose(y, _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d,fw,b", SHAPES)
def test_empty_state_is_block_softmax_attention(d, fw, b):
    rng = _rng(11)
    q, k, v, _, _, w, S, Z = _case(rng, d, fw, b, 16)
    y = oracle.block_forward(q, k, v, w, 0.7, np.zeros_like(S), np.zeros_like(Z))
    np.testing.assert_allclose(y, _sdpa(q, k, v), rtol=1e-12, atol=1e-13)


def test_explicit_softmax_scale_is_used():
    rng = _rng(12)
    q, k, v, _, _, w, S, Z = _case(rng, 8, 4, 6, 10)
    y = oracle.block_forward(q, k, v, w, 0.0, S, Z, scale=0.3)
    np.testing.assert_allclose(y, _sdpa(q, k, v, scale=0.3), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("d,fw,b", SHAPES)
@pytest.mark.parametrize("gamma", [0.5, 3.0])
def test_forward_equals_bruteforce_over_prefix(d, fw, b, gamma):
    # No state and no row maximum: y_i = (sum_j e^{s_ij} v_j + g sum_t kap_it v_t)
    # / (sum_j e^{s_ij} + g sum_t kap_it), kap_it = phi(q_i) . phi(k_t), summed
    # token by token over the whole prefix. Equal in exact arithmetic to the
    # stabilised form the oracle evaluates.
    rng = _rng(13)
    n = 3 * b + 2
    q, k, v, kp, vp, w, S, Z = _case(rng, d, fw, b, n)
    y = oracle.block_forward(q, k, v, w, gamma, S, Z)
    pq, pk = oracle.phi(q, w), oracle.phi(kp, w)
    c = 1.0 / np.sqrt(d)
    for i in range(b):
        num = np.zeros(d)
        den = 0.0
        for j in range(b):
            e = np.exp(c * np.dot(q[i], k[j]))
            num += e * v[j]
            den += e
        for t in range(n):
            kap = float(np.dot(pq[i], pk[t]))
            num += gamma * kap * vp[t]
            den += gamma * kap
        np.testing.assert_allclose(y[i], num / den, rtol=1e-11, atol=1e-13)


def test_constant_values_give_constant_output():
    rng = _rng(14)
    d, fw, b, n = 8, 4, 5, 20
    q, k = rng.standard_normal((b, d)), rng.standard_normal((b, d))
    kp = rng.standard_normal((n, d))
    cval = rng.standard_normal(d)
    v = np.tile(cval, (b, 1))
    vp = np.tile(cval, (n, 1))
    w = _w(rng, fw, d, 2.0)
    S, Z = oracle.state_build(kp, vp, w)
    y = oracle.block_forward(q, k, v, w, 2.5, S, Z)
    np.testing.assert_allclose(y, np.tile(cval, (b, 1)), rtol=1e-12, atol=1e-13)


def test_output_in_convex_hull_of_values():
    rng = _rng(15)
    d, fw, b, n = 6, 3, 4, 12
    q, k, v, kp, vp, w, S, Z = _case(rng, d, fw, b, n)
    y = oracle.block_forward(q, k, v, w, 1.3, S, Z)
    allv = np.concatenate([v, vp])
    assert np.all(y <= allv.max(0) + 1e-12)
    assert np.all(y >= allv.min(0) - 1e-12)


def test_large_gate_limit_is_normalised_linear_attention():
    rng = _rng(16)
    d, fw, b, n = 8, 4, 3, 15
    q, k, v, _, _, w, S, Z = _case(rng, d, fw, b, n)
    y = oracle.block_forward(q, k, v, w, 1e30, S, Z)
    pq = oracle.phi(q, w)
    np.testing.assert_allclose(y, (pq @ S) / (pq @ Z)[:, None], rtol=1e-12, atol=1e-14)


def test_zero_matrix_closed_form():
    # W = 0: phi = 1/FW in every entry, phi(q) . phi(k) = 2/FW = 4/F, so the
    # linear branch is (4/F) sum_t v_t over (4/F) N.
    rng = _rng(17)
    d, fw, b, n, g = 6, 3, 4, 10, 0.8
    q, k, v = (rng.standard_normal((b, d)) for _ in range(3))
    kp, vp = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    w = np.zeros((fw, d))
    S, Z = oracle.state_build(kp, vp, w)
    y = oracle.block_forward(q, k, v, w, g, S, Z)
    s = (q @ k.T) / np.sqrt(d)
    F = 2 * fw
    for i in range(b):
        m = s[i].max()
        a = np.exp(s[i] - m)
        num = a @ v + g * np.exp(-m) * (4.0 / F) * vp.sum(0)
        den = a.sum() + g * np.exp(-m) * (4.0 / F) * n
        np.testing.assert_allclose(y[i], num / den, rtol=1e-12, atol=1e-14)


def test_state_and_gate_rescaling_invariance():
    rng = _rng(18)
    q, k, v, _, _, w, S, Z = _case(rng, 8, 4, 5, 11)
    y1 = oracle.block_forward(q, k, v, w, 0.9, S, Z)
    y2 = oracle.block_forward(q, k, v, w, 0.9 / 7.0, 7.0 * S, 7.0 * Z)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-14)


def test_single_token_block_closed_form():
    rng = _rng(19)
    d, fw = 8, 4
    q, k, v, _, _, w, S, Z = _case(rng, d, fw, 1, 9)
    g = 0.6
    y = oracle.block_forward(q, k, v, w, g, S, Z)
    s = float(q[0] @ k[0]) / np.sqrt(d)
    pq = oracle.phi(q, w)[0]
    ref = (v[0] + g * np.exp(-s) * (pq @ S)) / (1.0 + g * np.exp(-s) * (pq @ Z))
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- batched drivers
def test_batched_forward_matches_pairs():
    rng = _rng(20)
    R, H, B, d, fw = 3, 2, 4, 8, 4
    q, k, v = (rng.standard_normal((R, H, B, d)) for _ in range(3))
    w = rng.standard_normal((H, fw, d)) / np.sqrt(d)
    gamma = rng.random(H)
    S = rng.random((R, H, 2 * fw, d))
    Z = rng.random((R, H, 2 * fw)) + 1.0
    out = oracle.block_forward_batch(q, k, v, w, gamma, S, Z, nthreads=3)
    for r in range(R):
        for h in range(H):
            ref = oracle.block_forward(q[r, h], k[r, h], v[r, h], w[h], gamma[h], S[r, h], Z[r, h])
            np.testing.assert_array_equal(out[r, h], ref)


def test_batched_commit_matches_pairs():
    rng = _rng(21)
    R, H, B, d, fw = 2, 3, 5, 6, 3
    k, v = rng.standard_normal((R, H, B, d)), rng.standard_normal((R, H, B, d))
    w = rng.standard_normal((H, fw, d)) / np.sqrt(d)
    S = rng.random((R, H, 2 * fw, d))
    Z = rng.random((R, H, 2 * fw))
    S0, Z0 = S.copy(), Z.copy()
    oracle.state_commit_batch(S, Z, k, v, w, nthreads=4)
    for r in range(R):
        for h in range(H):
            s1, z1 = S0[r, h].copy(), Z0[r, h].copy()
            oracle.state_commit(s1, z1, k[r, h], v[r, h], w[h])
            np.testing.assert_array_equal(S[r, h], s1)
            np.testing.assert_array_equal(Z[r, h], z1)


# ---------------------------------------------------------------- softmax prefix attention
@pytest.mark.parametrize("d,b,n", [(8, 4, 0), (8, 4, 13), (16, 1, 5), (6, 7, 40)])
def test_prefix_attention_is_softmax_attention_over_prefix_and_block(d, b, n):
    # one softmax over the prefix keys followed by the block's keys, no mask:
    # PyTorch's CPU attention on the concatenated keys and values
    rng = _rng(30)
    q, k, v = (rng.standard_normal((b, d)) for _ in range(3))
    kp, vp = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    y = oracle.prefix_attention(q, k, v, kp, vp)
    ref = _sdpa(q, np.concatenate([kp, k]), np.concatenate([vp, v]))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_prefix_attention_is_order_invariant_over_prefix():
    rng = _rng(31)
    q, k, v = (rng.standard_normal((3, 8)) for _ in range(3))
    kp, vp = rng.standard_normal((9, 8)), rng.standard_normal((9, 8))
    p = rng.permutation(9)
    np.testing.assert_allclose(oracle.prefix_attention(q, k, v, kp[p], vp[p]),
                               oracle.prefix_attention(q, k, v, kp, vp), rtol=1e-12, atol=1e-14)


def test_prefix_attention_explicit_scale_and_constant_values():
    rng = _rng(32)
    q, k = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    kp = rng.standard_normal((6, 8))
    cval = rng.standard_normal(8)
    y = oracle.prefix_attention(q, k, np.tile(cval, (4, 1)), kp, np.tile(cval, (6, 1)), scale=0.25)
    np.testing.assert_allclose(y, np.tile(cval, (4, 1)), rtol=1e-12, atol=1e-13)
    kp2, vp2 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    v = rng.standard_normal((4, 8))
    y2 = oracle.prefix_attention(q, k, v, kp2, vp2, scale=0.25)
    np.testing.assert_allclose(y2, _sdpa(q, np.concatenate([kp2, k]), np.concatenate([vp2, v]), scale=0.25),
                               rtol=1e-12, atol=1e-13)
