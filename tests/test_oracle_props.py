"""Property tests of the fp64 oracle over tiny random shapes (no GPU).

Hypothesis draws the shape (d in {4, 8}, FW in {2, 4}, B in {1, 2, 3, 8},
prefix length N in 0..40), the input scale and a seed; every property is one
the definitions fix independently of how the oracle evaluates them:
* phi: both halves positive and summing to 1; phi(-x) swaps the halves
  (pith.science review, "What carries the argument": phi(x) = [softmax(xW),
  softmax(-xW)]).
* state: each half of Z sums to the number of committed tokens; commits of
  any partition of the prefix into blocks equal one build over all of it
  (gist.science explainer, "Architecture Design": the states are sums over the
  committed tokens, changed only at a commit).
* forward: gate 0 or an empty state gives softmax attention within the block
  (scipy's softmax on the logits); the result equals the sum over every prior
  token of (phi(q) . phi(k_t)) v_t with no state and no row maximum; each
  output coordinate lies between the smallest and largest value of the
  tokens it averages; (S, Z, gamma) -> (lam S, lam Z, gamma / lam) leaves it
  unchanged.
"""
import numpy as np
import scipy.special as sp
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None)


@st.composite
def shapes(draw):
    d = draw(st.sampled_from([4, 8]))
    fw = draw(st.sampled_from([2, 4]))
    b = draw(st.sampled_from([1, 2, 3, 8]))
    n = draw(st.integers(0, 40))
    scale = draw(st.floats(0.1, 3.0))
    seed = draw(st.integers(0, 2**31 - 1))
    return d, fw, b, n, scale, seed


def _draw(d, fw, b, n, scale, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((b, d)) * scale for _ in range(3))
    kp, vp = rng.standard_normal((n, d)) * scale, rng.standard_normal((n, d))
    w = rng.standard_normal((fw, d)) * scale / np.sqrt(d)
    return rng, q, k, v, kp, vp, w


@SETTINGS
@given(shapes())
def test_phi_halves_and_sign_symmetry(sh):
    d, fw, b, n, scale, seed = sh
    _, q, _, _, _, _, w = _draw(*sh)
    ph, ng = oracle.phi(q, w), oracle.phi(-q, w)
    assert np.all(ph > 0)
    np.testing.assert_allclose(ph[:, :fw].sum(1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ph[:, fw:].sum(1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ng[:, :fw], ph[:, fw:], rtol=1e-13, atol=0)
    np.testing.assert_allclose(ng[:, fw:], ph[:, :fw], rtol=1e-13, atol=0)


@SETTINGS
@given(shapes())
def test_state_counts_tokens_and_ignores_block_boundaries(sh):
    d, fw, b, n, scale, seed = sh
    rng, _, _, _, kp, vp, w = _draw(*sh)
    S1, Z1 = oracle.state_build(kp, vp, w)
    assert abs(Z1[:fw].sum() - n) <= 1e-13 * max(n, 1)
    assert abs(Z1[fw:].sum() - n) <= 1e-13 * max(n, 1)
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(3, max(n - 1, 0)), replace=False)) if n > 1 else []
    S2, Z2 = np.zeros_like(S1), np.zeros_like(Z1)
    for a, c in zip(np.concatenate([[0], cuts]).astype(int), np.concatenate([cuts, [n]]).astype(int)):
        oracle.state_commit(S2, Z2, kp[a:c], vp[a:c], w)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Z2, Z1, rtol=1e-12, atol=1e-13)


def _block_softmax(q, k, v):
    s = q @ k.T / np.sqrt(q.shape[1])
    return sp.softmax(s, axis=1) @ v


@SETTINGS
@given(shapes(), st.floats(0.0, 5.0))
def test_gate_zero_and_empty_state_are_block_softmax(sh, gamma):
    _, q, k, v, kp, vp, w = _draw(*sh)
    S, Z = oracle.state_build(kp, vp, w)
    ref = _block_softmax(q, k, v)
    np.testing.assert_allclose(oracle.block_forward(q, k, v, w, 0.0, S, Z), ref, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(oracle.block_forward(q, k, v, w, gamma, np.zeros_like(S), np.zeros_like(Z)), ref,
                               rtol=1e-11, atol=1e-13)


@SETTINGS
@given(shapes(), st.floats(0.01, 10.0))
def test_forward_is_bruteforce_hybrid_attention(sh, gamma):
    d, fw, b, n, scale, seed = sh
    _, q, k, v, kp, vp, w = _draw(*sh)
    S, Z = oracle.state_build(kp, vp, w)
    y = oracle.block_forward(q, k, v, w, gamma, S, Z)
    pq, pk = oracle.phi(q, w), oracle.phi(kp, w) if n else np.zeros((0, 2 * fw))
    e = np.exp(q @ k.T / np.sqrt(d))     # [B][B], no row maximum
    kap = pq @ pk.T                      # [B][N]
    ref = (e @ v + gamma * kap @ vp) / (e.sum(1) + gamma * kap.sum(1))[:, None]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)
    allv = np.concatenate([v, vp])
    assert np.all(y <= allv.max(0) + 1e-12) and np.all(y >= allv.min(0) - 1e-12)


@SETTINGS
@given(shapes(), st.floats(0.01, 10.0), st.floats(0.05, 20.0))
def test_state_and_gate_rescaling(sh, gamma, lam):
    _, q, k, v, kp, vp, w = _draw(*sh)
    S, Z = oracle.state_build(kp, vp, w)
    y1 = oracle.block_forward(q, k, v, w, gamma, S, Z)
    y2 = oracle.block_forward(q, k, v, w, gamma / lam, lam * S, lam * Z)
    np.testing.assert_allclose(y2, y1, rtol=1e-11, atol=1e-13)
