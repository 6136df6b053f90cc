"""Pins of the oracle's gated linear recurrence (oracle.gated_recurrence)
against things other than itself: the recurrence unrolled into a closed-form
sum over earlier steps with gate products, causal linear attention (gate 1)
through a float64 library matmul, a hand-computed scalar example, and
structural properties (causality, column independence, linearity).

The recurrence is the one the POPCORNBENCH transcript "Kimi-K2.6 l2 p24"
analyses: per (batch, head) a D x D state from zero; at each step the gate
scales every column j of the state and the outer product k_t v_t^T is added,
then y_t = q_t^T S_t. Unrolled, y[t, j] = sum over tau <= t of
(q_t . k_tau) v_tau[j] times the product of gate[p, j] for tau < p <= t.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_amd.inputs import make_gated


def closed_form(q, k, v, g):
    """The unrolled sum, written directly (numpy float64, explicit loops)."""
    q, k, v, g = (np.asarray(x, np.float64) for x in (q, k, v, g))
    B, T, H, D = q.shape
    y = np.zeros((B, T, H, D))
    for b in range(B):
        for h in range(H):
            for t in range(T):
                for tau in range(t + 1):
                    dot = float(np.dot(q[b, t, h], k[b, tau, h]))
                    decay = np.prod(g[b, tau + 1:t + 1, h], axis=0)  # ones if empty
                    y[b, t, h] += dot * v[b, tau, h] * decay
    return y


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (2, 9, 3, 5), (1, 17, 2, 8), (2, 6, 4, 24)])
def test_closed_form(shape):
    q, k, v, g = make_gated(*shape, seed=sum(shape))
    y = oracle.gated_recurrence(q, k, v, g)
    want = closed_form(q, k, v, g)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_hand_computed_scalar():
    """D = 1, T = 3: s_t = g_t s_{t-1} + k_t v_t, y_t = q_t s_t, with values
    exact in binary: s = 2, 4, 3 and y = 2, 8, 9."""
    q = np.array([1, 2, 3], np.float32).reshape(1, 3, 1, 1)
    k = np.array([1, 1, 2], np.float32).reshape(1, 3, 1, 1)
    v = np.array([2, 3, 1], np.float32).reshape(1, 3, 1, 1)
    g = np.array([0.5, 0.5, 0.25], np.float32).reshape(1, 3, 1, 1)
    y = oracle.gated_recurrence(q, k, v, g)
    assert np.array_equal(y.reshape(-1), [2.0, 8.0, 9.0])


@pytest.mark.parametrize("T", [1, 40, 130])
def test_unit_gate_is_causal_linear_attention(T):
    """gate = 1: the state is the running sum of outer products, so y =
    tril(Q K^T) V per (batch, head), by float64 torch matmul."""
    q, k, v, _ = make_gated(2, T, 3, 16, seed=300 + T)
    g = torch.ones_like(q)
    y = oracle.gated_recurrence(q, k, v, g)
    qh, kh, vh = (x.double().permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    s = torch.tril(qh @ kh.transpose(-1, -2).contiguous())
    want = (s @ vh).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(y, want, rtol=1e-11, atol=1e-11)


def test_zero_gate_keeps_only_the_current_step():
    """gate = 0: the state forgets everything before the step, so y_t =
    (q_t . k_t) v_t."""
    q, k, v, _ = make_gated(2, 11, 3, 7, seed=310)
    y = oracle.gated_recurrence(q, k, v, torch.zeros_like(q))
    dot = (q.double() * k.double()).sum(-1, keepdim=True)
    np.testing.assert_allclose(y, (dot * v.double()).numpy(), rtol=1e-14, atol=1e-14)


def test_causal():
    """y_t depends on steps <= t only."""
    q, k, v, g = make_gated(1, 20, 2, 6, seed=320)
    y1 = oracle.gated_recurrence(q, k, v, g)
    q2, k2, v2, g2 = (x.clone() for x in (q, k, v, g))
    r = make_gated(1, 20, 2, 6, seed=321)
    for a, b in zip((q2, k2, v2, g2), r):
        a[:, 12:] = b[:, 12:]
    y2 = oracle.gated_recurrence(q2, k2, v2, g2)
    assert np.array_equal(y1[:, :12], y2[:, :12])
    assert not np.array_equal(y1[:, 12:], y2[:, 12:])


def test_columns_independent():
    """Output column j reads only column j of v and of the gate: changing
    every other column of both leaves it unchanged."""
    q, k, v, g = make_gated(2, 15, 2, 6, seed=330)
    j = 3
    y1 = oracle.gated_recurrence(q, k, v, g)
    _, _, v2, g2 = make_gated(2, 15, 2, 6, seed=331)
    v2[..., j], g2[..., j] = v[..., j], g[..., j]
    y2 = oracle.gated_recurrence(q, k, v2, g2)
    assert np.array_equal(y1[..., j], y2[..., j])
    assert not np.array_equal(y1[..., :j], y2[..., :j])


def test_heads_and_batches_independent():
    """Permuting heads (and batches) permutes the outputs the same way."""
    q, k, v, g = make_gated(3, 10, 4, 5, seed=340)
    y = oracle.gated_recurrence(q, k, v, g)
    perm_h, perm_b = [2, 0, 3, 1], [1, 2, 0]
    xs = [x[perm_b][:, :, perm_h].contiguous() for x in (q, k, v, g)]
    yp = oracle.gated_recurrence(*xs)
    assert np.array_equal(yp, y[perm_b][:, :, perm_h])


def test_linear_in_values_and_queries():
    """y is linear in v (for fixed q, k, gate) and in q; doubling is exact.
    Values on a 2^-10 grid keep v + v2 exact in float32."""
    q, k, v, g = make_gated(1, 25, 2, 8, seed=350)
    _, _, v2, _ = make_gated(1, 25, 2, 8, seed=351)
    v, v2 = (torch.round(x * 1024) / 1024 for x in (v, v2))
    assert torch.equal((v + v2).double(), v.double() + v2.double())
    ya = oracle.gated_recurrence(q, k, v, g)
    yb = oracle.gated_recurrence(q, k, v2, g)
    yab = oracle.gated_recurrence(q, k, v + v2, g)
    np.testing.assert_allclose(yab, ya + yb, rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.gated_recurrence(2 * q, k, v, g), 2 * ya)
    assert np.array_equal(oracle.gated_recurrence(q, k, 2 * v, g), 2 * ya)


def test_rejects_mismatched_shapes():
    q, k, v, g = make_gated(1, 4, 1, 3, seed=1)
    with pytest.raises(ValueError):
        oracle.gated_recurrence(q, k, v, g[:, :3])
