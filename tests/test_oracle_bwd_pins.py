"""Pins of the oracle's backward pass (oracle.attention_backward) against
things other than itself: central differences of the forward oracle, float64
autograd through torch's scaled_dot_product_attention, closed forms, and
identities the gradients of attention obey. The backward's definition is the
one of "Flash attention in PyTorch, then in Triton", section "Backwards, and
training with it"."""
import numpy as np
import pytest
import torch

import oracle


def grid_inputs(shape, seed, step=2.0 ** -6, lim=2.0):
    """Random values on a coarse binary grid, so that +-h perturbations with
    h a small power of two are exact in float32."""
    rng = np.random.default_rng(seed)
    x = rng.uniform(-lim, lim, size=shape)
    return (np.round(x / step) * step).astype(np.float32)


def loss(q, k, v, dout, causal, scale):
    o, _ = oracle.attention(q, k, v, causal, scale)
    return float(np.sum(o * dout.astype(np.float64)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,D,scale", [(1, 3, 0.37), (4, 5, 0.37), (9, 8, -0.29)])
def test_central_differences(T, D, scale, causal):
    """dL/dx of L = sum(O * dO), by a fourth-order central difference of the
    forward oracle on every input element, matches the backward."""
    shape = (1, 2, T, D)
    q, k, v = (grid_inputs(shape, s) for s in (11, 12, 13))
    dout = grid_inputs(shape, 14)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal, scale)
    h = 2.0 ** -8
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(g)
        for idx in np.ndindex(*shape):
            vals = []
            for step in (h, -h, 2 * h, -2 * h):
                y = x.copy()
                y[idx] += np.float32(step)
                args = {"q": q, "k": k, "v": v}
                args[name] = y
                vals.append(loss(args["q"], args["k"], args["v"], dout, causal, scale))
            num[idx] = (8 * (vals[0] - vals[1]) - (vals[2] - vals[3])) / (12 * h)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8, err_msg=f"d{name}")


def torch_grads(q, k, v, dout, causal, scale):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    return [g.numpy() for g in torch.autograd.grad(o, (tq, tk, tv),
                                                   torch.tensor(dout, dtype=torch.float64))]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T,scale", [(1, 0.125), (100, 0.125), (256, 0.3)])
def test_float64_autograd(T, scale, causal):
    """float64 autograd through torch's SDPA on the two-sequence, three-head
    shapes of the page's test agrees with the oracle's gradients."""
    shape = (2, 3, T, 64)
    rng = np.random.default_rng(T)
    q, k, v, dout = (rng.standard_normal(shape).astype(np.float32) for _ in range(4))
    ours = oracle.attention_backward(q, k, v, dout, causal, scale)
    theirs = torch_grads(q, k, v, dout, causal, scale)
    for name, a, b in zip("qkv", ours, theirs):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11 * max(1.0, np.abs(b).max()),
                                   err_msg=f"d{name}")


def test_single_token_closed_form():
    """T = 1: the one weight is exactly 1, so dV = dO and dQ = dK = 0."""
    rng = np.random.default_rng(5)
    q, k, v, dout = (rng.standard_normal((2, 3, 1, 64)).astype(np.float32) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal, 0.125)
        assert np.array_equal(dv, dout.astype(np.float64))
        assert np.array_equal(dq, np.zeros_like(dq))
        assert np.array_equal(dk, np.zeros_like(dk))


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0: uniform weights 1/|J_i|, so dV_j = sum of dO_i / |J_i| over the
    rows that see key j, and dK = 0."""
    T, D = 37, 64
    rng = np.random.default_rng(6)
    q = np.zeros((T, D), np.float32)
    k, v, dout = (rng.standard_normal((T, D)).astype(np.float32) for _ in range(3))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal, 0.125)
    want = np.zeros((T, D))
    for i in range(T):
        n = i + 1 if causal else T
        for j in range(n):
            want[j] += dout[i].astype(np.float64) / n
    np.testing.assert_allclose(dv, want, rtol=1e-13, atol=1e-13)
    assert np.array_equal(dk, np.zeros_like(dk))
    # and dQ_i = scale * sum_j (1/n) (dO_i.v_j - dO_i.O_i) k_j, O_i the mean
    scale = 0.125
    dq_want = np.zeros((T, D))
    for i in range(T):
        n = i + 1 if causal else T
        vv = v[:n].astype(np.float64)
        o = vv.mean(axis=0)
        ds = (vv @ dout[i].astype(np.float64) - o @ dout[i].astype(np.float64)) / n
        dq_want[i] = scale * ds @ k[:n].astype(np.float64)
    np.testing.assert_allclose(dq, dq_want, rtol=1e-11, atol=1e-12)


def random_case(seed, shape=(2, 2, 33, 16)):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(shape).astype(np.float32) for _ in range(4)]


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """Adding one vector to every key shifts each row's scores by a constant,
    which the softmax ignores; so the key gradients of a slice sum to 0."""
    q, k, v, dout = random_case(21)
    _, dk, _ = oracle.attention_backward(q, k, v, dout, causal, 0.3)
    total = dk.sum(axis=2)
    assert np.abs(total).max() < 1e-12 * max(1.0, np.abs(dk).max()) * dk.shape[2]


@pytest.mark.parametrize("causal", [False, True])
def test_value_gradient_independent_of_values(causal):
    """dV = P^T dO involves no V: another V gives the same dV."""
    q, k, v, dout = random_case(22)
    v2 = random_case(23)[2]
    dv1 = oracle.attention_backward(q, k, v, dout, causal, 0.3)[2]
    dv2 = oracle.attention_backward(q, k, v2, dout, causal, 0.3)[2]
    assert np.array_equal(dv1, dv2)


@pytest.mark.parametrize("causal", [False, True])
def test_value_affine(causal):
    """V -> a V + b (b one row added to every value row) scales dS, hence dQ
    and dK, by a, and leaves dV alone. Values on a 2^-10 grid keep a V + b
    exact in float32."""
    q, k, v, dout = random_case(24)
    v = np.round(v * 1024) / 1024
    b = np.round(np.random.default_rng(25).standard_normal(16) * 64) / 64
    a = 2.5
    v2 = (a * v + b).astype(np.float32)
    assert np.array_equal(v2.astype(np.float64), a * v.astype(np.float64) + b)
    g1 = oracle.attention_backward(q, k, v, dout, causal, 0.3)
    g2 = oracle.attention_backward(q, k, v2, dout, causal, 0.3)
    np.testing.assert_allclose(g2[0], a * g1[0], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g2[1], a * g1[1], rtol=1e-9, atol=1e-12)
    assert np.array_equal(g2[2], g1[2])


@pytest.mark.parametrize("causal", [False, True])
def test_query_key_gradient_identity(causal):
    """sum_i q_i.dQ_i = scale sum_ij dS_ij q_i.k_j = sum_j k_j.dK_j for each
    slice (a transposed operand or a lost scale breaks it)."""
    q, k, v, dout = random_case(26)
    dq, dk, _ = oracle.attention_backward(q, k, v, dout, causal, 0.3)
    lhs = np.einsum("bhtd,bhtd->bh", q.astype(np.float64), dq)
    rhs = np.einsum("bhtd,bhtd->bh", k.astype(np.float64), dk)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-11, atol=1e-12)
    assert np.abs(lhs).min() > 1e-3  # not trivially zero


def test_causal_rows_do_not_see_later_rows():
    """Causal: dQ_i uses only rows <= i of q, k, v and dO."""
    q, k, v, dout = random_case(27)
    r = 20
    q2, k2, v2, d2 = (x.copy() for x in (q, k, v, dout))
    rng = np.random.default_rng(28)
    for x in (q2, k2, v2, d2):
        x[:, :, r + 1:] = rng.standard_normal(x[:, :, r + 1:].shape)
    dq1 = oracle.attention_backward(q, k, v, dout, True, 0.3)[0]
    dq2 = oracle.attention_backward(q2, k2, v2, d2, True, 0.3)[0]
    assert np.array_equal(dq1[:, :, : r + 1], dq2[:, :, : r + 1])
    assert not np.array_equal(dq1[:, :, r + 1:], dq2[:, :, r + 1:])


def test_slices_subset_matches_full():
    """Selected slices equal the same slices of the full computation."""
    q, k, v, dout = random_case(29, shape=(2, 3, 17, 8))
    full = oracle.attention_backward(q, k, v, dout, True, 0.3)
    sel = np.array([4, 1])
    part = oracle.attention_backward(q, k, v, dout, True, 0.3, slices=sel)
    for a, b in zip(full, part):
        flat = a.reshape(6, 17, 8)
        assert np.array_equal(flat[sel], b)
