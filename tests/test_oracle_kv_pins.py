"""Pins of the oracle's decode function (oracle.attention_kv: Tq new queries
against a Tk-token key/value cache, the causal mask aligned to the
bottom-right) against things other than itself: the independently pinned
full-sequence oracle, float64 torch SDPA with an explicit mask, and closed
forms."""
import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("Tq,Tk", [(1, 1), (1, 9), (4, 33), (17, 17), (40, 200)])
def test_last_rows_of_a_causal_sequence(Tq, Tk):
    """A causal decode of the last Tq tokens equals those rows of causal
    attention over the whole sequence (the query at position Tk - Tq + i)."""
    qf, k, v = rand((2, 3, Tk, 16), 1), rand((2, 3, Tk, 16), 2), rand((2, 3, Tk, 16), 3)
    o_full, l_full = oracle.attention(qf, k, v, True, 0.3)
    o, l = oracle.attention_kv(np.ascontiguousarray(qf[:, :, Tk - Tq:]), k, v, True, 0.3)
    assert np.array_equal(o, o_full[:, :, Tk - Tq:])
    assert np.array_equal(l, l_full[:, :, Tk - Tq:])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(1, 100), (7, 100), (64, 256), (100, 100)])
def test_float64_sdpa_with_explicit_mask(Tq, Tk, causal):
    """float64 scaled_dot_product_attention with the bottom-right mask written
    out as a boolean table, and logsumexp of the masked scores."""
    q, k, v = rand((2, 3, Tq, 64), 4), rand((2, 3, Tk, 64), 5), rand((2, 3, Tk, 64), 6)
    o, lse = oracle.attention_kv(q, k, v, causal, 0.125)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    i = torch.arange(Tq)[:, None]
    j = torch.arange(Tk)[None, :]
    mask = (j <= Tk - Tq + i) if causal else torch.ones(Tq, Tk, dtype=torch.bool)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=0.125)
    s = 0.125 * tq @ tk.transpose(-1, -2)
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_single_key_closed_form():
    """Tk = 1 (so Tq = 1): the one weight is 1, O = V and lse = the score."""
    q, k, v = rand((2, 2, 1, 64), 7), rand((2, 2, 1, 64), 8), rand((2, 2, 1, 64), 9)
    for causal in (False, True):
        o, lse = oracle.attention_kv(q, k, v, causal, 0.25)
        assert np.array_equal(o, v.astype(np.float64))
        want = 0.25 * np.einsum("bhqd,bhkd->bhq", q.astype(np.float64), k.astype(np.float64))
        np.testing.assert_allclose(lse, want, rtol=0, atol=1e-13)


def test_one_new_token_sees_the_whole_cache():
    """Tq = 1: the new token is the last one, so the causal mask hides
    nothing and both masks agree."""
    q, k, v = rand((1, 4, 1, 32), 10), rand((1, 4, 57, 32), 11), rand((1, 4, 57, 32), 12)
    a = oracle.attention_kv(q, k, v, True, 0.2)
    b = oracle.attention_kv(q, k, v, False, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rejects_more_queries_than_keys():
    with pytest.raises(RuntimeError):
        oracle.attention_kv(rand((1, 1, 5, 8), 1), rand((1, 1, 4, 8), 2),
                            rand((1, 1, 4, 8), 3), True, 0.3)
