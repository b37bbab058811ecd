"""Pins of the gradient oracle (oracle/backward_oracle.py).

Its forward is pinned to the numpy oracle; its gradient to finite differences
(torch.autograd.gradcheck: the derivative's definition) and, where the method
reduces to softmax attention (every block exact, or blocks of one token), to
the gradients of the library's dense attention.
"""

import math

import numpy as np
import pytest
import torch

from oracle import backward_oracle as BO
from oracle import pisa_oracle as O


def rand(T, D, seed):
    r = np.random.default_rng(seed)
    return [r.standard_normal((T, D)) for _ in range(4)]


@pytest.mark.parametrize("T,B,topk,band,n_sink,so,fo", [
    (300, 64, 2, 1, 0, False, True), (300, 64, 1, 0, 2, True, True), (256, 32, 3, 1, 1, True, False),
    (77, 16, 2, 1, 0, False, False)])
def test_torch_forward_equals_numpy_oracle(T, B, topk, band, n_sink, so, fo):
    q, k, v, _ = rand(T, 8, T + B)
    s = 0.4
    o, parts = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=topk, band=band, n_sink=n_sink,
                                   second_order=so, first_order="global" if fo else "none",
                                   return_parts=True)
    keep = parts["w"] <= math.log(B) if so else None
    t = [torch.tensor(x) for x in (q, k, v)]
    ot = BO.forward_torch(*t, parts["idx"], B=B, scale=s, band=band, n_sink=n_sink, second_order=so,
                          first_order=fo, gate_keep=keep)
    np.testing.assert_allclose(ot.numpy(), o, rtol=0, atol=1e-12)


@pytest.mark.parametrize("so,fo,n_sink", [(False, True, 0), (True, True, 1), (True, False, 0)])
def test_gradcheck_finite_differences(so, fo, n_sink):
    T, B, D = 40, 8, 4
    q, k, v, _ = rand(T, D, 11)
    s = 0.7
    _, parts = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=1, band=0, n_sink=n_sink,
                                   second_order=so, return_parts=True)
    keep = parts["w"] <= math.log(B) if so else None
    idx = parts["idx"]
    f = lambda a, b, c: BO.forward_torch(a, b, c, idx, B=B, scale=s, band=0, n_sink=n_sink,
                                         second_order=so, first_order=fo, gate_keep=keep)
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    assert torch.autograd.gradcheck(f, t, eps=1e-6, atol=1e-6, rtol=1e-5)


def dense_grads(q, k, v, do, s):
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*(x[None, None] for x in t), scale=s)[0, 0]
    (o * torch.tensor(do)).sum().backward()
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("T,B", [(256, 64), (300, 64)])
def test_all_blocks_exact_gives_dense_gradients(T, B):
    q, k, v, do = rand(T, 16, 5)
    s = 0.25
    N = O.num_blocks(T, B)
    idx = np.array([([j for j in range(N) if abs(i - j) > 1] + [-1] * N)[:N] for i in range(N)], np.int32)
    got = BO.grads(q, k, v, do, idx, B=B, scale=s, band=1)
    for g, w in zip(got, dense_grads(q, k, v, do, s)):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)


def test_one_token_blocks_give_dense_gradients_for_any_routing():
    """B = 1: every virtual token is exact (kbar = k, H_j = 0), so any routing
    gives softmax attention and its gradient."""
    T = 24
    q, k, v, do = rand(T, 4, 9)
    s = 0.6
    r = np.random.default_rng(3)
    idx = np.stack([np.sort(r.choice([j for j in range(T) if j != i], 3, replace=False)) for i in range(T)])
    got = BO.grads(q, k, v, do, idx.astype(np.int32), B=1, scale=s, band=0)
    for g, w in zip(got, dense_grads(q, k, v, do, s)):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)


def test_o_used_equal_to_o_changes_nothing():
    T, B = 200, 32
    q, k, v, do = rand(T, 8, 21)
    _, parts = O.pisa_forward_head(q, k, v, B=B, scale=0.4, topk=2, band=1, return_parts=True)
    o = O.pisa_forward_head(q, k, v, B=B, scale=0.4, topk=2, band=1)
    a = BO.grads(q, k, v, do, parts["idx"], B=B, scale=0.4, band=1)
    b = BO.grads(q, k, v, do, parts["idx"], o_used=o, B=B, scale=0.4, band=1)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_o_used_closed_form_in_softmax_attention():
    """Every block exact: log den_t = logsumexp_k s q_t.k, so a delta error
    c_t moves dq_t by -c_t s E_P[k], dk_k by -sum_t c_t s P_tk q_t, and
    leaves dv unchanged."""
    T, B, D = 256, 64, 16
    q, k, v, do = rand(T, D, 22)
    s = 0.3
    N = O.num_blocks(T, B)
    idx = np.array([([j for j in range(N) if abs(i - j) > 1] + [-1] * N)[:N] for i in range(N)], np.int32)
    o = O.dense_attention(q, k, v, s)
    o_used = o + 1e-3 * np.random.default_rng(5).standard_normal(o.shape)
    base = BO.grads(q, k, v, do, idx, B=B, scale=s, band=1)
    got = BO.grads(q, k, v, do, idx, o_used=o_used, B=B, scale=s, band=1)
    c = (do * (o_used - o)).sum(1)
    z = s * q @ k.T
    Pm = np.exp(z - z.max(1, keepdims=True))
    Pm /= Pm.sum(1, keepdims=True)
    np.testing.assert_allclose(got[0] - base[0], -(c[:, None] * s * (Pm @ k)), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1] - base[1], -s * (Pm * c[:, None]).T @ q, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[2], base[2], rtol=0, atol=1e-13)


def test_dq_of_sampled_blocks_equals_full_gradient():
    T, B = 300, 32
    q, k, v, do = rand(T, 8, 23)
    for so in (False, True):
        _, parts = O.pisa_forward_head(q, k, v, B=B, scale=0.5, topk=2, band=1, second_order=so,
                                       return_parts=True)
        full = BO.grads(q, k, v, do, parts["idx"], B=B, scale=0.5, band=1, second_order=so)[0]
        blocks = [7, 0, 9]
        got = BO.grads_q_blocks(q, k, v, do, parts["idx"], blocks, B=B, scale=0.5, band=1, second_order=so)
        rows = np.concatenate([np.arange(32 * i, min(T, 32 * i + 32)) for i in blocks])
        np.testing.assert_allclose(got, full[rows], rtol=0, atol=1e-12)
