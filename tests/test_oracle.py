"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

No page prints a numeric worked example of the operator, so every pin is one
of: a hand-worked closed form, a special case that reduces to a library
routine (softmax attention), an inequality the paper proves (Jensen, Theorem
3.1 / C.2), an algebraic invariance that follows from the definitions, an
order-of-accuracy statement of the Taylor expansion, or brute force.

Sources: "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
Transformers" (§3.1-§3.4, Appendix C) and the "Piecewise-Taylor-Attention"
README ("Blog post" section, knobs, changelog).
"""

import math

import numpy as np
import pytest
import torch

from oracle import pisa_oracle as O

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def rand_qkv(T, D, seed, scale_q=1.0):
    r = np.random.default_rng(seed)
    return (scale_q * r.standard_normal((T, D)), r.standard_normal((T, D)), r.standard_normal((T, D)))


def sdpa(q, k, v, scale):
    """Library softmax attention (torch, float64 on the CPU)."""
    t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t, scale=scale)[0, 0].numpy()


# ---------------------------------------------------------------- dense / Eq. 1

def test_dense_matches_library_sdpa():
    q, k, v = rand_qkv(200, 16, 1)
    s = 0.3
    np.testing.assert_allclose(O.dense_attention(q, k, v, s), sdpa(q, k, v, s), rtol=0, atol=1e-13)


@pytest.mark.parametrize("T,B", [(256, 64), (300, 64), (100, 16), (77, 8)])
@pytest.mark.parametrize("second_order", [False, True])
@pytest.mark.parametrize("first_order", ["global", "blockwise", "none"])
def test_density_one_equals_dense(T, B, second_order, first_order):
    """Every KV block exact => U_i empty => o = softmax attention (Eq. 1)."""
    q, k, v = rand_qkv(T, 16, T + B)
    N = O.num_blocks(T, B)
    s = 1 / 4
    o = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=N, band=1, second_order=second_order,
                            first_order=first_order)
    np.testing.assert_allclose(o, sdpa(q, k, v, s), rtol=0, atol=1e-12)


def test_block_size_one_is_exact_for_any_routing():
    """B = 1: kbar = k, V-hat = v, H_j = 0, n_j = 1, so the virtual tokens are exact."""
    q, k, v = rand_qkv(40, 8, 5)
    r = np.random.default_rng(0)
    routing = np.sort(r.choice(40, size=(40, 3)), axis=1).astype(np.int32)
    for second_order in (False, True):
        o = O.pisa_forward_head(q, k, v, B=1, scale=0.5, topk=3, band=0, routing=routing,
                                second_order=second_order)
        np.testing.assert_allclose(o, sdpa(q, k, v, 0.5), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [256, 230])
def test_identical_keys_make_virtual_tokens_exact(T):
    """Identical keys inside every block: n_j e^{q'.kbar_j} is the exact block mass,
    e^{q'.kbar_j} V-hat_j the exact numerator, H_j = 0 and sigma^2_j = 0, so
    the output is softmax attention for any routing."""
    B, D = 64, 16
    q, _, v = rand_qkv(T, D, 7)
    kb = np.random.default_rng(8).standard_normal((O.num_blocks(T, B), D)) * 2
    k = np.repeat(kb, B, axis=0)[:T]
    for second_order in (False, True):
        for fo in ("global", "blockwise"):
            o = O.pisa_forward_head(q, k, v, B=B, topk=0, band=0, second_order=second_order,
                                    first_order=fo)
            np.testing.assert_allclose(o, sdpa(q, k, v, 0.25), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- hand-worked example

def test_hand_worked_example():
    """T=4, B=2, D=1, s=1, topk=0, band=0 (S_i = {i}, U_i = {1-i}).

    k = [0, 2 | 1, 1], v = [1, 3 | 2, 4], q = [1, 0 | 0, 1].
    Block 0: kbar=1, V-hat=4, H_0 = (0-1)*1 + (2-1)*3 = 2, sigma^2 = 1.
    Block 1: kbar=1, V-hat=6, H_1 = 0,                    sigma^2 = 0.   H = 2, T = 4.
    t=0 (q=1): exact e^0*1 + e^2*3 over 1 + e^2; virtual a = e, A_num = 6e,
               mass 2e; F = (2e/4)*1*2 = e       -> (1 + 7e + 3e^2) / (1 + e)^2
    t=1 (q=0): (1 + 3 + 6) / (2 + 2)                 = 5/2
    t=2 (q=0): (2 + 4 + 4) / (2 + 2)                 = 5/2
    t=3 (q=1): exact e(2+4), mass 2e; virtual a = e: 4e, mass 2e; F = e
               -> 11e / 4e                           = 11/4
    Block-wise first order (Eq. 6): F_0 = e*H_1 = 0, F_3 = e*1*H_0 = 2e.
    Second order (ln B = ln 2): q2bar = 1/2 in both blocks; w_01 = 0,
    w_10 = 1/2 * 1/2 * 1 = 1/4 (kept): t=2 -> (6 + 4c)/(2 + 2c), t=3 ->
    (6e + 5ec)/(2e + 2ec) with c = e^{1/4}.
    """
    e = math.e
    q = np.array([[1.0], [0.0], [0.0], [1.0]])
    k = np.array([[0.0], [2.0], [1.0], [1.0]])
    v = np.array([[1.0], [3.0], [2.0], [4.0]])
    kw = dict(B=2, scale=1.0, topk=0, band=0)
    o = O.pisa_forward_head(q, k, v, **kw)[:, 0]
    np.testing.assert_allclose(o, [(1 + 7 * e + 3 * e * e) / (1 + e) ** 2, 2.5, 2.5, 2.75], rtol=1e-14)
    ob = O.pisa_forward_head(q, k, v, first_order="blockwise", **kw)[:, 0]
    np.testing.assert_allclose(ob, [(1 + 6 * e + 3 * e * e) / (1 + e) ** 2, 2.5, 2.5, 3.0], rtol=1e-14)
    o0 = O.pisa_forward_head(q, k, v, first_order="none", **kw)[:, 0]
    np.testing.assert_allclose(o0, [(1 + 6 * e + 3 * e * e) / (1 + e) ** 2, 2.5, 2.5, 2.5], rtol=1e-14)
    c = math.exp(0.25)
    o2 = O.pisa_forward_head(q, k, v, second_order=True, **kw)[:, 0]
    np.testing.assert_allclose(
        o2, [(1 + 7 * e + 3 * e * e) / (1 + e) ** 2, 2.5, (6 + 4 * c) / (2 + 2 * c),
             (6 * e + 5 * e * c) / (2 * e + 2 * e * c)], rtol=1e-14)
    so = O.pisa_forward_head(q, k, v, sparse_only=True, **kw)[:, 0]
    np.testing.assert_allclose(so, [(1 + 3 * e * e) / (1 + e * e), 2.0, 3.0, 3.0], rtol=1e-14)


# ---------------------------------------------------------------- statistics

def test_stats_hc_free_identity_and_variance():
    """H = sum_j (K_j - kbar_j)^T V_j equals K^T V - sum_j kbar_j (x) V-hat_j (the
    README's hc-free identity); sigma^2 >= 0 and equals numpy's population variance."""
    T, B, D = 300, 64, 8
    _, k, v = rand_qkv(T, D, 11)
    k = k + 3.0
    st = O.kv_block_stats(k, v, B, per_block_H=True)
    ident = k.T @ v - sum(np.outer(st.kbar[j], st.vsum[j]) for j in range(len(st.n)))
    np.testing.assert_allclose(st.H, ident, rtol=0, atol=1e-11)
    np.testing.assert_allclose(st.Hj.sum(axis=0), st.H, rtol=0, atol=1e-11)
    for j, (a, b) in enumerate(O.block_slices(T, B)):
        np.testing.assert_allclose(st.kbar[j], np.mean(k[a:b], axis=0), rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(st.sig2[j], np.var(k[a:b], axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(st.vsum[j], v[a:b].sum(axis=0), rtol=1e-15, atol=1e-13)
        assert st.n[j] == b - a
    assert (st.sig2 >= 0).all()


def test_jensen_mass_bound():
    """n_j e^{q'.kbar_j} <= sum_n e^{q'.k_{j,n}} for every query and block (Eq. 13)."""
    T, B, D = 320, 64, 16
    q, k, v = rand_qkv(T, D, 13)
    s = 0.25
    st = O.kv_block_stats(k, v, B)
    for j, (a, b) in enumerate(O.block_slices(T, B)):
        true_mass = np.exp(s * q @ k[a:b].T).sum(axis=1)
        approx = st.n[j] * np.exp(s * q @ st.kbar[j])
        assert (approx <= true_mass * (1 + 1e-14)).all()


# ---------------------------------------------------------------- first order

def test_equal_block_matrices_make_global_equal_blockwise():
    """All H_j equal (same in-block deviations, same values) => M = 0 => the
    global first order equals the block-wise one (Theorem 3.1 with M = 0)."""
    T, B, D = 256, 32, 8
    r = np.random.default_rng(3)
    dev = r.standard_normal((B, D)) * 0.3
    dev -= dev.mean(axis=0)
    vblk = r.standard_normal((B, D))
    centres = r.standard_normal((T // B, D))
    k = np.concatenate([c + dev for c in centres])
    v = np.tile(vblk, (T // B, 1))
    q = r.standard_normal((T, D))
    kw = dict(B=B, topk=1, band=1, scale=0.4)
    og = O.pisa_forward_head(q, k, v, first_order="global", **kw)
    ob = O.pisa_forward_head(q, k, v, first_order="blockwise", **kw)
    np.testing.assert_allclose(og, ob, rtol=0, atol=1e-12)
    # and the first-order term is not trivially zero here
    o0 = O.pisa_forward_head(q, k, v, first_order="none", **kw)
    assert np.abs(og - o0).max() > 1e-3


def test_theorem_c2_bound():
    """||o_global - o_blockwise|| <= ||q'_t|| M sum_U alpha_tj / D_t (Eq. 12), 64 | T."""
    T, B, D = 512, 64, 16
    q, k, v = rand_qkv(T, D, 21)
    s = 0.25
    kw = dict(B=B, topk=2, band=1, scale=s)
    og, parts = O.pisa_forward_head(q, k, v, first_order="global", return_parts=True, **kw)
    ob = O.pisa_forward_head(q, k, v, first_order="blockwise", **kw)
    st = O.kv_block_stats(k, v, B, per_block_H=True)
    N = len(st.n)
    Hbar = st.Hj.mean(axis=0)
    for i in range(N):
        _, U = O.selected_sets(parts["idx"][i], i, N, 1)
        M = max(np.linalg.norm(st.Hj[j] - Hbar, 2) for j in U)
        for t in range(i * B, (i + 1) * B):
            qp = s * q[t]
            # parts["den"] and alpha share the same e^{-m_t} shift
            alpha = np.exp(qp @ st.kbar[U].T - parts["m"][t]).sum()
            bound = np.linalg.norm(qp) * M * alpha / parts["den"][t]
            assert np.linalg.norm(og[t] - ob[t]) <= bound * (1 + 1e-12) + 1e-15


@pytest.mark.parametrize("fo,order", [("none", 1), ("blockwise", 2)])
def test_order_of_accuracy(fo, order):
    """Scale the in-block key deviations by eps: the zeroth-order error is O(eps),
    the block-wise first-order error O(eps^2) (Taylor remainder, Appendix C remark 3)."""
    T, B, D = 256, 32, 8
    r = np.random.default_rng(4)
    q = r.standard_normal((T, D))
    v = r.standard_normal((T, D))
    centres = np.repeat(r.standard_normal((T // B, D)), B, axis=0)
    dev = r.standard_normal((T, D))
    errs = []
    for eps in (0.08, 0.04, 0.02):
        k = centres + eps * dev
        o = O.pisa_forward_head(q, k, v, B=B, topk=1, band=0, scale=0.5, first_order=fo)
        errs.append(np.abs(o - sdpa(q, k, v, 0.5)).max())
    rates = [math.log2(errs[i] / errs[i + 1]) for i in range(2)]
    assert all(abs(rt - order) < 0.25 for rt in rates), (errs, rates)


# ---------------------------------------------------------------- second order (PWT)

def _pm_block_case(a_dev, q_d, B=64, D=4, dim=1):
    """Every KV block: keys kbar_j +- a on one dim (half each), equal values;
    every query block: identical rows. Returns q, k, v and x = q'_d a."""
    N = 4
    r = np.random.default_rng(9)
    kb = r.standard_normal((N, D)) * 0.5
    sign = np.where(np.arange(B) % 2 == 0, 1.0, -1.0)
    k = np.concatenate([np.tile(kb[j], (B, 1)) + np.outer(sign, np.eye(D)[dim]) * a_dev for j in range(N)])
    v = np.repeat(r.standard_normal((N, D)), B, axis=0)
    qrow = r.standard_normal((N, D))
    qrow[:, dim] = q_d
    q = np.repeat(qrow, B, axis=0)
    return q, k, v


def test_second_order_closed_form():
    """Keys +-a on one dim, identical query rows: w = 1/2 (s q_d)^2 a^2 exactly; the
    true block mass is n e^{q'.kbar} cosh(q'_d a), the PWT mass n e^{q'.kbar + w}, so
    the log-mass error is at most x^4/12 with x = q'_d a (ln cosh x = x^2/2 - x^4/12 + ...)."""
    B, s, a_dev, q_d = 64, 0.5, 0.8, 1.0
    q, k, v = _pm_block_case(a_dev, q_d, B=B)
    st = O.kv_block_stats(k, v, B)
    qbar, q2bar = O.pool_queries(q, B, s)
    w, wg, wr = O.second_order_w(q2bar, st.sig2, B)
    x = s * q_d * a_dev
    np.testing.assert_allclose(w, 0.5 * x * x, rtol=1e-14)
    assert np.array_equal(wg, w) and np.array_equal(wr, w)
    # whole operator: only the diagonal block is exact
    dense = sdpa(q, k, v, s)
    e_pwt = np.abs(O.pisa_forward_head(q, k, v, B=B, scale=s, topk=0, band=0, second_order=True) - dense).max()
    e_pisa = np.abs(O.pisa_forward_head(q, k, v, B=B, scale=s, topk=0, band=0) - dense).max()
    assert e_pwt < e_pisa / 20
    # relative mass error per virtual block is e^{x^4/12 + O(x^6)} - 1; outputs move by less
    assert e_pwt <= (math.exp(x ** 4 / 12) - 1) * np.abs(v).max() * 2


def test_second_order_gate():
    """w > ln B is gated to 0 for the logits (the block falls back to the zeroth order)."""
    B, s = 64, 0.5
    q, k, v = _pm_block_case(4.0, 2.0, B=B)   # x = 4, w = 8 > ln 64
    qbar, q2bar = O.pool_queries(q, B, s)
    w, wg, wr = O.second_order_w(q2bar, O.kv_block_stats(k, v, B).sig2, B)
    assert (w > math.log(B)).all() and (wg == 0).all() and np.allclose(wr, math.log(B))
    o2 = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=0, band=0, second_order=True)
    o1 = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=0, band=0, second_order=False)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)


def test_gate_boundary_is_strict():
    q2bar = np.array([[2.0]])
    sig2 = np.array([[math.log(64.0)], [math.log(64.0) + 1e-9]])
    w, wg, wr = O.second_order_w(q2bar, sig2, 64)     # w = ln 64 and ln 64 + 1e-9
    assert wg[0, 0] == w[0, 0] and wg[0, 1] == 0.0


def test_router_uses_clamped_spread():
    """Ranking bonus is min(w, ln B): a block with a huge w gets only ln B."""
    lnB = math.log(64.0)
    qbar = np.array([[1.0, 0.0]])
    kbar = np.array([[0.0, 0.0], [0.0, 0.0], [1.0, 0.0], [0.0, 0.0]])
    # raw w: block 1 huge (clamped to lnB), block 2 base score 1 + w 3.5 = 4.5 > lnB
    w_rank = np.minimum(np.array([[0.0, 10.0, 3.5, 0.0]]), lnB)
    idx, r = O.route_topk(qbar, kbar, 1.0, 1, band=-1, w_rank=w_rank)
    assert idx.tolist() == [[2]]
    idx_raw, _ = O.route_topk(qbar, kbar, 1.0, 1, band=-1, w_rank=np.array([[0.0, 10.0, 3.5, 0.0]]))
    assert idx_raw.tolist() == [[1]]


def _pooling_case():
    """T = 14 tokens, B = 4, D = 2, s = 1/2: blocks 0-2 full, block 3 ragged
    (two rows). Query block 3 holds rows (1, 1) and (3, -1); key blocks:
      0: four rows (1.3, 0)                      kbar (1.3, 0), sigma^2 (0, 0)
      1: (1.3, 0), (-1.3, 0), (1.3, 0), (-1.3, 0) kbar (0, 0),   sigma^2 (1.69, 0)
      2: (1.8, 0), (0.2, 0), (1.8, 0), (0.2, 0)   kbar (1, 0),   sigma^2 (0.64, 0)
      3: (0, 0), (0, 0)."""
    k = np.zeros((14, 2))
    k[0:4, 0] = 1.3
    k[4:8, 0] = [1.3, -1.3, 1.3, -1.3]
    k[8:12, 0] = [1.8, 0.2, 1.8, 0.2]
    q = np.zeros((14, 2))
    q[0:12] = np.arange(24).reshape(12, 2) / 8.0
    q[12] = [1.0, 1.0]
    q[13] = [3.0, -1.0]
    return q, k, np.zeros((14, 2))


def test_pooled_queries_hand_worked_ragged_block():
    """qbar_i is the mean of the block's query rows and q2bar_i the mean of
    their squares after the softmax scale ([PISA] Algorithm 1 step 1 and
    Fig. 4: block means; [PWT] "Blog post": q^2 pooled per query block), both
    over the n_i rows present (R6). Worked by hand for the ragged block 3
    (rows (1, 1), (3, -1)) and the full block 0 (rows (0, 1/8), (2/8, 3/8),
    (4/8, 5/8), (6/8, 7/8))."""
    q, _, _ = _pooling_case()
    qbar, q2bar = O.pool_queries(q, 4, 0.5)
    assert qbar.shape == (4, 2)
    assert qbar[3].tolist() == [2.0, 0.0]
    # s^2 * mean of squares: 0.25 * ((1 + 9) / 2, (1 + 1) / 2)
    assert q2bar[3].tolist() == [1.25, 0.25]
    assert qbar[0].tolist() == [12 / 32, 16 / 32]
    # 0.25 * (0 + 4 + 16 + 36) / (4 * 64), 0.25 * (1 + 9 + 25 + 49) / (4 * 64)
    np.testing.assert_allclose(q2bar[0], [56 / 1024, 84 / 1024], rtol=1e-15)


def test_pooled_query_scale_decides_second_order_routing():
    """With the second-order term the routing score s qbar_i . kbar_j +
    min(w_ij, ln B) compares the pooled mean against the spread, so the scale of
    qbar matters ([PISA] Algorithm 1 step 2 with Eq. 11's pooled score;
    [PWT] router: min(w, ln B)). Query block 3 (ragged, n = 2), band 0,
    top-1 over key blocks 0, 1, 2, worked by hand:
      s qbar_3 . kbar_j = 0.5 * 2 * kbar_j0 = 1.3, 0, 1.0
      w_3j = 0.5 (1.25 sigma^2_j0 + 0.25 sigma^2_j1) = 0, 1.05625, 0.4
      r_3j = 1.3, 1.05625, 1.4  -> block 2.
    A qbar too large by the row count (a sum: x2) picks block 0 (2.6 > 2.4);
    one too small by half (s q instead of q, or dividing the two rows by B = 4
    instead of n = 2) picks block 1 (0.65, 1.05625, 0.9)."""
    q, k, v = _pooling_case()
    B, s = 4, 0.5
    st = O.kv_block_stats(k, v, B)
    assert st.kbar[:3, 0].tolist() == [1.3, 0.0, 1.0]
    np.testing.assert_allclose(st.sig2[:3, 0], [0.0, 1.69, 0.64], atol=1e-15)
    qbar, q2bar = O.pool_queries(q, B, s)
    w, wg, wr = O.second_order_w(q2bar, st.sig2, B)
    np.testing.assert_allclose(w[3, :3], [0.0, 1.05625, 0.4], atol=1e-15)
    idx, r = O.route_topk(qbar, st.kbar, s, 1, band=0, w_rank=wr)
    np.testing.assert_allclose(r[3, :3], [1.3, 1.05625, 1.4], atol=1e-15)
    assert idx[3].tolist() == [2]
    # the case tells the plausible mis-scalings of qbar apart
    for factor, want in ((2.0, 0), (0.5, 1)):
        bad = qbar.copy()
        bad[3] *= factor
        assert O.route_topk(bad, st.kbar, s, 1, band=0, w_rank=wr)[0][3].tolist() == [want]


# ---------------------------------------------------------------- covariance-aware routing (R19)

def _equal_block_matrices_case(T=256, B=16, D=4, seed=5):
    """Every block has the same in-block key deviations and the same V rows,
    so every H_j is the same matrix; the block means differ."""
    r = np.random.default_rng(seed)
    dev = r.standard_normal((B, D))
    dev -= dev.mean(axis=0)
    vrows = r.standard_normal((B, D))
    N = T // B
    k = np.concatenate([r.standard_normal(D)[None] * 2 + dev for _ in range(N)])
    v = np.tile(vrows, (N, 1))
    q = r.standard_normal((T, D))
    return q, k, v


def test_cov_bias_equal_block_matrices_leave_routing_unchanged():
    """All H_j equal => M_j = ||H_j - Hbar|| = 0 for every block => the prior
    log(M_j + eps) is the same for every block and the ranking is that of the
    plain pooled score ([PISA] Eq. 11)."""
    q, k, v = _equal_block_matrices_case()
    st = O.kv_block_stats(k, v, 16, per_block_H=True)
    M = O.block_heterogeneity(st.Hj)
    assert np.abs(M).max() < 1e-12
    s = 0.5
    qbar, _ = O.pool_queries(q, 16, s)
    plain, _ = O.route_topk(qbar, st.kbar, s, 3, band=1)
    biased, _ = O.route_topk(qbar, st.kbar, s, 3, band=1, bias=O.cov_bias(M))
    assert np.array_equal(plain, biased)
    assert np.array_equal(O.pisa_forward_head(q, k, v, B=16, scale=s, topk=3, cov_bias=True, return_parts=True)[1]["idx"],
                          plain)


def test_cov_bias_hand_worked_scalar_blocks():
    """D = 1, B = 2: H_j is the scalar sum_n (k_n - kbar_j) v_n.
      block 0: k (1, -1), v (1, 0)  ->  kbar 0, H_0 = 1
      block 1: k (2, 2),  v (5, 7)  ->  kbar 2, H_1 = 0
      block 2: k (0, 2),  v (0, 3)  ->  kbar 1, H_2 = (-1)(0) + (1)(3) = 3
      block 3: k (4, 4),  v (1, 1)  ->  kbar 4, H_3 = 0
    Hbar = (1 + 0 + 3 + 0) / 4 = 1, so M = (0, 1, 2, 1) and the prior is
    log(M + eps). Query block 3 (rows 0.5, 0.5: qbar 0.5), band 0, scale 1,
    top-1 over blocks 0, 1, 2 with pooled scores 0.5 kbar = (0, 1, 0.5):
    without the prior block 1 wins (1 > 0.5 > 0); with it the scores are
    (log 1e-6, 1 + log(1 + 1e-6), 0.5 + log(2 + 1e-6)) = (-13.8, 1.000001,
    1.193148): block 2."""
    k = np.array([1, -1, 2, 2, 0, 2, 4, 4], float)[:, None]
    v = np.array([1, 0, 5, 7, 0, 3, 1, 1], float)[:, None]
    q = np.full((8, 1), 0.5)
    st = O.kv_block_stats(k, v, 2, per_block_H=True)
    assert st.Hj[:, 0, 0].tolist() == [1.0, 0.0, 3.0, 0.0]
    M = O.block_heterogeneity(st.Hj)
    assert M.tolist() == [0.0, 1.0, 2.0, 1.0]
    b = O.cov_bias(M)
    np.testing.assert_allclose(b, [math.log(1e-6), math.log(1 + 1e-6), math.log(2 + 1e-6), math.log(1 + 1e-6)],
                               rtol=1e-15)
    qbar, _ = O.pool_queries(q, 2, 1.0)
    plain, _ = O.route_topk(qbar, st.kbar, 1.0, 1, band=0)
    assert plain[3].tolist() == [1]
    biased, r = O.route_topk(qbar, st.kbar, 1.0, 1, band=0, bias=b)
    assert biased[3].tolist() == [2]
    np.testing.assert_allclose(r[3, :3], [math.log(1e-6), 1 + math.log(1 + 1e-6), 0.5 + math.log(2 + 1e-6)],
                               rtol=1e-15)
    _, parts = O.pisa_forward_head(q, k, v, B=2, scale=1.0, topk=1, band=0, cov_bias=True, return_parts=True)
    assert parts["idx"][3].tolist() == [2]
    assert parts["M"].tolist() == [0.0, 1.0, 2.0, 1.0]


def test_cov_norm_frobenius_against_spectral():
    """R19 takes the Frobenius norm: for H_j - Hbar = +-diag(3, 4) it is 5 (the
    spectral norm, the alternative reading, is 4)."""
    Hj = np.array([[[3.0, 0.0], [0.0, 4.0]], [[-3.0, 0.0], [0.0, -4.0]]])
    assert O.block_heterogeneity(Hj, "fro").tolist() == [5.0, 5.0]
    np.testing.assert_allclose(O.block_heterogeneity(Hj, "spectral"), [4.0, 4.0], rtol=1e-15)


def test_cov_heterogeneity_invariances():
    """H_j is centred on the block mean: k -> k + c and v -> v + c leave every
    H_j, hence M_j, unchanged; v -> a v scales M_j by |a|."""
    r = np.random.default_rng(11)
    k, v = r.standard_normal((200, 8)), r.standard_normal((200, 8))
    M = O.block_heterogeneity(O.kv_block_stats(k, v, 32, per_block_H=True).Hj)
    c = r.standard_normal(8)
    Mk = O.block_heterogeneity(O.kv_block_stats(k + c, v, 32, per_block_H=True).Hj)
    Mv = O.block_heterogeneity(O.kv_block_stats(k, v + c, 32, per_block_H=True).Hj)
    Ma = O.block_heterogeneity(O.kv_block_stats(k, -2.5 * v, 32, per_block_H=True).Hj)
    np.testing.assert_allclose(Mk, M, rtol=1e-12)
    np.testing.assert_allclose(Mv, M, rtol=1e-12)
    np.testing.assert_allclose(Ma, 2.5 * M, rtol=1e-12)


def test_cov_heterogeneity_brute_force():
    """M_j from scalar loops over rows and matrix entries (ragged last block)."""
    r = np.random.default_rng(12)
    T, D, B = 45, 3, 8
    k, v = r.standard_normal((T, D)), r.standard_normal((T, D))
    N = -(-T // B)
    Hs = []
    for j in range(N):
        rows = range(j * B, min(T, j * B + B))
        kb = [sum(k[n][a] for n in rows) / len(rows) for a in range(D)]
        Hs.append([[sum((k[n][a] - kb[a]) * v[n][b] for n in rows) for b in range(D)] for a in range(D)])
    Hbar = [[sum(Hs[j][a][b] for j in range(N)) / N for b in range(D)] for a in range(D)]
    want = [math.sqrt(sum((Hs[j][a][b] - Hbar[a][b]) ** 2 for a in range(D) for b in range(D))) for j in range(N)]
    got = O.block_heterogeneity(O.kv_block_stats(k, v, B, per_block_H=True).Hj)
    np.testing.assert_allclose(got, want, rtol=1e-12)


# ---------------------------------------------------------------- routing

def test_routing_known_ranking_band_ties_padding():
    N = 10
    qbar = np.ones((N, 1))
    c = np.array([5.0, 1.0, 9.0, 9.0, 0.0, 7.0, 3.0, 9.0, 2.0, 8.0])
    kbar = c[:, None]
    idx, r = O.route_topk(qbar, kbar, 1.0, 3, band=1)
    # row 0: band {0,1}; candidates by score 9 (2,3,7) -> ties keep lowest: 2,3,7
    assert idx[0].tolist() == [2, 3, 7]
    # row 3: band {2,3,4}; best others: 7 (9), 9 (8), 5 (7)
    assert idx[3].tolist() == [5, 7, 9]
    # row 8: band {7,8,9}; best others: 2, 3 (9), 5 (7)
    assert idx[8].tolist() == [2, 3, 5]
    # fewer candidates than topk: ascending, then -1
    idx2, _ = O.route_topk(qbar[:3], kbar[:3], 1.0, 3, band=1)
    assert idx2.tolist() == [[2, -1, -1], [-1, -1, -1], [0, -1, -1]]
    # union reading: top-3 over all blocks, band not excluded
    idxu, _ = O.route_topk(qbar, kbar, 1.0, 3, band=1, band_mode="union")
    assert idxu[0].tolist() == [2, 3, 7]


def test_routing_with_sink_blocks_known_ranking():
    """Sinks (R16) are forced like the band: never routed, top-k over the rest."""
    N = 10
    qbar = np.ones((N, 1))
    c = np.array([5.0, 1.0, 9.0, 9.0, 0.0, 7.0, 3.0, 9.0, 2.0, 8.0])
    idx, _ = O.route_topk(qbar, c[:, None], 1.0, 3, band=1, n_sink=3)
    # row 0: band {0,1}, sinks {0,1,2}; best of 3..9: 3, 7 (9), 9 (8)
    assert idx[0].tolist() == [3, 7, 9]
    # row 8: band {7,8,9}, sinks {0,1,2}; best of 3..6: 3 (9), 5 (7), 6 (3)
    assert idx[8].tolist() == [3, 5, 6]
    # everything forced: no candidates, all padding
    idx2, _ = O.route_topk(qbar, c[:, None], 1.0, 3, band=1, n_sink=N)
    assert (idx2 == -1).all()
    S, U = O.selected_sets(idx[8], 8, N, 1, n_sink=3)
    assert S.tolist() == [0, 1, 2, 3, 5, 6, 7, 8, 9] and U.tolist() == [4]


@pytest.mark.parametrize("T,B", [(300, 64), (256, 32)])
def test_all_blocks_sinks_equals_dense(T, B):
    """n_sink >= N forces every block exact: o = softmax attention for any topk."""
    q, k, v = rand_qkv(T, 16, 3 * T)
    N = O.num_blocks(T, B)
    s = 0.25
    for topk in (0, 1):
        o = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=topk, band=0, n_sink=N)
        np.testing.assert_allclose(o, sdpa(q, k, v, s), rtol=0, atol=1e-12)


def test_sinks_equal_the_same_blocks_routed():
    """Forcing the sinks equals routing them by hand: the table with the sinks
    listed as routed ids gives the same output as n_sink with the rest."""
    T, B = 640, 64
    q, k, v = rand_qkv(T, 8, 77)
    N = T // B
    kw = dict(B=B, scale=0.3, band=1)
    o_s, parts = O.pisa_forward_head(q, k, v, topk=2, n_sink=2, return_parts=True, **kw)
    table = np.full((N, 4), -1, np.int32)
    for i in range(N):
        ids = sorted(set(int(j) for j in parts["idx"][i] if j >= 0) | {0, 1})
        table[i, :len(ids)] = ids
    o_r = O.pisa_forward_head(q, k, v, topk=4, routing=table, **kw)
    np.testing.assert_allclose(o_s, o_r, rtol=0, atol=1e-13)


def test_out_of_range_routing_entries_are_padding():
    """Table entries outside [0, N) are ignored like -1 (the ABI's reading)."""
    T, B = 640, 64
    q, k, v = rand_qkv(T, 8, 78)
    N = T // B
    kw = dict(B=B, scale=0.3, band=1, topk=3)
    o, parts = O.pisa_forward_head(q, k, v, return_parts=True, **kw)
    bad = np.concatenate([parts["idx"], np.full((N, 2), N + 4, np.int32)], axis=1)
    bad[:, [0, -1]] = bad[:, [-1, 0]]
    np.testing.assert_array_equal(O.pisa_forward_head(q, k, v, routing=bad, **kw), o)


def test_routing_invariant_to_key_translation():
    q, k, v = rand_qkv(640, 8, 31)
    qbar, _ = O.pool_queries(q, 64, 0.3)
    st1 = O.kv_block_stats(k, v, 64)
    st2 = O.kv_block_stats(k + np.linspace(-2, 2, 8), v, 64)
    i1, _ = O.route_topk(qbar, st1.kbar, 0.3, 3, 1)
    i2, _ = O.route_topk(qbar, st2.kbar, 0.3, 3, 1)
    assert np.array_equal(i1, i2)


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("second_order", [False, True])
def test_value_affine_and_key_translation_and_permutation(second_order):
    T, B, D = 300, 64, 8
    q, k, v = rand_qkv(T, D, 41)
    kw = dict(B=B, topk=2, band=1, scale=0.35, second_order=second_order)
    o = O.pisa_forward_head(q, k, v, **kw)
    c = np.linspace(-1, 2, D)
    np.testing.assert_allclose(O.pisa_forward_head(q, k, v + c, **kw), o + c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.pisa_forward_head(q, k, 2.5 * v, **kw), 2.5 * o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O.pisa_forward_head(q, k + c, v, **kw), o, rtol=0, atol=1e-11)
    perm = np.arange(T)
    r = np.random.default_rng(2)
    for a, b in O.block_slices(T, B):
        perm[a:b] = a + r.permutation(b - a)
    np.testing.assert_allclose(O.pisa_forward_head(q, k[perm], v[perm], **kw), o, rtol=0, atol=1e-12)
    # permuting query rows inside a block permutes the output rows
    np.testing.assert_allclose(O.pisa_forward_head(q[perm], k, v, **kw), o[perm], rtol=0, atol=1e-12)


def test_query_block_addressing_and_external_routing():
    T, B, D = 320, 64, 8
    q, k, v = rand_qkv(T, D, 51)
    o, parts = O.pisa_forward_head(q, k, v, B=B, topk=2, band=1, return_parts=True)
    o2 = O.pisa_forward_head(q, k, v, B=B, topk=2, band=1, routing=parts["idx"], query_blocks=[1, 3])
    np.testing.assert_array_equal(o2[64:128], o[64:128])
    assert np.isnan(o2[:64]).all()


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, B, s, idx, band, second_order, first_order):
    """Scalar loops straight from the definitions, no vectorisation."""
    T, D = len(q), len(q[0])
    N = -(-T // B)
    rows = [list(range(j * B, min((j + 1) * B, T))) for j in range(N)]
    kbar = [[sum(k[t][d] for t in rows[j]) / len(rows[j]) for d in range(D)] for j in range(N)]
    vsum = [[sum(v[t][d] for t in rows[j]) for d in range(D)] for j in range(N)]
    sig2 = [[sum((k[t][d] - kbar[j][d]) ** 2 for t in rows[j]) / len(rows[j]) for d in range(D)] for j in range(N)]
    Hj = [[[sum((k[t][a] - kbar[j][a]) * v[t][b] for t in rows[j]) for b in range(D)] for a in range(D)]
          for j in range(N)]
    H = [[sum(Hj[j][a][b] for j in range(N)) for b in range(D)] for a in range(D)]
    out = np.zeros((T, D))
    for i in range(N):
        sel = set(x for x in idx[i] if x >= 0) | {j for j in range(N) if abs(i - j) <= band}
        q2 = [sum((s * q[t][d]) ** 2 for t in rows[i]) / len(rows[i]) for d in range(D)]
        for t in rows[i]:
            qp = [s * q[t][d] for d in range(D)]
            num = [0.0] * D
            den = 0.0
            tail = 0.0
            bw = [0.0] * D
            for j in range(N):
                if j in sel:
                    for n in rows[j]:
                        e = math.exp(sum(qp[d] * k[n][d] for d in range(D)))
                        den += e
                        for d in range(D):
                            num[d] += e * v[n][d]
                else:
                    lam = sum(qp[d] * kbar[j][d] for d in range(D))
                    if second_order:
                        w = 0.5 * sum(q2[d] * sig2[j][d] for d in range(D))
                        lam += w if w <= math.log(B) else 0.0
                    a = math.exp(lam)
                    den += len(rows[j]) * a
                    tail += len(rows[j]) * a
                    for d in range(D):
                        num[d] += a * vsum[j][d]
                    for b in range(D):
                        bw[b] += a * sum(qp[c] * Hj[j][c][b] for c in range(D))
            for b in range(D):
                if first_order == "global":
                    num[b] += tail / T * sum(qp[c] * H[c][b] for c in range(D))
                elif first_order == "blockwise":
                    num[b] += bw[b]
            out[t] = [x / den for x in num]
    return out


@pytest.mark.parametrize("T,B", [(64, 16), (90, 16), (50, 4), (37, 1)])
@pytest.mark.parametrize("second_order", [False, True])
@pytest.mark.parametrize("first_order", ["global", "blockwise"])
def test_brute_force_tiny(T, B, second_order, first_order):
    D = 3
    q, k, v = rand_qkv(T, D, T * 7 + B)
    N = O.num_blocks(T, B)
    r = np.random.default_rng(T)
    topk = min(2, N)
    routing = np.full((N, topk), -1, dtype=np.int32)
    for i in range(N):
        cand = [j for j in range(N) if abs(i - j) > 1]
        ch = sorted(r.choice(cand, size=min(topk, len(cand)), replace=False).tolist()) if cand else []
        routing[i, :len(ch)] = ch
    s = 0.7
    o = O.pisa_forward_head(q, k, v, B=B, scale=s, topk=topk, band=1, routing=routing,
                            second_order=second_order, first_order=first_order)
    ref = brute_force(q.tolist(), k.tolist(), v.tolist(), B, s, routing.tolist(), 1, second_order, first_order)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
