"""Plain fp64 CPU oracle for PISA piecewise sparse attention (forward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the
HIP library and imports nothing from it.

Sources (cited by page title and section / equation, as printed there):

* [PISA] "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
  Transformers" (arXiv 2602.01077): §3.1 Eq. 1-2, §3.2 "Formulation" Eqs. 3-6,
  §3.3 Eqs. 7-10, Theorem 3.1, Eq. 11, §3.4 Algorithm 1, Appendix C.
* [PWT] "Piecewise-Taylor-Attention" README (GitHub HaoyiZhu): the opening
  "Blog post" section (second-order mass term w_j, gating at ln B), the knobs
  paragraph (band), and the changelog items on hc-free statistics and the
  router (clamped ranking spread, set-identical top-k).

Everything is float64 numpy. Inputs are taken as given (bf16 inputs are
upcast exactly by the caller). A library matmul stands in for each sum that
the pages write as a matrix product; there is no blocking, fusion or
reordering beyond the steps the pages state.

Readings adopted where the pages are silent or inconsistent (each one is a
convention that both this oracle and the HIP path follow):

R1  softmax scale s = 1/sqrt(D) on every logit (exact, virtual, routing); the
    Taylor terms use q' = s*q  ([PISA] App. C puts the scale back in alpha).
R3  H_j is centred on the block centroid k̄_j ([PISA] App. C notation).
R4  global first order: F_t = (l_tail_t / T) * q'_t H with H = sum_j H_j and
    l_tail_t the tail *mass* sum_{j in U} n_j a_tj  ([PISA] Algorithm 1
    Phase 3 with the virtual-token mass of Eq. 3; equals Eq. 10 when 64 | T).
R5  a virtual token carries mass n_j * exp(lambda)  ([PISA] Eq. 3).
R6  partial last block: n_j = rows present; the gate threshold stays ln B.
R7  routing score r_ij = s * qbar_i . kbar_j (+ min(w_ij, ln B) when the
    second-order term is on); the covariance prior only when asked for (R19).
R8  topk is an integer argument (callers use floor(density * N)).
R9  the +-band is forced exact and top-k is taken over the non-band blocks
    (band_mode="additive"); band_mode="union" is the alternative reading.
R10 ties in routing go to the lower block index; tables are ascending.
R11 q2bar = mean over the query block of (s*q)^2 (elementwise); sigma^2 is
    the population variance (1/n_j).
R12 gate: w > ln B  ->  0 (strict), w = ln B kept.
R13 the gated w enters the virtual logit, hence numerator, mass and l_tail.
R16 sink blocks ([PWT] knobs: n_sink_blocks=n forces the first n KV blocks,
    e.g. an MMDiT text prefix, into the exact branch): like the band they are
    forced for every query block and top-k is taken over the other blocks.
R19 covariance-aware routing ([PISA] §3.3 "Covariance-Aware Block Selection",
    Eq. 11, Appendix D Eq. 14; [PWT] knobs cov_bias=True and the changelog's
    per-block Frobenius norm in the router): the routing score gains
    log(M_j + eps) with M_j = ||H_j - Hbar||_F, Hbar = (1/N) sum_j H_j over all
    N blocks (the global statistic of Eq. 10), eps = 1e-6. The paper's own
    notation makes ||.||_2 the spectral norm; cov_norm="spectral" is that
    alternative reading. Eq. 11's softmax is dropped as in R7.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

COV_EPS = 1e-6   # eps of log(M_j + eps) (R19)

__all__ = [
    "COV_EPS",
    "block_heterogeneity",
    "cov_bias",
    "num_blocks",
    "block_slices",
    "kv_block_stats",
    "pool_queries",
    "second_order_w",
    "route_topk",
    "selected_sets",
    "dense_attention",
    "pisa_forward_head",
    "pisa_forward",
    "KVStats",
]


def num_blocks(T: int, B: int) -> int:
    """N = ceil(T / B)  ([PISA] Algorithm 1, loop bound)."""
    return -(-T // B)


def block_slices(T: int, B: int):
    """Row ranges of the block partition t = iB + m  ([PISA] §3.2 Formulation)."""
    return [(j * B, min((j + 1) * B, T)) for j in range(num_blocks(T, B))]


@dataclass
class KVStats:
    n: np.ndarray          # [N] rows per block
    kbar: np.ndarray       # [N, D] block centroid of keys
    vsum: np.ndarray       # [N, D] block sum of values  (V-hat)
    sig2: np.ndarray       # [N, D] per-dim population variance of keys
    H: np.ndarray          # [D, D] sum_j H_j
    Hj: np.ndarray | None  # [N, D, D] per-block first-order matrices (optional)


def kv_block_stats(k: np.ndarray, v: np.ndarray, B: int, per_block_H: bool = False) -> KVStats:
    """Block statistics of one (batch, head).

    kbar_j = (1/n_j) sum_n k_{j,n}; V-hat_j = sum_n v_{j,n}
        ([PISA] §3.2 Formulation and Eq. 5; Fig. 4 "Prepare Phase").
    H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n}, H = sum_j H_j
        ([PISA] Appendix C notation; R3).
    sigma^2_j = (1/n_j) sum_n (k_{j,n} - kbar_j)^2 per dimension
        ([PWT] "Blog post": per-dimension key variance of block j; R11).
    H is formed here from its definition (centred keys times values), not
    from the K^T V identity; the tests check the identity separately.
    """
    T, D = k.shape
    sl = block_slices(T, B)
    N = len(sl)
    n = np.array([b - a for a, b in sl], dtype=np.float64)
    kbar = np.empty((N, D))
    vsum = np.empty((N, D))
    sig2 = np.empty((N, D))
    kc = np.empty_like(k)
    for j, (a, b) in enumerate(sl):
        kbar[j] = k[a:b].sum(axis=0) / n[j]
        vsum[j] = v[a:b].sum(axis=0)
        kc[a:b] = k[a:b] - kbar[j]
        sig2[j] = (kc[a:b] ** 2).sum(axis=0) / n[j]
    H = kc.T @ v
    Hj = None
    if per_block_H:
        Hj = np.stack([kc[a:b].T @ v[a:b] for a, b in sl])
    return KVStats(n=n, kbar=kbar, vsum=vsum, sig2=sig2, H=H, Hj=Hj)


def pool_queries(q: np.ndarray, B: int, scale: float):
    """qbar_i = block mean of queries; q2bar_i = block mean of (s*q)^2.

    ([PISA] Algorithm 1 step 1 and Fig. 4: block means Q-bar;
    [PWT] "Blog post": q^2 pooled per query block; R11.)
    """
    T, D = q.shape
    sl = block_slices(T, B)
    qbar = np.empty((len(sl), D))
    q2bar = np.empty((len(sl), D))
    for i, (a, b) in enumerate(sl):
        qbar[i] = q[a:b].sum(axis=0) / (b - a)
        q2bar[i] = ((scale * q[a:b]) ** 2).sum(axis=0) / (b - a)
    return qbar, q2bar


def second_order_w(q2bar: np.ndarray, sig2: np.ndarray, B: int):
    """w_ij = 1/2 q2bar_i . sigma^2_j; gated and clamped forms.

    ([PWT] "Blog post": B e^{q.kbar + w}, w = 1/2 q2bar . sigma^2; gated to zero
    where w exceeds ln B; changelog "Router polish": ranking uses min(w, ln B).)
    Returns (w, w_gated, w_rank), each [Nq, Nk].
    """
    w = 0.5 * (q2bar @ sig2.T)
    lnB = math.log(B)
    w_gated = np.where(w > lnB, 0.0, w)
    w_rank = np.minimum(w, lnB)
    return w, w_gated, w_rank


def block_heterogeneity(Hj: np.ndarray, norm: str = "fro") -> np.ndarray:
    """M_j = ||H_j - Hbar|| per block, Hbar = (1/N) sum_j H_j  ([PISA] Eq. 10
    for Hbar, Eq. 11 and Appendix D for M_j; R19). Hj: [N, D, D]."""
    Hbar = Hj.sum(axis=0) / Hj.shape[0]
    diff = Hj - Hbar[None]
    if norm == "fro":
        return np.sqrt((diff * diff).sum(axis=(1, 2)))
    if norm == "spectral":
        return np.array([np.linalg.norm(d, ord=2) for d in diff])
    raise ValueError(norm)


def cov_bias(M: np.ndarray, eps: float = COV_EPS) -> np.ndarray:
    """The routing prior log(M_j + eps)  ([PISA] Eq. 11)."""
    return np.log(M + eps)


def route_topk(qbar, kbar, scale, topk, band, w_rank=None, band_mode="additive", n_sink=0, bias=None):
    """Per query block, the top-k KV blocks by pooled score.

    r_ij = s qbar_i . kbar_j (+ w_rank_ij) (+ bias_j)   ([PISA] Algorithm 1
    step 2 with Eq. 11, R7; [PWT] router with min(w, ln B); bias_j the
    covariance prior log(M_j + eps) of R19 when given).
    Band_i = {j : |i-j| <= band} is forced exact ([PWT] knobs: band=b).
    additive (R9): Top_i = the min(topk, |Cand_i|) best of Cand_i = all \\ Band_i
    \\ Sinks, Sinks = {j < n_sink} (R16).
    union: Top_i = the topk best of all blocks (the band is added afterwards).
    Ranking key (-r_ij, j): ties go to the lower index (R10).
    Returns (idx [Nq, topk] int32 ascending, -1 padded; scores r [Nq, Nk]).
    """
    Nq, Nk = qbar.shape[0], kbar.shape[0]
    r = scale * (qbar @ kbar.T)
    if w_rank is not None:
        r = r + w_rank
    if bias is not None:
        r = r + np.asarray(bias)[None, :]
    idx = np.full((Nq, topk), -1, dtype=np.int32)
    for i in range(Nq):
        if band_mode == "additive":
            cand = np.array([j for j in range(Nk) if abs(i - j) > band and j >= n_sink], dtype=np.int64)
        elif band_mode == "union":
            cand = np.arange(Nk, dtype=np.int64)
        else:
            raise ValueError(band_mode)
        # stable sort on -r keeps ascending j among equal scores
        order = cand[np.argsort(-r[i, cand], kind="stable")]
        chosen = np.sort(order[: min(topk, len(cand))])
        idx[i, : len(chosen)] = chosen
    return idx, r


def selected_sets(idx_row: np.ndarray, i: int, N: int, band: int, n_sink: int = 0):
    """S_i = Band_i union Sinks union Top_i, U_i = complement  ([PISA] §3.2
    Formulation; sinks R16)."""
    S = set(int(j) for j in idx_row if 0 <= j < N)
    S.update(j for j in range(max(0, i - band), min(N, i + band + 1)))
    S.update(range(min(n_sink, N)))
    Ssorted = np.array(sorted(S), dtype=np.int64)
    U = np.array([j for j in range(N) if j not in S], dtype=np.int64)
    return Ssorted, U


def dense_attention(q, k, v, scale):
    """O = softmax(s Q K^T) V  ([PISA] §3.1 Eq. 1)."""
    z = scale * (q @ k.T)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def pisa_forward_head(q, k, v, *, B=64, scale=None, topk, band=1, second_order=False,
                      first_order="global", sparse_only=False, routing=None,
                      query_blocks=None, band_mode="additive", return_parts=False, n_sink=0,
                      cov_bias=False, cov_norm="fro"):
    """PISA forward for one (batch, head); q, k, v are [T, D] float64.

    Per query block i and query row t (q' = s q_t):
      exact   E_num = sum_{j in S_i} sum_n e^{q'.k_{j,n}} v_{j,n},
              E_den = sum_{j in S_i} sum_n e^{q'.k_{j,n}}      ([PISA] Eqs. 3-4)
      virtual lambda_tj = q'.kbar_j + w_gated_ij,  a_tj = e^{lambda_tj},
              A_num = sum_{j in U_i} a_tj V-hat_j,
              A_den = l_tail_t = sum_{j in U_i} n_j a_tj          ([PISA] Eqs. 3, 5;
              [PWT] "Blog post"; R5, R13)
      first   global:    F_t = (l_tail_t / T) q'_t H            ([PISA] Eq. 10,
                         Algorithm 1 Phase 3; R4)
              blockwise: F_t = sum_{j in U_i} a_tj q'_t H_j     ([PISA] Eq. 6)
              none:      F_t = 0                                 ("-0th")
      output  o_t = (E_num + A_num + F_t) / (E_den + A_den)      ([PISA] Eq. 3,
              Algorithm 1 step 24)
    Every exponential is taken relative to m_t, the max over the exact logits
    and every lambda_tj + ln n_j; the shift cancels in the ratio ([PISA]
    Algorithm 1 omits the safe-softmax steps "for brevity").

    routing: None (computed here) or an [N, topk] table (-1 padded) that is
    used as Top_i verbatim ("fed the GPU's routing").
    n_sink: the first n_sink KV blocks are exact for every query block (R16).
    cov_bias: route with the covariance prior log(M_j + eps) (R19).
    query_blocks: iterable of block indices to evaluate (others stay NaN).
    Returns o [T, D] (and a dict of intermediate quantities if return_parts).
    """
    T, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    N = num_blocks(T, B)
    sl = block_slices(T, B)
    st = kv_block_stats(k, v, B, per_block_H=(first_order == "blockwise" or cov_bias))
    qbar, q2bar = pool_queries(q, B, scale)
    if second_order:
        w, w_gated, w_rank = second_order_w(q2bar, st.sig2, B)
    else:
        w = w_gated = w_rank = None
    M = block_heterogeneity(st.Hj, cov_norm) if cov_bias else None
    if routing is None:
        idx, _ = route_topk(qbar, st.kbar, scale, topk, band, w_rank, band_mode, n_sink,
                            bias=cov_bias_fn(M) if cov_bias else None)
    else:
        idx = np.asarray(routing)
    lnn = np.log(st.n)
    out = np.full((T, D), np.nan)
    parts = {"idx": idx, "l_tail": np.full(T, np.nan), "den": np.full(T, np.nan),
             "m": np.full(T, np.nan)}
    blocks = range(N) if query_blocks is None else query_blocks
    for i in blocks:
        a0, a1 = sl[i]
        S, U = selected_sets(idx[i], i, N, band, n_sink)
        qp = scale * q[a0:a1]                                   # [R, D]
        keys = np.concatenate([np.arange(*sl[j]) for j in S]) if len(S) else np.zeros(0, np.int64)
        logit_ex = qp @ k[keys].T                               # [R, |keys|]
        lam = qp @ st.kbar[U].T                                 # [R, |U|]
        if second_order:
            lam = lam + w_gated[i, U][None, :]
        if sparse_only:
            lam = lam[:, :0]
            U = U[:0]
        mass_logit = lam + lnn[U][None, :]
        m = np.full(a1 - a0, -np.inf)
        if logit_ex.shape[1]:
            m = np.maximum(m, logit_ex.max(axis=1))
        if mass_logit.shape[1]:
            m = np.maximum(m, mass_logit.max(axis=1))
        pe = np.exp(logit_ex - m[:, None])
        E_num = pe @ v[keys]
        E_den = pe.sum(axis=1)
        a = np.exp(lam - m[:, None])                            # [R, |U|]
        A_num = a @ st.vsum[U]
        l_tail = a @ st.n[U]
        if first_order == "global":
            F = (l_tail / T)[:, None] * (qp @ st.H)
        elif first_order == "blockwise":
            F = np.einsum("ru,rd,ude->re", a, qp, st.Hj[U]) if len(U) else np.zeros_like(qp)
        elif first_order == "none":
            F = np.zeros_like(qp)
        else:
            raise ValueError(first_order)
        if sparse_only:
            F = np.zeros_like(qp)
        den = E_den + l_tail
        out[a0:a1] = (E_num + A_num + F) / den[:, None]
        parts["l_tail"][a0:a1] = l_tail
        parts["den"][a0:a1] = den
        parts["m"][a0:a1] = m
    if return_parts:
        parts.update(stats=st, qbar=qbar, q2bar=q2bar, w=w, w_gated=w_gated, w_rank=w_rank, M=M)
        return out, parts
    return out


def pisa_forward(q, k, v, **kw):
    """Batched wrapper over [Bt, H, T, D] arrays; returns o of the same shape."""
    Bt, Hh, T, D = q.shape
    o = np.empty((Bt, Hh, T, D))
    for b in range(Bt):
        for h in range(Hh):
            o[b, h] = pisa_forward_head(q[b, h], k[b, h], v[b, h], **kw)
    return o


cov_bias_fn = cov_bias   # the function, under a name the keyword argument does not shadow
