"""Plain float64 CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP path, and the HIP path never calls it.

Sources (the pages, by title and section):
  * "FlashAttention" (interactiveprimer), intro and "The bottleneck is memory,
    not multiplication": attention over N tokens forms the N x N matrix of
    scaled query-key scores, applies a softmax per query row and multiplies the
    result by the values; FlashAttention returns exactly that result.
  * "FlashAttention, simplified", "The trick": the streaming form -- a running
    row maximum m, a running sum l of exponentials, an accumulator rescaled by
    exp(m_old - m_new) whenever the maximum grows, and one division by l at the
    end -- whose output equals standard attention.
  * "What FlashAttention actually buys", "The actual problem": the tiled result
    is exact attention, not an approximation.
  * "What FlashAttention actually buys", "Why the distinction matters
    downstream": the backward pass recomputes tiles rather than storing the
    score matrix; the gradient functions here differentiate the definition.

Readings taken where the pages are silent (each also listed with the design
notes of this repository):
  * causal (prefill) attention: the pages name the prefill case ("FlashAttention,
    simplified", "Why it matters for inference") but no mask; the plainest
    reading is the lower-triangular one -- query i of a sequence sees keys
    j <= i (the mask is aligned at the first token, N_q = N_k).
  * scale: the scores are ``scale * q_i . k_j`` with ``scale`` a caller value
    (the pages say "scaled" but give no value); workloads use 1/sqrt(d).
  * logsumexp: LSE_i = m_i + ln(l_i) in natural log of the scaled scores.  It is
    not on the pages; it is the per-row state (m, l) reduced to one number.
  * The streaming loop runs over K/V blocks only: query rows are independent,
    so all query rows are carried together.

Parity pins: every function here is checked by ``tests/test_oracle_pins.py``
against brute force in high-precision decimal arithmetic, closed forms,
invariants and an independent library attention routine; none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

# Upper bound on the float64 score block held at once (bytes); complete score
# rows are always kept, only the number of rows per block changes.
_BLOCK_BYTES = 1 << 28


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v):
    if q.ndim < 2 or k.ndim != q.ndim or v.ndim != q.ndim:
        raise ValueError("q, k, v must have the same rank >= 2")
    if q.shape[:-2] != k.shape[:-2] or q.shape[:-2] != v.shape[:-2]:
        raise ValueError("q, k, v leading dimensions differ")
    if q.shape[-1] != k.shape[-1]:
        raise ValueError("q and k must share the feature size")
    if k.shape[-2] != v.shape[-2]:
        raise ValueError("k and v must have the same number of rows")


def attention_reference(q, k, v, scale: float, causal: bool = False):
    """Exact attention by its definition, in float64, with complete score rows.

    For each leading index (batch, head) and each query row i:
        S_ij   = scale * sum_t q_it k_jt            (all N keys of the row)
        m_i    = max_j S_ij
        E_ij   = exp(S_ij - m_i),  l_i = sum_j E_ij
        P_ij   = E_ij / l_i                          (softmax of the row)
        O_i    = sum_j P_ij v_j
        LSE_i  = m_i + ln l_i
    ("FlashAttention" (interactiveprimer), intro: score matrix, softmax, values.)

    q: [..., Nq, d], k: [..., Nk, d], v: [..., Nk, dv]; any real dtype, upcast
    exactly to float64. ``scale`` is used as the float64 value of the argument.
    Returns (O float64 [..., Nq, dv], LSE float64 [..., Nq]). Rows are handled
    in blocks of complete rows, which leaves the row-wise definition unchanged.
    With Nk == 0 the softmax is undefined and a ValueError is raised.

    causal=True: row i's softmax runs over the keys j <= i only (S_ij = -inf
    for j > i, whose exponential is exactly 0); requires Nq == Nk.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v)
    lead = q.shape[:-2]
    nq, nk, dv = q.shape[-2], k.shape[-2], v.shape[-1]
    if nk == 0 and nq > 0:
        raise ValueError("softmax over zero keys is undefined")
    if causal and nq != nk:
        raise ValueError("causal attention needs as many queries as keys")
    s = np.float64(scale)
    out = np.empty(lead + (nq, dv), dtype=np.float64)
    lse = np.empty(lead + (nq,), dtype=np.float64)
    rows = max(1, _BLOCK_BYTES // max(1, 8 * nk))
    for idx in np.ndindex(*lead):
        qh, kh, vh = q[idx], k[idx], v[idx]
        for r0 in range(0, nq, rows):
            r1 = min(nq, r0 + rows)
            scores = s * (qh[r0:r1] @ kh.T)
            if causal:
                scores[_future(r0, r1, nk)] = -np.inf
            m = scores.max(axis=1)
            e = np.exp(scores - m[:, None])
            l = e.sum(axis=1)
            p = e / l[:, None]
            out[idx][r0:r1] = p @ vh
            lse[idx][r0:r1] = m + np.log(l)
    return out, lse


def _future(r0, r1, nk):
    """Boolean mask of the keys a causal row may not see: rows r0..r1-1
    (absolute query index i), columns j > i."""
    i = np.arange(r0, r1)[:, None]
    j = np.arange(nk)[None, :]
    return j > i


def attention_probabilities(q, k, scale: float, causal: bool = False):
    """The softmax matrix P = softmax(scale * q k^T) row by row, float64.

    Same definition as ``attention_reference``; materialises P, so it is meant
    for small sizes (invariant checks: rows are non-negative and sum to one).
    """
    q, k = _f64(q), _f64(k)
    if q.ndim < 2 or k.shape[:-2] != q.shape[:-2] or k.shape[-1] != q.shape[-1]:
        raise ValueError("q and k shapes do not match")
    scores = np.float64(scale) * (q @ np.swapaxes(k, -1, -2))
    if causal:
        if q.shape[-2] != k.shape[-2]:
            raise ValueError("causal attention needs as many queries as keys")
        scores[..., _future(0, q.shape[-2], k.shape[-2])] = -np.inf
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_online(q, k, v, scale: float, block: int, causal: bool = False):
    """The pages' streaming algorithm over K/V blocks, in float64.

    "FlashAttention, simplified", "The trick": starting from m = -inf, l = 0,
    acc = 0, for each block of ``block`` consecutive keys (the last one may be
    shorter):
        S     = scale * q k_blk^T
        m_new = max(m, rowmax(S))
        alpha = exp(m - m_new)
        l     = alpha * l + rowsum(exp(S - m_new))
        acc   = alpha * acc + exp(S - m_new) v_blk
        m     = m_new
    and finally O = acc / l.  LSE = m + ln l (the same reading as above).
    All query rows are carried together: query rows never interact.
    causal=True: scores of keys j > i are -inf in every block (they add
    exp(-inf) = 0); block 0 holds key 0, so no row starts from an empty block.
    Returns (O, LSE) like ``attention_reference``.
    """
    if block < 1:
        raise ValueError("block must be >= 1")
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v)
    lead = q.shape[:-2]
    nq, nk, dv = q.shape[-2], k.shape[-2], v.shape[-1]
    if nk == 0 and nq > 0:
        raise ValueError("softmax over zero keys is undefined")
    if causal and nq != nk:
        raise ValueError("causal attention needs as many queries as keys")
    s = np.float64(scale)
    out = np.empty(lead + (nq, dv), dtype=np.float64)
    lse = np.empty(lead + (nq,), dtype=np.float64)
    for idx in np.ndindex(*lead):
        qh, kh, vh = q[idx], k[idx], v[idx]
        m = np.full(nq, -np.inf)
        l = np.zeros(nq)
        acc = np.zeros((nq, dv))
        for j0 in range(0, nk, block):
            j1 = min(nk, j0 + block)
            scores = s * (qh @ kh[j0:j1].T)
            if causal:
                scores[np.arange(j0, j1)[None, :] > np.arange(nq)[:, None]] = -np.inf
            m_new = np.maximum(m, scores.max(axis=1))
            alpha = np.exp(m - m_new)
            e = np.exp(scores - m_new[:, None])
            l = alpha * l + e.sum(axis=1)
            acc = alpha[:, None] * acc + e @ vh[j0:j1]
            m = m_new
        out[idx] = acc / l[:, None]
        lse[idx] = m + np.log(l)
    return out, lse


def attention_backward_reference(q, k, v, do, scale: float, causal: bool = False):
    """Gradients of attention by the chain rule applied to its definition, float64.

    With S = scale * q k^T, P = softmax_rows(S) (causal: over keys j <= i),
    O = P v and an upstream gradient dO = dL/dO:
        dV     = P^T dO
        dP     = dO v^T
        D_i    = sum_j P_ij dP_ij            (= dO_i . O_i)
        dS     = P * (dP - D)                (softmax Jacobian, row by row)
        dQ     = scale * dS k
        dK     = scale * dS^T q
    The pages stop at the forward pass; "What FlashAttention actually buys",
    "Why the distinction matters downstream", mentions that the backward pass
    recomputes the score tiles instead of storing them -- the kernels do that,
    using the forward's LSE; this reference materialises P per head.

    q, k [..., N, d], v, do [..., N, dv]. Returns (dQ, dK, dV), float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check(q, k, v)
    if do.shape != q.shape[:-1] + (v.shape[-1],):
        raise ValueError("do must have the shape of the output")
    nq, nk = q.shape[-2], k.shape[-2]
    if causal and nq != nk:
        raise ValueError("causal attention needs as many queries as keys")
    s = np.float64(scale)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for idx in np.ndindex(*q.shape[:-2]):
        qh, kh, vh, doh = q[idx], k[idx], v[idx], do[idx]
        scores = s * (qh @ kh.T)
        if causal:
            scores[_future(0, nq, nk)] = -np.inf
        e = np.exp(scores - scores.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv[idx] = p.T @ doh
        dp = doh @ vh.T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[idx] = s * (ds @ kh)
        dk[idx] = s * (ds.T @ qh)
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, scale: float, rows, causal: bool = False):
    """dQ of attention for the query rows `rows` only, float64.

    Row i of dQ depends on row i alone: with s_j = scale * q_i . k_j over the
    keys row i sees (all N, or j <= i when causal), p = softmax(s),
    dp_j = dO_i . v_j and D_i = sum_j p_j dp_j,
        dQ_i = scale * sum_j p_j (dp_j - D_i) k_j.
    The same chain rule as attention_backward_reference, evaluated one row at
    a time, so that it fits very long sequences.

    q, k [..., N, d], v, do [..., N, dv]; rows: query indices. Returns dQ rows
    [..., len(rows), d], float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check(q, k, v)
    if do.shape != q.shape[:-1] + (v.shape[-1],):
        raise ValueError("do must have the shape of the output")
    nq, nk = q.shape[-2], k.shape[-2]
    if causal and nq != nk:
        raise ValueError("causal attention needs as many queries as keys")
    s = np.float64(scale)
    rows = [int(i) for i in rows]
    out = np.empty(q.shape[:-2] + (len(rows), q.shape[-1]), dtype=np.float64)
    for idx in np.ndindex(*q.shape[:-2]):
        qh, kh, vh, doh = q[idx], k[idx], v[idx], do[idx]
        for t, i in enumerate(rows):
            end = i + 1 if causal else nk
            sc = s * (kh[:end] @ qh[i])
            e = np.exp(sc - sc.max())
            p = e / e.sum()
            dp = vh[:end] @ doh[i]
            delta = p @ dp
            out[idx + (t,)] = s * ((p * (dp - delta)) @ kh[:end])
    return out
