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


def _block_partial(scores, v_blk):
    """Softmax state of one block of keys on its own, per query row.

    Returns (m_b, l_b, acc_b): the row maximum of the block's scores, the sum
    of exp(score - m_b) over the block, and those same exponentials times the
    block's value rows. A row that sees no key of the block (every score -inf,
    causal only) gets m_b = -inf, l_b = 0 and acc_b = 0.
    """
    m_b = scores.max(axis=1)
    shift = np.where(np.isfinite(m_b), m_b, 0.0)
    e = np.exp(scores - shift[:, None])  # exp(-inf) = 0 for hidden keys
    return m_b, e.sum(axis=1), e @ v_blk


def _merge_partial(m, l, acc, m_b, l_b, acc_b):
    """Fold one block's softmax state into the running state of the rows.

    Both states are re-expressed relative to the larger of the two maxima:
    the running sum and accumulator are multiplied by exp(m - m_new), which
    is 1 unless the block raised the maximum, and the block's by
    exp(m_b - m_new). The result is the state of the union of the two key
    sets, exactly (up to rounding).
    """
    m_new = np.maximum(m, m_b)
    ref = np.where(np.isfinite(m_new), m_new, 0.0)
    a = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
    b = np.where(np.isfinite(m_b), np.exp(m_b - ref), 0.0)
    return m_new, a * l + b * l_b, a[:, None] * acc + b[:, None] * acc_b


def attention_online(q, k, v, scale: float, block: int, causal: bool = False):
    """The pages' streaming algorithm over K/V blocks, in float64.

    "FlashAttention, simplified", "The trick": keys are visited one block at a
    time while each query row carries a running maximum m (starting at -inf),
    a running sum l of exponentials (starting at 0) and an unnormalised output
    accumulator (starting at 0). Each block's scores are formed, the running
    state is rescaled by exp(m_old - m_new) when the block raises the maximum,
    the block's exponentials and their weighted values are added, and after
    the last block the accumulator is divided by l once. Here a block's own
    softmax state is formed first (``_block_partial``) and then folded into
    the running state (``_merge_partial``), which is the same update written
    as an exact merge of two partial softmaxes. ``block`` keys per block; the
    last block may be shorter. LSE = m + ln l (the same reading as above).
    All query rows are carried together: query rows never interact.
    causal=True: scores of keys j > i are -inf in every block; block 0 holds
    key 0, so every row has a finite maximum after the first block.
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
            m, l, acc = _merge_partial(m, l, acc, *_block_partial(scores, vh[j0:j1]))
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


def attention_backward_cols(q, k, v, do, scale: float, cols, causal: bool = False):
    """dK and dV of attention for the key rows `cols` only, float64.

    Key j's gradients gather over every query row that sees it:
        dV_j = sum_i P_ij dO_i
        dK_j = scale * sum_i P_ij (dP_ij - D_i) q_i
    with P_ij the softmax of row i (over all N keys, or keys <= i when causal),
    dP_ij = dO_i . v_j and D_i = sum_j' P_ij' dP_ij'. P_ij and D_i depend on
    all of row i, so every query row is evaluated in full (in blocks of
    complete rows, as in ``attention_reference``), but only the chosen
    columns of P and dS are kept. The same chain rule as
    ``attention_backward_reference``, organised so that it fits very long
    sequences: the work is that of the forward definition, the memory one
    block of rows.

    q, k [..., N, d], v, do [..., N, dv]; cols: key indices. Returns
    (dK [..., len(cols), d], dV [..., len(cols), dv]), float64.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _check(q, k, v)
    if do.shape != q.shape[:-1] + (v.shape[-1],):
        raise ValueError("do must have the shape of the output")
    nq, nk = q.shape[-2], k.shape[-2]
    if causal and nq != nk:
        raise ValueError("causal attention needs as many queries as keys")
    cols = np.asarray([int(j) for j in cols], dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= nk):
        raise ValueError("key index out of range")
    s = np.float64(scale)
    lead = q.shape[:-2]
    dk = np.zeros(lead + (cols.size, q.shape[-1]), dtype=np.float64)
    dv = np.zeros(lead + (cols.size, v.shape[-1]), dtype=np.float64)
    rows = max(1, _BLOCK_BYTES // max(1, 16 * nk))  # two N-wide float64 blocks
    for idx in np.ndindex(*lead):
        qh, kh, vh, doh = q[idx], k[idx], v[idx], do[idx]
        for r0 in range(0, nq, rows):
            r1 = min(nq, r0 + rows)
            scores = s * (qh[r0:r1] @ kh.T)
            if causal:
                scores[_future(r0, r1, nk)] = -np.inf
            e = np.exp(scores - scores.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            dp = doh[r0:r1] @ vh.T
            delta = (p * dp).sum(axis=1, keepdims=True)
            p_c = p[:, cols]
            ds_c = p_c * (dp[:, cols] - delta)
            dv[idx] += p_c.T @ doh[r0:r1]
            dk[idx] += s * (ds_c.T @ qh[r0:r1])
    return dk, dv

