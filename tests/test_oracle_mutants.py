"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows the pins are discriminating: a dropped scale, a transposed score
matrix, a wrong logarithm base, a missing maximum shift, a wrong rescale factor
or a lost ragged block would not slip through. Everything here runs on the
CPU; nothing touches the GPU.
"""
import numpy as np
import pytest

from pins import failing_pins

MUTATIONS = [
    "drop_scale",
    "scale_twice",
    "negate_scores",
    "transpose_scores",
    "lse_log2",
    "lse_without_max",
    "no_max_shift",
    "softmax_wrong_axis",
    "no_normalisation",
    "online_alpha_inverted",
    "online_no_rescale_acc",
    "online_no_rescale_sum",
    "online_drop_ragged_block",
    "online_stale_max",
]


def _mutant(q, k, v, scale, mutation):
    """One head-batched attention with a single planted mistake."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale)
    if mutation.startswith("online_"):
        return _online_mutant(q, k, v, s, mutation, block=7)
    if mutation == "drop_scale":
        s = 1.0
    if mutation == "scale_twice":
        s = s * s
    if mutation == "negate_scores":
        s = -s
    kt = np.swapaxes(k, -1, -2)
    scores = s * (q @ kt)
    if mutation == "transpose_scores":
        if scores.shape[-1] != scores.shape[-2]:
            raise ValueError("shape")
        scores = np.swapaxes(scores, -1, -2)
    axis = -2 if mutation == "softmax_wrong_axis" else -1
    m = scores.max(axis=axis, keepdims=True)
    e = np.exp(scores) if mutation == "no_max_shift" else np.exp(scores - m)
    if mutation == "no_max_shift":
        m = np.zeros_like(m)
    l = e.sum(axis=axis, keepdims=True)
    p = e if mutation == "no_normalisation" else e / l
    o = p @ v
    if axis == -2:
        m, l = np.swapaxes(m, -1, -2), np.swapaxes(l, -1, -2)
    if mutation == "lse_log2":
        lse = m[..., 0] + np.log2(l[..., 0])
    elif mutation == "lse_without_max":
        lse = np.log(l[..., 0])
    else:
        lse = m[..., 0] + np.log(l[..., 0])
    return o, lse


def _online_mutant(q, k, v, s, mutation, block):
    """The streaming form as a merge of per-block softmax states (running
    state rescaled by exp(m - m_new), the block's by exp(m_b - m_new)), with
    one planted mistake."""
    lead = q.shape[:-2]
    nq, nk, dv = q.shape[-2], k.shape[-2], v.shape[-1]
    out = np.empty(lead + (nq, dv))
    lse = np.empty(lead + (nq,))
    stop = nk - nk % block if mutation == "online_drop_ragged_block" and nk > block else nk
    for idx in np.ndindex(*lead):
        m = np.full(nq, -np.inf)
        l = np.zeros(nq)
        acc = np.zeros((nq, dv))
        for j0 in range(0, stop, block):
            j1 = min(nk, j0 + block)
            sc = s * (q[idx] @ k[idx][j0:j1].T)
            m_b = sc[:, 0] if mutation == "online_stale_max" else sc.max(axis=1)  # stale: first key only
            e = np.exp(sc - m_b[:, None])
            l_b, acc_b = e.sum(axis=1), e @ v[idx][j0:j1]
            m_new = np.maximum(m, m_b)
            a = np.exp(m - m_new)  # 0 on the first block (m = -inf)
            if mutation == "online_alpha_inverted":
                a = np.where(np.isfinite(m), np.exp(m_new - m), 0.0)
            b = np.exp(m_b - m_new)
            l = (l if mutation == "online_no_rescale_sum" else a * l) + b * l_b
            acc = (acc if mutation == "online_no_rescale_acc" else a[:, None] * acc) + b[:, None] * acc_b
            m = m_new
        out[idx] = acc / l[:, None]
        lse[idx] = m + np.log(l)
    return out, lse


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_mistake_is_caught(mutation):
    bad = failing_pins(lambda q, k, v, s: _mutant(q, k, v, s, mutation))
    assert bad, f"mutation {mutation} passed every pin"


def test_unmutated_copy_passes():
    """The mutant scaffold itself, with no mutation, passes every pin (so the
    failures above come from the planted mistakes)."""
    assert failing_pins(lambda q, k, v, s: _mutant(q, k, v, s, "none")) == []
    assert failing_pins(lambda q, k, v, s: _online_mutant(
        np.asarray(q, float), np.asarray(k, float), np.asarray(v, float), float(s), "online_none", 7)) == []


# -- causal mask mistakes --------------------------------------------------------

from pins import CAUSAL_PINS  # noqa: E402

CAUSAL_MUTATIONS = ["exclude_diagonal", "upper_triangle", "one_key_ahead", "no_mask", "mask_rows_not_keys"]


def _causal_mutant(q, k, v, scale, mutation):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[-2]
    scores = float(scale) * (q @ np.swapaxes(k, -1, -2))
    i = np.arange(n)[:, None]
    j = np.arange(k.shape[-2])[None, :]
    hidden = {
        "exclude_diagonal": j >= i,
        "upper_triangle": j < i,
        "one_key_ahead": j > i + 1,
        "no_mask": np.zeros((n, k.shape[-2]), dtype=bool),
        "mask_rows_not_keys": i[::-1] < j,
    }[mutation]
    scores = np.where(hidden, -np.inf, scores)
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    l = e.sum(axis=-1, keepdims=True)
    return (e / l) @ v, (m + np.log(l))[..., 0]


@pytest.mark.parametrize("mutation", CAUSAL_MUTATIONS)
def test_causal_mutant_is_caught(mutation):
    bad = failing_pins(lambda q, k, v, s: _causal_mutant(q, k, v, s, mutation), CAUSAL_PINS)
    assert bad, f"causal mutation {mutation} passed every causal pin"


def test_causal_mutant_harness_is_sound():
    """The unmutated harness (mask j > i) passes every causal pin."""

    def correct(q, k, v, s):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        n = q.shape[-2]
        scores = float(s) * (q @ np.swapaxes(k, -1, -2))
        scores = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, scores)
        m = scores.max(axis=-1, keepdims=True)
        e = np.exp(scores - m)
        l = e.sum(axis=-1, keepdims=True)
        return (e / l) @ v, (m + np.log(l))[..., 0]

    assert failing_pins(correct, CAUSAL_PINS) == []


# -- backward-pass mistakes ------------------------------------------------------

from pins import BWD_PINS  # noqa: E402

BWD_MUTATIONS = ["dq_no_scale", "no_delta", "delta_wrong_axis", "dk_untransposed", "dv_untransposed",
                 "ds_sign", "dq_uses_v", "causal_mask_dropped"]


def _bwd_mutant(q, k, v, do, scale, causal, mutation):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = float(scale)
    out = [np.empty_like(q), np.empty_like(k), np.empty_like(v)]
    n = q.shape[-2]
    for idx in np.ndindex(*q.shape[:-2]):
        qh, kh, vh, doh = q[idx], k[idx], v[idx], do[idx]
        scores = s * (qh @ kh.T)
        if causal and mutation != "causal_mask_dropped":
            scores = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, scores)
        e = np.exp(scores - scores.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dv = p @ doh if mutation == "dv_untransposed" else p.T @ doh
        dp = doh @ vh.T
        axis = 0 if mutation == "delta_wrong_axis" else 1
        delta = 0.0 if mutation == "no_delta" else (p * dp).sum(axis=axis, keepdims=True)
        ds = p * (dp - delta)
        if mutation == "ds_sign":
            ds = -ds
        dq = (1.0 if mutation == "dq_no_scale" else s) * (ds @ (vh if mutation == "dq_uses_v" else kh))
        dk = s * (ds @ qh if mutation == "dk_untransposed" else ds.T @ qh)
        out[0][idx], out[1][idx], out[2][idx] = dq, dk, dv
    return tuple(out)


@pytest.mark.parametrize("mutation", BWD_MUTATIONS)
def test_backward_mutant_is_caught(mutation):
    bad = failing_pins(lambda *a: _bwd_mutant(*a, mutation), BWD_PINS)
    assert bad, f"backward mutation {mutation} passed every backward pin"


# -- column-wise dK, dV mistakes ---------------------------------------------------

from oracle import attention_backward_rows  # noqa: E402
from pins import pin_bwd_cols_subset  # noqa: E402

COLS_MUTATIONS = ["normalise_over_chosen", "no_delta", "delta_over_chosen", "dk_no_scale", "causal_mask_dropped",
                  "drop_last_row_block", "dv_uses_ds"]


def _cols_mutant(q, k, v, do, scale, cols, causal, mutation, rows_per_block=16):
    """Column-wise dK, dV over row blocks of complete rows, one planted mistake."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    s = float(scale)
    cols = np.asarray(list(cols), dtype=np.int64)
    n = q.shape[-2]
    dk = np.zeros(q.shape[:-2] + (cols.size, q.shape[-1]))
    dv = np.zeros(q.shape[:-2] + (cols.size, v.shape[-1]))
    starts = list(range(0, n, rows_per_block))
    if mutation == "drop_last_row_block" and len(starts) > 1:
        starts = starts[:-1]
    for idx in np.ndindex(*q.shape[:-2]):
        for r0 in starts:
            r1 = min(n, r0 + rows_per_block)
            sc = s * (q[idx][r0:r1] @ k[idx].T)
            if causal and mutation != "causal_mask_dropped":
                sc = np.where(np.arange(n)[None, :] > np.arange(r0, r1)[:, None], -np.inf, sc)
            if mutation == "normalise_over_chosen":
                e = np.exp(sc[:, cols] - sc[:, cols].max(axis=1, keepdims=True))
                p_c = e / e.sum(axis=1, keepdims=True)
                p = None
            else:
                e = np.exp(sc - sc.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                p_c = p[:, cols]
            dp = do[idx][r0:r1] @ v[idx].T
            if mutation == "no_delta":
                delta = 0.0
            elif mutation in ("delta_over_chosen", "normalise_over_chosen"):
                delta = (p_c * dp[:, cols]).sum(axis=1, keepdims=True)
            else:
                delta = (p * dp).sum(axis=1, keepdims=True)
            ds_c = p_c * (dp[:, cols] - delta)
            dv[idx] += (ds_c if mutation == "dv_uses_ds" else p_c).T @ do[idx][r0:r1]
            dk[idx] += (1.0 if mutation == "dk_no_scale" else s) * (ds_c.T @ q[idx][r0:r1])
    return dk, dv


def _failing_cols_pins(cols_fn):
    def bwd(q, k, v, do, scale, causal):
        n = np.asarray(q).shape[-2]
        dk, dv = cols_fn(q, k, v, do, scale, range(n), causal)
        return attention_backward_rows(q, k, v, do, scale, range(n), causal=causal), dk, dv

    bad = failing_pins(bwd, BWD_PINS)
    try:
        with np.errstate(all="ignore"):
            pin_bwd_cols_subset(cols_fn)
    except Exception:  # noqa: BLE001 - any failure counts
        bad.append("pin_bwd_cols_subset")
    return bad


@pytest.mark.parametrize("mutation", COLS_MUTATIONS)
def test_cols_mutant_is_caught(mutation):
    bad = _failing_cols_pins(lambda *a: _cols_mutant(*a, mutation))
    assert bad, f"column-wise mutation {mutation} passed every pin"


def test_cols_mutant_harness_is_sound():
    assert _failing_cols_pins(lambda *a: _cols_mutant(*a, "none")) == []
