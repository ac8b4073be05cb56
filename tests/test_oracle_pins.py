"""The CPU oracle held to brute force, closed forms, invariants and a library
routine (no GPU needed)."""
import math

import numpy as np
import pytest

from oracle import attention_online, attention_probabilities, attention_reference
from pins import ALL_PINS, CAUSAL_PINS, decimal_attention, support_function_bounds


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_reference_meets_pin(pin):
    pin(attention_reference)


@pytest.mark.parametrize("block", [1, 7, 128])
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_online_meets_pin(pin, block):
    pin(lambda q, k, v, s: attention_online(q, k, v, s, block))


@pytest.mark.parametrize("block", [1, 7, 16, 128, 300, 1000])
def test_tiling_invariance(block):
    """The streaming loop over any K/V tiling gives the definition's O to 1e-12
    ("FlashAttention, simplified", "The trick": the output is the same as
    standard attention). N = 300 leaves a ragged last block for most sizes."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 300, 32)) for _ in range(3))
    q *= 3.0  # peaky rows: the running maximum moves often
    o_ref, lse_ref = attention_reference(q, k, v, 1 / math.sqrt(32))
    o, lse = attention_online(q, k, v, 1 / math.sqrt(32), block)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_probabilities_rows():
    """Every softmax row is non-negative and sums to one."""
    rng = np.random.default_rng(12)
    q, k = (4.0 * rng.standard_normal((3, 120, 16)) for _ in range(2))
    p = attention_probabilities(q, k, 0.25)
    assert p.shape == (3, 120, 120)
    assert np.all(p >= 0.0)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-14


def test_probabilities_match_decimal():
    rng = np.random.default_rng(13)
    q, k = (rng.standard_normal((7, 5)) for _ in range(2))
    p = attention_probabilities(q[None], k[None], 0.9)[0]
    _, lse_ref = decimal_attention(q, k, np.eye(7), 0.9)
    # With V = I the decimal output rows are the softmax rows themselves.
    o_ref, _ = decimal_attention(q, k, np.eye(7), 0.9)
    assert np.max(np.abs(p - o_ref)) <= 1e-15
    assert np.all(np.isfinite(lse_ref))


def test_row_blocking_does_not_change_result(monkeypatch):
    """Blocks of complete rows leave the row-wise definition unchanged."""
    import oracle.attention as oa

    rng = np.random.default_rng(14)
    q, k, v = (rng.standard_normal((1, 2, 200, 16)) for _ in range(3))
    o1, l1 = attention_reference(q, k, v, 0.3)
    monkeypatch.setattr(oa, "_BLOCK_BYTES", 8 * 200 * 3)  # three rows per block
    o2, l2 = attention_reference(q, k, v, 0.3)
    # BLAS may block a matmul differently by shape: equal to rounding only.
    assert np.max(np.abs(o1 - o2)) <= 1e-14 and np.max(np.abs(l1 - l2)) <= 1e-14


def test_rows_subset_equal_full():
    """Oracle rows depend only on their own query row: a sampled subset of query
    rows gives exactly the rows of the full result."""
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((1, 1, 64, 8)) for _ in range(3))
    o, lse = attention_reference(q, k, v, 0.5)
    idx = np.array([0, 5, 63])
    o_s, lse_s = attention_reference(q[:, :, idx], k, v, 0.5)
    assert np.allclose(o_s, o[:, :, idx], rtol=0, atol=1e-15)
    assert np.allclose(lse_s, lse[:, :, idx], rtol=0, atol=1e-15)


def test_zero_keys_rejected_and_empty_queries_ok():
    z = np.zeros((1, 0, 4))
    with pytest.raises(ValueError):
        attention_reference(np.zeros((1, 2, 4)), z, z, 1.0)
    o, lse = attention_reference(z, np.zeros((1, 3, 4)), np.zeros((1, 3, 4)), 1.0)
    assert o.shape == (1, 0, 4) and lse.shape == (1, 0)


def test_support_function_detects_outside_point():
    v = np.array([[[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]]])
    inside = np.array([[[0.2, 0.2]]])
    outside = np.array([[[0.8, 0.8]]])
    assert support_function_bounds(inside, v) <= 0.0
    assert support_function_bounds(outside, v) > 0.0


# -- causal (prefill) attention ------------------------------------------------

@pytest.mark.parametrize("pin", CAUSAL_PINS, ids=lambda p: p.__name__)
def test_causal_reference_meets_pin(pin):
    pin(lambda q, k, v, s: attention_reference(q, k, v, s, causal=True))


@pytest.mark.parametrize("block", [1, 7, 128])
@pytest.mark.parametrize("pin", CAUSAL_PINS, ids=lambda p: p.__name__)
def test_causal_online_meets_pin(pin, block):
    pin(lambda q, k, v, s: attention_online(q, k, v, s, block, causal=True))


@pytest.mark.parametrize("block", [1, 5, 32, 128, 300])
def test_causal_tiling_invariance(block):
    """The streaming loop with the causal mask over any tiling gives the
    definition's result to 1e-12 (blocks straddling the diagonal included)."""
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((2, 300, 32)) for _ in range(3))
    q *= 3.0
    o_ref, lse_ref = attention_reference(q, k, v, 1 / math.sqrt(32), causal=True)
    o, lse = attention_online(q, k, v, 1 / math.sqrt(32), block, causal=True)
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12


def test_causal_probabilities_are_lower_triangular():
    rng = np.random.default_rng(22)
    q, k = (3.0 * rng.standard_normal((2, 90, 16)) for _ in range(2))
    p = attention_probabilities(q, k, 0.3, causal=True)
    assert np.all(np.triu(p, 1) == 0.0)
    assert np.all(p >= 0.0)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-14


def test_causal_needs_square():
    q = np.zeros((1, 3, 4))
    k = np.zeros((1, 5, 4))
    with pytest.raises(ValueError):
        attention_reference(q, k, k, 1.0, causal=True)


# -- backward pass ---------------------------------------------------------------

from oracle import attention_backward_reference  # noqa: E402
from pins import BWD_PINS  # noqa: E402


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_reference_meets_pin(pin):
    pin(lambda q, k, v, do, s, causal: attention_backward_reference(q, k, v, do, s, causal=causal))


# -- row-wise dQ (long sequences) -------------------------------------------------

from oracle import attention_backward_rows  # noqa: E402


def test_backward_rows_against_library_autograd():
    """torch's float64 autograd through its own CPU attention, sampled rows."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(410)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((2, 3, 57, 16)) for _ in range(4))
        scale = 0.3
        rows = [0, 1, 20, 55, 56]
        got = attention_backward_rows(q, k, v, do, scale, rows, causal=causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, is_causal=causal)
        o.backward(torch.from_numpy(do))
        assert np.max(np.abs(got - tq.grad.numpy()[:, :, rows])) <= 1e-12, causal


def test_backward_rows_finite_differences():
    """dQ entries against a central difference of L = sum(O * dO) with the
    (separately pinned) forward oracle."""
    from oracle import attention_reference

    rng = np.random.default_rng(411)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((1, 6, 4)) for _ in range(4))
        got = attention_backward_rows(q, k, v, do, 0.9, range(6), causal=causal)
        h = 1e-5
        for idx in np.ndindex(*q.shape):
            qp, qm = q.copy(), q.copy()
            qp[idx] += h
            qm[idx] -= h
            lp = np.sum(attention_reference(qp, k, v, 0.9, causal=causal)[0] * do)
            lm = np.sum(attention_reference(qm, k, v, 0.9, causal=causal)[0] * do)
            fd = (lp - lm) / (2 * h)
            assert abs(got[idx] - fd) <= 2e-8 * max(1.0, abs(fd)), (causal, idx)


def test_backward_rows_closed_forms():
    """One key, or scale 0 (uniform weights): dQ = 0 exactly in exact
    arithmetic; and the rows equal the full-matrix gradient's rows."""
    rng = np.random.default_rng(412)
    q, k, v, do = (rng.standard_normal((2, 1, 5)) for _ in range(4))
    assert np.max(np.abs(attention_backward_rows(q, k, v, do, 0.7, [0]))) <= 1e-15
    q, k, v, do = (rng.standard_normal((1, 30, 5)) for _ in range(4))
    for causal in (False, True):
        assert np.max(np.abs(attention_backward_rows(q, k, v, do, 0.0, [0, 7, 29], causal=causal))) <= 1e-15
        full = attention_backward_reference(q, k, v, do, 0.45, causal=causal)[0]
        got = attention_backward_rows(q, k, v, do, 0.45, [3, 0, 29], causal=causal)
        assert np.max(np.abs(got - full[:, [3, 0, 29]])) <= 1e-13


# -- column-wise dK, dV (long sequences) -------------------------------------------

from oracle import attention_backward_cols  # noqa: E402
from pins import BWD_PINS, pin_bwd_cols_subset  # noqa: E402


def _bwd_via_cols(q, k, v, do, scale, causal):
    """(dQ, dK, dV) with dK and dV from the column-wise function over every key
    (dQ from the separately pinned row-wise function), so that every backward
    pin applies to the column-wise gradients."""
    n = np.asarray(q).shape[-2]
    dk, dv = attention_backward_cols(q, k, v, do, scale, range(n), causal=causal)
    return attention_backward_rows(q, k, v, do, scale, range(n), causal=causal), dk, dv


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_cols_backward_pins(pin):
    pin(_bwd_via_cols)


def test_backward_cols_subset():
    pin_bwd_cols_subset(attention_backward_cols)


def test_backward_cols_against_library_autograd():
    """torch's float64 autograd through its own CPU attention, sampled keys."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(420)
    for causal in (False, True):
        q, k, v, do = (rng.standard_normal((2, 3, 57, 16)) for _ in range(4))
        scale = 0.3
        cols = [0, 1, 20, 55, 56]
        dk, dv = attention_backward_cols(q, k, v, do, scale, cols, causal=causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, is_causal=causal)
        o.backward(torch.from_numpy(do))
        assert np.max(np.abs(dk - tk.grad.numpy()[:, :, cols])) <= 1e-12, causal
        assert np.max(np.abs(dv - tv.grad.numpy()[:, :, cols])) <= 1e-12, causal


def test_backward_cols_row_blocks(monkeypatch):
    """Rows are gathered in blocks of complete rows (the last one ragged): the
    sums over blocks equal the full-matrix gradient's columns."""
    import oracle.attention as oa

    rng = np.random.default_rng(421)
    q, k, v, do = (1.5 * rng.standard_normal((2, 100, 8)) for _ in range(4))
    monkeypatch.setattr(oa, "_BLOCK_BYTES", 16 * 100 * 7)  # seven rows per block
    for causal in (False, True):
        full = attention_backward_reference(q, k, v, do, 0.6, causal=causal)
        dk, dv = attention_backward_cols(q, k, v, do, 0.6, [99, 0, 31, 64], causal=causal)
        assert np.max(np.abs(dk - full[1][:, [99, 0, 31, 64]])) <= 1e-13
        assert np.max(np.abs(dv - full[2][:, [99, 0, 31, 64]])) <= 1e-13


def test_backward_cols_rejects_bad_keys():
    x = np.zeros((1, 4, 2))
    with pytest.raises(ValueError):
        attention_backward_cols(x, x, x, x, 1.0, [4])
    with pytest.raises(ValueError):
        attention_backward_cols(x, x, x, x, 1.0, [-1])
