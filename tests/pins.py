"""Checks that pin an attention implementation to facts outside itself.

Each ``pin_*`` function takes an attention callable ``fn(q, k, v, scale) ->
(O, LSE)`` (float64 results, any leading dims) and raises AssertionError if the
callable disagrees with:
  * brute force in 40-digit decimal arithmetic on tiny inputs (exp and ln of
    ``decimal`` are correctly rounded; no numpy involved);
  * closed forms: N = 1, N = 2 (logistic weights), uniform scores (mean of V,
    LSE = ln N), constant value rows, V = identity, a huge score gap, exact ties,
    the augmented-feature shift of the scores;
  * invariants: permutation (in)variance, convex-hull bounds of O;
  * an independent library routine (torch's CPU scaled-dot-product attention
    and logsumexp, both in float64).
The oracle is held to these in ``test_oracle_pins.py``; planted mistakes are
shown to fail them in ``test_oracle_mutants.py``. GPU results reuse
``support_function_bounds`` for the convex-hull check at full size.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np


def decimal_attention(q, k, v, scale, prec: int = 40, causal: bool = False):
    """Attention of one head by brute force in ``prec``-digit decimal arithmetic.

    q [N, d], k [M, d], v [M, dv]; values and scale are converted exactly from
    binary floating point. Returns (O, LSE) as float64 arrays. causal=True:
    query i uses keys 0..i only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    with localcontext() as ctx:
        ctx.prec = prec
        sc = Decimal(float(scale))
        Q = [[Decimal(float(x)) for x in row] for row in q]
        K = [[Decimal(float(x)) for x in row] for row in k]
        V = [[Decimal(float(x)) for x in row] for row in v]
        n, m, dv = len(Q), len(K), v.shape[1]
        out = np.empty((n, dv))
        lse = np.empty(n)
        for i in range(n):
            keys = range(i + 1) if causal else range(m)
            s = [sc * sum(Q[i][t] * K[j][t] for t in range(len(Q[i]))) for j in keys]
            mx = max(s)
            e = [(x - mx).exp() for x in s]
            z = sum(e)
            for c in range(dv):
                out[i, c] = float(sum(e[j] * V[j][c] for j in range(len(e))) / z)
            lse[i] = float(mx + z.ln())
    return out, lse


def _rng(seed):
    return np.random.default_rng(seed)


def pin_brute_force(fn, tol=1e-13):
    """Tiny N and d against the decimal brute force."""
    cases = [(1, 1), (2, 4), (3, 4), (5, 1), (5, 64), (17, 4), (17, 64)]
    for n, d in cases:
        rng = _rng(100 + 7 * n + d)
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d + 1))
        for scale in (1.0 / math.sqrt(d), 0.37, 2.5):
            o, lse = fn(q[None], k[None], v[None], scale)
            o_ref, lse_ref = decimal_attention(q, k, v, scale)
            assert np.max(np.abs(o[0] - o_ref)) <= tol, (n, d, scale, "O")
            assert np.max(np.abs(lse[0] - lse_ref)) <= tol * max(1.0, np.max(np.abs(lse_ref))), (
                n, d, scale, "LSE")


def pin_single_key(fn):
    """N = 1: the output is the only value row, LSE is the single scaled score."""
    rng = _rng(1)
    for d in (1, 8, 64):
        q = rng.standard_normal((1, 1, d))
        k = rng.standard_normal((1, 1, d))
        v = rng.standard_normal((1, 1, d))
        scale = 0.3
        o, lse = fn(q, k, v, scale)
        assert np.max(np.abs(o - v)) <= 1e-15
        expect = scale * float(np.dot(q[0, 0], k[0, 0]))
        assert abs(lse[0, 0] - expect) <= 1e-14 * max(1.0, abs(expect))


def pin_two_keys(fn):
    """N = 2: weights are logistic functions of the score difference.

    Written with hand-chosen vectors so that S and its transpose differ.
    """
    q = np.array([[[1.0, 2.0], [0.5, -1.0]]])
    k = np.array([[[3.0, -1.0], [0.0, 2.0]]])
    v = np.array([[[1.0, 10.0], [-4.0, 0.5]]])
    scale = 0.7
    o, lse = fn(q, k, v, scale)
    for i in range(2):
        s0 = scale * float(q[0, i] @ k[0, 0])
        s1 = scale * float(q[0, i] @ k[0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        expect = w0 * v[0, 0] + w1 * v[0, 1]
        assert np.max(np.abs(o[0, i] - expect)) <= 1e-14, i
        big = max(s0, s1)
        expect_lse = big + math.log1p(math.exp(min(s0, s1) - big))
        assert abs(lse[0, i] - expect_lse) <= 1e-14, i


def pin_uniform_scores(fn):
    """scale = 0, or q = 0: every weight is 1/N, O is the mean of V, LSE = ln N."""
    rng = _rng(2)
    for n in (1, 3, 100, 257):
        k = rng.standard_normal((2, n, 16))
        v = rng.standard_normal((2, n, 16))
        q = rng.standard_normal((2, n, 16))
        for qq, sc in ((q, 0.0), (np.zeros_like(q), 0.25)):
            o, lse = fn(qq, k, v, sc)
            mean = v.mean(axis=1, keepdims=True)
            assert np.max(np.abs(o - mean)) <= 1e-13, n
            assert np.max(np.abs(lse - math.log(n))) <= 1e-13, n


def pin_constant_values(fn):
    """All value rows equal c: O_i = c whatever the weights."""
    rng = _rng(3)
    n, d = 50, 12
    q = 3.0 * rng.standard_normal((1, n, d))
    k = 3.0 * rng.standard_normal((1, n, d))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (1, n, d)).copy()
    o, _ = fn(q, k, v, 0.5)
    assert np.max(np.abs(o - c)) <= 1e-13


def pin_identity_values(fn):
    """V = I (N = d): row i of O is the softmax row of the scaled scores.

    The softmax row is computed here from scaled scores with math.exp/fsum.
    """
    rng = _rng(4)
    n = 9
    q = rng.standard_normal((1, n, n))
    k = rng.standard_normal((1, n, n))
    v = np.eye(n)[None]
    scale = 0.8
    o, _ = fn(q, k, v, scale)
    for i in range(n):
        s = [scale * math.fsum(q[0, i, t] * k[0, j, t] for t in range(n)) for j in range(n)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = math.fsum(e)
        assert np.max(np.abs(o[0, i] - np.array(e) / z)) <= 1e-14, i


def pin_huge_gap_and_ties(fn):
    """A score far above the rest selects its value row; exact ties average."""
    n, d = 6, 4
    q = np.zeros((1, n, d))
    q[0, :, 0] = 1.0
    k = np.zeros((1, n, d))
    k[0, 3, 0] = 1.0  # key 3 scores `scale`, the rest score 0
    v = np.arange(n * d, dtype=np.float64).reshape(1, n, d)
    o, lse = fn(q, k, v, 1.0e4)  # gap of 1e4: the others weigh exp(-1e4) == 0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o - v[0, 3])) <= 1e-12
    assert np.max(np.abs(lse - 1.0e4)) <= 1e-9
    k[0, 5, 0] = 1.0  # keys 3 and 5 tie at the top
    o, lse = fn(q, k, v, 1.0e4)
    assert np.max(np.abs(o - 0.5 * (v[0, 3] + v[0, 5]))) <= 1e-12
    assert np.max(np.abs(lse - (1.0e4 + math.log(2.0)))) <= 1e-9


def pin_permutations(fn):
    """Permuting K and V rows together leaves O, LSE unchanged; permuting Q rows
    permutes them."""
    rng = _rng(5)
    n, d = 40, 8
    q, k, v = (rng.standard_normal((2, n, d)) for _ in range(3))
    o, lse = fn(q, k, v, 0.6)
    pk = rng.permutation(n)
    o2, lse2 = fn(q, k[:, pk], v[:, pk], 0.6)
    assert np.max(np.abs(o - o2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13
    pq = rng.permutation(n)
    o3, lse3 = fn(q[:, pq], k, v, 0.6)
    assert np.max(np.abs(o[:, pq] - o3)) <= 1e-13 and np.max(np.abs(lse[:, pq] - lse3)) <= 1e-13


def pin_shift(fn):
    """q' = [q, c], k' = [k, 1]: every score of row i moves by scale*c_i, so O is
    unchanged and LSE moves by scale*c_i."""
    rng = _rng(6)
    n, d = 30, 6
    q, k, v = (rng.standard_normal((1, n, d)) for _ in range(3))
    c = 5.0 * rng.standard_normal((1, n, 1))
    q2 = np.concatenate([q, c], axis=-1)
    k2 = np.concatenate([k, np.ones((1, n, 1))], axis=-1)
    scale = 0.45
    o, lse = fn(q, k, v, scale)
    o2, lse2 = fn(q2, k2, v, scale)
    assert np.max(np.abs(o - o2)) <= 1e-13
    assert np.max(np.abs(lse2 - (lse + scale * c[..., 0]))) <= 1e-12


def support_function_bounds(o, v, n_dirs=16, seed=7):
    """Worst violation of the convex-hull bound of O's rows by V's rows.

    For random unit directions w: w.O_i must lie in [min_j w.v_j, max_j w.v_j].
    o [..., N, dv], v [..., N, dv]; returns the largest excess (<= 0 if inside).
    """
    o = np.asarray(o, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rng = _rng(seed)
    w = rng.standard_normal((v.shape[-1], n_dirs))
    w /= np.linalg.norm(w, axis=0, keepdims=True)
    pv = v @ w  # [..., N, n_dirs]
    po = o @ w
    hi = pv.max(axis=-2, keepdims=True)
    lo = pv.min(axis=-2, keepdims=True)
    return float(max(np.max(po - hi), np.max(lo - po)))


def pin_convex_hull(fn):
    rng = _rng(8)
    q, k, v = (2.0 * rng.standard_normal((3, 64, 10)) for _ in range(3))
    o, _ = fn(q, k, v, 0.9)
    assert support_function_bounds(o, v) <= 1e-13


def pin_library_sdpa(fn):
    """Against torch's own CPU attention and logsumexp in float64 (an
    independent implementation of the same definition)."""
    import torch
    import torch.nn.functional as F

    rng = _rng(9)
    for (b, h, n, d) in ((2, 3, 37, 16), (1, 2, 300, 64)):
        q, k, v = (rng.standard_normal((b, h, n, d)) for _ in range(3))
        scale = 1.0 / math.sqrt(d)
        o, lse = fn(q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        with torch.no_grad():
            o_t = F.scaled_dot_product_attention(tq, tk, tv, scale=scale).numpy()
            lse_t = torch.logsumexp(scale * (tq @ tk.transpose(-1, -2)), dim=-1).numpy()
        assert np.max(np.abs(o - o_t)) <= 1e-12, (b, h, n, d)
        assert np.max(np.abs(lse - lse_t)) <= 1e-12, (b, h, n, d)


ALL_PINS = [
    pin_brute_force,
    pin_single_key,
    pin_two_keys,
    pin_uniform_scores,
    pin_constant_values,
    pin_identity_values,
    pin_huge_gap_and_ties,
    pin_permutations,
    pin_shift,
    pin_convex_hull,
    pin_library_sdpa,
]


# ---------------------------------------------------------------------------
# Causal (prefill) attention: query i sees keys j <= i. Each pin takes
# fn(q, k, v, scale) -> (O, LSE) computing causal attention.
# ---------------------------------------------------------------------------


def pin_causal_brute_force(fn, tol=1e-13):
    """Tiny N against the decimal brute force over keys 0..i."""
    for n, d in [(1, 3), (2, 4), (3, 4), (6, 5), (17, 8)]:
        rng = _rng(300 + n + d)
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        for scale in (0.45, 2.0):
            o, lse = fn(q[None], k[None], v[None], scale)
            o_ref, lse_ref = decimal_attention(q, k, v, scale, causal=True)
            assert np.max(np.abs(o[0] - o_ref)) <= tol, (n, d, scale, "O")
            assert np.max(np.abs(lse[0] - lse_ref)) <= tol * max(1.0, np.max(np.abs(lse_ref))), (n, d, scale)


def pin_causal_first_row(fn):
    """Row 0 sees key 0 alone: O_0 = v_0 exactly and LSE_0 = scale q_0.k_0."""
    rng = _rng(301)
    q, k, v = (rng.standard_normal((2, 40, 16)) for _ in range(3))
    o, lse = fn(q, k, v, 0.3)
    assert np.max(np.abs(o[:, 0] - v[:, 0])) <= 1e-15
    expect = 0.3 * np.einsum("bd,bd->b", q[:, 0], k[:, 0])
    assert np.max(np.abs(lse[:, 0] - expect)) <= 1e-14


def pin_causal_uniform(fn):
    """scale = 0: row i is the mean of v_0..v_i and LSE_i = ln(i + 1)."""
    rng = _rng(302)
    n = 70
    q, k, v = (rng.standard_normal((2, n, 8)) for _ in range(3))
    o, lse = fn(q, k, v, 0.0)
    prefix_mean = np.cumsum(v, axis=1) / np.arange(1, n + 1)[None, :, None]
    assert np.max(np.abs(o - prefix_mean)) <= 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, n + 1))[None])) <= 1e-13


def pin_causal_prefix(fn):
    """No future token leaks: the first n rows of the full sequence equal the
    causal attention of the sequence cut after n tokens, and changing a later
    token leaves them unchanged."""
    rng = _rng(303)
    N = 60
    q, k, v = (2.0 * rng.standard_normal((1, N, 12)) for _ in range(3))
    o, lse = fn(q, k, v, 0.5)
    for n in (1, 7, 33, 59):
        o_n, lse_n = fn(q[:, :n], k[:, :n], v[:, :n], 0.5)
        assert np.max(np.abs(o[:, :n] - o_n)) <= 1e-14, n
        assert np.max(np.abs(lse[:, :n] - lse_n)) <= 1e-14, n
    k2, v2 = k.copy(), v.copy()
    k2[:, 40:] += 100.0
    v2[:, 40:] -= 50.0
    o2, lse2 = fn(q, k2, v2, 0.5)
    assert np.max(np.abs(o2[:, :40] - o[:, :40])) <= 1e-14
    assert np.max(np.abs(lse2[:, :40] - lse[:, :40])) <= 1e-14


def pin_causal_library(fn):
    """torch's CPU attention with is_causal=True and logsumexp over the
    lower-triangular scores, float64."""
    import torch
    import torch.nn.functional as F

    rng = _rng(304)
    for (b, h, n, d) in ((1, 2, 45, 16), (2, 1, 129, 32)):
        q, k, v = (rng.standard_normal((b, h, n, d)) for _ in range(3))
        scale = 1.0 / math.sqrt(d)
        o, lse = fn(q, k, v, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        with torch.no_grad():
            o_t = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, is_causal=True).numpy()
            s_t = scale * (tq @ tk.transpose(-1, -2))
            s_t = s_t.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
            lse_t = torch.logsumexp(s_t, dim=-1).numpy()
        assert np.max(np.abs(o - o_t)) <= 1e-12, (b, h, n, d)
        assert np.max(np.abs(lse - lse_t)) <= 1e-12, (b, h, n, d)


CAUSAL_PINS = [
    pin_causal_brute_force,
    pin_causal_first_row,
    pin_causal_uniform,
    pin_causal_prefix,
    pin_causal_library,
]


def failing_pins(fn, pins=None):
    """Names of the pins that ``fn`` fails (an exception counts as a failure)."""
    bad = []
    for pin in ALL_PINS if pins is None else pins:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts
            bad.append(pin.__name__)
    return bad


# ---------------------------------------------------------------------------
# Backward pass: each pin takes bwd(q, k, v, do, scale, causal) -> (dQ, dK, dV).
# ---------------------------------------------------------------------------


def _forward_loss(q, k, v, do, scale, causal):
    """L = sum(O * dO), with O from the (separately pinned) forward oracle."""
    from oracle import attention_reference

    o, _ = attention_reference(q, k, v, scale, causal=causal)
    return float(np.sum(o * do))


def pin_bwd_finite_differences(bwd, tol=2e-8):
    """Every gradient entry against a central difference of L = sum(O * dO)."""
    for causal in (False, True):
        rng = _rng(400 + causal)
        n, d = 5, 3
        q, k, v, do = (rng.standard_normal((1, n, d)) for _ in range(4))
        scale = 0.7
        grads = bwd(q, k, v, do, scale, causal)
        h = 1e-5
        for which, x in enumerate((q, k, v)):
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                fd = (_forward_loss(*args_p, do, scale, causal) - _forward_loss(*args_m, do, scale, causal)) / (2 * h)
                assert abs(grads[which][idx] - fd) <= tol * max(1.0, abs(fd)), (causal, which, idx, grads[which][idx], fd)


def pin_bwd_library(bwd):
    """torch's float64 autograd through its own CPU attention (causal too)."""
    import torch
    import torch.nn.functional as F

    rng = _rng(401)
    for causal in (False, True):
        for (b, h, n, d) in ((1, 2, 33, 8), (2, 1, 70, 16)):
            q, k, v, do = (rng.standard_normal((b, h, n, d)) for _ in range(4))
            scale = 1.0 / math.sqrt(d)
            dq, dk, dv = bwd(q, k, v, do, scale, causal)
            tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale, is_causal=causal)
            o.backward(torch.from_numpy(do))
            for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
                assert np.max(np.abs(mine - ref.numpy())) <= 1e-12, (causal, b, h, n, d)


def pin_bwd_single_key(bwd):
    """N = 1: O = v_0 whatever q, k, so dV = dO and dQ = dK = 0."""
    rng = _rng(402)
    q, k, v, do = (rng.standard_normal((2, 1, 7)) for _ in range(4))
    dq, dk, dv = bwd(q, k, v, do, 0.8, False)
    assert np.max(np.abs(dv - do)) <= 1e-15
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15


def pin_bwd_zero_scale(bwd):
    """scale = 0: uniform weights, so dQ = dK = 0 and dV_j = mean_i dO_i
    (causal: dV_j = sum over i >= j of dO_i / (i + 1))."""
    rng = _rng(403)
    n = 20
    q, k, v, do = (rng.standard_normal((1, n, 6)) for _ in range(4))
    dq, dk, dv = bwd(q, k, v, do, 0.0, False)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    assert np.max(np.abs(dv - do.mean(axis=1, keepdims=True))) <= 1e-14
    dq, dk, dv = bwd(q, k, v, do, 0.0, True)
    expect = np.stack([sum(do[0, i] / (i + 1) for i in range(j, n)) for j in range(n)])[None]
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    assert np.max(np.abs(dv - expect)) <= 1e-14


def pin_bwd_linear_in_upstream(bwd):
    """Gradients are linear in dO."""
    rng = _rng(404)
    q, k, v, d1, d2 = (rng.standard_normal((2, 25, 8)) for _ in range(5))
    for causal in (False, True):
        a = bwd(q, k, v, d1, 0.4, causal)
        b = bwd(q, k, v, d2, 0.4, causal)
        c = bwd(q, k, v, 2.0 * d1 - 3.0 * d2, 0.4, causal)
        for x, y, z in zip(a, b, c):
            assert np.max(np.abs(z - (2.0 * x - 3.0 * y))) <= 1e-12


def pin_bwd_key_shift(bwd):
    """Adding one vector to every key moves each row's scores by a constant, so
    the output does not change: the key gradients sum to zero over the keys."""
    rng = _rng(405)
    q, k, v, do = (2.0 * rng.standard_normal((2, 40, 8)) for _ in range(4))
    for causal in (False, True):
        _, dk, _ = bwd(q, k, v, do, 0.5, causal)
        assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12 * max(1.0, np.max(np.abs(dk)))


def pin_bwd_causal_future(bwd):
    """Causal: with dO zero after position t, keys and values after t get no
    gradient (no query that sees them has an upstream gradient)."""
    rng = _rng(406)
    q, k, v, do = (rng.standard_normal((1, 30, 8)) for _ in range(4))
    do[:, 18:] = 0.0
    _, dk, dv = bwd(q, k, v, do, 0.6, True)
    assert np.max(np.abs(dk[:, 18:])) == 0.0 and np.max(np.abs(dv[:, 18:])) == 0.0
    assert np.max(np.abs(dv[:, :18])) > 0.0


BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_library,
    pin_bwd_single_key,
    pin_bwd_zero_scale,
    pin_bwd_linear_in_upstream,
    pin_bwd_key_shift,
    pin_bwd_causal_future,
]


def pin_bwd_cols_subset(cols_fn):
    """A column-wise gradient (cols_fn(q, k, v, do, scale, cols, causal) ->
    (dK rows, dV rows)) of a few keys, in any order, equals those keys' rows of
    the same function over every key: each key's gradient is a sum over all
    query rows, whose softmax runs over every key the row sees, not only the
    chosen ones."""
    rng = _rng(407)
    q, k, v, do = (2.0 * rng.standard_normal((2, 45, 8)) for _ in range(4))
    for causal in (False, True):
        dk_all, dv_all = cols_fn(q, k, v, do, 0.55, range(45), causal)
        pick = [44, 3, 0, 21]
        dk, dv = cols_fn(q, k, v, do, 0.55, pick, causal)
        assert np.max(np.abs(dk - dk_all[:, pick])) <= 1e-13 * max(1.0, np.max(np.abs(dk_all)))
        assert np.max(np.abs(dv - dv_all[:, pick])) <= 1e-13 * max(1.0, np.max(np.abs(dv_all)))

