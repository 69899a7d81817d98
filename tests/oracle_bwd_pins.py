"""Pins for the fp64 backward oracle (gradients of O with respect to Q, K, V).

Each ``pin_bwd_*`` raises AssertionError when ``oracle.attention``'s
gradient functions disagree with a fact that does not come from them: the
forward oracle differentiated by central finite differences, closed forms
(one key, zero scale), invariants of the function (translating every key
leaves O unchanged; every row of P sums to one), the structure of grouped
and packed attention, and a library's automatic differentiation of the
plain expression. The functions look the oracle up at call time, so a test
can plant a mistake in ``oracle.attention`` and see which pins catch it.
"""
from __future__ import annotations

import numpy as np

import oracle.attention as A
from oracle_pins import _assert_close, _rng

FD_EPS = 1e-5     # central differences in fp64: truncation ~eps^2, rounding ~1e-16/eps
FD_TOL = 1e-8


def _loss_grads_fd(q, k, v, do, scale, causal, cu=None, directions=3, seed=0):
    """Directional derivatives of L = sum(dO * O(Q, K, V)) along random
    directions, by central differences of the forward oracle."""
    rng = _rng(seed)

    def loss(qq, kk, vv):
        o, _ = A.attention_ref(qq, kk, vv, scale, causal, cu)
        return float((o * do).sum())

    out = []
    for _ in range(directions):
        eq, ek, ev = (rng.standard_normal(x.shape) for x in (q, k, v))
        dq_fd = (loss(q + FD_EPS * eq, k, v) - loss(q - FD_EPS * eq, k, v)) / (2 * FD_EPS)
        dk_fd = (loss(q, k + FD_EPS * ek, v) - loss(q, k - FD_EPS * ek, v)) / (2 * FD_EPS)
        dv_fd = (loss(q, k, v + FD_EPS * ev) - loss(q, k, v - FD_EPS * ev)) / (2 * FD_EPS)
        out.append(((eq, dq_fd), (ek, dk_fd), (ev, dv_fd)))
    return out


def pin_bwd_finite_differences():
    """<dQ, E> etc. equal the directional derivatives of sum(dO * O) taken by
    central differences of the forward oracle: causal and not, GQA, Nq != Nk,
    packed sequences."""
    rng = _rng(101)
    cases = [
        (rng.standard_normal((2, 7, 4, 6)), rng.standard_normal((2, 9, 2, 6)), False, None),
        (rng.standard_normal((1, 9, 2, 5)), rng.standard_normal((1, 9, 1, 5)), True, None),
        (rng.standard_normal((1, 9, 2, 5)), rng.standard_normal((1, 6, 2, 5)), True, None),
    ]
    for qshape_arr, kshape_arr, causal, _ in cases:
        q = qshape_arr
        k = kshape_arr
        v = rng.standard_normal(k.shape)
        do = rng.standard_normal(q.shape)
        dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.7, causal)
        for (eq, a), (ek, b), (ev, c) in _loss_grads_fd(q, k, v, do, 0.7, causal):
            _assert_close(float((dq * eq).sum()), a, FD_TOL * max(1.0, abs(a)), "dQ directional")
            _assert_close(float((dk * ek).sum()), b, FD_TOL * max(1.0, abs(b)), "dK directional")
            _assert_close(float((dv * ev).sum()), c, FD_TOL * max(1.0, abs(c)), "dV directional")
    cu = np.array([0, 4, 4, 11, 12])
    q = rng.standard_normal((12, 4, 3))
    k = rng.standard_normal((12, 2, 3))
    v = rng.standard_normal((12, 2, 3))
    do = rng.standard_normal((12, 4, 3))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.9, True, cu_seqlens=cu)
    for (eq, a), (ek, b), (ev, c) in _loss_grads_fd(q, k, v, do, 0.9, True, cu):
        _assert_close(float((dq * eq).sum()), a, FD_TOL * max(1.0, abs(a)), "packed dQ")
        _assert_close(float((dk * ek).sum()), b, FD_TOL * max(1.0, abs(b)), "packed dK")
        _assert_close(float((dv * ev).sum()), c, FD_TOL * max(1.0, abs(c)), "packed dV")


def pin_bwd_elementwise_numeric_gradient():
    """Every element of dQ, dK, dV of a tiny causal case against its own
    central difference (brute force over all inputs)."""
    rng = _rng(102)
    q = rng.standard_normal((1, 3, 1, 2))
    k = rng.standard_normal((1, 4, 1, 2))
    v = rng.standard_normal((1, 4, 1, 2))
    do = rng.standard_normal((1, 3, 1, 2))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 1.1, True)

    def loss(qq, kk, vv):
        return float((A.attention_ref(qq, kk, vv, 1.1, True)[0] * do).sum())

    for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += FD_EPS
            xm[idx] -= FD_EPS
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = xp
            args_m[which] = xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * FD_EPS)
        _assert_close(g, num, FD_TOL, f"elementwise gradient {'QKV'[which]}")


def pin_bwd_single_key():
    """One key: P = 1, O = v for every row, so dQ = dK = 0 and dV is the sum
    of dO over all query rows of the heads that read it."""
    rng = _rng(103)
    q = rng.standard_normal((2, 5, 4, 3))
    k = rng.standard_normal((2, 1, 2, 3))
    v = rng.standard_normal((2, 1, 2, 3))
    do = rng.standard_normal((2, 5, 4, 3))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.8, False)
    _assert_close(dq, np.zeros_like(dq), 1e-14, "single key dQ")
    _assert_close(dk, np.zeros_like(dk), 1e-14, "single key dK")
    want = do.reshape(2, 5, 2, 2, 3).sum(axis=(1, 3))[:, None]
    _assert_close(dv, want, 1e-13, "single key dV")


def pin_bwd_zero_scale():
    """scale 0: P is uniform over the visible keys and does not depend on Q
    or K, so dQ = dK = 0; dV_j = sum_i dO_i / (number of keys row i sees)
    (all Lk keys, or i+1 keys under the causal mask)."""
    rng = _rng(104)
    q = rng.standard_normal((1, 6, 1, 4))
    k = rng.standard_normal((1, 6, 1, 4))
    v = rng.standard_normal((1, 6, 1, 4))
    do = rng.standard_normal((1, 6, 1, 4))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.0, False)
    _assert_close(dq, np.zeros_like(dq), 1e-14, "scale 0 dQ")
    _assert_close(dk, np.zeros_like(dk), 1e-14, "scale 0 dK")
    _assert_close(dv[0, :, 0], np.broadcast_to(do[0, :, 0].sum(0) / 6, (6, 4)), 1e-13,
                  "scale 0 dV")
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.0, True)
    want = np.stack([sum(do[0, i, 0] / (i + 1) for i in range(j, 6)) for j in range(6)])
    _assert_close(dv[0, :, 0], want, 1e-13, "scale 0 causal dV")
    _assert_close(dk, np.zeros_like(dk), 1e-14, "scale 0 causal dK")


def pin_bwd_key_translation():
    """Adding one vector u to every key adds scale q_i.u to every visible
    score of row i, which the row softmax ignores; so the directional
    derivative along (u, u, ..., u) vanishes: sum_j dK_j = 0 per sequence and
    K/V head, causal or not."""
    rng = _rng(105)
    for causal in (False, True):
        q = rng.standard_normal((2, 8, 4, 5))
        k = rng.standard_normal((2, 8, 2, 5))
        v = rng.standard_normal((2, 8, 2, 5))
        do = rng.standard_normal((2, 8, 4, 5))
        _, dk, _ = A.attention_bwd_ref(q, k, v, do, 0.6, causal)
        _assert_close(dk.sum(axis=1), np.zeros((2, 2, 5)), 1e-12, "sum of dK over keys")


def pin_bwd_dv_column_sum():
    """Rows of P sum to one, so sum_j dV_j = sum_j sum_i P_ij dO_i is the sum
    of dO over all query rows that see a key."""
    rng = _rng(106)
    q = rng.standard_normal((1, 7, 2, 3))
    k = rng.standard_normal((1, 5, 2, 3))
    v = rng.standard_normal((1, 5, 2, 3))
    do = rng.standard_normal((1, 7, 2, 3))
    for causal in (False, True):
        _, _, dv = A.attention_bwd_ref(q, k, v, do, 0.9, causal)
        _assert_close(dv.sum(axis=1), do.sum(axis=1), 1e-12, "sum of dV over keys")


def pin_bwd_gqa_is_repeated_heads():
    """Grouped K/V gradients equal the per-head gradients with K and V
    repeated for each query head, summed over each group."""
    rng = _rng(107)
    q = rng.standard_normal((1, 6, 6, 4))
    k = rng.standard_normal((1, 6, 2, 4))
    v = rng.standard_normal((1, 6, 2, 4))
    do = rng.standard_normal((1, 6, 6, 4))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.5, True)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    dq2, dk2, dv2 = A.attention_bwd_ref(q, kr, vr, do, 0.5, True)
    _assert_close(dq, dq2, 1e-13, "GQA dQ")
    _assert_close(dk, dk2.reshape(1, 6, 2, 3, 4).sum(axis=3), 1e-13, "GQA dK")
    _assert_close(dv, dv2.reshape(1, 6, 2, 3, 4).sum(axis=3), 1e-13, "GQA dV")


def pin_bwd_packed_is_independent():
    """Packed sequences give the gradients of separate fixed-length calls."""
    rng = _rng(108)
    cu = np.array([0, 5, 5, 12])
    q = rng.standard_normal((12, 2, 3))
    k = rng.standard_normal((12, 1, 3))
    v = rng.standard_normal((12, 1, 3))
    do = rng.standard_normal((12, 2, 3))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.7, True, cu_seqlens=cu)
    for s in range(3):
        lo, hi = cu[s], cu[s + 1]
        if hi == lo:
            continue
        a, b, c = A.attention_bwd_ref(q[None, lo:hi], k[None, lo:hi], v[None, lo:hi],
                                      do[None, lo:hi], 0.7, True)
        _assert_close(dq[lo:hi], a[0], 1e-14, "packed dQ")
        _assert_close(dk[lo:hi], b[0], 1e-14, "packed dK")
        _assert_close(dv[lo:hi], c[0], 1e-14, "packed dV")


def pin_bwd_library_autograd():
    """torch.autograd (CPU, float64) of the plain expression
    softmax(scale Q K^T + mask) V agrees with the oracle."""
    import torch
    rng = _rng(109)
    for causal in (False, True):
        q = rng.standard_normal((1, 10, 2, 6))
        k = rng.standard_normal((1, 10, 1, 6))
        v = rng.standard_normal((1, 10, 1, 6))
        do = rng.standard_normal((1, 10, 2, 6))
        dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.45, causal)
        tq = torch.tensor(q, requires_grad=True)
        tk = torch.tensor(k, requires_grad=True)
        tv = torch.tensor(v, requires_grad=True)
        kk = tk.repeat_interleave(2, dim=2)
        vv = tv.repeat_interleave(2, dim=2)
        s = torch.einsum("bihd,bjhd->bhij", tq, kk) * 0.45
        if causal:
            mask = torch.ones(10, 10, dtype=torch.bool).tril()
            s = s.masked_fill(~mask, float("-inf"))
        o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vv)
        (o * torch.tensor(do)).sum().backward()
        _assert_close(dq, tq.grad.numpy(), 1e-12, "autograd dQ")
        _assert_close(dk, tk.grad.numpy(), 1e-12, "autograd dK")
        _assert_close(dv, tv.grad.numpy(), 1e-12, "autograd dV")


def pin_bwd_picked_rows():
    """Picked gradient rows agree with the full backward oracle."""
    rng = _rng(110)
    q = rng.standard_normal((2, 15, 4, 5))
    k = rng.standard_normal((2, 15, 2, 5))
    v = rng.standard_normal((2, 15, 2, 5))
    do = rng.standard_normal((2, 15, 4, 5))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.4, True)
    qp = np.array([[0, 0, 0], [1, 3, 14], [0, 2, 6]])
    kp = np.array([[0, 0, 0], [1, 1, 14], [1, 0, 7]])
    pq, pk, pv = A.attention_bwd_picked(q, k, v, do, 0.4, True, qp, kp)
    for r, (b, h, i) in enumerate(qp):
        _assert_close(pq[r], dq[b, i, h], 1e-13, "picked dQ")
    for r, (b, g, j) in enumerate(kp):
        _assert_close(pk[r], dk[b, j, g], 1e-13, "picked dK")
        _assert_close(pv[r], dv[b, j, g], 1e-13, "picked dV")
    cu = np.array([0, 6, 13])
    q = rng.standard_normal((13, 2, 4))
    k = rng.standard_normal((13, 1, 4))
    v = rng.standard_normal((13, 1, 4))
    do = rng.standard_normal((13, 2, 4))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.4, True, cu_seqlens=cu)
    pq, pk, pv = A.attention_bwd_picked(q, k, v, do, 0.4, True, [[1, 1, 3]], [[0, 0, 2], [1, 0, 6]],
                                        cu_seqlens=cu)
    _assert_close(pq[0], dq[6 + 3, 1], 1e-13, "picked packed dQ")
    _assert_close(pk[0], dk[2, 0], 1e-13, "picked packed dK")
    _assert_close(pv[1], dv[6 + 6, 0], 1e-13, "picked packed dV")


def pin_bwd_empty_and_zero_upstream():
    """No keys, no queries or dO = 0: every gradient is zero."""
    rng = _rng(111)
    q = rng.standard_normal((1, 4, 1, 3))
    k = rng.standard_normal((1, 4, 1, 3))
    v = rng.standard_normal((1, 4, 1, 3))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, np.zeros_like(q), 0.5, True)
    for g in (dq, dk, dv):
        _assert_close(g, np.zeros_like(g), 0.0, "zero upstream gradient")
    dq, dk, dv = A.attention_bwd_ref(q, k[:, :0], v[:, :0], rng.standard_normal(q.shape), 0.5, False)
    _assert_close(dq, np.zeros_like(dq), 0.0, "no keys dQ")
    assert dk.shape == (1, 0, 1, 3) and dv.shape == (1, 0, 1, 3)


def pin_bwd_window_finite_differences():
    """Gradients with a sliding window (causal and not) against central
    differences of the windowed forward oracle."""
    rng = _rng(112)
    for causal, win in ((True, (3, -1)), (False, (2, 1))):
        q = rng.standard_normal((1, 10, 2, 4))
        k = rng.standard_normal((1, 10, 1, 4))
        v = rng.standard_normal((1, 10, 1, 4))
        do = rng.standard_normal((1, 10, 2, 4))
        dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.6, causal, window=win)

        def loss(qq, kk, vv):
            return float((A.attention_ref(qq, kk, vv, 0.6, causal, window=win)[0] * do).sum())

        for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            e = rng.standard_normal(x.shape)
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[which] = x + FD_EPS * e
            args_m[which] = x - FD_EPS * e
            fd = (loss(*args_p) - loss(*args_m)) / (2 * FD_EPS)
            _assert_close(float((g * e).sum()), fd, FD_TOL * max(1.0, abs(fd)),
                          f"window directional {'QKV'[which]}")


def pin_bwd_bias_finite_differences():
    """Gradients with an additive bias (held fixed; causal and not, a bias
    with -inf entries, GQA) against central differences of the biased
    forward oracle."""
    rng = _rng(113)
    for causal, dead in ((True, False), (False, True)):
        q = rng.standard_normal((1, 8, 2, 4))
        k = rng.standard_normal((1, 9, 1, 4))
        v = rng.standard_normal((1, 9, 1, 4))
        do = rng.standard_normal((1, 8, 2, 4))
        bias = rng.standard_normal((1, 2, 8, 9)) * 1.5
        if dead:
            bias[0, 0, :, 3] = -np.inf
            bias[0, 1, 2, :] = -np.inf
        dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.6, causal, bias=bias)

        def loss(qq, kk, vv):
            return float((A.attention_ref(qq, kk, vv, 0.6, causal, bias=bias)[0] * do).sum())

        for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            e = rng.standard_normal(x.shape)
            args_p, args_m = [q, k, v], [q, k, v]
            args_p[which] = x + FD_EPS * e
            args_m[which] = x - FD_EPS * e
            fd = (loss(*args_p) - loss(*args_m)) / (2 * FD_EPS)
            _assert_close(float((g * e).sum()), fd, FD_TOL * max(1.0, abs(fd)),
                          f"bias directional {'QKV'[which]}")


def pin_bwd_bias_library_autograd():
    """torch.autograd (CPU, float64) of softmax(scale Q K^T + B + mask) V
    agrees with the oracle, for a bias per head and the causal mask."""
    import torch
    rng = _rng(114)
    q = rng.standard_normal((2, 10, 2, 6))
    k = rng.standard_normal((2, 10, 1, 6))
    v = rng.standard_normal((2, 10, 1, 6))
    do = rng.standard_normal((2, 10, 2, 6))
    bias = rng.standard_normal((1, 2, 10, 10))
    dq, dk, dv = A.attention_bwd_ref(q, k, v, do, 0.45, True, bias=bias)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(2, dim=2)
    vv = tv.repeat_interleave(2, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kk) * 0.45 + torch.tensor(bias)
    s = s.masked_fill(~torch.ones(10, 10, dtype=torch.bool).tril(), float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(do)).sum().backward()
    _assert_close(dq, tq.grad.numpy(), 1e-12, "autograd bias dQ")
    _assert_close(dk, tk.grad.numpy(), 1e-12, "autograd bias dK")
    _assert_close(dv, tv.grad.numpy(), 1e-12, "autograd bias dV")
    qp = np.array([[0, 1, 9], [1, 0, 3]])
    kp = np.array([[1, 0, 0], [0, 0, 7]])
    pq, pk, pv = A.attention_bwd_picked(q, k, v, do, 0.45, True, qp, kp, bias=bias)
    for r, (b, h, i) in enumerate(qp):
        _assert_close(pq[r], dq[b, i, h], 1e-13, "picked bias dQ")
    for r, (b, g, j) in enumerate(kp):
        _assert_close(pk[r], dk[b, j, g], 1e-13, "picked bias dK")
        _assert_close(pv[r], dv[b, j, g], 1e-13, "picked bias dV")


ALL_BWD_PINS = [
    pin_bwd_finite_differences, pin_bwd_elementwise_numeric_gradient, pin_bwd_single_key,
    pin_bwd_zero_scale, pin_bwd_key_translation, pin_bwd_dv_column_sum,
    pin_bwd_gqa_is_repeated_heads, pin_bwd_packed_is_independent, pin_bwd_library_autograd,
    pin_bwd_picked_rows, pin_bwd_empty_and_zero_upstream, pin_bwd_window_finite_differences,
    pin_bwd_bias_finite_differences, pin_bwd_bias_library_autograd,
]
