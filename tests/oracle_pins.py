"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a fact that does not come from the oracle itself: a closed form, an
invariant, a special case that reduces to a textbook routine, a brute-force
evaluation on tiny inputs, a second route through the online recurrence, or
a library routine. The functions look the oracle up at call time, so a test
can plant a mistake in ``oracle.attention`` and see which pins catch it.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.attention as A

TIGHT = 1e-13          # fp64 agreement for identities that hold exactly
ROUTE = 1e-12          # fp64 agreement between two different summation routes


def _rng(seed):
    return np.random.default_rng(seed)


def _assert_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(both_inf, 0.0, np.abs(a - b))
    assert np.all(np.isfinite(diff)), f"{what}: non-finite mismatch"
    err = float(diff.max()) if diff.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# Independent routes (written here, sharing nothing with the oracle)
# ---------------------------------------------------------------------------

def brute_force(q, k, v, scale, causal, cu_seqlens=None):
    """Pure-Python per-row evaluation with math.exp and math.fsum.

    Follows "Softmax does not need the matrix", *Carry the Normalizer*:
    s_j = scale * q.k_j, m = max s, p_j = exp(s_j - m) / sum exp(s_i - m),
    o = sum p_j v_j; LSE = m + log(sum exp(s_j - m)). Tiny shapes only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if cu_seqlens is None:
        units = [(b, (b, slice(None)), q.shape[1], k.shape[1]) for b in range(q.shape[0])]
        hq, hkv, d = q.shape[2], k.shape[2], q.shape[3]
    else:
        cu = [int(x) for x in cu_seqlens]
        units = [(s, (slice(cu[s], cu[s + 1]),), cu[s + 1] - cu[s], cu[s + 1] - cu[s])
                 for s in range(len(cu) - 1)]
        hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    out = np.zeros_like(q)
    lse = (np.full((q.shape[0], hq, q.shape[1]), -np.inf) if cu_seqlens is None
           else np.full((hq, q.shape[0]), -np.inf))
    group = hq // hkv
    for s, idx, lq, lk in units:
        qs, ks, vs = q[idx], k[idx], v[idx]
        for h in range(hq):
            g = h // group
            for i in range(lq):
                keys = [j for j in range(lk) if (not causal or j <= i)]
                if not keys:
                    continue
                sc = [scale * math.fsum(float(qs[i, h, t]) * float(ks[j, g, t]) for t in range(d))
                      for j in keys]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                l = math.fsum(e)
                row = [math.fsum(e[n] * float(vs[j, g, t]) for n, j in enumerate(keys)) / l
                       for t in range(d)]
                if cu_seqlens is None:
                    out[s, i, h] = row
                    lse[s, h, i] = m + math.log(l)
                else:
                    base = int(cu_seqlens[s])
                    out[base + i, h] = row
                    lse[h, base + i] = m + math.log(l)
    return out, lse


def online_blockwise(q, k, v, scale, causal, block):
    """The online recurrence of "Softmax does not need the matrix",
    *Carry the Normalizer*, in fp64, over key blocks of size ``block``:
    m' = max(m, m_b); l' = e^(m-m') l + sum_b e^(s_j-m');
    a' = e^(m-m') a + sum_b e^(s_j-m') v_j; o = a / l.

    Single head: q [Lq, d], k and v [Lk, d]. Returns (O, LSE, rescales) where
    ``rescales`` counts block updates that raised a row's running maximum
    after its first block.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    m = np.full(lq, -np.inf)
    l = np.zeros(lq)
    a = np.zeros((lq, v.shape[1]))
    rescales = 0
    i = np.arange(lq)[:, None]
    for j0 in range(0, lk, block):
        kb, vb = k[j0:j0 + block], v[j0:j0 + block]
        s = scale * np.einsum("id,jd->ij", q, kb)
        if causal:
            j = np.arange(j0, j0 + len(kb))[None, :]
            s = np.where(j <= i, s, -np.inf)
        mb = s.max(axis=1)
        mn = np.maximum(m, mb)
        live = np.isfinite(mn)
        alpha = np.where(live & np.isfinite(m), np.exp(np.where(live, m - mn, 0.0)), 0.0)
        rescales += int(np.sum(np.isfinite(m) & (mn > m)))
        e = np.where(live[:, None], np.exp(s - np.where(live, mn, 0.0)[:, None]), 0.0)
        l = alpha * l + e.sum(axis=1)
        a = alpha[:, None] * a + e @ vb
        m = mn
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(l[:, None] > 0, a / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse, rescales


# ---------------------------------------------------------------------------
# Pins
# ---------------------------------------------------------------------------

def pin_rows_sum_to_one():
    """I1: every row of P sums to 1, and exp(S - LSE) sums to 1 per row."""
    rng = _rng(1)
    s = rng.standard_normal((7, 33)) * 5
    s[:, 20:] = -np.inf                      # a masked tail
    p, m, l = A.softmax_rows(s)
    _assert_close(p.sum(axis=1), np.ones(7), TIGHT, "sum P")
    assert np.all(p[:, 20:] == 0), "masked entries must get probability 0"
    _assert_close(m, s[:, :20].max(axis=1), 0.0, "row max")
    q = rng.standard_normal((1, 9, 2, 4))
    k = rng.standard_normal((1, 9, 2, 4))
    v = rng.standard_normal((1, 9, 2, 4))
    for causal in (False, True):
        _, lse = A.attention_ref(q, k, v, 0.7, causal)
        for h in range(2):
            sc = 0.7 * q[0, :, h] @ k[0, :, h].T
            if causal:
                sc = np.where(np.tril(np.ones((9, 9), bool)), sc, -np.inf)
            _assert_close(np.exp(sc - lse[0, h][:, None]).sum(axis=1), np.ones(9), TIGHT,
                          "sum exp(S-LSE)")


def pin_single_key():
    """I2: with one key, p = 1, so O = v exactly and LSE = scale * q.k."""
    rng = _rng(2)
    q = rng.standard_normal((2, 5, 3, 8))
    k = rng.standard_normal((2, 1, 3, 8))
    v = rng.standard_normal((2, 1, 3, 8))
    o, lse = A.attention_ref(q, k, v, 0.35, False)
    assert np.array_equal(o, np.broadcast_to(v, o.shape)), "O must equal v bit-exactly"
    want = np.empty_like(lse)
    for b in range(2):
        for h in range(3):
            for i in range(5):
                want[b, h, i] = 0.35 * math.fsum(q[b, i, h] * k[b, 0, h])
    _assert_close(lse, want, TIGHT, "LSE single key")


def pin_uniform_scores_mean():
    """I3: all scores equal (identical keys, or scale 0) -> O = mean(V) and
    LSE = s + log(n)."""
    rng = _rng(3)
    n, d = 11, 6
    q = rng.standard_normal((1, 4, 2, d))
    kk = rng.standard_normal(d)
    k = np.broadcast_to(kk, (1, n, 2, d)).copy()
    v = rng.standard_normal((1, n, 2, d))
    mean = np.array([[math.fsum(v[0, :, h, t]) / n for t in range(d)] for h in range(2)])
    o, lse = A.attention_ref(q, k, v, 0.9, False)
    for h in range(2):
        _assert_close(o[0, :, h], np.broadcast_to(mean[h], (4, d)), TIGHT, "identical keys")
        want = [0.9 * math.fsum(q[0, i, h] * kk) + math.log(n) for i in range(4)]
        _assert_close(lse[0, h], want, TIGHT, "LSE identical keys")
    k2 = rng.standard_normal((1, n, 2, d))
    o0, lse0 = A.attention_ref(q, k2, v, 0.0, False)
    for h in range(2):
        _assert_close(o0[0, :, h], np.broadcast_to(mean[h], (4, d)), TIGHT, "scale 0")
    _assert_close(lse0, np.full(lse0.shape, math.log(n)), TIGHT, "LSE scale 0")


def pin_two_key_closed_form():
    """Closed form: two keys with scores 0 and ln 3 give weights 1/4, 3/4."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.0]], [[math.log(3.0)]]]])
    v = np.array([[[[2.0]], [[-6.0]]]])
    o, lse = A.attention_ref(q, k, v, 1.0, False)
    _assert_close(o.ravel(), [0.25 * 2.0 + 0.75 * -6.0], TIGHT, "two-key O")
    _assert_close(lse.ravel(), [math.log(4.0)], TIGHT, "two-key LSE")
    # causal: row 0 sees only key 0
    q2 = np.array([[[[1.0]], [[1.0]]]])
    o2, lse2 = A.attention_ref(q2, k, v, 1.0, True)
    _assert_close(o2.ravel(), [2.0, -4.0], TIGHT, "two-key causal O")
    _assert_close(lse2.ravel(), [0.0, math.log(4.0)], TIGHT, "two-key causal LSE")


def pin_permutation_invariance():
    """I4: non-causal O and LSE do not depend on the order of the (k, v) pairs."""
    rng = _rng(4)
    q = rng.standard_normal((1, 6, 2, 5))
    k = rng.standard_normal((1, 13, 2, 5))
    v = rng.standard_normal((1, 13, 2, 5))
    o, lse = A.attention_ref(q, k, v, 0.6, False)
    perm = rng.permutation(13)
    o2, lse2 = A.attention_ref(q, k[:, perm], v[:, perm], 0.6, False)
    _assert_close(o, o2, TIGHT, "permuted O")
    _assert_close(lse, lse2, TIGHT, "permuted LSE")
    # the pairing matters: permuting V alone must change O
    o3, _ = A.attention_ref(q, k, v[:, perm], 0.6, False)
    assert np.abs(o3 - o).max() > 1e-3, "O must depend on which v goes with which k"


def pin_brute_force():
    """I5: brute force on tiny shapes: plain, causal, GQA, packed, Nq != Nk."""
    rng = _rng(5)
    cases = [
        dict(b=2, nq=5, nk=5, hq=2, hkv=2, d=3, causal=False),
        dict(b=1, nq=6, nk=6, hq=4, hkv=2, d=4, causal=True),
        dict(b=1, nq=4, nk=7, hq=3, hkv=1, d=2, causal=False),
        dict(b=1, nq=7, nk=4, hq=2, hkv=1, d=3, causal=True),
    ]
    for c in cases:
        q = rng.standard_normal((c["b"], c["nq"], c["hq"], c["d"])) * 2
        k = rng.standard_normal((c["b"], c["nk"], c["hkv"], c["d"]))
        v = rng.standard_normal((c["b"], c["nk"], c["hkv"], c["d"]))
        o, lse = A.attention_ref(q, k, v, 0.8, c["causal"])
        ob, lb = brute_force(q, k, v, 0.8, c["causal"])
        _assert_close(o, ob, TIGHT, f"brute force O {c}")
        _assert_close(lse, lb, TIGHT, f"brute force LSE {c}")
    cu = np.array([0, 3, 3, 8, 9])
    q = rng.standard_normal((9, 4, 3)) * 2
    k = rng.standard_normal((9, 2, 3))
    v = rng.standard_normal((9, 2, 3))
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.5, causal, cu_seqlens=cu)
        ob, lb = brute_force(q, k, v, 0.5, causal, cu_seqlens=cu)
        _assert_close(o, ob, TIGHT, "brute force packed O")
        _assert_close(lse, lb, TIGHT, "brute force packed LSE")


def pin_online_route():
    """I6: the online block recurrence agrees with the materialised oracle for
    every block size (the two routes of "Softmax does not need the matrix",
    *A Row You Can Stream*: the error stays at floating-point noise)."""
    rng = _rng(6)
    for n, causal, spread in [(37, False, 1.0), (37, True, 1.0), (64, True, 6.0), (50, False, 6.0)]:
        q = rng.standard_normal((1, n, 1, 16)) * spread
        k = rng.standard_normal((1, n, 1, 16))
        v = rng.standard_normal((1, n, 1, 16))
        o, lse = A.attention_ref(q, k, v, 0.25, causal)
        for block in (1, 2, 3, 7, n):
            o2, l2, _ = online_blockwise(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.25, causal, block)
            _assert_close(o[0, :, 0], o2, ROUTE, f"online O block={block}")
            _assert_close(lse[0, 0], l2, ROUTE, f"online LSE block={block}")


def pin_causal_structure():
    """I7: causal row i equals non-causal attention over keys 0..i; row 0 is
    v_0; with scale 0 causal rows are prefix means."""
    rng = _rng(7)
    n, d = 9, 4
    q = rng.standard_normal((1, n, 1, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    o, lse = A.attention_ref(q, k, v, 0.5, True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]), "causal row 0 must equal v_0"
    for i in range(n):
        oi, li = A.attention_ref(q[:, i:i + 1], k[:, :i + 1], v[:, :i + 1], 0.5, False)
        _assert_close(o[0, i], oi[0, 0], TIGHT, f"causal row {i}")
        _assert_close(lse[0, 0, i], li[0, 0, 0], TIGHT, f"causal LSE row {i}")
    o0, lse0 = A.attention_ref(q, k, v, 0.0, True)
    for i in range(n):
        want = [math.fsum(v[0, :i + 1, 0, t]) / (i + 1) for t in range(d)]
        _assert_close(o0[0, i, 0], want, TIGHT, f"prefix mean row {i}")
        _assert_close(lse0[0, 0, i], math.log(i + 1), TIGHT, f"prefix LSE row {i}")


def pin_gqa_is_repeated_heads():
    """I8: GQA equals MHA with each K/V head repeated for its query-head group."""
    rng = _rng(8)
    q = rng.standard_normal((2, 6, 8, 4))
    k = rng.standard_normal((2, 6, 2, 4))
    v = rng.standard_normal((2, 6, 2, 4))
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.5, causal)
        kr, vr = np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2)
        o2, lse2 = A.attention_ref(q, kr, vr, 0.5, causal)
        _assert_close(o, o2, 0.0, "GQA O")
        _assert_close(lse, lse2, 0.0, "GQA LSE")
        # and head 5 really reads kv-head 1: a per-head call
        oh, lh = A.attention_ref(q[:, :, 5:6], k[:, :, 1:2], v[:, :, 1:2], 0.5, causal)
        _assert_close(o[:, :, 5:6], oh, 0.0, "GQA head 5")


def pin_packed_is_independent():
    """I9: packed sequences equal separate calls, and changing one sequence's
    K/V changes no other sequence's output."""
    rng = _rng(9)
    lens = [4, 1, 6, 0, 3]
    cu = np.concatenate([[0], np.cumsum(lens)])
    t = int(cu[-1])
    q = rng.standard_normal((t, 4, 3))
    k = rng.standard_normal((t, 2, 3))
    v = rng.standard_normal((t, 2, 3))
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.7, causal, cu_seqlens=cu)
        for s in range(len(lens)):
            lo, hi = cu[s], cu[s + 1]
            os_, ls_ = A.attention_ref(q[None, lo:hi], k[None, lo:hi], v[None, lo:hi], 0.7, causal)
            _assert_close(o[lo:hi], os_[0], 0.0, f"packed seq {s} O")
            _assert_close(lse[:, lo:hi], ls_[0], 0.0, f"packed seq {s} LSE")
        k2, v2 = k.copy(), v.copy()
        k2[cu[2]:cu[3]] += 3.0
        v2[cu[2]:cu[3]] -= 2.0
        o2, lse2 = A.attention_ref(q, k2, v2, 0.7, causal, cu_seqlens=cu)
        other = np.ones(t, bool)
        other[cu[2]:cu[3]] = False
        _assert_close(o2[other], o[other], 0.0, "isolation O")
        assert np.abs(o2[cu[2]:cu[3]] - o[cu[2]:cu[3]]).max() > 1e-3


def pin_shift_invariance():
    """I10: adding the same constant c to every score of a row leaves O
    unchanged and shifts LSE by exactly c (here c = 1000, which overflows a
    float64 exp unless the row maximum is subtracted first)."""
    rng = _rng(10)
    n, d = 12, 5
    q = rng.standard_normal((1, n, 1, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    o, lse = A.attention_ref(q, k, v, 1.0, False)
    q2 = np.concatenate([q, np.full((1, n, 1, 1), 1000.0)], axis=3)
    k2 = np.concatenate([k, np.ones((1, n, 1, 1))], axis=3)
    v2 = np.concatenate([v, np.zeros((1, n, 1, 1))], axis=3)
    o2, lse2 = A.attention_ref(q2, k2, v2, 1.0, False)
    _assert_close(o2[..., :d], o, 1e-12, "shifted O")
    _assert_close(lse2 - 1000.0, lse, 1e-10, "shifted LSE")


def pin_hard_max_limit():
    """I11: when the top score of each row beats the runner-up by a margin
    that underflows exp, O is the argmax key's value row exactly."""
    rng = _rng(11)
    n, d = 10, 4
    q = rng.standard_normal((1, n, 1, d))
    k = rng.standard_normal((1, n, 1, d))
    v = rng.standard_normal((1, n, 1, d))
    s = q[0, :, 0] @ k[0, :, 0].T
    srt = np.sort(s, axis=1)
    gap = (srt[:, -1] - srt[:, -2]).min()
    scale = 800.0 / gap                       # gap * scale = 800 > 745 (exp underflow)
    assert gap > 1e-3, "rows need a clear winner for this pin"
    o, lse = A.attention_ref(q, k, v, scale, False)
    arg = s.argmax(axis=1)
    assert np.array_equal(o[0, :, 0], v[0, arg, 0]), "hard-max rows must pick v_argmax"
    _assert_close(lse[0, 0], scale * s.max(axis=1), 1e-9 * scale, "hard-max LSE")


def pin_library_sdpa():
    """I12: torch's scaled_dot_product_attention (CPU, float64) and
    torch.logsumexp agree with the oracle, for plain, causal and GQA inputs."""
    import torch
    import torch.nn.functional as F
    rng = _rng(12)
    for causal, hq, hkv in [(False, 4, 4), (True, 4, 4), (True, 8, 2)]:
        q = rng.standard_normal((2, 24, hq, 16))
        k = rng.standard_normal((2, 24, hkv, 16))
        v = rng.standard_normal((2, 24, hkv, 16))
        o, lse = A.attention_ref(q, k, v, 0.3, causal)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, hq // hkv, axis=2)).permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, hq // hkv, axis=2)).permute(0, 2, 1, 3)
        to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3)
        _assert_close(o, to.permute(0, 2, 1, 3).numpy(), ROUTE, "SDPA O")
        sc = torch.matmul(tq, tk.transpose(-1, -2)) * 0.3
        if causal:
            sc = sc.masked_fill(~torch.ones(24, 24, dtype=torch.bool).tril(), float("-inf"))
        _assert_close(lse, torch.logsumexp(sc, dim=-1).numpy(), ROUTE, "logsumexp LSE")


def pin_empty_cases():
    """A row that sees no key: O = 0 and LSE = -inf (reading for Nk = 0 and
    empty packed sequences)."""
    q = np.ones((1, 3, 2, 4))
    k = np.ones((1, 0, 2, 4))
    v = np.ones((1, 0, 2, 4))
    o, lse = A.attention_ref(q, k, v, 0.5, False)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = A.attention_ref(q, k, v, 0.5, True)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def pin_picked_rows():
    """Row picks agree bit-for-bit with the full oracle (same route)."""
    rng = _rng(13)
    q = rng.standard_normal((2, 20, 4, 8))
    k = rng.standard_normal((2, 20, 2, 8))
    v = rng.standard_normal((2, 20, 2, 8))
    o, lse = A.attention_ref(q, k, v, 0.4, True)
    picks = np.array([[0, 0, 0], [1, 3, 19], [0, 2, 7], [1, 1, 5], [0, 0, 19]])
    po, pl = A.attention_picked(q, k, v, 0.4, True, picks)
    for r, (b, h, i) in enumerate(picks):
        _assert_close(po[r], o[b, i, h], 1e-15, "picked O")
        _assert_close(pl[r], lse[b, h, i], 1e-15, "picked LSE")
    cu = np.array([0, 7, 20, 26])
    qp = rng.standard_normal((26, 4, 8))
    kp = rng.standard_normal((26, 2, 8))
    vp = rng.standard_normal((26, 2, 8))
    o, lse = A.attention_ref(qp, kp, vp, 0.4, True, cu_seqlens=cu)
    picks = np.array([[0, 1, 6], [1, 3, 0], [2, 0, 5], [1, 2, 12]])
    po, pl = A.attention_picked(qp, kp, vp, 0.4, True, picks, cu_seqlens=cu)
    for r, (s, h, i) in enumerate(picks):
        _assert_close(po[r], o[cu[s] + i, h], 1e-15, "picked packed O")
        _assert_close(pl[r], lse[h, cu[s] + i], 1e-15, "picked packed LSE")


def pin_window_wide_equals_plain():
    """A window wider than the sequence changes nothing."""
    rng = _rng(31)
    q = rng.standard_normal((2, 9, 2, 4))
    k = rng.standard_normal((2, 11, 1, 4))
    v = rng.standard_normal((2, 11, 1, 4))
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.6, causal)
        ow, lw = A.attention_ref(q, k, v, 0.6, causal, window=(100, 100))
        _assert_close(ow, o, 0.0, "wide window O")
        _assert_close(lw, lse, 0.0, "wide window LSE")
        ow, lw = A.attention_ref(q, k, v, 0.6, causal, window=(-1, -1))
        _assert_close(ow, o, 0.0, "unbounded window O")


def pin_window_zero_left_causal():
    """Left window 0 under the causal mask: row i sees key i only, so
    O_i = v_i and LSE_i = scale * q_i . k_i."""
    rng = _rng(32)
    q = rng.standard_normal((1, 7, 1, 5))
    k = rng.standard_normal((1, 7, 1, 5))
    v = rng.standard_normal((1, 7, 1, 5))
    o, lse = A.attention_ref(q, k, v, 0.8, True, window=(0, -1))
    _assert_close(o, v, 1e-15, "zero left window O")
    want = 0.8 * np.einsum("bihd,bihd->bhi", q, k)
    _assert_close(lse, want, 1e-14, "zero left window LSE")


def pin_window_by_slicing():
    """Each row of a windowed call equals the unmasked oracle over that
    row's own key slice [i - left, i + right] (cut at 0, Lk and, causal, at
    i): slicing instead of masking, a different route."""
    rng = _rng(33)
    lq, lk, d = 12, 10, 4
    q = rng.standard_normal((lq, d))
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, d))
    for causal, win in ((False, (2, 3)), (True, (3, -1)), (False, (0, 0)), (True, (1, 5)),
                        (False, (-1, 1))):
        o, lse = A.attention_head(q, k, v, 0.7, causal, window=win)
        for i in range(lq):
            lo = 0 if win[0] < 0 else max(0, i - win[0])
            hi = lk if win[1] < 0 else min(lk, i + win[1] + 1)
            if causal:
                hi = min(hi, i + 1)
            if hi <= lo:
                assert np.all(o[i] == 0) and np.isneginf(lse[i]), "empty window row"
                continue
            oi, li = A.attention_head(q[i:i + 1], k[lo:hi], v[lo:hi], 0.7, False)
            _assert_close(o[i], oi[0], 1e-14, f"window row {i} O")
            _assert_close(lse[i], li[0], 1e-14, f"window row {i} LSE")


def pin_window_brute_force():
    """Pure-Python per-row evaluation over the explicit key range."""
    rng = _rng(34)
    q = rng.standard_normal((6, 3))
    k = rng.standard_normal((8, 3))
    v = rng.standard_normal((8, 3))
    o, lse = A.attention_head(q, k, v, 0.9, True, window=(2, -1))
    for i in range(6):
        keys = [j for j in range(8) if i - 2 <= j <= i]
        s = [0.9 * math.fsum(q[i, c] * k[j, c] for c in range(3)) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        for c in range(3):
            _assert_close(o[i, c], math.fsum(e[n] * v[keys[n], c] for n in range(len(keys))) / den,
                          1e-13, "window brute-force O")
        _assert_close(lse[i], m + math.log(den), 1e-13, "window brute-force LSE")


def pin_bias_row_constant():
    """A bias constant along each row (B_ij = c_i) cancels in the softmax:
    O is unchanged and LSE_i moves by exactly c_i. Per (batch entry, head)
    constants, causal and not, GQA, Nq != Nk."""
    rng = _rng(41)
    q = rng.standard_normal((2, 6, 3, 4))
    k = rng.standard_normal((2, 8, 1, 4))
    v = rng.standard_normal((2, 8, 1, 4))
    c = rng.standard_normal((2, 3, 6))
    bias = np.broadcast_to(c[..., None], (2, 3, 6, 8)).copy()
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.6, causal)
        ob, lb = A.attention_ref(q, k, v, 0.6, causal, bias=bias)
        _assert_close(ob, o, 1e-14, "row-constant bias O")
        _assert_close(lb, lse + c, 1e-13, "row-constant bias LSE")


def pin_bias_log_weights():
    """With Q = 0 every score is 0, so B_ij = log w_j makes each row the
    w-weighted mean of the visible values: O_i = sum w_j v_j / sum w_j and
    LSE_i = log sum w_j (sums over j <= i when causal). A textbook weighted
    mean; the bias is shared by all entries and heads ([1, 1, N, N])."""
    rng = _rng(42)
    n, d = 7, 3
    w = rng.uniform(0.1, 3.0, n)
    v = rng.standard_normal((1, n, 1, d))
    q = np.zeros((1, n, 2, d))
    k = rng.standard_normal((1, n, 1, d))
    bias = np.broadcast_to(np.log(w)[None, None, None, :], (1, 1, n, n))
    for causal in (False, True):
        o, lse = A.attention_ref(q, k, v, 0.5, causal, bias=bias)
        for i in range(n):
            js = np.arange(i + 1 if causal else n)
            want = (w[js, None] * v[0, js, 0]).sum(axis=0) / w[js].sum()
            for h in range(2):
                _assert_close(o[0, i, h], want, 1e-14, "log-weight bias O")
                _assert_close(lse[0, h, i], np.log(w[js].sum()), 1e-14, "log-weight bias LSE")


def pin_bias_as_mask():
    """A bias of 0 and -inf is a mask: the lower-triangular pattern gives the
    causal call, a band gives the windowed call, a row of -inf gives O = 0
    and LSE = -inf, and -inf where the causal mask already hides changes
    nothing."""
    rng = _rng(43)
    q = rng.standard_normal((1, 9, 2, 4))
    k = rng.standard_normal((1, 9, 2, 4))
    v = rng.standard_normal((1, 9, 2, 4))
    i = np.arange(9)[:, None]
    j = np.arange(9)[None, :]
    tri = np.where(j <= i, 0.0, -np.inf)[None, None]
    o, lse = A.attention_ref(q, k, v, 0.7, True)
    ob, lb = A.attention_ref(q, k, v, 0.7, False, bias=tri)
    _assert_close(ob, o, 0.0, "triangular bias O")
    _assert_close(lb, lse, 0.0, "triangular bias LSE")
    ob, lb = A.attention_ref(q, k, v, 0.7, True, bias=tri)
    _assert_close(ob, o, 0.0, "triangular bias under causal O")
    band = np.where((j >= i - 2) & (j <= i + 1), 0.0, -np.inf)[None, None]
    o, lse = A.attention_ref(q, k, v, 0.7, False, window=(2, 1))
    ob, lb = A.attention_ref(q, k, v, 0.7, False, bias=band)
    _assert_close(ob, o, 0.0, "band bias O")
    _assert_close(lb, lse, 0.0, "band bias LSE")
    dead = np.zeros((1, 2, 9, 9))
    dead[0, 1, 4, :] = -np.inf
    ob, lb = A.attention_ref(q, k, v, 0.7, False, bias=dead)
    assert np.all(ob[0, 4, 1] == 0) and np.isneginf(lb[0, 1, 4]), "fully masked row"
    o, lse = A.attention_ref(q, k, v, 0.7, False)
    keep = np.ones(o.shape, dtype=bool)
    keep[0, 4, 1] = False
    _assert_close(ob[keep], o[keep], 0.0, "other rows untouched")


def pin_bias_brute_force():
    """Pure-Python per-row evaluation of softmax(scale q.k_j + B_ij) with a
    random bias (not square, causal)."""
    rng = _rng(44)
    lq, lk, d = 5, 7, 3
    q = rng.standard_normal((lq, d))
    k = rng.standard_normal((lk, d))
    v = rng.standard_normal((lk, d))
    b = rng.standard_normal((lq, lk)) * 2.0
    o, lse = A.attention_head(q, k, v, 0.8, True, bias=b)
    for i in range(lq):
        keys = range(min(lk, i + 1))
        s = [0.8 * math.fsum(q[i, c] * k[j, c] for c in range(d)) + b[i, j] for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        for c in range(d):
            _assert_close(o[i, c], math.fsum(e[n] * v[j, c] for n, j in enumerate(keys)) / den,
                          1e-13, "bias brute-force O")
        _assert_close(lse[i], m + math.log(den), 1e-13, "bias brute-force LSE")


def pin_bias_library_sdpa():
    """torch's scaled_dot_product_attention with an additive float mask
    (CPU, float64) and torch.logsumexp agree with the oracle: a bias per
    (entry, head), one shared over heads, and one combined with the causal
    mask."""
    import torch
    import torch.nn.functional as F
    rng = _rng(45)
    q = rng.standard_normal((2, 12, 4, 8))
    k = rng.standard_normal((2, 12, 2, 8))
    v = rng.standard_normal((2, 12, 2, 8))
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, 2, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, 2, axis=2)).permute(0, 2, 1, 3)
    tri = torch.zeros(12, 12, dtype=torch.float64).masked_fill(
        ~torch.ones(12, 12, dtype=torch.bool).tril(), float("-inf"))
    for shape, causal in (((2, 4, 12, 12), False), ((1, 4, 12, 12), True), ((2, 1, 12, 12), False)):
        bias = rng.standard_normal(shape) * 1.5
        o, lse = A.attention_ref(q, k, v, 0.35, causal, bias=bias)
        mask = torch.from_numpy(bias) + (tri if causal else 0.0)
        to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.35)
        _assert_close(o, to.permute(0, 2, 1, 3).numpy(), ROUTE, "SDPA bias O")
        sc = torch.matmul(tq, tk.transpose(-1, -2)) * 0.35 + mask
        _assert_close(lse, torch.logsumexp(sc, dim=-1).numpy(), ROUTE, "logsumexp bias LSE")


def pin_bias_packed():
    """Packed sequences with a per-sequence bias block [nseq, Hq, Lmax, Lmax]
    (local indices) equal separate fixed-length calls, each with its own
    block cut to its length."""
    rng = _rng(46)
    cu = np.array([0, 5, 5, 12])
    q = rng.standard_normal((12, 2, 4))
    k = rng.standard_normal((12, 1, 4))
    v = rng.standard_normal((12, 1, 4))
    bias = rng.standard_normal((3, 2, 7, 7))
    o, lse = A.attention_ref(q, k, v, 0.5, True, cu_seqlens=cu, bias=bias)
    for s in range(3):
        lo, hi = int(cu[s]), int(cu[s + 1])
        n = hi - lo
        os_, ls_ = A.attention_ref(q[None, lo:hi], k[None, lo:hi], v[None, lo:hi], 0.5, True,
                                   bias=bias[s:s + 1, :, :n, :n])
        _assert_close(o[lo:hi], os_[0], 0.0, "packed bias O")
        _assert_close(lse[:, lo:hi], ls_[0], 0.0, "packed bias LSE")
    picks = np.array([[0, 1, 4], [2, 0, 6], [2, 1, 0]])
    po, pl = A.attention_picked(q, k, v, 0.5, True, picks, cu_seqlens=cu, bias=bias)
    for r, (s, h, i) in enumerate(picks):
        _assert_close(po[r], o[cu[s] + i, h], 1e-15, "picked bias O")
        _assert_close(pl[r], lse[h, cu[s] + i], 1e-15, "picked bias LSE")


def pin_e4m3_codes():
    """OCP e4m3 values fixed by the format: zero, the smallest subnormal
    2^-9, the largest subnormal 7 * 2^-9, the smallest normal 2^-6, one,
    1.875, two, the largest value 448, signs, and NaN at 0x7f / 0xff."""
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
            0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    got = A.e4m3_value(np.array(list(want), dtype=np.uint8))
    _assert_close(got, np.array(list(want.values())), 0.0, "e4m3 codes")
    assert np.isnan(A.e4m3_value(np.array([0x7F, 0xFF], dtype=np.uint8))).all(), "e4m3 NaN codes"
    assert np.signbit(A.e4m3_value(np.array([0x80], dtype=np.uint8)))[0], "e4m3 negative zero"


def pin_e4m3_library():
    """All 256 e4m3 codes decode to torch's float8_e4m3fn values."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = A.e4m3_value(codes)
    same = (got == lib) | (np.isnan(got) & np.isnan(lib))
    assert same.all(), f"e4m3 codes differ at {np.nonzero(~same)[0][:8]}"


def pin_fp8_descale_laws():
    """The dequantization factors act on the function as the definition
    says: q_descale * 2 is the same call as scale * 2 (so is k_descale),
    v_descale scales O and leaves LSE; with descale 1, the call is the
    attention of the decoded codes (Q = 0.5 everywhere gives uniform
    weights: O = the mean of the visible values)."""
    rng = _rng(51)
    qb = rng.integers(0, 0x7E, (1, 6, 2, 8), dtype=np.uint8) | (rng.integers(0, 2, (1, 6, 2, 8),
                                                                              dtype=np.uint8) << 7)
    kb = rng.integers(0, 0x50, (1, 7, 1, 8), dtype=np.uint8)
    vb = rng.integers(0, 0x7E, (1, 7, 1, 8), dtype=np.uint8)
    for causal in (False, True):
        o1, l1 = A.attention_fp8_ref(qb, kb, vb, 0.02, 0.03, 1.5, 0.4, causal)
        o2, l2 = A.attention_fp8_ref(qb, kb, vb, 0.04, 0.03, 1.5, 0.2, causal)
        o3, l3 = A.attention_fp8_ref(qb, kb, vb, 0.02, 0.06, 3.0, 0.2, causal)
        _assert_close(o2, o1, 1e-14, "q_descale vs scale O")
        _assert_close(l2, l1, 1e-13, "q_descale vs scale LSE")
        _assert_close(o3, 2 * o1, 1e-13, "v_descale scales O")
        _assert_close(l3, l1, 1e-13, "v_descale leaves LSE")
    half = np.full((1, 5, 1, 4), 0x30, dtype=np.uint8)    # 0.5
    vb = rng.integers(0, 0x60, (1, 5, 1, 4), dtype=np.uint8)
    o, lse = A.attention_fp8_ref(half, np.zeros((1, 5, 1, 4), np.uint8), vb, 1.0, 1.0, 1.0, 0.7,
                                 True)
    vals = A.e4m3_value(vb)[0, :, 0]
    for i in range(5):
        _assert_close(o[0, i, 0], vals[:i + 1].mean(axis=0), 1e-13, "uniform fp8 rows")
        _assert_close(lse[0, 0, i], math.log(i + 1), 1e-15, "uniform fp8 LSE")


ALL_PINS = [
    pin_rows_sum_to_one, pin_single_key, pin_uniform_scores_mean, pin_two_key_closed_form,
    pin_permutation_invariance, pin_brute_force, pin_online_route, pin_causal_structure,
    pin_gqa_is_repeated_heads, pin_packed_is_independent, pin_shift_invariance,
    pin_hard_max_limit, pin_library_sdpa, pin_empty_cases, pin_picked_rows,
    pin_window_wide_equals_plain, pin_window_zero_left_causal, pin_window_by_slicing,
    pin_window_brute_force, pin_bias_row_constant, pin_bias_log_weights, pin_bias_as_mask,
    pin_bias_brute_force, pin_bias_library_sdpa, pin_bias_packed, pin_e4m3_codes,
    pin_e4m3_library, pin_fp8_descale_laws,
]
