"""fp64 CPU oracle for the exact scaled-dot-product attention forward pass.

TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the CPU-baseline
leg of the bench may call this module; the product path (the ``libfa`` C
library and its Python binding) never imports, links or runs it, and this
module imports nothing from the product path.

What it computes is the plain definition, written out and materialised on
purpose (it is the "standard" schedule that the tiled method avoids):

* "Softmax does not need the matrix" (sir-teo.github.io), opening equation
  and section *Carry the Normalizer*: scores s_j = q.k_j / sqrt(d), the stable
  softmax p_j = exp(s_j - m) / sum_i exp(s_i - m) with m = max_i s_i, and the
  output o = sum_j p_j v_j.
* "Understanding FlashAttention Pt 1: Personal Notes", section 0.2 Notation:
  S = Q K^T / sqrt(d) (+ B), P = softmax_row(S), O = P V; and the three-step
  standard algorithm of its introduction (form S, form P, form O).

Readings taken where the pages are silent:

* the caller passes ``scale`` (the pages' 1/sqrt(d) is the usual value);
* causal masking is top-left: query i sees key j iff j <= i (indices local to
  the sequence), and key j must exist (j < Lk);
* grouped-query attention groups contiguous heads: q-head h reads kv-head
  h // (Hq // Hkv);
* the retained row statistic is the natural-log log-sum-exp of the scaled,
  visible scores: LSE_i = m_i + log(sum_j exp(S_ij - m_i));
* a row that sees no key has O = 0 and LSE = -inf;
* V has the same width d as Q and K;
* the additive bias B of "Understanding FlashAttention Pt 1", section 0.2
  (S = Q K^T / sqrt(d) + B) is optional. It is added to the scaled scores of
  the visible pairs before the softmax; masked pairs stay masked whatever B
  holds there, and a bias entry of -inf removes its pair like the mask does.
  B is given per (batch entry or sequence, q-head) as a [Lq, Lk] block with
  indices local to the sequence; ``bias_of`` states the indexing. The bias
  is an input only: no gradient with respect to it is formed.

The backward pass (``attention_head_bwd`` and the functions after it) is
the gradient of the same function with respect to Q, K and V for a given
upstream gradient dO, written out by the chain rule through the
materialised S and P. The pages name this step only: "Understanding
FlashAttention Pt 1", contents, section 3.6 ("Backward pass: recompute
instead of save"), and semiaifoundry "attention-io-tiling", section
*Specifications and interfaces* (use the retained statistics and permitted
recomputation for the backward execution). The oracle recomputes nothing
from retained statistics: it forms S and P from Q and K again, exactly as
the forward definition reads, and differentiates that.

Everything is float64. bf16 and fp32 inputs are exactly representable in
float64, so the upcast adds no error.

Memory layouts (token-major, row-major, contiguous), the same ones the C ABI
uses:

* fixed length: q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d],
  O [B, Nq, Hq, d], LSE [B, Hq, Nq];
* packed variable length (``cu_seqlens`` = offsets [nseq + 1]):
  q [T, Hq, d], k and v [T, Hkv, d], O [T, Hq, d], LSE [Hq, T], with
  sequence s occupying tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of both the
  query and the key side (self-attention), never attending across sequences.
"""
from __future__ import annotations

import numpy as np

# Rows of S materialised at once. It bounds host memory only; every row is
# still formed whole, exactly as the definition reads.
ROW_CHUNK = 1024


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """K/V head read by query head ``h`` (grouped-query attention).

    "Softmax does not need the matrix", section *Quadratic Time Did Not
    Vanish*, names grouped-query attention; "Understanding FlashAttention
    Pt 1", section 1.1, lists MQA/GQA as compatible. Reading: the Hq/Hkv query
    heads of one group are contiguous, so h -> h // (Hq // Hkv).
    """
    if hkv <= 0 or hq % hkv != 0:
        raise ValueError(f"Hq={hq} must be a positive multiple of Hkv={hkv}")
    return h // (hq // hkv)


def visible_mask(rows: np.ndarray, lk: int, causal: bool, window=None) -> np.ndarray:
    """Boolean [len(rows), lk]: True where query ``rows[r]`` may see key j.

    Causal reading: top-left lower-triangular, j <= i, indices local to the
    sequence ("Understanding FlashAttention Pt 1", section 3.5 title, causal
    masking; the body of that section is not in the pages, so the plain
    lower-triangular mask is taken).

    ``window`` = (left, right), a sliding (local) window: query i also sees
    only keys i - left <= j <= i + right, a negative bound meaning unbounded.
    Reading: the pages name local attention and sliding windows only
    ("Understanding FlashAttention Pt 1", contents, section 4.2 title;
    "Softmax does not need the matrix", *Quadratic Time Did Not Vanish*), so
    the plain band around the diagonal is taken, combined with the causal
    mask by AND.
    """
    j = np.arange(lk)[None, :]
    i = np.asarray(rows)[:, None]
    m = (j <= i) if causal else np.broadcast_to(j >= 0, (len(rows), lk))
    if window is not None:
        left, right = window
        if left >= 0:
            m = m & (j >= i - left)
        if right >= 0:
            m = m & (j <= i + right)
    return m


def bias_of(bias, s: int, h: int):
    """The [Lq, Lk] bias block of batch entry (or sequence) ``s`` and q-head
    ``h``, or None.

    ``bias`` is None or an array indexed [s, h, i, j], i and j local to the
    sequence; an axis of length 1 among the first two is shared by every
    batch entry (or sequence) or every head. Reading: the pages define B
    only as a term of S ("Understanding FlashAttention Pt 1", section 0.2),
    so it is taken per (entry, head, query, key), the most general form, with
    sharing as the usual broadcast.
    """
    if bias is None:
        return None
    b = np.asarray(bias)
    if b.ndim != 4:
        raise ValueError(f"bias must be indexed [s, h, i, j], got shape {b.shape}")
    return b[s if b.shape[0] > 1 else 0, h if b.shape[1] > 1 else 0]


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * q_rows K^T, materialised ("Understanding FlashAttention
    Pt 1", section 0.2: S = Q K^T / sqrt(d); "Softmax does not need the
    matrix", s_j = q^T k_j / sqrt(d))."""
    return (q_rows @ k.T) * scale


def softmax_rows(s: np.ndarray):
    """Stable row softmax of a materialised score block.

    "Softmax does not need the matrix", section *Carry the Normalizer*:
    p_j = exp(s_j - m) / sum_i exp(s_i - m), m = max_i s_i. Masked entries
    arrive as -inf and get probability 0. Returns (P, m, l) with
    l = sum_j exp(s_j - m). A row with no finite entry has P = 0, m = -inf,
    l = 0.
    """
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    p = e / l_safe[:, None]
    return p, m, l


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, rows=None, window=None, bias=None):
    """One (sequence, head) of attention: q [Lq, d], k and v [Lk, d], bias
    None or [>= Lq, >= Lk] (row i, column j: query i, key j).

    Forms S (+ B), then P, then O = P V for the selected query rows (all
    rows if ``rows`` is None), and LSE = m + log(l). Returns (O [R, d],
    LSE [R]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    rows = np.arange(lq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), v.shape[1]), dtype=np.float64)
    lse = np.full(len(rows), -np.inf, dtype=np.float64)
    if lk == 0 or len(rows) == 0:
        return out, lse
    for c0 in range(0, len(rows), ROW_CHUNK):
        r = rows[c0:c0 + ROW_CHUNK]
        s = scores(q[r], k, scale)                                # write S
        if bias is not None:                                      # S + B
            s = s + np.asarray(np.asarray(bias)[r][:, :lk], dtype=np.float64)
        s = np.where(visible_mask(r, lk, causal, window), s, -np.inf)
        p, m, l = softmax_rows(s)                                 # write P
        out[c0:c0 + len(r)] = p @ v                               # O = P V
        with np.errstate(divide="ignore"):
            lse[c0:c0 + len(r)] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def attention_ref(q, k, v, scale: float, causal: bool, cu_seqlens=None, window=None,
                  bias=None):
    """Full forward pass in the token-major layouts of the module docstring.

    ``bias``: None or indexed [s, h, i, j] as ``bias_of`` states (fixed
    length: [B or 1, Hq or 1, >= Nq, >= Nk]; packed: [nseq or 1, Hq or 1,
    >= longest, >= longest], local indices). Returns (O, LSE) as float64
    arrays.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if cu_seqlens is None:
        bsz, nq, hq, d = q.shape
        hkv = k.shape[2]
        out = np.zeros_like(q)
        lse = np.full((bsz, hq, nq), -np.inf)
        for b in range(bsz):
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                o_bh, l_bh = attention_head(q[b, :, h], k[b, :, g], v[b, :, g], scale, causal,
                                            window=window, bias=bias_of(bias, b, h))
                out[b, :, h] = o_bh
                lse[b, h] = l_bh
        return out, lse
    t, hq, d = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.zeros_like(q)
    lse = np.full((hq, t), -np.inf)
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            o_sh, l_sh = attention_head(q[lo:hi, h], k[lo:hi, g], v[lo:hi, g], scale, causal,
                                        window=window, bias=bias_of(bias, s, h))
            out[lo:hi, h] = o_sh
            lse[h, lo:hi] = l_sh
    return out, lse


def attention_picked(q, k, v, scale: float, causal: bool, picks, cu_seqlens=None, window=None,
                     bias=None):
    """Selected outputs only, one (batch-or-sequence, q-head, row) at a time.

    For parity checks at sizes where the full oracle would take too long:
    each picked row is formed from the definition exactly as in
    ``attention_ref``. ``picks`` is an int array [P, 3] of (s, h, i) with i
    local to the sequence. Returns (O [P, d], LSE [P]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    picks = np.asarray(picks, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    out = np.zeros((len(picks), d), dtype=np.float64)
    lse = np.full(len(picks), -np.inf)
    if cu_seqlens is None:
        hq, hkv = q.shape[2], k.shape[2]
    else:
        hq, hkv = q.shape[1], k.shape[1]
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    # group picks by (s, h) so each K/V head slice is upcast once
    order = np.lexsort((picks[:, 2], picks[:, 1], picks[:, 0]))
    i0 = 0
    while i0 < len(order):
        s, h = picks[order[i0], 0], picks[order[i0], 1]
        i1 = i0
        while i1 < len(order) and picks[order[i1], 0] == s and picks[order[i1], 1] == h:
            i1 += 1
        sel = order[i0:i1]
        g = kv_head_of(int(h), hq, hkv)
        if cu_seqlens is None:
            qs, ks, vs = q[s, :, h], k[s, :, g], v[s, :, g]
        else:
            lo, hi = int(cu[s]), int(cu[s + 1])
            qs, ks, vs = q[lo:hi, h], k[lo:hi, g], v[lo:hi, g]
        o_sel, l_sel = attention_head(np.asarray(qs, dtype=np.float64),
                                      np.asarray(ks, dtype=np.float64),
                                      np.asarray(vs, dtype=np.float64),
                                      scale, causal, rows=picks[sel, 2],
                                      window=window, bias=bias_of(bias, int(s), int(h)))
        out[sel] = o_sel
        lse[sel] = l_sel
        i0 = i1
    return out, lse


# ---------------------------------------------------------------------------
# Backward pass: gradients of O = softmax(scale Q K^T) V
# ---------------------------------------------------------------------------

def softmax_rows_bwd(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Chain rule through the row softmax: given P = softmax_row(S) and
    dP = dL/dP, returns dS = dL/dS with dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).

    Derivation: dP_ik/dS_ij = P_ik (delta_kj - P_ij) for a row softmax
    ("Softmax does not need the matrix", *Carry the Normalizer*, stable
    softmax p_j = exp(s_j - m) / sum exp(s_i - m); the shift m cancels).
    Masked entries have P = 0, hence dS = 0.
    """
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def attention_head_bwd(q, k, v, do, scale: float, causal: bool, window=None, bias=None):
    """Gradients of one (sequence, head): q, do [Lq, d]; k, v [Lk, d]; bias
    None or [>= Lq, >= Lk] as in ``attention_head``.

    Forms S = scale q K^T (+ B), the mask, P = softmax_row(S) (as the forward
    definition), then
      dV = P^T dO,   dP = dO V^T,   dS = softmax_rows_bwd(P, dP),
      dQ = scale dS K,   dK = scale dS^T Q.
    Returns (dq [Lq, d], dk [Lk, d], dv [Lk, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lq, lk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if lq == 0 or lk == 0:
        return dq, dk, dv
    for c0 in range(0, lq, ROW_CHUNK):
        r = np.arange(c0, min(lq, c0 + ROW_CHUNK))
        s = scores(q[r], k, scale)
        if bias is not None:
            s = s + np.asarray(np.asarray(bias)[r][:, :lk], dtype=np.float64)
        s = np.where(visible_mask(r, lk, causal, window), s, -np.inf)
        p, _, _ = softmax_rows(s)
        dv += p.T @ do[r]
        dp = do[r] @ v.T
        ds = softmax_rows_bwd(p, dp)
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool, cu_seqlens=None, window=None,
                      bias=None):
    """Gradients in the layouts of the module docstring (dO like O); ``bias``
    as in ``attention_ref``.

    Returns (dQ like q, dK like k, dV like v) as float64 arrays. With
    grouped-query attention a K/V head's gradients are the sums over the
    query heads that read it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if cu_seqlens is None:
        bsz, _, hq, _ = q.shape
        hkv = k.shape[2]
        for b in range(bsz):
            for h in range(hq):
                g = kv_head_of(h, hq, hkv)
                a, bk, bv = attention_head_bwd(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h],
                                               scale, causal, window=window,
                                               bias=bias_of(bias, b, h))
                dq[b, :, h] = a
                dk[b, :, g] += bk
                dv[b, :, g] += bv
        return dq, dk, dv
    hq, hkv = q.shape[1], k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            a, bk, bv = attention_head_bwd(q[lo:hi, h], k[lo:hi, g], v[lo:hi, g], do[lo:hi, h],
                                           scale, causal, window=window,
                                           bias=bias_of(bias, s, h))
            dq[lo:hi, h] = a
            dk[lo:hi, g] += bk
            dv[lo:hi, g] += bv
    return dq, dk, dv


def attention_bwd_picked(q, k, v, do, scale: float, causal: bool, q_picks, kv_picks,
                         cu_seqlens=None, window=None, bias=None):
    """Selected gradient rows, for parity checks at sizes where the full
    oracle would take too long.

    ``q_picks`` [P, 3] of (s, h, i): the dQ row of query i of q-head h.
    ``kv_picks`` [R, 3] of (s, g, j): the dK and dV rows of key j of K/V head
    g, summed over the query heads that read g. Every row is formed from the
    definition as in ``attention_head_bwd``: the whole rows of S, P and dP of
    the queries involved are materialised. Returns (dq [P, d], dk [R, d],
    dv [R, d]).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    q_picks = np.asarray(q_picks, dtype=np.int64).reshape(-1, 3)
    kv_picks = np.asarray(kv_picks, dtype=np.int64).reshape(-1, 3)
    d = q.shape[-1]
    if cu_seqlens is None:
        hq, hkv = q.shape[2], k.shape[2]
    else:
        hq, hkv = q.shape[1], k.shape[1]
        cu = np.asarray(cu_seqlens, dtype=np.int64)

    def head_scores(qh, kh, s, h, r):
        sc = scores(qh[r], kh, scale)
        b = bias_of(bias, int(s), int(h))
        if b is not None:
            sc = sc + np.asarray(np.asarray(b)[r][:, :kh.shape[0]], dtype=np.float64)
        return np.where(visible_mask(r, kh.shape[0], causal, window), sc, -np.inf)

    def head(s, h):
        g = kv_head_of(int(h), hq, hkv)
        if cu_seqlens is None:
            return (np.asarray(q[s, :, h], np.float64), np.asarray(k[s, :, g], np.float64),
                    np.asarray(v[s, :, g], np.float64), np.asarray(do[s, :, h], np.float64))
        lo, hi = int(cu[s]), int(cu[s + 1])
        return (np.asarray(q[lo:hi, h], np.float64), np.asarray(k[lo:hi, g], np.float64),
                np.asarray(v[lo:hi, g], np.float64), np.asarray(do[lo:hi, h], np.float64))

    dq = np.zeros((len(q_picks), d))
    for n, (s, h, i) in enumerate(q_picks):
        qh, kh, vh, doh = head(s, h)
        r = np.array([i])
        p, _, _ = softmax_rows(head_scores(qh, kh, s, h, r))
        ds = softmax_rows_bwd(p, doh[r] @ vh.T)
        dq[n] = scale * (ds @ kh)[0]
    dk = np.zeros((len(kv_picks), d))
    dv = np.zeros((len(kv_picks), d))
    group = hq // hkv
    # picks of one (sequence, K/V head) share the materialised rows
    keys = sorted({(int(s), int(g)) for s, g, _ in kv_picks})
    for s, g in keys:
        sel = [n for n, (s2, g2, _) in enumerate(kv_picks) if s2 == s and g2 == g]
        cols = np.array([kv_picks[n][2] for n in sel], dtype=np.int64)
        for h in range(g * group, (g + 1) * group):
            qh, kh, vh, doh = head(s, h)
            lq, lk = qh.shape[0], kh.shape[0]
            for c0 in range(0, lq, ROW_CHUNK):
                r = np.arange(c0, min(lq, c0 + ROW_CHUNK))
                p, _, _ = softmax_rows(head_scores(qh, kh, s, h, r))
                ds = softmax_rows_bwd(p, doh[r] @ vh.T)
                dv[sel] += p[:, cols].T @ doh[r]
                dk[sel] += scale * (ds[:, cols].T @ qh[r])
    return dq, dk, dv


# ---------------------------------------------------------------------------
# FP8 inputs
# ---------------------------------------------------------------------------

def e4m3_value(bits) -> np.ndarray:
    """Values of OCP e4m3 codes (uint8) as float64, from the format's
    definition: sign bit s, exponent field e (4 bits, bias 7), mantissa
    field m (3 bits); e > 0 gives (-1)^s 2^(e-7) (1 + m/8), e = 0 gives the
    subnormal (-1)^s 2^-6 (m/8); e = 15 with m = 7 is NaN (no infinities).
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    return np.where((e == 15) & (m == 7), np.nan, s * mag)


def attention_fp8_ref(q_bits, k_bits, v_bits, q_descale: float, k_descale: float,
                      v_descale: float, scale: float, causal: bool):
    """Attention of FP8 inputs: the exact attention (``attention_ref``) of the
    dequantized tensors q = q_descale * Q, k = k_descale * K,
    v = v_descale * V, fixed-length layouts. The pages list FP8 only as
    FlashAttention-3's low-precision variant ("Understanding FlashAttention
    Pt 1", contents, section 5.6); reading: the inputs are e4m3 with one
    dequantization factor per tensor, and the function computed is unchanged.
    Returns (O, LSE) as float64."""
    q = e4m3_value(q_bits) * float(q_descale)
    k = e4m3_value(k_bits) * float(k_descale)
    v = e4m3_value(v_bits) * float(v_descale)
    return attention_ref(q, k, v, scale, causal)

