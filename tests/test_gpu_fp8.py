"""GPU parity of the FP8 forward (fa_fwd_fp8) against the fp64 oracle of
the dequantized inputs.

Tolerance, from the arithmetic of the kernel and of the fp8 matrix
instruction:

* P rounding. Each block stores a row's weights as ws = 2^(x - m - t + 8)
  with t = ceil(block max - m), so the block's largest stored weight lies
  in (2^7, 2^8]; the MFMA's per-lane operand scale 2^(t-8) restores the
  true weights, and the normaliser l is the float32 sum of the unrounded
  ones. Rounding ws to e4m3 costs at most 2^-4 ws for a normal and 2^-10
  (half the subnormal step) below 2^-6, i.e. 2^(t-18) in true units, while
  l exceeds the block's largest true weight 2^(t-1): at most 2^-17 of l.
* Accumulation inside v_mfma_f32_32x32x64_f8f6f4. Its 64-product dot
  products are not exact: measured with one wave on the GPU (B = 1, rows of
  A with known sums), low bits of products next to a larger one in the same
  group of 8 are dropped (448 + 63 * 2^-9 comes out as 448.109375, the 7
  small terms grouped with 448 lost; 256 + 63 * 0.28125 loses 7 * 2^-6),
  each term losing less than 2^-13 of its group's largest product, so an
  instruction's error is below 7 * 2^-13 * sum_k |a_k b_k| < 2^-10 sum_k
  |a_k b_k|. Over random e4m3 operands (512 waves, 1024 outputs each) the
  largest error seen was 2^-11.8 sum_k |a_k b_k|. Hence eps = 2^-10.
  Partial sums across instructions are float32.

With Pabs_i = sum_j P_ij |V_j| (the oracle's attention of |V|), Vsum_i =
sum of |V_j| over the keys row i sees, and Sabs_ij = |scale| |q_i|.|k_j|
(the absolute score sum), elementwise

    |O_gpu - O_ref|_i <= 2^-4 Pabs_i + 2^-17 Vsum_i                  (P rounding)
                         + eps (1 + 2^-4) Pabs_i                      (P V sums)
                         + eps sum_j P_ij Sabs_ij (|V_j| + |O_i|)     (score sums)
                         + 2^-8 |O_ref|_i + 1e-6                      (bf16 O),
    |LSE_gpu - LSE_ref|_i <= eps sum_j P_ij Sabs_ij + 1e-5 (1 + |LSE_i|).

When every score is an integer and the scale is ln 2 (the "signs" inputs:
4 entries of +-1 per row of Q and K), every weight is a power of two within
e4m3's exact range and every score sum is exact, so the P rounding and score
terms vanish and only the P V sums and the bf16 rounding remain.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_63_amd  # noqa: F401


def _dev(bits):
    import torch
    return torch.from_numpy(bits).to("cuda")


def _run(x, causal, scale):
    import torch

    import exact_io_aware_63_amd as fa
    o, lse = fa.attention_fwd_fp8(_dev(x.q_bits), _dev(x.k_bits), _dev(x.v_bits),
                                  q_descale=x.q_descale, k_descale=x.k_descale,
                                  v_descale=x.v_descale, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _deq(x):
    return (oracle.e4m3_value(x.q_bits) * x.q_descale, oracle.e4m3_value(x.k_bits) * x.k_descale,
            oracle.e4m3_value(x.v_bits) * x.v_descale)


EPS = 2.0 ** -10


def _row_terms(qh, kh, vh, scale, causal, rows, o_rows):
    """Bound terms of the given rows of one head (fp64): Pabs, Vsum,
    sum_j P Sabs (|V_j| + |O_i|) per column, and sum_j P Sabs."""
    lk = kh.shape[0]
    vis = oracle.visible_mask(rows, lk, causal)
    p, _, _ = oracle.softmax_rows(np.where(vis, oracle.scores(qh[rows], kh, scale), -np.inf))
    sabs = abs(scale) * (np.abs(qh[rows]) @ np.abs(kh).T)
    ps = p * sabs
    va = np.abs(vh)
    return (p @ va, vis.astype(np.float64) @ va,
            ps @ va + ps.sum(axis=1, keepdims=True) * np.abs(o_rows), ps.sum(axis=1))


def _bounds(q, k, v, scale, causal, o_ref, lse_ref, exact):
    """Elementwise O and LSE bounds of the module docstring, fixed-length
    layouts (q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d])."""
    bo = np.zeros_like(o_ref)
    bl = np.zeros_like(lse_ref)
    bsz, nq, hq, _ = q.shape
    hkv = k.shape[2]
    rows = np.arange(nq)
    for b in range(bsz):
        for h in range(hq):
            g = oracle.kv_head_of(h, hq, hkv)
            pabs, vsum, psv, ps = _row_terms(q[b, :, h], k[b, :, g], v[b, :, g], scale, causal,
                                             rows, o_ref[b, :, h])
            round_p = 0.0 if exact else 2.0 ** -4 * pabs + 2.0 ** -17 * vsum
            bo[b, :, h] = (round_p + EPS * (1 + 2.0 ** -4) * pabs + EPS * psv +
                           2.0 ** -8 * np.abs(o_ref[b, :, h]) + 1e-6)
            bl[b, h] = EPS * ps + 1e-5 * (1 + np.abs(np.where(np.isfinite(lse_ref[b, h]),
                                                              lse_ref[b, h], 0.0)))
    return bo, bl


def _check(name, o, lse, o_ref, lse_ref, bo, bl):
    err = np.abs(o - o_ref)
    assert np.all(np.isfinite(o)), f"{name}: non-finite O"
    ratio = float((err / bo).max()) if err.size else 0.0
    same_inf = np.isinf(lse) & np.isinf(lse_ref) & (np.sign(lse) == np.sign(lse_ref))
    el = np.where(same_inf, 0.0, np.abs(lse - lse_ref))
    lratio = float((el / bl).max()) if el.size else 0.0
    say(f"[fp8 parity] {name}: max|dO| {float(err.max()) if err.size else 0:.3e}, "
        f"O err/bound {ratio:.3f}, max|dLSE| {float(el.max()) if el.size else 0:.2e}, "
        f"LSE err/bound {lratio:.3f}")
    assert ratio <= 1.0, f"{name}: O error exceeds the bound (ratio {ratio:.3f})"
    assert lratio <= 1.0, f"{name}: LSE error exceeds the bound (ratio {lratio:.3f})"


CASES = [
    # name, B, Hq, Hkv, Nq, Nk, causal, mode, sigma
    ("signs_causal", 1, 8, 2, 1500, 1500, True, "signs", (1.0, 1.0, 1.0)),
    ("signs_full_ragged", 2, 4, 4, 600, 333, False, "signs", (1.0, 1.0, 1.0)),
    ("normal_causal", 2, 4, 2, 700, 700, True, "normal", (1.0, 1.0, 1.0)),
    ("normal_full_ragged", 1, 8, 2, 333, 517, False, "normal", (1.0, 1.0, 1.0)),
    ("wide_scores_rescale", 1, 4, 4, 1000, 1000, True, "normal", (3.0, 3.0, 1.0)),
    ("tail_130", 1, 4, 1, 130, 130, True, "normal", (1.0, 1.0, 1.0)),
    ("tiny", 1, 2, 1, 1, 3, False, "normal", (1.0, 1.0, 1.0)),
    ("rows_past_keys", 1, 2, 2, 300, 70, True, "normal", (1.0, 1.0, 1.0)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_parity(case):
    name, b, hq, hkv, nq, nk, causal, mode, sigma = case
    say(f"[case] fp8 {name}")
    x = W.draw_fp8(b, hq, hkv, nq, nk, 128, zlib.crc32(name.encode()), sigma, mode)
    scale = math.log(2.0) if mode == "signs" else 1.0 / math.sqrt(128)
    o, lse = _run(x, causal, scale)
    q, k, v = _deq(x)
    o_ref, lse_ref = oracle.attention_fp8_ref(x.q_bits, x.k_bits, x.v_bits, x.q_descale,
                                              x.k_descale, x.v_descale, scale, causal)
    _check(name, o, lse, o_ref, lse_ref, *_bounds(q, k, v, scale, causal, o_ref, lse_ref,
                                                  mode == "signs"))


def test_fp8_no_keys():
    """Nk = 0: every row gets O = 0 and LSE = -inf (no workspace needed)."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] fp8 no keys")
    q = torch.full((1, 40, 2, 128), 0x38, dtype=torch.uint8, device="cuda")
    kv = torch.empty((1, 0, 1, 128), dtype=torch.uint8, device="cuda")
    o, lse = fa.attention_fwd_fp8(q, kv, kv, causal=False)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_fp8_deterministic_and_negative_scale():
    """Repeated calls agree bitwise; a negative scale is the attention of the
    negated scores (the oracle with the same scale)."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] fp8 determinism, negative scale")
    x = W.draw_fp8(1, 4, 2, 500, 500, 128, 91)
    args = [_dev(x.q_bits), _dev(x.k_bits), _dev(x.v_bits)]
    kw = dict(q_descale=x.q_descale, k_descale=x.k_descale, v_descale=x.v_descale, causal=True)
    o1, l1 = fa.attention_fwd_fp8(*args, **kw)
    o2, l2 = fa.attention_fwd_fp8(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o, lse = _run(x, True, -0.2)
    q, k, v = _deq(x)
    o_ref, lse_ref = oracle.attention_fp8_ref(x.q_bits, x.k_bits, x.v_bits, x.q_descale,
                                              x.k_descale, x.v_descale, -0.2, True)
    _check("negative scale", o, lse, o_ref, lse_ref, *_bounds(q, k, v, -0.2, True, o_ref, lse_ref,
                                                              False))


def test_fp8_full_size_sampled():
    """Causal GQA 32/8 heads, N = 8192, d = 128 (the bf16 workload's shape)
    with amax-scaled N(0, 1) inputs: 32 rows of every head (tile edges and
    random rows, 1024 in all), each formed whole by the oracle, against the
    bound."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] fp8 full size: causal GQA 32/8, N=8192, d=128")
    w = W.WORKLOADS[4]
    x = W.draw_fp8(1, w.hq, w.hkv, w.n, w.n, w.d, 4008)
    o, lse = fa.attention_fwd_fp8(_dev(x.q_bits), _dev(x.k_bits), _dev(x.v_bits),
                                  q_descale=x.q_descale, k_descale=x.k_descale,
                                  v_descale=x.v_descale, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    q, k, v = _deq(x)
    rng = np.random.default_rng(4008)
    edges = {0, 1, 63, 64, 255, 256, 4095, 4096, w.n - 2, w.n - 1}
    n_rows = 0
    for h in range(w.hq):
        rows = np.array(sorted(edges | set(rng.choice(w.n, 32 - len(edges) + 4,
                                                      replace=False).tolist()))[:32])
        g = oracle.kv_head_of(h, w.hq, w.hkv)
        ro, rl = oracle.attention_head(q[0, :, h], k[0, :, g], v[0, :, g], w.scale, True,
                                       rows=rows)
        pabs, vsum, psv, ps = _row_terms(q[0, :, h], k[0, :, g], v[0, :, g], w.scale, True, rows,
                                         ro)
        bo = (2.0 ** -4 * pabs + 2.0 ** -17 * vsum + EPS * (1 + 2.0 ** -4) * pabs + EPS * psv +
              2.0 ** -8 * np.abs(ro) + 1e-6)
        bl = EPS * ps + 1e-5 * (1 + np.abs(rl))
        _check(f"full size head {h}", o[0, rows, h], lse[0, h, rows], ro, rl, bo, bl)
        n_rows += len(rows)
    assert n_rows >= 1000


def _codes(x):
    """e4m3 codes of values that e4m3 holds exactly (checked)."""
    b = W.to_e4m3_bits(np.asarray(x, np.float32))
    assert np.array_equal(oracle.e4m3_value(b), np.asarray(x, np.float64)), "not exact in e4m3"
    return b


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_far_rescale_every_block(causal):
    """Scores that climb by about 82 (base 2) from one 64-key block to the
    next: every block maximum lies more than 64 above the row's reference,
    so each block moves the reference and rescales the accumulators (the
    rare path kept for float32 range). Inputs have descale 1: N(0, 1) codes,
    with q's last column 40 and key j's last column 16 floor(j / 64)."""
    say(f"[case] fp8 far rescale every block, causal={causal}")
    n, hq, hkv, d = 700, 4, 2, 128
    rng = np.random.default_rng(77)
    qv = oracle.e4m3_value(W.to_e4m3_bits(rng.standard_normal((1, n, hq, d), np.float32)))
    kv = oracle.e4m3_value(W.to_e4m3_bits(rng.standard_normal((1, n, hkv, d), np.float32)))
    vv = oracle.e4m3_value(W.to_e4m3_bits(rng.standard_normal((1, n, hkv, d), np.float32)))
    qv[..., -1] = 40.0
    kv[0, :, :, -1] = (16.0 * np.floor(np.arange(n) / 64.0))[:, None]
    x = W.Fp8Inputs(_codes(qv), _codes(kv), _codes(vv), 1.0, 1.0, 1.0)
    scale = 1.0 / math.sqrt(d)
    # precondition, from the definition: consecutive full blocks' maxima
    # (base 2) differ by more than 64 for every row of every head
    for h in range(hq):
        g = oracle.kv_head_of(h, hq, hkv)
        s2 = oracle.scores(qv[0, :, h], kv[0, :, g], scale) * 1.4426950408889634
        full = s2[:, :(n // 64) * 64].reshape(n, n // 64, 64).max(axis=2)
        assert float(np.diff(full, axis=1).min()) > 64.0
    o, lse = _run(x, causal, scale)
    o_ref, lse_ref = oracle.attention_fp8_ref(x.q_bits, x.k_bits, x.v_bits, 1.0, 1.0, 1.0, scale,
                                              causal)
    _check("far rescale", o, lse, o_ref, lse_ref,
           *_bounds(qv, kv, vv, scale, causal, o_ref, lse_ref, False))


def test_fp8_score_accumulation_within_eps():
    """The fp8 matrix instruction's accumulation error, seen through the
    scores: with one key, LSE = scale q.k as the kernel sums it (a weight
    sum of exactly one block-scaled 2^8), so |LSE - scale q.k| bounds that
    instruction's error on each row's 128 products. It must stay within
    eps = 2^-10 of |scale| sum_k |q_k k_k| (plus float32 rounding of the
    final products). Rows: one 448 and seven 2^-9 in every group of 8
    products at each position of the large term, mixed signs, and
    amax-scaled normal codes; head 0's key is all ones, head 1's random."""
    say("[case] fp8 score accumulation against eps = 2^-10")
    d, nq = 128, 512
    rng = np.random.default_rng(515)
    rows = []
    for pos in range(8):                       # large product at each group position
        r = np.full(d, 2.0 ** -9)
        r[pos::8] = 448.0
        rows.append(r)
        rows.append(r * np.where(rng.random(d) < 0.5, -1.0, 1.0))
    while len(rows) < nq:
        z = rng.standard_normal(d)
        rows.append(oracle.e4m3_value(W.to_e4m3_bits((z * (448.0 / np.abs(z).max()))
                                                      .astype(np.float32))))
    qv = np.stack(rows)[None, :, None, :].repeat(2, axis=2)          # [1, nq, 2, d]
    k_rand = oracle.e4m3_value(W.to_e4m3_bits((rng.standard_normal(d) * 16).astype(np.float32)))
    kv = np.stack([np.ones(d), k_rand])[None, None]                   # [1, 1, 2, d]
    x = W.Fp8Inputs(_codes(qv), _codes(kv), _codes(np.ones_like(kv)), 1.0, 1.0, 1.0)
    scale = 1.0 / math.sqrt(d)
    _, lse = _run(x, False, scale)
    worst = 0.0
    for h in range(2):
        exact = scale * (qv[0, :, h] @ kv[0, 0, h])
        absum = abs(scale) * (np.abs(qv[0, :, h]) @ np.abs(kv[0, 0, h]))
        err = np.abs(lse[0, h] - exact)
        assert np.all(err <= EPS * absum + 1e-6 * np.abs(exact) + 1e-30), (
            f"head {h}: worst err/(eps sum|ab|) {float((err / (EPS * absum)).max()):.3f}")
        worst = max(worst, float((err / absum).max()))
    say(f"[fp8 accumulation] largest error / sum|a b| = 2^{math.log2(max(worst, 1e-300)):.1f}")
