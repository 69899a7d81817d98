"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle.

The GPU runs its own forward pass first (O and LSE), then fa_bwd; the oracle
differentiates the exact function of the same bf16 inputs. Tolerance,
derived from the arithmetic of the kernels: every error source is a
relative bf16 perturbation (at most 2^-9) of one term of the gradient sums:
P and dS rounded to bf16 before their products, the final rounding of each
output, and D = dO.O formed from the forward pass's O, whose own error is a
few bf16 roundings of the terms of sum_j P_ij V_j. With the absolute-value
forms dPa = |dO| |V|^T and Da_i = sum_j P_ij dPa_ij (>= |dP|, >= |D|, and
bounding the error of D in units of 2^-9), elementwise

    |dV_gpu - dV| <= c |P|^T |dO|,
    |dQ_gpu - dQ| <= c scale (P * (dPa + Da)) |K|,
    |dK_gpu - dK| <= c scale (P * (dPa + Da))^T |Q|,

with c = 2^-6 (eight roundings' worth per term). A wrong index, sign or
dropped term makes errors of the size of the bound itself.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu

C_BOUND = 2.0 ** -6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_63_amd  # noqa: F401  (fails loudly if libfa.so is missing)


def _draw_do(shape, seed):
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    bits = W.round_to_bf16_bits(x)
    return W.bf16_bits_to_f32(bits), bits


def _run(inp, do_bits, causal, scale, window=None, bias=None):
    """GPU forward then backward; returns float64 numpy (dq, dk, dv).
    ``bias``: a workloads.Bias, passed to both passes."""
    import torch

    import exact_io_aware_63_amd as fa
    q, k, v, cu = to_device(inp)
    ms = inp.max_seqlen if cu is not None else None
    bt = None
    if bias is not None:
        bt = torch.from_numpy(bias.bits.view(np.int16)).view(torch.bfloat16).to(q.device)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu, max_seqlen=ms,
                              window=window, bias=bt)
    do = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(q.device)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, do, causal=causal, scale=scale, cu_seqlens=cu,
                                  max_seqlen=ms, window=window, bias=bt)
    torch.cuda.synchronize()
    return tuple(t.float().cpu().double().numpy() for t in (dq, dk, dv))


def _head_terms(qh, kh, vh, doh, scale, causal, rows=None, window=None, bias_block=None):
    """P and dPa + Da (module docstring) of the given rows of one head
    (fp64; P from the definition, as the oracle forms it)."""
    lq, lk = qh.shape[0], kh.shape[0]
    rows = np.arange(lq) if rows is None else np.asarray(rows)
    sc = oracle.scores(qh[rows], kh, scale)
    if bias_block is not None:
        sc = sc + np.asarray(bias_block[rows][:, :lk], dtype=np.float64)
    sc = np.where(oracle.visible_mask(rows, lk, causal, window), sc, -np.inf)
    p, _, _ = oracle.softmax_rows(sc)
    dpa = np.abs(doh[rows]) @ np.abs(vh).T
    da = (p * dpa).sum(axis=1, keepdims=True)
    return p, dpa + da


def _heads(inp, do):
    """(unit, q-head, K/V head, q, k, v, do) per (sequence or batch, head)."""
    q, k, v = inp.q.astype(np.float64), inp.k.astype(np.float64), inp.v.astype(np.float64)
    do = do.astype(np.float64)
    packed = inp.cu_seqlens is not None
    hq, hkv = (q.shape[1], k.shape[1]) if packed else (q.shape[2], k.shape[2])
    units = range(len(inp.cu_seqlens) - 1) if packed else range(q.shape[0])
    for s in units:
        for h in range(hq):
            g = oracle.kv_head_of(h, hq, hkv)
            if packed:
                lo, hi = int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])
                yield s, h, g, q[lo:hi, h], k[lo:hi, g], v[lo:hi, g], do[lo:hi, h]
            else:
                yield s, h, g, q[s, :, h], k[s, :, g], v[s, :, g], do[s, :, h]


def _bounds_full(inp, do, scale, causal, window=None, bias=None):
    """Elementwise magnitude sums of the module docstring, full tensors."""
    bq, bk, bv = (np.zeros(x.shape) for x in (inp.q, inp.k, inp.v))
    packed = inp.cu_seqlens is not None
    for s, h, g, qh, kh, vh, doh in _heads(inp, do):
        if qh.shape[0] == 0 or kh.shape[0] == 0:
            continue
        p, w = _head_terms(qh, kh, vh, doh, scale, causal, window=window,
                           bias_block=oracle.bias_of(bias, s, h))
        a = abs(scale) * ((p * w) @ np.abs(kh))
        b = abs(scale) * ((p * w).T @ np.abs(qh))
        c = p.T @ np.abs(doh)
        if packed:
            lo, hi = int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])
            bq[lo:hi, h] = a
            bk[lo:hi, g] += b
            bv[lo:hi, g] += c
        else:
            bq[s, :, h] = a
            bk[s, :, g] += b
            bv[s, :, g] += c
    return bq, bk, bv


def _check(name, got, ref, bound):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    tol = C_BOUND * bound + 1e-6 * max(float(bound.max()) if bound.size else 0.0, 1e-30)
    ratio = float((err / np.maximum(bound, 1e-30)).max()) if err.size else 0.0
    say(f"[bwd parity] {name}: max|err| {float(err.max()) if err.size else 0:.3e}, "
        f"max err/bound {ratio:.2e} (limit {C_BOUND:.2e})")
    bad = err > tol
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements exceed the bound; worst at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}")


SMALL_BWD = [
    # B, Hq, Hkv, Nq, Nk, d, causal, lens
    (2, 4, 2, 300, 300, 128, True, None),
    (2, 4, 2, 300, 300, 128, False, None),
    (1, 4, 4, 257, 257, 64, True, None),
    (1, 4, 4, 257, 257, 64, False, None),
    (1, 4, 1, 200, 333, 64, False, None),
    (1, 2, 1, 333, 200, 128, True, None),
    (1, 2, 1, 200, 333, 128, True, None),
    (3, 2, 2, 1, 1, 128, True, None),
    (1, 4, 2, 0, 0, 128, True, [1, 127, 128, 129, 300, 0, 64, 513]),
    (1, 4, 2, 0, 0, 128, False, [1, 127, 128, 129, 300, 0, 64, 513]),
    (1, 8, 2, 0, 0, 64, True, [5, 260, 0, 128, 77]),
    (2, 16, 4, 700, 700, 128, True, None),
]


def _id(c):
    b, hq, hkv, nq, nk, d, causal, lens = c
    shape = f"lens{len(lens)}" if lens else f"B{b}_Nq{nq}_Nk{nk}"
    return f"bwd_{shape}_H{hq}x{hkv}_d{d}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case", SMALL_BWD, ids=[_id(c) for c in SMALL_BWD])
def test_bwd_small_full_parity(case):
    b, hq, hkv, nq, nk, d, causal, lens = case
    name = _id(case)
    say(f"[case] {name}")
    seed = zlib.crc32(name.encode())
    inp = W.draw(len(lens) if lens else b, hq, hkv, nq, nk, d, "bf16", seed=seed, lens=lens)
    do, do_bits = _draw_do(inp.q.shape, seed + 1)
    scale = 1.0 / math.sqrt(d)
    got = _run(inp, do_bits, causal, scale)
    ref = oracle.attention_bwd_ref(inp.q, inp.k, inp.v, do, scale, causal, inp.cu_seqlens)
    bounds = _bounds_full(inp, do, scale, causal)
    for nm, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        _check(f"{name} {nm}", g, r, bd)


WINDOW_BWD = [
    # B, Hq, Hkv, Nq, Nk, d, causal, lens, window
    (2, 4, 2, 700, 700, 128, True, None, (100, -1)),
    (1, 4, 4, 600, 600, 64, False, None, (64, 64)),
    (1, 2, 1, 900, 900, 128, True, None, (257, 3)),
    (1, 4, 1, 333, 200, 128, False, None, (-1, 30)),
    (1, 4, 2, 0, 0, 128, True, [1, 127, 300, 0, 513, 64], (130, -1)),
]


@pytest.mark.parametrize("case", WINDOW_BWD,
                         ids=[f"win{c[8][0]}_{c[8][1]}_" + _id(c[:8]) for c in WINDOW_BWD])
def test_bwd_window_parity(case):
    b, hq, hkv, nq, nk, d, causal, lens, win = case
    name = f"win{win[0]}_{win[1]}_" + _id(case[:8])
    say(f"[case] {name}")
    seed = zlib.crc32(name.encode())
    inp = W.draw(len(lens) if lens else b, hq, hkv, nq, nk, d, "bf16", seed=seed, lens=lens)
    do, do_bits = _draw_do(inp.q.shape, seed + 1)
    scale = 1.0 / math.sqrt(d)
    got = _run(inp, do_bits, causal, scale, window=win)
    ref = oracle.attention_bwd_ref(inp.q, inp.k, inp.v, do, scale, causal, inp.cu_seqlens,
                                   window=win)
    bounds = _bounds_full(inp, do, scale, causal, window=win)
    for nm, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        _check(f"{name} {nm}", g, r, bd)


BIAS_BWD = [
    # name, B, Hq, Hkv, Nq, Nk, d, causal, lens, (bias entries, bias heads), sigma, extras
    ("per_head", 2, 4, 2, 300, 300, 128, True, None, (2, 4), 1.0, {}),
    ("head_shared_ragged", 1, 4, 1, 200, 333, 64, False, None, (1, 1), 2.0, {}),
    ("key_padding_dead_rows", 2, 4, 2, 300, 300, 128, False, None, (2, 4), 1.0,
     dict(key_lens=[300, 97], dead_rows=[(0, 1, 5), (1, 3, 299)])),
    ("causal_dead_row0", 1, 4, 4, 257, 257, 64, True, None, (1, 1), 1.0,
     dict(dead_rows=[(0, 0, 0)])),
    ("large_bias", 1, 2, 1, 333, 200, 128, True, None, (1, 2), 8.0, {}),
    ("packed", 1, 4, 2, 0, 0, 128, True, [1, 127, 300, 0, 513, 64], (6, 4), 1.0, {}),
]


@pytest.mark.parametrize("case", BIAS_BWD, ids=[c[0] for c in BIAS_BWD])
def test_bwd_bias_parity(case):
    name, b, hq, hkv, nq, nk, d, causal, lens, (be, bh), sigma, extra = case
    say(f"[case] bwd bias {name}")
    seed = zlib.crc32(("bwd bias " + name).encode())
    inp = W.draw(len(lens) if lens else b, hq, hkv, nq, nk, d, "bf16", seed=seed, lens=lens)
    rows = inp.max_seqlen if lens else nq
    cols = inp.max_seqlen if lens else nk
    bias = W.draw_bias(be, bh, rows, cols, seed + 2, sigma, **extra)
    do, do_bits = _draw_do(inp.q.shape, seed + 1)
    scale = 1.0 / math.sqrt(d)
    got = _run(inp, do_bits, causal, scale, bias=bias)
    ref = oracle.attention_bwd_ref(inp.q, inp.k, inp.v, do, scale, causal, inp.cu_seqlens,
                                   bias=bias.values)
    bounds = _bounds_full(inp, do, scale, causal, bias=bias.values)
    for nm, g, r, bd in zip(("dQ", "dK", "dV"), got, ref, bounds):
        _check(f"bias {name} {nm}", g, r, bd)


def test_bwd_one_sided_calls_write_zeros():
    """Nq == 0: dK = dV = 0; Nk == 0: dQ = 0 (no key is seen)."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] bwd one-sided")
    dev = torch.device("cuda")
    k = torch.randn(1, 70, 2, 64, device=dev).bfloat16()
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    st = fa.fa_bwd(0, k.data_ptr(), k.data_ptr(), 0, 0, 0, 0, dk.data_ptr(), dv.data_ptr(), 0,
                   1, 4, 2, 0, 70, 64, 0.125, 1, None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_last_error()
    q = torch.randn(1, 50, 4, 64, device=dev).bfloat16()
    lse = torch.full((1, 4, 50), float("-inf"), device=dev)
    dq = torch.full_like(q, 7.0)
    dsum = torch.empty_like(lse)
    st = fa.fa_bwd(q.data_ptr(), 0, 0, q.data_ptr(), q.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                   0, 0, dsum.data_ptr(), 1, 4, 2, 50, 0, 64, 0.125, 0, None,
                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_last_error()
    torch.cuda.synchronize()
    assert bool((dk == 0).all()) and bool((dv == 0).all())
    assert bool((dq == 0).all())


def test_bwd_deterministic():
    """Two calls on the same inputs give bitwise-identical gradients."""
    say("[case] bwd determinism")
    inp = W.draw(1, 8, 2, 900, 900, 128, "bf16", seed=77)
    _, do_bits = _draw_do(inp.q.shape, 78)
    a = _run(inp, do_bits, True, 1 / math.sqrt(128))
    b = _run(inp, do_bits, True, 1 / math.sqrt(128))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_workload4_sampled():
    """Causal GQA 32/8, N=8192, d=128 at full size: sampled dQ rows (every
    256-row tile boundary kind plus random rows) and the dK/dV rows of
    sampled keys of two K/V heads, formed one by one by the oracle."""
    import torch

    import exact_io_aware_63_amd as fa
    w = W.WORKLOADS[4]
    say("[case] bwd workload 4 (sampled)")
    inp = W.draw_workload(4)
    do, do_bits = _draw_do(inp.q.shape, 2004)
    q, k, v, _ = to_device(inp)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=w.scale)
    dod = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(q.device)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, dod, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    n = w.n
    qrows = sorted({0, 1, 63, 64, 127, 128, 255, 256, n // 2, n - 2, n - 1} |
                   set(rng.integers(0, n, 12).tolist()))
    q_picks = np.array([(0, int(rng.integers(w.hq)), i) for i in qrows])
    krows = sorted({0, 1, 127, 128, 4095, n - 1} | set(rng.integers(0, n, 6).tolist()))
    kv_picks = np.array([(0, g, j) for g in (0, 5) for j in krows])
    ref_dq, ref_dk, ref_dv = oracle.attention_bwd_picked(inp.q, inp.k, inp.v, do, w.scale, True,
                                                         q_picks, kv_picks)
    got_dq = dq[0, q_picks[:, 2], q_picks[:, 1]].float().cpu().double().numpy()
    got_dk = dk[0, kv_picks[:, 2], kv_picks[:, 1]].float().cpu().double().numpy()
    got_dv = dv[0, kv_picks[:, 2], kv_picks[:, 1]].float().cpu().double().numpy()
    # magnitude bounds of the picked rows
    bq = np.zeros_like(ref_dq)
    for r, (s, h, i) in enumerate(q_picks):
        g = oracle.kv_head_of(h, w.hq, w.hkv)
        p, wt = _head_terms(inp.q[0, :, h].astype(np.float64), inp.k[0, :, g].astype(np.float64),
                            inp.v[0, :, g].astype(np.float64), do[0, :, h].astype(np.float64),
                            w.scale, True, rows=[i])
        bq[r] = w.scale * ((p * wt) @ np.abs(inp.k[0, :, g].astype(np.float64)))[0]
    bk = np.zeros_like(ref_dk)
    bv = np.zeros_like(ref_dv)
    group = w.hq // w.hkv
    for g in (0, 5):
        sel = np.nonzero(kv_picks[:, 1] == g)[0]
        cols = kv_picks[sel, 2]
        kh, vh = inp.k[0, :, g].astype(np.float64), inp.v[0, :, g].astype(np.float64)
        for h in range(g * group, (g + 1) * group):
            qh, doh = inp.q[0, :, h].astype(np.float64), do[0, :, h].astype(np.float64)
            for c0 in range(0, n, 1024):
                rows = np.arange(c0, min(n, c0 + 1024))
                p, wt = _head_terms(qh, kh, vh, doh, w.scale, True, rows=rows)
                bv[sel] += p[:, cols].T @ np.abs(doh[rows])
                bk[sel] += w.scale * ((p * wt)[:, cols].T @ np.abs(qh[rows]))
    _check("workload 4 dQ rows", got_dq, ref_dq, bq)
    _check("workload 4 dK rows", got_dk, ref_dk, bk)
    _check("workload 4 dV rows", got_dv, ref_dv, bv)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
