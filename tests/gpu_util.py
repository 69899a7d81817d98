"""Helpers shared by the GPU tests: move seeded inputs to the device, call
the library through its binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the parity bar: max |O_gpu - O_ref| and max |LSE_gpu - LSE_ref|
# against the unrounded fp64 oracle.
TOL_O = {"bf16": 2e-2, "fp32": 1e-5}
TOL_LSE = {"bf16": 1e-3, "fp32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda"):
    import torch
    if inp.dtype == "bf16":
        def t(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        q, k, v = t(inp.q_bits), t(inp.k_bits), t(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(x).to(device) for x in (inp.q, inp.k, inp.v))
    cu = None
    if inp.cu_seqlens is not None:
        cu = torch.from_numpy(inp.cu_seqlens).to(device)
    return q, k, v, cu


def run_gpu(inp, causal, scale, device="cuda"):
    """Run the library on ``inp``; returns (O float64 numpy, LSE float64 numpy)."""
    import torch

    import exact_io_aware_63_amd as fa
    q, k, v, cu = to_device(inp, device)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu,
                              max_seqlen=inp.max_seqlen if cu is not None else None)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(same_inf, 0.0, np.abs(a - b))
    if not np.all(np.isfinite(d)):
        return float("inf")
    return float(d.max()) if d.size else 0.0


def assert_parity(o, lse, o_ref, lse_ref, dtype, what):
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    say(f"[parity] {what}: max|dO|={eo:.3e} (tol {TOL_O[dtype]:.0e}) "
        f"max|dLSE|={el:.3e} (tol {TOL_LSE[dtype]:.0e})")
    assert eo <= TOL_O[dtype], f"{what}: max|dO| {eo:.3e} > {TOL_O[dtype]}"
    assert el <= TOL_LSE[dtype], f"{what}: max|dLSE| {el:.3e} > {TOL_LSE[dtype]}"


def pick_rows(inp, n_random, seed, hq):
    """(s, h, i) picks: boundary rows of every sequence plus random ones."""
    rng = np.random.default_rng(seed)
    if inp.lens is None:
        nseq, lens = inp.q.shape[0], [inp.q.shape[1]] * inp.q.shape[0]
    else:
        nseq, lens = len(inp.lens), [int(x) for x in inp.lens]
    picks = []
    for s in range(nseq):
        L = lens[s]
        if L == 0:
            continue
        for i in {0, 1, 31, 32, 63, 64, 127, 128, 129, L // 2, L - 2, L - 1}:
            if 0 <= i < L:
                picks.append((s, int(rng.integers(hq)), i))
    for _ in range(n_random):
        s = int(rng.integers(nseq))
        if lens[s] == 0:
            continue
        picks.append((s, int(rng.integers(hq)), int(rng.integers(lens[s]))))
    return np.array(picks, dtype=np.int64)


def gather_picks(o, lse, picks, inp):
    """Select picked rows from full GPU outputs (layouts of the C ABI)."""
    if inp.cu_seqlens is None:
        return (o[picks[:, 0], picks[:, 2], picks[:, 1]],
                lse[picks[:, 0], picks[:, 1], picks[:, 2]])
    cu = inp.cu_seqlens.astype(np.int64)
    tok = cu[picks[:, 0]] + picks[:, 2]
    return o[tok, picks[:, 1]], lse[picks[:, 1], tok]


def oracle_sequence(q, k, v, scale, causal, workers=8):
    """The fp64 oracle on every head of one sequence, heads run in a thread
    pool (numpy's matrix products and exponentials release the GIL).
    q [L, Hq, d], k and v [L, Hkv, d]; returns (O [L, Hq, d], LSE [Hq, L])."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    lq, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((lq, hq, d), dtype=np.float64)
    lse = np.full((hq, lq), -np.inf)

    def one(h):
        g = oracle.kv_head_of(h, hq, hkv)
        out[:, h], lse[h] = oracle.attention_head(q[:, h], k[:, g], v[:, g], scale, causal)

    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, range(hq)))
    return out, lse
