"""GPU parity of the split-K/V (decode) forward against the fp64 oracle.

Each batch entry is compared with the oracle's plain forward over its own
valid keys (``seqlens_k``); the bar is the forward's bf16 tolerance (the
partial outputs are float32, P is rounded to bf16 for P V as in fa_fwd,
and the merge is float32 with one final rounding).
"""
import math
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_LSE, TOL_O, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_63_amd  # noqa: F401


def _dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _reference(inp, lens, scale, causal):
    b_, nq, hq, d = inp.q.shape
    hkv = inp.k.shape[2]
    o = np.zeros((b_, nq, hq, d))
    lse = np.full((b_, hq, nq), -np.inf)
    for b in range(b_):
        L = lens[b]
        for h in range(hq):
            g = oracle.kv_head_of(h, hq, hkv)
            ob, lb = oracle.attention_head(inp.q[b, :, h], inp.k[b, :L, g], inp.v[b, :L, g], scale,
                                           causal)
            o[b, :, h] = ob
            lse[b, h] = lb
    return o, lse


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, seqlens_k (None = all Nk), splits
    (4, 32, 8, 1, 5000, 128, False, [5000, 1, 4097, 0], 1),
    (4, 32, 8, 1, 5000, 128, False, [5000, 1, 4097, 0], 7),
    (4, 32, 8, 1, 5000, 128, False, [5000, 1, 4097, 0], 64),
    (2, 16, 2, 4, 300, 128, True, None, 3),
    (3, 16, 1, 2, 1000, 64, False, [1000, 999, 64], 5),
    (2, 8, 8, 1, 129, 64, True, None, 2),
]


def _id(c):
    b, hq, hkv, nq, nk, d, causal, lens, n = c
    return (f"B{b}_H{hq}x{hkv}_Nq{nq}_Nk{nk}_d{d}_{'causal' if causal else 'full'}"
            f"_{'lens' if lens else 'fixed'}_splits{n}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_splitkv_parity(case):
    import torch

    import exact_io_aware_63_amd as fa
    b, hq, hkv, nq, nk, d, causal, lens, n = case
    name = _id(case)
    say(f"[case] splitkv {name}")
    inp = W.draw(b, hq, hkv, nq, nk, d, "bf16", seed=zlib.crc32(name.encode()))
    scale = 1.0 / math.sqrt(d)
    sk = torch.tensor(lens, dtype=torch.int32).cuda() if lens else None
    o, lse = fa.attention_fwd_splitkv(_dev(inp.q_bits), _dev(inp.k_bits), _dev(inp.v_bits),
                                      num_splits=n, causal=causal, scale=scale, seqlens_k=sk)
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    o_ref, lse_ref = _reference(inp, lens or [nk] * b, scale, causal)
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    say(f"[parity] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE["bf16"]


def test_splitkv_no_keys():
    """Nk == 0: every row sees no key, O = 0 and LSE = -inf."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] splitkv Nk=0")
    q = torch.randn(2, 1, 8, 64).bfloat16().cuda()
    k = torch.zeros(2, 0, 2, 64).bfloat16().cuda()
    o, lse = fa.attention_fwd_splitkv(q, k, k.clone(), num_splits=3)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_splitkv_matches_fwd():
    """The split path and fa_fwd compute the same function: on one decode
    input their outputs agree to the bf16 bar."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] splitkv vs fa_fwd")
    inp = W.draw(2, 32, 8, 1, 3000, 128, "bf16", seed=91)
    q, k, v = _dev(inp.q_bits), _dev(inp.k_bits), _dev(inp.v_bits)
    o1, l1 = fa.attention_fwd_splitkv(q, k, v, num_splits=16)
    o2, l2 = fa.attention_fwd(q, k, v)
    torch.cuda.synchronize()
    assert max_err(o1.float().cpu().numpy(), o2.float().cpu().numpy()) <= TOL_O["bf16"]
    assert max_err(l1.cpu().numpy(), l2.cpu().numpy()) <= TOL_LSE["bf16"]


def test_splitkv_recommended_splits_parity():
    """The split count the library recommends for this device (used by the
    decode benchmark) on a bench-like decode shape with ragged lengths."""
    import torch

    import exact_io_aware_63_amd as fa
    b, hq, hkv, nk, d = 16, 32, 8, 2048, 128
    n = fa.fa_fwd_splitkv_num_splits(b, hkv, nk, 0)
    say(f"[case] splitkv recommended splits: {n}")
    assert 1 <= n <= 1024
    lens = [nk - 97 * i for i in range(b)]
    inp = W.draw(b, hq, hkv, 1, nk, d, "bf16", seed=4242)
    scale = 1.0 / math.sqrt(d)
    sk = torch.tensor(lens, dtype=torch.int32).cuda()
    o, lse = fa.attention_fwd_splitkv(_dev(inp.q_bits), _dev(inp.k_bits), _dev(inp.v_bits),
                                      num_splits=n, causal=False, scale=scale, seqlens_k=sk)
    torch.cuda.synchronize()
    o_ref, lse_ref = _reference(inp, lens, scale, False)
    eo = max_err(o.float().cpu().double().numpy(), o_ref)
    el = max_err(lse.cpu().double().numpy(), lse_ref)
    say(f"[parity] recommended splits {n}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE["bf16"]
