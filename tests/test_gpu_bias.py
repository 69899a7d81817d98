"""GPU parity of the biased forward (fa_fwd_bias) against the fp64 oracle
with the same bias: per-head, head-shared and fully shared biases, -inf key
padding and fully masked rows, large biases that force the rescale path,
packed sequences, ragged tails and a full-size sampled check."""
import math
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_parity, gather_picks, pick_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_63_amd  # noqa: F401


def _bias_tensor(bias):
    import torch
    return torch.from_numpy(bias.bits.view(np.int16)).view(torch.bfloat16).to("cuda")


CASES = [
    # name, B, Hq, Hkv, Nq, Nk, d, causal, (bias entries, bias heads), sigma, lens, extras
    ("per_head", 2, 4, 2, 700, 700, 128, True, (2, 4), 1.0, None, {}),
    ("head_shared_ragged", 2, 4, 1, 333, 517, 64, False, (2, 1), 2.0, None, {}),
    ("all_shared", 1, 8, 2, 1000, 1000, 128, False, (1, 1), 1.0, None, {}),
    ("key_padding", 3, 4, 2, 600, 600, 128, False, (3, 4), 1.0, None,
     dict(key_lens=[600, 257, 1], dead_rows=[(0, 1, 5), (2, 3, 599)])),
    ("key_padding_causal", 2, 4, 4, 300, 300, 64, True, (2, 1), 0.5, None,
     dict(key_lens=[70, 300], dead_rows=[(1, 0, 0)])),
    ("large_bias_rescale", 1, 2, 1, 900, 900, 128, True, (1, 2), 20.0, None, {}),
    ("packed", 0, 4, 2, 0, 0, 128, True, (6, 4), 1.0, [1, 127, 300, 0, 513, 64], {}),
    ("tail_130", 1, 4, 4, 130, 130, 64, True, (1, 4), 1.0, None, {}),
    ("tiny", 1, 2, 1, 1, 3, 128, False, (1, 2), 1.0, None, {}),
]


def _run(case):
    import torch

    import exact_io_aware_63_amd as fa
    name, b, hq, hkv, nq, nk, d, causal, (be, bh), sigma, lens, extra = case
    say(f"[case] bias {name}")
    seed = zlib.crc32(name.encode())
    inp = W.draw(len(lens) if lens else b, hq, hkv, nq, nk, d, "bf16", seed=seed, lens=lens)
    rows = cols = inp.max_seqlen if lens else None
    bias = W.draw_bias(be, bh, rows or nq, cols or nk, seed + 1, sigma, **extra)
    q, k, v, cu = to_device(inp)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu,
                              max_seqlen=inp.max_seqlen if cu is not None else None,
                              bias=_bias_tensor(bias))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, scale, causal, inp.cu_seqlens,
                                          bias=bias.values)
    return inp, o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bias_parity(case):
    inp, o, lse, o_ref, lse_ref = _run(case)
    assert_parity(o, lse, o_ref, lse_ref, "bf16", f"bias {case[0]}")


def test_bias_dead_rows_are_empty():
    """Rows whose bias is -inf everywhere get O = 0 and LSE = -inf exactly."""
    case = [c for c in CASES if c[0] == "key_padding"][0]
    inp, o, lse, _, _ = _run(case)
    for e, h, r in case[-1]["dead_rows"]:
        assert np.all(o[e, r, h] == 0.0), (e, h, r)
        assert np.isneginf(lse[e, h, r]), (e, h, r)


def test_zero_bias_matches_fa_fwd():
    """A zero bias reproduces fa_fwd within bf16 rounding of O (the score
    path differs only in the order of the scale multiplications)."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] zero bias vs fa_fwd")
    inp = W.draw(1, 8, 2, 800, 800, 128, "bf16", seed=77)
    q, k, v, _ = to_device(inp)
    zero = torch.zeros(1, 1, 800, 800, dtype=torch.bfloat16, device="cuda")
    for causal in (True, False):
        o1, l1 = fa.attention_fwd(q, k, v, causal=causal)
        o2, l2 = fa.attention_fwd(q, k, v, causal=causal, bias=zero)
        torch.cuda.synchronize()
        do = (o1.float() - o2.float()).abs().max().item()
        dl = (l1 - l2).abs().max().item()
        say(f"[parity] zero bias causal={causal}: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
        assert do <= 8e-3 and dl <= 1e-5


def test_bias_is_deterministic():
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] bias determinism")
    inp = W.draw(1, 4, 2, 600, 600, 128, "bf16", seed=78)
    bias = _bias_tensor(W.draw_bias(1, 4, 600, 600, 79, 3.0))
    q, k, v, _ = to_device(inp)
    o1, l1 = fa.attention_fwd(q, k, v, causal=True, bias=bias)
    o2, l2 = fa.attention_fwd(q, k, v, causal=True, bias=bias)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bias_full_size_sampled():
    """Causal GQA 32/8 heads, N = 8192, d = 128 with one bias shared by
    every head ([1, 1, 8192, 8192]); rows sampled at tile edges and at
    random, each formed whole by the oracle."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] bias full size: causal GQA 32/8, N=8192, d=128, shared bias")
    w = W.WORKLOADS[4]
    inp = W.draw_workload(4)
    bias = W.draw_bias(1, 1, w.n, w.n, 4004, 1.0)
    q, k, v, _ = to_device(inp)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=w.scale, bias=_bias_tensor(bias))
    torch.cuda.synchronize()
    picks = pick_rows(inp, 48, seed=4004, hq=w.hq)
    go, gl = gather_picks(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), picks, inp)
    ro, rl = oracle.attention_picked(inp.q, inp.k, inp.v, w.scale, True, picks, bias=bias.values)
    assert_parity(go, gl, ro, rl, "bf16", "bias full size sampled")
