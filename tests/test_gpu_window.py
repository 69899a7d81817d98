"""GPU parity of the sliding-window forward (fa_fwd_window) against the
fp64 oracle with the same window, and agreement with fa_fwd when the
window covers everything."""
import math
import zlib

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_parity, pick_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_63_amd  # noqa: F401


CASES = [
    # B, Hq, Hkv, Nq, Nk, d, causal, (left, right), lens
    (2, 4, 2, 700, 700, 128, True, (100, -1), None),
    (2, 4, 2, 700, 700, 128, True, (0, -1), None),
    (1, 4, 4, 600, 600, 64, True, (63, -1), None),
    (1, 4, 4, 600, 600, 64, True, (64, -1), None),
    (1, 2, 1, 900, 900, 128, True, (255, -1), None),
    (1, 2, 1, 900, 900, 128, True, (256, -1), None),
    (1, 2, 1, 900, 900, 128, True, (257, 3), None),
    (2, 4, 2, 500, 500, 128, False, (64, 64), None),
    (1, 4, 1, 333, 200, 64, False, (0, 0), None),
    (1, 4, 1, 200, 333, 128, False, (-1, 30), None),
    (1, 4, 2, 0, 0, 128, True, (130, -1), [1, 127, 300, 0, 513, 64]),
]


def _id(c):
    b, hq, hkv, nq, nk, d, causal, win, lens = c
    shape = f"lens{len(lens)}" if lens else f"B{b}_Nq{nq}_Nk{nk}"
    return f"win{win[0]}_{win[1]}_{shape}_H{hq}x{hkv}_d{d}_{'causal' if causal else 'full'}"


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_window_parity(case):
    import torch

    import exact_io_aware_63_amd as fa
    b, hq, hkv, nq, nk, d, causal, win, lens = case
    name = _id(case)
    say(f"[case] {name}")
    inp = W.draw(len(lens) if lens else b, hq, hkv, nq, nk, d, "bf16",
                 seed=zlib.crc32(name.encode()), lens=lens)
    q, k, v, cu = to_device(inp)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.attention_fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu,
                              max_seqlen=inp.max_seqlen if cu is not None else None, window=win)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, scale, causal, inp.cu_seqlens,
                                          window=win)
    assert_parity(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref,
                  "bf16", name)


def test_wide_window_is_fa_fwd():
    """A window wider than every sequence gives fa_fwd's result bit for bit
    (the same blocks in the same order). The non-causal case uses a grid of
    more 256-row tiles than compute units (2 x 48 heads x 4 tiles), where
    fa_fwd does not split the keys between wave pairs either."""
    import torch

    import exact_io_aware_63_amd as fa
    say("[case] wide window vs fa_fwd")
    for causal in (True, False):
        inp = W.draw(2 if not causal else 1, 48 if not causal else 8, 2, 1000, 1000, 128, "bf16",
                     seed=5)
        q, k, v, _ = to_device(inp)
        o1, l1 = fa.attention_fwd(q, k, v, causal=causal)
        o2, l2 = fa.attention_fwd(q, k, v, causal=causal, window=(5000, 5000))
        # the widest bounds an int holds: the host clamps them to max(Nq, Nk)
        o3, l3 = fa.attention_fwd(q, k, v, causal=causal, window=(2**31 - 1, 2**31 - 1))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_window_workload4_sampled():
    """Causal GQA 32/8, N=8192, d=128 with a 1024-key left window at full
    size, on sampled rows (the oracle forms each picked row alone)."""
    import torch

    import exact_io_aware_63_amd as fa
    w = W.WORKLOADS[4]
    say("[case] window 1024 on workload 4 (sampled)")
    inp = W.draw_workload(4)
    q, k, v, _ = to_device(inp)
    o, lse = fa.attention_fwd(q, k, v, causal=True, scale=w.scale, window=(1024, -1))
    torch.cuda.synchronize()
    picks = pick_rows(inp, 40, seed=44, hq=w.hq)
    pt = torch.from_numpy(picks).to(o.device)
    og = o[pt[:, 0], pt[:, 2], pt[:, 1]].float().cpu().double().numpy()
    lg = lse[pt[:, 0], pt[:, 1], pt[:, 2]].cpu().double().numpy()
    o_ref, lse_ref = oracle.attention_picked(inp.q, inp.k, inp.v, w.scale, True, picks,
                                             window=(1024, -1))
    assert_parity(og, lg, o_ref, lse_ref, "bf16", f"window 1024, {len(picks)} rows")
