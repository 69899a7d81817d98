"""fa_fwd_splitkv_noalloc (the allocation-free split-K/V forward) against
fa_fwd_splitkv with a caller workspace, through the C ABI: two calls in a
row, the second smaller, each compared with the workspace entry point on the
same inputs. Both run the same kernels on the same partial-result layout,
so the outputs must agree bit for bit; the first call's outputs are also
checked against the fp64 oracle at the forward's bf16 tolerance."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_LSE, TOL_O, max_err, say

pytestmark = pytest.mark.gpu


def _dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def _both(fa, b, hq, hkv, nq, nk, d, causal, lens, splits, seed):
    """(O, LSE) of the no-alloc entry point, then of fa_fwd_splitkv."""
    import torch
    inp = W.draw(b, hq, hkv, nq, nk, d, "bf16", seed=seed)
    q, k, v = _dev(inp.q_bits), _dev(inp.k_bits), _dev(inp.v_bits)
    sk = torch.tensor(lens, dtype=torch.int32).cuda() if lens is not None else None
    sk_ptr = sk.data_ptr() if sk is not None else None
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (True, False):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((b, hq, nq), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = fa.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                           lse.data_ptr(), b, hq, hkv, nq, nk, d, scale, causal,
                                           sk_ptr, splits, stream)
        else:
            nbytes = fa.fa_fwd_splitkv_workspace_bytes(b, hq, nq, d, splits)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), b, hq, hkv, nq, nk, d, scale, causal, sk_ptr,
                                   splits, ws.data_ptr(), nbytes, stream)
        assert st == 0, fa.fa_last_error()
        torch.cuda.synchronize()
        outs.append((o, lse))
    return inp, scale, outs


def test_noalloc_matches_workspace_entry_point_twice():
    import torch

    import exact_io_aware_63_amd as fa
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 4 entries, GQA 32/8, 2000-key cache with ragged lengths, 8 splits
    say("[case] noalloc call 1: B4 H32x8 Nq1 Nk2000 d128 splits8")
    lens = [2000, 1, 1337, 0]
    inp, scale, ((o1, l1), (o2, l2)) = _both(fa, 4, 32, 8, 1, 2000, 128, False, lens, 8, 71)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "first call differs from fa_fwd_splitkv"
    o_ref = np.zeros((4, 1, 32, 128))
    lse_ref = np.full((4, 32, 1), -np.inf)
    for b in range(4):
        for h in range(32):
            g = oracle.kv_head_of(h, 32, 8)
            ob, lb = oracle.attention_head(inp.q[b, :, h], inp.k[b, :lens[b], g],
                                           inp.v[b, :lens[b], g], scale, False)
            o_ref[b, :, h], lse_ref[b, h] = ob, lb
    eo = max_err(o1.float().cpu().double().numpy(), o_ref)
    el = max_err(l1.cpu().double().numpy(), lse_ref)
    say(f"[parity] noalloc call 1: max|dO| {eo:.3e} max|dLSE| {el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE["bf16"]
    # second call, smaller: the scratch still holds the first call's partials
    say("[case] noalloc call 2: B2 H16x2 Nq2 Nk300 d64 causal splits3")
    _, _, ((o1, l1), (o2, l2)) = _both(fa, 2, 16, 2, 2, 300, 64, True, None, 3, 72)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "second call differs from fa_fwd_splitkv"
    assert bool(torch.isfinite(o1.float()).all()) and bool(torch.isfinite(l1).all())
