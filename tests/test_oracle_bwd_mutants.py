"""Plant plausible mistakes in the backward oracle and check the pins
catch each one.

Every mutant replaces one step of ``oracle.attention``'s gradient code (on
the CPU, through monkeypatch) with a wrong variant: a dropped or sign-flipped
term, a sum over the wrong axis, a missing scale, a swapped operand or
output, an ignored mask, a group sum that overwrites. The backward pin suite
must fail for each of them.
"""
import numpy as np
import pytest

import oracle.attention as A
from oracle_bwd_pins import ALL_BWD_PINS

_orig_head_bwd = A.attention_head_bwd


def _head_bwd_variant(change):
    """The oracle's per-head gradient steps with one planted change."""
    def f(q, k, v, do, scale, causal, window=None, bias=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        lq, lk = q.shape[0], k.shape[0]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        if lq == 0 or lk == 0:
            return dq, dk, dv
        r = np.arange(lq)
        s = A.scores(q, k, scale)
        if bias is not None and change != "bias_ignored":
            s = s + np.asarray(bias, dtype=np.float64)[:lq, :lk]
        if change != "mask_ignored":
            s = np.where(A.visible_mask(r, lk, causal, window), s, -np.inf)
        p, _, _ = A.softmax_rows(s)
        dp = do @ v.T
        ds = A.softmax_rows_bwd(p, dp)
        dv = (ds.T @ do) if change == "dv_from_ds" else (p.T @ do)
        dq = (ds @ k) if change == "dq_unscaled" else scale * (ds @ k)
        dk = scale * (ds.T @ (v if change == "dk_from_v" else q))
        if change == "dk_dv_swapped":
            dk, dv = dv, dk
        return dq, dk, dv
    return f


def _bwd_ref_group_overwrites(q, k, v, do, scale, causal, cu_seqlens=None, window=None,
                              bias=None):
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if cu_seqlens is None:
        hq, hkv = q.shape[2], k.shape[2]
        for b in range(q.shape[0]):
            for h in range(hq):
                g = A.kv_head_of(h, hq, hkv)
                a, bk, bv = A.attention_head_bwd(q[b, :, h], k[b, :, g], v[b, :, g], do[b, :, h],
                                                 scale, causal, window, A.bias_of(bias, b, h))
                dq[b, :, h], dk[b, :, g], dv[b, :, g] = a, bk, bv
        return dq, dk, dv
    hq, hkv = q.shape[1], k.shape[1]
    cu = np.asarray(cu_seqlens)
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for h in range(hq):
            g = A.kv_head_of(h, hq, hkv)
            a, bk, bv = A.attention_head_bwd(q[lo:hi, h], k[lo:hi, g], v[lo:hi, g], do[lo:hi, h],
                                             scale, causal, window, A.bias_of(bias, s, h))
            dq[lo:hi, h], dk[lo:hi, g], dv[lo:hi, g] = a, bk, bv
    return dq, dk, dv


MUTANTS = {
    "softmax_bwd_no_rowsum": ("softmax_rows_bwd", lambda p, dp: p * dp),
    "softmax_bwd_plus_rowsum": ("softmax_rows_bwd",
                                lambda p, dp: p * (dp + (p * dp).sum(axis=1, keepdims=True))),
    "softmax_bwd_wrong_axis": ("softmax_rows_bwd",
                               lambda p, dp: p * (dp - (p * dp).sum(axis=0, keepdims=True))),
    "softmax_bwd_no_p_factor": ("softmax_rows_bwd",
                                lambda p, dp: (dp - (p * dp).sum(axis=1, keepdims=True)) * (p > 0)),
    "head_dq_unscaled": ("attention_head_bwd", _head_bwd_variant("dq_unscaled")),
    "head_dk_from_v": ("attention_head_bwd", _head_bwd_variant("dk_from_v")),
    "head_dv_from_ds": ("attention_head_bwd", _head_bwd_variant("dv_from_ds")),
    "head_dk_dv_swapped": ("attention_head_bwd", _head_bwd_variant("dk_dv_swapped")),
    "head_mask_ignored": ("attention_head_bwd", _head_bwd_variant("mask_ignored")),
    "head_bias_ignored": ("attention_head_bwd", _head_bwd_variant("bias_ignored")),
    "gqa_group_overwrites": ("attention_bwd_ref", _bwd_ref_group_overwrites),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    for pin in ALL_BWD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_variant_passes(monkeypatch):
    """The mutant scaffold itself, with no change, passes every pin."""
    monkeypatch.setattr(A, "attention_head_bwd", _head_bwd_variant("none"))
    for pin in ALL_BWD_PINS:
        pin()
