"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def fa():
    import exact_io_aware_63_amd as fa
    return fa


def test_header_declares_expected_entry_points():
    assert _declared_functions() == sorted(
        ["fa_fwd", "fa_fwd_fp32", "fa_fwd_window", "fa_fwd_bias", "fa_bwd", "fa_bwd_window",
         "fa_bwd_bias", "fa_fwd_splitkv", "fa_fwd_fp8", "fa_fwd_fp8_workspace_bytes",
         "fa_fwd_splitkv_workspace_bytes", "fa_fwd_splitkv_num_splits", "fa_fwd_splitkv_noalloc",
         "fa_check_cu_seqlens", "fa_status_string", "fa_last_error", "fa_version"])


def test_library_exports_every_declared_symbol(fa):
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), f"libfa.so does not export {name}"
    assert set(fa.EXPORTED) == set(_declared_functions())


def test_binding_names_match_c_names(fa):
    for name in _declared_functions():
        assert callable(getattr(fa, name))


def test_version_and_status_strings(fa):
    assert fa.fa_version() == 10000
    for st in (0, -1, -2, -3, -4, -5):
        assert fa.fa_status_string(st)
    assert fa.fa_status_string(0) == "FA_OK"
    assert "unknown" in fa.fa_status_string(7)


# Fake, 16-byte aligned, never dereferenced addresses: every case below must
# be rejected before the library touches a pointer or the HIP runtime.
P = 0x10000
GOOD = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=64, scale=0.125,
            causal=0, cu=None, stream=None)


def _call(fa, fn, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
              a["Nk"], a["d"], a["scale"], a["causal"], a["cu"], a["stream"])


BAD = [
    ("null_q", dict(q=0), -1),
    ("null_k", dict(k=0), -1),
    ("null_v", dict(v=0), -1),
    ("null_o", dict(o=0), -1),
    ("null_lse", dict(lse=0), -1),
    ("neg_batch", dict(B=-1), -2),
    ("neg_nq", dict(Nq=-3), -2),
    ("neg_nk", dict(Nk=-1), -2),
    ("zero_hq", dict(Hq=0), -2),
    ("zero_hkv", dict(Hkv=0), -2),
    ("hq_not_multiple", dict(Hq=6, Hkv=4), -2),
    ("packed_nq_ne_nk", dict(cu=P, Nq=8, Nk=9), -2),
    ("d_96", dict(d=96), -3),
    ("d_256", dict(d=256), -3),
    ("d_0", dict(d=0), -3),
    ("scale_nan", dict(scale=math.nan), -4),
    ("scale_inf", dict(scale=math.inf), -4),
    ("misaligned_q", dict(q=P + 8), -4),
    ("misaligned_o", dict(o=P + 2), -4),
    ("misaligned_lse", dict(lse=P + 2), -4),
    ("misaligned_cu", dict(cu=P + 2), -4),
    ("grid_too_large", dict(B=1 << 20, Hq=1 << 10, Hkv=1, Nq=1 << 16, Nk=8), -2),
]


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_fp32"])
@pytest.mark.parametrize("name,kw,status", BAD, ids=[b[0] for b in BAD])
def test_rejects_bad_arguments(fa, entry, name, kw, status):
    st = _call(fa, getattr(fa, entry), **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error(), "a failing call must leave a message"


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_fp32"])
@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0),
                                dict(Nq=0, cu=P, Nk=0)])
def test_empty_work_is_a_noop(fa, entry, kw):
    assert _call(fa, getattr(fa, entry), **kw) == 0
    assert fa.fa_last_error() == ""


def test_valid_call_without_gpu_fails_cleanly(fa):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _call(fa, fa.fa_fwd)
    assert st == fa.FA_ERR_HIP
    assert "hip" in fa.fa_last_error().lower()


def _call_bias(fa, bias=P, sb=0, sh=64, sr=8, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_bias(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], bias, sb, sh, sr,
                          a["cu"], a["stream"])


BAD_BIAS = [
    ("null_bias", dict(bias=0), -1),
    ("misaligned_bias", dict(bias=P + 4), -4),
    ("negative_entry_stride", dict(sb=-4), -4),
    ("negative_head_stride", dict(sh=-64), -4),
    ("row_stride_below_nk", dict(sr=4), -4),
    ("row_stride_not_multiple_of_4", dict(sr=10), -4),
    ("head_stride_not_multiple_of_4", dict(sh=66), -4),
    ("entry_stride_not_multiple_of_4", dict(sb=2), -4),
    ("base_checks_still_apply", dict(Hq=6, Hkv=4), -2),
    ("null_q", dict(q=0), -1),
]


@pytest.mark.parametrize("name,kw,status", BAD_BIAS, ids=[b[0] for b in BAD_BIAS])
def test_bias_rejects_bad_arguments(fa, name, kw, status):
    st = _call_bias(fa, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error()


def test_bias_empty_work_is_a_noop(fa):
    assert _call_bias(fa, B=0, bias=0) == 0
    assert _call_bias(fa, Nq=0) == 0


def test_bias_valid_call_without_gpu_fails_cleanly(fa):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_bias(fa) == fa.FA_ERR_HIP
    assert _call_bias(fa, sb=0, sh=0, sr=8, causal=1) == fa.FA_ERR_HIP


def test_attention_fwd_checks_tensors(fa):
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention_fwd(q, q, q)          # host tensors are refused
    with pytest.raises(TypeError):
        fa.attention_fwd(q.half(), q.half(), q.half())


# fa_bwd: the same fake addresses; every buffer 16-byte aligned.
GOOD_BWD = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, dsum=P, B=1, Hq=4, Hkv=2, Nq=8,
                Nk=8, d=64, scale=0.125, causal=1, cu=None, stream=None)


def _call_bwd(fa, **kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                     a["dsum"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"],
                     a["causal"], a["cu"], a["stream"])


BAD_BWD = [(f"null_{n}", {n: 0}, -1) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv",
                                                "dsum")] + [
    (f"misaligned_{n}", {n: P + 8}, -4) for n in ("q", "k", "v", "o", "do", "dq", "dk", "dv")] + [
    ("misaligned_lse_4", dict(lse=P + 4), -4),
    ("misaligned_dsum_4", dict(dsum=P + 4), -4),
    ("misaligned_cu", dict(cu=P + 2), -4),
    ("neg_batch", dict(B=-1), -2),
    ("neg_nq", dict(Nq=-1), -2),
    ("hq_not_multiple", dict(Hq=6, Hkv=4), -2),
    ("packed_nq_ne_nk", dict(cu=P, Nq=8, Nk=9), -2),
    ("d_96", dict(d=96), -3),
    ("scale_nan", dict(scale=math.nan), -4),
    ("query_side_null_with_queries", dict(Nk=0, dq=0), -1),
    ("key_side_null_with_keys", dict(Nq=0, dk=0), -1),
]


@pytest.mark.parametrize("name,kw,status", BAD_BWD, ids=[b[0] for b in BAD_BWD])
def test_bwd_rejects_bad_arguments(fa, name, kw, status):
    st = _call_bwd(fa, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error(), "a failing call must leave a message"


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0, Nk=0),
                                dict(B=0, q=0, k=0, v=0, o=0, do=0, lse=0, dq=0, dk=0, dv=0, dsum=0),
                                dict(Nq=0, Nk=0, cu=P)])
def test_bwd_empty_work_is_a_noop(fa, kw):
    assert _call_bwd(fa, **kw) == 0
    assert fa.fa_last_error() == ""


@pytest.mark.parametrize("kw", [dict(Nq=0, q=0, o=0, do=0, lse=0, dsum=0, dq=0),
                                dict(Nk=0, k=0, v=0, dk=0, dv=0), dict()])
def test_bwd_one_sided_and_full_calls_reach_the_device(fa, kw):
    """Nq == 0 (dK = dV = 0 to write) or Nk == 0 (dQ = 0) is not a no-op:
    with the other side's buffers absent it still passes validation and,
    without a GPU, fails at the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = _call_bwd(fa, **kw)
    assert st == fa.FA_ERR_HIP, (st, fa.fa_last_error())


# fa_fwd_splitkv
def _ws(B=2, Hq=8, Nq=1, d=64, n=4):
    rows = B * Hq * Nq * n
    return (rows * d * 4 + 255) // 256 * 256 + rows * 4


def _call_bwd_bias(fa, bias=P, sb=0, sh=64, sr=8, **kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return fa.fa_bwd_bias(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                          a["dv"], a["dsum"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                          a["scale"], a["causal"], bias, sb, sh, sr, a["cu"], a["stream"])


@pytest.mark.parametrize("name,kw,status", BAD_BIAS[:8] + [
    ("bwd_checks_still_apply", dict(dq=0), -1), ("bwd_alignment", dict(dsum=P + 4), -4)],
    ids=[b[0] for b in BAD_BIAS[:8]] + ["bwd_checks_still_apply", "bwd_alignment"])
def test_bwd_bias_rejects_bad_arguments(fa, name, kw, status):
    st = _call_bwd_bias(fa, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error()


def test_bwd_bias_noop_and_no_gpu(fa):
    import torch
    assert _call_bwd_bias(fa, B=0, bias=0) == 0
    assert _call_bwd_bias(fa, Nq=0, Nk=0) == 0
    if not torch.cuda.is_available():
        assert _call_bwd_bias(fa) == fa.FA_ERR_HIP


def test_splitkv_workspace_size(fa):
    assert fa.fa_fwd_splitkv_workspace_bytes(2, 8, 1, 64, 4) == _ws()
    assert fa.fa_fwd_splitkv_workspace_bytes(3, 32, 2, 128, 7) == _ws(3, 32, 2, 128, 7)
    assert fa.fa_fwd_splitkv_workspace_bytes(0, 8, 1, 64, 4) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(2, 8, 1, 64, 0) == 0


GOOD_SKV = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nq=1, Nk=100, d=64, scale=0.125,
                causal=0, seqlens=None, n=4, ws=P * 16, wsb=_ws(), stream=None)


def _call_skv(fa, **kw):
    a = dict(GOOD_SKV)
    a.update(kw)
    return fa.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["seqlens"], a["n"],
                             a["ws"], a["wsb"], a["stream"])


BAD_SKV = [
    ("null_q", dict(q=0), -1), ("null_k", dict(k=0), -1), ("null_o", dict(o=0), -1),
    ("null_lse", dict(lse=0), -1), ("null_ws", dict(ws=0), -1),
    ("neg_nk", dict(Nk=-1), -2), ("hq_not_multiple", dict(Hq=6, Hkv=4), -2),
    ("d_96", dict(d=96), -3),
    ("too_many_rows", dict(Hq=16, Hkv=1, Nq=3), -3),
    ("zero_splits", dict(n=0), -4), ("too_many_splits", dict(n=1025), -4),
    ("scale_nan", dict(scale=math.nan), -4),
    ("workspace_short", dict(wsb=_ws() - 1), -4),
    ("misaligned_ws", dict(ws=P * 16 + 16), -4),
    ("misaligned_q", dict(q=P + 8), -4),
    ("misaligned_seqlens", dict(seqlens=P + 2), -4),
]


@pytest.mark.parametrize("name,kw,status", BAD_SKV, ids=[b[0] for b in BAD_SKV])
def test_splitkv_rejects_bad_arguments(fa, name, kw, status):
    st = _call_skv(fa, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(B=0, q=0, k=0, v=0, o=0, lse=0, ws=0)])
def test_splitkv_empty_work_is_a_noop(fa, kw):
    assert _call_skv(fa, **kw) == 0
    assert fa.fa_last_error() == ""


def test_splitkv_valid_call_without_gpu_fails_cleanly(fa):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_skv(fa) == fa.FA_ERR_HIP
    assert _call_skv(fa, Nk=0, k=0, v=0) == fa.FA_ERR_HIP  # no keys: O = 0, LSE = -inf to write


# fa_fwd_fp8: fake addresses, workspace 256-byte aligned.
GOOD_FP8 = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=4, Hkv=2, Nq=100, Nk=130, d=128, scale=0.1,
                qd=0.5, kd=0.25, vd=2.0, causal=1, ws=P, wsb=1 << 20, stream=None)


def _call_fp8(fa, **kw):
    a = dict(GOOD_FP8)
    a.update(kw)
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                         a["Nq"], a["Nk"], a["d"], a["scale"], a["qd"], a["kd"], a["vd"],
                         a["causal"], a["ws"], a["wsb"], a["stream"])


def test_fp8_workspace_size(fa):
    assert fa.fa_fwd_fp8_workspace_bytes(2, 2, 130) == 2 * 2 * 3 * 8192
    assert fa.fa_fwd_fp8_workspace_bytes(1, 8, 8192) == 8 * 128 * 8192
    assert fa.fa_fwd_fp8_workspace_bytes(0, 2, 10) == 0
    assert fa.fa_fwd_fp8_workspace_bytes(1, 2, 0) == 0


BAD_FP8 = [
    ("null_q", dict(q=0), -1), ("null_k", dict(k=0), -1), ("null_v", dict(v=0), -1),
    ("null_o", dict(o=0), -1), ("null_lse", dict(lse=0), -1), ("null_ws", dict(ws=0), -1),
    ("neg_batch", dict(B=-1), -2), ("hq_not_multiple", dict(Hq=6, Hkv=4), -2),
    ("d_64", dict(d=64), -3), ("d_256", dict(d=256), -3),
    ("scale_nan", dict(scale=math.nan), -4), ("qd_inf", dict(qd=math.inf), -4),
    ("vd_nan", dict(vd=math.nan), -4), ("c_overflow", dict(scale=1e30, qd=1e10, kd=1.0), -4),
    ("misaligned_q", dict(q=P + 8), -4), ("misaligned_o", dict(o=P + 4), -4),
    ("misaligned_ws", dict(ws=P + 16), -4), ("workspace_small", dict(wsb=2 * 2 * 3 * 8192 - 1), -4),
]


@pytest.mark.parametrize("name,kw,status", BAD_FP8, ids=[b[0] for b in BAD_FP8])
def test_fp8_rejects_bad_arguments(fa, name, kw, status):
    st = _call_fp8(fa, **kw)
    assert st == status, (st, fa.fa_last_error())
    assert fa.fa_last_error()


def test_fp8_noop_and_no_gpu(fa):
    import torch
    assert _call_fp8(fa, B=0, q=0, k=0, v=0, o=0, lse=0, ws=0) == 0
    assert _call_fp8(fa, Nq=0) == 0
    if not torch.cuda.is_available():
        assert _call_fp8(fa) == fa.FA_ERR_HIP
        assert _call_fp8(fa, Nk=0, k=0, v=0, ws=0, wsb=0) == fa.FA_ERR_HIP



def _call_window(fa, left, right, **kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], left, right,
                            a["cu"], a["stream"])


@pytest.mark.parametrize("left,right", [(2**31 - 1, 2**31 - 1), (2**31 - 1, -1), (0, 2**31 - 1),
                                        (-5, -7)])
def test_window_any_int_bound_passes_host_checks(fa, left, right):
    """Bounds up to INT_MAX are legal (the host clamps them to max(Nq, Nk));
    without a GPU the call gets as far as the device check."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _call_window(fa, left, right) == fa.FA_ERR_HIP
    assert _call_window(fa, left, right, causal=1, Nq=8, Nk=1000) == fa.FA_ERR_HIP


def test_window_rejects_sequences_beyond_2_pow_30(fa):
    """A window with Nq or Nk above 2^30 could overflow i + bound in int."""
    big = (1 << 30) + 1
    assert _call_window(fa, 4, 4, Hq=1, Hkv=1, Nq=big, Nk=8) == fa.FA_ERR_SHAPE
    assert "2^30" in fa.fa_last_error()
    assert _call_window(fa, -1, 4, Hq=1, Hkv=1, Nq=8, Nk=big) == fa.FA_ERR_SHAPE


def test_attention_fwd_checks_output_buffers(fa):
    """Wrong caller-supplied O or LSE buffers are refused before any call."""
    import torch
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 4, dtype=torch.float32)
    bad_out = [torch.zeros(1, 4, 2, 32, dtype=torch.bfloat16),      # shape
               torch.zeros(1, 4, 2, 64, dtype=torch.float32),       # dtype
               torch.zeros(1, 4, 64, 2, dtype=torch.bfloat16).transpose(2, 3)]  # layout
    for out in bad_out:
        with pytest.raises(ValueError, match="out"):
            fa.attention_fwd(q, q, q, out=out, lse=lse)
    bad_lse = [torch.zeros(1, 4, 2, dtype=torch.float32),           # [B, Nq, Hq]
               torch.zeros(1, 2, 4, dtype=torch.bfloat16),          # dtype
               torch.zeros(1, 4, 2, dtype=torch.float32).transpose(1, 2)]  # layout
    for l in bad_lse:
        with pytest.raises(ValueError, match="lse"):
            fa.attention_fwd(q, q, q, out=torch.zeros_like(q), lse=l)
    # packed: LSE is [Hq, T]
    qp = torch.zeros(6, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 2, 6], dtype=torch.int32)
    with pytest.raises(ValueError, match="lse"):
        fa.attention_fwd(qp, qp, qp, cu_seqlens=cu, max_seqlen=4,
                         lse=torch.zeros(6, 2, dtype=torch.float32))
    # right buffers on the host: refused only for not being device tensors
    with pytest.raises(ValueError, match="device"):
        fa.attention_fwd(q, q, q, out=torch.zeros_like(q), lse=lse)


def test_attention_fwd_fp8_checks_shapes(fa):
    import torch
    q = torch.zeros(2, 4, 2, 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="B or d"):
        fa.attention_fwd_fp8(q, q[:1], q[:1])                       # batch differs
    k = torch.zeros(2, 4, 2, 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="B or d"):
        fa.attention_fwd_fp8(q, k, k)                               # d differs
    q64 = torch.zeros(2, 4, 2, 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="d=128"):
        fa.attention_fwd_fp8(q64, q64, q64)
    with pytest.raises(ValueError, match="device"):
        fa.attention_fwd_fp8(q, q, q)
    with pytest.raises(TypeError):
        fa.attention_fwd_fp8(q.float(), q, q)


CU_CASES = [
    ("valid", [0, 3, 3, 10], 7, 0),
    ("valid_empty_batch", [0], 7, 0),
    ("first_not_zero", [1, 3, 10], 7, -4),
    ("decreasing", [0, 5, 4, 10], 7, -4),
    ("longer_than_max", [0, 3, 11], 7, -4),
    ("exactly_max", [0, 7, 14], 7, 0),
]


@pytest.mark.parametrize("name,cu,mx,status", CU_CASES, ids=[c[0] for c in CU_CASES])
def test_check_cu_seqlens(fa, name, cu, mx, status):
    import numpy as np
    a = np.asarray(cu, dtype=np.int32)
    st = fa.fa_check_cu_seqlens(a.ctypes.data, len(cu) - 1, mx)
    assert st == status, (st, fa.fa_last_error())
    assert bool(fa.fa_last_error()) == (status != 0)


def test_check_cu_seqlens_null_and_negative(fa):
    assert fa.fa_check_cu_seqlens(None, 2, 8) == fa.FA_ERR_NULL
    assert fa.fa_check_cu_seqlens(None, 0, 8) == fa.FA_OK
    assert fa.fa_check_cu_seqlens(None, -1, 8) == fa.FA_ERR_SHAPE


def _call_noalloc(fa, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=8, Hkv=2, Nq=1, Nk=300, d=128, scale=0.1,
             causal=0, lens=None, splits=4, stream=None)
    a.update(kw)
    return fa.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                     a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                     a["lens"], a["splits"], a["stream"])


def test_noalloc_rejects_calls_beyond_its_scratch(fa):
    """The allocation-free entry point refuses, on the host, any call whose
    split scratch exceeds the fixed array; just below the limit it passes
    the host checks (and stops at the device check without a GPU)."""
    import torch
    lim = fa.FA_NOALLOC_SCRATCH_BYTES
    # B * Hq * Nq * splits rows of (d + 1) floats, the O part padded to 256 B
    big = dict(B=64, Hq=32, Hkv=8, Nq=1, splits=64)
    assert fa.fa_fwd_splitkv_workspace_bytes(64, 32, 1, 128, 64) > lim
    assert _call_noalloc(fa, **big) == fa.FA_ERR_ARG
    assert "scratch" in fa.fa_last_error()
    ok = dict(B=64, Hq=32, Hkv=8, Nq=1, splits=15)
    assert fa.fa_fwd_splitkv_workspace_bytes(64, 32, 1, 128, 15) <= lim
    if not torch.cuda.is_available():
        assert _call_noalloc(fa, **ok) == fa.FA_ERR_HIP


@pytest.mark.parametrize("kw,status", [(dict(q=0), -1), (dict(splits=0), -4), (dict(d=96), -3),
                                       (dict(Hq=6, Hkv=4), -2), (dict(Nq=9), -3),
                                       (dict(B=0), 0), (dict(Nq=0), 0)])
def test_noalloc_shares_the_host_checks(fa, kw, status):
    assert _call_noalloc(fa, **kw) == status, fa.fa_last_error()


def test_splitkv_num_splits(fa):
    """About three split workgroups per compute unit, each range >= 512 keys."""
    assert fa.fa_fwd_splitkv_num_splits(16, 8, 8192, 256) == 6     # 768 / 128
    assert fa.fa_fwd_splitkv_num_splits(1, 8, 8192, 256) == 16     # 96 capped by 8192 / 512
    assert fa.fa_fwd_splitkv_num_splits(2, 1, 1 << 20, 256) == 384  # 768 / 2
    assert fa.fa_fwd_splitkv_num_splits(1, 1, 1 << 30, 1024) == 1024
    assert fa.fa_fwd_splitkv_num_splits(64, 32, 8192, 256) == 1    # more units than slots
    assert fa.fa_fwd_splitkv_num_splits(4, 8, 300, 256) == 1       # fewer than 512 keys
    for bad in ((0, 8, 8192), (4, 0, 8192), (4, 8, 0)):
        assert fa.fa_fwd_splitkv_num_splits(*bad, 256) == fa.FA_ERR_SHAPE
