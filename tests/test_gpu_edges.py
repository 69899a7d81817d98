"""GPU edge cases and invariants, each pinned by a fact other than the
oracle (closed forms, exact special cases, structural identities), plus
determinism and the empty-input contract."""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_O, assert_parity, max_err, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fa():
    import exact_io_aware_63_amd as fa
    return fa


def _bf16_tensor(x, device="cuda"):
    import torch
    return torch.from_numpy(W.round_to_bf16_bits(np.asarray(x, np.float32)).view(np.int16)) \
        .view(torch.bfloat16).to(device)


@pytest.mark.parametrize("d", [64, 128])
def test_single_key_returns_v_exactly(d):
    """One key: p = 2^0 = 1 and l = 1, so O equals that key's value row
    bit-exactly in bf16, and LSE = scale * q.k."""
    say(f"[case] single key d={d}")
    inp = W.draw(2, 4, 2, 150, 1, d, "bf16", seed=21)
    for causal in (False, True):
        o, lse = run_gpu(inp, causal, 0.3)
        want = np.repeat(inp.v[:, :, :, None, :], 2, axis=3).reshape(2, 1, 4, d)
        assert np.array_equal(o, np.broadcast_to(want, o.shape)), "O must equal v"
        kk = np.repeat(inp.k, 2, axis=2)
        s = 0.3 * np.einsum("bihd,bjhd->bhij", inp.q.astype(np.float64), kk.astype(np.float64))[..., 0]
        assert max_err(lse, s) <= 1e-3


def test_identical_keys_and_zero_scale_give_mean():
    """All scores equal (identical keys, or scale 0): O = mean(V),
    LSE = s + ln(n)."""
    say("[case] identical keys / scale 0")
    n, d = 300, 128
    inp = W.draw(1, 2, 1, 200, n, d, "bf16", seed=22)
    inp.k[:] = inp.k[:, :1]
    inp.k_bits[:] = inp.k_bits[:, :1]
    mean = inp.v.astype(np.float64).mean(axis=1)            # [1, 1, d]
    o, lse = run_gpu(inp, False, 1 / math.sqrt(d))
    assert max_err(o, np.broadcast_to(mean[:, None], o.shape)) <= TOL_O["bf16"]
    s = (inp.q.astype(np.float64) @ inp.k[0, 0, 0].astype(np.float64)) / math.sqrt(d)
    assert max_err(lse, np.moveaxis(s, 1, 2) + math.log(n)) <= 1e-3
    o0, lse0 = run_gpu(W.draw(1, 2, 1, 200, n, d, "bf16", seed=23), False, 0.0)
    inp0 = W.draw(1, 2, 1, 200, n, d, "bf16", seed=23)
    mean0 = inp0.v.astype(np.float64).mean(axis=1)
    assert max_err(o0, np.broadcast_to(mean0[:, None], o0.shape)) <= TOL_O["bf16"]
    assert max_err(lse0, np.full(lse0.shape, math.log(n))) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_causal_zero_scale_prefix_means(dtype):
    """scale 0 with the causal mask: row i is the mean of V[0..i]."""
    say(f"[case] causal prefix means {dtype}")
    n, d = 390, 64
    inp = W.draw(1, 2, 2, n, n, d, dtype, seed=24)
    o, lse = run_gpu(inp, True, 0.0)
    v = inp.v.astype(np.float64)
    pref = np.cumsum(v, axis=1) / np.arange(1, n + 1)[None, :, None, None]
    tol = TOL_O[dtype]
    assert max_err(o, pref) <= tol
    assert max_err(lse, np.broadcast_to(np.log(np.arange(1, n + 1)), lse.shape)) <= 1e-4


def _scale_with_power_of_two_factor(min_factor):
    """A float32 scale whose base-2 factor c = fp32(fp64(scale) * log2 e) is a
    power of two >= min_factor. With such a c every product c * s is exact
    in float32, so the weight of a row's maximum is exactly 2^0 = 1."""
    k = math.ceil(math.log2(min_factor))
    target = np.float32(2.0 ** k)
    s0 = np.float32(2.0 ** k / math.log2(math.e))
    for cand in (s0, np.nextafter(s0, np.float32(np.inf)), np.nextafter(s0, np.float32(0))):
        c = np.float32(np.float64(cand) * 1.4426950408889634)
        if c == target:
            return float(cand)
    raise AssertionError("no float32 scale with a power-of-two base-2 factor")


def test_hard_max_limit_exact():
    """When the top score beats the runner-up by >= 200 in base-2 units, all
    other weights underflow to 0 and O is v_argmax exactly (bf16)."""
    say("[case] hard-max limit")
    n, d = 256, 64
    inp = W.draw(1, 1, 1, n, n, d, "bf16", seed=25)
    s = inp.q[0, :, 0].astype(np.float64) @ inp.k[0, :, 0].astype(np.float64).T
    srt = np.sort(s, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    keep = gap > 0.05                                        # clear winners only
    assert keep.sum() > 100
    scale = _scale_with_power_of_two_factor(200.0 / gap[keep].min())
    o, _ = run_gpu(inp, False, scale)
    arg = s.argmax(axis=1)
    got = o[0, keep, 0]
    want = inp.v[0, arg[keep], 0].astype(np.float64)
    assert np.array_equal(got, want)


def test_shift_invariance_large_offset():
    """Adding c to every score of a row (q gets 800 in a column where every
    key has 1, so c = 800 * scale = 100) leaves O unchanged and shifts LSE by
    exactly 100; 2^(100*log2 e) overflows float32 without the max shift."""
    say("[case] shift invariance")
    n, d = 333, 64
    inp = W.draw(1, 4, 2, n, n, d, "bf16", seed=26)
    for arr, bits in ((inp.q, inp.q_bits), (inp.k, inp.k_bits), (inp.v, inp.v_bits)):
        arr[..., -1] = 0.0
        bits[..., -1] = 0
    o, lse = run_gpu(inp, True, 0.125)
    inp.q[..., -1] = 800.0
    inp.q_bits[..., -1] = W.round_to_bf16_bits(np.float32([800.0]))[0]
    inp.k[..., -1] = 1.0
    inp.k_bits[..., -1] = W.round_to_bf16_bits(np.float32([1.0]))[0]
    o2, lse2 = run_gpu(inp, True, 0.125)
    assert max_err(o2, o) <= TOL_O["bf16"]
    assert max_err(lse2 - 100.0, lse) <= 1e-3
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, 0.125, True)
    assert_parity(o2, lse2, o_ref, lse_ref, "bf16", "shifted scores")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_heads_bitwise(causal):
    """GQA reads K/V head h // (Hq/Hkv): identical to MHA on repeated heads,
    bit for bit (the same arithmetic on the same values)."""
    import torch
    say(f"[case] GQA == repeated heads causal={causal}")
    inp = W.draw(2, 8, 2, 300, 300, 128, "bf16", seed=27)
    q, k, v, _ = to_device(inp)
    fa = _fa()
    o, lse = fa.attention_fwd(q, k, v, causal=causal)
    o2, lse2 = fa.attention_fwd(q, k.repeat_interleave(4, dim=2).contiguous(),
                                v.repeat_interleave(4, dim=2).contiguous(), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_packed_equals_separate_calls_and_isolation(causal):
    """Packed sequences give the same bits as one call per sequence, and a
    change to one sequence's K/V leaves every other sequence untouched."""
    import torch
    say(f"[case] packed == separate causal={causal}")
    lens = [130, 1, 0, 257, 64, 500]
    inp = W.draw(len(lens), 4, 2, 0, 0, 128, "bf16", seed=28, lens=lens)
    q, k, v, cu = to_device(inp)
    fa = _fa()
    o, lse = fa.attention_fwd(q, k, v, causal=causal, cu_seqlens=cu, max_seqlen=max(lens))
    c = inp.cu_seqlens
    for s, L in enumerate(lens):
        if L == 0:
            continue
        sl = slice(int(c[s]), int(c[s + 1]))
        os_, ls_ = fa.attention_fwd(q[sl][None].contiguous(), k[sl][None].contiguous(),
                                    v[sl][None].contiguous(), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o[sl], os_[0]), f"sequence {s} O"
        assert torch.equal(lse[:, sl], ls_[0]), f"sequence {s} LSE"
    k2, v2 = k.clone(), v.clone()
    sl = slice(int(c[3]), int(c[4]))
    k2[sl] = k2[sl] * 2 + 1
    v2[sl] = -v2[sl]
    o2, lse2 = fa.attention_fwd(q, k2, v2, causal=causal, cu_seqlens=cu, max_seqlen=max(lens))
    torch.cuda.synchronize()
    mask = torch.ones(q.shape[0], dtype=torch.bool, device=q.device)
    mask[sl] = False
    assert torch.equal(o2[mask], o[mask]) and torch.equal(lse2[:, mask], lse[:, mask])
    assert not torch.equal(o2[sl], o[sl])


def test_empty_keys_give_zero_and_neg_inf():
    import torch
    say("[case] Nk = 0 and empty packed sequences")
    fa = _fa()
    # non-causal bf16 takes the key-halves schedule at this size: both halves
    # are empty and the merge must still give O = 0, LSE = -inf
    for dtype in (torch.bfloat16, torch.float32):
        for causal in (1, 0):
            q = torch.randn(2, 70, 4, 64, device="cuda").to(dtype)
            o = torch.full_like(q, 7.0)
            lse = torch.zeros(2, 4, 70, device="cuda")
            # Nk = 0 still needs valid (non-NULL) pointers: pass q's storage.
            st = (fa.fa_fwd if dtype == torch.bfloat16 else fa.fa_fwd_fp32)(
                q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                2, 4, 2, 70, 0, 64, 0.125, causal, None, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert st == 0, fa.fa_last_error()
            assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_noop_calls_leave_outputs_untouched():
    import torch
    say("[case] no-op calls")
    fa = _fa()
    q = torch.randn(1, 8, 2, 64, device="cuda").to(torch.bfloat16)
    o = torch.full_like(q, 3.0)
    lse = torch.full((1, 2, 8), 5.0, device="cuda")
    for B, Nq in ((0, 8), (1, 0)):
        st = fa.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, 2, 2, Nq, 8, 64, 0.125, 0, None, None)
        assert st == 0
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 5.0).all())


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_deterministic_bitwise(wid):
    """No atomics and a fixed reduction order: two identical calls at the
    full workload size agree bit for bit (a mismatch would flag a race).
    Workload 2 takes the key-halves schedule, whose two wave pairs hand
    their partial state over through LDS."""
    import torch
    say(f"[case] determinism workload {wid}")
    w = W.WORKLOADS[wid]
    inp = W.draw_workload(wid)
    q, k, v, _ = to_device(inp)
    fa = _fa()
    o1, l1 = fa.attention_fwd(q, k, v, causal=w.causal, scale=w.scale)
    o2, l2 = fa.attention_fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_side_stream_matches_default_stream():
    import torch
    say("[case] side stream")
    inp = W.draw(1, 4, 2, 300, 300, 128, "bf16", seed=29)
    q, k, v, _ = to_device(inp)
    fa = _fa()
    o1, l1 = fa.attention_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = fa.attention_fwd(q, k, v, causal=True)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_negative_scale():
    say("[case] negative scale")
    inp = W.draw(1, 2, 2, 200, 200, 64, "bf16", seed=30)
    o, lse = run_gpu(inp, True, -0.2)
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, -0.2, True)
    assert_parity(o, lse, o_ref, lse_ref, "bf16", "negative scale")


def test_peaky_rows_parity():
    """Q ~ N(0, 3^2) raises the running max often (many rescales)."""
    say("[case] peaky rows")
    inp = W.draw(1, 4, 2, 700, 700, 128, "bf16", seed=31, sigma=(3.0, 1.0, 1.0))
    o, lse = run_gpu(inp, True, 1 / math.sqrt(128))
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, 1 / math.sqrt(128), True)
    assert_parity(o, lse, o_ref, lse_ref, "bf16", "peaky rows")


def _ramp_inputs(n, d, hq, hkv, seed, per_tile):
    """Seeded bf16 inputs plus a key-position ramp in the last d column: q
    holds A there for every row and key j holds floor(j / 32), so each run of
    32 keys scores per_tile more (base-2 units) than the run before it."""
    inp = W.draw(1, hq, hkv, n, n, d, "bf16", seed=seed)
    scale = 1.0 / math.sqrt(d)
    a = float(W.bf16_bits_to_f32(W.round_to_bf16_bits(
        np.float32([per_tile / (scale * 1.4426950408889634)])))[0])
    ramp = np.floor(np.arange(n) / 32.0).astype(np.float32)
    inp.q[..., -1] = a
    inp.q_bits[..., -1] = W.round_to_bf16_bits(np.float32([a]))[0]
    inp.k[0, :, :, -1] = ramp[:, None]
    inp.k_bits[0, :, :, -1] = W.round_to_bf16_bits(ramp)[:, None]
    return inp, scale


@pytest.mark.parametrize("d,causal", [(128, True), (128, False), (64, True)])
def test_raising_reference_every_tile(d, causal):
    """Scores that climb by about 20 (base 2) every 32 keys: each later tile
    exceeds the row's reference by more than 2^16, so the reference is raised
    and the accumulators rescaled many times per row."""
    say(f"[case] rising scores d={d} causal={causal}")
    inp, scale = _ramp_inputs(700, d, 4, 2, 41, 20.0)
    o, lse = run_gpu(inp, causal, scale)
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, "bf16", "rising scores")


def test_falling_scores_underflow_later_tiles():
    """Scores that drop by about 20 (base 2) every 32 keys: the first tile
    sets the reference and later weights underflow, as in the definition."""
    say("[case] falling scores")
    inp, scale = _ramp_inputs(700, 128, 4, 2, 42, -20.0)
    o, lse = run_gpu(inp, True, scale)
    o_ref, lse_ref = oracle.attention_ref(inp.q, inp.k, inp.v, scale, True)
    assert_parity(o, lse, o_ref, lse_ref, "bf16", "falling scores")


def test_check_inputs_env_rejects_bad_offsets(monkeypatch):
    """With FA_CHECK_INPUTS set, packed calls copy cu_seqlens to the host and
    refuse a bad array before any launch. The bad arrays used here stay
    inside the buffers (a sequence longer than max_seqlen, a first offset
    that is not 0), so a launch would not read out of bounds either."""
    import torch
    fa = _fa()
    say("[case] FA_CHECK_INPUTS on packed offsets")
    T, hq, hkv, d = 6, 2, 1, 64
    q = torch.zeros(T, hq, d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(T, hkv, d, dtype=torch.bfloat16, device="cuda")
    good = torch.tensor([0, 2, 6], dtype=torch.int32, device="cuda")
    long_seq = torch.tensor([0, 6], dtype=torch.int32, device="cuda")
    not_zero = torch.tensor([2, 6], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("FA_CHECK_INPUTS", "1")
    fa.attention_fwd(q, k, k, causal=True, cu_seqlens=good, max_seqlen=4)
    for cu, mx, what in ((long_seq, 4, "max_seqlen"), (not_zero, 4, "must be 0")):
        with pytest.raises(fa.FaError) as ei:
            fa.attention_fwd(q, k, k, causal=True, cu_seqlens=cu, max_seqlen=mx)
        assert ei.value.status == fa.FA_ERR_ARG and what in ei.value.detail
    torch.cuda.synchronize()
