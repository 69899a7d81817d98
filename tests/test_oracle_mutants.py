"""Plant plausible mistakes in the oracle and check the pins catch each one.

Every mutant below replaces one step of ``oracle.attention`` (on the CPU,
through monkeypatch) with a wrong variant: a dropped term, a wrong sign or
index, a swapped operand. The pin suite must fail for each of them; a mutant
that every pin lets through would mean the pins do not constrain that step.
"""
import numpy as np
import pytest

import oracle.attention as A
from oracle_pins import ALL_PINS

_orig_head = A.attention_head
_orig_softmax = A.softmax_rows
_orig_visible = A.visible_mask


def _softmax_no_max(s):
    e = np.exp(s)
    l = e.sum(axis=1)
    with np.errstate(invalid="ignore"):
        return e / l[:, None], np.zeros(len(s)), l


def _softmax_wrong_axis(s):
    p, m, l = _orig_softmax(s)
    e = np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None])
    col = e.sum(axis=0)
    return e / np.where(col > 0, col, 1.0)[None, :], m, l


def _softmax_lse_no_l(s):
    p, m, l = _orig_softmax(s)
    return p, m, np.ones_like(l)


def _visible_strict(rows, lk, causal, window=None):
    j = np.arange(lk)[None, :]
    i = np.asarray(rows)[:, None]
    return (j < i) if causal else np.broadcast_to(j >= 0, (len(rows), lk))


def _visible_reversed(rows, lk, causal, window=None):
    j = np.arange(lk)[None, :]
    i = np.asarray(rows)[:, None]
    return (j >= i) if causal else np.broadcast_to(j >= 0, (len(rows), lk))


def _visible_ignores_causal(rows, lk, causal, window=None):
    return np.broadcast_to(np.arange(lk)[None, :] >= 0, (len(rows), lk))


def _window_left_off_by_one(rows, lk, causal, window=None):
    m = _orig_visible(rows, lk, causal, None)
    if window is not None:
        j = np.arange(lk)[None, :]
        i = np.asarray(rows)[:, None]
        if window[0] >= 0:
            m = m & (j > i - window[0])
        if window[1] >= 0:
            m = m & (j <= i + window[1])
    return m


def _window_right_off_by_one(rows, lk, causal, window=None):
    m = _orig_visible(rows, lk, causal, None)
    if window is not None:
        j = np.arange(lk)[None, :]
        i = np.asarray(rows)[:, None]
        if window[0] >= 0:
            m = m & (j >= i - window[0])
        if window[1] >= 0:
            m = m & (j < i + window[1])
    return m


_orig_bias_of = A.bias_of


def _head_with_bias(fn):
    """attention_head with the bias block replaced by fn(bias, q)."""
    def f(q, k, v, scale, causal, rows=None, window=None, bias=None):
        return _orig_head(q, k, v, scale, causal, rows, window,
                          None if bias is None else fn(np.asarray(bias, dtype=np.float64), scale))
    return f


def _head_bias_replaces_mask(q, k, v, scale, causal, rows=None, window=None, bias=None):
    if bias is None:
        return _orig_head(q, k, v, scale, causal, rows, window, bias)
    return _orig_head(q, k, v, scale, False, rows, None, bias)


def _bias_of_swapped(bias, s, h):
    if bias is None:
        return None
    b = np.asarray(bias)
    return b[h if b.shape[0] > 1 else 0, s if b.shape[1] > 1 else 0]


_orig_e4m3 = A.e4m3_value


def _e4m3_bias8(bits):
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e, m = (b >> 3) & 0xF, (b & 7).astype(np.float64)
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 8), np.ldexp(m / 8.0, -7))
    return np.where(b & 0x80, -1.0, 1.0) * mag


def _e4m3_no_subnormals(bits):
    v = _orig_e4m3(bits)
    e = (np.asarray(bits, dtype=np.uint8) >> 3) & 0xF
    return np.where(e == 0, 0.0, v)


MUTANTS = {
    "e4m3_exponent_bias_8": ("e4m3_value", _e4m3_bias8),
    "e4m3_subnormals_flushed": ("e4m3_value", _e4m3_no_subnormals),
    "e4m3_sign_dropped": ("e4m3_value", lambda bits: np.abs(_orig_e4m3(bits))),
    "bias_ignored": ("attention_head", _head_with_bias(lambda b, scale: np.zeros_like(b))),
    "bias_transposed": ("attention_head", _head_with_bias(lambda b, scale: b.T)),
    "bias_negated": ("attention_head", _head_with_bias(lambda b, scale: -b)),
    "bias_scaled": ("attention_head", _head_with_bias(lambda b, scale: b * scale)),
    "bias_replaces_mask": ("attention_head", _head_bias_replaces_mask),
    "bias_entry_head_swapped": ("bias_of", _bias_of_swapped),
    "window_ignored": ("visible_mask", lambda rows, lk, causal, window=None:
                       _orig_visible(rows, lk, causal, None)),
    "window_left_off_by_one": ("visible_mask", _window_left_off_by_one),
    "window_right_off_by_one": ("visible_mask", _window_right_off_by_one),
    "gqa_modulo_grouping": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "causal_strict_lower": ("visible_mask", _visible_strict),
    "causal_reversed": ("visible_mask", _visible_reversed),
    "causal_ignored": ("visible_mask", _visible_ignores_causal),
    "scale_dropped": ("scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("scores", lambda q, k, scale: (q @ k.T) * scale * scale),
    "softmax_no_max_shift": ("softmax_rows", _softmax_no_max),
    "softmax_wrong_axis": ("softmax_rows", _softmax_wrong_axis),
    "lse_without_denominator": ("softmax_rows", _softmax_lse_no_l),
    "values_are_keys": ("attention_head",
                        lambda q, k, v, scale, causal, rows=None, window=None, bias=None:
                        _orig_head(q, k, k, scale, causal, rows, window, bias)),
    "lse_log2": ("attention_head",
                 lambda q, k, v, scale, causal, rows=None, window=None, bias=None:
                 (lambda o, l: (o, l / np.log(2.0)))(*_orig_head(q, k, v, scale, causal, rows,
                                                                 window, bias))),
    "last_key_dropped": ("attention_head",
                         lambda q, k, v, scale, causal, rows=None, window=None, bias=None:
                         _orig_head(q, k[:-1], v[:-1], scale, causal, rows, window, bias)),
    "first_row_skipped": ("attention_head",
                          lambda q, k, v, scale, causal, rows=None, window=None, bias=None:
                          (lambda o, l: (np.concatenate([np.zeros_like(o[:1]), o[1:]]), l))(
                              *_orig_head(q, k, v, scale, causal, rows, window, bias))),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"
