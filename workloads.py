"""Seeded synthetic inputs for the attention forward workloads.

This module draws Q, K, V (and, for packed batches, the sequence lengths)
from a seeded generator and rounds them to their storage type. It holds no
attention arithmetic; the oracle and the GPU path both consume what it
returns, and nothing else is shared between them.

Recipe (identical for every consumer):

* ``rng = numpy.random.default_rng(seed)``, seed ``1000 + workload id`` by
  default;
* packed workloads draw the lengths first:
  ``rng.integers(lo, hi, nseq, endpoint=True)``;
* then Q, K, V in that order, each ``rng.standard_normal(shape, float32) * sigma``
  in the token-major layout ([B, N, H, d], or [T, H, d] when packed);
* bf16 workloads round each float32 value to the nearest bf16, ties to even.

The five workloads are synthetic shapes; none stands for a dataset.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    dtype: str                 # "fp32" or "bf16" (storage and input type)
    batch: int                 # B, or the number of packed sequences
    hq: int
    hkv: int
    n: int                     # Nq = Nk for fixed length; unused when packed
    d: int
    causal: bool
    sigma_q: float = 1.0
    sigma_k: float = 1.0
    sigma_v: float = 1.0
    packed_len_range: Optional[tuple] = None   # (lo, hi) inclusive, packed only

    @property
    def packed(self) -> bool:
        return self.packed_len_range is not None

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    1: Workload(1, "fp32 single head, N=256, d=64, non-causal", "fp32",
                1, 1, 1, 256, 64, False),
    2: Workload(2, "bf16 16 heads, N=2048, d=64, non-causal", "bf16",
                1, 16, 16, 2048, 64, False),
    3: Workload(3, "bf16 causal 32 heads, N=4096, d=128", "bf16",
                1, 32, 32, 4096, 128, True),
    4: Workload(4, "bf16 causal GQA 32/8 heads, N=8192, d=128", "bf16",
                1, 32, 8, 8192, 128, True),
    5: Workload(5, "bf16 packed causal GQA 32/8, 16 sequences, L~U[128,16384], d=128, "
                   "Q~N(0,3^2)", "bf16",
                16, 32, 8, 0, 128, True, sigma_q=3.0, packed_len_range=(128, 16384)),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Inputs here are finite draws, so no NaN
    handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Q, K, V as float32 values exactly representable in the storage type,
    plus the bf16 bit patterns when the storage type is bf16."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    cu_seqlens: Optional[np.ndarray]      # int32 [nseq + 1] or None
    lens: Optional[np.ndarray]            # int64 [nseq] or None
    q_bits: Optional[np.ndarray] = None
    k_bits: Optional[np.ndarray] = None
    v_bits: Optional[np.ndarray] = None

    @property
    def max_seqlen(self) -> int:
        if self.lens is None:
            return self.q.shape[1]
        return int(self.lens.max()) if len(self.lens) else 0


def _draw(rng, shape, sigma, dtype):
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)
    if dtype == "bf16":
        bits = round_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    return x, None


def draw(batch: int, hq: int, hkv: int, nq: int, nk: int, d: int, dtype: str,
         seed: int, sigma=(1.0, 1.0, 1.0), lens=None) -> Inputs:
    """Draw one input set.

    Fixed length when ``lens`` is None: q [batch, nq, hq, d], k and v
    [batch, nk, hkv, d]. Packed when ``lens`` is a sequence of lengths (or the
    tuple ``("uniform", lo, hi)``, drawn first from the same generator):
    q [T, hq, d], k and v [T, hkv, d], T = sum(lens).
    """
    rng = np.random.default_rng(seed)
    cu = None
    if lens is not None:
        if isinstance(lens, tuple) and lens and lens[0] == "uniform":
            lens = rng.integers(lens[1], lens[2], batch, endpoint=True)
        lens = np.asarray(lens, dtype=np.int64)
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens).astype(np.int32)
        total = int(cu[-1])
        qs, ks = (total, hq, d), (total, hkv, d)
    else:
        qs, ks = (batch, nq, hq, d), (batch, nk, hkv, d)
    q, qb = _draw(rng, qs, sigma[0], dtype)
    k, kb = _draw(rng, ks, sigma[1], dtype)
    v, vb = _draw(rng, ks, sigma[2], dtype)
    return Inputs(q, k, v, dtype, cu, lens, qb, kb, vb)


def draw_workload(wid: int, seed: Optional[int] = None) -> Inputs:
    w = WORKLOADS[wid]
    seed = 1000 + wid if seed is None else seed
    sig = (w.sigma_q, w.sigma_k, w.sigma_v)
    if w.packed:
        lo, hi = w.packed_len_range
        return draw(w.batch, w.hq, w.hkv, 0, 0, w.d, w.dtype, seed, sig,
                    lens=("uniform", lo, hi))
    return draw(w.batch, w.hq, w.hkv, w.n, w.n, w.d, w.dtype, seed, sig)


@dataclasses.dataclass
class Bias:
    """An additive bias as bf16 bit patterns and the float32 values they
    hold, indexed [entry or 1, head or 1, row, column]; the columns are
    padded with zeros to a multiple of 4 (the row stride the bf16 kernels
    read in runs of 4)."""
    values: np.ndarray
    bits: np.ndarray


def draw_bias(entries: int, heads: int, rows: int, cols: int, seed: int, sigma: float = 1.0,
              key_lens=None, dead_rows=()) -> Bias:
    """Draw a bias [entries, heads, rows, round_up(cols, 4)].

    Entries are ``rng.standard_normal(float32) * sigma`` from
    ``numpy.random.default_rng(seed)``, rounded to bf16. ``key_lens`` (one
    length per entry) sets columns at or past that length to -inf, a key
    padding pattern; ``dead_rows`` lists (entry, head, row) triples whose
    whole row is -inf. Padding columns past ``cols`` hold 0.
    """
    rng = np.random.default_rng(seed)
    cpad = (cols + 3) // 4 * 4
    x = np.zeros((entries, heads, rows, cpad), dtype=np.float32)
    x[..., :cols] = rng.standard_normal((entries, heads, rows, cols), dtype=np.float32) * np.float32(
        sigma)
    if key_lens is not None:
        for e, n in enumerate(key_lens):
            x[e, :, :, int(n):cols] = -np.inf
    for e, h, r in dead_rows:
        x[e, h, r, :cols] = -np.inf
    bits = round_to_bf16_bits_inf(x)
    return Bias(bf16_bits_to_f32(bits), bits)


def round_to_bf16_bits_inf(x: np.ndarray) -> np.ndarray:
    """``round_to_bf16_bits`` that also keeps infinities (their bit patterns
    are exact in bf16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = round_to_bf16_bits(np.where(np.isfinite(x), x, 0.0).astype(np.float32))
    u = x.view(np.uint32)
    inf = np.isinf(x)
    bits[inf] = (u[inf] >> np.uint32(16)).astype(np.uint16)
    return bits


@dataclasses.dataclass
class Fp8Inputs:
    """FP8 (OCP e4m3) inputs: the codes of Q, K, V (uint8, fixed-length
    layouts) and one dequantization factor per tensor."""
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    q_descale: float
    k_descale: float
    v_descale: float


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values (finite, |x| <= 448) to e4m3 codes with torch's
    float8_e4m3fn cast (round to nearest, ties to even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def draw_fp8(batch: int, hq: int, hkv: int, nq: int, nk: int, d: int, seed: int,
             sigma=(1.0, 1.0, 1.0), mode: str = "normal") -> Fp8Inputs:
    """Draw FP8 inputs q [batch, nq, hq, d], k and v [batch, nk, hkv, d].

    ``mode="normal"``: ``rng.standard_normal(float32) * sigma`` for Q, K, V in
    that order, each quantized with the per-tensor factor
    descale = max|x| / 448 (the largest value maps to the largest e4m3
    normal): codes = e4m3(x / descale).
    ``mode="signs"``: Q and K rows hold 4 entries of +-1 at random positions
    and zeros elsewhere (descale 1), so every score q.k is an integer in
    [-4, 4]; V as in "normal".
    """
    rng = np.random.default_rng(seed)
    qs, ks = (batch, nq, hq, d), (batch, nk, hkv, d)

    def quant(x):
        amax = float(np.abs(x).max()) if x.size else 0.0
        ds = amax / 448.0 if amax > 0 else 1.0
        return to_e4m3_bits(x / np.float32(ds)), ds

    def signs(shape):
        x = np.zeros(shape, dtype=np.float32)
        flat = x.reshape(-1, shape[-1])
        cols = np.argsort(rng.random(flat.shape), axis=1)[:, :4]
        vals = np.where(rng.random((flat.shape[0], 4)) < 0.5, -1.0, 1.0).astype(np.float32)
        np.put_along_axis(flat, cols, vals, axis=1)
        return to_e4m3_bits(x), 1.0

    if mode == "normal":
        (qb, qd), (kb, kd) = (quant(rng.standard_normal(s, dtype=np.float32) * np.float32(sg))
                              for s, sg in ((qs, sigma[0]), (ks, sigma[1])))
    elif mode == "signs":
        (qb, qd), (kb, kd) = signs(qs), signs(ks)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    vb, vd = quant(rng.standard_normal(ks, dtype=np.float32) * np.float32(sigma[2]))
    return Fp8Inputs(qb, kb, vb, qd, kd, vd)
