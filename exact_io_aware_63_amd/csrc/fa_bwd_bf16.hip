// Exact attention backward by recomputation, bf16 in / bf16 out, float32
// accumulation, for gfx950 (CDNA4) matrix cores.
//
// The forward pass keeps only O and the per-row log-sum-exp; the backward
// pass recomputes the probabilities block by block from Q, K and that LSE
// instead of reading a stored P ("Understanding FlashAttention Pt 1:
// Personal Notes", contents, section 3.6: recompute instead of save;
// semiaifoundry "attention-io-tiling", section Specifications and
// interfaces: the retained statistics and permitted recomputation serve
// the backward execution). With S = scale Q K^T and P = exp(S - LSE) on the
// visible pairs, the gradients of O = P V for an upstream gradient dO are
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = dO_i . O_i,
//   dQ = scale dS K,   dK = scale dS^T Q
// (D_i equals sum_j P_ij dP_ij because O_i = sum_j P_ij V_j).
//
// Two launches in order on one stream: bwd_dot_kernel, then
// bwd_main_kernel, whose workgroups run one of two bodies:
//   * bwd_dot_kernel: D = rowsum(dO * O) in float32, one value per (query
//     row, q-head), laid out like the LSE;
//   * dK/dV body: a workgroup owns 128 keys of one (batch or sequence,
//     K/V head); wave w holds keys 32w .. 32w+31 of K and V in registers and
//     accumulates dK^T and dV^T in registers while 64-row blocks of Q and dO
//     (and their LSE and D) stream through LDS, for every query head of the
//     K/V head's group, so grouped-query gradients are summed without
//     atomics. Per 32 x 32 block: S = Q K^T and dP = dO V^T (lane = key,
//     registers = queries), then P and dS, packed to bf16 as the B operands
//     of dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read from the
//     row-major LDS tiles through ds_read_b64_tr_b16;
//   * dQ body: a workgroup owns 128 query rows of one (batch or
//     sequence, q-head); wave w holds rows 32w .. 32w+31 of Q and dO in
//     registers (lane = query, one LSE and one D value per lane) and
//     accumulates dQ^T while 64-key blocks of K and V stream through LDS:
//     S^T = K Q^T and dP^T = V dO^T, then P^T and dS^T, and
//     dQ^T += K^T dS^T with K^T read through transposing LDS reads.
// The causal mask is top-left (key j visible to query i iff j <= i, indices
// local to the batch entry or sequence); blocks entirely above the diagonal
// are skipped per wave, and partial blocks are masked element by element.
// With an additive bias B (the BIAS variants) the recomputed probabilities
// are P = exp(scale Q K^T + B - LSE), the LSE being the forward's with the
// same bias; each lane loads the bias values of its own score registers
// before the score MFMAs of a block. A row that saw no finite score in the
// forward (LSE = -inf) gets P = 0 on every pair.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <type_traits>

#include "fa_bf16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdRows = 128;  // keys (dK/dV kernel) or query rows (dQ kernel) per workgroup

// Output register r of a 32x32 MFMA block sits at row 8(r/4) + 4*h2 + (r%4)
// and column lane % 32, h2 = lane / 32.
__device__ __forceinline__ constexpr int mrow(int r, int h2) { return 8 * (r >> 2) + 4 * h2 + (r & 3); }

// Transposed A operand (32 rows of the tile's d columns, 16 of its rows) of
// a 64-row LDS tile, e.g. dO^T, Q^T or K^T: two transposing reads give tile
// rows 16g + 8r + 4*tr_h + (0..3), r = 0, 1, at d column 32t + 16*tr_dgrp +
// tr_i; lane tr_i of each 16-lane group supplies the address of 4
// consecutive d values of tile row 16g + 8r + 4*tr_h + tr_i/4. The row order
// matches the MFMA output registers 8g .. 8g+7 (mrow) of a score block,
// which become the B operand.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int row0, int t, int g,
                                             int lane) {
  using T = Tile<D>;
  const int tr_i = lane & 15;
  const int tr_dgrp = (lane >> 4) & 1;
  const int tr_h = lane >> 5;
  s16x4 half[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = row0 + 16 * g + 8 * r + 4 * tr_h + (tr_i >> 2);
    const int unit = (4 * t + 2 * tr_dgrp + ((tr_i & 3) >> 1)) ^ swz<T::kUnits>(row);
    const int off = row * T::kRowBytes + unit * 16 + (tr_i & 1) * 8;
    half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + off));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row-major A operand (32 tile rows from row0, 16 d values of chunk cc) of a
// 64-row LDS tile: lane reads row row0 + lane%32, d = 16cc + 8*h2 .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const unsigned char* tile, int row0, int cc, int lane) {
  using T = Tile<D>;
  const int row = row0 + (lane & 31);
  const int unit = (2 * cc + (lane >> 5)) ^ swz<T::kUnits>(row);
  return *reinterpret_cast<const bf16x8*>(tile + row * T::kRowBytes + unit * 16);
}

// B operand pair of registers 8g .. 8g+7 of a float32 MFMA output block,
// rounded to bf16 (nearest even).
__device__ __forceinline__ bf16x8 pack_chunk(const f32x16& x, int g) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(x[8 * g + i]);
  return r;
}

// Component i (a compile-time constant after unrolling) of a float4.
__device__ __forceinline__ float f4_at(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Key `key` visible to query `q` (sequence-local): inside both sequences,
// under the causal mask, and inside the sliding window when WIN.
template <bool CAUSAL, bool WIN>
__device__ __forceinline__ bool visible(const BwdParams& p, int q, int key, int Lq, int Lk) {
  bool v = q < Lq && key < Lk && (!CAUSAL || key <= q);
  if constexpr (WIN)
    v = v && (p.win_left < 0 || key >= q - p.win_left) && (p.win_right < 0 || key <= q + p.win_right);
  return v;
}

// Index of the LSE / D value of token `tok` (sequence-local row i) of q-head
// h: fixed length [B, Hq, Nq], packed [Hq, T].
struct RowIndex {
  long base;  // index of row 0 of this (batch or sequence, head)
  __device__ __forceinline__ long at(int i) const { return base + i; }
};

// Sequence bounds of batch entry or sequence b.
struct SeqBounds {
  long q_tok0, k_tok0;  // first token of the sequence in Q/O/dO and in K/V
  int Lq, Lk;
  long total;           // packed: total tokens (LSE row stride), else Nq
};
__device__ __forceinline__ SeqBounds seq_bounds(const BwdParams& p, int b) {
  SeqBounds s;
  if (p.cu_seqlens != nullptr) {
    const int s0 = p.cu_seqlens[b];
    const int s1 = p.cu_seqlens[b + 1];
    s.Lq = s.Lk = s1 - s0;
    s.q_tok0 = s.k_tok0 = s0;
    s.total = p.cu_seqlens[p.batch];
  } else {
    s.Lq = p.nq;
    s.Lk = p.nk;
    s.q_tok0 = static_cast<long>(b) * p.nq;
    s.k_tok0 = static_cast<long>(b) * p.nk;
    s.total = p.nq;
  }
  return s;
}
__device__ __forceinline__ RowIndex row_index(const BwdParams& p, const SeqBounds& s, int b, int h) {
  RowIndex r;
  r.base = p.cu_seqlens != nullptr ? static_cast<long>(h) * s.total + s.q_tok0
                                   : (static_cast<long>(b) * p.hq + h) * p.nq;
  return r;
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O)
// ---------------------------------------------------------------------------

// One (token, q-head) row per D/8 lanes: each lane multiplies 8 bf16 pairs,
// the row's lanes then add their partial sums. Rows are enumerated token by
// token (tok * Hq + h); tokens of a fixed-length batch are b * Nq + i. The
// grid covers B * Nq * Hq rows, a bound of the packed token count, which is
// read from the device here.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dot_kernel(BwdParams p) {
  constexpr int kLanes = D / 8;
  const long n_rows = (p.cu_seqlens != nullptr ? static_cast<long>(p.cu_seqlens[p.batch])
                                               : static_cast<long>(p.batch) * p.nq) * p.hq;
  const long row = (static_cast<long>(blockIdx.x) * kThreads + threadIdx.x) / kLanes;
  const int part = threadIdx.x % kLanes;
  float acc = 0.f;
  if (row < n_rows) {
    const long off = row * D + part * 8;  // Q/O/dO rows are tok * Hq + h, each D wide
    const u32x4 a = ld16(static_cast<const u16*>(p.o) + off);
    const u32x4 c = ld16(static_cast<const u16*>(p.dout) + off);
    const bf16x8 ao = as_bf16x8(a), ad = as_bf16x8(c);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      acc = __builtin_fmaf(static_cast<float>(ao[e]), static_cast<float>(ad[e]), acc);
  }
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
  if (row < n_rows && part == 0) {
    const long tok = row / p.hq;
    const int h = static_cast<int>(row % p.hq);
    long idx;
    if (p.cu_seqlens != nullptr) {
      idx = static_cast<long>(h) * p.cu_seqlens[p.batch] + tok;
    } else {
      const long b = tok / p.nq;
      idx = (b * p.hq + h) * p.nq + (tok % p.nq);
    }
    p.dsum[idx] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

// Score MFMAs for the interleaved plan below: as mfma_qk_first/acc, with
// two wait states first, because vector instructions now sit right before
// them and the compiler does not see the asm as a matrix instruction (a
// vector write of an operand register needs two wait states before an MFMA
// reads it).
__device__ __forceinline__ f32x16 mfma_qk_first_w(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
__device__ __forceinline__ void mfma_qk_acc_w(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}

// Exponent offset of a row: -LSE in base 2, or -inf for a row with
// LSE = -inf when a bias is present (its pairs may be visible with B = -inf,
// and every probability of the row is 0).
template <bool BIAS>
__device__ __forceinline__ float neg_lse2(float lse) {
  if constexpr (BIAS) return lse == -INFINITY ? -INFINITY : -lse * kLog2e;
  return -lse * kLog2e;
}

__device__ __forceinline__ float bf16_bits_to_float(u16 x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// dK/dV of workgroup `bid` (see bwd_main_kernel for the launch).
template <int D, bool CAUSAL, bool WIN, bool BIAS>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p, int n_kt, int bid) {
  using T = Tile<D>;
  constexpr int NC = D / 16;  // 16-wide d chunks of the score contractions
  constexpr int ND = D / 32;  // 32-row d tiles of dK^T, dV^T
  // Two slots per staged tensor as separate arrays, chosen at compile time
  // (the block loop is unrolled by two): with one array indexed at run time
  // the compiler cannot tell the slot being loaded from the slot being read
  // and waits for the next block's loads before every read of this one.
  __shared__ __attribute__((aligned(1024))) unsigned char q_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char q_st1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char do_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char do_st1[T::kBytes];
  __shared__ __attribute__((aligned(16))) float lse_st0[kTileRows];
  __shared__ __attribute__((aligned(16))) float lse_st1[kTileRows];
  __shared__ __attribute__((aligned(16))) float d_st0[kTileRows];
  __shared__ __attribute__((aligned(16))) float d_st1[kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // Workgroup -> (key tile, batch-or-sequence, K/V head); the key tiles near
  // the start of a sequence see the most queries under the causal mask and
  // go first.
  const int units = p.batch * p.hkv;
  const int kt = bid / units;
  const int b = (bid % units) / p.hkv;
  const int kvh = (bid % units) % p.hkv;
  const int gq = p.hq / p.hkv;
  const SeqBounds sb = seq_bounds(p, b);
  const int k0 = kt * kBwdRows;
  if (k0 >= sb.Lk) return;
  const int kw0 = k0 + 32 * w;  // first key of this wave
  const int key = kw0 + j;      // this lane's key (column of every score block)

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const u16* kg = static_cast<const u16*>(p.k) + sb.k_tok0 * kstride + static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + sb.k_tok0 * kstride + static_cast<long>(kvh) * D;

  // K and V of this wave's keys: the B operands of S = Q K^T and dP = dO V^T
  // (column = key, 8 consecutive d values per lane).
  bf16x8 kf[NC], vf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (key < sb.Lk) {
      a = ld16(kg + static_cast<long>(key) * kstride + 16 * cc + 8 * h2);
      c = ld16(vg + static_cast<long>(key) * kstride + 16 * cc + 8 * h2);
    }
    kf[cc] = as_bf16x8(a);
    vf[cc] = as_bf16x8(c);
    asm volatile("" : "+a"(kf[cc]), "+a"(vf[cc]));  // only the matrix cores read them: AGPRs
  }
  asm volatile("s_nop 4" ::: "memory");  // AGPR writes before the inline MFMAs read them
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int t = 0; t < ND; ++t) {
    dk[t] = dv[t] = f32x16{};
    asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));  // the accumulators live in AGPRs
  }

  // Query blocks: every q-head of the group, rows from the block that holds
  // key k0 (causal) or from 0, to the end of the sequence; with a window,
  // only the rows whose windows reach keys k0 .. k0+127.
  int qlo = CAUSAL ? k0 : 0;
  int qhi = sb.Lq;
  if constexpr (WIN) {
    if (p.win_right >= 0) qlo = max(qlo, k0 - p.win_right);
    if (p.win_left >= 0) qhi = min(qhi, k0 + kBwdRows - 1 + p.win_left + 1);
  }
  const int qb0 = (max(qlo, 0) / kTileRows) * kTileRows;
  const int nqb = qhi > qb0 ? (qhi - qb0 + kTileRows - 1) / kTileRows : 0;
  const int n_it = nqb * gq;
  const float c = p.scale_log2;

  auto head_of = [&](int it) { return kvh * gq + it / nqb; };
  auto issue = [&](int it, unsigned char* q_dst, unsigned char* do_dst, float* lse_dst,
                   float* d_dst) {
    const int h = head_of(it);
    const int q0 = qb0 + (it % nqb) * kTileRows;
    const u16* qg = static_cast<const u16*>(p.q) + sb.q_tok0 * qstride + static_cast<long>(h) * D;
    const u16* dg = static_cast<const u16*>(p.dout) + sb.q_tok0 * qstride + static_cast<long>(h) * D;
    issue_tile<D>(qg, qstride, q0, sb.Lq, q_dst, tid, w);
    issue_tile<D>(dg, qstride, q0, sb.Lq, do_dst, tid, w);
    if (w < 2) {
      // 64 floats of LSE (wave 0) or D (wave 1): one 4-byte load per lane
      const RowIndex ri = row_index(p, sb, b, h);
      const float* src = (w == 0 ? p.lse : p.dsum) + ri.at(q0);
      const int rows = min(sb.Lq - q0, kTileRows);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(src), 0, static_cast<uint32_t>(rows) * 4u, kBufferFlags);
      float* dst = w == 0 ? lse_dst : d_dst;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 4, lane * 4, 0, 0, 0);
    }
  };

  if (n_it > 0) issue(0, q_st0, do_st0, lse_st0, d_st0);
  auto step = [&](auto par_tag, int it) {
    constexpr int PAR = decltype(par_tag)::value;  // it & 1
    const int q0 = qb0 + (it % nqb) * kTileRows;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block `it` landed; every wave is done with block it-1
    if (it + 1 < n_it) {
      if constexpr (PAR) issue(it + 1, q_st0, do_st0, lse_st0, d_st0);
      else issue(it + 1, q_st1, do_st1, lse_st1, d_st1);
    }
    const unsigned char* qs = PAR ? q_st1 : q_st0;
    const unsigned char* ds_ = PAR ? do_st1 : do_st0;
    const float* ls = PAR ? lse_st1 : lse_st0;
    const float* dsm = PAR ? d_st1 : d_st0;
    // Sub-block `sub` alone: scores, then its vector work, then its
    // products (the biased kernels).
    auto serial_item = [&](int sub) {
      const int r0 = 32 * sub;  // tile row of this 32-row sub-block
      const int qs0 = q0 + r0;  // its first query
      // Bias of this lane's key against the block's 16 queries of this
      // half-wave (indices clamped into the sequence; clamped values belong
      // to invisible pairs and are never used).
      u16 bias_v[16];
      if constexpr (BIAS) {
        const u16* bgh = static_cast<const u16*>(p.bias) + b * p.bias_sb +
                         head_of(it) * p.bias_sh + min(key, sb.Lk - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          bias_v[r] = bgh[static_cast<long>(min(qs0 + mrow(r, h2), sb.Lq - 1)) * p.bias_sr];
      }
      // S = Q K^T and dP = dO V^T: lane = key, register r = query qs0 + mrow(r)
      // (inline-asm MFMAs: results in VGPRs for the vector work that follows,
      // read only after mfma_result_guard())
      f32x16 s = mfma_qk_first(row_operand<D>(qs, r0, 0, lane), kf[0]);
      f32x16 dp = mfma_qk_first(row_operand<D>(ds_, r0, 0, lane), vf[0]);
#pragma unroll
      for (int cc = 1; cc < NC; ++cc) {
        mfma_qk_acc(s, row_operand<D>(qs, r0, cc, lane), kf[cc]);
        mfma_qk_acc(dp, row_operand<D>(ds_, r0, cc, lane), vf[cc]);
      }
      mfma_result_guard();
      // P = 2^(c s - LSE log2 e) on visible pairs, dS = P (dP - D). A
      // sub-block whose pairs all exist and are visible (wave-uniform; most
      // of them under the causal mask) skips the per-element test.
      f32x16 pr, dsr;
      auto probs = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int rr = r0 + 8 * g4 + 4 * h2;
          const float4 l4 = *reinterpret_cast<const float4*>(ls + rr);
          const float4 d4 = *reinterpret_cast<const float4*>(dsm + rr);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float off = neg_lse2<BIAS>(lv[e]);
            if constexpr (BIAS) off = __builtin_fmaf(bf16_bits_to_float(bias_v[r]), kLog2e, off);
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, off));
            if constexpr (MASKED) {
              const int q = qs0 + mrow(r, h2);
              pr[r] = visible<CAUSAL, WIN>(p, q, key, sb.Lq, sb.Lk) ? pe : 0.f;
            } else {
              pr[r] = pe;
            }
            dsr[r] = pr[r] * (dp[r] - dvv[e]);
          }
        }
      };
      const bool full = !WIN && qs0 + 31 < sb.Lq && kw0 + 31 < sb.Lk && (!CAUSAL || qs0 >= kw0 + 31);
      if (full) probs(std::false_type{});
      else probs(std::true_type{});
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries (two 16-chunks)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const bf16x8 pb = pack_chunk(pr, g);
        const bf16x8 sbv = pack_chunk(dsr, g);
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(ds_, r0, t, g, lane), pb, dv[t], 0, 0, 0);
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(qs, r0, t, g, lane), sbv, dk[t], 0, 0, 0);
          asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));
        }
      }
    };
    // Is sub-block `sub` of this tile active for this wave (rows in the
    // sequence, some pair possibly visible)?
    auto active = [&](int sub) {
      const int qs0 = q0 + 32 * sub;
      if (qs0 >= sb.Lq) return false;
      if (CAUSAL && qs0 + 31 < kw0) return false;  // every query before every key of the wave
      if constexpr (WIN) {  // every query outside every window of the wave's keys
        if (p.win_right >= 0 && qs0 + 31 < kw0 - p.win_right) return false;
        if (p.win_left >= 0 && qs0 > kw0 + 31 + p.win_left) return false;
      }
      return true;
    };
    // every pair of sub-block `sub` exists and is visible: no per-element test
    auto all_visible = [&](int sub) {
      const int qs0 = q0 + 32 * sub;
      return !WIN && qs0 + 31 < sb.Lq && kw0 + 31 < sb.Lk && (!CAUSAL || qs0 >= kw0 + 31);
    };
    // P and dS of register r of a sub-block, in place (s becomes P, dp
    // becomes dS), from the row's LSE and D (lv, dvv). No mask here: masked
    // tiles are cleared afterwards by mask_sub.
    auto prob_elem = [&](int r, f32x16& sv, f32x16& dpv, float lv, float dvv) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, neg_lse2<false>(lv)));
      const float dd = dpv[r] - dvv;
      sv[r] = pe;
      dpv[r] = pe * dd;
    };
    // Zero P and dS of the invisible pairs of sub-block `sub` (a select, so
    // whatever the exponential gave for such a pair, inf included, is gone).
    auto mask_sub = [&](int sub, f32x16& pv, f32x16& dsv) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vis = visible<CAUSAL, WIN>(p, q0 + 32 * sub + mrow(r, h2), key, sb.Lq, sb.Lk);
        pv[r] = vis ? pv[r] : 0.f;
        dsv[r] = vis ? dsv[r] : 0.f;
      }
    };
    // Both sub-blocks active: a software pipeline over the tile. The matrix
    // cores form the second sub-block's S and dP while the vector unit turns
    // the first one's scores into P and dS, then accumulate the first one's
    // dV and dK while the vector unit does the second one's; one MFMA per
    // step, the vector work spread evenly over the steps.
    auto pipelined = [&](bool full0, bool full1) {
      constexpr int NS = 2 * NC;        // score steps: S and dP chains interleaved
      constexpr int NP = 4 * ND;        // product steps: 2 chunks x ND tiles x (dV, dK)
      constexpr int EPS = 16 / NS;      // elements per score step
      constexpr int EPP = 16 / NP;      // elements per product step
      static_assert(EPS * NS == 16 && EPP * NP == 16, "element spread");
      // LSE and D of a sub-block's rows: registers 4g4 .. 4g4+3 are rows
      // 32*sub + 8g4 + 4*h2 + (0..3); each group is read two steps before
      // its first element
      float4 l4[4], d4[4];
      auto load_ld = [&](int sub, int g4) {
        l4[g4] = *reinterpret_cast<const float4*>(ls + 32 * sub + 8 * g4 + 4 * h2);
        d4[g4] = *reinterpret_cast<const float4*>(dsm + 32 * sub + 8 * g4 + 4 * h2);
      };
      load_ld(0, 0);
      // phase 1: S and dP of sub-block 0, operands read two steps ahead
      f32x16 s0, p0;
      {
        bf16x8 op0[NS];
        auto load_op0 = [&](int k) {
          op0[k] = row_operand<D>((k & 1) ? ds_ : qs, 0, k >> 1, lane);
        };
        load_op0(0);
        load_op0(1);
        static_for<NS>([&](auto K) {
          constexpr int k = decltype(K)::value;
          if constexpr (k + 2 < NS) load_op0(k + 2);
          constexpr int cc = k >> 1;
          if constexpr ((k & 1) == 0) {
            if constexpr (cc == 0) s0 = mfma_qk_first(op0[k], kf[0]);
            else mfma_qk_acc(s0, op0[k], kf[cc]);
          } else {
            if constexpr (cc == 0) p0 = mfma_qk_first(op0[k], vf[0]);
            else mfma_qk_acc(p0, op0[k], vf[cc]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      mfma_result_guard();
      // phase 2: S and dP of sub-block 1 on the matrix cores, P and dS of
      // sub-block 0 on the vector unit. Operands are read two steps ahead.
      f32x16 s1, p1;
      bf16x8 op[NS];
      auto load_op = [&](int k) {
        op[k] = row_operand<D>((k & 1) ? ds_ : qs, 32, k >> 1, lane);
      };
      load_op(0);
      load_op(1);
      static_for<NS>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NS) load_op(k + 2);
        static_for<3>([&](auto G) {  // groups 1..3
          constexpr int g4 = decltype(G)::value + 1;
          constexpr int at = (4 * g4) / EPS - 2;
          if constexpr (at == k || (at < 0 && k == 0)) load_ld(0, g4);
        });
        constexpr int cc = k >> 1;
        if constexpr ((k & 1) == 0) {
          if constexpr (cc == 0) s1 = mfma_qk_first_w(op[k], kf[0]);
          else mfma_qk_acc_w(s1, op[k], kf[cc]);
        } else {
          if constexpr (cc == 0) p1 = mfma_qk_first_w(op[k], vf[0]);
          else mfma_qk_acc_w(p1, op[k], vf[cc]);
        }
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
          constexpr int r0e = k * EPS;
          const int r = r0e + e;
          prob_elem(r, s0, p0, f4_at(l4[r >> 2], r & 3), f4_at(d4[r >> 2], r & 3));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (!full0) mask_sub(0, s0, p0);
      bf16x8 pb0[2], sbv0[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        pb0[g] = pack_chunk(s0, g);
        sbv0[g] = pack_chunk(p0, g);
      }
      load_ld(1, 0);
      mfma_result_guard();  // sub-block 1's chains finished before its vector work
      // phase 3: dV and dK of sub-block 0 on the matrix cores, P and dS of
      // sub-block 1 on the vector unit; transposed operands two steps ahead.
      bf16x8 top[NP];
      auto load_top = [&](int k) {
        const int g = k / (2 * ND), t = (k >> 1) % ND;
        top[k] = tr_operand<D>((k & 1) ? qs : ds_, 0, t, g, lane);
      };
      load_top(0);
      load_top(1);
      static_for<NP>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NP) load_top(k + 2);
        static_for<3>([&](auto G) {
          constexpr int g4 = decltype(G)::value + 1;
          constexpr int at = (4 * g4) / EPP - 2;
          if constexpr (at == k || (at < 0 && k == 0)) load_ld(1, g4);
        });
        constexpr int g = k / (2 * ND), t = (k >> 1) % ND;
        if constexpr ((k & 1) == 0)
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[k], pb0[g], dv[t], 0, 0, 0);
        else
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[k], sbv0[g], dk[t], 0, 0, 0);
        asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));
#pragma unroll
        for (int e = 0; e < EPP; ++e) {
          const int r = k * EPP + e;
          prob_elem(r, s1, p1, f4_at(l4[r >> 2], r & 3), f4_at(d4[r >> 2], r & 3));
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      // phase 4: dV and dK of sub-block 1; transposed operands two steps
      // ahead, the first two read before the mask and the packing
      bf16x8 top1[NP];
      auto load_top1 = [&](int k) {
        const int g = k / (2 * ND), t = (k >> 1) % ND;
        top1[k] = tr_operand<D>((k & 1) ? qs : ds_, 32, t, g, lane);
      };
      load_top1(0);
      load_top1(1);
      if (!full1) mask_sub(1, s1, p1);
      bf16x8 pb1[2], sbv1[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        pb1[g] = pack_chunk(s1, g);
        sbv1[g] = pack_chunk(p1, g);
      }
      static_for<NP>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NP) load_top1(k + 2);
        constexpr int g = k / (2 * ND), t = (k >> 1) % ND;
        if constexpr ((k & 1) == 0)
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top1[k], pb1[g], dv[t], 0, 0, 0);
        else
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top1[k], sbv1[g], dk[t], 0, 0, 0);
        asm volatile("" : "+a"(dk[t]), "+a"(dv[t]));
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    const bool act0 = active(0), act1 = active(1);
    if constexpr (!BIAS) {
      // An inactive sub-block of an active tile goes through the pipeline
      // too, under the per-element test, so all its probabilities are 0
      // (it happens only near the diagonal and at a ragged end).
      if (act0 || act1) {
        pipelined(act0 && all_visible(0), act1 && all_visible(1));
      }
    } else {
      if (act0) serial_item(0);
      if (act1) serial_item(1);
    }
  };
  {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int it = 0; it < n_it; it += 2) {
      step(P0{}, it);
      if (it + 1 >= n_it) break;
      step(P1{}, it + 1);
    }
  }

  // dK = scale (dK^T)^T, dV = (dV^T)^T: lane = key, register r of d-tile t =
  // d column 32t + mrow(r); four consecutive d values per 8-byte store.
  // Explicit reads out of the AGPRs, after the last MFMAs have written them.
  mfma_result_guard();
#pragma unroll
  for (int t = 0; t < ND; ++t) {
    dk[t] = read_agpr(dk[t]);
    dv[t] = read_agpr(dv[t]);
  }
  if (key < sb.Lk) {
    u16* dkg = static_cast<u16*>(p.dk) + (sb.k_tok0 + key) * kstride + static_cast<long>(kvh) * D;
    u16* dvg = static_cast<u16*>(p.dv) + (sb.k_tok0 + key) * kstride + static_cast<long>(kvh) * D;
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 a4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a4[e] = static_cast<__bf16>(dk[t][4 * g4 + e] * p.scale);
          v4[e] = static_cast<__bf16>(dv[t][4 * g4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dkg + 32 * t + 8 * g4 + 4 * h2) = a4;
        *reinterpret_cast<bf16x4*>(dvg + 32 * t + 8 * g4 + 4 * h2) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

// dQ of workgroup `bid` (see bwd_main_kernel for the launch).
template <int D, bool CAUSAL, bool WIN, bool BIAS>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p, int n_qt, int bid) {
  using T = Tile<D>;
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  // two slots per tensor, separate arrays chosen at compile time (see the
  // dK/dV body)
  __shared__ __attribute__((aligned(1024))) unsigned char k_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st1[T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // Workgroup -> (query tile, batch-or-sequence, q-head), longest causal
  // tiles first.
  const int bh = p.hq * p.batch;
  const int qt = n_qt - 1 - bid / bh;
  const int b = (bid % bh) / p.hq;
  const int h = (bid % bh) % p.hq;
  const int kvh = h / (p.hq / p.hkv);
  const SeqBounds sb = seq_bounds(p, b);
  const int q0 = qt * kBwdRows;
  if (q0 >= sb.Lq) return;
  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + j;     // this lane's query (column of every S^T block)

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const u16* qg = static_cast<const u16*>(p.q) + sb.q_tok0 * qstride + static_cast<long>(h) * D;
  const u16* dg = static_cast<const u16*>(p.dout) + sb.q_tok0 * qstride + static_cast<long>(h) * D;
  const u16* kg = static_cast<const u16*>(p.k) + sb.k_tok0 * kstride + static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + sb.k_tok0 * kstride + static_cast<long>(kvh) * D;

  // Q and dO of this wave's rows: the B operands of S^T = K Q^T and
  // dP^T = V dO^T (column = query, 8 consecutive d values per lane); the
  // row's LSE (in base 2) and D.
  bf16x8 qf[NC], dof[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
    if (qrow < sb.Lq) {
      a = ld16(qg + static_cast<long>(qrow) * qstride + 16 * cc + 8 * h2);
      c = ld16(dg + static_cast<long>(qrow) * qstride + 16 * cc + 8 * h2);
    }
    qf[cc] = as_bf16x8(a);
    dof[cc] = as_bf16x8(c);
    asm volatile("" : "+a"(qf[cc]), "+a"(dof[cc]));  // only the matrix cores read them: AGPRs
  }
  asm volatile("s_nop 4" ::: "memory");  // AGPR writes before the inline MFMAs read them
  const RowIndex ri = row_index(p, sb, b, h);
  const float nlse2 = qrow < sb.Lq ? neg_lse2<BIAS>(p.lse[ri.at(qrow)]) : 0.f;
  // this lane's bias row (clamped into the sequence), 4 * h2 keys in: a run
  // of 4 keys starts at every multiple of 4 and never crosses the row's end
  const u16* brow = nullptr;
  if constexpr (BIAS)
    brow = static_cast<const u16*>(p.bias) + b * p.bias_sb + h * p.bias_sh +
           static_cast<long>(min(qrow, sb.Lq - 1)) * p.bias_sr + 4 * h2;
  const float drow = qrow < sb.Lq ? p.dsum[ri.at(qrow)] : 0.f;
  const float c = p.scale_log2;

  f32x16 dq[ND];
#pragma unroll
  for (int t = 0; t < ND; ++t) {
    dq[t] = f32x16{};
    asm volatile("" : "+a"(dq[t]));  // the accumulators live in AGPRs
  }

  // Key blocks: from 0 (or, with a window, the block holding the first
  // row's window start) to the last key any row of the tile sees.
  int kend = sb.Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBwdRows, sb.Lq));
  int key_base = 0;
  if constexpr (WIN) {
    if (p.win_right >= 0) kend = min(kend, min(q0 + kBwdRows, sb.Lq) - 1 + p.win_right + 1);
    if (p.win_left >= 0) key_base = (max(0, q0 - p.win_left) / kTileRows) * kTileRows;
  }
  const int nkb = kend > key_base ? (kend - key_base + kTileRows - 1) / kTileRows : 0;
  if (nkb > 0) {
    issue_tile<D>(kg, kstride, key_base, sb.Lk, k_st0, tid, w);
    issue_tile<D>(vg, kstride, key_base, sb.Lk, v_st0, tid, w);
  }
  auto step = [&](auto par_tag, int kb) {
    constexpr int PAR = decltype(par_tag)::value;  // kb & 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 1 < nkb) {
      unsigned char* k_nxt = PAR ? k_st0 : k_st1;
      unsigned char* v_nxt = PAR ? v_st0 : v_st1;
      issue_tile<D>(kg, kstride, key_base + (kb + 1) * kTileRows, sb.Lk, k_nxt, tid, w);
      issue_tile<D>(vg, kstride, key_base + (kb + 1) * kTileRows, sb.Lk, v_nxt, tid, w);
    }
    const unsigned char* ks = PAR ? k_st1 : k_st0;
    const unsigned char* vs = PAR ? v_st1 : v_st0;
    // Sub-block `sub` alone (the biased kernels): scores, then its vector
    // work, then its product.
    auto serial_item = [&](int sub) {
      const int r0 = 32 * sub;
      const int ks0 = key_base + kb * kTileRows + r0;  // first key of this 32-key sub-block
      // bias of keys ks0 + 8g + 4*h2 + (0..3) = registers 4g .. 4g+3
      u32x2 bias_v[4];
      if constexpr (BIAS) {
        const int kmax = ((sb.Lk - 1) & ~3) - 4 * h2;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          bias_v[g] = *reinterpret_cast<const u32x2*>(brow + min(ks0 + 8 * g, kmax));
      }
      // S^T = K Q^T and dP^T = V dO^T: lane = query, register r = key ks0 + mrow(r)
      // (inline-asm MFMAs: results in VGPRs, read only after mfma_result_guard())
      f32x16 st = mfma_qk_first(row_operand<D>(ks, r0, 0, lane), qf[0]);
      f32x16 dpt = mfma_qk_first(row_operand<D>(vs, r0, 0, lane), dof[0]);
#pragma unroll
      for (int cc = 1; cc < NC; ++cc) {
        mfma_qk_acc(st, row_operand<D>(ks, r0, cc, lane), qf[cc]);
        mfma_qk_acc(dpt, row_operand<D>(vs, r0, cc, lane), dof[cc]);
      }
      mfma_result_guard();
      f32x16 dst;
      auto dscores = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float off = nlse2;
          if constexpr (BIAS) {
            const uint32_t wd = bias_v[r >> 2][(r >> 1) & 1];
            off = __builtin_fmaf(__uint_as_float((r & 1) ? (wd & 0xffff0000u) : (wd << 16)),
                                 kLog2e, off);
          }
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], c, off));
          if constexpr (MASKED) {
            const int kk = ks0 + mrow(r, h2);
            dst[r] = visible<CAUSAL, WIN>(p, qrow, kk, sb.Lq, sb.Lk) ? pe * (dpt[r] - drow) : 0.f;
          } else {
            dst[r] = pe * (dpt[r] - drow);
          }
        }
      };
      // all pairs of the sub-block exist and are visible: no per-element test
      const bool full = !WIN && ks0 + 31 < sb.Lk && wq0 + 31 < sb.Lq && (!CAUSAL || ks0 + 31 <= wq0);
      if (full) dscores(std::false_type{});
      else dscores(std::true_type{});
      // dQ^T += K^T dS^T over the 32 keys (two 16-chunks)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const bf16x8 sbv = pack_chunk(dst, g);
#pragma unroll
        for (int t = 0; t < ND; ++t)
        {
          dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(ks, r0, t, g, lane), sbv, dq[t], 0, 0, 0);
          asm volatile("" : "+a"(dq[t]));
        }
      }
    };
    // Is 32-key sub-block `sub` of this tile active for this wave?
    auto active = [&](int sub) {
      const int ks0 = key_base + kb * kTileRows + 32 * sub;
      if (ks0 >= sb.Lk) return false;
      if (CAUSAL && ks0 > wq0 + 31) return false;  // every key after every query of the wave
      if constexpr (WIN) {  // every key outside every window of the wave's rows
        if (p.win_right >= 0 && ks0 > wq0 + 31 + p.win_right) return false;
        if (p.win_left >= 0 && ks0 + 31 < wq0 - p.win_left) return false;
      }
      return true;
    };
    // every pair of sub-block `sub` exists and is visible
    auto all_visible = [&](int sub) {
      const int ks0 = key_base + kb * kTileRows + 32 * sub;
      return !WIN && ks0 + 31 < sb.Lk && wq0 + 31 < sb.Lq && (!CAUSAL || ks0 + 31 <= wq0);
    };
    // dS^T of register r, in place into dpv: P (dP - D), P = 2^(c s - LSE)
    auto dscore_elem = [&](int r, const f32x16& sv, f32x16& dpv) {
      const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c, nlse2));
      dpv[r] = pe * (dpv[r] - drow);
    };
    // zero dS^T of the invisible pairs of sub-block `sub` (a select)
    auto mask_sub = [&](int sub, f32x16& dsv) {
      const int ks0 = key_base + kb * kTileRows + 32 * sub;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dsv[r] = visible<CAUSAL, WIN>(p, qrow, ks0 + mrow(r, h2), sb.Lq, sb.Lk) ? dsv[r] : 0.f;
    };
    // Software pipeline over the tile's two sub-blocks (as in the dK/dV
    // body): the second sub-block's S^T and dP^T chains run on the matrix
    // cores while the vector unit forms the first one's dS^T, then the first
    // one's dQ^T product runs while the vector unit does the second one's.
    auto pipelined = [&](bool full0, bool full1) {
      constexpr int NS = 2 * NC;   // score steps
      constexpr int NP = 2 * ND;   // product steps: 2 chunks x ND tiles
      constexpr int EPS = 16 / NS, EPP = 16 / NP;
      static_assert(EPS * NS == 16 && EPP * NP == 16, "element spread");
      // phase 1: S^T and dP^T of sub-block 0, operands read two steps ahead
      f32x16 s0, p0;
      {
        bf16x8 op0[NS];
        auto load_op0 = [&](int k) { op0[k] = row_operand<D>((k & 1) ? vs : ks, 0, k >> 1, lane); };
        load_op0(0);
        load_op0(1);
        static_for<NS>([&](auto K) {
          constexpr int k = decltype(K)::value;
          if constexpr (k + 2 < NS) load_op0(k + 2);
          constexpr int cc = k >> 1;
          if constexpr ((k & 1) == 0) {
            if constexpr (cc == 0) s0 = mfma_qk_first(op0[k], qf[0]);
            else mfma_qk_acc(s0, op0[k], qf[cc]);
          } else {
            if constexpr (cc == 0) p0 = mfma_qk_first(op0[k], dof[0]);
            else mfma_qk_acc(p0, op0[k], dof[cc]);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      mfma_result_guard();
      // phase 2: sub-block 1's chains with sub-block 0's dS^T
      f32x16 s1, p1;
      bf16x8 op[NS];
      auto load_op = [&](int k) { op[k] = row_operand<D>((k & 1) ? vs : ks, 32, k >> 1, lane); };
      load_op(0);
      load_op(1);
      static_for<NS>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NS) load_op(k + 2);
        constexpr int cc = k >> 1;
        if constexpr ((k & 1) == 0) {
          if constexpr (cc == 0) s1 = mfma_qk_first_w(op[k], qf[0]);
          else mfma_qk_acc_w(s1, op[k], qf[cc]);
        } else {
          if constexpr (cc == 0) p1 = mfma_qk_first_w(op[k], dof[0]);
          else mfma_qk_acc_w(p1, op[k], dof[cc]);
        }
#pragma unroll
        for (int e = 0; e < EPS; ++e) dscore_elem(k * EPS + e, s0, p0);
        __builtin_amdgcn_sched_barrier(0);
      });
      if (!full0) mask_sub(0, p0);
      bf16x8 sbv0[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) sbv0[g] = pack_chunk(p0, g);
      mfma_result_guard();  // sub-block 1's chains finished before its vector work
      // phase 3: sub-block 0's dQ^T product with sub-block 1's dS^T
      bf16x8 top[NP];
      auto load_top = [&](int k) { top[k] = tr_operand<D>(ks, 0, k % ND, k / ND, lane); };
      load_top(0);
      load_top(1);
      static_for<NP>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NP) load_top(k + 2);
        constexpr int g = k / ND, t = k % ND;
        dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top[k], sbv0[g], dq[t], 0, 0, 0);
        asm volatile("" : "+a"(dq[t]));
#pragma unroll
        for (int e = 0; e < EPP; ++e) dscore_elem(k * EPP + e, s1, p1);
        __builtin_amdgcn_sched_barrier(0);
      });
      // phase 4: sub-block 1's product; transposed operands two steps
      // ahead, the first two read before the mask and the packing
      bf16x8 top1[NP];
      auto load_top1 = [&](int k) { top1[k] = tr_operand<D>(ks, 32, k % ND, k / ND, lane); };
      load_top1(0);
      load_top1(1);
      if (!full1) mask_sub(1, p1);
      bf16x8 sbv1[2];
#pragma unroll
      for (int g = 0; g < 2; ++g) sbv1[g] = pack_chunk(p1, g);
      static_for<NP>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (k + 2 < NP) load_top1(k + 2);
        constexpr int g = k / ND, t = k % ND;
        dq[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top1[k], sbv1[g], dq[t], 0, 0, 0);
        asm volatile("" : "+a"(dq[t]));
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    const bool act0 = active(0), act1 = active(1);
    if constexpr (!BIAS) {
      // inactive sub-blocks of an active tile go through the pipeline and
      // are cleared by mask_sub
      if (act0 || act1) pipelined(act0 && all_visible(0), act1 && all_visible(1));
    } else {
      if (act0) serial_item(0);
      if (act1) serial_item(1);
    }
  };
  {
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (int kb = 0; kb < nkb; kb += 2) {
      step(P0{}, kb);
      if (kb + 1 >= nkb) break;
      step(P1{}, kb + 1);
    }
  }

  // dQ = scale (dQ^T)^T: lane = query, register r of d-tile t = d column
  // 32t + mrow(r); explicit reads out of the AGPRs after the last MFMAs.
  mfma_result_guard();
#pragma unroll
  for (int t = 0; t < ND; ++t) dq[t] = read_agpr(dq[t]);
  if (qrow < sb.Lq) {
    u16* dqg = static_cast<u16*>(p.dq) + (sb.q_tok0 + qrow) * qstride + static_cast<long>(h) * D;
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 a4;
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = static_cast<__bf16>(dq[t][4 * g4 + e] * p.scale);
        *reinterpret_cast<bf16x4*>(dqg + 32 * t + 8 * g4 + 4 * h2) = a4;
      }
  }
}

// Both gradient kernels in one launch: they depend on the row dots D but
// not on each other, so workgroups 0 .. n_dkdv-1 run the dK/dV body (the
// longest key tiles first) and the rest the dQ body (the longest query
// tiles first). Short dQ tiles then fill compute units as the long dK/dV
// tiles finish, instead of each kernel draining its own tail. Either part
// may be empty.
template <int D, bool CAUSAL, bool WIN, bool BIAS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(BwdParams p, int n_qt, int n_kt, int n_dkdv) {
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < n_dkdv) bwd_dkdv_body<D, CAUSAL, WIN, BIAS>(p, n_kt, bid);
  else bwd_dq_body<D, CAUSAL, WIN, BIAS>(p, n_qt, bid - n_dkdv);
}

}  // namespace

// One object file per (head width, causal) pair, like the forward kernels.
// An empty side launches no workgroups for it: with Nq == 0 only dK/dV
// workgroups run and write zeros (no query sees any key), with Nk == 0
// only dQ workgroups run and write zeros.
template <int D, bool CAUSAL, bool WIN, bool BIAS>
hipError_t launch_bwd_main(const BwdParams& p, hipStream_t stream) {
  const long n_rows = static_cast<long>(p.batch) * p.nq * p.hq;
  if (n_rows > 0) {
    const long dot_blocks = (n_rows * (D / 8) + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3(static_cast<unsigned>(dot_blocks)),
                       dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qt = (p.nq + kBwdRows - 1) / kBwdRows;
  const int n_kt = (p.nk + kBwdRows - 1) / kBwdRows;
  const long n_dq = n_rows > 0 ? static_cast<long>(n_qt) * p.hq * p.batch : 0;
  const long n_dkdv = p.nk > 0 ? static_cast<long>(n_kt) * p.hkv * p.batch : 0;
  if (n_dq + n_dkdv == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, WIN, BIAS>),
                     dim3(static_cast<unsigned>(n_dkdv + n_dq)), dim3(kThreads), 0, stream, p,
                     n_qt, n_kt, static_cast<int>(n_dkdv));
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  // the host never combines a bias with a window
  if (p.bias != nullptr) return launch_bwd_main<D, CAUSAL, false, true>(p, stream);
  if (p.win_left >= 0 || p.win_right >= 0) return launch_bwd_main<D, CAUSAL, true, false>(p, stream);
  return launch_bwd_main<D, CAUSAL, false, false>(p, stream);
}

#if !defined(FA_BF16_D) || !defined(FA_BF16_CAUSAL)
#error "compile with -DFA_BF16_D=64|128 -DFA_BF16_CAUSAL=0|1"
#endif
template hipError_t launch_bwd_bf16<FA_BF16_D, (FA_BF16_CAUSAL != 0)>(const BwdParams&,
                                                                    hipStream_t);

}  // namespace fa
