// Exact tiled attention forward, bf16 in / bf16 out, float32 softmax state
// and accumulation, for gfx950 (CDNA4) matrix cores.
//
// The schedule is the IO-aware tiling of "Understanding FlashAttention Pt 1:
// Personal Notes" (section 1.2: compute a small S tile, softmax it, use it
// with V_j, discard it, go to the next tile) with the online row state of
// "Softmax does not need the matrix" (section "Carry the Normalizer":
// m' = max(m, m_b), l' = e^(m-m') l + sum e^(s-m'), a' = e^(m-m') a +
// sum e^(s-m') v). Scores are kept in base 2: x = s * scale * log2(e), so
// every exponential is one v_exp_f32 and e^(m-m') becomes 2^(m-m').
//
// Work decomposition (one workgroup = 4 wavefronts of 64 lanes, one
// wavefront per SIMD, so each wavefront has the whole register file):
//   * a workgroup owns 256 query rows of one (batch or sequence, q-head);
//     wavefront w owns rows 64w .. 64w+63 of that tile as two 32-row query
//     tiles, so every K or V operand read from LDS feeds two MFMAs;
//   * K/V blocks of 64 keys stream through LDS with buffer-to-LDS loads (no
//     VGPR staging); K runs one block ahead of V, each with two buffers;
//     rows past the end of the sequence lie outside the buffer range and
//     arrive as zeros;
//   * each wave computes the transposed score block S^T = K_j Q_i^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 32 scores of ONE query row
//     per query tile: row max and row sum are lane-local plus one
//     v_permlane32_swap with the other half-wave, and the rescale factor is
//     a per-lane scalar;
//   * the output is accumulated transposed as well, O^T += V_j^T P^T: P^T
//     feeds the B operand straight from the score registers, and V^T comes
//     from the row-major V tile through ds_read_b64_tr_b16 transposing reads;
//   * the key loop is software-pipelined: while the exponentials of block j
//     are computed, the matrix cores form the scores of block j+1 and
//     accumulate P_j V_j, in a fixed compile-time interleave (Plan);
//   * K/V tiles are stored with an XOR swizzle of the 16-byte units of each
//     row so that the score reads (16 consecutive rows, same column) and the
//     transposing V reads (4 consecutive rows, 64 bytes each) spread over the
//     LDS banks.
//
// Reference point of the exponentials. The invariant of "Carry the
// Normalizer" holds for ANY common reference m of l and a: o = a / l and
// LSE = m + log l do not depend on it, as long as nothing overflows. A row's
// first visible block sets m (its accumulator is still zero, so nothing is
// rescaled); afterwards m is kept while the weights stay below 2^kRaise.
// Only when some row of a wave would exceed that are the wave's references
// raised to the block maxima and the accumulators rescaled, a path realistic
// inputs rarely take; it passes the accumulator through private memory so
// that the vector unit never reads it and it stays in AGPRs.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <type_traits>
#include <utility>

#include "fa_bf16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBR = kBf16TileRows;  // query rows per workgroup

// issue_tile for a tile that may not be wanted: an unwanted tile gets an
// empty buffer range (its loads read nothing and write zeros to its LDS),
// so every wave issues the same number of loads either way.
template <int D>
__device__ __forceinline__ void issue_tile_if(const u16* g, long stride, int r0, int L, bool want,
                                              unsigned char* dst, int tid, int w) {
  using T = Tile<D>;
  const int rows = min(L - r0, kTileRows);
  const uint32_t stride_b = static_cast<uint32_t>(stride * 2);
  const uint32_t nrec = want ? static_cast<uint32_t>(rows - 1) * stride_b + T::kRowBytes : 0u;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(g + static_cast<long>(want ? r0 : 0) * stride), 0, nrec, kBufferFlags);
  const int lane = tid & 63;
  unsigned char* const base = dst + w * (T::kLoads * 1024);
  static_for<T::kLoads>([&](auto IT) {
    constexpr int it = decltype(IT)::value;
    const int u = (w * T::kLoads + it) * 64 + lane;
    const int row = u / T::kUnits;
    const int gc = (u % T::kUnits) ^ swz<T::kUnits>(row);
    const uint32_t voff = row * stride_b + gc * 16 - it * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)base, 16, voff, 0, it * 1024, 0);
  });
}
constexpr int kBC = kTileRows;      // keys per K/V block
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRaise = 16.f;      // the main loop keeps m while the block max is <= m + 16

// Instruction plan of one key block for one wave (two 32-row query tiles).
// The block has M matrix steps: 4*NC score MFMAs of the NEXT block (two
// 32-key tiles x NC d-chunks x two query tiles) and 8*ND P V MFMAs of THIS
// block (four 16-key chunks x ND d-tiles x two query tiles). Consecutive
// steps share one LDS operand (the two query tiles). The 64 exponentials of
// this block (32 score registers per query tile) are spread evenly over the
// first M - 2*ND steps; P V chunk g is placed right after the step that
// finishes its 16 probabilities (8 per query tile), and score MFMAs fill the
// remaining steps. The last 2*ND steps (chunk 3's P V MFMAs) carry the row
// maxima of the next block's scores, whose MFMAs are done by then, so the
// next block starts with its reference update instead of a serial reduction.
template <int D>
struct Plan {
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int M = 4 * NC + 8 * ND;
  static constexpr int VS = M - 2 * ND;  // steps that carry exponentials
  static constexpr int elem_step(int e) { return e * VS / 64; }
  // elements of step s: first_elem(s) .. first_elem(s + 1) - 1
  static constexpr int first_elem(int s) { return (s * 64 + VS - 1) / VS; }
  static constexpr int pv_start(int g) { return elem_step(16 * g + 15) + 1; }
  // -1 if step s is a score MFMA, else the P V chunk it belongs to
  static constexpr int pv_chunk(int s) {
    for (int g = 0; g < 4; ++g)
      if (s >= pv_start(g) && s < pv_start(g) + 2 * ND) return g;
    return -1;
  }
  // index of the score MFMA at step s (number of score steps before it)
  static constexpr int qk_index(int s) {
    int n = 0;
    for (int i = 0; i < s; ++i) n += pv_chunk(i) < 0 ? 1 : 0;
    return n;
  }
  // Score MFMA q: key tile q / (2NC), d-chunk (q / 2) % NC, query tile q % 2,
  // so the first key tile of the next block is formed while the first key
  // tile of this block is consumed. Operand p = q / 2 (K tile p / NC,
  // d-chunk p % NC) serves both query tiles.
  // first step that uses score operand p
  static constexpr int qk_first(int p) {
    for (int s = 0; s < M; ++s)
      if (pv_chunk(s) < 0 && qk_index(s) == 2 * p) return s;
    return -1;
  }
  // last step that forms a score MFMA of key tile kt, query tile qt
  static constexpr int last_qk_step(int kt, int qt) {
    int last = -1;
    for (int s = 0; s < M; ++s)
      if (pv_chunk(s) < 0 && qk_index(s) / (2 * NC) == kt && qk_index(s) % 2 == qt) last = s;
    return last;
  }
  static constexpr bool valid() {
    int qk = 0;
    for (int s = 0; s < M; ++s) qk += pv_chunk(s) < 0 ? 1 : 0;
    for (int g = 0; g + 1 < 4; ++g)
      if (pv_start(g + 1) < pv_start(g) + 2 * ND) return false;
    return qk == 4 * NC && pv_start(3) + 2 * ND == M;
  }
};
static_assert(Plan<128>::valid() && Plan<64>::valid(), "block plan");

// WIN: sliding window, query i sees keys i - win_left .. i + win_right
// (a negative bound is unbounded), on top of the causal mask. The
// workgroup streams only the key blocks its rows' windows reach; blocks
// are indexed from the first of them, kb_base.
// BIAS: an additive bf16 bias B joins the scores of the visible pairs
// before the softmax ("Understanding FlashAttention Pt 1", section 0.2:
// S = Q K^T / sqrt(d) + B). Each lane loads the bias values of its own
// score registers (runs of 4 consecutive keys, 8 bytes) straight into
// registers, one block ahead; scores then carry t = scale * s + b in
// natural units and the base-2 factor becomes log2(e).
// SPLIT (no mask but the key count, no window, no bias): for grids that
// would leave compute units idle, a workgroup owns 128 query rows and its
// two wave pairs take the first and the second half of the key blocks;
// at the end the second pair hands its (m, l, a) to the first through LDS,
// which merges them by the rule for two blocks of "Carry the Normalizer"
// (common reference m = max(m1, m2), each part scaled by e^(m_i - m)).
template <int D, bool CAUSAL, bool WIN, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_kernel(FwdParams p, int n_qt) {
  static_assert(!SPLIT || (!CAUSAL && !WIN && !BIAS), "key halves only for the plain mask");
  using T = Tile<D>;
  using PL = Plan<D>;
  constexpr int NC = D / 16;  // 16-wide d chunks of the QK^T contraction
  constexpr int ND = D / 32;  // 32-row tiles of O^T
  constexpr int NH = SPLIT ? 2 : 1;               // key ranges per workgroup
  constexpr int ROWS = SPLIT ? kBR / 2 : kBR;     // query rows per workgroup
  // K runs one block ahead of V: block j+1's scores are formed while block
  // j's probabilities meet V, so each tensor has its own two buffers (one
  // per key half with SPLIT).
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[NH * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[NH * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[NH * T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[NH * T::kBytes];
  // the workgroup's Q rows, staged once (a smaller alignment places them
  // after the K/V buffers, whose LDS offsets then fit the 16-bit immediate
  // of the key loop's LDS reads)
  __shared__ __attribute__((aligned(256))) unsigned char qst[(ROWS / 64) * T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = SPLIT ? (w >> 1) : 0;   // key half of this wave
  const int wrow = SPLIT ? (w & 1) : w;    // 64-row group of this wave
  const int j = lane & 31;   // query column of S^T / O^T; key row of the K operand
  const int h2 = lane >> 5;  // half-wave

  // Map the workgroup to (tile, batch-or-sequence, q-head). Workgroup ids are
  // dealt round-robin to the 8 XCDs (id % 8), each with its own L2. When the
  // K/V heads (over all batch entries) split evenly over the XCDs, every
  // query tile that reads K/V head u runs on XCD u % 8, so that head's K/V
  // stay in one L2. Within an XCD, and in the fallback order, the longest
  // causal tiles go first and the q-heads sharing a K/V head are adjacent.
  const int gq = p.hq / p.hkv;
  const int units = p.batch * p.hkv;
  int tile, b, h;
  if ((units & 7) == 0) {
    const int x = blockIdx.x & 7;
    const int idx = blockIdx.x >> 3;
    const int hh = idx % gq;
    const int t2 = idx / gq;
    const int upx = units >> 3;
    // With many tiles per unit (long sequences, whose K/V heads outgrow an
    // L2), chunks of ch tiles of one unit (up to 32 workgroups, one XCD's
    // CUs) run together, so the XCD streams one K/V head at a time. Chunks
    // run longest first across the XCD's units, a partial chunk (n_qt % ch
    // tiles) last; ch <= n_qt / 8 keeps the last chunks short. ch = 1 is
    // plain longest-first order across units.
    const int ch = n_qt >= 32 ? max(1, min(32 / gq, n_qt / 8)) : 1;
    const int n_full = n_qt / ch;
    const int full_slots = n_full * upx * ch;
    int ui, rank;
    if (t2 < full_slots) {
      const int r2 = t2 / ch;
      ui = r2 % upx;
      rank = (r2 / upx) * ch + t2 % ch;
    } else {
      const int rem = n_qt - n_full * ch;
      const int t3 = t2 - full_slots;
      ui = t3 / rem;
      rank = n_full * ch + t3 % rem;
    }
    const int u = ui * 8 + x;
    tile = n_qt - 1 - rank;
    b = u / p.hkv;
    h = (u % p.hkv) * gq + hh;
  } else {
    const int bh = p.hq * p.batch;
    tile = n_qt - 1 - static_cast<int>(blockIdx.x / bh);
    const int rem = static_cast<int>(blockIdx.x % bh);
    b = rem / p.hq;
    h = rem % p.hq;
  }
  const int kvh = h / gq;

  long q_tok0, k_tok0, lse_base;
  int Lq, Lk;
  if (p.cu_seqlens != nullptr) {
    const int s0 = p.cu_seqlens[b];
    const int s1 = p.cu_seqlens[b + 1];
    const int total = p.cu_seqlens[p.batch];
    Lq = Lk = s1 - s0;
    q_tok0 = k_tok0 = s0;
    lse_base = static_cast<long>(h) * total + s0;
  } else {
    Lq = p.nq;
    Lk = p.nk;
    q_tok0 = static_cast<long>(b) * p.nq;
    k_tok0 = static_cast<long>(b) * p.nk;
    lse_base = (static_cast<long>(b) * p.hq + h) * p.nq;
  }
  const int q0 = tile * ROWS;
  if (q0 >= Lq) return;

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const u16* qg = static_cast<const u16*>(p.q) + q_tok0 * qstride + static_cast<long>(h) * D;
  const u16* kg = static_cast<const u16*>(p.k) + k_tok0 * kstride + static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + k_tok0 * kstride + static_cast<long>(kvh) * D;

  // Blocks the workgroup streams, and blocks this wave computes: a causal
  // wave stops at the block holding its own diagonal, and a wave whose rows
  // all lie past the end of the queries computes nothing (it still loads
  // its share of every tile and meets every barrier).
  int kend = Lk;
  if (CAUSAL) kend = min(kend, min(q0 + ROWS, Lq));
  int kb_base = 0;  // first key block of the workgroup
  if constexpr (WIN) {
    if (p.win_right >= 0) kend = min(kend, min(q0 + kBR, Lq) - 1 + p.win_right + 1);
    if (p.win_left >= 0) kb_base = max(0, q0 - p.win_left) / kBC;
  }
  int nblk;
  if constexpr (WIN) nblk = kend > kb_base * kBC ? (kend + kBC - 1) / kBC - kb_base : 0;
  else nblk = (kend + kBC - 1) / kBC;
  // With SPLIT, half h streams blocks h*nh0 .. of the nblk (nh0 of them for
  // half 0, the rest for half 1); the loop runs nh0 steps for both.
  int nbh[NH];
  if constexpr (SPLIT) {
    const int nh0 = (nblk + 1) / 2;
    nbh[0] = nh0;
    nbh[1] = nblk - nh0;
    kb_base = half * nh0;
    nblk = nh0;
  } else {
    nbh[0] = nblk;
  }
  const int key_base = kb_base * kBC;  // first key of local block 0 (of this wave's half)
  const int wq0 = q0 + 64 * wrow;      // first query row of this wave
  int nblk_w = wq0 >= Lq ? 0 : (SPLIT ? nbh[half] : nblk);
  if (CAUSAL) nblk_w = min(nblk_w, wq0 / kBC + 1 - kb_base);
  if constexpr (WIN) {
    if (p.win_right >= 0) nblk_w = min(nblk_w, (wq0 + 63 + p.win_right) / kBC + 1 - kb_base);
  }

  // Every tile is loaded by all four waves; hk(h) is the first key of
  // half h, and a half streams nbh[h] blocks.
  auto hk = [&](int h) { return SPLIT ? h * nblk * kBC : key_base; };
  // K_0 and the workgroup's Q rows first, then V_0 and K_1: a fixed number
  // of loads per wave, so the first scores wait for the first group only.
#pragma unroll
  for (int h = 0; h < NH; ++h)
    issue_tile_if<D>(kg, kstride, hk(h), Lk, nbh[h] > 0, kb0 + h * T::kBytes, tid, w);
#pragma unroll
  for (int sub = 0; sub < ROWS / 64; ++sub)
    issue_tile_if<D>(qg, qstride, q0 + 64 * sub, Lq, q0 + 64 * sub < Lq, qst + sub * T::kBytes,
                     tid, w);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    issue_tile_if<D>(vg, kstride, hk(h), Lk, nbh[h] > 0, vb0 + h * T::kBytes, tid, w);
    issue_tile_if<D>(kg, kstride, hk(h) + kBC, Lk, nbh[h] > 1, kb1 + h * T::kBytes, tid, w);
  }
  __builtin_amdgcn_sched_barrier(0);
  constexpr int kLater = NH * 2 * T::kLoads;  // loads issued after K_0 and Q
  static_assert(kLater <= 63, "vmcnt range");
  // this wave's view of the buffers (its key half)
  unsigned char* const kw0 = kb0 + half * T::kBytes;
  unsigned char* const kw1 = kb1 + half * T::kBytes;
  unsigned char* const vw0 = vb0 + half * T::kBytes;
  unsigned char* const vw1 = vb1 + half * T::kBytes;

  // A negative scale is applied by negating Q (exact in bf16), so that the
  // base-2 factor c below is >= 0 and max(c*s) = c*max(s). With a bias the
  // scores become t = cn * s + b first and the base-2 factor is log2(e).
  const float c = fmaxf(fabsf(p.scale_log2), FLT_MIN);
  const float cn = fmaxf(fabsf(p.scale), FLT_MIN);
  const float ce = BIAS ? 1.4426950408889634f : c;
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Bias rows of this lane, one per query tile (rows past the end read the
  // last row; they are never stored), and the bias values of one block:
  // bb[qt][kt][g] holds keys k0 + 32kt + 8g + 4*h2 + (0..3), i.e. score
  // registers 4g .. 4g+3 of sc[qt][kt]. A run never crosses the end of a
  // row: the row stride is a multiple of 4 and at least Nk, and in a block
  // that reaches past the keys every run start is clamped to the last run.
  const u16* brow[2] = {nullptr, nullptr};
  u32x2 bb[2][2][4];
  if constexpr (BIAS) {
    const u16* bg = static_cast<const u16*>(p.bias) + b * p.bias_sb + h * p.bias_sh;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
      brow[qt] = bg + static_cast<long>(min(wq0 + 32 * qt + j, Lq - 1)) * p.bias_sr + 4 * h2;
  }
  auto load_bias = [&](int jb) {
    const int k0 = key_base + jb * kBC;
    if (k0 + kBC <= Lk) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            bb[qt][kt][g] = *reinterpret_cast<const u32x2*>(brow[qt] + k0 + 32 * kt + 8 * g);
    } else {
      const int kmax = ((Lk - 1) & ~3) - 4 * h2;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            bb[qt][kt][g] =
                *reinterpret_cast<const u32x2*>(brow[qt] + min(k0 + 32 * kt + 8 * g, kmax));
    }
  };

  // Q fragments, held in registers for the whole key loop: the B operand of
  // S^T = K Q^T (column = query, 8 consecutive d values per lane). Query
  // tile qt of this wave covers rows wq0 + 32qt .. +31; this lane's row is
  // wq0 + 32qt + j.
  // They are read from the staged rows once this wave's K_0 and Q loads are
  // done (at most kLater of its loads still in flight) and the barrier has
  // made every wave's part visible. The barrier is a bare one: the fence of
  // __syncthreads would also wait for V_0 and K_1. A row past the end is
  // zero in LDS and its fragment is zeroed again below.
  bf16x8 qf[2][NC];
  u32x4 qv[2][NC];
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLater) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  {
    const unsigned char* qs = qst + wrow * T::kBytes;  // rows wq0 .. wq0+63
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int row = 32 * qt + j;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const int unit = (2 * cc + h2) ^ swz<T::kUnits>(row);
        qv[qt][cc] = *reinterpret_cast<const u32x4*>(qs + row * T::kRowBytes + unit * 16);
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const bool live = wq0 + 32 * qt + j < Lq;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const u32x4 v = live ? (qv[qt][cc] ^ qflip) : u32x4{0u, 0u, 0u, 0u};
      qf[qt][cc] = as_bf16x8(v);
      asm volatile("" : "+a"(qf[qt][cc]));  // move to an AGPR now
    }
  }
  asm volatile("s_nop 4" ::: "memory");     // AGPR writes before MFMA reads
  if constexpr (BIAS) {
    if (nblk_w > 0) load_bias(0);
  }

  f32x16 acc[2][ND];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < ND; ++t) {
      acc[qt][t] = f32x16{};
      asm volatile("" : "+a"(acc[qt][t]));
    }
  float m_run[2] = {-INFINITY, -INFINITY};  // running reference of x = c * s
  float l_run[2] = {0.f, 0.f};              // this lane's part of l (unrounded weights)
  // the same sum with each block's largest weight taken as the bf16 value
  // that P V multiplies: O = a / lt cancels the rounding of a row's dominant
  // weight (LSE keeps l)
  float lt_run[2] = {0.f, 0.f};

  // Per-lane constants of the LDS reads.
  const int k_row_off = j * T::kRowBytes;            // + kt * 32 rows
  const int k_swz = swz<T::kUnits>(j);               // same for row j + 32kt
  const int tr_i = lane & 15;                        // lane within a 16-lane group
  const int tr_dgrp = (lane >> 4) & 1;               // which 16 d-columns of the 32-row tile
  const int tr_h = lane >> 5;                        // which 4-key quarter of each 8 keys

  // K operand of S^T = K_j Q^T: 32 key rows (tile kt) x 16 d values (chunk cc).
  auto k_operand = [&](const unsigned char* ks, int kt, int cc) {
    const int unit = (2 * cc + h2) ^ k_swz;
    return *reinterpret_cast<const bf16x8*>(ks + kt * 32 * T::kRowBytes + k_row_off + unit * 16);
  };
  // V^T A operand for 32 d-rows (tile t) and 16 keys (chunk g): two
  // transposing reads give keys 16g + 8r + 4*tr_h + (0..3), r = 0, 1, at
  // d column 32t + 16*tr_dgrp + tr_i. Lane tr_i of each 16-lane group
  // supplies the address of 4 consecutive d values of key row
  // (16g + 8r + 4*tr_h + tr_i/4).
  auto v_operand = [&](const unsigned char* vs, int t, int g) {
    s16x4 half[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 16 * g + 8 * r + 4 * tr_h + (tr_i >> 2);
      const int unit = (4 * t + 2 * tr_dgrp + ((tr_i & 3) >> 1)) ^ swz<T::kUnits>(row);
      const int off = row * T::kRowBytes + unit * 16 + (tr_i & 1) * 8;
      half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs + off));
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T of one block: s[qt][kt][r] is the score of key
  // k0 + 32kt + 8(r/4) + 4*h2 + (r%4) against query wq0 + 32qt + j.
  f32x16 sa[2][2], sb[2][2];
  if (nblk_w > 0) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = k_operand(kw0, kt, cc);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          if (cc == 0) sa[qt][kt] = mfma_qk_first(a, qf[qt][cc]);
          else mfma_qk_acc(sa[qt][kt], a, qf[qt][cc]);
        }
      }
  }
  // Row maxima of the next block's scores, formed ahead of it (unmasked
  // blocks use them; masked ones form their own after the mask).
  float nmax[2] = {-INFINITY, -INFINITY};
  if constexpr (!BIAS) {
    mfma_result_guard();
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = sa[qt][0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sa[qt][0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[qt][1][r]);
      nmax[qt] = xhalf_max(mx);
    }
  }

  // One key block j: its scores sc are in registers. On entry the loads of
  // K_{j+1} and V_j are in flight (issued one block earlier).
  //   head: wait for them, barrier (every wave is done with block j-1, so
  //      the buffers of K_j and V_{j-1} are free), start the loads of
  //      K_{j+2} and V_{j+1} into those buffers;
  //   body: mask (then the row maxima of a masked block), reference; then
  //      the M steps of Plan<D>: the scores of block j+1 (sn) from K_{j+1},
  //      the exponentials of block j, and O^T += V_j^T P_j^T, one MFMA per
  //      step, so the matrix cores run while the vector unit computes
  //      exponentials; the last steps form the row maxima of sn. Operands
  //      are read from LDS kAhead steps early.
  constexpr int kAhead = 3;
  auto head = [&](auto par_tag, int jb) {
    constexpr int PAR = decltype(par_tag)::value;  // jb & 1
    unsigned char* k_free = PAR ? kb1 : kb0;        // K_j, consumed
    unsigned char* v_free = PAR ? vb0 : vb1;        // V_{j-1}, consumed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      if (jb + 2 < nbh[h])
        issue_tile<D>(kg, kstride, hk(h) + (jb + 2) * kBC, Lk, k_free + h * T::kBytes, tid, w);
      if (jb + 1 < nbh[h])
        issue_tile<D>(vg, kstride, hk(h) + (jb + 1) * kBC, Lk, v_free + h * T::kBytes, tid, w);
    }
  };
  auto body = [&](auto par_tag, int jb, f32x16(&sc)[2][2], f32x16(&sn)[2][2]) {
    constexpr int PAR = decltype(par_tag)::value;  // jb & 1
    const unsigned char* k_next = PAR ? kw0 : kw1;  // K_{j+1}
    const unsigned char* v_cur = PAR ? vw1 : vw0;   // V_j
    if (jb >= nblk_w) return;
    const int k0 = key_base + jb * kBC;
    // the last score MFMAs of sc may still be in flight (without a bias the
    // previous block's last steps already read every score register)
    if constexpr (BIAS) mfma_result_guard();
    bool masked = false;

    // LDS operands: score operand p (K tile p/NC, d-chunk p%NC) is first used
    // at step qk_first(p); value operand (t, g) at pv_start(g) + 2t.
    bf16x8 kop[2 * NC];
    bf16x8 vop[4][ND];
    auto load_for_step = [&](auto S) {
      static_for<2 * NC>([&](auto P) {
        if constexpr (PL::qk_first(P) == S) kop[P] = k_operand(k_next, P / NC, P % NC);
      });
      static_for<4>([&](auto G) {
        static_for<ND>([&](auto TT) {
          if constexpr (PL::pv_start(G) + 2 * TT == S) vop[G][TT] = v_operand(v_cur, TT, G);
        });
      });
    };

    // Only blocks that reach past the end of the keys or cross the causal
    // diagonal of this wave are masked: visible iff key <= lim, with
    // key - k0 - 4*h2 = 32kt + 8(r/4) + (r%4). c >= FLT_MIN keeps
    // 2^(c * -inf - m) = 0.
    if constexpr (!WIN) {
      if ((k0 + kBC > Lk) || (CAUSAL && k0 + kBC - 1 > wq0)) {
        masked = true;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int qrow = wq0 + 32 * qt + j;
          const int lim = (CAUSAL ? min(Lk - 1, qrow) : Lk - 1) - k0 - 4 * h2;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sc[qt][kt][r] = (32 * kt + 8 * (r >> 2) + (r & 3) <= lim) ? sc[qt][kt][r] : -INFINITY;
        }
      }
    } else {  // also the window's edges: visible iff lim_lo <= key - k0 - 4*h2 <= lim
      if ((k0 + kBC > Lk) || (CAUSAL && k0 + kBC - 1 > wq0) ||
          (p.win_left >= 0 && k0 < wq0 + 63 - p.win_left) ||
          (p.win_right >= 0 && k0 + kBC - 1 > wq0 + p.win_right)) {
        masked = true;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int qrow = wq0 + 32 * qt + j;
          int hi = CAUSAL ? min(Lk - 1, qrow) : Lk - 1;
          if (p.win_right >= 0) hi = min(hi, qrow + p.win_right);
          const int lo = p.win_left >= 0 ? qrow - p.win_left : 0;
          const int lim = hi - k0 - 4 * h2;
          const int lim_lo = lo - k0 - 4 * h2;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 32 * kt + 8 * (r >> 2) + (r & 3);
              sc[qt][kt][r] = (off <= lim && off >= lim_lo) ? sc[qt][kt][r] : -INFINITY;
            }
        }
      }
    }
    if constexpr (BIAS) {  // t = cn * s + b; masked scores stay -inf
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wd = bb[qt][kt][g][e >> 1];
              const float bv = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
              sc[qt][kt][4 * g + e] = __builtin_fmaf(sc[qt][kt][4 * g + e], cn, bv);
            }
      if (jb + 1 < nblk_w) load_bias(jb + 1);
    }
    float mb[2], smax[2];
    bool up = false;
    if (BIAS || masked) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = fmaxf(sc[qt][0][0], sc[qt][0][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[qt][0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[qt][1][r]);
        nmax[qt] = xhalf_max(mx);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      smax[qt] = nmax[qt];
      mb[qt] = smax[qt] * ce;
      // A row's first visible block sets its reference (its accumulator and
      // denominator are still zero); later raises need the rescale.
      if (m_run[qt] == -INFINITY) m_run[qt] = mb[qt];
      up = up || (mb[qt] > m_run[qt] + kRaise);
    }
    if (__any(up)) {  // wave-uniform, rare
      mfma_result_guard();  // the last P V MFMAs may still be in flight
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        // raise each row of this wave to its block maximum (alpha = 1 for
        // rows that do not gain)
        const float m_new = fmaxf(m_run[qt], mb[qt]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
        m_run[qt] = m_new;
        l_run[qt] *= alpha;
        lt_run[qt] *= alpha;
#pragma unroll
        for (int t = 0; t < ND; ++t) acc[qt][t] = scale_via_scratch(acc[qt][t], alpha);
      }
      asm volatile("s_nop 1" ::: "memory");  // AGPR writes before MFMA reads
    }
    static_for<kAhead>(load_for_step);
    // A row that has seen no visible key keeps m = -inf; 0 is used as the
    // reference then, so that 2^(-inf - ref) = 0 instead of NaN.
    float m_ref[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) m_ref[qt] = (m_run[qt] == -INFINITY) ? 0.f : m_run[qt];
    // bf16 rounding residual of each row's largest weight of this block (the
    // same arithmetic as that weight's own exponential below)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float pm = __builtin_amdgcn_exp2f(__builtin_fmaf(smax[qt], ce, -m_ref[qt]));
      lt_run[qt] += static_cast<float>(static_cast<__bf16>(pm)) - pm;
    }

    // P^T as the B operand of O^T += V^T P^T: 16-key chunk g takes score
    // registers 8(g%2) .. 8(g%2)+7 of key tile g/2, i.e. keys
    // 16g + 8(s/4) + 4*h2 + (s%4) for slot s. Element e of the block is
    // chunk e/16, query tile (e/8)%2, slot e%8.
    float rs[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    bf16x8 pb[2][4];
    float tmax[2];
    static_for<PL::M>([&](auto S) {
      if constexpr (S + kAhead < PL::M) load_for_step(std::integral_constant<int, S + kAhead>{});
      constexpr int g = PL::pv_chunk(S);
      if constexpr (g < 0) {
        constexpr int q = PL::qk_index(S);
        constexpr int qt = q & 1, pp = q >> 1, kt = pp / NC, cc = pp % NC;
        if constexpr (cc == 0) sn[qt][kt] = mfma_qk_first(kop[pp], qf[qt][cc]);
        else mfma_qk_acc(sn[qt][kt], kop[pp], qf[qt][cc]);
      } else {
        constexpr int i = S - PL::pv_start(g);
        constexpr int t = i >> 1, qt = i & 1;
        acc[qt][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[g][t], pb[qt][g], acc[qt][t],
                                                             0, 0, 0);
        asm volatile("" : "+a"(acc[qt][t]));  // the accumulator lives in AGPRs
      }
      if constexpr (!BIAS && S >= PL::M - 2 * ND) {
        // steps without exponentials: row maxima of the next block, a
        // score tile (qt, kt) per ND/2 steps, kt = 0 first
        constexpr int i = S - (PL::M - 2 * ND), spt = ND / 2;
        constexpr int tt = i / spt, part = i % spt, qt = tt & 1, kt = tt >> 1;
        constexpr int r0 = part * 16 / spt, r1 = (part + 1) * 16 / spt;
        static_assert(kt == 0 || S - PL::last_qk_step(kt, qt) >= 4, "score results ready");
        if constexpr (tt == 0 && part == 0) { tmax[0] = -INFINITY; tmax[1] = -INFINITY; }
        static_for<r1 - r0>([&](auto R) { tmax[qt] = fmaxf(tmax[qt], sn[qt][kt][r0 + R]); });
        if constexpr (kt == 1 && part == spt - 1) nmax[qt] = xhalf_max(tmax[qt]);
      }
      constexpr int e0 = PL::first_elem(S);
      static_for<PL::first_elem(S + 1) - e0>([&](auto EI) {
        constexpr int E = e0 + EI;
        if constexpr (E < 64) {
          constexpr int eg = E / 16, eq = (E / 8) & 1, es = E % 8;
          const float x = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sc[eq][eg >> 1][8 * (eg & 1) + es], ce, -m_ref[eq]));
          rs[eq][eg] += x;
          pb[eq][eg][es] = static_cast<__bf16>(x);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      l_run[qt] += (rs[qt][0] + rs[qt][1]) + (rs[qt][2] + rs[qt][3]);
      lt_run[qt] += (rs[qt][0] + rs[qt][1]) + (rs[qt][2] + rs[qt][3]);
    }
  };

  // Key loop, unrolled by two so every LDS address has a fixed buffer. A
  // wave's last computed block also forms the scores of the block after it
  // (from whatever the K buffer holds, discarded): one branch-free region
  // for every block.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int jb = 0; jb < nblk; jb += 2) {
    head(P0{}, jb);
    body(P0{}, jb, sa, sb);
    if (jb + 1 >= nblk) break;
    head(P1{}, jb + 1);
    body(P1{}, jb + 1, sb, sa);
  }

  // Epilogue: o = a / l, rounded once to bf16; LSE = ln(2) * (m + log2 l).
  mfma_result_guard();  // the last P V MFMAs may still be in flight
  // SPLIT: the second key half's (m, l, a) of each lane, staged in the
  // (now free) K and V buffers of the wave pair's row group.
  const float* xa = reinterpret_cast<const float*>(wrow ? kb1 : kb0);  // 2*ND*16 per lane
  const float* xm = reinterpret_cast<const float*>(wrow ? vb1 : vb0);  // m, l per query tile
  if constexpr (SPLIT) {
    __syncthreads();  // every wave is done with the K/V buffers
    if (half == 1) {
      float* ya = reinterpret_cast<float*>(wrow ? kb1 : kb0);
      float* ym = reinterpret_cast<float*>(wrow ? vb1 : vb0);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          const f32x16 a = read_agpr(acc[qt][t]);
#pragma unroll
          for (int r = 0; r < 16; ++r) ya[((qt * ND + t) * 16 + r) * 64 + lane] = a[r];
        }
        ym[qt * 64 + lane] = m_run[qt];
        ym[(2 + qt) * 64 + lane] = l_run[qt];
        ym[(4 + qt) * 64 + lane] = lt_run[qt];
      }
    }
    __syncthreads();
    if (half == 1) return;
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    f32x16 o_t[ND];
#pragma unroll
    for (int t = 0; t < ND; ++t) o_t[t] = read_agpr(acc[qt][t]);
    if constexpr (SPLIT) {  // both parts to the common reference max(m0, m1)
      const float m0 = m_run[qt];
      const float m1 = xm[qt * 64 + lane];
      const float mm = fmaxf(m0, m1);
      const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
      const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      l_run[qt] = l_run[qt] * a0 + xm[(2 + qt) * 64 + lane] * a1;
      lt_run[qt] = lt_run[qt] * a0 + xm[(4 + qt) * 64 + lane] * a1;
      m_run[qt] = mm;
#pragma unroll
      for (int t = 0; t < ND; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o_t[t][r] = o_t[t][r] * a0 + xa[((qt * ND + t) * 16 + r) * 64 + lane] * a1;
    }
    const int qrow = wq0 + 32 * qt + j;
    const float l_tot = xhalf_sum(l_run[qt]);
    const float lt_tot = xhalf_sum(lt_run[qt]);
    if (qrow < Lq) {
      // o = a / lt, LSE from l
      const float inv = l_tot > 0.f ? 1.f / lt_tot : 0.f;
      u16* og = static_cast<u16*>(p.o) + (q_tok0 + qrow) * qstride + static_cast<long>(h) * D;
#pragma unroll
      for (int t = 0; t < ND; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = static_cast<__bf16>(o_t[t][4 * g + e] * inv);
          *reinterpret_cast<bf16x4*>(og + 32 * t + 8 * g + 4 * h2) = o4;
        }
      if (h2 == 0)
        p.lse[lse_base + qrow] = l_tot > 0.f ? (m_run[qt] + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

// One object file per (head width, causal) pair: the build compiles this
// source once for each, with FA_BF16_D in {64, 128} and FA_BF16_CAUSAL in
// {0, 1}, so the four kernels compile in parallel.
template <int D, bool CAUSAL>
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  const int n_qt = (p.nq + kBR - 1) / kBR;
  const unsigned grid = static_cast<unsigned>(n_qt) * p.hq * p.batch;
  const bool plain = p.bias == nullptr && p.win_left < 0 && p.win_right < 0;
  if constexpr (!CAUSAL) {
    // A grid of 256-row tiles that leaves compute units idle: 128-row
    // workgroups whose wave pairs split the keys, twice as many of them.
    if (plain && grid <= static_cast<unsigned>(p.num_cus)) {
      const int n_qt2 = (p.nq + kBR / 2 - 1) / (kBR / 2);
      const unsigned grid2 = static_cast<unsigned>(n_qt2) * p.hq * p.batch;
      hipLaunchKernelGGL((fwd_bf16_kernel<D, false, false, false, true>), dim3(grid2),
                         dim3(kThreads), 0, stream, p, n_qt2);
      return hipGetLastError();
    }
  }
  if (p.bias != nullptr)  // the host never combines a bias with a window
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, true, false>), dim3(grid),
                       dim3(kThreads), 0, stream, p, n_qt);
  else if (!plain)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, true, false, false>), dim3(grid),
                       dim3(kThreads), 0, stream, p, n_qt);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, false, false, false>), dim3(grid),
                       dim3(kThreads), 0, stream, p, n_qt);
  return hipGetLastError();
}

#if !defined(FA_BF16_D) || !defined(FA_BF16_CAUSAL)
#error "compile with -DFA_BF16_D=64|128 -DFA_BF16_CAUSAL=0|1"
#endif
template hipError_t launch_fwd_bf16<FA_BF16_D, (FA_BF16_CAUSAL != 0)>(const FwdParams&,
                                                                    hipStream_t);

}  // namespace fa
