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
// Work decomposition (one workgroup = 4 wavefronts of 64 lanes):
//   * a workgroup owns 128 query rows of one (batch or sequence, q-head);
//     wavefront w owns rows 32w .. 32w+31 of that tile;
//   * K/V blocks of 64 keys stream through LDS in two stages: while the
//     waves compute on block j, buffer-to-LDS loads (no VGPR staging) bring
//     block j+1 into the other stage; rows past the end of the sequence lie
//     outside the buffer range and arrive as zeros;
//   * each wave computes the transposed score block S^T = K_j Q_i^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 32 scores of ONE query row:
//     row max and row sum are lane-local plus one v_permlane32_swap with the
//     other half-wave, and the rescale factor is a per-lane scalar;
//   * the output is accumulated transposed as well, O^T += V_j^T P^T: P^T
//     feeds the B operand straight from the score registers, and V^T comes
//     from the row-major V tile through ds_read_b64_tr_b16 transposing reads.
//   * K/V tiles are stored with an XOR swizzle of the 16-byte units of each
//     row so that the score reads (16 consecutive rows, same column) and the
//     transposing V reads (4 consecutive rows, 64 bytes each) spread over the
//     LDS banks.
//
// Reference point of the exponentials. The invariant of "Carry the
// Normalizer" holds for ANY common reference m of l and a: o = a / l and
// LSE = m + log l do not depend on it, as long as nothing overflows. The
// kernel raises m to the new block maximum only when some row of the wave
// would otherwise see a weight above 2^kLazy; otherwise it keeps m. Each
// row's first block sets m, so every weight stays below 2^kLazy (far inside
// the float32 range), and the accumulator rescale, which costs one multiply
// per accumulator register, becomes rare.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <type_traits>
#include <utility>

#include "fa_launch.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kBR = kBf16TileRows;  // query rows per workgroup
constexpr int kBC = 64;             // keys per K/V block
constexpr int kThreads = 256;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.f;        // keep m while the block max is <= m + 8
// Third descriptor word of a raw buffer resource on gfx9-family parts
// (32-bit data format, no swizzle); the range check uses num_records.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
  static constexpr int kUnits = D / 8;               // 16-byte units per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kBC * kRowBytes;     // one K or V tile
  static constexpr int kLoads = kBC * kUnits / kThreads;  // loads per lane per tile
};

// XOR swizzle of the 16-byte unit index within a row.
template <int UNITS>
__device__ __forceinline__ int swz(int row) {
  if constexpr (UNITS == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

__device__ __forceinline__ u32x4 ld16(const u16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max and sum of a value with the same lane of the other half-wave
__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Compile-time loop: f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction plan of one key block for one wave. The block has M matrix
// steps: 2*NC score MFMAs of the NEXT block (two 32-key tiles x NC d-chunks)
// and 4*ND P V MFMAs of THIS block (four 16-key chunks x ND d-tiles). The 32
// exponentials of this block (one per score register of the lane) are
// spread evenly over the first M - ND steps; P V chunk g is placed right
// after the step that finishes its 8 probabilities, and score MFMAs fill the
// remaining steps.
template <int D>
struct Plan {
  static constexpr int NC = D / 16;
  static constexpr int ND = D / 32;
  static constexpr int M = 2 * NC + 4 * ND;
  static constexpr int VS = M - ND;  // steps that carry exponentials
  static constexpr int elem_step(int e) { return e * VS / 32; }
  static constexpr int pv_start(int g) { return elem_step(8 * g + 7) + 1; }
  // -1 if step s is a score MFMA, else the P V chunk it belongs to
  static constexpr int pv_chunk(int s) {
    for (int g = 0; g < 4; ++g)
      if (s >= pv_start(g) && s < pv_start(g) + ND) return g;
    return -1;
  }
  // index of the score MFMA at step s (number of score steps before it)
  static constexpr int qk_index(int s) {
    int n = 0;
    for (int i = 0; i < s; ++i) n += pv_chunk(i) < 0 ? 1 : 0;
    return n;
  }
  static constexpr bool valid() {
    int qk = 0;
    for (int s = 0; s < M; ++s) qk += pv_chunk(s) < 0 ? 1 : 0;
    for (int g = 0; g + 1 < 4; ++g)
      if (pv_start(g + 1) < pv_start(g) + ND) return false;
    return qk == 2 * NC && pv_start(3) + ND == M;
  }
};
static_assert(Plan<128>::valid() && Plan<64>::valid(), "block plan");

// Start the loads of one 64-key tile of K or V (keys k0 .. k0+63) into LDS.
// Each lane moves kLoads 16-byte units; a wave instruction fills 1 KiB of
// contiguous LDS. Rows at or past Lk are outside the buffer range and are
// written as zeros.
template <int D>
__device__ __forceinline__ void issue_tile(const u16* g, long stride, int k0, int Lk,
                                           unsigned char* dst, int tid, int w) {
  using T = Tile<D>;
  const int rows = min(Lk - k0, kBC);
  const uint32_t stride_b = static_cast<uint32_t>(stride * 2);
  const uint32_t nrec = static_cast<uint32_t>(rows - 1) * stride_b + T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(g + static_cast<long>(k0) * stride), 0, nrec, kBufferFlags);
#pragma unroll
  for (int it = 0; it < T::kLoads; ++it) {
    const int u = it * kThreads + tid;
    const int row = u / T::kUnits;
    const int gc = (u % T::kUnits) ^ swz<T::kUnits>(row);
    const uint32_t voff = row * stride_b + gc * 16;
    const int lds_off = (it * kThreads + w * 64) * 16;  // wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + lds_off), 16, voff, 0, 0, 0);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdParams p, int n_qt) {
  using T = Tile<D>;
  constexpr int NC = D / 16;  // 16-wide d chunks of the QK^T contraction
  constexpr int ND = D / 32;  // 32-row tiles of O^T
  // K runs one block ahead of V: block j's scores are formed while block
  // j-1's probabilities meet V, so each tensor has its own two buffers.
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int u = (t2 % upx) * 8 + x;
    tile = n_qt - 1 - t2 / upx;
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
  const int q0 = tile * kBR;
  if (q0 >= Lq) return;

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const u16* qg = static_cast<const u16*>(p.q) + q_tok0 * qstride + static_cast<long>(h) * D;
  const u16* kg = static_cast<const u16*>(p.k) + k_tok0 * kstride + static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + k_tok0 * kstride + static_cast<long>(kvh) * D;

  int kend = Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBR, Lq));
  const int nblk = (kend + kBC - 1) / kBC;
  if (nblk > 0) {
    issue_tile<D>(kg, kstride, 0, Lk, kb0, tid, w);
    issue_tile<D>(vg, kstride, 0, Lk, vb0, tid, w);
    if (nblk > 1) issue_tile<D>(kg, kstride, kBC, Lk, kb1, tid, w);
  }

  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + j;     // this lane's query row

  // A negative scale is applied by negating Q (exact in bf16), so that the
  // base-2 factor c below is >= 0 and max(c*s) = c*max(s).
  const float c = fmaxf(fabsf(p.scale_log2), FLT_MIN);
  const uint32_t qflip = p.scale_log2 < 0.f ? 0x80008000u : 0u;

  // Q fragment, held in registers for the whole key loop: the B operand of
  // S^T = K Q^T (column = query, 8 consecutive d values per lane).
  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < Lq) v = ld16(qg + static_cast<long>(qrow) * qstride + 16 * cc + 8 * h2) ^ qflip;
    qf[cc] = as_bf16x8(v);
  }

  f32x16 acc[ND];
#pragma unroll
  for (int t = 0; t < ND; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY;  // running reference of x = c * s
  float l_run = 0.f;        // this lane's part of the running denominator

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
  // V^T A operand for 32 d-rows (tile t) and 16 keys (chunk cc): two
  // transposing reads give keys 16cc + 8r + 4*tr_h + (0..3), r = 0, 1, at
  // d column 32t + 16*tr_dgrp + tr_i. Lane tr_i of each 16-lane group
  // supplies the address of 4 consecutive d values of key row
  // (16cc + 8r + 4*tr_h + tr_i/4).
  auto v_operand = [&](const unsigned char* vs, int t, int cc) {
    s16x4 half[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = 16 * cc + 8 * r + 4 * tr_h + (tr_i >> 2);
      const int unit = (4 * t + 2 * tr_dgrp + ((tr_i & 3) >> 1)) ^ swz<T::kUnits>(row);
      const int off = row * T::kRowBytes + unit * 16 + (tr_i & 1) * 8;
      half[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vs + off));
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T for two 32-key tiles of one block: s[kt][r] is the score of key
  // k0 + 32kt + 8(r/4) + 4*h2 + (r%4) against query qrow.
  f32x16 sa[2], sb[2];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nblk > 0) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sa[kt] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        sa[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(kb0, kt, cc), qf[cc], sa[kt],
                                                         0, 0, 0);
    }
  }

  // One key block j: its scores sc are in registers. On entry the loads of
  // K_{j+1} and V_j are in flight (issued one block earlier).
  //   1. wait for them, barrier (every wave is done with block j-1, so the
  //      buffers of K_j and V_{j-1} are free), start the loads of K_{j+2}
  //      and V_{j+1} into those buffers;
  //   2. mask, row maximum, reference update (rare rescale);
  //   3. the M steps of Plan<D>: the scores of block j+1 (sn) from K_{j+1},
  //      the exponentials of block j, and O^T += V_j^T P_j^T, one MFMA per
  //      step, so the matrix cores run while the vector unit computes
  //      exponentials. Operands are read from LDS kAhead steps early.
  using PL = Plan<D>;
  constexpr int kAhead = 2;
  auto iter = [&](auto par_tag, int jb, f32x16(&sc)[2], f32x16(&sn)[2]) {
    constexpr int PAR = decltype(par_tag)::value;  // jb & 1
    unsigned char* k_next = PAR ? kb0 : kb1;        // K_{j+1}
    unsigned char* k_free = PAR ? kb1 : kb0;        // K_j, consumed
    unsigned char* v_cur = PAR ? vb1 : vb0;         // V_j
    unsigned char* v_free = PAR ? vb0 : vb1;        // V_{j-1}, consumed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (jb + 2 < nblk) issue_tile<D>(kg, kstride, (jb + 2) * kBC, Lk, k_free, tid, w);
    if (jb + 1 < nblk) issue_tile<D>(vg, kstride, (jb + 1) * kBC, Lk, v_free, tid, w);
    const int k0 = jb * kBC;

    bf16x8 opnd[PL::M];
    auto load_operand = [&](auto S) {
      constexpr int g = PL::pv_chunk(S);
      if constexpr (g < 0) {
        constexpr int q = PL::qk_index(S);
        opnd[S] = k_operand(k_next, q & 1, q >> 1);
      } else {
        opnd[S] = v_operand(v_cur, S - PL::pv_start(g), g);
      }
    };
    static_for<kAhead>(load_operand);

    // Only blocks that reach past the end of the keys or cross the causal
    // diagonal are masked: visible iff key <= lim, with key - k0 - 4*h2 =
    // 32kt + 8(r/4) + (r%4). c >= FLT_MIN keeps 2^(c * -inf - m) = 0.
    if ((k0 + kBC > Lk) || (CAUSAL && k0 + kBC - 1 > wq0)) {
      const int lim = (CAUSAL ? min(Lk - 1, qrow) : Lk - 1) - k0 - 4 * h2;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kt][r] = (32 * kt + 8 * (r >> 2) + (r & 3) <= lim) ? sc[kt][r] : -INFINITY;
    }
    float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    const float mb = xhalf_max(mx) * c;
    // The reference point moves only when some row of the wave gains more
    // than kLazy over it (wave-uniform decision).
    const bool raise = __any(mb > m_run + kLazy);
    if (raise) {
      const float m_new = fmaxf(m_run, mb);
      // A row that has seen no visible key keeps m = -inf; 0 is used as the
      // reference then, so that 2^(-inf - ref) = 0 instead of NaN.
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < ND; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    }
    const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;

    // P^T as the B operand of O^T += V^T P^T: 16-key chunk g takes score
    // registers 8(g%2) .. 8(g%2)+7 of tile g/2, i.e. keys
    // 16g + 8(s/4) + 4*h2 + (s%4) for slot s.
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8 pb[4];
    static_for<PL::M>([&](auto S) {
      if constexpr (S + kAhead < PL::M) load_operand(std::integral_constant<int, S + kAhead>{});
      constexpr int g = PL::pv_chunk(S);
      if constexpr (g < 0) {
        constexpr int q = PL::qk_index(S);
        constexpr int kt = q & 1, cc = q >> 1;
        sn[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[S], qf[cc],
                                                         cc == 0 ? f32x16{} : sn[kt], 0, 0, 0);
      } else {
        constexpr int t = S - PL::pv_start(g);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[S], pb[g], acc[t], 0, 0, 0);
      }
      static_for<32>([&](auto E) {
        if constexpr (PL::elem_step(E) == S) {
          constexpr int eg = E / 8, es = E % 8;
          const float x = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sc[eg >> 1][8 * (eg & 1) + es], c, -m_ref));
          rs[eg] += x;
          pb[eg][es] = static_cast<__bf16>(x);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);  // from the unrounded float32 P
  };

  // The last block also forms the scores of a block past the end (from the
  // stale K buffer, discarded): one branch-free loop body for every block.
  for (int jb = 0; jb < nblk; jb += 2) {
    iter(std::integral_constant<int, 0>{}, jb, sa, sb);
    if (jb + 1 >= nblk) break;
    iter(std::integral_constant<int, 1>{}, jb + 1, sb, sa);
  }

  // Epilogue: o = a / l, rounded once to bf16; LSE = ln(2) * (m + log2 l).
  const float l_tot = xhalf_sum(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    u16* og = static_cast<u16*>(p.o) + (q_tok0 + qrow) * qstride + static_cast<long>(h) * D;
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = static_cast<__bf16>(acc[t][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(og + 32 * t + 8 * g + 4 * h2) = o4;
      }
    if (h2 == 0)
      p.lse[lse_base + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int n_qt = (p.nq + kBR - 1) / kBR;
  const unsigned grid = static_cast<unsigned>(n_qt) * p.hq * p.batch;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(kThreads), 0, stream, p, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
