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
//   * K/V blocks of 64 keys are staged in LDS and shared by the 4 waves;
//   * each wave computes the transposed score block S^T = K_j Q_i^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 32 scores of ONE query row
//     (its column): row max and row sum are lane-local plus one exchange with
//     lane ^ 32, and the rescale factor is a per-lane scalar;
//   * the output is accumulated transposed as well, O^T += V_j^T P^T, so
//     P^T feeds the B operand straight from the score registers and V^T is
//     read from LDS, where V is stored transposed with keys permuted to match
//     the score registers' key order.
#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

constexpr int kBR = kBf16TileRows;  // query rows per workgroup
constexpr int kBC = 64;             // keys per K/V block
constexpr int kThreads = 256;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 ld16(const u16* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Position of key k (0..63 within a block) inside a row of the transposed V
// tile. Lanes 0-31 of a 32x32x16 score tile hold keys {0-3, 8-11} of every
// 16-key group and lanes 32-63 hold keys {4-7, 12-15}; storing V^T in that
// order lets each lane read its 8 keys as one 16-byte LDS load.
__device__ __forceinline__ int vt_pos(int k) {
  const int grp = k >> 4, u = k & 15;
  const int half = (u >> 2) & 1;
  const int slot = ((u >> 3) << 2) | (u & 3);
  return (grp << 4) | (half << 3) | slot;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(FwdParams p, int n_qt) {
  constexpr int KSTR = D + 8;    // K tile row stride in LDS (elements)
  constexpr int VSTR = kBC + 8;  // V^T tile row stride in LDS (elements)
  constexpr int NC = D / 16;     // 16-wide d chunks of the QK^T contraction
  constexpr int ND = D / 32;     // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) u16 ks[kBC * KSTR];
  __shared__ __attribute__((aligned(16))) u16 vt[D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int j = lane & 31;   // query column within the wave / key row in A
  const int h2 = lane >> 5;  // which half of the wave

  // Heaviest query tiles first: with the causal mask tile t costs ~t+1
  // blocks, so starting from the last tile shortens the tail.
  const int bh = p.hq * p.batch;
  const int tile = n_qt - 1 - static_cast<int>(blockIdx.x / bh);
  const int rem = static_cast<int>(blockIdx.x % bh);
  const int b = rem / p.hq;
  const int h = rem % p.hq;
  const int kvh = h / (p.hq / p.hkv);

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

  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + j;     // this lane's query row

  // Q fragment, held in registers for the whole key loop: the B operand of
  // S^T = K Q^T (column = query, 8 consecutive d values per lane).
  bf16x8 qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (qrow < Lq) v = ld16(qg + static_cast<long>(qrow) * qstride + 16 * c + 8 * h2);
    qf[c] = as_bf16x8(v);
  }

  int kend = Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBR, Lq));
  const int nblk = (kend + kBC - 1) / kBC;

  f32x16 acc[ND];
#pragma unroll
  for (int t = 0; t < ND; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY;  // running max of x = s * scale * log2(e)
  float l_run = 0.f;        // this lane's part of the running denominator

  for (int blk = 0; blk < nblk; ++blk) {
    const int k0 = blk * kBC;
    __syncthreads();  // the previous block's LDS reads are done
    // Stage K (row-major) and V (transposed, permuted) for keys k0..k0+63.
    // Keys past the end are zero-filled so that masked lanes multiply zeros.
#pragma unroll
    for (int c = tid; c < kBC * (D / 8); c += kThreads) {
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      const int key = k0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u};
      u32x4 vv = {0u, 0u, 0u, 0u};
      if (key < Lk) {
        kv = ld16(kg + static_cast<long>(key) * kstride + col);
        vv = ld16(vg + static_cast<long>(key) * kstride + col);
      }
      *reinterpret_cast<u32x4*>(&ks[row * KSTR + col]) = kv;
      const int pos = vt_pos(row);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[(col + 2 * e) * VSTR + pos] = static_cast<u16>(vv[e] & 0xFFFFu);
        vt[(col + 2 * e + 1) * VSTR + pos] = static_cast<u16>(vv[e] >> 16);
      }
    }
    __syncthreads();
    if (CAUSAL && k0 > wq0 + 31) continue;  // every key is after every row

    // S^T for two 32-key tiles: st[kt][r] is the score of key
    // k0 + 32kt + 8(r/4) + 4*h2 + (r%4) against query qrow.
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const bf16x8 a = as_bf16x8(ld16(&ks[(kt * 32 + j) * KSTR + 16 * c + 8 * h2]));
        st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], st[kt], 0, 0, 0);
      }
    }

    float x[32];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kt * 16 + r] = st[kt][r] * p.scale_log2;

    const bool need_mask = (k0 + kBC > Lk) || (CAUSAL && k0 + kBC - 1 > wq0);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * h2 + (r & 3);
          const bool vis = key < Lk && (!CAUSAL || key <= qrow);
          if (!vis) x[kt * 16 + r] = -INFINITY;
        }
    }

    float mb = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mb = fmaxf(mb, x[i]);
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float m_new = fmaxf(m_run, mb);
    // A row that has seen no visible key yet keeps m = -inf; use 0 as the
    // reference so that 2^(-inf - ref) = 0 instead of NaN.
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
      rs += x[i];
    }
    l_run = l_run * alpha + rs;  // from the unrounded float32 P
    m_run = m_new;
    if (!__all(alpha == 1.f)) {
#pragma unroll
      for (int t = 0; t < ND; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    }

    // P^T as the B operand of O^T += V^T P^T: 16-key chunk c takes score
    // registers 8(c%2) .. 8(c%2)+7 of tile c/2 (keys 16c + {0-3, 8-11} on
    // lanes 0-31, 16c + {4-7, 12-15} on lanes 32-63; vt_pos matches).
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int s = 0; s < 8; ++s) pb[c][s] = static_cast<__bf16>(x[(c >> 1) * 16 + 8 * (c & 1) + s]);

#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 a = as_bf16x8(ld16(&vt[(32 * t + j) * VSTR + 16 * c + 8 * h2]));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], acc[t], 0, 0, 0);
      }
  }

  // Epilogue: o = a / l, rounded once to bf16; LSE = ln(2) * (m + log2 l).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
