// Exact tiled attention forward in float32 throughout (inputs, scores,
// softmax state, accumulation and output), for gfx950.
//
// Same schedule as the bf16 kernel ("Understanding FlashAttention Pt 1",
// section 1.2; "Softmax does not need the matrix", section "Carry the
// Normalizer"), on the vector ALUs: one lane owns one query row and carries
// (m, l, a) for it while 16-key blocks of K and V stream through LDS.
// This path serves small float32 problems where no bf16 rounding is
// acceptable; it is not tuned for throughput.
#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBQ = kFp32TileRows;  // query rows per workgroup (one wave)
constexpr int kBK = 16;             // keys per block (LDS stays under 64 KiB at d = 128)
constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBQ) void fwd_fp32_kernel(FwdParams p, int n_qt) {
  __shared__ float qs[kBQ][D + 1];  // +1: each lane reads its own row
  __shared__ float kt[kBK][D];      // read as broadcasts
  __shared__ float vs[kBK][D];

  const int lane = threadIdx.x;
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
  const int q0 = tile * kBQ;
  if (q0 >= Lq) return;

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const float* qg = static_cast<const float*>(p.q) + q_tok0 * qstride + static_cast<long>(h) * D;
  const float* kg = static_cast<const float*>(p.k) + k_tok0 * kstride + static_cast<long>(kvh) * D;
  const float* vg = static_cast<const float*>(p.v) + k_tok0 * kstride + static_cast<long>(kvh) * D;

  for (int i = lane; i < kBQ * D; i += kBQ) {
    const int r = i / D, c = i % D;
    qs[r][c] = (q0 + r < Lq) ? qg[static_cast<long>(q0 + r) * qstride + c] : 0.f;
  }
  const int qrow = q0 + lane;

  int kend = Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBQ, Lq));

  float acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) acc[t] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int k0 = 0; k0 < kend; k0 += kBK) {
    __syncthreads();
    for (int i = lane; i < kBK * D; i += kBQ) {
      const int r = i / D, c = i % D;
      const int key = k0 + r;
      const bool in = key < Lk;
      kt[r][c] = in ? kg[static_cast<long>(key) * kstride + c] : 0.f;
      vs[r][c] = in ? vg[static_cast<long>(key) * kstride + c] : 0.f;
    }
    __syncthreads();

    float x[kBK];
    float mb = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kBK; ++jj) {
      float dot = 0.f;
#pragma unroll 16
      for (int t = 0; t < D; ++t) dot = fmaf(qs[lane][t], kt[jj][t], dot);
      const int key = k0 + jj;
      const bool vis = key < Lk && (!CAUSAL || key <= qrow);
      x[jj] = vis ? dot * p.scale_log2 : -INFINITY;
      mb = fmaxf(mb, x[jj]);
    }
    const float m_new = fmaxf(m_run, mb);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_ref);
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < kBK; ++jj) {
      x[jj] = exp2f(x[jj] - m_ref);
      rs += x[jj];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < D; ++t) {
      float a = acc[t] * alpha;
#pragma unroll
      for (int jj = 0; jj < kBK; ++jj) a = fmaf(x[jj], vs[jj][t], a);
      acc[t] = a;
    }
  }

  if (qrow < Lq) {
    float* og = static_cast<float*>(p.o) + (q_tok0 + qrow) * qstride + static_cast<long>(h) * D;
#pragma unroll
    for (int t = 0; t < D; ++t) og[t] = l_run > 0.f ? acc[t] / l_run : 0.f;
    p.lse[lse_base + qrow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int n_qt = (p.nq + kBQ - 1) / kBQ;
  const unsigned grid = static_cast<unsigned>(n_qt) * p.hq * p.batch;
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3(grid), dim3(kBQ), 0, stream, p, n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
