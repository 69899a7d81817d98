// Exact tiled attention forward in float32 throughout (inputs, scores,
// softmax state, accumulation and output), for gfx950.
//
// Same schedule as the bf16 kernel ("Understanding FlashAttention Pt 1",
// section 1.2; "Softmax does not need the matrix", section "Carry the
// Normalizer"), on the vector ALUs. A workgroup owns 64 query rows and has
// four waves: 64-key blocks of K and V stream through LDS, and wave w takes
// keys 16w .. 16w+15 of each block, so lane i of every wave carries its own
// (m, l, a) of query row i over a quarter of the keys. At the end the four
// states are merged through LDS by the two-block rule of "Carry the
// Normalizer" (common reference max(m1, m2), each part scaled by
// e^(m_i - m)), in two rounds (waves 2, 3 into 0, 1, then 1 into 0).
// This path serves small float32 problems where no bf16 rounding is
// acceptable; it is not tuned for throughput.
#include <hip/hip_runtime.h>

#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kBQ = kFp32TileRows;  // query rows per workgroup
constexpr int kWaves = 4;           // waves per workgroup, one key quarter each
constexpr int kBK = 16;             // keys per wave per block
constexpr int kBlk = kWaves * kBK;  // keys per block
constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBQ * kWaves) void fwd_fp32_kernel(FwdParams p, int n_qt) {
  __shared__ float qs[kBQ][D + 1];  // +1: each lane reads its own row
  // K and V of one block (read as broadcasts); at the end, the accumulators
  // of two waves, a[w'][t][lane], for the merge.
  __shared__ float kv[2 * kBlk * D];
  __shared__ float ml[2][2][kBQ];   // m and l of two waves for the merge
  float (*kt)[D] = reinterpret_cast<float (*)[D]>(kv);
  float (*vs)[D] = reinterpret_cast<float (*)[D]>(kv + kBlk * D);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  for (int i = tid; i < kBQ * D; i += kBQ * kWaves) {
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

  for (int kb = 0; kb < kend; kb += kBlk) {
    __syncthreads();
    for (int i = tid; i < kBlk * D; i += kBQ * kWaves) {
      const int r = i / D, c = i % D;
      const int key = kb + r;
      const bool in = key < Lk;
      kt[r][c] = in ? kg[static_cast<long>(key) * kstride + c] : 0.f;
      vs[r][c] = in ? vg[static_cast<long>(key) * kstride + c] : 0.f;
    }
    __syncthreads();
    const int k0 = kb + w * kBK;  // this wave's keys k0 .. k0+15 of the block
    const int r0 = w * kBK;       // and their rows in the LDS block

    float x[kBK];
    float mb = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kBK; ++jj) {
      float dot = 0.f;
#pragma unroll 16
      for (int t = 0; t < D; ++t) dot = fmaf(qs[lane][t], kt[r0 + jj][t], dot);
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
      for (int jj = 0; jj < kBK; ++jj) a = fmaf(x[jj], vs[r0 + jj][t], a);
      acc[t] = a;
    }
  }

  // Merge the four key quarters: waves 2 and 3 into 0 and 1, then 1 into 0.
  float* ka = kv;  // a[slot][t][lane], two slots
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    const int span = round == 0 ? 2 : 1;  // wave w + span merges into wave w
    __syncthreads();                      // the K/V block (or the last round) is consumed
    if (w >= span && w < 2 * span) {
      const int slot = w - span;
#pragma unroll
      for (int t = 0; t < D; ++t) ka[(slot * D + t) * kBQ + lane] = acc[t];
      ml[slot][0][lane] = m_run;
      ml[slot][1][lane] = l_run;
    }
    __syncthreads();
    if (w < span) {
      const float m1 = ml[w][0][lane];
      const float mm = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.f : exp2f(m_run - mm);
      const float a1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mm);
      l_run = l_run * a0 + ml[w][1][lane] * a1;
      m_run = mm;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = acc[t] * a0 + ka[(w * D + t) * kBQ + lane] * a1;
    }
  }
  if (w != 0) return;

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
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3(grid), dim3(kBQ * kWaves), 0, stream, p,
                     n_qt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace fa
