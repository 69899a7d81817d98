// Split-K/V attention forward for decode-shaped problems (few query rows per
// head, a long K/V cache), bf16 in / bf16 out, float32 state.
//
// The keys of every (batch entry, K/V head) are cut into `n_splits` ranges.
// A workgroup computes, for one range, the softmax-normalised output and the
// log-sum-exp of every query row of the K/V head's group over that range
// alone; a second kernel merges the ranges with the block merge rule of
// "Softmax does not need the matrix", section "Carry the Normalizer": for
// partial results (o_s, LSE_s) over disjoint key sets,
//   LSE = log sum_s exp(LSE_s),   o = sum_s exp(LSE_s - LSE) o_s.
// "Understanding FlashAttention Pt 1: Personal Notes", contents, section 8.1
// names the prefill and decode regimes; here decode has too few query rows
// per head to fill the chip with one workgroup per query tile, so the key
// axis supplies the parallelism instead.
//
// Query rows: the Hq/Hkv query heads that share K/V head g, times Nq rows,
// form one 32-row query tile (row r = group head r / Nq, query r % Nq), so
// one pass over the K/V tiles serves the whole group. One wavefront per
// workgroup owns one (batch entry, K/V head, key range): it forms the scores
// S^T = K Q^T of 32 keys at a time (lane = query row, registers = keys),
// keeps the online state (m, l) and accumulates all of O^T += V^T P^T, so
// no state is merged inside a workgroup and no key is scored twice. The
// problem is bound by HBM reads of K and V: each wave keeps the next stage's
// loads in flight while it computes, the loads bypass reuse in the caches
// (each K/V byte is read once), and small per-wave LDS rings let five waves
// share a compute unit.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <mutex>

#include "fa_bf16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr float kLn2d = 0.6931471805599453f;
constexpr float kLog2ed = 1.4426950408889634f;

__device__ __forceinline__ constexpr int drow(int r, int h2) { return 8 * (r >> 2) + 4 * h2 + (r & 3); }

// Rows 16g + 8r + 4*tr_h + (0..3) of a 64-row LDS tile at d columns of d-tile
// t, as the transposed A operand (see the forward kernel's V^T reads).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand_dec(const unsigned char* tile, int row0, int t, int g,
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

template <int D>
__device__ __forceinline__ bf16x8 row_operand_dec(const unsigned char* tile, int row0, int cc,
                                                  int lane) {
  using T = Tile<D>;
  const int row = row0 + (lane & 31);
  const int unit = (2 * cc + (lane >> 5)) ^ swz<T::kUnits>(row);
  return *reinterpret_cast<const bf16x8*>(tile + row * T::kRowBytes + unit * 16);
}

// One wavefront per workgroup: it streams its own key range through a ring
// of kDecStages LDS slots of kDecKeys keys (K and V), filled by
// buffer-to-LDS loads that no other wave touches, so the ring needs no
// barrier, only the wave's own count of loads in flight.
constexpr int kDecKeys = 32;    // keys per stage (one 32x32 score tile)
constexpr int kDecStages = 2;   // ring slots: one stage in flight while one is read
constexpr int kDecThreads = 64;
constexpr int kDecLoadAux = 2;  // cache policy of the K/V loads: non-temporal (read once)

template <int D>
struct DecStage {
  static constexpr int kUnits = D / 8;                        // 16-byte units per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kDecKeys * kRowBytes;         // one tensor of one stage
  static constexpr int kLoads = kDecKeys * kUnits / kDecThreads;  // 16-byte loads per lane
};

// Keys [kbeg, kend) of split s of a sequence with Lk keys: equal ranges,
// rounded up to whole stages.
__device__ __forceinline__ void split_range(int Lk, int n_splits, int s, int& kbeg, int& kend) {
  const int per = ((Lk + n_splits - 1) / n_splits + kDecKeys - 1) / kDecKeys * kDecKeys;
  kbeg = min(Lk, s * per);
  kend = min(Lk, kbeg + per);
}

// Loads of keys r0 .. r0+31 of one tensor into an LDS slot, in the
// swizzled row layout the operand reads expect; keys at or past kend lie
// outside the buffer range and arrive as zeros.
template <int D>
__device__ __forceinline__ void issue_stage(const u16* g, uint32_t stride_b, int r0, int kend,
                                            unsigned char* dst, int lane) {
  using T = DecStage<D>;
  const int rows = min(kend - r0, kDecKeys);
  const uint32_t nrec = static_cast<uint32_t>(rows - 1) * stride_b + T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(g + static_cast<long>(r0) * (stride_b / 2)), 0, nrec, kBufferFlags);
#pragma unroll
  for (int it = 0; it < T::kLoads; ++it) {
    const int u = it * kDecThreads + lane;
    const int row = u / T::kUnits;
    const int gc = (u % T::kUnits) ^ swz<T::kUnits>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + it * kDecThreads * 16), 16,
                                             row * stride_b + gc * 16, 0, 0, kDecLoadAux);
  }
}

// Wait until at most n stages (2 * kLoads loads each) are still in flight.
template <int D>
__device__ __forceinline__ void wait_stages(int n) {
  constexpr int L = 2 * DecStage<D>::kLoads;
  if (n >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * L) : "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(L) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
static_assert(kDecStages >= 2 && kDecStages <= 4, "wait_stages covers up to two newer stages");

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeParams p) {
  using T = DecStage<D>;
  constexpr int NC = D / 16;  // 16-wide d chunks of the score contraction
  constexpr int ND = D / 32;  // 32-row d tiles of O^T
  __shared__ __attribute__((aligned(1024))) unsigned char ring[kDecStages][2][T::kBytes];

  const int lane = threadIdx.x;
  const int j = lane & 31;
  const int h2 = lane >> 5;

  const int split = static_cast<int>(blockIdx.x % p.n_splits);
  const int bk = static_cast<int>(blockIdx.x / p.n_splits);
  const int b = bk / p.hkv;
  const int kvh = bk % p.hkv;
  const int gq = p.hq / p.hkv;
  const int Lk = p.seqlens_k != nullptr ? min(max(p.seqlens_k[b], 0), p.nk) : p.nk;
  int kbeg, kend;
  split_range(Lk, p.n_splits, split, kbeg, kend);

  // This lane's query row: group head j / Nq, query j % Nq.
  const int nrows = gq * p.nq;
  const bool row_ok = j < nrows;
  const int gh = row_ok ? j / p.nq : 0;
  const int qi = row_ok ? j % p.nq : 0;
  const int h = kvh * gq + gh;

  const long qstride = static_cast<long>(p.hq) * D;
  const long kstride = static_cast<long>(p.hkv) * D;
  const uint32_t stride_b = static_cast<uint32_t>(kstride * 2);
  const u16* kg = static_cast<const u16*>(p.k) + static_cast<long>(b) * p.nk * kstride +
                  static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + static_cast<long>(b) * p.nk * kstride +
                  static_cast<long>(kvh) * D;

  const int nst = (kend - kbeg + kDecKeys - 1) / kDecKeys;  // stages of this split
  auto issue = [&](int s) {
    unsigned char* slot = &ring[s % kDecStages][0][0];
    issue_stage<D>(kg, stride_b, kbeg + s * kDecKeys, kend, slot, lane);
    issue_stage<D>(vg, stride_b, kbeg + s * kDecKeys, kend, slot + T::kBytes, lane);
  };
#pragma unroll
  for (int s = 0; s < kDecStages - 1; ++s)
    if (s < nst) issue(s);

  bf16x8 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u};
    if (row_ok)
      a = ld16(static_cast<const u16*>(p.q) + (static_cast<long>(b) * p.nq + qi) * qstride +
               static_cast<long>(h) * D + 16 * cc + 8 * h2);
    qf[cc] = as_bf16x8(a);
  }
  const float c = p.scale_log2;
  float m = -INFINITY;  // running max of c * s (base 2)
  float l = 0.f;        // this lane's part of the denominator
  f32x16 acc[ND];
#pragma unroll
  for (int t = 0; t < ND; ++t) acc[t] = f32x16{};

  for (int s = 0; s < nst; ++s) {
    // stage s has landed once at most the stages issued after it remain
    wait_stages<D>(min(kDecStages - 2, nst - 1 - s));
    // the slot read in the previous iteration is free: refill it
    if (s + kDecStages - 1 < nst) issue(s + kDecStages - 1);
    const unsigned char* kst = &ring[s % kDecStages][0][0];
    const unsigned char* vst = kst + T::kBytes;
    const int ks0 = kbeg + s * kDecKeys;
    f32x16 st = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand_dec<D>(kst, 0, cc, lane), qf[cc],
                                                   st, 0, 0, 0);
    // x = c * s on visible keys, -inf elsewhere
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = ks0 + drow(r, h2);
      const bool vis = key < kend && (!p.causal || key <= qi);
      st[r] = vis ? st[r] * c : -INFINITY;
      mx = fmaxf(mx, st[r]);
    }
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m, mx);
    const float ref = m_new == -INFINITY ? 0.f : m_new;  // a row with no visible key yet
    const float alpha = __builtin_amdgcn_exp2f(m - ref);
    m = m_new;
    float rs = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = __builtin_amdgcn_exp2f(st[r] - ref);
      rs += x;
      pb[r >> 3][r & 7] = static_cast<__bf16>(x);
    }
    l = l * alpha + rs;
#pragma unroll
    for (int t = 0; t < ND; ++t) {
      acc[t] *= alpha;
#pragma unroll
      for (int g = 0; g < 2; ++g)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand_dec<D>(vst, 0, t, g, lane),
                                                         pb[g], acc[t], 0, 0, 0);
    }
  }

  // Partial results of this split: o_s = a / l (float32) and LSE_s (natural
  // log); a split with no visible key stores LSE_s = -inf and o_s = 0.
  const float l_tot = xhalf_sum(l);
  if (row_ok) {
    const long prow = ((static_cast<long>(split) * p.batch + b) * p.hq + h) * p.nq + qi;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* og = p.part_o + prow * D;
#pragma unroll
    for (int t = 0; t < ND; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 o4;
        o4.x = acc[t][4 * g4 + 0] * inv;
        o4.y = acc[t][4 * g4 + 1] * inv;
        o4.z = acc[t][4 * g4 + 2] * inv;
        o4.w = acc[t][4 * g4 + 3] * inv;
        *reinterpret_cast<float4*>(og + 32 * t + 8 * g4 + 4 * h2) = o4;
      }
    if (h2 == 0) p.part_lse[prow] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2d : -INFINITY;
  }
}

// Merge the splits of one (batch entry, q-head, query row) per wave: the
// row's LSE = log sum_s exp(LSE_s) and o = sum_s exp(LSE_s - LSE) o_s, then
// o rounded once to bf16. A row no split sees gets o = 0, LSE = -inf. Lane
// s holds split s's LSE and weight (64 splits at a time), so the maximum
// and the weight sum are wave reductions and the partial rows' loads do not
// wait on each other.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeParams p) {
  const long row = static_cast<long>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long n_rows = static_cast<long>(p.batch) * p.hq * p.nq;
  if (row >= n_rows) return;
  const long split_stride = n_rows;  // part rows of consecutive splits
  const int ns = p.n_splits;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) mx = fmaxf(mx, p.part_lse[(s0 + lane) * split_stride + row]);
  mx = wave_max(mx);
  float o[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) o[e] = 0.f;
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      // this lane's split weight (0 for a split that saw no key)
      float wgt = 0.f;
      if (s0 + lane < ns) {
        const float ls = p.part_lse[(s0 + lane) * split_stride + row];
        wgt = ls == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ls - mx) * kLog2ed);
      }
      sum += wgt;
      const int n = min(64, ns - s0);
      int s = 0;
      for (; s + 4 <= n; s += 4) {  // four partial rows in flight
        float src[4][D / 64];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < D / 64; ++e)
            src[u][e] = p.part_o[((s0 + s + u) * split_stride + row) * D + e * 64 + lane];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float wu = __shfl(wgt, s + u);
#pragma unroll
          for (int e = 0; e < D / 64; ++e) o[e] = __builtin_fmaf(wu, src[u][e], o[e]);
        }
      }
      for (; s < n; ++s) {
        const float wu = __shfl(wgt, s);
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
          o[e] = __builtin_fmaf(wu, p.part_o[((s0 + s) * split_stride + row) * D + e * 64 + lane],
                                o[e]);
      }
    }
    sum = wave_sum(sum);
    const float inv = 1.f / sum;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) o[e] *= inv;
    lse = mx + __logf(sum);
  }
  // row = (b * Hq + h) * Nq + i  ->  O [B, Nq, Hq, D], LSE [B, Hq, Nq]
  const long i = row % p.nq;
  const long bh = row / p.nq;
  const long h = bh % p.hq;
  const long b = bh / p.hq;
  u16* og = static_cast<u16*>(p.o) + ((b * p.nq + i) * p.hq + h) * D;
#pragma unroll
  for (int e = 0; e < D / 64; ++e)
    reinterpret_cast<__bf16*>(og)[e * 64 + lane] = static_cast<__bf16>(o[e]);
  if (lane == 0) p.lse[row] = lse;
}

}  // namespace

template <int D>
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.batch) * p.hkv * p.n_splits;
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3(grid), dim3(kDecThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n_rows = static_cast<long>(p.batch) * p.hq * p.nq;
  const unsigned cgrid = static_cast<unsigned>((n_rows + kThreads / 64 - 1) / (kThreads / 64));
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(cgrid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template hipError_t launch_decode_bf16<64>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_bf16<128>(const DecodeParams&, hipStream_t);

// Partial O and LSE of every split for fa_fwd_splitkv_noalloc. Each GPU
// that loads the library holds its own copy until the process ends; every
// call on a GPU reuses it (the split pass writes every partial row that the
// combine pass reads, so nothing needs clearing between calls).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kScratchDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  ScratchSlot& slot = g_scratch[dev];
  // in host code `scratch` names a host-side stand-in: only the address the
  // runtime reports for the current device may reach a kernel
  std::call_once(slot.once, [&] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
  });
  if (slot.err != hipSuccess) return slot.err;
  *ptr = slot.ptr;
  return hipSuccess;
}

}  // namespace fa
