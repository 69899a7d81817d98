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
// one pass over the K/V tiles serves the whole group. All four waves of a
// workgroup form the same scores S^T = K Q^T (lane = query row, registers =
// keys) and the same online state (m, l); wave w accumulates output columns
// 32w .. 32w+31 (d = 128) of O^T += V^T P^T, so no state is merged across
// waves. The problem is bound by HBM reads of K and V; the repeated score
// MFMAs cost matrix-core time that is otherwise idle.
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

// Keys [kbeg, kend) of split s of a sequence with Lk keys: equal ranges,
// rounded up to whole 64-key tiles.
__device__ __forceinline__ void split_range(int Lk, int n_splits, int s, int& kbeg, int& kend) {
  const int per = ((Lk + n_splits - 1) / n_splits + kTileRows - 1) / kTileRows * kTileRows;
  kbeg = min(Lk, s * per);
  kend = min(Lk, kbeg + per);
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  using T = Tile<D>;
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;  // d-tiles of O^T; waves >= ND idle in the P V product
  // Two slots per tensor as separate arrays, chosen at compile time (the
  // loop is unrolled by two): with one array indexed at run time the
  // compiler cannot tell the slot being loaded from the slot being read,
  // and waits for the new tile's loads before every read of the current one.
  __shared__ __attribute__((aligned(1024))) unsigned char k_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_st1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_st1[T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const u16* kg = static_cast<const u16*>(p.k) + static_cast<long>(b) * p.nk * kstride +
                  static_cast<long>(kvh) * D;
  const u16* vg = static_cast<const u16*>(p.v) + static_cast<long>(b) * p.nk * kstride +
                  static_cast<long>(kvh) * D;

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
  f32x16 acc = f32x16{};

  const int nkb = (kend - kbeg + kTileRows - 1) / kTileRows;
  if (nkb > 0) {
    issue_tile<D>(kg, kstride, kbeg, kend, k_st0, tid, w);
    issue_tile<D>(vg, kstride, kbeg, kend, v_st0, tid, w);
  }
  auto step = [&](auto par_tag, int it) {
    constexpr int PAR = decltype(par_tag)::value;  // it & 1
    const unsigned char* k_cur = PAR ? k_st1 : k_st0;
    const unsigned char* v_cur = PAR ? v_st1 : v_st0;
    unsigned char* k_nxt = PAR ? k_st0 : k_st1;
    unsigned char* v_nxt = PAR ? v_st0 : v_st1;
    const int k0 = kbeg + it * kTileRows;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < nkb) {
      issue_tile<D>(kg, kstride, k0 + kTileRows, kend, k_nxt, tid, w);
      issue_tile<D>(vg, kstride, k0 + kTileRows, kend, v_nxt, tid, w);
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ks0 = k0 + 32 * sub;
      if (ks0 >= kend) break;
      f32x16 st = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_operand_dec<D>(k_cur, 32 * sub, cc, lane),
                                                     qf[cc], st, 0, 0, 0);
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
      f32x16 pr;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(st[r] - ref);
        rs += pr[r];
      }
      l = l * alpha + rs;
      if (w < ND) {
        acc *= alpha;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          bf16x8 pb;
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[i] = static_cast<__bf16>(pr[8 * g + i]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand_dec<D>(v_cur, 32 * sub, w, g, lane),
                                                        pb, acc, 0, 0, 0);
        }
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int it = 0; it < nkb; it += 2) {
    step(P0{}, it);
    if (it + 1 >= nkb) break;
    step(P1{}, it + 1);
  }

  // Partial results of this split: o_s = a / l (float32) and LSE_s (natural
  // log); a split with no visible key stores LSE_s = -inf and o_s = 0.
  const float l_tot = xhalf_sum(l);
  if (row_ok) {
    const long prow = ((static_cast<long>(split) * p.batch + b) * p.hq + h) * p.nq + qi;
    if (w < ND) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* og = p.part_o + prow * D;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4 o4;
        o4.x = acc[4 * g4 + 0] * inv;
        o4.y = acc[4 * g4 + 1] * inv;
        o4.z = acc[4 * g4 + 2] * inv;
        o4.w = acc[4 * g4 + 3] * inv;
        *reinterpret_cast<float4*>(og + 32 * w + 8 * g4 + 4 * h2) = o4;
      }
    }
    if (w == 0 && h2 == 0)
      p.part_lse[prow] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2d : -INFINITY;
  }
}

// Merge the splits of one (batch entry, q-head, query row) per wave: the
// row's LSE = log sum_s exp(LSE_s) and o = sum_s exp(LSE_s - LSE) o_s, then
// o rounded once to bf16. A row no split sees gets o = 0, LSE = -inf.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeParams p) {
  const long row = static_cast<long>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const long n_rows = static_cast<long>(p.batch) * p.hq * p.nq;
  if (row >= n_rows) return;
  const long split_stride = n_rows;  // part rows of consecutive splits
  float mx = -INFINITY;
  for (int s = 0; s < p.n_splits; ++s) mx = fmaxf(mx, p.part_lse[s * split_stride + row]);
  float o[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) o[e] = 0.f;
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < p.n_splits; ++s) {
      const float ls = p.part_lse[s * split_stride + row];
      if (ls == -INFINITY) continue;
      const float wgt = __builtin_amdgcn_exp2f((ls - mx) * kLog2ed);
      sum += wgt;
      const float* src = p.part_o + (s * split_stride + row) * D;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) o[e] = __builtin_fmaf(wgt, src[e * 64 + lane], o[e]);
    }
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
  hipLaunchKernelGGL((decode_split_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, p);
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
