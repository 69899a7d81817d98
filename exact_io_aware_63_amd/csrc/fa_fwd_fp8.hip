// Exact tiled attention forward with FP8 (OCP e4m3) Q, K, V for gfx950
// (CDNA4) matrix cores; bf16 output, float32 softmax state and LSE.
//
// The function is attention of the dequantized inputs: with per-tensor
// factors dq, dk, dv the inputs are q = dq * Q8, k = dk * K8, v = dv * V8,
// S = scale q k^T, P = softmax_row(S), O = P v. The pages name FP8 as the
// FlashAttention-3 variant whose speed comes with a precision cost
// ("Understanding FlashAttention Pt 1: Personal Notes", contents, section
// 5.6). Here the cost is exactly one rounding: the scores are exact (e4m3
// products are exact in the float32 accumulator), and the probabilities
// are rounded to e4m3 for the P V product on the fp8 matrix cores.
//
// Schedule: the tiling and online softmax of the bf16 kernel ("Softmax
// does not need the matrix", section "Carry the Normalizer"; "Understanding
// FlashAttention Pt 1", section 1.2), with v_mfma_f32_32x32x64_f8f6f4 for
// both products:
//   * a workgroup owns 256 query rows of one (batch entry, q-head); wave w
//     owns 64 of them as two 32-row query tiles;
//   * 64-key blocks of K (row-major, 16-byte units swizzled) and of V^T
//     stream through LDS by buffer-to-LDS loads, double-buffered;
//   * S^T = K Q^T: a lane holds 32 scores of one query row;
//   * the weights of a block are stored per row as ws = 2^(x - m - t + 8),
//     x = c s in base 2, t = ceil(block max - m), so the block's largest
//     weight lies in (2^7, 2^8]; they are rounded to e4m3 and packed straight
//     into the B operand of O^T += V^T P^T, whose per-lane e8m0 scale
//     (the row's 2^(t-8)) restores the true weights 2^(x - m) in the
//     product. Their byte order
//     (key tile kt, register r: key 32kt + 8(r/4) + 4*h2 + (r%4)) is what
//     the V^T tiles are laid out for: a pre-pass (vt_pack_kernel) writes
//     each 64-key block of V as a [128 d rows x 64 bytes] tile whose byte
//     32*h2 + i of row d is V[key(h2, i)][d], so the A operand of a lane is
//     32 contiguous bytes.
// Reference point: the first visible block of a row sets m; the block scale
// absorbs any later growth of the maxima, so m moves again only when a
// block maximum exceeds m + 64 (to keep the float32 sums far from
// overflow), a rescale through private memory that realistic inputs never
// reach. Stored weights down to 2^-14 of the block maximum are e4m3 normals
// (3 mantissa bits).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <type_traits>

#include "fa_bf16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kD8 = 128;                 // head width of the fp8 path
constexpr int kBR8 = 256;                // query rows per workgroup
constexpr int kBlk = 64;                 // keys per block
constexpr int kVtRowBytes = kBlk;        // one V^T tile row: 64 keys of one d
constexpr int kVtBytes = kD8 * kBlk;     // 8 KiB
constexpr float kRaiseFar = 64.f;        // a block maximum above m + 64 moves m
constexpr int kTmin = -100;              // t is clamped to [-100, 64]: scale 2^(t-8)
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kScaleOne = 127;           // e8m0 scale 2^0 of the scaled MFMA form

// Key of byte i (0..31) of half-wave h2 in a 64-key block: key tile i/16,
// MFMA output register r = i % 16 at row 8(r/4) + 4*h2 + (r%4).
__host__ __device__ constexpr int key_of_byte(int h2, int i) {
  return 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * h2 + (i & 3);
}

// LDS swizzles. A ds_read_b128 serves 16 lanes per pass from one 256-byte
// bank window, so the 16 rows read by 16 consecutive lanes (same logical
// unit) must fall on 16 different 16-byte bank groups.
// V^T tile rows are 64 bytes: row d sits at bank groups 4(d%4) .. +3, and
// logical unit u is stored at unit u ^ ((d / 4) % 4).
__device__ __forceinline__ int vt_swz(int d) { return (d >> 2) & 3; }

// K tile: 64 keys x 128 bytes; row r sits at bank groups 8(r%2) .. +7, and
// logical unit u is stored at unit u ^ ((r / 2) % 8).
constexpr int kKRowBytes = kD8;
constexpr int kKBytes = kBlk * kKRowBytes;
__device__ __forceinline__ int k_swz8(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0,
                                                         kScaleOne);
}

// Score MFMAs (S^T tile = K operand x Q fragment) as inline asm, with the
// Q fragment in AGPRs and the scores written to VGPRs, where the next
// block's vector work reads them. The compiler does not see these as
// MFMAs, so nothing reads a score tile before mfma8_result_guard() at the
// end of the region that formed it.
__device__ __forceinline__ f32x16 mfma8_qk_first(i32x8 a, i32x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
__device__ __forceinline__ void mfma8_qk_acc(f32x16& d, i32x8 a, i32x8 b) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// 32 wait states: more than a 16-pass MFMA result needs before a dependent
// vector read.
__device__ __forceinline__ void mfma8_result_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Step plan of one block: 16 matrix steps. Steps 0..7: the score MFMAs of
// the NEXT block, s -> key tile s/4, d chunk (s/2)%2, query tile s%2 (each
// LDS operand serves both query tiles); steps 8..11: P V of query tile 0,
// d tile s-8; steps 12..15: P V of query tile 1. The 16 groups of 4
// weights (exp, e4m3 pack, row sum) of THIS block are spread over steps
// 0..11: tile 0's group g at step g, tile 1's groups at steps 1, 3, 5, 7,
// 8, 9, 10, 11, so each tile's P bytes are complete before its P V.
constexpr int kQt1GroupStep[8] = {1, 3, 5, 7, 8, 9, 10, 11};

// ---------------------------------------------------------------------------
// V -> V^T tiles
// ---------------------------------------------------------------------------

// One workgroup per (batch entry, K/V head, 64-key block): stage the 64 rows
// of V (8 KiB) in LDS, then write the 128 x 64-byte V^T tile (each 16-byte
// unit gathered from 16 keys). Keys at or past Nk are written as zeros.
__global__ __launch_bounds__(kThreads) void vt_pack_kernel(Fp8Params p) {
  __shared__ __attribute__((aligned(16))) unsigned char vs[kBlk * kD8];
  const int tid = threadIdx.x;
  const int blk = static_cast<int>(blockIdx.x % p.nblk);
  const int unit = static_cast<int>(blockIdx.x / p.nblk);  // b * Hkv + g
  const int b = unit / p.hkv;
  const int g = unit % p.hkv;
  const long kstride = static_cast<long>(p.hkv) * kD8;
  const unsigned char* vg = static_cast<const unsigned char*>(p.v) +
                            static_cast<long>(b) * p.nk * kstride + static_cast<long>(g) * kD8;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = it * kThreads + tid;  // 512 units: key u / 8, unit u % 8
    const int key = blk * kBlk + u / 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < p.nk) x = *reinterpret_cast<const u32x4*>(vg + key * kstride + (u % 8) * 16);
    *reinterpret_cast<u32x4*>(vs + u * 16) = x;
  }
  __syncthreads();
  unsigned char* out = static_cast<unsigned char*>(p.vt) + (static_cast<long>(unit) * p.nblk + blk) * kVtBytes;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int o = it * kThreads + tid;  // 512 units: row d = o / 4, physical unit o % 4
    const int d = o >> 2;
    const int lu = (o & 3) ^ vt_swz(d);  // logical unit: bytes 16*lu .. 16*lu+15 of the row
    uint32_t wv[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint32_t acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bi = 16 * lu + 4 * q4 + e;  // byte of the row: half bi / 32, byte bi % 32
        const int key = key_of_byte(bi >> 5, bi & 31);
        acc |= static_cast<uint32_t>(vs[key * kD8 + d]) << (8 * e);
      }
      wv[q4] = acc;
    }
    *reinterpret_cast<u32x4*>(out + d * kVtRowBytes + (o & 3) * 16) = u32x4{wv[0], wv[1], wv[2], wv[3]};
  }
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------

// Start the buffer-to-LDS loads of one K tile (keys r0 .. r0+63 of one
// K/V head, rows `stride` bytes apart); rows at or past L lie outside the
// buffer range and arrive as zeros. Two 16-byte units per lane.
__device__ __forceinline__ void issue_k8(const unsigned char* g, long stride, int r0, int L,
                                         unsigned char* dst, int tid, int w) {
  const int rows = min(L - r0, kBlk);
  const uint32_t sb = static_cast<uint32_t>(stride);
  const uint32_t nrec = static_cast<uint32_t>(rows - 1) * sb + kKRowBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(g + static_cast<long>(r0) * stride), 0, nrec, kBufferFlags);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int u = it * kThreads + tid;  // physical unit u % 8 of row u / 8
    const int row = u >> 3;
    const uint32_t voff = row * sb + ((u & 7) ^ k_swz8(row)) * 16;
    const int lds_off = (it * kThreads + w * 64) * 16;  // wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + lds_off), 16, voff, 0, 0, 0);
  }
}

// Buffer-to-LDS copy of one contiguous 8 KiB V^T tile (two 16-byte units
// per lane; a wave instruction fills 1 KiB).
__device__ __forceinline__ void issue_vt(const unsigned char* src, unsigned char* dst, int tid,
                                         int w) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src), 0, kVtBytes, kBufferFlags);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int lds_off = (it * kThreads + w * 64) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + lds_off), 16,
                                             (it * kThreads + tid) * 16, 0, 0, 0);
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_fp8_kernel(Fp8Params p, int n_qt) {
  __shared__ __attribute__((aligned(1024))) unsigned char kb[2][kKBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vb[2][kVtBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int h2 = lane >> 5;

  // Workgroup -> (tile, batch entry, q-head), XCD-aware as the bf16 kernel:
  // when the K/V heads split evenly over the 8 XCDs (ids dealt id % 8), all
  // tiles of one K/V head run on one XCD; longest causal tiles first.
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
  const int Lq = p.nq, Lk = p.nk;
  const int q0 = tile * kBR8;
  if (q0 >= Lq) return;

  const long qstride = static_cast<long>(p.hq) * kD8;
  const long kstride = static_cast<long>(p.hkv) * kD8;
  const unsigned char* qg = static_cast<const unsigned char*>(p.q) +
                            static_cast<long>(b) * Lq * qstride + static_cast<long>(h) * kD8;
  const unsigned char* kg = static_cast<const unsigned char*>(p.k) +
                           static_cast<long>(b) * Lk * kstride + static_cast<long>(kvh) * kD8;
  const unsigned char* vtg = static_cast<const unsigned char*>(p.vt) +
                             (static_cast<long>(b) * p.hkv + kvh) * p.nblk * kVtBytes;

  int kend = Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBR8, Lq));
  const int nblk = (kend + kBlk - 1) / kBlk;
  const int wq0 = q0 + 64 * w;
  int nblk_w = wq0 >= Lq ? 0 : nblk;
  if (CAUSAL) nblk_w = min(nblk_w, wq0 / kBlk + 1);

  if (nblk > 0) {
    issue_k8(kg, kstride, 0, Lk, kb[0], tid, w);
    issue_vt(vtg, vb[0], tid, w);
    if (nblk > 1) issue_k8(kg, kstride, kBlk, Lk, kb[1], tid, w);
  }

  // A negative c is applied by flipping the sign bits of Q (exact in e4m3).
  const float c = fmaxf(fabsf(p.c), FLT_MIN);
  const uint32_t qflip = p.c < 0.f ? 0x80808080u : 0u;

  // Q fragments (B operand of S^T = K Q^T): query tile qt, 64-wide d chunk
  // cc, bytes 64cc + 32*h2 .. +31 of this lane's row.
  i32x8 qf[2][2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = wq0 + 32 * qt + j;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
      if (qrow < Lq) {
        const unsigned char* src = qg + static_cast<long>(qrow) * qstride + 64 * cc + 32 * h2;
        lo = *reinterpret_cast<const u32x4*>(src) ^ qflip;
        hi = *reinterpret_cast<const u32x4*>(src + 16) ^ qflip;
      }
      qf[qt][cc] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      asm volatile("" : "+a"(qf[qt][cc]));  // only the matrix cores read Q: AGPRs
    }
  }
  asm volatile("s_nop 4" ::: "memory");  // AGPR writes before the inline MFMAs read them

  f32x16 acc[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[qt][t] = f32x16{};
      asm volatile("" : "+a"(acc[qt][t]));  // the accumulators live in AGPRs
    }
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  // K operand: key tile kt (rows 32kt + j), d chunk cc: logical 16-byte
  // units 4cc + 2*h2 and 4cc + 2*h2 + 1 of the row.
  const int k_swz = k_swz8(j);  // equal for rows j and j + 32
  auto k_operand = [&](const unsigned char* ks, int kt, int cc) {
    const unsigned char* row = ks + (32 * kt + j) * kKRowBytes;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + ((4 * cc + 2 * h2) ^ k_swz) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + ((4 * cc + 2 * h2 + 1) ^ k_swz) * 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // V^T operand: d tile t (rows 32t + j), bytes 32*h2 .. +31 of the row.
  auto v_operand = [&](const unsigned char* vs, int t) {
    const int d = 32 * t + j;
    const unsigned char* row = vs + d * kVtRowBytes;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(row + ((2 * h2) ^ vt_swz(d)) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(row + ((2 * h2 + 1) ^ vt_swz(d)) * 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  // S^T of one block from the K tile ks: s[qt][kt][r] is key
  // k0 + 32kt + 8(r/4) + 4*h2 + (r%4) against query wq0 + 32qt + j.
  // two score sets: a block reads its scores from one while its region forms
  // the next block's in the other (the key loop swaps them)
  f32x16 sa[2][2], sb[2][2];
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (nblk_w > 0) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const i32x8 a0 = k_operand(kb[0], kt, 0);
      const i32x8 a1 = k_operand(kb[0], kt, 1);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        sa[qt][kt] = mfma8_qk_first(a0, qf[qt][0]);
        mfma8_qk_acc(sa[qt][kt], a1, qf[qt][1]);
      }
    }
    mfma8_result_guard();
  }

  // One key block j; its scores sc are in registers and the loads of
  // K_{j+1} and V^T_j are in flight (issued one block earlier).
  //   head: wait for them; barrier (every wave is done with block j-1, so
  //      the buffers of K_j and V^T_{j-1} are free); start the loads of
  //      K_{j+2} and V^T_{j+1} into them;
  //   body: mask, row maxima, reference; then one branch-free region in
  //      which the matrix cores form the scores of block j+1 (sn) and
  //      O^T += V^T_j P_j^T while the vector unit computes the weights of
  //      block j: each score MFMA shares its slot with 14 vector
  //      instructions of query tile 0, each P V MFMA of tile 0 with 28 of
  //      tile 1 (sched_group_barrier fixes that interleave).
  auto head = [&](auto par_tag, int jb) {
    constexpr int PAR = decltype(par_tag)::value;  // jb & 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (jb + 2 < nblk) issue_k8(kg, kstride, (jb + 2) * kBlk, Lk, kb[PAR], tid, w);
    if (jb + 1 < nblk)
      issue_vt(vtg + static_cast<long>(jb + 1) * kVtBytes, vb[PAR ^ 1], tid, w);
  };
  auto body = [&](auto par_tag, int jb, f32x16(&sc)[2][2], f32x16(&sn)[2][2]) {
    constexpr int PAR = decltype(par_tag)::value;  // jb & 1
    if (jb >= nblk_w) return;
    const int k0 = jb * kBlk;
    const unsigned char* k_next = kb[PAR ^ 1];  // K_{j+1}
    const unsigned char* v_cur = vb[PAR];       // V^T_j
    // Mask the blocks that reach past the keys or cross this wave's diagonal.
    if ((k0 + kBlk > Lk) || (CAUSAL && k0 + kBlk - 1 > wq0)) {
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
    float mb[2];
    bool up = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // two running maxima (shorter dependency chains), one v_max3 per two scores
      float ma = fmaxf(sc[qt][0][0], sc[qt][1][0]);
      float mc = fmaxf(sc[qt][0][1], sc[qt][1][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        ma = max3(ma, sc[qt][0][r], sc[qt][1][r]);
        mc = max3(mc, sc[qt][0][r + 1], sc[qt][1][r + 1]);
      }
      mb[qt] = xhalf_max(fmaxf(ma, mc)) * c;
      if (m_run[qt] == -INFINITY) m_run[qt] = mb[qt];
      up = up || (mb[qt] > m_run[qt] + kRaiseFar);
    }
    if (__any(up)) {  // wave-uniform, rare
      // after the last P V MFMAs have written the accumulators
      mfma8_result_guard();
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float m_new = fmaxf(m_run[qt], mb[qt]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);
        m_run[qt] = m_new;
        l_run[qt] *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[qt][t] = scale_via_scratch(acc[qt][t], alpha);
      }
      asm volatile("s_nop 1" ::: "memory");  // AGPR writes before MFMA reads
    }
    // per-row block exponent t, exp offset 8 - m - t, B-operand scale byte
    // 127 + (t - 8); a row with no visible key so far keeps t = 0 (its
    // weights are all 0)
    float off[2];
    int tq[2], sbq[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const bool none = m_run[qt] == -INFINITY;
      tq[qt] = none ? 0 : static_cast<int>(ceilf(fmaxf(mb[qt] - m_run[qt], static_cast<float>(kTmin))));
      off[qt] = (none ? 0.f : -m_run[qt]) + static_cast<float>(8 - tq[qt]);
      sbq[qt] = kScaleOne + tq[qt] - 8;
    }

    // The region (Plan above): LDS operands are read two steps before their
    // first use; score operand p = 2kt + cc is first used at step 2p, value
    // operand t (shared by both query tiles) at step 8 + t.
    i32x8 kop[2][2], vop[4];
    int pw[2][8];
    float rs[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    auto loads_for = [&](auto S) {
      constexpr int s = decltype(S)::value;
      if constexpr (s < 8 && (s & 1) == 0) {
        constexpr int pp = s / 2;
        kop[pp >> 1][pp & 1] = k_operand(k_next, pp >> 1, pp & 1);
      }
      if constexpr (s >= 8 && s < 12) vop[s - 8] = v_operand(v_cur, s - 8);
    };
    // group g of query tile qt: score registers 4(g%4) .. +3 of key tile
    // g/4, packed into B-operand word g
    auto group = [&](int qt, int g) {
      const int kt = g >> 2, r0 = 4 * (g & 3);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qt][kt][r0 + e], c, off[qt]));
      rs[qt][g & 1] += (x[0] + x[1]) + (x[2] + x[3]);
      const int wd = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __float_as_int(x[0]), false);
      pw[qt][g] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], wd, true);
    };
    static_for<2>(loads_for);
    static_for<16>([&](auto S) {
      constexpr int s = decltype(S)::value;
      if constexpr (s + 2 < 16) loads_for(std::integral_constant<int, s + 2>{});
      if constexpr (s < 8) {
        constexpr int kt = s >> 2, cc = (s >> 1) & 1, qt = s & 1;
        if constexpr (cc == 0) sn[qt][kt] = mfma8_qk_first(kop[kt][0], qf[qt][0]);
        else mfma8_qk_acc(sn[qt][kt], kop[kt][1], qf[qt][1]);
      } else {
        constexpr int qt = s >= 12 ? 1 : 0, tt = s - 8 - 4 * qt;
        const i32x8 pb = {pw[qt][0], pw[qt][1], pw[qt][2], pw[qt][3],
                          pw[qt][4], pw[qt][5], pw[qt][6], pw[qt][7]};
        acc[qt][tt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            vop[tt], pb, acc[qt][tt], 0, 0, 0, kScaleOne, 0, sbq[qt]);
        asm volatile("" : "+a"(acc[qt][tt]));
      }
      if constexpr (s < 8) group(0, s);
      static_for<8>([&](auto G) {
        if constexpr (kQt1GroupStep[decltype(G)::value] == s) group(1, decltype(G)::value);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) l_run[qt] += ldexpf(rs[qt][0] + rs[qt][1], tq[qt] - 8);
    // the next block's scores are read only after the score MFMAs of this
    // region have finished
    mfma8_result_guard();
  };

  // Key loop, unrolled by two so every LDS address has a fixed buffer. A
  // wave's last computed block also forms the scores of the block after it
  // (from whatever the K buffer holds, discarded).
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int jb = 0; jb < nblk; jb += 2) {
    head(P0{}, jb);
    body(P0{}, jb, sa, sb);
    if (jb + 1 >= nblk) break;
    head(P1{}, jb + 1);
    body(P1{}, jb + 1, sb, sa);
  }

  // Epilogue: o = dv * a / l, rounded once to bf16; LSE = ln 2 (m + log2 l).
  mfma8_result_guard();  // the last P V MFMAs may still be in flight
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    f32x16 o_t[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o_t[t] = read_agpr(acc[qt][t]);
    const int qrow = wq0 + 32 * qt + j;
    const float l_tot = xhalf_sum(l_run[qt]);
    if (qrow < Lq) {
      const float f = l_tot > 0.f ? p.v_descale / l_tot : 0.f;
      u16* og = static_cast<u16*>(p.o) + (static_cast<long>(b) * Lq + qrow) * qstride +
                static_cast<long>(h) * kD8;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = static_cast<__bf16>(o_t[t][4 * g + e] * f);
          *reinterpret_cast<bf16x4*>(og + 32 * t + 8 * g + 4 * h2) = o4;
        }
      if (h2 == 0)
        p.lse[(static_cast<long>(b) * p.hq + h) * Lq + qrow] =
            l_tot > 0.f ? (m_run[qt] + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream) {
  const unsigned packs = static_cast<unsigned>(p.batch) * p.hkv * p.nblk;
  if (packs > 0) {  // no keys: no V^T tiles, every row gets O = 0, LSE = -inf
    hipLaunchKernelGGL(vt_pack_kernel, dim3(packs), dim3(kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_qt = (p.nq + kBR8 - 1) / kBR8;
  const unsigned grid = static_cast<unsigned>(n_qt) * p.hq * p.batch;
  if (p.causal)
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, p, n_qt);
  else
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, p, n_qt);
  return hipGetLastError();
}

}  // namespace fa
