// Pieces shared by the matrix-core kernels of libfa (bf16 forward and
// backward, fp8 forward): vector types, the 64-row tile of K, V, Q or dO as
// staged in LDS (16-byte units of each row XOR-swizzled), its buffer-to-LDS
// loader, lane reductions, accumulator moves out of AGPRs and a
// compile-time loop. Device code only; every definition has internal
// linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

constexpr int kTileRows = 64;  // rows of one staged tile
constexpr int kThreads = 256;  // threads per workgroup of the bf16 kernels
// Third descriptor word of a raw buffer resource on gfx9-family parts
// (32-bit data format, no swizzle); the range check uses num_records.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Tile {
  static constexpr int kUnits = D / 8;                          // 16-byte units per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kTileRows * kRowBytes;          // one tile
  static constexpr int kLoads = kTileRows * kUnits / kThreads;  // loads per lane per tile
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

// Score MFMA (S^T tile = K operand x Q fragment), written as inline asm so
// that the score accumulator is a VGPR (the vector unit reads it next) while
// the Q fragment stays in an AGPR (only the matrix cores read it). The
// compiler does not see these as MFMAs: the dependent vector reads of a
// score tile are kept at least 19 wait states after its last MFMA by the
// instruction plan and by explicit s_nop guards.
__device__ __forceinline__ f32x16 mfma_qk_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  return d;
}
__device__ __forceinline__ void mfma_qk_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// 21 wait states: covers a 16-pass MFMA result before a dependent read.
__device__ __forceinline__ void mfma_result_guard() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Read an accumulator tile held in AGPRs into VGPRs (explicit moves, so
// that the compiler keeps the tile itself in AGPRs).
__device__ __forceinline__ f32x16 read_agpr(f32x16 a) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(a[i]));
    r[i] = x;
  }
  return r;
}

// Multiply an accumulator tile that lives in AGPRs by a per-lane factor,
// passing it through private memory: memory instructions take AGPR data
// directly, so no vector instruction reads the tile and the compiler keeps
// it in AGPRs everywhere else. Used only on the rare rescale path.
__device__ __forceinline__ f32x16 scale_via_scratch(f32x16 a, float f) {
  volatile f32x16 tmp;
  tmp = a;
  f32x16 x = tmp;
  x *= f;
  tmp = x;
  f32x16 r = tmp;
  asm volatile("" : "+a"(r));
  return r;
}

// Start the loads of one 64-row tile of a bf16 tensor with rows of D values
// at element stride `stride` (rows r0 .. r0+63: keys of K or V, or queries
// of Q or dO) into LDS. Each lane moves kLoads 16-byte units; a wave
// instruction fills 1 KiB of contiguous LDS. Rows at or past L (the length
// of the sequence) are outside the buffer range and are written as zeros.
template <int D>
__device__ __forceinline__ void issue_tile(const u16* g, long stride, int r0, int L,
                                           unsigned char* dst, int tid, int w) {
  using T = Tile<D>;
  const int rows = min(L - r0, kTileRows);
  const uint32_t stride_b = static_cast<uint32_t>(stride * 2);
  const uint32_t nrec = static_cast<uint32_t>(rows - 1) * stride_b + T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(g + static_cast<long>(r0) * stride), 0, nrec, kBufferFlags);
  // Wave w fills 1 KiB chunks w*kLoads .. w*kLoads + kLoads-1 of the tile
  // from one LDS base (M0), the chunk's offset in the instruction offset
  // field, which the hardware adds to the global offset as well.
  static_assert(T::kLoads <= 4, "chunk offsets fit the 12-bit instruction offset");
  const int lane = tid & 63;
  unsigned char* const base = dst + w * (T::kLoads * 1024);
  static_for<T::kLoads>([&](auto IT) {
    constexpr int it = decltype(IT)::value;
    const int u = (w * T::kLoads + it) * 64 + lane;
    const int row = u / T::kUnits;
    const int gc = (u % T::kUnits) ^ swz<T::kUnits>(row);
    // >= 0: row >= 64 * it / kUnits and stride_b >= kRowBytes = 16 * kUnits
    const uint32_t voff = row * stride_b + gc * 16 - it * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)base, 16, voff, 0, it * 1024, 0);
  });
}

}  // namespace
}  // namespace fa
