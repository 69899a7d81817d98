// Internal interface between the host entry points (fa_api.cpp) and the
// device kernels. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// One attention-forward problem, already validated on the host.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;  // device pointer, or nullptr for fixed length
  int batch;                  // B, or number of packed sequences
  int hq;
  int hkv;
  int nq;                     // packed: maximum sequence length
  int nk;
  int d;
  float scale_log2;           // scale * log2(e): scores are kept in base 2
  int causal;
  int win_left;               // sliding window: query i sees keys >= i - win_left (-1: all)
  int win_right;              // and keys <= i + win_right (-1: all); bf16 kernels only
  float scale;                // the score scale itself (bias variant)
  const void* bias;           // additive bias, bf16, or nullptr; bf16 kernels only:
  long bias_sb;               //   element (s, h, i, j) at bias[s*sb + h*sh + i*sr + j]
  long bias_sh;
  long bias_sr;
  int num_cus;                // compute units of the device (choice of launch shape)
};

// Launch the bf16 kernel for head width D (64 or 128), causal or not.
// Returns the hipError_t of the launch. Each of the four instances is
// compiled in its own object file.
template <int D, bool CAUSAL>
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
extern template hipError_t launch_fwd_bf16<64, false>(const FwdParams&, hipStream_t);
extern template hipError_t launch_fwd_bf16<64, true>(const FwdParams&, hipStream_t);
extern template hipError_t launch_fwd_bf16<128, false>(const FwdParams&, hipStream_t);
extern template hipError_t launch_fwd_bf16<128, true>(const FwdParams&, hipStream_t);

// One attention-backward problem, already validated on the host.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;                // D = rowsum(dO * O), laid out like lse
  const int32_t* cu_seqlens;  // device pointer, or nullptr for fixed length
  int batch;
  int hq;
  int hkv;
  int nq;
  int nk;
  int d;
  float scale;
  float scale_log2;           // scale * log2(e)
  int causal;
  int win_left;               // sliding window as FwdParams (-1: unbounded)
  int win_right;
  const void* bias;           // additive bias as FwdParams, or nullptr
  long bias_sb;
  long bias_sh;
  long bias_sr;
};

// Launch the bf16 backward (D = rowsum(dO * O), then dQ, then dK and dV)
// for head width D, causal or not; one object file per instance.
template <int D, bool CAUSAL>
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);
extern template hipError_t launch_bwd_bf16<64, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd_bf16<64, true>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd_bf16<128, false>(const BwdParams&, hipStream_t);
extern template hipError_t launch_bwd_bf16<128, true>(const BwdParams&, hipStream_t);

// One split-K/V (decode) forward problem, already validated on the host.
struct DecodeParams {
  const void* q;              // [B, Nq, Hq, d] bf16
  const void* k;              // [B, Nk, Hkv, d] bf16
  const void* v;
  void* o;                    // [B, Nq, Hq, d] bf16
  float* lse;                 // [B, Hq, Nq]
  const int32_t* seqlens_k;   // device int32 [B] (keys of each entry), or nullptr: Nk
  float* part_o;              // workspace: [n_splits, B, Hq, Nq, d] float32
  float* part_lse;            // workspace: [n_splits, B, Hq, Nq] float32
  int batch;
  int hq;
  int hkv;
  int nq;
  int nk;
  int d;
  float scale_log2;
  int causal;
  int n_splits;
};

// Split pass then combine pass, head width D.
template <int D>
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
extern template hipError_t launch_decode_bf16<64>(const DecodeParams&, hipStream_t);
extern template hipError_t launch_decode_bf16<128>(const DecodeParams&, hipStream_t);

// Scratch of fa_fwd_splitkv_noalloc: a file-scope device array of this many
// bytes in fa_decode_bf16.hip takes the place of the caller's workspace.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;

// Device address of that array on the current device, looked up with
// hipGetSymbolAddress on the first call for each device (thread-safe).
hipError_t decode_scratch(void** ptr);

// One FP8 (e4m3) attention-forward problem, already validated on the host:
// fixed length, d = 128, Q [B, Nq, Hq, 128], K and V [B, Nk, Hkv, 128]
// (bytes), O [B, Nq, Hq, 128] bf16, LSE [B, Hq, Nq].
struct Fp8Params {
  const void* q;
  const void* k;
  const void* v;
  void* vt;                   // workspace: [B, Hkv, nblk] V^T tiles of 8 KiB
  void* o;
  float* lse;
  int batch;
  int hq;
  int hkv;
  int nq;
  int nk;
  int nblk;                   // ceil(Nk / 64)
  float c;                    // scale * dq * dk * log2(e)
  float v_descale;            // dv
  int causal;
};

// V^T pre-pass, then the forward kernel.
hipError_t launch_fwd_fp8(const Fp8Params& p, hipStream_t stream);

// Launch the float32 kernel (d in {64, 128}).
hipError_t launch_fwd_fp32(const FwdParams& p, hipStream_t stream);

// Query tile height of each kernel (rows of Q per workgroup); the host uses
// it to bound the grid size.
constexpr int kBf16TileRows = 256;
constexpr int kFp32TileRows = 64;

}  // namespace fa
