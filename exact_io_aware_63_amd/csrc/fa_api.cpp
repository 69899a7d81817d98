// C ABI of libfa: argument validation, device check and kernel launch.
//
// Every argument check runs on the host before the first HIP call, so the
// error paths work (and are tested) on machines without a GPU.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr int kMaxDevices = 64;

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device architecture check, done once per device.
struct DeviceCheck {
  std::once_flag once;
  int status = FA_OK;
  int cus = 0;  // compute units, for the choice of launch shape
  char msg[256] = "";
};
DeviceCheck g_devices[kMaxDevices];

int check_device(int* cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  DeviceCheck& dc = g_devices[dev];
  std::call_once(dc.once, [&] {
    hipDeviceProp_t prop;
    hipError_t pe = hipGetDeviceProperties(&prop, dev);
    if (pe != hipSuccess) {
      dc.status = FA_ERR_HIP;
      snprintf(dc.msg, sizeof(dc.msg), "hipGetDeviceProperties failed: %s", hipGetErrorString(pe));
      return;
    }
    dc.cus = prop.multiProcessorCount;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      dc.status = FA_ERR_UNSUPPORTED;
      snprintf(dc.msg, sizeof(dc.msg), "device %d is %s; libfa is built for gfx950 only", dev,
               prop.gcnArchName);
    }
  });
  if (dc.status != FA_OK) return fail(dc.status, "%s", dc.msg);
  if (cus != nullptr) *cus = dc.cus;
  return FA_OK;
}

// Shared validation for both element types. `elem` is the element size in
// bytes, `tile_rows` the query rows per workgroup of the kernel.
int validate(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             const int32_t* cu_seqlens, int tile_rows, bool* noop) {
  *noop = false;
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B=%d, Nq=%d, Nk=%d must be >= 0", B, Nq, Nk);
  if (Hq <= 0 || Hkv <= 0)
    return fail(FA_ERR_SHAPE, "Hq=%d and Hkv=%d must be > 0", Hq, Hkv);
  if (Hq % Hkv != 0)
    return fail(FA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (cu_seqlens != nullptr && Nq != Nk)
    return fail(FA_ERR_SHAPE, "packed sequences need Nq == Nk (the maximum length); got %d, %d",
                Nq, Nk);
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head width d=%d; supported: 64, 128", d);
  if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale is not finite");
  if (B == 0 || Nq == 0) {
    *noop = true;
    return FA_OK;
  }
  if (!Q || !K || !V || !O || !LSE)
    return fail(FA_ERR_NULL, "Q, K, V, O and LSE must all be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(FA_ERR_ARG, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(LSE, 4) || (cu_seqlens && !aligned(cu_seqlens, 4)))
    return fail(FA_ERR_ARG, "LSE and cu_seqlens must be 4-byte aligned");
  const int64_t n_qt = (static_cast<int64_t>(Nq) + tile_rows - 1) / tile_rows;
  const int64_t grid = n_qt * Hq * static_cast<int64_t>(B);
  if (grid > 0x7fffffffLL)
    return fail(FA_ERR_SHAPE, "grid of %lld workgroups exceeds the launch limit",
                static_cast<long long>(grid));
  // Element offsets are 64-bit in the kernels; the token counts only need
  // to fit the int arguments, which they do by type.
  return FA_OK;
}

// Additive bias of fa_fwd_bias: bf16 element (s, h, i, j) at
// ptr[s*sb + h*sh + i*sr + j].
struct BiasArg {
  const void* ptr;
  int64_t sb, sh, sr;
};

int validate_bias(const BiasArg& b, int Nk) {
  if (b.ptr == nullptr) return fail(FA_ERR_NULL, "bias must be non-NULL");
  if (!aligned(b.ptr, 8)) return fail(FA_ERR_ARG, "bias must be 8-byte aligned");
  if (b.sb < 0 || b.sh < 0)
    return fail(FA_ERR_ARG, "bias strides of the batch and head axes must be >= 0 (0 shares)");
  if (b.sr < Nk)
    return fail(FA_ERR_ARG, "bias row stride %lld is smaller than Nk=%d",
                static_cast<long long>(b.sr), Nk);
  if (b.sb % 4 != 0 || b.sh % 4 != 0 || b.sr % 4 != 0)
    return fail(FA_ERR_ARG, "bias strides must be multiples of 4 elements");
  return FA_OK;
}

// Packed offsets in host memory: 0 first, non-decreasing, no sequence
// longer than max_seqlen.
int check_cu_host(const int32_t* cu, int B, int max_seqlen) {
  if (B < 0) return fail(FA_ERR_SHAPE, "B=%d must be >= 0", B);
  if (B == 0) return FA_OK;
  if (cu == nullptr) return fail(FA_ERR_NULL, "cu_seqlens is NULL");
  if (cu[0] != 0) return fail(FA_ERR_ARG, "cu_seqlens[0] = %d, must be 0", cu[0]);
  for (int s = 0; s < B; ++s) {
    const long len = static_cast<long>(cu[s + 1]) - cu[s];
    if (len < 0)
      return fail(FA_ERR_ARG, "cu_seqlens decreases at %d: %d then %d", s, cu[s], cu[s + 1]);
    if (len > max_seqlen)
      return fail(FA_ERR_ARG, "sequence %d has %ld tokens, more than max_seqlen=%d", s, len,
                  max_seqlen);
  }
  return FA_OK;
}

// FA_CHECK_INPUTS set (and not "0"): copy the device cu_seqlens to the host
// on the call's stream, wait for it, and check it before any launch.
int check_cu_device_if_asked(const int32_t* cu, int B, int max_seqlen, hipStream_t stream) {
  const char* env = std::getenv("FA_CHECK_INPUTS");
  if (cu == nullptr || env == nullptr || env[0] == '\0' || std::strcmp(env, "0") == 0)
    return FA_OK;
  std::vector<int32_t> host(static_cast<size_t>(B) + 1);
  hipError_t e = hipMemcpyAsync(host.data(), cu, host.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "copying cu_seqlens to the host failed: %s", hipGetErrorString(e));
  return check_cu_host(host.data(), B, max_seqlen);
}

// A window bound of max(Nq, Nk) or more restricts nothing (local indices
// differ by less than that), so larger bounds are clamped there: the
// kernels then form i + bound without int overflow. -1 (any negative)
// stays "unbounded".
int clamp_window(int bound, int Nq, int Nk) {
  if (bound < 0) return -1;
  return std::min(bound, std::max(Nq, Nk));
}

int run(bool bf16, const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
        int Hkv, int Nq, int Nk, int d, float scale, int causal, const int32_t* cu_seqlens,
        void* stream, int win_left = -1, int win_right = -1, const BiasArg* bias = nullptr) {
  g_last_error[0] = '\0';
  bool noop = false;
  const int tile_rows = bf16 ? fa::kBf16TileRows : fa::kFp32TileRows;
  int st = validate(Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, cu_seqlens, tile_rows, &noop);
  if (st != FA_OK || noop) return st;
  if (bias != nullptr && (st = validate_bias(*bias, Nk)) != FA_OK) return st;
  if ((win_left >= 0 || win_right >= 0) && std::max(Nq, Nk) > (1 << 30))
    return fail(FA_ERR_SHAPE, "a sliding window needs Nq, Nk <= 2^30");
  int cus = 0;
  st = check_device(&cus);
  if (st != FA_OK) return st;
  st = check_cu_device_if_asked(cu_seqlens, B, Nq, static_cast<hipStream_t>(stream));
  if (st != FA_OK) return st;
  fa::FwdParams p;
  p.num_cus = cus;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.cu_seqlens = cu_seqlens;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.nq = Nq;
  p.nk = Nk;
  p.d = d;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.causal = causal ? 1 : 0;
  p.win_left = clamp_window(win_left, Nq, Nk);
  p.win_right = clamp_window(win_right, Nq, Nk);
  p.scale = scale;
  p.bias = bias ? bias->ptr : nullptr;
  p.bias_sb = bias ? bias->sb : 0;
  p.bias_sh = bias ? bias->sh : 0;
  p.bias_sr = bias ? bias->sr : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!bf16)
    e = fa::launch_fwd_fp32(p, s);
  else if (d == 64)
    e = causal ? fa::launch_fwd_bf16<64, true>(p, s) : fa::launch_fwd_bf16<64, false>(p, s);
  else
    e = causal ? fa::launch_fwd_bf16<128, true>(p, s) : fa::launch_fwd_bf16<128, false>(p, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

// Checks of fa_bwd. Unlike the forward, an empty side does not make the
// call a no-op: with Nq == 0 every dK and dV row is zero, and with Nk == 0
// every dQ row is zero, and the kernels write those zeros.
int validate_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                 const float* LSE, const void* dQ, const void* dK, const void* dV,
                 const float* Dsum, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                 const int32_t* cu_seqlens, bool* noop) {
  *noop = false;
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B=%d, Nq=%d, Nk=%d must be >= 0", B, Nq, Nk);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_SHAPE, "Hq=%d and Hkv=%d must be > 0", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (cu_seqlens != nullptr && Nq != Nk)
    return fail(FA_ERR_SHAPE, "packed sequences need Nq == Nk (the maximum length); got %d, %d",
                Nq, Nk);
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head width d=%d; supported: 64, 128", d);
  if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale is not finite");
  if (B == 0 || (Nq == 0 && Nk == 0)) {
    *noop = true;
    return FA_OK;
  }
  const bool has_q = Nq > 0, has_k = Nk > 0;
  if ((has_q && (!Q || !O || !dO || !LSE || !Dsum || !dQ)) || (has_k && (!K || !V || !dK || !dV)))
    return fail(FA_ERR_NULL,
                "every buffer of a non-empty side must be non-NULL (query side: Q, O, dO, LSE, "
                "Dsum, dQ; key side: K, V, dK, dV)");
  const void* p16[] = {Q, K, V, O, dO, dQ, dK, dV};
  for (const void* ptr : p16)
    if (ptr && !aligned(ptr, 16))
      return fail(FA_ERR_ARG, "Q, K, V, O, dO, dQ, dK and dV must be 16-byte aligned");
  if ((LSE && !aligned(LSE, 16)) || (Dsum && !aligned(Dsum, 16)))
    return fail(FA_ERR_ARG, "LSE and Dsum must be 16-byte aligned");
  if (cu_seqlens && !aligned(cu_seqlens, 4))
    return fail(FA_ERR_ARG, "cu_seqlens must be 4-byte aligned");
  const long tiles = (static_cast<long>(std::max(Nq, Nk)) + 127) / 128;
  if (tiles * std::max(Hq, Hkv) * static_cast<long>(B) > 0x7fffffffL ||
      static_cast<long>(B) * Nq * Hq * (d / 8) > 0x7fffffffL * 256L)
    return fail(FA_ERR_SHAPE, "problem exceeds the launch limits");
  return FA_OK;
}

int run_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
            const float* LSE, void* dQ, void* dK, void* dV, float* Dsum, int B, int Hq, int Hkv,
            int Nq, int Nk, int d, float scale, int causal, const int32_t* cu_seqlens,
            void* stream, int win_left = -1, int win_right = -1, const BiasArg* bias = nullptr) {
  g_last_error[0] = '\0';
  bool noop = false;
  int st = validate_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, Dsum, B, Hq, Hkv, Nq, Nk, d, scale,
                        cu_seqlens, &noop);
  if (st != FA_OK || noop) return st;
  if (bias != nullptr && (st = validate_bias(*bias, Nk)) != FA_OK) return st;
  if ((win_left >= 0 || win_right >= 0) && std::max(Nq, Nk) > (1 << 30))
    return fail(FA_ERR_SHAPE, "a sliding window needs Nq, Nk <= 2^30");
  st = check_device();
  if (st != FA_OK) return st;
  st = check_cu_device_if_asked(cu_seqlens, B, Nq, static_cast<hipStream_t>(stream));
  if (st != FA_OK) return st;
  fa::BwdParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.dout = dO;
  p.lse = LSE;
  p.dq = dQ;
  p.dk = dK;
  p.dv = dV;
  p.dsum = Dsum;
  p.cu_seqlens = cu_seqlens;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.nq = Nq;
  p.nk = Nk;
  p.d = d;
  p.scale = scale;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.causal = causal ? 1 : 0;
  p.win_left = clamp_window(win_left, Nq, Nk);
  p.win_right = clamp_window(win_right, Nq, Nk);
  p.bias = bias ? bias->ptr : nullptr;
  p.bias_sb = bias ? bias->sb : 0;
  p.bias_sh = bias ? bias->sh : 0;
  p.bias_sr = bias ? bias->sr : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (d == 64)
    e = causal ? fa::launch_bwd_bf16<64, true>(p, s) : fa::launch_bwd_bf16<64, false>(p, s);
  else
    e = causal ? fa::launch_bwd_bf16<128, true>(p, s) : fa::launch_bwd_bf16<128, false>(p, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

constexpr int kMaxSplits = 1024;
constexpr int kDecodeRows = 32;  // query rows of one K/V head's group per split workgroup

size_t decode_workspace(int B, int Hq, int Nq, int d, int n_splits) {
  const size_t rows = static_cast<size_t>(B) * Hq * Nq * n_splits;
  const size_t o_bytes = rows * d * 4;
  return ((o_bytes + 255) / 256) * 256 + rows * 4;
}

// use_scratch: the library's own device array takes the place of the
// workspace (fa_fwd_splitkv_noalloc); `workspace` is then ignored.
int run_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
                int Hkv, int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
                int n_splits, void* workspace, size_t workspace_bytes, void* stream,
                bool use_scratch = false) {
  g_last_error[0] = '\0';
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B=%d, Nq=%d, Nk=%d must be >= 0", B, Nq, Nk);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_SHAPE, "Hq=%d and Hkv=%d must be > 0", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d != 64 && d != 128)
    return fail(FA_ERR_UNSUPPORTED, "head width d=%d; supported: 64, 128", d);
  if (static_cast<long>(Hq / Hkv) * Nq > kDecodeRows)
    return fail(FA_ERR_UNSUPPORTED,
                "(Hq/Hkv) * Nq = %d query rows per K/V head; the split-K/V path takes at most %d "
                "(use fa_fwd for longer query blocks)", (Hq / Hkv) * Nq, kDecodeRows);
  if (n_splits < 1 || n_splits > kMaxSplits)
    return fail(FA_ERR_ARG, "num_splits=%d must be in 1..%d", n_splits, kMaxSplits);
  if (!std::isfinite(scale)) return fail(FA_ERR_ARG, "scale is not finite");
  if (B == 0 || Nq == 0) return FA_OK;
  if (!Q || !O || !LSE || (!use_scratch && !workspace) || (Nk > 0 && (!K || !V)))
    return fail(FA_ERR_NULL, "Q, O, LSE, workspace (and K, V when Nk > 0) must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      (!use_scratch && !aligned(workspace, 256)))
    return fail(FA_ERR_ARG, "Q, K, V and O must be 16-byte aligned, workspace 256-byte aligned");
  if (!aligned(LSE, 4) || (seqlens_k && !aligned(seqlens_k, 4)))
    return fail(FA_ERR_ARG, "LSE and seqlens_k must be 4-byte aligned");
  const size_t need = decode_workspace(B, Hq, Nq, d, n_splits);
  if (use_scratch && need > fa::kNoAllocScratchBytes)
    return fail(FA_ERR_ARG,
                "the call needs %zu bytes of split scratch; fa_fwd_splitkv_noalloc holds %zu "
                "(fewer splits or a smaller batch, or fa_fwd_splitkv with a workspace)",
                need, fa::kNoAllocScratchBytes);
  if (!use_scratch && workspace_bytes < need)
    return fail(FA_ERR_ARG, "workspace of %zu bytes; %zu needed", workspace_bytes, need);
  if (static_cast<long>(B) * Hkv * n_splits > 0x7fffffffL)
    return fail(FA_ERR_SHAPE, "grid exceeds the launch limit");
  int st = check_device();
  if (st != FA_OK) return st;
  if (use_scratch) {
    const hipError_t se = fa::decode_scratch(&workspace);
    if (se != hipSuccess)
      return fail(FA_ERR_HIP, "looking up the scratch array failed: %s", hipGetErrorString(se));
  }
  fa::DecodeParams p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.o = O;
  p.lse = LSE;
  p.seqlens_k = seqlens_k;
  const size_t rows = static_cast<size_t>(B) * Hq * Nq * n_splits;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        ((rows * d * 4 + 255) / 256) * 256);
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.nq = Nq;
  p.nk = Nk;
  p.d = d;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  p.causal = causal ? 1 : 0;
  p.n_splits = n_splits;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d == 64 ? fa::launch_decode_bf16<64>(p, s) : fa::launch_decode_bf16<128>(p, s);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

constexpr int kFp8D = 128;
constexpr int kFp8Block = 64;       // keys per V^T tile
constexpr size_t kFp8TileBytes = 8192;

size_t fp8_workspace(int B, int Hkv, int Nk) {
  const size_t nblk = (static_cast<size_t>(Nk) + kFp8Block - 1) / kFp8Block;
  return static_cast<size_t>(B) * Hkv * nblk * kFp8TileBytes;
}

int run_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq, int Hkv,
            int Nq, int Nk, int d, float scale, float q_descale, float k_descale,
            float v_descale, int causal, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (B < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B=%d, Nq=%d, Nk=%d must be >= 0", B, Nq, Nk);
  if (Hq <= 0 || Hkv <= 0) return fail(FA_ERR_SHAPE, "Hq=%d and Hkv=%d must be > 0", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(FA_ERR_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (d != kFp8D) return fail(FA_ERR_UNSUPPORTED, "head width d=%d; the fp8 path takes 128", d);
  if (!std::isfinite(scale) || !std::isfinite(q_descale) || !std::isfinite(k_descale) ||
      !std::isfinite(v_descale))
    return fail(FA_ERR_ARG, "scale and descale factors must be finite");
  const double c = static_cast<double>(scale) * q_descale * k_descale * 1.4426950408889634;
  if (!(std::fabs(c) <= 3.0e38)) return fail(FA_ERR_ARG, "scale * q_descale * k_descale overflows");
  if (B == 0 || Nq == 0) return FA_OK;
  if (!Q || !O || !LSE || (Nk > 0 && (!K || !V || !workspace)))
    return fail(FA_ERR_NULL, "Q, O, LSE (and with keys K, V, workspace) must be non-NULL");
  if (!aligned(Q, 16) || (K && !aligned(K, 16)) || (V && !aligned(V, 16)) || !aligned(O, 16))
    return fail(FA_ERR_ARG, "Q, K, V and O must be 16-byte aligned");
  if (!aligned(LSE, 4)) return fail(FA_ERR_ARG, "LSE must be 4-byte aligned");
  if (workspace && !aligned(workspace, 256))
    return fail(FA_ERR_ARG, "workspace must be 256-byte aligned");
  const size_t need = fp8_workspace(B, Hkv, Nk);
  if (Nk > 0 && workspace_bytes < need)
    return fail(FA_ERR_ARG, "workspace of %zu bytes is below the %zu the call needs",
                workspace_bytes, need);
  const int64_t n_qt = (static_cast<int64_t>(Nq) + 255) / 256;
  const int64_t nblk = (static_cast<int64_t>(Nk) + kFp8Block - 1) / kFp8Block;
  if (n_qt * Hq * static_cast<int64_t>(B) > 0x7fffffffLL ||
      nblk * Hkv * static_cast<int64_t>(B) > 0x7fffffffLL)
    return fail(FA_ERR_SHAPE, "problem exceeds the launch limits");
  int st = check_device();
  if (st != FA_OK) return st;
  fa::Fp8Params p;
  p.q = Q;
  p.k = K;
  p.v = V;
  p.vt = workspace;
  p.o = O;
  p.lse = LSE;
  p.batch = B;
  p.hq = Hq;
  p.hkv = Hkv;
  p.nq = Nq;
  p.nk = Nk;
  p.nblk = static_cast<int>(nblk);
  p.c = static_cast<float>(c);
  p.v_descale = v_descale;
  p.causal = causal ? 1 : 0;
  const hipError_t e = fa::launch_fwd_fp8(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq, int Hkv,
           int Nq, int Nk, int d, float scale, int causal, const int32_t* cu_seqlens,
           void* stream) {
  return run(true, Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream);
}

int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
                  int Hkv, int Nq, int Nk, int d, float scale, int causal, int window_left,
                  int window_right, const int32_t* cu_seqlens, void* stream) {
  return run(true, Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream,
             window_left, window_right);
}

int fa_fwd_bias(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
                int Hkv, int Nq, int Nk, int d, float scale, int causal, const void* bias,
                int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_row,
                const int32_t* cu_seqlens, void* stream) {
  const BiasArg b{bias, bias_stride_b, bias_stride_h, bias_stride_row};
  return run(true, Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream, -1,
             -1, &b);
}

int fa_fwd_fp32(const float* Q, const float* K, const float* V, float* O, float* LSE, int B,
                int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                const int32_t* cu_seqlens, void* stream) {
  return run(false, Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, cu_seqlens, stream);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV, float* Dsum, int B, int Hq, int Hkv,
           int Nq, int Nk, int d, float scale, int causal, const int32_t* cu_seqlens,
           void* stream) {
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, Dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 cu_seqlens, stream);
}

int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* LSE, void* dQ, void* dK, void* dV, float* Dsum, int B, int Hq,
                  int Hkv, int Nq, int Nk, int d, float scale, int causal, int window_left,
                  int window_right, const int32_t* cu_seqlens, void* stream) {
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, Dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 cu_seqlens, stream, window_left, window_right);
}

int fa_bwd_bias(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, void* dQ, void* dK, void* dV, float* Dsum, int B, int Hq,
                int Hkv, int Nq, int Nk, int d, float scale, int causal, const void* bias,
                int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_row,
                const int32_t* cu_seqlens, void* stream) {
  const BiasArg b{bias, bias_stride_b, bias_stride_h, bias_stride_row};
  return run_bwd(Q, K, V, O, dO, LSE, dQ, dK, dV, Dsum, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 cu_seqlens, stream, -1, -1, &b);
}

size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || d <= 0 || num_splits <= 0) return 0;
  return decode_workspace(B, Hq, Nq, d, num_splits);
}

int fa_fwd_splitkv_num_splits(int B, int Hkv, int Nk, int num_cus) {
  g_last_error[0] = '\0';
  if (B < 1 || Hkv < 1 || Nk < 1)
    return fail(FA_ERR_SHAPE, "B=%d, Hkv=%d and Nk=%d must all be at least 1", B, Hkv, Nk);
  if (num_cus <= 0) {
    const int st = check_device(&num_cus);
    if (st != FA_OK) return st;
  }
  const int64_t units = static_cast<int64_t>(B) * Hkv;
  const int64_t want = (3 * static_cast<int64_t>(num_cus) + units / 2) / units;
  const int64_t cap = std::min<int64_t>(1024, std::max<int64_t>(1, Nk / 512));
  return static_cast<int>(std::max<int64_t>(1, std::min(want, cap)));
}

int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   const int32_t* seqlens_k, int num_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return run_splitkv(Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, seqlens_k, num_splits,
                     workspace, workspace_bytes, stream);
}

static_assert(FA_NOALLOC_SCRATCH_BYTES == fa::kNoAllocScratchBytes, "scratch size in the header");

int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                           const int32_t* seqlens_k, int num_splits, void* stream) {
  return run_splitkv(Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, causal, seqlens_k, num_splits,
                     nullptr, 0, stream, /*use_scratch=*/true);
}

size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Nk) {
  if (B <= 0 || Hkv <= 0 || Nk <= 0) return 0;
  return fp8_workspace(B, Hkv, Nk);
}

int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
               int Hkv, int Nq, int Nk, int d, float scale, float q_descale, float k_descale,
               float v_descale, int causal, void* workspace, size_t workspace_bytes,
               void* stream) {
  return run_fp8(Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, d, scale, q_descale, k_descale, v_descale,
                 causal, workspace, workspace_bytes, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head width or device not supported";
    case FA_ERR_ARG: return "FA_ERR_ARG: non-finite scale or misaligned pointer";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_last_error; }

int fa_check_cu_seqlens(const int32_t* cu_seqlens_host, int B, int max_seqlen) {
  g_last_error[0] = '\0';
  return check_cu_host(cu_seqlens_host, B, max_seqlen);
}

int fa_version(void) { return kVersion; }

}  // extern "C"
