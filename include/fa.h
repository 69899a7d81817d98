/*
 * libfa: exact tiled scaled-dot-product attention, forward pass and its
 * backward pass by recomputation, for AMD Instinct MI355X (gfx950). C ABI.
 *
 * The operation ("Softmax does not need the matrix", opening equation and
 * section "Carry the Normalizer"; "Understanding FlashAttention Pt 1:
 * Personal Notes", section 0.2 Notation):
 *
 *     S = scale * Q K^T,   P = softmax_row(S),   O = P V,
 *     LSE_i = ln sum_{visible j} exp(S_ij)
 *
 * computed exactly (up to floating-point rounding order) without ever
 * storing S or P: for each query tile the kernel streams K/V blocks through
 * on-chip memory, updates the running row state (m, l, a) with the
 * exp(m - m') rescale ("Carry the Normalizer"), and writes only O and the
 * per-row log-sum-exp ("Understanding FlashAttention Pt 1", section 1.2: a
 * score tile is computed, used with V_j and discarded; semiaifoundry
 * "attention-io-tiling", section The mechanism).
 *
 * Layout. Every buffer is contiguous, row-major and token-major.
 *   Fixed length (cu_seqlens == NULL):
 *     Q [B, Nq, Hq, d]   K, V [B, Nk, Hkv, d]   O [B, Nq, Hq, d]
 *     LSE [B, Hq, Nq] (float32)
 *   Packed variable length (cu_seqlens != NULL):
 *     B is the number of sequences; cu_seqlens is int32 [B + 1] in DEVICE
 *     memory, cu_seqlens[0] = 0, non-decreasing; sequence s owns tokens
 *     cu_seqlens[s] .. cu_seqlens[s+1]-1 on both the query and key side
 *     (self-attention; no attention across sequences).
 *     Q, O [T, Hq, d]   K, V [T, Hkv, d]   LSE [Hq, T],  T = cu_seqlens[B].
 *     Nq and Nk must both equal the largest sequence length (it sizes the
 *     grid); rows of a longer sequence beyond Nq are not written.
 *
 * Semantics.
 *   - scale is applied to Q K^T (the usual value is 1/sqrt(d)).
 *   - causal != 0 keeps key j for query i iff j <= i (top-left
 *     lower-triangular, indices local to the batch entry or sequence).
 *   - Grouped-query attention: Hq % Hkv == 0 and query head h reads K/V
 *     head h / (Hq / Hkv) (contiguous groups; Hkv == 1 is multi-query).
 *   - A row that sees no key (Nk == 0, or an empty sequence) gets O = 0 and
 *     LSE = -inf.
 *   - fa_fwd: Q, K, V, O are bfloat16 (stored as 16-bit words); scores,
 *     softmax state and accumulation are float32; P is rounded to bf16 for
 *     the P V product; O is normalised in float32 and rounded to bf16 once
 *     (round to nearest even). fa_fwd_fp32: everything float32.
 *   - Results are exact up to rounding order, not bitwise equal to another
 *     implementation; repeated calls with the same inputs on the same device
 *     give bitwise-identical outputs.
 *
 * Ownership. The caller allocates every buffer on the current HIP device
 * and keeps it alive until the work on `stream` completes. The library
 * allocates no device memory, keeps no pointer after returning, and does
 * not synchronise. `stream` is a hipStream_t (NULL = the null stream).
 * Calls are thread-safe.
 *
 * Errors. Every function returns a status (FA_OK or a negative FA_ERR_*);
 * no exception crosses the ABI. All argument checks run on the host before
 * any HIP call. fa_last_error() gives a thread-local message for the last
 * failing call on this thread. Device-side faults are asynchronous and
 * surface at the caller's next synchronisation. The contents of cu_seqlens
 * live on the device and are not checked by default: offsets that are
 * decreasing or exceed the buffers are undefined behaviour. With the
 * environment variable FA_CHECK_INPUTS set to a value other than "0", every
 * call that takes cu_seqlens first copies it to the host (synchronising
 * `stream`) and checks it with fa_check_cu_seqlens; a bad array fails the
 * call with FA_ERR_ARG before any kernel is launched.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* B/Hq/Hkv/Nq/Nk inconsistent or out of range */
  FA_ERR_UNSUPPORTED = -3, /* head width d not in {64, 128}, or not gfx950 */
  FA_ERR_ARG = -4,         /* scale not finite, or a pointer misaligned */
  FA_ERR_HIP = -5          /* a HIP runtime call or the launch failed */
};

/*
 * Attention forward, bf16 inputs and output, float32 LSE.
 *   Q, K, V, O : device pointers, bf16, 16-byte aligned, layouts above.
 *   LSE        : device pointer, float32, 4-byte aligned (required).
 *   B          : batch size, or number of sequences when packed (B >= 0;
 *                B == 0 is a no-op).
 *   Hq, Hkv    : query and K/V head counts, Hq % Hkv == 0.
 *   Nq, Nk     : query and key lengths (>= 0; Nq == 0 is a no-op); packed:
 *                both the maximum sequence length.
 *   d          : head width, 64 or 128.
 *   scale      : finite float applied to Q K^T.
 *   causal     : 0 or non-zero (top-left mask, see above).
 *   cu_seqlens : NULL for fixed length, else device int32 [B + 1].
 *   stream     : hipStream_t to launch on.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int Hq, int Hkv, int Nq, int Nk, int d,
           float scale, int causal, const int32_t* cu_seqlens, void* stream);

/*
 * fa_fwd with a sliding (local) window: query i sees only keys j with
 * i - window_left <= j <= i + window_right (indices local to the batch entry
 * or sequence), ANDed with the causal mask when causal != 0; a negative
 * bound is unbounded, and with both negative the call is fa_fwd. The pages
 * name local attention and sliding windows as variants of the mask
 * ("Understanding FlashAttention Pt 1: Personal Notes", contents, section
 * 4.2; "Softmax does not need the matrix", section "Quadratic Time Did Not
 * Vanish"). Key blocks outside every window of a query tile are not read.
 * A row whose window holds no key gets O = 0 and LSE = -inf. bf16; other
 * arguments and errors as fa_fwd.
 */
int fa_fwd_window(const void* Q, const void* K, const void* V, void* O,
                  float* LSE, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                  float scale, int causal, int window_left, int window_right,
                  const int32_t* cu_seqlens, void* stream);

/*
 * fa_fwd with an additive bias B in the scores: S = scale * Q K^T + B,
 * P = softmax_row(S) over the visible keys ("Understanding FlashAttention
 * Pt 1: Personal Notes", section 0.2 Notation, where B is an optional
 * additive mask or bias).
 *   bias : device pointer, bf16, 8-byte aligned. Element (s, h, i, j), for
 *          batch entry (or packed sequence) s, query head h, query i and
 *          key j (i, j local to the entry or sequence), is
 *          bias[s*bias_stride_b + h*bias_stride_h + i*bias_stride_row + j].
 *   bias_stride_b, bias_stride_h : >= 0, in elements; 0 shares one bias
 *          over every entry or every head.
 *   bias_stride_row : in elements, >= Nk.
 *   All three strides must be multiples of 4. Bias rows are read in aligned
 *   runs of 4 elements, so positions up to the next multiple of 4 past a
 *   row's last key must be readable (values read past the last key are
 *   ignored); a row stride that is a multiple of 4 and >= Nk guarantees
 *   this inside a row.
 * The causal mask still applies (a masked pair stays masked whatever B
 * holds). B may hold -inf, which removes a pair; a row left with no visible
 * pair gets O = 0 and LSE = -inf. +inf or NaN in B give undefined results.
 * LSE is the log-sum-exp of the biased scores. No sliding window with a
 * bias (a window is a bias of 0 and -inf). No gradient with respect to B.
 * Other arguments and errors as fa_fwd.
 */
int fa_fwd_bias(const void* Q, const void* K, const void* V, void* O, float* LSE,
                int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                int causal, const void* bias, int64_t bias_stride_b,
                int64_t bias_stride_h, int64_t bias_stride_row,
                const int32_t* cu_seqlens, void* stream);

/* Same contract with float32 Q, K, V, O (no bf16 rounding anywhere). */
int fa_fwd_fp32(const float* Q, const float* K, const float* V, float* O,
                float* LSE, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, const int32_t* cu_seqlens,
                void* stream);

/*
 * Attention backward by recomputation, bf16. The gradients of the forward
 * function above for an upstream gradient dO ("Understanding FlashAttention
 * Pt 1: Personal Notes", contents, section 3.6 "Backward pass: recompute
 * instead of save"; semiaifoundry "attention-io-tiling", section
 * Specifications and interfaces: the retained statistics and permitted
 * recomputation serve the backward execution):
 *
 *     P = exp(scale Q K^T - LSE) on visible pairs (recomputed, never stored)
 *     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
 *     dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q
 *
 * with the mask, grouped-query mapping and packed-sequence rules of fa_fwd;
 * a K/V head's dK and dV are the sums over the query heads that read it.
 *   Q, K, V    : the forward inputs (bf16, layouts as fa_fwd).
 *   O, LSE     : what fa_fwd wrote for these inputs (LSE float32).
 *   dO         : upstream gradient, bf16, laid out like O.
 *   dQ, dK, dV : outputs, bf16, laid out like Q, K, V; every row of a
 *                token that exists is written (rows that no query or key
 *                sees get zeros). Float32 accumulation, one rounding.
 *   Dsum       : float32 scratch laid out like LSE, owned by the caller; the
 *                call writes D there first and reads it back.
 *   other arguments as fa_fwd. Alignment: 16 bytes for every tensor,
 *   including LSE and Dsum.
 * B == 0, or Nq == Nk == 0, is a no-op. With Nq == 0 only K, V, dK, dV are
 * used (dK = dV = 0); with Nk == 0 only the query-side buffers (dQ = 0).
 * Errors as fa_fwd; d must be 64 or 128.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
           float* Dsum, int B, int Hq, int Hkv, int Nq, int Nk, int d,
           float scale, int causal, const int32_t* cu_seqlens, void* stream);

/* fa_bwd for the sliding-window forward of fa_fwd_window: the same window
 * (LSE and O from fa_fwd_window with these window bounds). */
int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O,
                  const void* dO, const float* LSE, void* dQ, void* dK,
                  void* dV, float* Dsum, int B, int Hq, int Hkv, int Nq,
                  int Nk, int d, float scale, int causal, int window_left,
                  int window_right, const int32_t* cu_seqlens, void* stream);

/* fa_bwd for the biased forward of fa_fwd_bias: the same bias (bias and
 * strides as fa_fwd_bias; LSE and O from fa_fwd_bias with this bias). The
 * probabilities are recomputed as P = exp(scale Q K^T + B - LSE); a row
 * whose LSE is -inf (no finite biased score) contributes nothing. No
 * gradient with respect to B is formed. */
int fa_bwd_bias(const void* Q, const void* K, const void* V, const void* O,
                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                float* Dsum, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, const void* bias, int64_t bias_stride_b,
                int64_t bias_stride_h, int64_t bias_stride_row,
                const int32_t* cu_seqlens, void* stream);

/*
 * Split-K/V attention forward for decode-shaped problems, bf16: the same
 * function as fa_fwd (fixed-length layout, same mask and grouping) for few
 * query rows per head and a long K/V cache ("Understanding FlashAttention
 * Pt 1: Personal Notes", contents, section 8.1: prefill and decode are
 * different regimes). The keys of every (batch entry, K/V head) are cut into
 * num_splits ranges; each range yields a softmax-normalised partial output
 * and its log-sum-exp, and a second pass merges them with the block merge
 * rule of "Softmax does not need the matrix", section "Carry the
 * Normalizer": LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *   Q, O       : [B, Nq, Hq, d] bf16; K, V : [B, Nk, Hkv, d] bf16 (a cache
 *                with room for Nk keys per batch entry); LSE : [B, Hq, Nq].
 *   seqlens_k  : NULL (every entry has Nk keys) or device int32 [B], the
 *                number of valid keys of each entry (clamped to 0 .. Nk);
 *                keys past it are never read.
 *   causal     : top-left mask as fa_fwd (query i sees keys j <= i); for
 *                one new token attending to a whole cache pass 0.
 *   num_splits : 1 .. 1024 key ranges per (batch entry, K/V head).
 *   workspace  : device memory of at least
 *                fa_fwd_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits)
 *                bytes, 256-byte aligned, owned by the caller (partial O
 *                and LSE of every split); its contents on return are
 *                unspecified.
 * (Hq / Hkv) * Nq must be at most 32: the query rows of one K/V head's group
 * form one tile (FA_ERR_UNSUPPORTED otherwise; use fa_fwd). B == 0 or
 * Nq == 0 is a no-op. Other arguments and errors as fa_fwd.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits);

/*
 * A split count for fa_fwd_splitkv: enough key ranges that the split pass
 * fills about three workgroups per compute unit, round(3 * num_cus / (B *
 * Hkv)), clamped to 1 .. min(1024, max(1, Nk / 512)) so that a range keeps
 * at least 512 keys. num_cus <= 0 takes the current device's count. Returns
 * the count (>= 1), or a negative FA_ERR_* (B, Hkv or Nk < 1: FA_ERR_SHAPE;
 * no usable device when num_cus <= 0: as fa_fwd). Host only; launches
 * nothing.
 */
int fa_fwd_splitkv_num_splits(int B, int Hkv, int Nk, int num_cus);
int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O,
                   float* LSE, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   float scale, int causal, const int32_t* seqlens_k,
                   int num_splits, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * fa_fwd_splitkv without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The partial results live in a
 * device array the library holds, FA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU
 * for the life of the process; a call whose
 * fa_fwd_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits) exceeds that
 * fails with FA_ERR_ARG before any HIP call. The call allocates nothing.
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (different streams, or threads without ordering) race and their
 * results are undefined; calls ordered on one stream are safe. Other
 * arguments, results and errors as fa_fwd_splitkv.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O,
                           float* LSE, int B, int Hq, int Hkv, int Nq, int Nk,
                           int d, float scale, int causal,
                           const int32_t* seqlens_k, int num_splits,
                           void* stream);

/*
 * Attention forward with FP8 inputs: Q, K, V in OCP e4m3 (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities, 0x7f / 0xff
 * are NaN) with one dequantization factor per tensor. The function is the
 * attention of the dequantized inputs q = q_descale * Q, k = k_descale * K,
 * v = v_descale * V: S = scale q k^T, P = softmax_row(S), O = P v, LSE as
 * fa_fwd. The pages list FP8 as FlashAttention-3's low-precision variant
 * and state that its speed has a precision cost ("Understanding
 * FlashAttention Pt 1: Personal Notes", contents, section 5.6). The cost
 * here is one rounding: the scores are exact products summed in float32;
 * the probabilities are rounded to e4m3 for the P V product (an absolute
 * error of at most 2^-4 P_ij, or 2^-17 of the row's weight sum when
 * that is larger, per term); O is rounded once to bf16.
 *   Q [B, Nq, Hq, 128], K, V [B, Nk, Hkv, 128] : device, e4m3 bytes,
 *            16-byte aligned. Fixed length only; d must be 128.
 *   O [B, Nq, Hq, 128] : device, bf16, 16-byte aligned.
 *   LSE [B, Hq, Nq] : device, float32.
 *   scale, q_descale, k_descale, v_descale : finite floats.
 *   causal : top-left mask as fa_fwd.
 *   workspace : device memory of at least fa_fwd_fp8_workspace_bytes(B,
 *            Hkv, Nk) bytes, 256-byte aligned, owned by the caller; the call
 *            writes V, transposed in 64-key tiles, there first (its contents
 *            on return are unspecified). May be NULL when Nk == 0.
 * B == 0 or Nq == 0 is a no-op. Errors as fa_fwd; FA_ERR_UNSUPPORTED for
 * d != 128.
 */
size_t fa_fwd_fp8_workspace_bytes(int B, int Hkv, int Nk);
int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
               float q_descale, float k_descale, float v_descale, int causal,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host-side check of a packed-sequence offset array (the one fa_fwd and
 * fa_bwd take as cu_seqlens), here in HOST memory: cu_seqlens_host[0] == 0,
 * non-decreasing, and no sequence longer than max_seqlen. Returns FA_OK,
 * FA_ERR_NULL (NULL array with B > 0), FA_ERR_SHAPE (B < 0) or FA_ERR_ARG
 * (the first violation, named in fa_last_error()). Reads B + 1 values; no
 * HIP call.
 */
int fa_check_cu_seqlens(const int32_t* cu_seqlens_host, int B, int max_seqlen);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* fa_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
