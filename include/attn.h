/*
 * attn.h -- C ABI of the exact IO-aware attention library for MI355X (gfx950).
 *
 * What it computes. For every batch b, query head h (KV head h / (Hq/Hkv)),
 * query row i and key j:
 *     s_ij  = scale * q_i . k_j                      (masked keys: s_ij = -inf)
 *     O_i   = sum_j softmax_j(s_i.) v_j,   lse_i = ln sum_j exp(s_ij)
 * exactly as the plain definition (Attention = softmax(QK^T/sqrt(d_k))V of
 * "Flash Attention FA1->FA4 / pre-training practice", §1.1), but computed
 * tile by tile with the online-softmax recurrence of the same page, §1.2, in
 * the unnormalised (m, l, u) form of "AI 大模型之 FlashAttention_01",
 * §4.1 and section "瓦片状态如何保持精确语义". The score matrix never
 * reaches device memory; the forward keeps only O and the per-row lse, and
 * the backward rebuilds the probabilities tile by tile from them (same page,
 * section "反向传播为什么可以重算").
 *
 * Layout. Every tensor is contiguous, row-major [B, H, S, d]:
 *   q, o, dout, dq : [B, Hq,  Sq, d]      k, v, dk, dv : [B, Hkv, Sk, d]
 *   lse            : [B, Hq,  Sq] float32, natural log
 * Element type is given by `dtype` (ATTN_F32 or ATTN_BF16) for q, k, v, o,
 * dout, dq, dk, dv; lse is always float32. All pointers are device pointers
 * (memory from hipMalloc or a PyTorch CUDA/HIP tensor) except `buf` of
 * attn_last_dispatch, which is host memory.
 *
 * Masks (`causal`): 0 = none; 1 = top-left, key j visible to query i iff
 * j <= i; 2 = bottom-right, j <= i + Sk - Sq. The two coincide when Sq == Sk.
 * A query row that sees no key (Sk == 0, or causal == 2 with i < Sq - Sk)
 * gets O = 0, lse = -inf, dq = 0, and adds nothing to dk or dv. This is the
 * explicit rule for fully masked rows that "AI 大模型之 FlashAttention_01"
 * (section "工程实操") asks an interface to define.
 *
 * Alignment: the kernels move data in 16-byte vectors, so every tensor
 * pointer (q, k, v, o, dout, dq, dk, dv, the FP8 code arrays, the bf16 input
 * of the quantisers) and the workspace must be 16-byte aligned; lse and the
 * FP8 scale arrays must be 4-byte aligned. A misaligned pointer returns
 * ATTN_ERR_ALIGN before anything is launched. (Memory from hipMalloc or a
 * PyTorch allocation is 256-byte aligned; a view that starts at an odd
 * element offset may not be.)
 *
 * Restrictions (the kernels are specialised, as that page's limitations
 * section notes for high-performance attention kernels): d in {64, 128};
 * Hq a multiple of Hkv (grouped heads are contiguous); scale finite and > 0;
 * Sq and Sk below 2^24 per head, B*Hq*Sq and B*Hkv*Sk below 2^31;
 * backward in ATTN_BF16 only; gfx950 only.
 *
 * Ownership and errors. The caller allocates every buffer, including the
 * workspace (size from the *_workspace_bytes queries); the library allocates
 * no device memory and keeps no pointer after a call returns. Arguments are
 * validated on the host before anything is launched: on error the function
 * returns a negative status, launches nothing and leaves every output
 * untouched. Work is enqueued asynchronously on `stream` (a hipStream_t; NULL
 * means the default stream); the library never synchronises, so a device
 * fault surfaces at the caller's next synchronisation. A failed launch returns
 * ATTN_ERR_HIP. No C++ exception crosses this interface. Calls may come from
 * several host threads; the dispatch record is per thread.
 */
#ifndef EXACT_ATTN_MI355X_H
#define EXACT_ATTN_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,       /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,      /* B, Hq, Hkv, Sq < 1, or Sk < 0, or a size past its limit */
  ATTN_ERR_GQA = -3,        /* Hq is not a multiple of Hkv */
  ATTN_ERR_HEADDIM = -4,    /* d not in {64, 128} */
  ATTN_ERR_DTYPE = -5,      /* unknown dtype, or not supported by this entry point */
  ATTN_ERR_CAUSAL = -6,     /* causal not in {0, 1, 2} */
  ATTN_ERR_WORKSPACE = -7,  /* workspace smaller than the query says, or NULL when needed */
  ATTN_ERR_HIP = -8,        /* a HIP runtime call or kernel launch failed */
  ATTN_ERR_SCALE = -9,      /* scale not finite or not > 0 */
  ATTN_ERR_DROPOUT = -10,   /* dropout probability not in [0, 1) or rounding to 1 */
  ATTN_ERR_ALIGN = -11,     /* a data pointer lacks the alignment stated above */
  ATTN_ERR_SCRATCH = -12    /* attn_fwd_noalloc: more scratch needed than its static buffer holds */
};

enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1 };

/* Bytes of device workspace attn_fwd needs for these arguments (0 if none).
 * Only the ATTN_BF16 split-key decode path (Hq/Hkv * Sq <= 32, e.g. one
 * query row) needs any: it keeps per-split partial results there. The bf16
 * prefill and ATTN_F32 read their inputs in place and need none. Returns 0
 * for invalid arguments too; the call then reports the error. */
size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d,
                                int causal, int dtype);

/* Forward: o (and lse, if non-NULL) from q, k, v. lse may be NULL when no
 * backward follows (inference keeps no state). k and v may be NULL only when
 * Sk == 0. workspace may be NULL only if attn_fwd_workspace_bytes returns 0. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* attn_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and dispatch as attn_fwd, minus the workspace: the
 * split-key decode path keeps its per-slice partials in a static device array
 * of the library (ATTN_NOALLOC_SCRATCH_BYTES = 16 MiB per GPU, held until the
 * process ends) instead of a caller's workspace; the prefill and fp32 paths
 * need none. No call here allocates or frees device memory. A problem whose
 * partials need more than the array holds (attn_fwd_workspace_bytes above
 * 16 MiB, e.g. decode with B * Hq * Sq * nsplit past about 32K rows at
 * d = 128) returns ATTN_ERR_SCRATCH before anything is launched. Every call
 * on one GPU uses that GPU's one array, and every partial a call reads was
 * written by that call, so nothing needs clearing between calls; but calls
 * that overlap on one GPU (concurrent streams or threads) race on it: run them
 * in order on one stream. The caller's current device must be the stream's. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
                     int dtype, void* stream);

/* Bytes of device workspace attn_bwd needs: the per-row terms D_i = dO_i . O_i
 * and lse_i * log2(e) (float32, 2 * B * Hq * Sq' values with Sq' = Sq rounded
 * up to 64, stored per 32 rows as [lse2 x 32 | -D x 32]), rounded up to 256
 * bytes. The contents are scratch: nothing is kept between calls. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d,
                                int causal, int dtype);

/* Backward of the forward above, given its o and lse and the upstream
 * gradient dout (all required). Writes dq, dk, dv (dk/dv summed over the query
 * heads that share a KV head). Must be called with the same mask, scale and
 * shapes as the forward that produced o and lse. k, v, dk and dv may be NULL
 * only when Sk == 0 (then dq = 0). ATTN_BF16 only. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
             int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* The backward in one pass. attn_bwd runs a dK/dV pass and a separate dQ
 * pass, which rebuilds S and dP a second time, and its results are the same
 * bits on every run. attn_bwd_fused instead forms dV, dK and dQ in a single
 * pass over the (key tile, query tile) pairs, adding each pair's dQ share into
 * float32 sums with atomic adds (the single-pass backward with accumulated dQ
 * that "Flash Attention FA1->FA4 / pre-training practice", §2.3, describes for
 * FA4), then rounds the sums into dq. The order of those additions varies
 * between runs, so dq can differ in its last bits from run to run, and dk/dv
 * differ from attn_bwd's by rounding (another summation order). On MI355X it
 * is slower than attn_bwd (float32 atomic adds are the bottleneck); it is kept
 * for comparison. Same arguments and errors as attn_bwd, with the workspace
 * of attn_bwd_fused_workspace_bytes: attn_bwd's block followed by the float32
 * dQ sums (B * Hq * Sq' * d values, rounded up to 256 bytes). */
size_t attn_bwd_fused_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d,
                                      int causal, int dtype);
int attn_bwd_fused(const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
                   int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Packed variable-length batches ("ragged layout" of the second page,
 * section on interface constraints, where a packed row number and a logical
 * row number are distinct). B sequences of different lengths are stored
 * head-major and back to back: q, o and dout/dq are [Hq, total_q, d], lse is
 * [Hq, total_q], k, v and dk/dv are [Hkv, total_k, d], all contiguous, with
 * total_q = cu_seqlens_q[B] and total_k = cu_seqlens_k[B]. Sequence b holds
 * the packed query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of every head; cu_seqlens_q and
 * cu_seqlens_k are HOST arrays of B+1 ints that start at 0 and never
 * decrease (else ATTN_ERR_SHAPE). Within a sequence the mask uses the logical
 * positions (query i, key j counted from the sequence's first row), exactly
 * as attn_fwd/attn_bwd with Sq and Sk set to that sequence's lengths; rows
 * never attend across sequences. A sequence without queries writes nothing
 * in the forward and zero dk/dv rows in the backward; one without keys gives
 * o = 0, lse = -inf, dq = 0. Every other argument means what it means for
 * attn_fwd/attn_bwd (the per-sequence shape checks apply to each sequence;
 * Hq * total_q and Hkv * total_k must stay below 2^31). All launches go to
 * the given stream. Forward: decode-shaped sequences (Hq/Hkv * length <= 32)
 * and every ATTN_F32 sequence run first, one split-key (or fp32) launch per
 * sequence in batch order, each reusing the start of the one workspace; the
 * remaining bf16 sequences then run as packed grids of up to 64 sequences
 * each (largest work first), which need no workspace. Backward: packed grids
 * of up to 64 sequences (dQ, then dK/dV kernels per grid) over every
 * sequence with queries or keys, in the same order; the workspace holds the
 * lse2/D rows of every sequence at once. So one workspace of the size the
 * query returns serves the whole call. */
size_t attn_fwd_varlen_workspace_bytes(const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                                       int Hq, int Hkv, int d, int causal, int dtype);
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int d, int causal, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream);
size_t attn_bwd_varlen_workspace_bytes(const int* cu_seqlens_q, const int* cu_seqlens_k, int B,
                                       int Hq, int Hkv, int d, int causal, int dtype);
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dout, void* dq, void* dk, void* dv,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int d, int causal, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Dropout on the attention probabilities, regenerated identically by the
 * forward and the backward ("AI 大模型之 FlashAttention_01", section
 * "接口与实现约束": with dropout on, the mapping to random numbers is part of
 * the contract between the two passes). The mapping is Philox4x32-10 (Salmon,
 * Moraes, Dror, Shaw, SC 2011) keyed by the 64-bit `seed`: for query head h of
 * batch b, the 4x4 block of query rows 4a..4a+3 and keys 4c..4c+3 (positions
 * within the problem) takes counter (c, a, b*Hq + h, offset); byte t of output
 * word w belongs to query 4a+w, key 4c+t. The probability P_ij is kept when
 * its byte is >= thr = round(256 * dropout_p), and kept values are scaled by
 * 1 / (1 - thr / 256): the effective dropout probability is thr / 256.
 * dropout_p must lie in [0, 1) with thr <= 255 (else ATTN_ERR_DROPOUT). The
 * forward keeps lse of the undropped probabilities; O = (P o Z) V with
 * Z = keep / (1 - thr / 256). The backward with the same seed, offset and
 * dropout_p returns the gradients of that O. bf16 only, dense [B, H, S, d]
 * layout as attn_fwd/attn_bwd; the forward needs no workspace, the backward
 * the one attn_bwd_workspace_bytes gives. `offset` selects an independent
 * stream for the same seed (e.g. one per layer or step). */
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int d, int causal, float scale, float dropout_p, unsigned long long seed,
                     unsigned int offset, void* stream);
int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, int causal, float scale, float dropout_p, unsigned long long seed, unsigned int offset,
                     void* workspace, size_t workspace_bytes, void* stream);
/* The keep mask itself, as bytes keep[B, Hq, Sq, Sk] (1 = kept) on the device,
 * from the same generator (for checking and debugging; causal masks are not
 * applied). B, Hq, Sq >= 1, Sk >= 0. */
int attn_dropout_mask(unsigned char* keep, int B, int Hq, int Sq, int Sk, float dropout_p,
                      unsigned long long seed, unsigned int offset, void* stream);

/* ---- FP8 forward ("Flash Attention FA1->FA4 / pre-training practice", section
 * 2.2: FA3 runs attention in FP8 at twice the bf16 matrix rate and keeps it
 * accurate with per-block quantisation). Format: MXFP8 (OCP Microscaling
 * v1.0): OCP E4M3 element codes (bias 7, max 448, S.1111.111 = NaN) in blocks
 * of 32 that share one E8M0 scale byte s (scale 2^(s - 127)). Q and K are
 * blocked along the head dimension, V along the keys. d = 128 only
 * (ATTN_ERR_HEADDIM otherwise). All buffers are device memory the caller
 * owns; nothing is allocated or kept. */

/* Key count of the transposed FP8 V: Sk rounded up to a multiple of 64, or
 * ATTN_ERR_SHAPE for Sk outside [0, 2^24). */
int attn_fp8_padded_keys(int Sk);

/* Quantise rows of bf16 (Q or K, [rows, d] contiguous, e.g. [B, H, S, d]) to
 * codes [rows, d] (uint8) and scales [rows, d/32] (uint8). Per block of 32:
 * e = the smallest integer with amax <= 448 * 2^e (0 for an all-zero block,
 * clamped to [-127, 127]), scale byte e + 127, codes E4M3(x * 2^-e) rounded
 * to nearest even (never saturating). rows >= 0; x 16-byte aligned. */
int attn_mxfp8_quantize_rows(const void* x, void* codes, void* scales, long long rows, int d, void* stream);

/* Quantise V (bf16 [BH, Sk, d]) along the keys into its transposed form,
 * tiled by 64 keys: codes [BH, Skp/64, d, 64] (Skp = attn_fp8_padded_keys(Sk);
 * element (t, c, j) is key 64t + j of channel c; padding keys hold 0) and
 * scales [BH, Skp/64, d, 2]: byte kb of channel c in tile t covers keys
 * 64t + 32kb .. +31. Same block rule as above, keys past Sk counting as
 * zeros. Each tile's codes (8 KB at d = 128) and scales are contiguous. */
int attn_mxfp8_quantize_vt(const void* v, void* vt_codes, void* vt_scales, int BH, int Sk, int d, void* stream);

/* Bytes of device workspace attn_fwd_fp8 needs (0 if none): decode-shaped
 * problems (Hq/Hkv * Sq <= 32) split the keys over several wavefronts and
 * keep per-split partial results there, as attn_fwd does. 0 for invalid
 * arguments too; the call then reports the error. */
size_t attn_fwd_fp8_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal);

/* Forward on MXFP8 inputs: O (bf16 [B, Hq, Sq, d]) and lse (float [B, Hq, Sq],
 * natural log, may be NULL) of exact attention of the dequantised inputs,
 * with the same masks, GQA grouping, scale and empty-row rule as attn_fwd.
 * q8/q_scales as attn_mxfp8_quantize_rows gives them for [B, Hq, Sq, d],
 * k8/k_scales for [B, Hkv, Sk, d], vt8/vt_scales as attn_mxfp8_quantize_vt
 * gives them for [B*Hkv, Sk, d]. The probabilities are rounded to E4M3
 * before the P V product (the score product and the softmax run in fp32).
 * Dispatch as attn_fwd: tiled prefill, or split-key decode when
 * Hq/Hkv * Sq <= 32 (then workspace must hold attn_fwd_fp8_workspace_bytes,
 * else ATTN_ERR_WORKSPACE). Errors as attn_fwd; k8, k_scales, vt8, vt_scales
 * may be NULL only when Sk == 0. */
int attn_fwd_fp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales, const void* vt8,
                 const void* vt_scales, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                 int causal, float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code (never NULL). */
const char* attn_strerror(int status);

/* Dispatch record. "AI 大模型之 FlashAttention_01", section "性能验证方法",
 * asks that a benchmark confirm which kernel actually ran and keep a log of
 * the dispatch decision; this is that record.
 * Copies into buf (host memory, n bytes, NUL-terminated) a description of
 * the kernels the calling thread's last successful call launched: kernel
 * names, grid and tile shapes. Returns the full length of
 * the description (like snprintf), or a negative status if buf is NULL with
 * n > 0. When the environment variable ATTN_LOG is set to 1 the same line is
 * also printed to stderr on every call. */
int attn_last_dispatch(char* buf, size_t n);

/* Diagnostics: per-kernel device timing of the calling thread's calls.
 * attn_timing_start() clears the record and, until attn_timing_stop(), makes
 * every kernel launch of attn_fwd/attn_bwd on this thread be bracketed by two
 * HIP events recorded on the launch's own stream (the events are created
 * lazily and reused; timing adds two event records per kernel and changes
 * nothing else). attn_timing_stop() ends the record, waits for the recorded
 * events, and writes one line per kernel name into buf (host memory, n bytes,
 * NUL-terminated): "<kernel> <launches> <total milliseconds>". It returns the
 * full length of the text, ATTN_ERR_NULL if buf is NULL with n > 0, or
 * ATTN_ERR_HIP if an event could not be created, recorded or read. The record
 * lives only in host memory; no kernel argument or output depends on it. */
int attn_timing_start(void);
int attn_timing_stop(char* buf, size_t n);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_MI355X_H */
