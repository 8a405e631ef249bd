/*
 * fa.h - exact attention forward (FlashAttention-2 style) and split-KV decode
 * for AMD Instinct MI355X (gfx950). C ABI: plain pointers and sizes only.
 *
 * What is computed (the plain definition, "Flash Attention: Revolutionizing
 * Transformer Efficiency", unite.ai, standard-attention listing):
 *
 *     O = softmax(scale * Q K^T [+ causal mask]) V,   LSE = log sum exp(...)
 *
 * per (batch, q-head, query row), without ever forming the score matrix: K/V
 * tiles stream through on-chip memory and the row maximum and row sum are
 * carried block to block with the softmax-merge identity of the same page
 * (section "The math of Flash Attention"). The result equals the plain
 * definition up to floating-point rounding (same page, "Impact", point 3).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, contiguous, row-major, on the device that is
 *     current for the calling thread, 16-byte aligned.
 *   - Element type of q, k, v, o, caches: bf16 or fp16 (argument `dtype`);
 *     arithmetic: fp32 accumulation on matrix cores; O is rounded to
 *     nearest-even into `dtype`; LSE is fp32 (natural log).
 *   - Grouped-query attention (SDPA page, devhandbook.co.kr, Example 5): q-head
 *     h reads kv-head h / (Hq / Hkv); Hq must be a multiple of Hkv. Hkv = 1 is
 *     multi-query attention.
 *   - `stream` is a hipStream_t passed as void* (NULL = legacy default stream).
 *     Work is only enqueued; the call never synchronises, allocates or frees.
 *     Results are valid once the stream has completed.
 *   - Inputs are read-only. Outputs and workspaces must not overlap an input
 *     (index arrays such as seqlens and cu_seqlens included) or each other;
 *     every call checks this on the byte ranges its arguments span and
 *     returns FA_ERR_INVALID_ARG when they do.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     decode workspace. The library keeps only per-device properties.
 *   - Errors: every argument is validated before anything is enqueued; on
 *     failure nothing is written and the call returns a status. The text of
 *     the most recent failure on the calling thread is fa_last_error().
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, bad scale, ... */
  FA_ERR_UNSUPPORTED = 2,  /* head dim, dtype or device not supported */
  FA_ERR_HIP = 3           /* the HIP runtime reported an error */
} fa_status;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP16 = 1 } fa_dtype;

/*
 * fa_fwd - prefill attention forward.
 *
 * Source of the operation: "Flash Attention: Revolutionizing Transformer
 * Efficiency" (unite.ai): standard-attention listing (definition), sections
 * "Flash Attention algorithm" and "Implementation details" (tiled loop over
 * query blocks and key/value blocks with running max and sum). Causal masking
 * as `is_causal` in the SDPA page (devhandbook.co.kr), Example 3.
 *
 *   q   [B, Hq,  Nq, d]  input, dtype
 *   k   [B, Hkv, Nk, d]  input, dtype
 *   v   [B, Hkv, Nk, d]  input, dtype
 *   o   [B, Hq,  Nq, d]  output, dtype
 *   lse [B, Hq,  Nq]     output, fp32, natural-log sum of exp of the visible
 *                        scaled scores; may be NULL (then not written)
 *   d      head width: 64 or 128 (else FA_ERR_UNSUPPORTED)
 *   scale  multiplies Q K^T; finite and > 0 (typically 1/sqrt(d))
 *   causal 0 or 1. With causal, key j is visible to query i iff
 *          j <= i + (Nk - Nq) (bottom-right alignment); requires Nq <= Nk.
 *   dtype  FA_DTYPE_BF16 or FA_DTYPE_FP16
 *
 * Sizes must be positive; B*Hq*Nq*d and B*Hkv*Nk*d must fit in int64.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 int dtype, void* stream);

/*
 * fa_fwd_varlen - fa_fwd over a packed batch of sequences of different
 * lengths, with no padding.
 *
 * Source: "Advanced techniques for enhancing LLM throughput" (cabseo.com),
 * section "Continuous batching": requests of different lengths are batched
 * together, and padding the short ones to the longest wastes work. Each
 * sequence is attended to exactly as by fa_fwd (same arithmetic, same causal
 * alignment per sequence); sequences never see each other's keys.
 *
 *   q      [Hq, total_q, d]   input, dtype: sequence b's query rows are rows
 *          cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of each head's slab
 *   k, v   [Hkv, total_k, d]  input, dtype: its keys are rows
 *          cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1
 *   o      [Hq, total_q, d]   output, dtype (rows of no sequence untouched)
 *   lse    [Hq, total_q] fp32 output, may be NULL
 *   cu_seqlens_q, cu_seqlens_k  [B+1] int32, device memory, non-decreasing
 *          from 0. Offsets are clamped into [0, total] (and an end below its
 *          start to the start), so no offset array can send the kernels
 *          outside the tensors.
 *   max_seqlen_q  upper bound on every sequence's query length: query rows
 *          past it are not computed.
 *   causal 0/1, per sequence bottom-right aligned (key j visible to query i
 *          iff j <= i + Nk_b - Nq_b). A row that sees no key (a sequence with
 *          Nk_b = 0, or causal with Nq_b > Nk_b) gets O = 0 and LSE = -inf.
 *   B, Hq, Hkv, d, scale, dtype, stream: as in fa_fwd.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                        int d, float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_strided - fa_fwd with q, k, v and o at any element strides, e.g. the
 * (batch, seq, heads, dim) layout.
 *
 * Source: "FlashAttention complete guide for beginners" (cloud-allstudy
 * tistory), section 5 "Usage (code examples)": flash_attn_func takes q, k, v
 * laid out (batch, seq, heads, dim); the SDPA page (devhandbook.co.kr),
 * Example 1, lays the same tensors out (B, H, L, D). The operation is the
 * one of fa_fwd; only the addressing differs, and the result is bitwise that
 * of fa_fwd on the same values.
 *
 *   strides  host array of 12 int64: the element strides of (batch, head,
 *            row) for q, then k, v and o. Element (b, h, i, c) of q is at
 *            q + b*strides[0] + h*strides[1] + i*strides[2] + c. Every stride
 *            is a non-negative multiple of 8 (16-byte rows); row strides are
 *            below 2^24 and the others below 2^40. The strides of o must not
 *            make two of its elements share memory; o must not overlap q, k
 *            or v (checked on the spans the strides reach).
 *            The (batch, seq, heads, dim) layout is {Nq*Hq*d, d, Hq*d} for q
 *            and o and {Nk*Hkv*d, d, Hkv*d} for k and v.
 *   lse      [B, Hq, Nq] fp32, contiguous, or NULL.
 *   all other arguments as in fa_fwd.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int64_t* strides, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_varlen_strided - fa_fwd_varlen with q, k, v and o at any element
 * strides, e.g. the packed (total, heads, dim) layout.
 *
 * Source: as fa_fwd_varlen ("Continuous batching", cabseo.com) with the
 * addressing of fa_fwd_strided.
 *
 *   strides  host array of 8 int64: the element strides of (head, token) for
 *            q, then k, v and o; token t of head h of q is at
 *            q + h*strides[0] + t*strides[1]. The (total, heads, dim) layout
 *            is {d, Hq*d} for q and o and {d, Hkv*d} for k and v. Same rules
 *            as in fa_fwd_strided.
 *   lse      [Hq, total_q] fp32, contiguous, or NULL.
 *   all other arguments as in fa_fwd_varlen.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int64_t* strides, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q,
                                int total_k, int max_seqlen_q, int d, float scale, int causal,
                                int dtype, void* stream);

/*
 * fa_fwd_fp8 - prefill attention forward with 8-bit float inputs.
 *
 * Source: "Flash Attention: Revolutionizing Transformer Efficiency"
 * (unite.ai), section "FlashAttention-3", point 2: computing in low-precision
 * FP8 for speed (point 3 names a technique against quantization error without
 * describing it; none is applied here). The operation is fa_fwd's on the
 * values the 8-bit inputs stand for: element x of the (b, head) slab of q
 * stands for x * q_descale[b, head], likewise k and v with their kv-head.
 * The probabilities are rounded to FP8 for the second product (after scaling
 * by 2^4, which keeps small values in E4M3's normal range while the running
 * reference keeps every scaled value at most 448), which bounds the accuracy:
 * about 4% relative error on O for nearly flat attention rows; the LSE is
 * computed in fp32.
 *
 *   q          [B, Hq, Nq, 128]  input, OCP FP8 E4M3 bytes (no infinities;
 *              0x7F/0xFF are NaN; largest finite 448)
 *   k, v       [B, Hkv, Nk, 128] input, E4M3 bytes
 *   o          [B, Hq, Nq, 128]  output, bf16
 *   lse        [B, Hq, Nq] fp32 output or NULL
 *   q_descale  [B, Hq] fp32, device memory; k_descale, v_descale [B, Hkv]
 *   d          must be 128 (else FA_ERR_UNSUPPORTED)
 *   scale, causal: as in fa_fwd (scale multiplies the dequantized Q K^T)
 *
 * Contiguous row-major tensors; o and lse must not overlap the inputs.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     const float* q_descale, const float* k_descale, const float* v_descale,
                     int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     void* stream);

/*
 * fa_bwd_workspace_bytes - bytes of device workspace fa_bwd needs (one fp32
 * per query row, rounded up to 256). Returns 0 if the sizes are invalid.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq);

/*
 * fa_bwd - gradients dQ, dK, dV of the prefill forward for an upstream
 * gradient dO of its output.
 *
 * Source: "Flash Attention: Revolutionizing Transformer Efficiency"
 * (unite.ai): the forward is the standard-attention definition of that page
 * (as fa_fwd); its "Enter Flash Attention" list (point 2) has the backward
 * pass recompute the parts of the attention matrix it needs rather than store
 * it, and its FlashAttention-2 section (point 2) names the backward pass as
 * the part brought close to forward speed. The gradients are those of the
 * forward definition (the chain rule; the pages give no formulas):
 *     P = exp(scale Q K^T - LSE) (0 where masked),  dV = P^T dO,
 *     dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale dS K,  dK = scale dS^T Q.
 * A kv-head's dK and dV sum the contributions of every q-head that reads it.
 *
 *   q, o, dout  [B, Hq, Nq, d]  inputs, dtype; o is fa_fwd's output for q, k, v
 *   k, v        [B, Hkv, Nk, d] inputs, dtype
 *   lse         [B, Hq, Nq] fp32 input, fa_fwd's LSE for the same call
 *   dq          [B, Hq, Nq, d]  output, dtype
 *   dk, dv      [B, Hkv, Nk, d] output, dtype
 *   workspace, workspace_bytes: device scratch of at least
 *               fa_bwd_workspace_bytes(B, Hq, Nq) bytes, 256-byte aligned,
 *               owned by the caller; contents on entry are ignored.
 *   d, scale, causal, dtype: as in fa_fwd (the same values as the forward).
 *
 * All tensors contiguous row-major. Outputs and the workspace must not
 * overlap each other or any input. The result is deterministic (no atomics).
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, void* workspace,
                 size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                 int causal, int dtype, void* stream);

/*
 * fa_decode_workspace_bytes - bytes of device workspace fa_decode needs for
 * these sizes and this `num_splits` (0 = the library's choice). Returns 0 if
 * the sizes are invalid. The workspace holds the partial outputs and their
 * LSE (the merge identity in LSE form), at most splits + 1 of them per
 * (sequence, q-head) with splits = num_splits or the library's choice, and a
 * small header that the split pass leaves for the merge pass.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Lcap, int d, int num_splits);

/*
 * fa_decode - one new query token per sequence against its KV cache, split
 * along the keys, then merged.
 *
 * Source: "Advanced techniques for enhancing LLM throughput" (cabseo.com),
 * sections "Memory requirements" (each new token attends to the cached K/V of
 * every earlier token) and "Autoregressive and memory-bound operations"
 * (decode is a matrix-vector product bound by memory traffic). The split
 * results are merged with the softmax-merge identity of the unite.ai page
 * ("The math of Flash Attention"), in LSE form:
 *     LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
 *
 *   q        [B, Hq, d]          input, dtype
 *   k_cache  [B, Hkv, Lcap, d]   input, dtype; rows >= seqlens[b] are never read
 *   v_cache  [B, Hkv, Lcap, d]   input, dtype; rows >= seqlens[b] are never read
 *   seqlens  [B] int32, device memory; values are clamped to [0, Lcap]. A
 *            sequence of length 0 yields O = 0 and LSE = -inf.
 *   o        [B, Hq, d]          output, dtype
 *   lse      [B, Hq] fp32 output, may be NULL
 *   workspace, workspace_bytes: device scratch of at least
 *            fa_decode_workspace_bytes(...) bytes, 256-byte aligned, owned by
 *            the caller; contents on entry are ignored.
 *   d        64 or 128; Hq / Hkv must be <= 32
 *   scale    finite and > 0
 *   num_splits  sets the smallest share of cached rows one wave takes,
 *            ceil(Lcap / num_splits) rounded up to a multiple of 128 (shares
 *            are otherwise equal across the waves the GPU holds at once);
 *            0 = chosen by the library. The result does not depend on it
 *            beyond rounding.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG (including a too-small workspace),
 * FA_ERR_UNSUPPORTED (d, dtype or Hq / Hkv outside the ranges above, B or
 * Hkv above 65535, or B * Hkv * ceil(Lcap / 32) above 2^31 - 1)
 * or FA_ERR_HIP.
 */
fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                    void* o, float* lse, void* workspace, size_t workspace_bytes,
                    int B, int Hq, int Hkv, int Lcap, int d, float scale, int num_splits,
                    int dtype, void* stream);

/*
 * fa_decode_noalloc - fa_decode without a caller-supplied workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, layouts, results and errors are those of fa_decode without
 * `workspace` and `workspace_bytes`. The workspace is a static device array
 * of FA_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU,
 * held until the process ends; its address is looked up on the first call
 * on each device (with that device current). The call allocates nothing
 * and frees nothing. Sizes whose fa_decode_workspace_bytes(...) exceeds the
 * array are refused with FA_ERR_INVALID_ARG before anything is launched.
 *
 * Every call on one GPU uses the same array and the last call's contents
 * stay in it (nothing in it needs to start at zero): calls that overlap on
 * one GPU (different streams, or threads, without ordering between them)
 * race. Order them on one stream, or use fa_decode with separate workspaces.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* seqlens,
                            void* o, float* lse, int B, int Hq, int Hkv, int Lcap, int d, float scale,
                            int num_splits, int dtype, void* stream);

/*
 * fa_decode_paged - fa_decode with the KV cache held in fixed-size pages
 * reached through a per-sequence page table.
 *
 * Source: "Advanced techniques for enhancing LLM throughput" (cabseo.com),
 * section "Paged attention": the cache of each sequence is split into pages,
 * in the manner of operating-system paging, so that caches of different and
 * growing lengths do not fragment memory, and attention walks a sequence's
 * cache page by page. The arithmetic, the split along the keys and the merge
 * are those of fa_decode.
 *
 *   q        [B, Hq, d]                          input, dtype
 *   k_pages  [num_pages, Hkv, page_size, d]      input, dtype: page p holds,
 *            per kv-head, page_size consecutive cache rows of one sequence
 *   v_pages  [num_pages, Hkv, page_size, d]      input, dtype (same layout)
 *   block_table [B, max_pages] int32, device memory: logical cache row j of
 *            sequence b is row j % page_size of page
 *            block_table[b * max_pages + j / page_size]. Only the entries that
 *            cover rows [0, seqlens[b]) are followed. An entry outside
 *            [0, num_pages) is not followed (no memory outside k_pages /
 *            v_pages is read); O and LSE of that sequence come out NaN.
 *   seqlens  [B] int32, device memory; clamped to [0, max_pages * page_size].
 *   o, lse   as in fa_decode
 *   workspace, workspace_bytes: at least
 *            fa_decode_workspace_bytes(B, Hq, Hkv, max_pages * page_size, d,
 *            num_splits) bytes, 256-byte aligned, owned by the caller.
 *   page_size   a multiple of 32
 *   d, scale, num_splits, dtype, stream: as in fa_decode.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED (page_size not a
 * multiple of 32, or as in fa_decode) or FA_ERR_HIP.
 */
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                          int num_pages, int page_size, int max_pages, int d, float scale,
                          int num_splits, int dtype, void* stream);

/*
 * fa_set_prefill_schedule - how the causal prefill entry points (fa_fwd,
 * fa_fwd_strided) spread query tiles over workgroups. Results are the same
 * up to the order of floating-point sums; only the work division changes.
 *
 *   FA_SCHEDULE_AUTO   (default) split when a causal grid of 256-row
 *                      workgroups fits on the device at once, else tiles
 *   FA_SCHEDULE_TILES  one 256-row query tile per workgroup, heaviest first
 *   FA_SCHEDULE_SPLIT  one workgroup per pair of 128-row blocks (nb-1-p, p)
 *                      of a head, the two halves of each key tile taken by
 *                      two wave groups and joined by the merge identity of
 *                      "The math of Flash Attention" (unite.ai)
 *
 * Process-wide, for all devices; takes effect at the next launch. Returns
 * the previous mode, or -1 (and changes nothing) for an unknown mode.
 */
#define FA_SCHEDULE_AUTO 0
#define FA_SCHEDULE_TILES 1
#define FA_SCHEDULE_SPLIT 2
int fa_set_prefill_schedule(int mode);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* fa_last_error(void);

/* Library ABI version (incremented on incompatible changes). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
