/*
 * fa.h -- C ABI of libfa: exact tiled attention (FlashAttention forward) and
 * split-KV decode for AMD Instinct MI355X (gfx950).
 *
 * Every pointer argument that names a tensor is a DEVICE pointer owned by the
 * caller; the library keeps no reference to it after the call returns and
 * never frees it.  All calls are asynchronous: they validate their arguments
 * on the host, enqueue kernels on `stream` (0 = the null stream) and return.
 * No call allocates device memory and no call synchronises the device.
 *
 * Errors are returned as a status code, never thrown.  On a non-OK status no
 * kernel has been enqueued (except FA_ERR_HIP, where a launch itself failed),
 * and fa_last_error() returns a description (thread-local).
 *
 * Tensor layouts (all contiguous, row-major, element strides implied):
 *   q  [B, Lq, Hq, D]      k, v [B, Lk, Hkv, D]     o [B, Lq, Hq, D]
 *   lse [B, Hq, Lq] float32, natural-log logsumexp of the scaled scores.
 * This is the [batch, seq, heads, head_dim] layout of the usage example in
 * "FlashAttention in the CANN ops-transformer library" (ai6s.net), section 4.
 */
#ifndef FA_GFX950_FA_H
#define FA_GFX950_FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, bad split count, small workspace */
  FA_ERR_UNSUPPORTED = 2,      /* head_dim not in {64,128,256} or unknown dtype */
  FA_ERR_HIP = 3               /* a kernel launch failed (text from hipGetErrorString) */
} fa_status;

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

/* Storage of one side (keys or values) of a paged KV cache. */
typedef enum {
  FA_KV_NATIVE = 0, /* elements of the call's dtype (fp16 / bf16) */
  FA_KV_INT8 = 1    /* int8 codes; the cached value is code * the row's float scale */
} fa_kv_format;

/*
 * fa_fwd -- O = softmax(scale * Q K^T + mask) V, computed tile by tile with an
 * online softmax; the score matrix is never stored.
 *
 * Defined by "FlashAttention in the CANN ops-transformer library" (ai6s.net),
 * section 2 (tiling, per-block running max/sum, blockwise O and L write-back)
 * and section 4 (arguments q, k, v, softmax_scale, is_causal); GQA head
 * sharing as in "Enable Flash Attention with llama.cpp" (qualllm.com), FAQ.
 *
 *   q, k, v, o  device pointers, elements of type `dtype`, layouts above;
 *               each must be 16-byte aligned.
 *   lse         device float32 [B, Hq, Lq]; receives, per query row, the
 *               logsumexp (natural log) of the scaled scores over the keys
 *               the row may see.  16-byte aligned.
 *   B, Lq, Lk   >= 1.   Hq, Hkv >= 1 with Hq % Hkv == 0; query head h reads
 *               key/value head h / (Hq / Hkv).  B*Lq*Hq and B*Lk*Hkv must be
 *               below 2^31 and Hkv*D below 2^25 (FA_ERR_INVALID_ARGUMENT).
 *   D           head dimension: 64, 128 or 256 (others -> FA_ERR_UNSUPPORTED;
 *               the head-dim set of the same page, section 5).
 *   scale       any finite float; scores are scale * q.k.
 *   causal      0: every query row sees every key (bidirectional, encoder
 *               use); nonzero: row i sees keys j <= i + (Lk - Lq)
 *               (bottom-right aligned; the usual lower triangle if Lq == Lk).
 *               Rows that see no key get o = 0 and lse = -inf.
 *   dtype       FA_F16 or FA_BF16 for q, k, v and o.  Accumulation is fp32.
 *   stream      HIP stream to enqueue on.
 * Returns FA_OK once enqueued.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                 fa_dtype dtype, hipStream_t stream);

/*
 * fa_fwd_ex -- fa_fwd plus structured masks: a sliding window and
 * block-diagonal packing of several sequences.  The masks are the "local" and
 * "block-diagonal" structured masks that "5 years, 10K stars: xformers"
 * (cloud.tencent.com) lists as the way to avoid reading a dense mask; as in
 * fa_fwd, no mask tensor is read.
 *
 *   window_left, window_right
 *               row i sees keys j with i + (Lk-Lq) - window_left <= j <=
 *               i + (Lk-Lq) + window_right; a negative value leaves that side
 *               unbounded.  causal additionally caps j <= i + (Lk-Lq).
 *               (-1, -1) is no window; (w, 0) with causal=0 equals causal
 *               attention limited to the last w+1 keys.  A side at least as
 *               wide as the query plus key rows is the same as unbounded;
 *               with a window, query plus key rows must be <= 2^30.
 *   cu_seqlens_q, cu_seqlens_k
 *               NULL: dense batch, exactly as fa_fwd (q [B,Lq,Hq,D], k/v
 *               [B,Lk,Hkv,D], lse [B,Hq,Lq]); total_q/total_k are ignored.
 *               Otherwise device int32 arrays of B+1 non-decreasing offsets
 *               starting at 0: sequence b is rows cu_seqlens_q[b] ..
 *               cu_seqlens_q[b+1]-1 of q/o [total_q, Hq, D] and rows
 *               cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k/v [total_k, Hkv,
 *               D]; each sequence attends only to its own keys (the causal and
 *               window rules apply inside it, with its own lengths); lse is
 *               [Hq, total_q] float32.  Lq and Lk must then be at least the
 *               longest query / key sequence (rows past Lq of a longer
 *               sequence are not computed).  Offsets are clamped into
 *               [0, total] on the device, so inconsistent offsets give wrong
 *               results but no out-of-bounds access.
 *   other arguments as in fa_fwd, which is fa_fwd_ex with NULL offsets and
 *   no window.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                    int Lq, int Lk, int total_q, int total_k, int D, float scale, int causal,
                    int window_left, int window_right, fa_dtype dtype, hipStream_t stream);

/*
 * fa_fwd_fp8 -- the forward of fa_fwd_ex (dense batch, causal / window masks)
 * on FP8 inputs: Q, K and V stored as OCP e4m3 codes, each with one float
 * descale (the real value is code * descale), P rounded to e4m3 for the PV
 * product, fp32 accumulation, O in bf16 or fp16.
 *
 * The FP8 variant is the FlashAttention-3 item of "FlashAttention-2 (TH)"
 * (systems-analysis.info); the page fixes neither the format nor the
 * scaling, read here as above.  Because P is rounded to e4m3 (relative error
 * <= 2^-4), O is exact only to about 2^-4 * sum_j P_ij |v_j|; lse is computed
 * from unrounded probabilities.
 *
 *   q8          device e4m3 [B, Lq, Hq, D], 16-byte aligned.
 *   k8          device e4m3 [B, Lk, Hkv, D], 16-byte aligned.
 *   vt8         device e4m3 [B, Hkv, D, vt_stride]: V transposed, key j of
 *               dimension d at column j.  vt_stride is a multiple of 64,
 *               >= Lk; columns Lk .. vt_stride-1 are read and must hold finite
 *               codes (zeros), their probabilities being 0.
 *   o, lse      as fa_fwd; o in out_dtype.
 *   D           64, 128 or 256 (at 256 two workgroups share each query tile,
 *               each forming the scores and probabilities and the P V
 *               product for 128 of the output dimensions).
 *   scale       softmax scale applied to the real (descaled) scores.
 *   q_descale, k_descale, v_descale   finite, > 0.
 *   other arguments as in fa_fwd_ex.  D * vt_stride must be below 2^32.
 */
fa_status fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, void* o, float* lse, int B,
                     int Hq, int Hkv, int Lq, int Lk, int D, int vt_stride, float scale,
                     float q_descale, float k_descale, float v_descale, int causal,
                     int window_left, int window_right, fa_dtype out_dtype, hipStream_t stream);

/*
 * fa_fwd_fp8_ex -- fa_fwd_fp8 also for sequences packed back to back, the
 * block-diagonal structured mask of "5 years, 10K stars: xformers"
 * (cloud.tencent.com), as fa_fwd_ex has it for 16-bit inputs.
 *
 *   cu_seqlens_q, cu_seqlens_k   NULL (dense: exactly fa_fwd_fp8) or device
 *               int32 [B + 1] offsets, as in fa_fwd_ex: sequence b is query
 *               rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 *               cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 and attends only to
 *               itself.  Offsets are clamped into [0, total] on the device.
 *   packed:  q8 [total_q, Hq, D], k8 [total_k, Hkv, D], o [total_q, Hq, D],
 *            lse float32 [Hq, total_q];
 *            vt8 [Hkv, D, vt_stride]: V transposed, key row r of k8 at column r;
 *            vt_stride a multiple of 64 and >= total_k + 64.  Columns
 *            total_k .. vt_stride-1 are read (each sequence's key tiles start
 *            at its first key rounded down to 16) and must hold finite codes.
 *   Lq, Lk      dense: the lengths; packed: the longest query / key sequence
 *               (the grid is sized by Lq).
 *   total_q, total_k   packed: the row counts of q8 / k8 (ignored when dense).
 *   other arguments as in fa_fwd_fp8.
 */
fa_status fa_fwd_fp8_ex(const void* q8, const void* k8, const void* vt8, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                        int Lq, int Lk, int total_q, int total_k, int D, int vt_stride,
                        float scale, float q_descale, float k_descale, float v_descale,
                        int causal, int window_left, int window_right, fa_dtype out_dtype,
                        hipStream_t stream);

/*
 * fa_decode_workspace_size -- bytes of device workspace fa_decode needs for
 * these sizes: float32 partial outputs [B, Hq, num_splits, D] followed by
 * float32 partial logsumexps [B, Hq, num_splits].  Returns 0 for invalid sizes.
 */
size_t fa_decode_workspace_size(int B, int Hq, int D, int num_splits);

/*
 * fa_decode -- one query token per sequence attending to its KV cache, split
 * over key chunks and merged by logsumexp.
 *
 * The per-token decode step whose latency the ai6s.net page reports in
 * section 3; the split-KV form is the split-K decoding backend named by
 * "5 years, 10K stars: xformers" (cloud.tencent.com).  Chunk c of sequence b
 * covers keys [c*C_b, min(len_b, (c+1)*C_b)) with C_b = ceil(len_b /
 * num_splits); each chunk yields a normalised partial output and its
 * logsumexp, and a second kernel merges them with weights
 * exp(lse_c - lse_total).
 *
 *   q          device [B, Hq, D] (dtype)              16-byte aligned
 *   k_cache,   device [B, Lk_max, Hkv, D] (dtype); rows j >= seqlens[b] of
 *   v_cache    sequence b are never read (they may hold anything).
 *   seqlens    device int32 [B]; sequence b attends to keys 0 .. seqlens[b]-1.
 *              Values are clamped to [0, Lk_max] on the device; a sequence of
 *              length 0 gets o = 0 and lse = -inf.
 *   o          device [B, Hq, D] (dtype);   lse  device float32 [B, Hq].
 *   num_splits 1 .. 64.
 *   workspace  device buffer of at least fa_decode_workspace_size(B,Hq,D,
 *              num_splits) bytes, 16-byte aligned, owned by the caller; its
 *              contents need not be initialised and are garbage afterwards.
 *   other arguments as in fa_fwd.
 * Returns FA_OK once both kernels are enqueued.
 */
fa_status fa_decode(const void* q, const void* k_cache, const void* v_cache, const int* seqlens,
                    void* o, float* lse, int B, int Hq, int Hkv, int Lk_max, int D, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    fa_dtype dtype, hipStream_t stream);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, kernels and results as fa_decode, minus
 * the workspace: the split partials live in a fixed 32 MiB array in device
 * memory that the library holds on each GPU it runs on until the process
 * ends.  Limit: B * Hq * num_splits * (D + 1) * 4 bytes must fit in 32 MiB
 * (65,027 (head, split) pairs at D = 128); larger calls return
 * FA_ERR_INVALID_ARGUMENT before any device call.  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress); no
 * call allocates or frees memory.  Every call on one GPU uses the same array:
 * calls that overlap on one GPU (different streams or host threads without
 * ordering between them) race and give wrong results; calls ordered on one
 * stream are safe.
 */
fa_status fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                            int Lk_max, int D, float scale, int num_splits, fa_dtype dtype,
                            hipStream_t stream);

/*
 * fa_decode_paged -- fa_decode over a paged KV cache whose keys, or keys and
 * values, may be stored as int8.
 *
 * The cache layout is the PagedAttention one cited in the references of
 * "FlashAttention-2 (TH)" (systems-analysis.info); the int8 modes are the
 * KV-INT8 modes of "MNN LLM attention_mode" (lpnh.cn), encoding section
 * (keys int8 with native values, or both int8).  The pages fix neither the
 * page layout nor the quantiser; the readings used:
 *
 *   k_pages,    device [num_pages, page_size, Hkv, D], elements of `dtype`
 *   v_pages     (FA_KV_NATIVE) or int8 (FA_KV_INT8); 16-byte aligned.  Key j
 *               of sequence b is slot j % page_size of page
 *               block_table[b * max_pages + j / page_size].
 *   k_scales,   device float32 [num_pages, Hkv, page_size], 16-byte aligned:
 *   v_scales    the scale of each cached row of an int8 side (its value is
 *               code * scale); ignored, and may be NULL, for a native side.
 *               Slots past a sequence's end may hold anything (NaN too).
 *   block_table device int32 [B, max_pages]; entries are clamped to
 *               [0, num_pages-1] on the device (bad entries read wrong rows,
 *               never out of bounds).  Entries past a sequence's length are
 *               not read.
 *   seqlens     device int32 [B], clamped to [0, max_pages * page_size].
 *   page_size   a power of two in [16, 65536].
 *   k_format,   FA_KV_NATIVE / FA_KV_NATIVE, FA_KV_INT8 / FA_KV_NATIVE or
 *   v_format    FA_KV_INT8 / FA_KV_INT8 (int8 values with native keys:
 *               FA_ERR_UNSUPPORTED).
 *   workspace   as fa_decode: fa_decode_workspace_size(B, Hq, D, num_splits)
 *               bytes.  Chunks are rounded up to whole 16-key steps here, so
 *               chunk c covers keys [c*C_b, min(len_b, (c+1)*C_b)) with
 *               C_b = 16 * ceil(len_b / (16 * num_splits)).
 *   other arguments as in fa_decode.
 * Returns FA_OK once both kernels are enqueued.
 */
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                          const float* k_scales, const float* v_scales, const int* block_table,
                          const int* seqlens, void* o, float* lse, int B, int Hq, int Hkv, int D,
                          int num_pages, int page_size, int max_pages, float scale,
                          int num_splits, fa_kv_format k_format, fa_kv_format v_format,
                          void* workspace, size_t workspace_bytes, fa_dtype dtype,
                          hipStream_t stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs: two float32
 * arrays [B, Hq, Lq rounded up to a multiple of 32] (per-row lse * log2(e)
 * and rowsum(dO * O)).  Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Lq);

/*
 * fa_bwd -- gradients dQ, dK, dV of fa_fwd / fa_fwd_ex (dense batch) given
 * the gradient dO of its output, from the forward's q, k, v, o and lse.
 *
 * The gradient of the forward's definition: with P_ij = exp(scale q_i.k_j -
 * lse_i) on the keys row i may see, dV_j = sum_i P_ij dO_i, dS_ij = P_ij
 * (dO_i.v_j - dO_i.o_i), dQ_i = scale sum_j dS_ij k_j, dK_j = scale sum_i
 * dS_ij q_i; grouped K/V heads sum their query heads' dK, dV.  The pages only
 * report training with the method ("FlashAttention-2 (TH)",
 * systems-analysis.info, performance) and pair every forward operator with a
 * backward ("5 years, 10K stars: xformers", cloud.tencent.com); the formulas
 * are calculus on the forward.  No atomics: results are bitwise reproducible.
 *
 *   q, o, dout  device [B, Lq, Hq, D] (dtype), 16-byte aligned.
 *   k, v        device [B, Lk, Hkv, D] (dtype), 16-byte aligned.
 *   lse         device float32 [B, Hq, Lq], as written by the forward.
 *   dq          device [B, Lq, Hq, D] (dtype), written.
 *   dk, dv      device [B, Lk, Hkv, D] (dtype), written (summed over each
 *               K/V head's query heads).
 *   D           64, 128 or 256 (others: FA_ERR_UNSUPPORTED).
 *   causal, window_left, window_right, scale: as in fa_fwd_ex; must be the
 *               forward's.
 *   workspace   fa_bwd_workspace_size(B, Hq, Lq) bytes, 16-byte aligned,
 *               caller-owned, contents need not be initialised.
 *   B*Lq*Hq and B*Lk*Hkv below 2^31, Hq*D and Hkv*D below 2^25.
 * Returns FA_OK once the three kernels are enqueued.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Lq,
                 int Lk, int D, float scale, int causal, int window_left, int window_right,
                 void* workspace, size_t workspace_bytes, fa_dtype dtype, hipStream_t stream);

/*
 * fa_bwd_ex -- fa_bwd for the structured masks of fa_fwd_ex: also for several
 * sequences packed back to back (block-diagonal), the backward of fa_fwd_ex
 * with the same offsets.
 *
 *   cu_seqlens_q, cu_seqlens_k, total_q, total_k
 *               as in fa_fwd_ex: NULL for a dense batch (then exactly
 *               fa_bwd); otherwise q, o, dout, dq are [total_q, Hq, D], k, v,
 *               dk, dv are [total_k, Hkv, D], lse is [Hq, total_q], and Lq /
 *               Lk must be at least the longest query / key sequence.  Each
 *               sequence's dk, dv rows are written (zero for keys no query of
 *               the sequence sees).  Offsets are clamped on the device and
 *               lengths past Lq / Lk are cut to them: inconsistent offsets
 *               give wrong results but no out-of-bounds access.
 *   workspace   fa_bwd_workspace_size(B, Hq, Lq) bytes, Lq the longest.
 *   other arguments as in fa_bwd, which is fa_bwd_ex with NULL offsets.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int B, int Hq, int Hkv, int Lq, int Lk, int total_q,
                    int total_k, int D, float scale, int causal, int window_left,
                    int window_right, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                    hipStream_t stream);

/* Text for the last non-OK status returned on this thread ("" if none). */
const char* fa_last_error(void);

/* Static description of the build: target arch, head dims, dtypes, tiles,
 * version.  Touches no device. */
const char* fa_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_GFX950_FA_H */
