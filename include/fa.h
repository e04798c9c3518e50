/*
 * fa.h -- C ABI of libfa_amd.so for AMD Instinct MI355X (gfx950): exact
 * attention forward (FlashAttention tiling, online softmax, log-sum-exp) on
 * 16-bit and FP8 inputs and on packed variable-length batches; its backward
 * (dQ, dK, dV); and split-KV flash-decode over dense or paged caches.
 *
 * Plain pointers and sizes only.  Every tensor pointer is a DEVICE pointer
 * owned by the caller; the library keeps none of them after a call returns
 * and frees nothing it did not allocate.  All calls enqueue work on `stream`
 * (0 = the null stream) and return without synchronising; a fault inside a
 * kernel surfaces at the caller's next synchronisation.  Argument checks run
 * before any HIP call, so a rejected call has enqueued nothing.
 *
 * Layouts are contiguous with head_dim fastest, the (batch, heads, seq_len,
 * head_dim) convention of the benchmark listing on the dailyaiworld page
 * "FlashAttention-3 vs Triton Kernels: Warp-Specialization on GPUs",
 * section "Benchmarking Triton vs FlashAttention-3 Kernels".
 */
#ifndef FA_AMD_FA_H
#define FA_AMD_FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    FA_ERR_SHAPE = 2,       /* a size is negative, inconsistent or too large  */
    FA_ERR_UNSUPPORTED = 3, /* head_dim not in {64, 128}, or unknown dtype    */
    FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned        */
    FA_ERR_WORKSPACE = 5,   /* caller workspace missing or too small          */
    FA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed     */
    FA_ERR_INTERNAL = 7,    /* unexpected internal error                      */
    FA_ERR_VALUE = 8        /* a non-finite scale                             */
} fa_status_t;

/* Storage type of q, k, v and the caches.  Arithmetic is bf16/fp16 products
 * with fp32 accumulation; outputs are always fp32. */
typedef enum { FA_BF16 = 0, FA_FP16 = 1 } fa_dtype_t;

/* Size of fa_decode_noalloc's fixed per-device buffer, in bytes. */
#define FA_DECODE_NOALLOC_MAX_BYTES ((size_t)8 << 20)

/*
 * fa_fwd -- exact softmax attention, computed tile by tile without storing
 * the N x N score matrix (dailyaiworld page, introduction: FlashAttention's
 * IO-aware tiling).  For every b < B, h < H, i < N:
 *     s_ij  = scale * <q[b,h,i,:], k[b,h,j,:]>     over visible keys j
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,h,j,:]
 *     lse[b,h,i] = log(sum_j exp(s_ij))            (natural log)
 * Key j is visible to query i iff causal == 0 or j <= i.
 *
 *   q, k, v : [B, H, N, d] 16-bit (dtype), device, 16-byte aligned
 *   o       : [B, H, N, d] fp32, device, 16-byte aligned (written)
 *   lse     : [B, H, N]    fp32, device, 4-byte aligned, or NULL to skip
 *   d       : 64 or 128;  N <= 2^23 (else FA_ERR_SHAPE)
 *   scale   : finite; 1/sqrt(d) reproduces the usual default
 * B == 0, H == 0 or N == 0 is a no-op returning FA_OK.
 */
fa_status_t fa_fwd(const void *q, const void *k, const void *v, float *o,
                   float *lse, int B, int H, int N, int d, int causal,
                   float scale, hipStream_t stream, fa_dtype_t dtype);

/*
 * fa_fwd_varlen -- fa_fwd over a packed batch of sequences of different
 * lengths (jagged / variable-length attention; the "jagged attention" item
 * of the roadmap in the Triton warp-specialisation note).  Sequence b is
 * rows [cu_seqlens[b], cu_seqlens[b+1]) of the packed tensors and attends
 * only to itself (causal: key j visible to query i iff j <= i, both counted
 * within the sequence).
 *
 *   q, k, v    : [total_tokens, H, d] 16-bit, device, 16-byte aligned
 *   o          : [total_tokens, H, d] fp32, device, 16-byte aligned
 *   lse        : [H, total_tokens] fp32, device, or NULL
 *   cu_seqlens : [B + 1] int32, device: 0 = cu[0] <= cu[1] <= ... <= cu[B]
 *                = total_tokens
 *   max_seqlen : >= every cu[b+1] - cu[b] (host value; sizes the grid)
 *   d          : 64 or 128;  max_seqlen * H * d < 2^30 (else FA_ERR_SHAPE)
 * Device-side cu_seqlens are not validated: offsets are clamped to
 * [0, total_tokens] and lengths to max_seqlen, so a bad table gives wrong
 * results but no out-of-range access.  B == 0, H == 0 or total_tokens == 0
 * is a no-op returning FA_OK.
 */
fa_status_t fa_fwd_varlen(const void *q, const void *k, const void *v, float *o,
                          float *lse, const int *cu_seqlens, int B, int H,
                          int total_tokens, int max_seqlen, int d, int causal,
                          float scale, hipStream_t stream, fa_dtype_t dtype);

/*
 * fa_fwd_fp8 -- fa_fwd for FP8 inputs with per-tensor dequantization
 * factors: the FP8 variant of the tiled forward that the dailyaiworld page
 * features (introduction and pipeline figure).  q, k, v hold OCP E4M3
 * ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 fraction bits, largest
 * finite 448, no infinities) bytes; the result is fa_fwd's definition
 * applied to the dequantized tensors
 *     q = q_descale * q8,   k = k_descale * k8,   v = v_descale * v8
 * (same mask, lse and output layout).  Both products run in E4M3 with fp32
 * accumulation: the attention weights are rounded to E4M3 for the PV product
 * (relative error up to 2^-4 per weight), while the row sums and lse use the
 * fp32 weights.
 *
 *   q, k, v : [B, H, N, d] bytes, device, 16-byte aligned
 *   o, lse  : as fa_fwd (lse may be NULL)
 *   d       : 64 or 128;  N <= 2^23
 *   scale, q_descale, k_descale, v_descale : finite (else FA_ERR_VALUE)
 * Bytes holding the E4M3 NaN pattern (0x7f, 0xff) give undefined results.
 * B == 0, H == 0 or N == 0 is a no-op returning FA_OK.
 */
fa_status_t fa_fwd_fp8(const void *q, const void *k, const void *v, float *o,
                       float *lse, int B, int H, int N, int d, int causal,
                       float scale, float q_descale, float k_descale,
                       float v_descale, hipStream_t stream);

/*
 * fa_bwd -- gradients of fa_fwd's attention (the attention backward, which
 * "Warp Specialization in Triton: Design and Roadmap" lists on its roadmap
 * as the next kernel after the forward).  For O = softmax(scale Q K^T
 * [+ causal mask]) V and an upstream gradient dO = dL/dO, with
 * P_ij = exp(scale <q_i, k_j> - lse_i) on the visible keys:
 *     dV_j = sum_i P_ij dO_i
 *     dS_ij = P_ij (<dO_i, v_j> - <dO_i, O_i>)
 *     dQ_i = scale sum_j dS_ij k_j,    dK_j = scale sum_i dS_ij q_i
 * o and lse are fa_fwd's outputs for the same q, k, v, causal and scale;
 * P is rebuilt from lse, and nothing of size N x N is stored.  P and dS are
 * rounded to the storage dtype for the products that consume them, with
 * fp32 accumulation.  Two kernels run in stream order (dQ, then dK and dV);
 * results are deterministic (no atomics).
 *
 *   q, k, v, dout : [B, H, N, d]  16-bit (dtype), device, 16-byte aligned
 *   o             : [B, H, N, d]  fp32, device, 16-byte aligned
 *   lse           : [B, H, N]     fp32, device (natural log, as fa_fwd writes)
 *   dq, dk, dv    : [B, H, N, d]  fp32, device, 16-byte aligned (written)
 *   d             : 64 or 128;  N <= 2^23
 *   workspace     : device memory of at least fa_bwd_workspace_bytes(B, H, N)
 *                   bytes, 256-byte aligned (FA_ERR_WORKSPACE otherwise);
 *                   overwritten.  Calls sharing one workspace must not overlap.
 * B == 0, H == 0 or N == 0 is a no-op returning FA_OK.
 */
fa_status_t fa_bwd(const void *q, const void *k, const void *v, const float *o,
                   const void *dout, const float *lse, float *dq, float *dk,
                   float *dv, int B, int H, int N, int d, int causal, float scale,
                   hipStream_t stream, fa_dtype_t dtype, void *workspace,
                   size_t workspace_bytes);

/* Bytes of workspace fa_bwd needs: two fp32 values per query row, each array
 * 256-byte aligned (0 for negative sizes). */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_bwd_varlen -- fa_bwd for a packed variable-length batch, the backward of
 * fa_fwd_varlen (same layout and bounds): sequence b occupies rows
 * [cu_seqlens[b], cu_seqlens[b+1]) of tensors shaped [total_tokens, H, d],
 * and each sequence attends only to itself.
 *
 *   q, k, v, dout : [total_tokens, H, d]  16-bit (dtype), device, 16-byte aligned
 *   o             : [total_tokens, H, d]  fp32 (fa_fwd_varlen's output)
 *   lse           : [H, total_tokens]     fp32 (fa_fwd_varlen's output)
 *   dq, dk, dv    : [total_tokens, H, d]  fp32 (written; rows that belong to
 *                   no sequence are left untouched)
 *   cu_seqlens    : [B + 1] int32, device, non-decreasing, cu_seqlens[B] <=
 *                   total_tokens (bounds are clamped to [0, total_tokens]);
 *                   max_seqlen >= the longest sequence (longer ones are cut
 *                   to max_seqlen, as in fa_fwd_varlen)
 *   d             : 64 or 128;  max_seqlen * H * d < 2^30
 *   workspace     : at least fa_bwd_workspace_bytes(1, H, total_tokens) bytes,
 *                   256-byte aligned (FA_ERR_WORKSPACE otherwise)
 * B, H, total_tokens or max_seqlen == 0 is a no-op returning FA_OK.
 */
fa_status_t fa_bwd_varlen(const void *q, const void *k, const void *v,
                          const float *o, const void *dout, const float *lse,
                          float *dq, float *dk, float *dv, const int *cu_seqlens,
                          int B, int H, int total_tokens, int max_seqlen, int d,
                          int causal, float scale, hipStream_t stream,
                          fa_dtype_t dtype, void *workspace,
                          size_t workspace_bytes);

/*
 * fa_decode -- attention of one new query token per sequence against a
 * key/value cache, split along the cache length into nsplit shards whose
 * partial results (O_s, lse_s) are combined by log-sum-exp reweighting
 * (post.smzdm.com digest on Triton warp specialisation, section 5: shard
 * outputs cannot simply be added; each carries its lse and the combine
 * re-normalises with it):
 *     lse = log sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * O_s
 * Grouped-query attention: query head hq reads key/value head
 * hq / (Hq / Hkv).  Every cached key is visible; scale is 1/sqrt(d).
 *
 *   q              : [B, Hq, d]       16-bit, device, 16-byte aligned
 *   kcache, vcache : [B, Hkv, L, d]   16-bit, device, 16-byte aligned
 *   o              : [B, Hq, d]       fp32, device, 16-byte aligned (written)
 *   Hq % Hkv == 0; 1 <= L <= 2^23; nsplit >= 1 (clamped to L; shard s covers keys
 *   [s*C, min(L, (s+1)*C)) with C = ceil(L / nsplit)).
 * Partial results live in a per-device workspace that the library allocates
 * on first use and grows when a larger call needs it (guarded by a mutex;
 * calls on different streams of one device share it, so such calls must not
 * overlap in time).  B == 0 or Hq == 0 is a no-op returning FA_OK.
 */
fa_status_t fa_decode(const void *q, const void *kcache, const void *vcache,
                      float *o, int B, int Hq, int Hkv, int L, int d,
                      int nsplit, hipStream_t stream, fa_dtype_t dtype);

/* Bytes of workspace fa_decode_ex needs for these sizes (0 on bad sizes). */
size_t fa_decode_workspace_bytes(int B, int Hq, int d, int nsplit);

/*
 * fa_decode_ex -- fa_decode with the final lse (optional) and a
 * caller-owned device workspace of at least fa_decode_workspace_bytes()
 * bytes, 256-byte aligned (FA_ERR_WORKSPACE otherwise).  Calls sharing one
 * workspace must not overlap in time.
 *   lse : [B, Hq] fp32, device, or NULL
 */
fa_status_t fa_decode_ex(const void *q, const void *kcache,
                         const void *vcache, float *o, float *lse, int B,
                         int Hq, int Hkv, int L, int d, int nsplit,
                         hipStream_t stream, fa_dtype_t dtype,
                         void *workspace, size_t workspace_bytes);

/*
 * fa_decode_noalloc -- fa_decode_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops or harnesses that
 * forbid hipMalloc): same arguments minus the workspace, same results, and
 * no allocation of any kind.  The shard partials go to a fixed buffer of
 * FA_DECODE_NOALLOC_MAX_BYTES (8 MiB) that the library keeps in device memory
 * on every GPU it runs on, from the module load until the process ends; its
 * address is looked up (not allocated) on the first call on each device.
 * A call needing fa_decode_workspace_bytes(B, Hq, d, min(nsplit, L)) bytes
 * more than that returns FA_ERR_WORKSPACE before any HIP call (at d = 128:
 * about B * Hq * min(nsplit, L) <= 16000).  Every call on
 * one GPU shares that buffer: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give wrong results.
 *   lse : [B, Hq] fp32, device, or NULL
 */
fa_status_t fa_decode_noalloc(const void *q, const void *kcache,
                              const void *vcache, float *o, float *lse, int B,
                              int Hq, int Hkv, int L, int d, int nsplit,
                              hipStream_t stream, fa_dtype_t dtype);

/*
 * fa_decode_paged -- fa_decode_ex over a paged key/value cache with a length
 * per sequence (variable-length batches; the pages mention PagedAttention as
 * the serving-side cache layout next to FlashAttention).  Sequence b owns
 * seq_lens[b] cached keys; key j of it lives in page block_table[b][j / P],
 * slot j % P, of the shared pools
 *   kpages, vpages : [num_pages, P, Hkv, d] 16-bit, device, 16-byte aligned
 *   block_table    : [B, pages_per_seq] int32, device
 *   seq_lens       : [B] int32, device
 * with P = page_size, a positive multiple of 16.  Shard s of sequence b
 * covers keys [s*C_b, min(L_b, (s+1)*C_b)) with C_b = ceil(L_b / nsplit)
 * rounded up to a multiple of 32 (trailing shards may be empty and get
 * weight 0).  q, o, lse, nsplit, workspace and the definition are those of
 * fa_decode_ex (workspace from fa_decode_workspace_bytes(B, Hq, d, nsplit));
 * nsplit is not clamped.  A sequence with no keys gets O = 0 and lse = -inf.
 * Device-side contents are not validated: lengths are clamped to
 * [0, pages_per_seq * P] and page ids to [0, num_pages), so bad tables give
 * wrong results but no out-of-range access.
 */
fa_status_t fa_decode_paged(const void *q, const void *kpages, const void *vpages,
                            const int *block_table, const int *seq_lens, float *o,
                            float *lse, int B, int Hq, int Hkv, int page_size,
                            int pages_per_seq, int num_pages, int d, int nsplit,
                            hipStream_t stream, fa_dtype_t dtype, void *workspace,
                            size_t workspace_bytes);

/* Static English description of a status code. */
const char *fa_status_string(fa_status_t status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_AMD_FA_H */
