/*
 * libfa_mi355x — FlashAttention forward (and its backward) for AMD Instinct
 * MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes; no C++ or framework types cross it.
 *
 * What fa_fwd computes, per (batch b, head h) and query row i:
 *
 *   S_ij = scale * sum_d q[b,h,i,d] * k[b,h,j,d]
 *   S_ij = -inf where causal and j > i           (top-left aligned)
 *   O[b,h,i,:] = sum_j softmax_j(S_i.) * v[b,h,j,:]
 *   lse[b,h,i] = ln sum_j exp(S_ij)              (natural log)
 *
 * The definition follows the PyTorch reference used for the correctness
 * check in "ops-transformer FlashAttention on Ascend: build, run and tune"
 * (ai6s.net/6a31724f..., section 4.3): scores scaled by `scale` before the
 * mask, the strict upper triangle filled with -inf, softmax over keys, then
 * the product with V. The call shape (q, k, v, head count, input_layout
 * "BNSD", scale, keep_prob) is the one of npu_flash_attention in "Tracing
 * npu_flash_attention through the CANN runtime" (ai6s.net/6a114bb2...,
 * layer 1). The computation order is FlashAttention-2's: the outer loop runs
 * over blocks of query rows, an online softmax keeps the running row maximum
 * and row sum, and S and P never reach device memory (first page, section
 * 1.2). The per-row logsumexp output is not defined on the pages; it is the
 * natural-log logsumexp of the scaled, masked score row.
 *
 * Layout: contiguous BNSD (fa_fwd_ex also takes BSHD, see fa_layout_t). q
 * and o: element (b,h,s,d) at ((b*H+h)*Sq+s)*D+d; k and v:
 * ((b*H+h)*Sk+s)*D+d; lse: fp32 [B,H,Sq] at (b*H+h)*Sq+s. All offsets are
 * computed in 64-bit integers.
 *
 * Supported (in_dtype -> o_dtype): F16 -> {F16, F32}; BF16 -> {BF16, F32};
 * FP8_E4M3 -> {F16, F32}. Head dim D in {64, 128}. FP8_E4M3 is OCP e4m3fn;
 * the value of an fp8 element is code * descale, with one fp32 descale per
 * tensor (a device pointer to a single float, read with stride 0, as the
 * fp8 scale tensors are broadcast in "Hygon FlashAttention: fixed-defect
 * review", chatdocs.ruinique.com/hygon/flash-attention-fixed-bugs, item 17).
 *
 * Ownership: the caller owns every buffer. The library allocates and frees
 * no device memory, never synchronises, and enqueues its kernels on `stream`
 * before returning. q, k, v and the descales are read only; o and lse are
 * written only in their valid region [B,H,Sq,D] and [B,H,Sq].
 *
 * Errors: the entry points return a status code and never throw. On any
 * error other than FA_ERR_HIP nothing is launched and the outputs are
 * untouched.
 *
 * Thread safety: the entry points keep no mutable state (except the
 * per-device address cache of fa_fwd_splitkv_noalloc, taken under a lock)
 * and may be called from several threads on different streams; calls of
 * fa_fwd_splitkv_noalloc that overlap on one GPU race on its array.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 8

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_POINTER = 1,         /* q, k, v, o or lse is NULL, or an fp8 descale is NULL */
  FA_ERR_BAD_SHAPE = 2,            /* B, H, Sq or Sk < 1, or a size overflows 64-bit offsets or the grid */
  FA_ERR_UNSUPPORTED_HEAD_DIM = 3, /* D not in {64, 128} */
  FA_ERR_UNSUPPORTED_DTYPE = 4,    /* (in_dtype, o_dtype) pair not supported */
  FA_ERR_UNSUPPORTED_LAYOUT = 5,   /* layout not one of fa_layout_t */
  FA_ERR_UNSUPPORTED_DROPOUT = 6,  /* keep_prob != 1.0 on an entry point without dropout, or
                                      keep_prob outside (0, 1] for fa_fwd_dropout / fa_bwd_dropout */
  FA_ERR_BAD_SCALE = 7,            /* scale is NaN or infinite */
  FA_ERR_MISALIGNED = 8,           /* a tensor pointer is not 16-byte aligned (lse: 4-byte) */
  FA_ERR_ALIASING = 9,             /* o or lse overlaps q, k, v, or each other */
  FA_ERR_HIP = 10,                 /* a kernel launch failed */
  FA_ERR_WORKSPACE = 11,           /* split-KV: workspace NULL or smaller than needed */
  FA_ERR_UNSUPPORTED_MASK = 12,    /* fa_fwd_ex: mask not one of fa_mask_t */
  FA_ERR_SCRATCH = 13              /* fa_fwd_splitkv_noalloc: the problem needs more than its
                                      static workspace, or `stream` is not on the current device */
} fa_status_t;

/* Memory layouts of q, k, v and o (contiguous): BNSD = [B, heads, S, D];
 * BSHD = [B, S, heads, D] (the sequence-major [B, S, H*D] tensors of the
 * first page's data generator and verifier, section 4, with the hidden
 * size split into heads). lse is [B, H, Sq] fp32 in either layout. */
typedef enum { FA_LAYOUT_BNSD = 0, FA_LAYOUT_BSHD = 1 } fa_layout_t;

typedef enum { FA_F16 = 0, FA_BF16 = 1, FA_FP8_E4M3 = 2, FA_F32 = 3 } fa_dtype_t;

/* Causal masks. TOP_LEFT: key j visible to query i iff j <= i (the
 * verifier's upper-triangle mask in "ops-transformer FlashAttention on
 * Ascend: build, run and tune", section 4.3; every row sees key 0).
 * BOTTOM_RIGHT: iff j <= i + (Sk - Sq), the diagonal through the last query
 * and the last key (the same as TOP_LEFT when Sq == Sk); with Sq > Sk the
 * first Sq - Sk rows see no key and get O = 0, lse = -inf. */
typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL_TOP_LEFT = 1, FA_MASK_CAUSAL_BOTTOM_RIGHT = 2 } fa_mask_t;

/*
 * fa_fwd — attention forward on one GPU.
 *
 * q [B,H,Sq,D], k [B,H,Sk,D], v [B,H,Sk,D] in in_dtype (device pointers);
 * o [B,H,Sq,D] in o_dtype and lse [B,H,Sq] fp32 (device pointers, written).
 * scale: any finite float (the configurations use 1/sqrt(D)).
 * causal: 0 = no mask; any other value = top-left causal mask (key j is
 *   visible to query i iff j <= i), so every row has at least one key.
 * keep_prob: must be 1.0.
 * descale_q/k/v: device pointers to one fp32 each for FA_FP8_E4M3 inputs;
 *   ignored (may be NULL) otherwise.
 * stream: HIP stream to enqueue on (0 = the null stream).
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                   fa_layout_t layout, float scale, int causal, float keep_prob,
                   fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                   const float* descale_q, const float* descale_k, const float* descale_v,
                   hipStream_t stream);

/*
 * fa_fwd_splitkv — the same computation as fa_fwd, with the keys of every
 * block of query rows split into num_splits ranges that run as separate
 * workgroups, for shapes whose blocks alone would leave most of the GPU
 * idle (few heads, short or causal sequences). Each range writes its own
 * normalised output O_s and logsumexp lse_s (fp32, in the workspace); a
 * second kernel merges them: lse = ln sum_s exp(lse_s), O = sum_s
 * exp(lse_s - lse) * O_s. This is the softmax identity for a split key set,
 * the merge that the per-row logsumexp output exists for; the partition
 * reduce of "Hygon FlashAttention: fixed-defect review" (item 7) combines
 * split partitions the same way. Results equal fa_fwd's up to rounding.
 *
 * Arguments as fa_fwd, plus:
 * num_splits: ranges per block of query rows, 0..256; 0 chooses the count:
 *   more than one only when the blocks of query rows would fill fewer than
 *   half of the GPU's resident workgroup slots and every range keeps at
 *   least 16 tiles of 32 keys (then about one full round of the slots), 1
 *   otherwise. Ranges past the last key are empty and cost one workgroup
 *   each.
 * workspace, workspace_size: device memory of at least
 *   fa_fwd_splitkv_workspace_size(...) bytes, 256-byte aligned, owned by the
 *   caller, not overlapping any other argument; its contents on entry do not
 *   matter and on return are unspecified. May be NULL when that size is 0
 *   (a single range: one kernel, as fa_fwd).
 * Enqueues two kernels on `stream` (one when a single range is used).
 * Errors as fa_fwd, plus FA_ERR_BAD_SHAPE for num_splits out of range,
 * FA_ERR_WORKSPACE for a missing or short workspace, FA_ERR_MISALIGNED and
 * FA_ERR_ALIASING for the workspace; nothing is launched on error.
 */
fa_status_t fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                           fa_layout_t layout, float scale, int causal, float keep_prob,
                           fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                           const float* descale_q, const float* descale_k, const float* descale_v,
                           int num_splits, void* workspace, int64_t workspace_size,
                           hipStream_t stream);

/*
 * Bytes of workspace fa_fwd_splitkv needs for these sizes and num_splits
 * (0: the automatic count); 0 when a single range is used; -1 for sizes or
 * num_splits that fa_fwd_splitkv would reject. Host only; no HIP call.
 */
int64_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                      int causal, int num_splits);

/*
 * fa_fwd_splitkv_noalloc — fa_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid it): it allocates nothing and takes no workspace.
 * The partial results live in a static 64 MiB device array of the library
 * (each GPU the library runs on holds one until the process ends), so a
 * problem whose fa_fwd_splitkv_workspace_size(B, H, Sq, Sk, D, causal,
 * num_splits) exceeds 67108864 bytes is rejected with FA_ERR_SCRATCH, and
 * so is a `stream` that does not belong to the current device. Nothing in
 * the array needs to start at zero. All calls on one GPU share its array:
 * calls that overlap in time on one GPU (several streams, several host
 * threads) race and give wrong results; serialise them. Other arguments,
 * results and errors as fa_fwd_splitkv.
 */
fa_status_t fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                   fa_layout_t layout, float scale, int causal, float keep_prob,
                                   fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                                   const float* descale_q, const float* descale_k,
                                   const float* descale_v, int num_splits, hipStream_t stream);

/*
 * fa_fwd_ex — the general entry point behind fa_fwd and fa_fwd_splitkv:
 * grouped key/value heads, the causal mask alignment, and the split-KV
 * arguments.
 *
 * k, v: [B, H_kv, Sk, D] with H_kv dividing H; query head h attends to
 *   key/value head h / (H / H_kv) (H_kv = H: one each; H_kv = 1: one shared
 *   head). Layout of k, v: ((b*H_kv+g)*Sk+s)*D+d.
 * mask: one of fa_mask_t (FA_ERR_UNSUPPORTED_MASK otherwise).
 * num_splits, workspace, workspace_size: as fa_fwd_splitkv (num_splits = 1
 *   and a NULL workspace give one kernel, as fa_fwd); the workspace size
 *   comes from fa_fwd_splitkv_workspace_size(B, H, Sq, Sk, D, mask != 0,
 *   num_splits).
 * Other arguments, ownership and errors as fa_fwd; H_kv < 1, H_kv > H or
 * H % H_kv != 0 is FA_ERR_BAD_SHAPE. The variants follow the pages' call
 * and lessons: the npu_flash_attention call takes head_num and a layout;
 * grouped heads and the bottom-right diagonal are the Sq != Sk and
 * layout-contract lessons of "Hygon FlashAttention: fixed-defect review",
 * item 12.
 */
fa_status_t fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                      fa_layout_t layout, float scale, fa_mask_t mask, float keep_prob,
                      fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                      const float* descale_q, const float* descale_k, const float* descale_v,
                      int num_splits, void* workspace, int64_t workspace_size,
                      hipStream_t stream);

/*
 * fa_fwd_varlen — B sequences of different lengths in packed, sequence-major
 * tensors: q and o [total_q, H, D], k and v [total_k, H_kv, D] (element
 * (t, h, d) at (t*H + h)*D + d), sequence b owning query rows
 * cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1. cu_seqlens_q, cu_seqlens_k: device int32 arrays of
 * B+1 nondecreasing offsets from 0 to total_q (total_k). max_seqlen_q: the
 * longest query length (sizes the grid; rows beyond it are not computed).
 * lse: fp32 [H, total_q]. Each sequence is attended on its own, with the
 * mask (and the bottom-right diagonal) placed per sequence; a sequence
 * with no key gives O = 0 and lse = -inf. The library does not read the
 * offsets on the host: offsets that break the rules above give undefined
 * results (the kernel clamps them into the packed tensors, so it never
 * reads or writes outside them). Other arguments and errors as fa_fwd_ex;
 * no split-KV. One kernel on `stream`.
 */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int64_t B, int64_t H, int64_t H_kv, int64_t total_q, int64_t total_k,
                          int64_t max_seqlen_q, int64_t D, float scale, fa_mask_t mask,
                          float keep_prob, fa_dtype_t in_dtype, fa_dtype_t o_dtype,
                          const float* descale_q, const float* descale_k, const float* descale_v,
                          hipStream_t stream);

/*
 * fa_fwd_dropout — the forward of fa_fwd_ex (one key range) with dropout on
 * the normalised probabilities: O = (P * Z / keep_prob) V, lse over all
 * visible keys as without dropout. The pages pass keep_prob through the
 * call ("Tracing npu_flash_attention through the CANN runtime", layer 1)
 * without defining it; this is inverted dropout with a stated mask:
 * Philox4x64-10 (Salmon et al., SC 2011) keyed by (seed, offset); for query
 * head index bh = b*H + h, query row i, 32-key tile t and half u in {0, 1},
 * the counter (2t + u, i, bh, 0) gives 256 bits read as sixteen 16-bit
 * values (value n = bits 16n .. 16n+15, first output word lowest); key
 * 32t + 8m + 4u + e (m, e in 0..3) takes value 4m + e and is kept iff it is
 * below round(keep_prob * 65536) (clamped to 1..65535). The same (seed,
 * offset) give the same mask on every call. keep_prob in (0, 1] (1: no
 * dropout); otherwise FA_ERR_UNSUPPORTED_DROPOUT. Other arguments and errors
 * as fa_fwd_ex.
 */
fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                           fa_layout_t layout, float scale, fa_mask_t mask, float keep_prob,
                           uint64_t seed, uint64_t offset, fa_dtype_t in_dtype,
                           fa_dtype_t o_dtype, const float* descale_q, const float* descale_k,
                           const float* descale_v, hipStream_t stream);

/*
 * Backward pass: the gradients of O = softmax(scale * Q K^T + mask) V for a
 * cotangent dO, recomputing P from the forward's lse (the backward whose dQ
 * pass "Hygon FlashAttention: fixed-defect review",
 * chatdocs.ruinique.com/hygon/flash-attention-fixed-bugs, item 13,
 * discusses; the formulas are the derivative of the forward):
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale * dS K, dK = scale * dS^T Q,
 * dK and dV of a key/value head summed over the query heads that share it
 * (deterministic: no atomics).
 *
 * q, o, dout: [B, H, Sq, D] and k, v: [B, H_kv, Sk, D], contiguous BNSD, in
 * in_dtype (FA_F16 or FA_BF16); lse: fp32 [B, H, Sq] as fa_fwd writes it (a
 * row without a visible key: -inf). dq [B, H, Sq, D], dk, dv [B, H_kv, Sk, D]
 * in grad_dtype (in_dtype or FA_F32), written whole. D 64 or 128; mask and
 * scale as fa_fwd_ex. workspace: device memory of at least
 * fa_bwd_workspace_size(B, H, Sq) bytes, 256-byte aligned, owned by the
 * caller (per-row lse in log2 units and rowsum(dO * O)); contents on entry
 * do not matter. Device pointers 16-byte aligned (lse: 4). Three kernels on
 * `stream`. Errors as fa_fwd_ex (FA_ERR_WORKSPACE: missing or small
 * workspace; FA_ERR_ALIASING: an output or the workspace overlaps another
 * tensor).
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H,
                   int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, float scale, fa_mask_t mask,
                   fa_dtype_t in_dtype, fa_dtype_t grad_dtype, void* workspace,
                   int64_t workspace_size, hipStream_t stream);

/*
 * fa_bwd_dropout — the backward of fa_fwd_dropout: the same arguments as
 * fa_bwd plus keep_prob, seed and offset, which must be those of the
 * forward call (the mask is drawn again from them, as fa_fwd_dropout
 * states it). o is the dropped forward output. With the mask Z fixed,
 * dV = (P * Z / keep_prob)^T dO and dP * Z / keep_prob is the gradient
 * reaching P (the derivative of the dropped forward). keep_prob in (0, 1]
 * (1: fa_bwd); otherwise FA_ERR_UNSUPPORTED_DROPOUT.
 */
fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D,
                           float scale, fa_mask_t mask, float keep_prob, uint64_t seed,
                           uint64_t offset, fa_dtype_t in_dtype, fa_dtype_t grad_dtype,
                           void* workspace, int64_t workspace_size, hipStream_t stream);

/* Workspace bytes fa_bwd needs (8 bytes per query row, rows rounded up to a
 * multiple of 32 per head); -1 for sizes it rejects: the kernels address
 * the workspace with 32-bit byte offsets, so B * H * (Sq rounded up to 32)
 * * 8 must not exceed INT32_MAX (at most 268,435,455 padded query rows over
 * all heads), and fa_bwd returns FA_ERR_BAD_SHAPE for larger problems. */
int64_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t Sq);

/* Human-readable name of a status code ("FA_OK", ...); never NULL. */
const char* fa_status_str(fa_status_t s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
