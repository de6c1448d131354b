/*
 * fa.h -- C ABI of libfa, an MI355X (gfx950) FlashAttention forward pass.
 *
 * Operations:
 *
 *   fa_fwd     exact softmax attention O = softmax(scale * Q K^T + mask) V for
 *              prefill, computed tile by tile with a running row maximum and
 *              running row sum so the N x N score and probability matrices never
 *              reach device memory; it also returns the per-row log-sum-exp.
 *              (Defined in "How FlashAttention Reduces HBM Traffic Exactly",
 *              section "The performance problem is data movement, not the
 *              attention formula"; the loop is the one in "FlashAttention and GPU
 *              Data Movement", sections 2 and 3.1; the log-sum-exp output is the
 *              statistic of "FlashAttention Explained: IO-Aware Attention,
 *              Tiling, Online Softmax and FP8 on Hopper", section "Why the
 *              statistics are cheap to store".)
 *
 *   fa_fwd_varlen  the same over packed variable-length sequences, with an
 *              optional sliding-window mask.
 *
 *   fa_bwd     gradients of fa_fwd with respect to q, k and v, recomputing the
 *              probabilities from the saved log-sum-exp.
 *
 *   fa_fp8_quantize, fa_fwd_fp8  FP8 (e4m3) prefill with incoherent processing.
 *
 *   fa_decode  single-token decode against a KV cache, with the key axis split
 *              across workgroups; every split writes a partial output and its
 *              log-sum-exp, and a second small kernel merges the partials
 *              ("FlashAttention Explained", section "Decoding, Paged and
 *              Split-KV Variants"; "FlashAttention and GPU Data Movement",
 *              section 6.1). fa_decode_paged reads the cache through a
 *              block table of fixed-size pages.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     allocates and frees nothing. Its only state between calls is the calling
 *     thread's last error message and a per-device cache of the compute-unit
 *     count (read once from the runtime, held in atomics).
 *   - Calls are asynchronous: FA_OK means the work was enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream). Results are
 *     valid once the caller synchronises that stream. Device faults surface at
 *     that synchronisation.
 *   - Every argument is validated before anything is launched: a non-OK
 *     status means nothing was enqueued and no output was written.
 *   - Supported combinations are finite. Anything outside them returns
 *     FA_ERR_UNSUPPORTED; there is no silent fallback to another algorithm.
 *   - Strides are in ELEMENTS of the tensor's own dtype. The head dimension is
 *     always contiguous (stride 1).
 *   - GQA: query head h reads key/value head h / (heads_q / heads_kv), i.e.
 *     consecutive query heads share one kv head.
 *   - The log-sum-exp is natural-log over the scaled, masked scores,
 *     LSE = m + ln(sum_c exp(s_c - m)), stored as float32.
 *   - Concurrent calls on different streams are safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FA_API __attribute__((visibility("default")))
#else
#define FA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, non-finite or non-positive scale */
  FA_ERR_UNSUPPORTED = 2,        /* valid request outside the implemented set (see each call) */
  FA_ERR_WORKSPACE_TOO_SMALL = 3,/* decode workspace smaller than fa_decode_workspace_bytes() */
  FA_ERR_HIP = 4                 /* the HIP runtime reported an error at launch */
} fa_status_t;

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP32 = 1 } fa_dtype_t;
typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1 } fa_mask_t;

/*
 * fa_fwd -- prefill attention forward.
 *
 * q   [batch, heads_q,  seqlen_q, head_dim]  in_dtype, strides q_stride  = {b, h, n}
 * k   [batch, heads_kv, seqlen_k, head_dim]  in_dtype, strides k_stride  = {b, h, n}
 * v   [batch, heads_kv, seqlen_k, head_dim]  in_dtype, strides v_stride  = {b, h, n}
 * o   [batch, heads_q,  seqlen_q, head_dim]  out_dtype, strides o_stride = {b, h, n}
 * lse [batch, heads_q,  seqlen_q] float32, contiguous; may be NULL (not written).
 *
 * in_dtype  BF16, or FP32 (values are rounded to bf16, nearest-even, as they are
 *           staged, and the products run on the bf16 matrix cores).
 * out_dtype BF16 (O rounded once, nearest-even, from the float32 result) or FP32.
 * mask      FA_MASK_NONE, or FA_MASK_CAUSAL: key c is visible to query row r iff
 *           c <= r; requires seqlen_q == seqlen_k. Key tiles wholly in a row
 *           tile's future are skipped; tiles on the diagonal are masked.
 * softmax_scale  multiplies Q K^T before the softmax (typically 1/sqrt(head_dim)).
 *
 * Supported: head_dim 64 or 128; heads_q % heads_kv == 0; every pointer 16-byte
 * aligned; every stride a multiple of 8 elements (bf16) or 4 elements (fp32);
 * the row strides k_stride[2] and v_stride[2] at most 2^24 elements (a key
 * tile is addressed with 32-bit offsets). Otherwise FA_ERR_UNSUPPORTED. q, k, v
 * must not overlap o or lse.
 */
FA_API fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int32_t batch, int32_t heads_q, int32_t heads_kv,
                   int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                   const int64_t q_stride[3], const int64_t k_stride[3],
                   const int64_t v_stride[3], const int64_t o_stride[3],
                   fa_dtype_t in_dtype, fa_dtype_t out_dtype, fa_mask_t mask,
                   float softmax_scale, void* stream);

/*
 * fa_fwd_varlen -- prefill over a packed batch of variable-length sequences,
 * optionally with a sliding-window mask.
 *
 * Sequences are concatenated on the token axis and described by cumulative
 * offsets, so no work is spent on padding ("FlashAttention Explained: IO-Aware
 * Attention, Tiling, Online Softmax and FP8 on Hopper", section "Trade-offs,
 * Gotchas, and What Goes Wrong"). Sequence b owns tokens cu_seqlens[b] ..
 * cu_seqlens[b+1]-1 of q, k, v and o alike and attends only to itself, with
 * positions counted from its own first token. The sliding window is the
 * causal mask restricted to the last window+1 keys: key c is visible to row r
 * iff c <= r and r - c <= window (same page, section "FlexAttention"; key
 * tiles wholly outside every row's window are skipped, as the causal mask
 * skips future tiles: "FlashAttention and Why Attention Is a Memory-Traffic
 * Problem").
 *
 * q   [total_tokens, heads_q,  head_dim] bf16, strides q_stride = {token, head}
 * k   [total_tokens, heads_kv, head_dim] bf16, strides k_stride = {token, head}
 * v   [total_tokens, heads_kv, head_dim] bf16, strides v_stride = {token, head}
 * o   [total_tokens, heads_q,  head_dim] out_dtype, strides o_stride = {token, head}
 * lse [heads_q, total_tokens] float32, contiguous; may be NULL.
 * cu_seqlens  DEVICE int32 [batch + 1], non-decreasing, cu_seqlens[0] = 0 and
 *             cu_seqlens[batch] <= total_tokens. Entries are clamped into
 *             [0, total_tokens] on the device, so no access leaves the buffers.
 * max_seqlen  an upper bound of every sequence's length (sizes the grid); rows
 *             of a longer sequence past max_seqlen are not written.
 * mask        FA_MASK_NONE or FA_MASK_CAUSAL (within each sequence).
 * window      -1 for none, else >= 0 and only with FA_MASK_CAUSAL.
 *
 * Supported: bf16 inputs; head_dim 64 or 128; heads_q % heads_kv == 0;
 * 16-byte aligned pointers; strides multiples of 16 bytes; k/v token strides at
 * most 2^24 elements. Otherwise FA_ERR_UNSUPPORTED. o must not overlap q, k, v.
 * With uniform lengths and a token-major layout this computes exactly what
 * fa_fwd computes on the same memory (same kernels, same tiles, same bits).
 */
FA_API fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                          int32_t total_tokens, int32_t max_seqlen, int32_t head_dim,
                          const int64_t q_stride[2], const int64_t k_stride[2],
                          const int64_t v_stride[2], const int64_t o_stride[2],
                          fa_dtype_t out_dtype, fa_mask_t mask, int32_t window, float softmax_scale,
                          void* stream);

/*
 * fa_decode_workspace_bytes -- device workspace fa_decode (and fa_decode_paged)
 * needs for these sizes and this split_tokens: float32 partial outputs and
 * log-sum-exps, one set of heads_q/heads_kv heads per piece of work. A piece
 * is the part of one (sequence, kv head) slab that falls in one workgroup's
 * range; the ranges cut the slabs at most (grid size - 1) times, so there are
 * at most batch*heads_kv plus the decode grid's size pieces for any
 * split_tokens, and the size returned does not change with it (the argument
 * is kept so a caller sizes the workspace for exactly the call it makes).
 * Returns 0 for invalid sizes.
 */
FA_API size_t fa_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t max_seqlen_k, int32_t head_dim, int32_t split_tokens);

/*
 * fa_decode -- one query token per sequence against a contiguous KV cache.
 *
 * q        [batch, heads_q, head_dim] bf16, contiguous
 * k_cache  [batch, heads_kv, max_seqlen_k, head_dim] bf16, strides kv_stride = {b, h, n}
 * v_cache  same shape and strides as k_cache
 * seqlens_k  DEVICE int32 [batch]: sequence b attends to cache rows
 *          0 .. seqlens_k[b]-1 and never reads rows at or past that length.
 *          Values are clamped to [0, max_seqlen_k]; a length of 0 yields O = 0
 *          and LSE = -inf for that sequence.
 * o        [batch, heads_q, head_dim] out_dtype, contiguous
 * lse      [batch, heads_q] float32, contiguous; may be NULL.
 * split_tokens  the cached rows of all sequences are cut into equal contiguous
 *          ranges, one per workgroup of a fixed grid; split_tokens > 0 is a
 *          lower bound on the keys of one range, <= 0 leaves the ranges as even
 *          as the grid allows. LSE does not depend on it beyond float32
 *          rounding; O may move by the bf16 rounding of the probabilities,
 *          which each range takes relative to its own running maximum.
 * workspace      device buffer of at least fa_decode_workspace_bytes(batch,
 *          heads_q, heads_kv, max_seqlen_k, head_dim, split_tokens) bytes,
 *          16-byte aligned; its contents on entry do not matter and are
 *          overwritten. Two calls that share a workspace must be ordered.
 *
 * Supported: head_dim 64 or 128; heads_q % heads_kv == 0 and heads_q / heads_kv <= 32;
 * bf16 q and cache; pointers 16-byte aligned; kv strides multiples of 8.
 * Every cache row a sequence may read (index < its length) must lie inside
 * the caches; rows at or past a sequence's length are never read.
 */
FA_API fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens_k, void* o, float* lse,
                      int32_t batch, int32_t heads_q, int32_t heads_kv,
                      int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                      fa_dtype_t out_dtype, float softmax_scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc -- fa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. The arguments, the kernels and the result are
 * fa_decode's (on the same inputs the two return identical bits); only the
 * partials workspace differs: it is a static array inside the library, 16 MiB
 * on each GPU the library runs on, held until the process ends. Nothing is
 * allocated or freed by this call.
 *
 * Limit: fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen_k,
 * head_dim, split_tokens) must not exceed 16 MiB (16777216 bytes); larger
 * sizes return FA_ERR_UNSUPPORTED before anything is launched. (The bench's
 * 64 sequences x 64 query heads over 8 kv heads at head_dim 128 need about
 * 5.3 MB.)
 *
 * All calls on one GPU share that GPU's array and nothing in it needs to start
 * at zero (every partial the merge reads is written first by the same call).
 * Two calls whose kernels overlap on one GPU race on it: order them (one
 * stream, or events), or use fa_decode with separate workspaces. The first
 * call on a device looks up the array's device address (hipGetSymbolAddress);
 * a failure there returns FA_ERR_HIP.
 */
FA_API fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* seqlens_k, void* o, float* lse,
                                     int32_t batch, int32_t heads_q, int32_t heads_kv,
                                     int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                                     fa_dtype_t out_dtype, float softmax_scale, int32_t split_tokens,
                                     void* stream);

/*
 * fa_decode_paged -- fa_decode against a paged KV cache: the cache lives in
 * fixed-size pages that need not be contiguous or in order, and a block table
 * maps each sequence's logical blocks of page_size tokens to physical pages
 * ("FlashAttention Explained: IO-Aware Attention, Tiling, Online Softmax and
 * FP8 on Hopper", section "Decoding, Paged and Split-KV Variants": a paged
 * kernel reads keys and values through the block table). Token t of sequence
 * b is slot t % page_size of page block_table[b * max_blocks_per_seq +
 * t / page_size]. The split, the arithmetic and the merge are those of
 * fa_decode, so on the same cached values the two return identical bits.
 *
 * q            [batch, heads_q, head_dim] bf16, contiguous
 * k_pages      num_pages pages of page_size tokens x heads_kv heads, bf16;
 *              element (page, kv head, slot, d) at
 *              page * page_stride[0] + head * page_stride[1] + slot * page_stride[2] + d
 *              (any order of the three outer axes, head_dim contiguous)
 * v_pages      same layout and strides as k_pages
 * block_table  DEVICE int32 [batch, max_blocks_per_seq]; only the entries of
 *              blocks that hold one of the first seqlens_k[b] tokens are read.
 *              An entry outside [0, num_pages) is clamped into it (the result is
 *              then meaningless, but no access leaves the page arrays).
 * seqlens_k    DEVICE int32 [batch], clamped to [0, max_blocks_per_seq * page_size];
 *              a length of 0 yields O = 0 and LSE = -inf
 * o, lse, out_dtype, softmax_scale, split_tokens: as for fa_decode
 * workspace    at least fa_decode_workspace_bytes(batch, heads_q, heads_kv,
 *              max_blocks_per_seq * page_size, head_dim, split_tokens) bytes,
 *              16-byte aligned
 *
 * Supported: head_dim 64 or 128; heads_q % heads_kv == 0 and heads_q / heads_kv <= 32;
 * page_size >= 16 (a 32-key block then spans at most three pages); pointers
 * 16-byte aligned; page strides multiples of 8 elements; page_size *
 * page_stride[2] < 2^31 elements. Otherwise FA_ERR_UNSUPPORTED.
 */
FA_API fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, const int32_t* seqlens_k, void* o, float* lse,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                            int32_t num_pages, int32_t page_size, int32_t max_blocks_per_seq,
                            const int64_t page_stride[3], fa_dtype_t out_dtype, float softmax_scale,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_workspace_bytes -- device workspace fa_bwd needs: one float per query
 * row (rowsum(dO * O)). 0 for non-positive sizes.
 */
FA_API size_t fa_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t seqlen_q);

/*
 * fa_bwd -- gradients of fa_fwd with respect to q, k and v, by recomputation:
 * the probabilities are rebuilt tile by tile from q, k and the forward pass's
 * log-sum-exp instead of being stored ("FlashAttention Explained: IO-Aware
 * Attention, Tiling, Online Softmax and FP8 on Hopper", section "Backward
 * Pass: Recomputation Beats Storage"). With P = exp(scale q k^T - lse) under
 * the mask: D = rowsum(dout * o), dv = P^T dout, dP = dout v^T,
 * dS = P * (dP - D), dq = scale dS k, dk = scale dS^T q. Under GQA dk and dv
 * of a kv head sum the contributions of its query heads. No atomics: the
 * result is deterministic.
 *
 * q, dout    [batch, heads_q, seqlen_q, head_dim] bf16, strides q_stride = {b, h, n}
 * o           the same shape and element strides, o_dtype: BF16 or FP32. D is
 *             computed from o as given; with a peaked softmax dP - D cancels,
 *             so an FP32 o (fa_fwd with out_dtype FP32) gives visibly more
 *             accurate dq and dk than the bf16-rounded one.
 * k, v        [batch, heads_kv, seqlen_k, head_dim] bf16, strides kv_stride
 * lse         [batch, heads_q, seqlen_q] float32, contiguous, as fa_fwd wrote it
 *             (with the same q, k, v, mask and softmax_scale; o is fa_fwd's output)
 * dq          [batch, heads_q, seqlen_q, head_dim] grad_dtype, strides dq_stride
 * dk, dv      [batch, heads_kv, seqlen_k, head_dim] grad_dtype, strides dkv_stride
 * grad_dtype  BF16 (rounded once, nearest-even) or FP32
 * mask        FA_MASK_NONE, or FA_MASK_CAUSAL (seqlen_q == seqlen_k)
 * workspace   at least fa_bwd_workspace_bytes(batch, heads_q, seqlen_q) bytes,
 *             16-byte aligned
 *
 * Supported: head_dim 64 or 128; heads_q % heads_kv == 0; 16-byte aligned
 * pointers; input strides multiples of 8 elements, gradient strides multiples
 * of 16 bytes. Otherwise FA_ERR_UNSUPPORTED. Gradients must not overlap any
 * input, each other or the workspace (FA_ERR_INVALID_ARGUMENT).
 */
FA_API fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q,
                          int32_t heads_kv, int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                          const int64_t q_stride[3], const int64_t kv_stride[3], const int64_t dq_stride[3],
                          const int64_t dkv_stride[3], fa_dtype_t o_dtype, fa_dtype_t grad_dtype, fa_mask_t mask,
                          float softmax_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fp8_quantize -- the quantiser of the FP8 path ("FlashAttention Explained:
 * IO-Aware Attention, Tiling, Online Softmax and FP8 on Hopper", section "FP8
 * Attention and Incoherent Processing"). Q and K rows are multiplied by the
 * same orthogonal matrix diag(signs) H / sqrt(128) (H the Sylvester Hadamard
 * matrix; a fast Walsh-Hadamard transform in float32), which leaves Q K^T
 * unchanged, then stored as OCP e4m3 (largest finite 448, nearest-even) with
 * one float32 scale per block: codes = e4m3(x * 448 / amax), scale =
 * amax / 448 (1 for an all-zero block). V is not rotated; it gets one scale
 * per kv head.
 *
 * q       [batch, heads_q, seqlen, 128] bf16, strides q_stride = {b, h, n}
 * k, v    [batch, heads_kv, seqlen, 128] bf16, strides kv_stride
 * signs   DEVICE float [128] of +1/-1 drawn by the caller, or NULL for no
 *         rotation (plain block quantisation)
 * outputs (contiguous, caller-owned):
 *   q8       [batch, heads_q, seqlen, 128] e4m3 bytes
 *   q_scale  [batch, heads_q, ceil(seqlen / 128)] float32 (one per 128 rows)
 *   k8       [batch, heads_kv, seqlen, 128] e4m3 bytes
 *   k_scale  [batch, heads_kv, ceil(seqlen / 64)] float32 (one per 64 keys)
 *   v8t      [batch, heads_kv, 128, npad] e4m3 bytes, npad = 64 ceil(seqlen / 64):
 *            V transposed; inside every 64-key tile key kappa sits at position
 *            32 ((kappa / 4) % 2) + 16 (kappa / 32) + 4 ((kappa % 32) / 8) + kappa % 4;
 *            padding keys are zero
 *   v_scale  [batch, heads_kv] float32 (while the call's kernels run on the
 *            stream it holds V's running maximum: read it after them)
 * Supported: head_dim 128; heads_q % heads_kv == 0; 16-byte aligned tensors;
 * strides multiples of 8 elements. Otherwise FA_ERR_UNSUPPORTED.
 */
FA_API fa_status_t fa_fp8_quantize(const void* q, const void* k, const void* v, const float* signs,
                                   int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen,
                                   int32_t head_dim, const int64_t q_stride[3], const int64_t kv_stride[3],
                                   void* q8, void* k8, void* v8t, float* q_scale, float* k_scale, float* v_scale,
                                   void* stream);

/*
 * fa_fwd_fp8 -- prefill attention on fa_fp8_quantize's outputs: both products
 * on the e4m3 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), the softmax in
 * float32. The probabilities are quantised too, as e4m3(2^8 * 2^(x - m)) with
 * x the scaled score in base 2 and m an integer base at or above the row's
 * running maximum; O is divided by the sum of the quantised weights; the LSE
 * is the float32 log-sum-exp of the dequantised scores. FP8 changes numerics:
 * results differ from fa_fwd by the quantisation error (about 1% mean on O).
 *
 * o    [batch, heads_q, seqlen, 128] out_dtype (BF16 or FP32), contiguous
 * lse  [batch, heads_q, seqlen] float32, contiguous; may be NULL
 * mask FA_MASK_NONE or FA_MASK_CAUSAL
 * Supported: head_dim 128; heads_q % heads_kv == 0; 16-byte aligned tensors.
 */
FA_API fa_status_t fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale,
                              const float* k_scale, const float* v_scale, void* o, float* lse, int32_t batch,
                              int32_t heads_q, int32_t heads_kv, int32_t seqlen, int32_t head_dim,
                              fa_dtype_t out_dtype, fa_mask_t mask, float softmax_scale, void* stream);

/* Static description of a status code. Never NULL. */
FA_API const char* fa_status_string(fa_status_t status);

/* Detail of the calling thread's most recent non-OK return ("" if none). */
FA_API const char* fa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
