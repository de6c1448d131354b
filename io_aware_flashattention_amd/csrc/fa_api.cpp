// C ABI of libfa: argument validation, instantiation choice and launch.
// Every check runs before anything is enqueued, so an error return means no
// work was launched and no output was touched. Unsupported combinations fail
// loudly instead of falling back to another algorithm.
#include "../../include/fa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "fa_launch.h"

namespace {

thread_local std::string g_last_error;

fa_status_t fail(fa_status_t s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

fa_status_t ok() {
  g_last_error.clear();
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte span [lo, hi) a strided [batch, heads, rows, head_dim] tensor touches.
void span(const void* base, const int64_t st[3], int64_t nb, int64_t nh, int64_t nr, int64_t d,
          int64_t elem, uintptr_t* lo, uintptr_t* hi) {
  int64_t last = (nb - 1) * st[0] + (nh - 1) * st[1] + (nr - 1) * st[2] + d;
  *lo = reinterpret_cast<uintptr_t>(base);
  *hi = *lo + static_cast<uintptr_t>(last * elem);
}

bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

extern "C" {

fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, const int32_t* seqlens_k, void* o, float* lse,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t head_dim,
                            int32_t num_pages, int32_t page_size, int32_t max_blocks_per_seq,
                            const int64_t page_stride[3], fa_dtype_t out_dtype, float softmax_scale,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seqlens_k || !o || !page_stride)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "fa_decode_paged: q, pages, block_table, seqlens_k, o and page_stride must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || head_dim <= 0 || num_pages <= 0 || page_size <= 0 ||
      max_blocks_per_seq <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_paged: sizes must be positive");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_paged: softmax_scale must be finite and positive (got %g)",
                (double)softmax_scale);
  if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_paged: unknown out_dtype %d", (int)out_dtype);
  for (int i = 0; i < 3; ++i)
    if (page_stride[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_paged: strides must be non-negative");
  if ((int64_t)max_blocks_per_seq * page_size > 0x7fffffffLL - 64)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_decode_paged: max_blocks_per_seq * page_size overflows int32");
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: head_dim %d not supported (64 or 128)", head_dim);
  if (heads_q % heads_kv != 0 || heads_q / heads_kv > 32)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_decode_paged: heads_q (%d) must be a multiple of heads_kv (%d) with at most 32 query heads per kv head",
                heads_q, heads_kv);
  if (page_size < 16)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: page_size %d not supported (at least 16)", page_size);
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(workspace))
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: q, pages, o and workspace must be 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (page_stride[i] % 8) return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: page strides must be multiples of 8 elements");
  if ((int64_t)page_size * page_stride[2] >= (int64_t(1) << 31))
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: page_size * slot stride must stay below 2^31 elements");
  const int max_seqlen = max_blocks_per_seq * page_size;
  const size_t need = fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen, head_dim, split_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "fa_decode_paged: workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  if ((int64_t)batch * heads_q > 0x7fffffffLL / 4 || (int64_t)batch * max_blocks_per_seq > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_decode_paged: problem too large for one launch");

  fa::DecodeParams p{};
  p.q = q; p.k = k_pages; p.v = v_pages; p.seqlens = seqlens_k; p.o = o; p.lse = lse;
  const int64_t parts = ((int64_t)batch * heads_kv + fa::decode_waves()) * (heads_q / heads_kv);
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + parts * head_dim;
  for (int i = 0; i < 3; ++i) p.kv_stride[i] = page_stride[i];
  p.block_table = block_table;
  p.page_size = page_size; p.max_blocks = max_blocks_per_seq; p.num_pages = num_pages;
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
  p.max_seqlen = max_seqlen; p.head_dim = head_dim;
  p.split_tokens = split_tokens > 0 ? split_tokens : 0;
  p.n_waves = fa::decode_waves();
  p.scale_log2 = softmax_scale * kLog2e;
  p.out_fp32 = out_dtype == FA_DTYPE_FP32;
  hipError_t e = fa::launch_decode(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_decode_paged: launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t fa_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t seqlen_q) {
  if (batch <= 0 || heads_q <= 0 || seqlen_q <= 0) return 0;
  return (size_t)batch * heads_q * seqlen_q * sizeof(float);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int32_t batch, int32_t heads_q, int32_t heads_kv,
                   int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim, const int64_t q_stride[3],
                   const int64_t kv_stride[3], const int64_t dq_stride[3], const int64_t dkv_stride[3],
                   fa_dtype_t o_dtype, fa_dtype_t grad_dtype, fa_mask_t mask, float softmax_scale,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: tensor pointers must be non-null");
  if (!q_stride || !kv_stride || !dq_stride || !dkv_stride)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: stride arrays must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: sizes must be positive");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: softmax_scale must be finite and positive (got %g)",
                (double)softmax_scale);
  if (grad_dtype != FA_DTYPE_BF16 && grad_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: unknown grad_dtype %d", (int)grad_dtype);
  if (o_dtype != FA_DTYPE_BF16 && o_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: unknown o_dtype %d", (int)o_dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: unknown mask %d", (int)mask);
  for (int i = 0; i < 3; ++i)
    if (q_stride[i] < 0 || kv_stride[i] < 0 || dq_stride[i] < 0 || dkv_stride[i] < 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: strides must be non-negative");
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: head_dim %d not supported (64 or 128)", head_dim);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
  if (mask == FA_MASK_CAUSAL && seqlen_q != seqlen_k)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: causal mask needs seqlen_q == seqlen_k (got %d, %d)", seqlen_q, seqlen_k);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) || !aligned16(lse))
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: pointers must be 16-byte aligned");
  const int gvec = grad_dtype == FA_DTYPE_BF16 ? 8 : 4;
  for (int i = 0; i < 3; ++i) {
    if (q_stride[i] % 8 || kv_stride[i] % 8)
      return fail(FA_ERR_UNSUPPORTED, "fa_bwd: input strides must be multiples of 8 elements");
    if (dq_stride[i] % gvec || dkv_stride[i] % gvec)
      return fail(FA_ERR_UNSUPPORTED, "fa_bwd: gradient strides must be multiples of %d elements", gvec);
  }
  const size_t need = fa_bwd_workspace_bytes(batch, heads_q, seqlen_q);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "fa_bwd: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  // no gradient may overlap an input, another gradient, or the workspace
  const int64_t gb = grad_dtype == FA_DTYPE_BF16 ? 2 : 4;
  uintptr_t lo[10], hi[10];
  span(q, q_stride, batch, heads_q, seqlen_q, head_dim, 2, &lo[0], &hi[0]);
  span(o, q_stride, batch, heads_q, seqlen_q, head_dim, o_dtype == FA_DTYPE_FP32 ? 4 : 2, &lo[1], &hi[1]);
  span(dout, q_stride, batch, heads_q, seqlen_q, head_dim, 2, &lo[2], &hi[2]);
  span(k, kv_stride, batch, heads_kv, seqlen_k, head_dim, 2, &lo[3], &hi[3]);
  span(v, kv_stride, batch, heads_kv, seqlen_k, head_dim, 2, &lo[4], &hi[4]);
  lo[5] = reinterpret_cast<uintptr_t>(lse);
  hi[5] = lo[5] + (uintptr_t)batch * heads_q * seqlen_q * sizeof(float);
  lo[6] = reinterpret_cast<uintptr_t>(workspace);
  hi[6] = lo[6] + need;
  span(dq, dq_stride, batch, heads_q, seqlen_q, head_dim, gb, &lo[7], &hi[7]);
  span(dk, dkv_stride, batch, heads_kv, seqlen_k, head_dim, gb, &lo[8], &hi[8]);
  span(dv, dkv_stride, batch, heads_kv, seqlen_k, head_dim, gb, &lo[9], &hi[9]);
  for (int gi = 7; gi < 10; ++gi)
    for (int j = 0; j < 10; ++j)
      if (j != gi && overlap(lo[gi], hi[gi], lo[j], hi[j]))
        return fail(FA_ERR_INVALID_ARGUMENT, "fa_bwd: gradient buffers must not overlap inputs, each other or the workspace");
  if ((int64_t)batch * heads_q * ((seqlen_q + 127) / 128) > 0x7fffffffLL ||
      (int64_t)batch * heads_q * seqlen_q * (head_dim / 8) > 0x7fffffffLL * 256LL)
    return fail(FA_ERR_UNSUPPORTED, "fa_bwd: problem too large for one launch");

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dsum = static_cast<float*>(workspace);
  p.dq = dq; p.dk = dk; p.dv = dv;
  for (int i = 0; i < 3; ++i) {
    p.q_stride[i] = q_stride[i]; p.kv_stride[i] = kv_stride[i];
    p.dq_stride[i] = dq_stride[i]; p.dkv_stride[i] = dkv_stride[i];
  }
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
  p.seqlen_q = seqlen_q; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = mask == FA_MASK_CAUSAL;
  p.grad_fp32 = grad_dtype == FA_DTYPE_FP32;
  p.o_fp32 = o_dtype == FA_DTYPE_FP32;
  hipError_t e = fa::launch_bwd(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_bwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status_t fa_fp8_quantize(const void* q, const void* k, const void* v, const float* signs,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen, int32_t head_dim,
                            const int64_t q_stride[3], const int64_t kv_stride[3], void* q8, void* k8, void* v8t,
                            float* q_scale, float* k_scale, float* v_scale, void* stream) {
  if (!q || !k || !v || !q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fp8_quantize: tensor pointers must be non-null (signs may be NULL)");
  if (!q_stride || !kv_stride) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fp8_quantize: stride arrays must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fp8_quantize: sizes must be positive");
  for (int i = 0; i < 3; ++i)
    if (q_stride[i] < 0 || kv_stride[i] < 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_fp8_quantize: strides must be non-negative");
  if (head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "fa_fp8_quantize: head_dim %d not supported (128)", head_dim);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_UNSUPPORTED, "fa_fp8_quantize: heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8t))
    return fail(FA_ERR_UNSUPPORTED, "fa_fp8_quantize: tensors must be 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (q_stride[i] % 8 || kv_stride[i] % 8)
      return fail(FA_ERR_UNSUPPORTED, "fa_fp8_quantize: strides must be multiples of 8 elements");
  if (heads_q > 65535 || heads_kv > 65535 || batch > 65535)
    return fail(FA_ERR_UNSUPPORTED, "fa_fp8_quantize: problem too large for one launch");
  fa::Fp8QuantParams p{};
  p.q = q; p.k = k; p.v = v; p.signs = signs;
  p.q8 = q8; p.k8 = k8; p.v8t = v8t; p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  for (int i = 0; i < 3; ++i) { p.q_stride[i] = q_stride[i]; p.kv_stride[i] = kv_stride[i]; }
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.seqlen = seqlen;
  hipError_t e = fa::launch_fp8_quant(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fp8_quantize: launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status_t fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale, const float* k_scale,
                       const float* v_scale, void* o, float* lse, int32_t batch, int32_t heads_q, int32_t heads_kv,
                       int32_t seqlen, int32_t head_dim, fa_dtype_t out_dtype, fa_mask_t mask, float softmax_scale,
                       void* stream) {
  if (!q8 || !k8 || !v8t || !q_scale || !k_scale || !v_scale || !o)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_fp8: tensor pointers must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_fp8: sizes must be positive");
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_fp8: softmax_scale must be finite and positive (got %g)",
                (double)softmax_scale);
  if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_fp8: unknown out_dtype %d", (int)out_dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_fp8: unknown mask %d", (int)mask);
  if (head_dim != 128) return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: head_dim %d not supported (128)", head_dim);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8t) || !aligned16(o))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: tensors must be 16-byte aligned");
  if ((int64_t)batch * heads_q * ((seqlen + 127) / 128) > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_fp8: problem too large for one launch");
  fa::Fp8FwdParams p{};
  p.q8 = q8; p.k8 = k8; p.v8t = v8t; p.q_scale = q_scale; p.k_scale = k_scale; p.v_scale = v_scale;
  p.o = o; p.lse = lse;
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv; p.seqlen = seqlen;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = mask == FA_MASK_CAUSAL;
  p.out_fp32 = out_dtype == FA_DTYPE_FP32;
  hipError_t e = fa::launch_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_fp8: launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_WORKSPACE_TOO_SMALL: return "FA_ERR_WORKSPACE_TOO_SMALL";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error_message(void) { return g_last_error.c_str(); }

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int32_t batch, int32_t heads_q, int32_t heads_kv,
                   int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                   const int64_t q_stride[3], const int64_t k_stride[3],
                   const int64_t v_stride[3], const int64_t o_stride[3],
                   fa_dtype_t in_dtype, fa_dtype_t out_dtype, fa_mask_t mask,
                   float softmax_scale, void* stream) {
  if (!q || !k || !v || !o) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: q, k, v and o must be non-null");
  if (!q_stride || !k_stride || !v_stride || !o_stride)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: stride arrays must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || seqlen_q <= 0 || seqlen_k <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: sizes must be positive (batch=%d heads_q=%d heads_kv=%d seqlen_q=%d seqlen_k=%d head_dim=%d)",
                batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: softmax_scale must be finite and positive (got %g)", (double)softmax_scale);
  if (in_dtype != FA_DTYPE_BF16 && in_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: unknown in_dtype %d", (int)in_dtype);
  if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: unknown out_dtype %d", (int)out_dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: unknown mask %d", (int)mask);
  for (int i = 0; i < 3; ++i)
    if (q_stride[i] < 0 || k_stride[i] < 0 || v_stride[i] < 0 || o_stride[i] < 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: strides must be non-negative");

  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: head_dim %d not supported (64 or 128)", head_dim);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
  if (mask == FA_MASK_CAUSAL && seqlen_q != seqlen_k)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: causal mask needs seqlen_q == seqlen_k (got %d, %d)", seqlen_q, seqlen_k);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: q, k, v and o must be 16-byte aligned");
  const int in_vec = in_dtype == FA_DTYPE_BF16 ? 8 : 4;
  const int out_vec = out_dtype == FA_DTYPE_BF16 ? 8 : 4;
  for (int i = 0; i < 3; ++i) {
    if (q_stride[i] % in_vec || k_stride[i] % in_vec || v_stride[i] % in_vec)
      return fail(FA_ERR_UNSUPPORTED, "fa_fwd: q/k/v strides must be multiples of %d elements", in_vec);
    if (o_stride[i] % out_vec)
      return fail(FA_ERR_UNSUPPORTED, "fa_fwd: o strides must be multiples of %d elements", out_vec);
  }
  if (k_stride[2] > (int64_t(1) << 24) || v_stride[2] > (int64_t(1) << 24))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: k/v row strides above 2^24 elements are not supported");
  const int64_t in_b = in_dtype == FA_DTYPE_BF16 ? 2 : 4, out_b = out_dtype == FA_DTYPE_BF16 ? 2 : 4;
  uintptr_t o0, o1, a0, a1;
  span(o, o_stride, batch, heads_q, seqlen_q, head_dim, out_b, &o0, &o1);
  span(q, q_stride, batch, heads_q, seqlen_q, head_dim, in_b, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: o overlaps q");
  span(k, k_stride, batch, heads_kv, seqlen_k, head_dim, in_b, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: o overlaps k");
  span(v, v_stride, batch, heads_kv, seqlen_k, head_dim, in_b, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd: o overlaps v");
  const int64_t n_qtiles = (seqlen_q + 63) / 64;          // bound over every kernel's row tile
  if ((int64_t)batch * heads_q * n_qtiles > 0x7fffffffLL)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd: problem too large for one launch");

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  for (int i = 0; i < 3; ++i) {
    p.q_stride[i] = q_stride[i]; p.k_stride[i] = k_stride[i];
    p.v_stride[i] = v_stride[i]; p.o_stride[i] = o_stride[i];
  }
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
  p.seqlen_q = seqlen_q; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = mask == FA_MASK_CAUSAL;
  p.in_fp32 = in_dtype == FA_DTYPE_FP32;
  p.out_fp32 = out_dtype == FA_DTYPE_FP32;
  p.cu_seqlens = nullptr;
  p.total = 0;
  p.window = -1;
  hipError_t e = fa::launch_fwd(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens, int32_t batch, int32_t heads_q, int32_t heads_kv,
                          int32_t total_tokens, int32_t max_seqlen, int32_t head_dim,
                          const int64_t q_stride[2], const int64_t k_stride[2],
                          const int64_t v_stride[2], const int64_t o_stride[2],
                          fa_dtype_t out_dtype, fa_mask_t mask, int32_t window, float softmax_scale,
                          void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: q, k, v, o and cu_seqlens must be non-null");
  if (!q_stride || !k_stride || !v_stride || !o_stride)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: stride arrays must be non-null");
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || total_tokens <= 0 || max_seqlen <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT,
                "fa_fwd_varlen: sizes must be positive (batch=%d heads_q=%d heads_kv=%d total=%d max_seqlen=%d head_dim=%d)",
                batch, heads_q, heads_kv, total_tokens, max_seqlen, head_dim);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: softmax_scale must be finite and positive (got %g)",
                (double)softmax_scale);
  if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: unknown out_dtype %d", (int)out_dtype);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL)
    return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: unknown mask %d", (int)mask);
  if (window < -1) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: window must be -1 (none) or >= 0");
  for (int i = 0; i < 2; ++i)
    if (q_stride[i] < 0 || k_stride[i] < 0 || v_stride[i] < 0 || o_stride[i] < 0)
      return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: strides must be non-negative");

  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: head_dim %d not supported (64 or 128)", head_dim);
  if (heads_q % heads_kv != 0)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: heads_q (%d) must be a multiple of heads_kv (%d)", heads_q,
                heads_kv);
  if (window >= 0 && mask != FA_MASK_CAUSAL)
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: a sliding window needs the causal mask");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: q, k, v and o must be 16-byte aligned");
  for (int i = 0; i < 2; ++i)
    if (q_stride[i] % 8 || k_stride[i] % 8 || v_stride[i] % 8 || o_stride[i] % (out_dtype == FA_DTYPE_BF16 ? 8 : 4))
      return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: strides must be multiples of 16 bytes");
  if (k_stride[0] > (int64_t(1) << 24) || v_stride[0] > (int64_t(1) << 24))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: k/v token strides above 2^24 elements are not supported");
  // byte spans as [1, heads, total, d] tensors with {0, head, token} strides
  const int64_t out_b = out_dtype == FA_DTYPE_BF16 ? 2 : 4;
  const int64_t qs3[3] = {0, q_stride[1], q_stride[0]}, ks3[3] = {0, k_stride[1], k_stride[0]};
  const int64_t vs3[3] = {0, v_stride[1], v_stride[0]}, os3[3] = {0, o_stride[1], o_stride[0]};
  uintptr_t o0, o1, a0, a1;
  span(o, os3, 1, heads_q, total_tokens, head_dim, out_b, &o0, &o1);
  span(q, qs3, 1, heads_q, total_tokens, head_dim, 2, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: o overlaps q");
  span(k, ks3, 1, heads_kv, total_tokens, head_dim, 2, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: o overlaps k");
  span(v, vs3, 1, heads_kv, total_tokens, head_dim, 2, &a0, &a1);
  if (overlap(o0, o1, a0, a1)) return fail(FA_ERR_INVALID_ARGUMENT, "fa_fwd_varlen: o overlaps v");
  const int64_t n_qtiles = (max_seqlen + 63) / 64;        // bound over every kernel's row tile
  if ((int64_t)batch * heads_q * n_qtiles > 0x7fffffffLL || (int64_t)heads_q * total_tokens > (int64_t(1) << 40))
    return fail(FA_ERR_UNSUPPORTED, "fa_fwd_varlen: problem too large for one launch");

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.q_stride[0] = 0; p.q_stride[1] = q_stride[1]; p.q_stride[2] = q_stride[0];
  p.k_stride[0] = 0; p.k_stride[1] = k_stride[1]; p.k_stride[2] = k_stride[0];
  p.v_stride[0] = 0; p.v_stride[1] = v_stride[1]; p.v_stride[2] = v_stride[0];
  p.o_stride[0] = 0; p.o_stride[1] = o_stride[1]; p.o_stride[2] = o_stride[0];
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
  p.seqlen_q = max_seqlen; p.seqlen_k = max_seqlen; p.head_dim = head_dim;
  p.scale_log2 = softmax_scale * kLog2e;
  p.causal = mask == FA_MASK_CAUSAL;
  p.in_fp32 = false;
  p.out_fp32 = out_dtype == FA_DTYPE_FP32;
  p.cu_seqlens = cu_seqlens;
  p.total = total_tokens;
  p.window = window;
  hipError_t e = fa::launch_fwd(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fa_fwd_varlen: launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t fa_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                 int32_t max_seqlen_k, int32_t head_dim, int32_t split_tokens) {
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || max_seqlen_k <= 0 || head_dim <= 0) return 0;
  if (heads_q % heads_kv != 0) return 0;
  // One partial (G heads x (d + 1) floats) per piece, a piece being the part
  // of one (sequence, kv head) slab inside one wave's range. The W ranges cut
  // the stream of B*Hkv slabs at no more than W - 1 interior points, so there
  // are at most B*Hkv + W pieces whatever split_tokens is: a larger split only
  // leaves some waves without a range. The bound is the same for every split.
  (void)split_tokens;
  const int64_t parts = (int64_t)batch * heads_kv + fa::decode_waves();
  return static_cast<size_t>(parts * (heads_q / heads_kv) * (head_dim + 1) * 4);
}

}  // extern "C"

namespace {

// Argument checks shared by fa_decode and fa_decode_noalloc (everything but
// the workspace), run before anything touches the GPU.
fa_status_t decode_checks(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seqlens_k, const void* o, int32_t batch, int32_t heads_q,
                          int32_t heads_kv, int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                          fa_dtype_t out_dtype, float softmax_scale) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !o || !kv_stride)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: q, caches, seqlens_k, o and kv_stride must be non-null", fn);
  if (batch <= 0 || heads_q <= 0 || heads_kv <= 0 || max_seqlen_k <= 0 || head_dim <= 0)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: sizes must be positive", fn);
  if (!std::isfinite(softmax_scale) || softmax_scale <= 0.f)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: softmax_scale must be finite and positive (got %g)", fn,
                (double)softmax_scale);
  if (out_dtype != FA_DTYPE_BF16 && out_dtype != FA_DTYPE_FP32)
    return fail(FA_ERR_INVALID_ARGUMENT, "%s: unknown out_dtype %d", fn, (int)out_dtype);
  for (int i = 0; i < 3; ++i)
    if (kv_stride[i] < 0) return fail(FA_ERR_INVALID_ARGUMENT, "%s: strides must be non-negative", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(FA_ERR_UNSUPPORTED, "%s: head_dim %d not supported (64 or 128)", fn, head_dim);
  if (heads_q % heads_kv != 0 || heads_q / heads_kv > 32)
    return fail(FA_ERR_UNSUPPORTED,
                "%s: heads_q (%d) must be a multiple of heads_kv (%d) with at most 32 query heads per kv head", fn,
                heads_q, heads_kv);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(FA_ERR_UNSUPPORTED, "%s: q, caches and o must be 16-byte aligned", fn);
  for (int i = 0; i < 3; ++i)
    if (kv_stride[i] % 8) return fail(FA_ERR_UNSUPPORTED, "%s: kv strides must be multiples of 8 elements", fn);
  if ((int64_t)batch * heads_q > 0x7fffffffLL / 4)
    return fail(FA_ERR_UNSUPPORTED, "%s: problem too large for one launch", fn);
  return FA_OK;
}

fa_status_t decode_launch(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* seqlens_k, void* o, float* lse, int32_t batch, int32_t heads_q,
                          int32_t heads_kv, int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                          fa_dtype_t out_dtype, float softmax_scale, int32_t split_tokens, void* workspace,
                          void* stream) {
  fa::DecodeParams p{};
  p.q = q; p.k = k_cache; p.v = v_cache; p.seqlens = seqlens_k; p.o = o; p.lse = lse;
  const int64_t parts = ((int64_t)batch * heads_kv + fa::decode_waves()) * (heads_q / heads_kv);
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = p.part_o + parts * head_dim;
  for (int i = 0; i < 3; ++i) p.kv_stride[i] = kv_stride[i];
  p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
  p.max_seqlen = max_seqlen_k; p.head_dim = head_dim;
  p.split_tokens = split_tokens > 0 ? split_tokens : 0;
  p.n_waves = fa::decode_waves();
  p.scale_log2 = softmax_scale * kLog2e;
  p.out_fp32 = out_dtype == FA_DTYPE_FP32;
  hipError_t e = fa::launch_decode(p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens_k, void* o, float* lse,
                      int32_t batch, int32_t heads_q, int32_t heads_kv,
                      int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                      fa_dtype_t out_dtype, float softmax_scale, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const fa_status_t st = decode_checks("fa_decode", q, k_cache, v_cache, seqlens_k, o, batch, heads_q, heads_kv,
                                       max_seqlen_k, head_dim, kv_stride, out_dtype, softmax_scale);
  if (st != FA_OK) return st;
  if (!aligned16(workspace))
    return fail(FA_ERR_UNSUPPORTED, "fa_decode: workspace must be 16-byte aligned");
  const size_t need = fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen_k, head_dim, split_tokens);
  if (!workspace || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE_TOO_SMALL, "fa_decode: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  return decode_launch("fa_decode", q, k_cache, v_cache, seqlens_k, o, lse, batch, heads_q, heads_kv, max_seqlen_k,
                       head_dim, kv_stride, out_dtype, softmax_scale, split_tokens, workspace, stream);
}

fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* seqlens_k, void* o, float* lse,
                              int32_t batch, int32_t heads_q, int32_t heads_kv,
                              int32_t max_seqlen_k, int32_t head_dim, const int64_t kv_stride[3],
                              fa_dtype_t out_dtype, float softmax_scale, int32_t split_tokens, void* stream) {
  const fa_status_t st = decode_checks("fa_decode_noalloc", q, k_cache, v_cache, seqlens_k, o, batch, heads_q,
                                       heads_kv, max_seqlen_k, head_dim, kv_stride, out_dtype, softmax_scale);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(batch, heads_q, heads_kv, max_seqlen_k, head_dim, split_tokens);
  if (need > fa::kDecodeScratchBytes)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_decode_noalloc: these sizes need %zu bytes of partials, more than the %zu-byte static scratch "
                "(use fa_decode with a workspace)", need, fa::kDecodeScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = fa::decode_scratch(&scratch);
  if (e != hipSuccess)
    return fail(FA_ERR_HIP, "fa_decode_noalloc: static scratch lookup failed: %s", hipGetErrorString(e));
  return decode_launch("fa_decode_noalloc", q, k_cache, v_cache, seqlens_k, o, lse, batch, heads_q, heads_kv,
                       max_seqlen_k, head_dim, kv_stride, out_dtype, softmax_scale, split_tokens, scratch, stream);
}

}  // extern "C"
