// Internal interface between the C ABI (fa_api.hip) and the kernel launchers.
// Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  int batch, heads_q, heads_kv, group, seqlen_q, seqlen_k, head_dim;
  int n_qtiles;
  int n_items;       // batch * (heads_q >> hp_log2) * n_qtiles logical work items
  float scale_log2;  // softmax scale * log2(e)
  bool causal, in_fp32, out_fp32;
  // Packed batch (null: dense): sequence b owns tokens cu_seqlens[b] ..
  // cu_seqlens[b+1]-1 of q, k, v and o; strides[2] is the token stride,
  // strides[1] the head stride, strides[0] unused; seqlen_q = seqlen_k = the
  // longest sequence; LSE is [heads_q, total].
  const int32_t* cu_seqlens;
  int total;
  int window;        // sliding window (causal only): row r sees keys r-window .. r; -1 for none
  // Reciprocals of group, n_qtiles and heads_kv for the work-item decode
  // (filled in by the launchers): n / d = umulhi(n, m) >> (s - 1) for
  // 0 <= n < 2^31, with s = ceil(log2 d) and m = ceil(2^(31+s) / d); m = 0
  // stands for d = 1.
  uint32_t div_m[3];
  int div_s[3];
  bool persist;      // d = 128 kernel: a persistent grid walks the items (set by its launcher)
  // d = 128 kernel: an item is 256 >> hp_log2 query rows of 1 << hp_log2 query
  // heads that share a kv head (set by its launcher; 0 elsewhere)
  int hp_log2;
  int cu_count;      // d = 64 kernel: compute units of the device (set by its launcher)
};

// The reciprocal (m, s) of d >= 1 described at FwdParams::div_m. With
// e = m d - 2^(31+s) < d <= 2^s, n m / 2^(31+s) exceeds n / d by less than
// n 2^-(31+s) < 2^-s <= 1/d, which never reaches the next integer.
inline void fa_reciprocal(int d, uint32_t* m, int* s) {
  int k = 0;
  while ((1LL << k) < d) ++k;
  *s = k;
  *m = d == 1 ? 0u : (uint32_t)((((uint64_t)1 << (31 + k)) + (uint64_t)d - 1) / (uint64_t)d);
}

struct DecodeParams {
  const void* q;       // [B, Hq, d] bf16
  const void* k;       // cache [B, Hkv, Lmax, d] bf16
  const void* v;
  const int32_t* seqlens;
  void* o;             // [B, Hq, d]
  float* lse;          // [B, Hq] or null
  float* part_o;       // workspace [B*Hkv + n_waves][G][d]
  float* part_lse;     // workspace [B*Hkv + n_waves][G]
  int64_t kv_stride[3];     // contiguous cache: {b, h, n}; paged cache: {page, h, slot}
  const int32_t* block_table;   // paged cache only: [batch][max_blocks] page ids (null: contiguous)
  int page_size, max_blocks, num_pages;
  int batch, heads_q, heads_kv, group, max_seqlen, head_dim;
  int split_tokens;    // lower bound on the keys per wave range (0: none)
  int n_waves;         // decode grid (one-wave workgroups)
  float scale_log2;
  bool out_fp32;
};

struct BwdParams {
  const void* q;       // [B, Hq, Nq, d] bf16, strides q_stride (shared by o, dout)
  const void* k;       // [B, Hkv, Nk, d] bf16, strides kv_stride (shared by v)
  const void* v;
  const void* o;       // bf16 or float32 (o_fp32), q_stride in its own elements
  const void* dout;
  const float* lse;    // [B, Hq, Nq] natural log, from the forward pass
  float* dsum;         // workspace [B, Hq, Nq]: rowsum(dO * O)
  void* dq;            // strides dq_stride
  void* dk;            // strides dkv_stride (shared by dv)
  void* dv;
  int64_t q_stride[3], kv_stride[3], dq_stride[3], dkv_stride[3];
  int batch, heads_q, heads_kv, group, seqlen_q, seqlen_k, head_dim;
  float scale, scale_log2;
  bool causal, grad_fp32, o_fp32;
};

// FP8 path (head_dim 128): the quantiser's inputs and outputs, then the
// attention kernel's. Quantised tensors are contiguous:
//   q8 [B, Hq, N, 128] e4m3 (rotated), q_scale [B, Hq, ceil(N/128)]
//   k8 [B, Hkv, N, 128] e4m3 (rotated), k_scale [B, Hkv, ceil(N/64)]
//   v8t [B, Hkv, 128, Npad] e4m3, Npad = 64 ceil(N/64), keys permuted in
//   every 64-key tile; v_scale [B, Hkv]
struct Fp8QuantParams {
  const void* q;       // bf16 [B, Hq, N, 128], strides q_stride
  const void* k;       // bf16 [B, Hkv, N, 128], strides kv_stride (shared by v)
  const void* v;
  const float* signs;  // [128] +-1, or null (no rotation)
  void* q8;
  void* k8;
  void* v8t;
  float* q_scale;
  float* k_scale;
  float* v_scale;
  int64_t q_stride[3], kv_stride[3];
  int batch, heads_q, heads_kv, seqlen;
};

struct Fp8FwdParams {
  const void* q8;
  const void* k8;
  const void* v8t;
  const float* q_scale;
  const float* k_scale;
  const float* v_scale;
  void* o;             // [B, Hq, N, 128] contiguous, bf16 or float32
  float* lse;          // [B, Hq, N] or null
  int batch, heads_q, heads_kv, group, seqlen;
  float scale_log2;
  bool causal, out_fp32;
};

hipError_t launch_fp8_quant(const Fp8QuantParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);

// n_qtiles is filled in by the launchers (it depends on the kernel's row tile).
hipError_t launch_fwd(const FwdParams& p, hipStream_t stream);       // dispatches on in_fp32
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream);

int decode_waves();
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Size of the static decode workspace behind fa_decode_noalloc, and its
// device address on the current device (looked up on the first call there).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
