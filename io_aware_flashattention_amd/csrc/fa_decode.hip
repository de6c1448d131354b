// Split-KV single-token decode for gfx950.
//
// With one query token per sequence the query-tile axis collapses to a single
// tile, so the key axis is the only long one: it is cut into splits of
// `split_tokens` keys, every split computes a partial output and its
// log-sum-exp, and a small second kernel merges the partials with the same
// rescaling identity the tile loop uses ("FlashAttention Explained: IO-Aware
// Attention, Tiling, Online Softmax and FP8 on Hopper", section "Decoding,
// Paged and Split-KV Variants"; "FlashAttention and GPU Data Movement",
// section 6.1).
//
// Work item = (sequence b, kv head, split s), one wave each; a workgroup is
// one wave by default, so a workgroup whose split lies past a short
// sequence's end exits at once and holds no LDS. All G query heads of the kv head are processed together, so each
// cached K/V byte is read from memory exactly once. Per 32-key block the wave
//   * loads 8 KB of K and 8 KB of V with fully coalesced 16-byte loads (the
//     next block's loads are issued before the current block is computed),
//   * re-lays them through a wave-private LDS region (K as [key][d], V
//     transposed as [d][key], XOR-swizzled chunks),
//   * computes S^T = K q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with
//     the G heads on the N axis (the kernel is bound by memory, not by the
//     matrix cores, so the padding of N to 32 costs nothing that matters),
//   * updates the running max / sum of each head (one lane per head).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

#ifndef FA_DEC_WAVES
#define FA_DEC_WAVES 1       // independent work items (waves) per workgroup
#endif
#ifndef FA_DEC_SPLIT
#define FA_DEC_SPLIT 1024    // default keys per split
#endif

constexpr int D = 128;
constexpr int KB = 32;                 // keys per block
constexpr int WAVES = FA_DEC_WAVES;
constexpr int NT = 64 * WAVES;
constexpr int DEFAULT_SPLIT = FA_DEC_SPLIT;

// Vt rows are 32 keys (64 bytes, four 16-byte chunks); the XOR keeps both the
// fragment reads (8 consecutive d rows) and the transposing writes spread.
__device__ __forceinline__ int vswz32(int d) { return ((d >> 1) & 3) ^ ((d >> 3) & 3); }

template <typename TOut>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(const DecodeParams p) {
  constexpr int DCH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 smem[WAVES][2 * KB * D];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  const int64_t item = (int64_t)blockIdx.x * WAVES + wave;
  const int s = (int)(item % p.max_splits);
  const int64_t bh = item / p.max_splits;
  if (bh >= (int64_t)p.batch * p.heads_kv) return;
  const int kvh = (int)(bh % p.heads_kv);
  const int b = (int)(bh / p.heads_kv);
  const int len = min(max(p.seqlens[b], 0), p.max_seqlen);
  const int k_begin = s * p.split_tokens;
  if (k_begin >= len) return;                     // this split holds no key
  const int k_end = min(len, k_begin + p.split_tokens);

  const __bf16* __restrict__ kp = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  const __bf16* __restrict__ vp = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  const int G = p.group;
  const int head = kvh * G + r32;                 // this lane's query head (valid if r32 < G)

  // query of this lane's head as B-operand fragments (heads past G are zero)
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + ((int64_t)b * p.heads_q + head) * D;
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc)
      qf[kc] = as_bf16x8(r32 < G ? load16(qp + 16 * kc + 8 * half) : u32x4{0, 0, 0, 0});
  }

  __bf16* ks = smem[wave];
  __bf16* vs = ks + KB * D;

  // lane's share of a 32-key block: keys 8*kg + i (i = 0..7) of d-chunk dc
  const int dc = lane % DCH, kg = lane / DCH;
  u32x4 kreg[8], vreg[8];
  auto load_block = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = k0 + 8 * kg + i;
      const bool ok = key < k_end;
      kreg[i] = ok ? load16(kp + (int64_t)key * p.kv_stride[2] + 8 * dc) : u32x4{0, 0, 0, 0};
      vreg[i] = ok ? load16(vp + (int64_t)key * p.kv_stride[2] + 8 * dc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 8 * kg + i;
      *reinterpret_cast<u32x4*>(ks + key * D + 8 * (dc ^ kswz(key))) = kreg[i];
    }
    // element e of keys 8kg..8kg+7 -> Vt[8*dc + e][8kg .. 8kg+7]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      uint32_t w[4];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const uint32_t lo = (vreg[2 * i2][e >> 1] >> sh) & 0xffffu;
        const uint32_t hi = (vreg[2 * i2 + 1][e >> 1] >> sh) & 0xffffu;
        w[i2] = lo | (hi << 16);
      }
      const int d = 8 * dc + e;
      *reinterpret_cast<u32x4*>(vs + d * KB + 8 * (kg ^ vswz32(d))) = u32x4{w[0], w[1], w[2], w[3]};
    }
  };

  const float c2 = p.scale_log2;
  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};

  load_block(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += KB) {
    store_block();
    if (k0 + KB < k_end) load_block(k0 + KB);      // in flight while this block computes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    f32x16 sc = f32x16{};
    {
      const int key = sigma32(r32);
#pragma unroll
      for (int kc = 0; kc < KSTEPS; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + key * D + 8 * ((2 * kc + half) ^ kswz(key)));
        sc = mfma32(a, qf[kc], sc);
      }
    }
    if (k0 + KB > k_end) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) sc[jj] = (k0 + acc_key(jj, half) >= k_end) ? kNegInf : sc[jj];
    }
    float mx = sc[0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, sc[jj]);
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float pv = fast_exp2(fmaf(sc[jj], c2, -m_use));
      sc[jj] = pv;
      rs += pv;
    }
    rs = half_swap_sum(rs);
    l_run = fmaf(l_run, alpha, rs);
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = sc[8 * c + e];
      pb[c] = to_bf16x8(f);
    }
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int d = 32 * db + r32;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + d * KB + 8 * ((2 * c + half) ^ vswz32(d)));
        o[db] = mfma32(a, pb[c], o[db]);
      }
    }
    // the next store_block overwrites this wave's LDS: keep the reads first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // partial of this split: normalised output and its log-sum-exp
  if (r32 < G) {
    const float inv_l = 1.f / l_run;                // l_run >= 1: the split holds a key
    float* po = p.part_o + (((int64_t)b * p.heads_q + head) * p.max_splits + s) * D;
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * half;
        *reinterpret_cast<f32x4*>(po + d) = f32x4{o[db][4 * gq] * inv_l, o[db][4 * gq + 1] * inv_l,
                                                  o[db][4 * gq + 2] * inv_l, o[db][4 * gq + 3] * inv_l};
      }
    if (half == 0)
      p.part_lse[((int64_t)b * p.heads_q + head) * p.max_splits + s] = (m_run + __log2f(l_run)) * kLn2;
  }
}

// One wave per (b, query head): LSE = log sum_s exp(lse_s), O = sum_s exp(lse_s - LSE) o_s.
template <typename TOut>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)p.batch * p.heads_q) return;
  const int b = (int)(row / p.heads_q);
  const int len = min(max(p.seqlens[b], 0), p.max_seqlen);
  const int ns = (len + p.split_tokens - 1) / p.split_tokens;
  const float* pl = p.part_lse + row * p.max_splits;
  const float* po = p.part_o + row * p.max_splits * D;
  float mx = kNegInf;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, pl[s]);
  float den = 0.f, n0 = 0.f, n1 = 0.f;
  if (ns > 0) {
    for (int s = 0; s < ns; ++s) {
      const float w = __expf(pl[s] - mx);
      const float2 v = *reinterpret_cast<const float2*>(po + (int64_t)s * D + 2 * lane);
      den += w;
      n0 = fmaf(w, v.x, n0);
      n1 = fmaf(w, v.y, n1);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  TOut* op = reinterpret_cast<TOut*>(p.o) + row * D + 2 * lane;
  op[0] = (TOut)(n0 * inv);
  op[1] = (TOut)(n1 * inv);
  if (p.lse != nullptr && lane == 0) p.lse[row] = den > 0.f ? mx + __logf(den) : kNegInf;
}

template <typename TOut>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t items = (int64_t)p.batch * p.heads_kv * p.max_splits;
  const int64_t wgs = (items + WAVES - 1) / WAVES;
  hipLaunchKernelGGL((decode_split_kernel<TOut>), dim3((unsigned)wgs), dim3(NT), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.batch * p.heads_q;
  hipLaunchKernelGGL((decode_merge_kernel<TOut>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int decode_default_split() { return DEFAULT_SPLIT; }

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  return p.out_fp32 ? launch_t<float>(p, stream) : launch_t<__bf16>(p, stream);
}

}  // namespace fa
