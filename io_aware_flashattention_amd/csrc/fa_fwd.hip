// Prefill attention forward for bf16 inputs on gfx950: exact softmax attention
// computed one 64-key tile at a time with a running row maximum and running
// row sum, so the N x N scores never leave the chip.
//
// The loop is the FlashAttention-2 order ("FlashAttention and GPU Data
// Movement", section 2 and the recurrence of section 3.1): a workgroup owns a
// tile of query rows, streams K/V tiles through LDS, keeps an unnormalised
// float32 accumulator in registers, divides once at the end and writes O and
// the per-row log-sum-exp once. Under the causal mask, tiles wholly in the
// future are not loaded (the skip bound) and only tiles crossing the diagonal
// are masked, elementwise, before the row statistics see them (section 2.1).
//
// Mapping onto the CDNA4 compute unit:
//   * NW waves per workgroup, wave w owns query rows q0+32w .. q0+32w+31 and
//     lane l owns row l % 32; two waves share each SIMD so one wave's softmax
//     overlaps the other's matrix work;
//   * K/V tiles move global -> LDS by direct DMA loads (no register staging),
//     STAGES tiles deep, one barrier per tile; rows past the sequence end are
//     clamped to the last row and masked, so the loads need no branches;
//   * S^T = K_tile Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, rows on N). K
//     rows are read in sigma order so the score accumulator is already the B
//     operand of O^T += V^T P^T; V stays row-major in LDS and its A operand
//     (eight consecutive keys of one d per lane) comes from transposing
//     ds_read_b64_tr_b16 reads;
//   * the softmax runs in base 2 with scale*log2(e) folded into one FMA per
//     score; a row's keys are split between lane l and lane l^32 and joined
//     with one permlane32 swap;
//   * the accumulator is rescaled only when some row's maximum grows by more
//     than 2^8 (between rescales exp2 arguments stay <= 8): O / l and
//     m + log2 l use one consistent base, so the result is unchanged. This is
//     the conditional rescaling of "FlashAttention Explained: IO-Aware
//     Attention, Tiling, Online Softmax and FP8 on Hopper" (FlashAttention-4
//     section). With a stale base the dominant weight is no longer exactly 1,
//     so two row sums are kept: O is divided by the sum of the bf16-rounded
//     weights that actually enter P V (an exactly normalised combination of V
//     rows), and the log-sum-exp uses the float32 sum of the weights.
#include "fa_device.h"
#include "fa_launch.h"

#ifndef FA_FWD_NW128
#define FA_FWD_NW128 8       // waves per workgroup at head_dim 128
#endif
#ifndef FA_FWD_STAGES128
#define FA_FWD_STAGES128 3   // K/V tiles in flight at head_dim 128
#endif

namespace fa {

namespace {

constexpr int BC = 64;       // keys per tile
constexpr float kRescaleThreshold = 8.f;

// LDS swizzles, measured against gfx950's 64 banks x 4 bytes: a ds_read_b128
// is served 16 lanes at a time and a ds_read_b64_tr_b16 32 lanes at a time;
// either is conflict-free when those lanes hit 16 distinct 16-byte slots of a
// 256-byte bank line. XOR patterns on the 16-byte chunk index of a row:
//   K (fragment rows sigma(0..15) at one chunk): D = 128 rows are 256 bytes,
//     so the chunk is XOR-ed with sigma(row) & 15 (= the lane number); D = 64
//     rows are 128 bytes (two rows per bank line), XOR with (row >> 1) & 7;
//   V (transposing reads: 4 consecutive rows x 64 bytes per 32 lanes): XOR
//     with 4 * (row % 4) for D = 128 and 4 * ((row >> 1) % 2) for D = 64.
template <int D> __device__ __forceinline__ int kswz_t(int r) {
  return D == 128 ? (sigma32(r & 31) & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int vswz_t(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// LDS pointer type for the direct global -> LDS loads (the host pass of the
// compiler needs the address space spelled out).
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace

namespace detail {

template <int D, bool CAUSAL, typename TOut, int NW, int STAGES>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(const FwdParams p) {
  constexpr int BRW = 32 * NW;               // query rows per workgroup
  constexpr int KSTEPS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  constexpr int TILE = BC * D;               // bf16 elements per K or V tile
  constexpr int ROWB = 2 * D;                // bytes per K/V row
  constexpr int NLD = TILE * 2 / 1024;       // 1-KB DMA writes per operand tile
  constexpr int LPW = NLD / NW;              // of those, per wave
  static_assert(NLD % NW == 0, "tile / wave mismatch");
  static_assert(STAGES == 3, "the software pipeline keeps tiles j, j+1 and j+2 in LDS");

  __shared__ __attribute__((aligned(16))) __bf16 smem[STAGES * 2 * TILE];   // [stage][K, V][TILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // ---- which (batch, head, query tile): XCD-aware, heavy causal tiles first,
  // the query heads of one kv head next to each other
  const int n = gridDim.x;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, slot = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  int L = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int g = L % p.group;
  L /= p.group;
  const int t = L % p.n_qtiles;
  L /= p.n_qtiles;
  const int kvh = L % p.heads_kv;
  const int b = L / p.heads_kv;
  const int hq = kvh * p.group + g;
  const int qt = CAUSAL ? p.n_qtiles - 1 - t : t;

  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(p.q) + b * p.q_stride[0] + hq * p.q_stride[1];
  const __bf16* __restrict__ kp = reinterpret_cast<const __bf16*>(p.k) + b * p.k_stride[0] + kvh * p.k_stride[1];
  const __bf16* __restrict__ vp = reinterpret_cast<const __bf16*>(p.v) + b * p.v_stride[0] + kvh * p.v_stride[1];
  const int64_t ks2 = p.k_stride[2], vs2 = p.v_stride[2];

  const int q0 = qt * BRW;
  const int wrow0 = q0 + wave * 32;
  const int row = wrow0 + r32;
  const int nq = p.seqlen_q, nk = p.seqlen_k;
  const int kv_end = CAUSAL ? min(nk, q0 + BRW) : nk;    // skip bound
  const int ntiles = (kv_end + BC - 1) / BC;

  // ---- DMA plan: this lane's 16-byte chunk of each 1-KB write
  int dma_row[LPW], dma_k[LPW], dma_v[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (wave * LPW + i) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    dma_row[i] = r;
    dma_k[i] = 8 * (pc ^ kswz_t<D>(r));
    dma_v[i] = 8 * (pc ^ vswz_t<D>(r));
  }
  auto issue = [&](int tile, int ST) {
    const int kv0 = tile * BC;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int key = min(kv0 + dma_row[i], nk - 1);
      __bf16* dk = smem + ST * 2 * TILE + (wave * LPW + i) * 512;
      __builtin_amdgcn_global_load_lds((const void*)(kp + key * ks2 + dma_k[i]), (lds_void*)dk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vp + key * vs2 + dma_v[i]), (lds_void*)(dk + TILE), 16, 0, 0);
    }
  };

  // ---- this lane's query row as B-operand fragments (rows past the end are 0)
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int kc = 0; kc < KSTEPS; ++kc)
    qf[kc] = as_bf16x8(row < nq ? load16(qp + (int64_t)row * p.q_stride[2] + 16 * kc + 8 * half)
                                : u32x4{0, 0, 0, 0});

  // ---- lane-constant LDS offsets (elements) of the fragment reads
  int koff[KSTEPS];
  {
    const int r = sigma32(r32);
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) koff[kc] = r * D + 8 * ((2 * kc + half) ^ kswz_t<D>(r));
  }
  int voff[DBLK];
  {
    const int gg = lane >> 4, i = lane & 15;
    const int r = 8 * (gg >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = 32 * db + 16 * (gg & 1) + 4 * (i & 3);
      voff[db] = r * D + 8 * ((col >> 3) ^ vswz_t<D>(r)) + (col & 7);
    }
  }

  // ---- running state of this lane's row
  const float c2 = p.scale_log2;
  float m_run = kNegInf;          // base of the exponentials (base-2 units)
  float l_run = 0.f;              // float32 sum of the weights (for the log-sum-exp)
  float l_o = 0.f;                // sum of the bf16-rounded weights (normalises O)
  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};

  // tiles this wave needs (under the causal mask, the rest lie in its future)
  const int nt_w = CAUSAL ? min(ntiles, (wrow0 + 31) / BC + 1) : ntiles;

  // S^T of one 64-key tile (K in stage ST): two 32-key blocks, chains interleaved
  auto scores = [&](int ST, f32x16& a0, f32x16& a1) {
    const __bf16* ks = smem + ST * 2 * TILE;
    a0 = f32x16{};
    a1 = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks + koff[kc]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(ks + 32 * D + koff[kc]);
      a0 = mfma32(k0, qf[kc], a0);
      a1 = mfma32(k1, qf[kc], a1);
    }
  };

  // diagonal / ragged tiles: -inf where the key is in the row's future or past the end
  auto mask = [&](int kv0, f32x16& a0, f32x16& a1) {
    if ((CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > nk)) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int k0 = kv0 + acc_key(jj, half), k1 = k0 + 32;
        a0[jj] = ((CAUSAL && k0 > row) || k0 >= nk) ? kNegInf : a0[jj];
        a1[jj] = ((CAUSAL && k1 > row) || k1 >= nk) ? kNegInf : a1[jj];
      }
    }
  };

  // row maximum of a tile; moves the base (rescaling O and the sums) only when
  // some row's maximum grows by more than the threshold (wave-uniform, rare)
  auto row_max = [&](const f32x16& a0, const f32x16& a1) {
    float mx = fmaxf(a0[0], a1[0]);          // three-input max chain (v_max3_f32)
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, fmaxf(a0[jj], a1[jj]));
    return half_swap_max(mx) * c2;
  };
  auto move_base = [&](float mt) {
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
      l_o *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
      m_run = m_new;
    }
  };

  // weights of a tile against the current base: float32 and bf16 row sums,
  // bf16 P^T chunks of 16 keys as B operands
  auto weights = [&](f32x16& a0, f32x16& a1, bf16x8 (&pb)[4]) {
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float p0 = fast_exp2(fmaf(a0[jj], c2, -m_use));
      const float p1 = fast_exp2(fmaf(a1[jj], c2, -m_use));
      a0[jj] = p0;
      a1[jj] = p1;
      rs += p0 + p1;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[0][e] = (__bf16)a0[e];
      pb[1][e] = (__bf16)a0[8 + e];
      pb[2][e] = (__bf16)a1[e];
      pb[3][e] = (__bf16)a1[8 + e];
    }
    float ro = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2 pr;
        pr[0] = pb[c][2 * e];
        pr[1] = pb[c][2 * e + 1];
        ro = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ro, false);
      }
    l_run += half_swap_sum(rs);
    l_o += half_swap_sum(ro);
  };

  // O^T += V^T P^T (V in stage ST); V^T fragments by transposing reads, 4 keys each
  auto accumulate = [&](int ST, const bf16x8 (&pb)[4]) {
    const __bf16* vs = smem + ST * 2 * TILE + TILE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const __bf16* va = vs + voff[db] + 16 * c * D;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(va));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(va + 4 * D));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma32(a, pb[c], o[db]);
      }
    }
  };

  // Software pipeline over tiles. Iteration j holds tile j (V) and tile j+1
  // (K) in LDS and loads tile j+2: the scores of tile j+1 go to the matrix
  // cores while the exponentials of tile j run on the vector ALUs, then
  // O += V_j P_j overlaps the row maximum of tile j+1.
  f32x16 c0, c1;                    // scores of tile j (the current tile)
  issue(0, 0);
  if (1 < ntiles) issue(1, 1);
  wait_vmcnt<0>();
  __syncthreads();
  if (0 < nt_w) {
    scores(0, c0, c1);
    mask(0, c0, c1);
    move_base(row_max(c0, c1));
  }

  auto step = [&](int j, int SV) {          // SV = j % 3: stage of tile j
    if (j >= ntiles) return;
    const int SK = (SV + 1) % 3;             // stage of tile j+1
    if (j > 0) {
      wait_vmcnt<0>();                       // tile j+1 landed (this wave's share)
      __syncthreads();                       // ... everyone's; tile j-1's stage is free
    }
    if (j + 2 < ntiles) issue(j + 2, (SV + 2) % 3);
    const bool cur = j < nt_w, nxt = j + 1 < nt_w;
    bf16x8 pb[4];
    f32x16 n0, n1;
    if (cur && nxt) {
      scores(SK, n0, n1);                    // matrix cores ...
      weights(c0, c1, pb);                   // ... alongside the exponentials
      mask((j + 1) * BC, n0, n1);
      accumulate(SV, pb);                    // matrix cores ...
      const float mt = row_max(n0, n1);      // ... alongside the next maximum
      move_base(mt);
      c0 = n0;
      c1 = n1;
    } else if (cur) {                        // this wave's last tile
      weights(c0, c1, pb);
      accumulate(SV, pb);
    }
  };

  for (int j = 0; j < ntiles; j += 3) {
    step(j, 0);
    step(j + 1, 1);
    step(j + 2, 2);
  }

  // ---- epilogue: O = acc / l (one division per row), LSE = ln 2 * (m + log2 l)
  if (row < nq) {
    const float inv_l = l_o > 0.f ? 1.f / l_o : 0.f;
    TOut* op = reinterpret_cast<TOut*>(p.o) + b * p.o_stride[0] + hq * p.o_stride[1] + (int64_t)row * p.o_stride[2];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * db + 8 * gq + 4 * half;
        const float v0 = o[db][4 * gq + 0] * inv_l, v1 = o[db][4 * gq + 1] * inv_l;
        const float v2 = o[db][4 * gq + 2] * inv_l, v3 = o[db][4 * gq + 3] * inv_l;
        if constexpr (sizeof(TOut) == 4) {
          *reinterpret_cast<f32x4*>(op + d) = f32x4{v0, v1, v2, v3};
        } else {
          bf16x4 h;
          h[0] = (__bf16)v0; h[1] = (__bf16)v1; h[2] = (__bf16)v2; h[3] = (__bf16)v3;
          *reinterpret_cast<bf16x4*>(op + d) = h;
        }
      }
    if (p.lse != nullptr && half == 0) {
      const float lse = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
      p.lse[((int64_t)b * p.heads_q + hq) * nq + row] = lse;
    }
  }
}

}  // namespace detail

namespace {

template <int D, bool CAUSAL, typename TOut, int NW, int STAGES>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  q.n_qtiles = (p.seqlen_q + 32 * NW - 1) / (32 * NW);
  const int64_t wgs = (int64_t)q.batch * q.heads_q * q.n_qtiles;
  hipLaunchKernelGGL((detail::fwd_bf16_kernel<D, CAUSAL, TOut, NW, STAGES>), dim3((unsigned)wgs), dim3(NW * 64), 0, stream, q);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int NW, int STAGES>
hipError_t launch_out(const FwdParams& p, hipStream_t stream) {
  return p.out_fp32 ? launch<D, CAUSAL, float, NW, STAGES>(p, stream)
                    : launch<D, CAUSAL, __bf16, NW, STAGES>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.in_fp32) return launch_fwd_f32(p, stream);
  if (p.head_dim == 64)
    return p.causal ? launch_out<64, true, 4, 3>(p, stream) : launch_out<64, false, 4, 3>(p, stream);
  return p.causal ? launch_out<128, true, FA_FWD_NW128, FA_FWD_STAGES128>(p, stream)
                  : launch_out<128, false, FA_FWD_NW128, FA_FWD_STAGES128>(p, stream);
}

}  // namespace fa
