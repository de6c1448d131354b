// Attention backward for bf16 inputs on gfx950, by recomputation: the
// probabilities are rebuilt tile by tile from Q, K and the forward pass's
// per-row log-sum-exp, never stored ("FlashAttention Explained: IO-Aware
// Attention, Tiling, Online Softmax and FP8 on Hopper", section "Backward
// Pass: Recomputation Beats Storage"; "How FlashAttention Reduces HBM Traffic
// Exactly", section "Training: recomputation replaces saved attention
// probabilities"). With P = exp(scale Q K^T - LSE) and the incoming dO:
//   D  = rowsum(dO * O)                       (pre-pass, one value per row)
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)
//   dK = scale dS^T Q,          dQ = scale dS K
// Two kernels share the work without atomics, so results are deterministic:
//   dkdv: a workgroup owns 128 keys of one kv head (32 per wave) and walks the
//         query rows of every query head of its group, accumulating dK and dV
//         in registers (the GQA sum happens in place); under the causal mask
//         it takes key tiles t and T-1-t so every workgroup has equal work;
//   dq:   a workgroup owns 128 query rows of one head (32 per wave) and walks
//         the key tiles, accumulating dQ in registers.
// Both stream their operand tiles 64 rows at a time through LDS by direct
// global -> LDS loads, issued a step or two before the matrix work reads them.
// Each of the five products runs on v_mfma_f32_32x32x16_bf16. Operand tiles
// are staged in LDS and read two ways: 16-byte row fragments in sigma order
// (so the score accumulator comes out in the B-operand layout of the next
// product, as in the forward kernel) and transposing ds_read_b64_tr_b16
// reads (the transposed operand of the accumulation products).
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int BB = 32;       // rows (or keys) per matrix-core block and per wave
constexpr int NWB = 4;       // waves per workgroup
#ifndef FA_BWD_AHEAD
#define FA_BWD_AHEAD 2       // LDS fragment reads issued this many matrix steps ahead (dK/dV)
#endif

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16-byte chunk swizzle of a tile row (any XOR pattern is correct as long as
// every access of row r uses this row's value). It depends on r % 16 only,
// so a 32-row block at row offset 32 b of a taller tile is addressed as a
// 32-row tile at t + 32 b D. These tiles are read both ways, and the pattern
// keeps both conflict-free on gfx950's 64 banks x 4 bytes:
//   row fragments (ds_read_b128, 16 lanes at a time: rows 0-15 or 16-31 of a
//     block at one chunk) need the pattern to permute the chunk slots of
//     those 16 rows (for D = 64, two rows per 256-byte bank line: of its 8
//     even and 8 odd rows);
//   transposing reads (ds_read_b64_tr_b16, 32 lanes: 4 consecutive rows x 4
//     consecutive chunks) need bit 2 and 3 of the pattern to differ across
//     the 4 rows (for D = 64, bit 2 across the two rows of each parity).
// 4 (r % 4) + (r / 4) % 4 meets both for D = 128; 4 ((r / 2) % 2) + (r / 4) % 4
// for D = 64.
template <int D> __device__ __forceinline__ int bswz(int r) {
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int D> __device__ __forceinline__ int tile_off(int r, int c) {   // element offset of (row, column)
  return r * D + 8 * ((c >> 3) ^ bswz<D>(r)) + (c & 7);
}

// A operand of X Y^T with X a 32-row LDS tile read in sigma order: lane l
// gets row sigma(l % 32), elements 16 kc + 8 (l / 32) .. +7.
template <int D> __device__ __forceinline__ bf16x8 frag_sigma(const __bf16* t, int lane, int kc) {
  const int r = sigma32(lane & 31);
  return *reinterpret_cast<const bf16x8*>(t + tile_off<D>(r, 16 * kc + 8 * (lane >> 5)));
}

// A operand of X^T Z for a 32-row LDS tile X: rows 16 c .. 16 c + 15 of X as
// the K dimension, columns 32 db .. 32 db + 31 as M (two transposing reads).
template <int D> __device__ __forceinline__ bf16x8 frag_trans(const __bf16* t, int lane, int db, int c) {
  const int gg = lane >> 4, i = lane & 15;
  const int r = 16 * c + 8 * (gg >> 1) + (i >> 2);
  const int col = 32 * db + 16 * (gg & 1) + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + tile_off<D>(r, col)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + tile_off<D>(r + 4, col)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed accumulator (32 x 32 block of [d, row]) to a row: lane l owns
// row l % 32 and writes d = 32 db + 8 gq + 4 (l / 32) .. +3.
template <int D, typename TOut>
__device__ __forceinline__ void store_rows(TOut* dst, const f32x16 (&acc)[D / 32], float mul, int lane) {
  const int half = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * half;
      const float v0 = acc[db][4 * gq] * mul, v1 = acc[db][4 * gq + 1] * mul;
      const float v2 = acc[db][4 * gq + 2] * mul, v3 = acc[db][4 * gq + 3] * mul;
      if constexpr (sizeof(TOut) == 4) {
        *reinterpret_cast<f32x4*>(dst + d) = f32x4{v0, v1, v2, v3};
      } else {
        bf16x4 h;
        h[0] = (__bf16)v0; h[1] = (__bf16)v1; h[2] = (__bf16)v2; h[3] = (__bf16)v3;
        *reinterpret_cast<bf16x4*>(dst + d) = h;
      }
    }
}


// S and dP of a 32-row block (rows of the LDS tiles qt and gt) against this
// wave's 32 keys: register j holds row acc_key(j, half), key = lane % 32.
// Each k-step's two fragments are read FA_BWD_AHEAD steps before the MFMAs
// that consume them (a scheduling barrier per step keeps that order), so
// the LDS latency hides behind matrix work even with one wave per SIMD.
template <int D>
__device__ __forceinline__ void dkdv_sdp(const __bf16* qt, const __bf16* gt, const bf16x8 (&kf)[D / 16],
                                         const bf16x8 (&vf)[D / 16], int lane, f32x16& sa, f32x16& dp) {
  constexpr int KS = D / 16, AHEAD = FA_BWD_AHEAD;
  bf16x8 fq[KS], fg[KS];
  auto read = [&](int kc) {
    if (kc < KS) {
      fq[kc] = frag_sigma<D>(qt, lane, kc);
      fg[kc] = frag_sigma<D>(gt, lane, kc);
    }
  };
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) read(x);
  sa = f32x16{};
  dp = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KS; ++kc) {
    __builtin_amdgcn_sched_barrier(0);
    read(kc + AHEAD);
    sa = mfma32(fq[kc], kf[kc], sa);
    dp = mfma32(fg[kc], vf[kc], dp);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// P = exp2(S scale log2 e - LSE log2 e) and dS = P (dP - D), as bf16 B
// operands; lse2 and dsum point at the block's 32 rows. EDGE applies the
// mask (key past the end, or in the row's future under the causal mask).
template <bool EDGE, bool CAUSAL>
__device__ __forceinline__ void dkdv_probs(const f32x16& sa, const f32x16& dp, const float* lse2, const float* dsum,
                                           int rs0, int key, int nk, float c2, int half, bf16x8 (&pb)[2],
                                           bf16x8 (&sd)[2]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int rr = acc_key(j, half);
    float x = fmaf(sa[j], c2, -lse2[rr]);
    if (EDGE) x = key < nk && (!CAUSAL || key <= rs0 + rr) ? x : kNegInf;
    const float pr = fast_exp2(x);
    pb[j >> 3][j & 7] = (__bf16)pr;
    sd[j >> 3][j & 7] = (__bf16)(pr * (dp[j] - dsum[rr]));
  }
}

// dV^T += dO^T P and dK^T += Q^T dS for a 32-row block (rows are the
// contraction), with the transposing reads FA_BWD_AHEAD steps ahead.
template <int D>
__device__ __forceinline__ void dkdv_acc(const __bf16* qt, const __bf16* gt, int lane, const bf16x8 (&pb)[2],
                                         const bf16x8 (&sd)[2], f32x16 (&dv)[D / 32], f32x16 (&dk)[D / 32]) {
  constexpr int DB = D / 32, NS = 2 * DB, AHEAD = FA_BWD_AHEAD;   // step i: row chunk i / DB, d block i % DB
  bf16x8 fg[NS], fq[NS];
  auto read = [&](int i) {
    if (i < NS) {
      fg[i] = frag_trans<D>(gt, lane, i % DB, i / DB);
      fq[i] = frag_trans<D>(qt, lane, i % DB, i / DB);
    }
  };
#pragma unroll
  for (int x = 0; x < AHEAD; ++x) read(x);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    read(i + AHEAD);
    dv[i % DB] = mfma32(fg[i], pb[i / DB], dv[i % DB]);
    dk[i % DB] = mfma32(fq[i], sd[i / DB], dk[i % DB]);
  }
  __builtin_amdgcn_sched_barrier(0);
}
}  // namespace

namespace detail {

// D[b, h, i] = sum_d dO[i, d] * O[i, d]: 16 lanes per row, 16 bytes each
// (head_dim 128; 8 lanes for 64).
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;                 // lanes per row
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int c = (int)(gid % LPR);
  float s = 0.f;
  if (row < rows) {
    const int i = (int)(row % p.seqlen_q);
    const int64_t bh = row / p.seqlen_q;
    const int h = (int)(bh % p.heads_q), b = (int)(bh / p.heads_q);
    const int64_t off = (int64_t)b * p.q_stride[0] + (int64_t)h * p.q_stride[1] + (int64_t)i * p.q_stride[2] + 8 * c;
    const bf16x8 g = as_bf16x8(load16(reinterpret_cast<const __bf16*>(p.dout) + off));
    if (p.o_fp32) {
      const float* op = reinterpret_cast<const float*>(p.o) + off;
      const f32x4 a = *reinterpret_cast<const f32x4*>(op), c4 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(a[e], (float)g[e], s);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(c4[e], (float)g[4 + e], s);
    } else {
      const bf16x8 o = as_bf16x8(load16(reinterpret_cast<const __bf16*>(p.o) + off));
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf((float)o[e], (float)g[e], s);
    }
  }
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) s += __shfl_xor(s, w, LPR);
  if (row < rows && c == 0) p.dsum[row] = s;
}

// dK and dV for 128 keys of one (batch, kv head), walking the query rows 64
// at a time (two 32-row blocks). Under the causal mask key tile t sees the
// rows from 128 t on, so a workgroup takes tiles t and T-1-t in turn and
// every workgroup does the same amount of work.
// Row order: the first pass walks down from the last row block, the second
// up from its tile's first one, and each row block takes every query head of
// the group before the next block. A row block costs every workgroup about
// the same, so all workgroups of a kv head stand on the same row block at the
// same time in either pass (workgroup u ends its first pass where its second
// starts): with the kv head's workgroups on one XCD, its L2 serves each Q/dO
// row block to all of them (counter fetch per launch at GQA-8, 8192 tokens:
// 8.8 -> 0.4 GB).
// Q and dO tiles reach LDS by direct global -> LDS loads into a three-stage
// ring, two steps ahead, with one barrier per step. Rows past the end are
// clamped to the last row: their LSE slot is set to +inf, so their weights
// are 0. LSE and D come in by 4-byte loads (waves 0 and 1), which then put
// LSE in base 2 and set the slots past the end before the barrier.
template <int D, bool CAUSAL, typename TOut>
__global__ __launch_bounds__(NWB * 64) void bwd_dkdv_kernel(const BwdParams p) {
  constexpr int KS = D / 16, DB = D / 32, RB = 2 * BB;
  constexpr int TILE = RB * D;               // elements of one Q or dO tile
  constexpr int LPW = TILE * 2 / 1024 / NWB; // 1-KB loads per wave and tensor
  constexpr int RPL = 1024 / (2 * D);        // rows per 1-KB load
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NST = 3;                     // ring depth
  static_assert(TILE * 2 % (1024 * NWB) == 0 && RB == 64, "");
  __shared__ __attribute__((aligned(16))) __bf16 ring[NST][2][TILE];    // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float lring[NST][2][RB];      // [stage][LSE log2 e, D]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int ktiles = (p.seqlen_k + NWB * BB - 1) / (NWB * BB);
  const int units = CAUSAL ? (ktiles + 1) / 2 : ktiles;
  int u = blockIdx.x % units;
  int bk = blockIdx.x / units;
  if ((p.batch * p.heads_kv) % 8 == 0) {     // one kv head's units on one XCD (workgroups go round-robin)
    const int x = blockIdx.x & 7, sl = blockIdx.x >> 3;
    u = sl % units;
    bk = x + 8 * (sl / units);
  }
  const int kvh = bk % p.heads_kv, b = bk / p.heads_kv;
  const int nq = p.seqlen_q, nk = p.seqlen_k;
  const float c2 = p.scale_log2;
  const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  const int64_t rs = p.q_stride[2];
  // this lane's row and source chunk in each of its loads: LDS chunk slot
  // lane % CPR of row r holds the row's logical chunk slot ^ bswz(r)
  int drow[LPW], dchk[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * RPL + lane / CPR;
    drow[i] = r;
    dchk[i] = 8 * ((lane % CPR) ^ bswz<D>(r));
  }

  for (int pass = 0; pass < (CAUSAL ? 2 : 1); ++pass) {
    const int kt = pass == 0 ? u : ktiles - 1 - u;
    if (pass == 1 && kt == u) break;         // odd tile count: the middle tile has no partner
    const int k0 = kt * NWB * BB;
    const int kw0 = k0 + wave * BB;          // this wave's keys kw0 .. kw0 + 31
    const int key = kw0 + (lane & 31);
    bf16x8 kf[KS], vf[KS];
#pragma unroll
    for (int kc = 0; kc < KS; ++kc) {
      kf[kc] = as_bf16x8(key < nk ? load16(kp + (int64_t)key * p.kv_stride[2] + 16 * kc + 8 * half) : u32x4{0, 0, 0, 0});
      vf[kc] = as_bf16x8(key < nk ? load16(vp + (int64_t)key * p.kv_stride[2] + 16 * kc + 8 * half) : u32x4{0, 0, 0, 0});
    }
    f32x16 dv[DB], dk[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) dv[i] = dk[i] = f32x16{};

    const int r_begin = CAUSAL ? k0 : 0;     // earlier rows see none of these keys
    const int nblk = (nq - r_begin + RB - 1) / RB;
    const int total = p.group * nblk;        // (query head, row block) steps
    auto issue = [&](int step, int st) {
      const int rb = step / p.group, g = step - rb * p.group;
      const int r0 = r_begin + (pass == 0 ? nblk - 1 - rb : rb) * RB;
      const int hq = kvh * p.group + g;
      const int64_t qo = (int64_t)b * p.q_stride[0] + (int64_t)hq * p.q_stride[1];
      const __bf16* qb = reinterpret_cast<const __bf16*>(p.q) + qo;
      const __bf16* gb = reinterpret_cast<const __bf16*>(p.dout) + qo;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int64_t e = (int64_t)min(r0 + drow[i], nq - 1) * rs + dchk[i];
        __builtin_amdgcn_global_load_lds((const void*)(qb + e), (lds_void*)&ring[st][0][(wave * LPW + i) * 512], 16, 0,
                                         0);
        __builtin_amdgcn_global_load_lds((const void*)(gb + e), (lds_void*)&ring[st][1][(wave * LPW + i) * 512], 16, 0,
                                         0);
      }
      if (wave < 2) {
        const int64_t so = ((int64_t)b * p.heads_q + hq) * nq + min(r0 + lane, nq - 1);
        __builtin_amdgcn_global_load_lds((const void*)(wave == 0 ? p.lse + so : p.dsum + so),
                                         (lds_void*)&lring[st][wave][0], 4, 0, 0);
      }
    };
    // every wave waits for its own loads of this step's tile (the next tile's may fly)
    auto wait_tile = [&](bool next_in_flight) {
      if (!next_in_flight) wait_vmcnt<0>();
      else if (wave < 2) wait_vmcnt<2 * LPW + 1>();
      else wait_vmcnt<2 * LPW>();
    };

    __syncthreads();                         // the previous pass's readers are done with the ring
    if (total > 0) issue(0, 0);
    if (total > 1) issue(1, 1);
    for (int step = 0; step < total; ++step) {
      const int st = step % NST;
      const int r0 = r_begin + (pass == 0 ? nblk - 1 - step / p.group : step / p.group) * RB;
      wait_tile(step + 1 < total);
      if (wave < 2) {                        // LSE in base 2; rows past the end: LSE +inf, D 0
        float* x = &lring[st][wave][lane];
        const float v = *x;
        *x = r0 + lane < nq ? (wave == 0 ? v * kLog2e : v) : (wave == 0 ? __builtin_huge_valf() : 0.f);
      }
      // tile `step` is published; the stage of step-1 is free for step+2
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (step + 2 < total) issue(step + 2, (step + 2) % NST);
      const __bf16* qs = ring[st][0];
      const __bf16* gs = ring[st][1];
      const float* ls = lring[st][0];
      const float* ds = lring[st][1];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int rs0 = r0 + sb * BB;
        if (CAUSAL && kw0 > rs0 + BB - 1) continue;   // every key of this wave is in these rows' future
        f32x16 sa, dp;
        bf16x8 pb[2], sd[2];
        dkdv_sdp<D>(qs + sb * BB * D, gs + sb * BB * D, kf, vf, lane, sa, dp);
        // a masked element exists only on diagonal blocks and ragged keys;
        // rows past the end carry LSE = +inf, so their weights are 0 already
        if ((CAUSAL && kw0 + BB - 1 > rs0) || kw0 + BB > nk)
          dkdv_probs<true, CAUSAL>(sa, dp, ls + sb * BB, ds + sb * BB, rs0, key, nk, c2, half, pb, sd);
        else
          dkdv_probs<false, CAUSAL>(sa, dp, ls + sb * BB, ds + sb * BB, rs0, key, nk, c2, half, pb, sd);
        dkdv_acc<D>(qs + sb * BB * D, gs + sb * BB * D, lane, pb, sd, dv, dk);
      }
    }
    if (key < nk) {
      const int64_t o = (int64_t)b * p.dkv_stride[0] + (int64_t)kvh * p.dkv_stride[1] + (int64_t)key * p.dkv_stride[2];
      store_rows<D, TOut>(reinterpret_cast<TOut*>(p.dk) + o, dk, p.scale, lane);
      store_rows<D, TOut>(reinterpret_cast<TOut*>(p.dv) + o, dv, 1.f, lane);
    }
  }
}

// dQ for 128 query rows of one (batch, query head), walking the keys 64 at a
// time (two 32-key blocks) with the next 64 in flight. Under the causal mask
// the heaviest query tiles are dispatched first.
// (Capped at two waves per SIMD: 256 registers hold it without spills, and
// the second wave's matrix work overlaps this one's softmax.)
template <int D, bool CAUSAL, typename TOut>
__global__ __launch_bounds__(NWB * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const BwdParams p) {
  constexpr int KS = D / 16, DB = D / 32, KB2 = 2 * BB;
  constexpr int TILE = KB2 * D;              // elements of one K or V tile
  constexpr int LPW = TILE * 2 / 1024 / NWB; // 1-KB loads per wave and tensor
  constexpr int RPL = 1024 / (2 * D);        // rows per 1-KB load
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static_assert(TILE * 2 % (1024 * NWB) == 0, "");
  __shared__ __attribute__((aligned(16))) __bf16 ring[2][2][TILE];     // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int qtiles = (p.seqlen_q + NWB * BB - 1) / (NWB * BB);
  const int tq = blockIdx.x / (p.batch * p.heads_q);      // heavy (late) tiles first under the mask
  int bh = blockIdx.x % (p.batch * p.heads_q);
  if ((p.batch * p.heads_kv) % 8 == 0) {     // the query heads of a kv head on one XCD, whose L2 holds its K/V
    const int x = bh & 7, sl = bh >> 3;
    bh = (x + 8 * (sl / p.group)) * p.group + sl % p.group;
  }
  const int qt = CAUSAL ? qtiles - 1 - tq : tq;
  const int hq = bh % p.heads_q, b = bh / p.heads_q;
  const int kvh = hq / p.group;
  const int nq = p.seqlen_q, nk = p.seqlen_k;
  const int q0 = qt * NWB * BB;
  const int rw0 = q0 + wave * BB;
  const int row = rw0 + (lane & 31);

  const int64_t qo = (int64_t)b * p.q_stride[0] + (int64_t)hq * p.q_stride[1];
  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int kc = 0; kc < KS; ++kc) {
    const int64_t e = (int64_t)row * p.q_stride[2] + 16 * kc + 8 * half;
    qf[kc] = as_bf16x8(row < nq ? load16(reinterpret_cast<const __bf16*>(p.q) + qo + e) : u32x4{0, 0, 0, 0});
    gf[kc] = as_bf16x8(row < nq ? load16(reinterpret_cast<const __bf16*>(p.dout) + qo + e) : u32x4{0, 0, 0, 0});
  }
  const int64_t so = ((int64_t)b * p.heads_q + hq) * nq;
  const float lse2 = row < nq ? p.lse[so + row] * kLog2e : __builtin_huge_valf();
  const float dsum = row < nq ? p.dsum[so + row] : 0.f;

  const __bf16* kp = reinterpret_cast<const __bf16*>(p.k) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  const __bf16* vp = reinterpret_cast<const __bf16*>(p.v) + b * p.kv_stride[0] + kvh * p.kv_stride[1];
  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  const float c2 = p.scale_log2;
  const int k_end = CAUSAL ? min(nk, q0 + NWB * BB) : nk;
  // K and V tiles by direct global -> LDS loads into a two-stage ring: tile
  // t+1 is issued right after the barrier that opens tile t. Keys past the
  // end are clamped to the last key; the mask removes them.
  int drow[LPW], dchk[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int r = (wave * LPW + i) * RPL + lane / CPR;
    drow[i] = r;
    dchk[i] = 8 * ((lane % CPR) ^ bswz<D>(r));
  }
  auto issue = [&](int kv0, int st) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int64_t e = (int64_t)min(kv0 + drow[i], nk - 1) * p.kv_stride[2] + dchk[i];
      __builtin_amdgcn_global_load_lds((const void*)(kp + e), (lds_void*)&ring[st][0][(wave * LPW + i) * 512], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vp + e), (lds_void*)&ring[st][1][(wave * LPW + i) * 512], 16, 0, 0);
    }
  };
  const int nt = (k_end + KB2 - 1) / KB2;
  if (nt > 0) issue(0, 0);
  for (int t = 0; t < nt; ++t) {
    const int kv0 = t * KB2, st = t & 1;
    wait_vmcnt<0>();                         // this wave's loads of tile t
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // tile t published; tile t-1's stage free
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 < nt) issue(kv0 + KB2, st ^ 1);   // in flight during this tile's matrix work
    const __bf16* ks = ring[st][0];
    const __bf16* vs = ring[st][1];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int kb0 = kv0 + sb * BB;
      if (CAUSAL && kb0 > rw0 + BB - 1) continue;   // these keys are in the future of every row of the wave
      const __bf16* kt = ks + sb * BB * D;
      const __bf16* vt = vs + sb * BB * D;
      // S^T and dP^T for (keys, rows): register j holds key acc_key(j, half), row = lane % 32
      f32x16 sa = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kc = 0; kc < KS; ++kc) {
        sa = mfma32(frag_sigma<D>(kt, lane, kc), qf[kc], sa);
        dp = mfma32(frag_sigma<D>(vt, lane, kc), gf[kc], dp);
      }
      bf16x8 sbf[2];
      // key kb0 + acc_key(j, half) is visible when acc_key(j, 0) <= lim (a
      // row past the end has LSE = +inf, so its weights are 0 already)
      const int lim = (CAUSAL ? min(row, nk - 1) : nk - 1) - kb0 - 8 * half;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float x = acc_key(j, 0) <= lim ? fmaf(sa[j], c2, -lse2) : kNegInf;
        sbf[j >> 3][j & 7] = (__bf16)(fast_exp2(x) * (dp[j] - dsum));
      }
      // dQ^T += K^T dS^T (keys are the contraction)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < DB; ++db) dq[db] = mfma32(frag_trans<D>(kt, lane, db, c), sbf[c], dq[db]);
    }
  }
  if (row < nq) {
    const int64_t o = (int64_t)b * p.dq_stride[0] + (int64_t)hq * p.dq_stride[1] + (int64_t)row * p.dq_stride[2];
    store_rows<D, TOut>(reinterpret_cast<TOut*>(p.dq) + o, dq, p.scale, lane);
  }
}

}  // namespace detail

namespace {

template <int D, bool CAUSAL, typename TOut>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
  const int64_t pre_threads = rows * (D / 8);
  hipLaunchKernelGGL((detail::bwd_pre_kernel<D>), dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0, stream,
                     p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ktiles = (p.seqlen_k + NWB * BB - 1) / (NWB * BB);
  const int64_t kwg = (int64_t)p.batch * p.heads_kv * (CAUSAL ? (ktiles + 1) / 2 : ktiles);
  hipLaunchKernelGGL((detail::bwd_dkdv_kernel<D, CAUSAL, TOut>), dim3((unsigned)kwg), dim3(NWB * 64), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t qwg = (int64_t)p.batch * p.heads_q * ((p.seqlen_q + NWB * BB - 1) / (NWB * BB));
  hipLaunchKernelGGL((detail::bwd_dq_kernel<D, CAUSAL, TOut>), dim3((unsigned)qwg), dim3(NWB * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t stream) {
  return p.grad_fp32 ? launch_bwd_t<D, CAUSAL, float>(p, stream) : launch_bwd_t<D, CAUSAL, __bf16>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.head_dim == 64) return p.causal ? launch_bwd_d<64, true>(p, stream) : launch_bwd_d<64, false>(p, stream);
  return p.causal ? launch_bwd_d<128, true>(p, stream) : launch_bwd_d<128, false>(p, stream);
}

}  // namespace fa
