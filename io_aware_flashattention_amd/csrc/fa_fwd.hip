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
#include <algorithm>
#include <atomic>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int BC = 64;       // keys per tile
constexpr int kPpStages = 3; // K/V ring depth of the ping-pong kernel
constexpr int kAhead = 4;    // its fragment-read steps issued ahead of their MFMA
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

template <int N> struct int_c { static constexpr int value = N; };

// LDS pointer type for the direct global -> LDS loads (the host pass of the
// compiler needs the address space spelled out).
typedef __attribute__((address_space(3))) void lds_void;

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Offsets (elements) of one (sequence, query head) in q, k, v, o and the LSE,
// and its lengths. A packed batch reads its offsets at wave-uniform
// addresses (scalar loads); they are clamped into [0, total] so a bad offset
// array cannot move an access outside the packed buffers.
typedef __attribute__((address_space(4))) const int32_t const_i32;

struct SeqView {
  int64_t q, k, v, o, lse;
  int nq, nk;
};

__device__ __forceinline__ SeqView seq_view(const FwdParams& p, int b, int hq, int kvh) {
  SeqView s;
  int64_t tq = 0, tk = 0, tv = 0, to = 0;
  if (p.cu_seqlens != nullptr) {
    const const_i32* cu = (const const_i32*)p.cu_seqlens;
    const int s0 = min(max(cu[b], 0), p.total);
    const int s1 = min(max(cu[b + 1], s0), p.total);
    s.nq = s.nk = s1 - s0;
    tq = (int64_t)s0 * p.q_stride[2];
    tk = (int64_t)s0 * p.k_stride[2];
    tv = (int64_t)s0 * p.v_stride[2];
    to = (int64_t)s0 * p.o_stride[2];
    s.lse = (int64_t)hq * p.total + s0;
  } else {
    s.nq = p.seqlen_q;
    s.nk = p.seqlen_k;
    tq = (int64_t)b * p.q_stride[0];
    tk = (int64_t)b * p.k_stride[0];
    tv = (int64_t)b * p.v_stride[0];
    to = (int64_t)b * p.o_stride[0];
    s.lse = ((int64_t)b * p.heads_q + hq) * p.seqlen_q;
  }
  s.q = tq + (int64_t)hq * p.q_stride[1];
  s.k = tk + (int64_t)kvh * p.k_stride[1];
  s.v = tv + (int64_t)kvh * p.v_stride[1];
  s.o = to + (int64_t)hq * p.o_stride[1];
  return s;
}

// Logical work item (batch, kv head, query tile, query head of the group, or
// group of 2^hp_log2 of them; head fastest) of hardware workgroup wg, or -1
// for grid padding. Workgroups
// are dealt to the 8 XCDs round-robin (wg % 8), each XCD with its own L2.
//   Dense batch: every (batch, kv head) row of query tiles costs the same, so
//   each XCD takes a contiguous range of the logical order; its resident
//   workgroups then share one kv head's K/V in its L2.
//   Packed batch: rows cost what their sequence's length makes them cost, and
//   contiguous ranges would leave some XCDs with long sequences and others
//   idle. With a multiple of 8 kv heads, XCD x takes kv heads x, x + 8, ...
//   of every sequence: every kv head carries the same work, so the XCDs stay
//   balanced, and each L2 holds only its own kv heads' K/V. An XCD's
//   workgroups take its (sequence, kv head) rows one after another, each row
//   heaviest query tile first, so the workgroups in flight share that row's
//   K/V (ordering the XCD's items by cost across sequences instead was 37%
//   slower on 16 packed sequences: their K/V no longer fit the L2 together).
//   Otherwise chunks of G >> hp_log2 workgroups (the query heads that share a
//   kv head and a query tile, kept on one XCD) are dealt to the XCDs in a
//   snake order: 0..7, 7..0, 0..7, ... Along one row, XCD x then gets tiles
//   x, 15-x, 16+x, 31-x, ..., whose causal costs pair up heavy with light,
//   and the XCDs stay balanced whatever the length mix. The grid is padded to
//   whole rounds.
__device__ __forceinline__ int work_item(int wg, int n, const FwdParams& p) {
  if (p.cu_seqlens != nullptr && p.heads_kv % 8 == 0) {
    const int G = p.group >> p.hp_log2, nkh = p.heads_kv >> 3;
    const int x = wg & 7;
    int k = wg >> 3;                         // k-th workgroup of XCD x
    const int g = k % G;
    k /= G;
    const int t = k % p.n_qtiles;
    k /= p.n_qtiles;
    const int kh = k % nkh, b = k / nkh;
    return ((b * p.heads_kv + x + 8 * kh) * p.n_qtiles + t) * G + g;
  }
  if (p.cu_seqlens != nullptr) {
    const int G = p.group >> p.hp_log2;
    const int x = wg & 7, k = wg >> 3;
    const int r = k / G, g = k - r * G;
    const int j = (r & 1) ? 7 - x : x;
    const int L = (8 * r + j) * G + g;
    return L < p.n_items ? L : -1;
  }
  const int xcd = wg & 7, slot = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  return (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Grid for the logical work items of a launch.
inline int64_t grid_for(const FwdParams& p) {
  if (p.cu_seqlens == nullptr || p.heads_kv % 8 == 0) return p.n_items;
  const int G = p.group >> p.hp_log2;
  const int64_t chunks = p.n_items / G;
  return (chunks + 7) / 8 * 8 * G;
}

}  // namespace

namespace detail {

// (head_dim 64 under the causal mask: held to 168 registers, three waves per
// SIMD and three workgroups per CU, which the short causal launches of GPT-2's
// shape need more than registers: 33.8 -> 31.9 us there)
template <int D, bool CAUSAL, typename TOut, int NW, int R, int STAGES>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D == 64 && CAUSAL ? 3 : (R == 1 ? 2 : 1),
                                                                          D == 64 && CAUSAL ? 3 : (R == 1 ? 2 : 1))))
void fwd_bf16_kernel(const FwdParams p) {
  constexpr int BRW = 32 * R * NW;           // query rows per workgroup (R 32-row blocks per wave)
  constexpr int KSTEPS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  constexpr int TILE = BC * D;               // bf16 elements per K or V tile
  constexpr int ROWB = 2 * D;                // bytes per K/V row
  constexpr int NLD = TILE * 2 / 1024;       // 1-KB DMA writes per operand tile
  constexpr int LPW = NLD / NW;              // of those, per wave
  static_assert(NLD % NW == 0, "tile / wave mismatch");
  static_assert(STAGES == 3 || STAGES == 4, "the pipeline keeps tiles j and j+1 resident and loads ahead");

  __shared__ __attribute__((aligned(16))) __bf16 smem[STAGES * 2 * TILE];   // [stage][K, V][TILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // ---- which (batch, head, query tile). Dense causal: in dispatch order,
  // every head's heaviest query tile first, then every head's next one, so
  // the longest workgroups start first and the short ones fill in behind
  // them (these launches are small: a head-major order left the heavy tiles
  // of the last heads to start late, 45 against 34 us on GPT-2's shape).
  // Otherwise XCD-aware, with the query heads of one kv head side by side.
  int L = work_item(blockIdx.x, gridDim.x, p);
  if (L < 0) return;                         // padding of the last XCD round (whole workgroup)
  int g, t, kvh, b;
  if (CAUSAL && p.cu_seqlens == nullptr) {
    // Block b shares a compute unit with b + C, b + 2C, ... (C = the CU
    // count) while they are all resident, so the heavy-first ranks snake
    // across those slots: the CU that takes a heavy tile first takes a light
    // one next, and every CU's blocks add up to about the same work.
    const int C = p.cu_count, k = blockIdx.x / C, j = blockIdx.x - k * C;
    const int cnt = min(C, (int)gridDim.x - k * C);
    L = k * C + ((k & 1) ? cnt - 1 - j : j);
    const int nh = p.batch * p.heads_q;
    t = L / nh;
    L -= t * nh;
    g = L % p.group;
    L /= p.group;
    kvh = L % p.heads_kv;
    b = L / p.heads_kv;
  } else {
    g = L % p.group;
    L /= p.group;
    t = L % p.n_qtiles;
    L /= p.n_qtiles;
    kvh = L % p.heads_kv;
    b = L / p.heads_kv;
  }
  const int hq = kvh * p.group + g;
  const int qt = CAUSAL ? p.n_qtiles - 1 - t : t;

  const SeqView sv = seq_view(p, b, hq, kvh);
  const int q0 = qt * BRW;
  const int nq = sv.nq, nk = sv.nk;
  if (q0 >= nq) return;                      // a packed sequence shorter than the longest (whole workgroup)
  const __bf16* __restrict__ qp = reinterpret_cast<const __bf16*>(p.q) + sv.q;
  const __bf16* __restrict__ kp = reinterpret_cast<const __bf16*>(p.k) + sv.k;
  const __bf16* __restrict__ vp = reinterpret_cast<const __bf16*>(p.v) + sv.v;
  const int64_t ks2 = p.k_stride[2], vs2 = p.v_stride[2];

  const int wrow0 = q0 + wave * 32 * R;      // first row of this wave; block rb starts at wrow0 + 32 rb
  const int W = CAUSAL ? p.window : -1;      // sliding window (row r sees keys r-W .. r)
  const int kv_end = CAUSAL ? min(nk, q0 + BRW) : nk;    // skip bound
  // tiles wholly behind every row's window are skipped too; tile indices
  // below are counted from the workgroup's first needed tile jbase
  const int jbase = W >= 0 ? max(0, q0 - W) / BC : 0;
  const int ntiles = (kv_end + BC - 1) / BC - jbase;

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
    const int kv0 = (jbase + tile) * BC;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int key = min(kv0 + dma_row[i], nk - 1);
      __bf16* dk = smem + ST * 2 * TILE + (wave * LPW + i) * 512;
      __builtin_amdgcn_global_load_lds((const void*)(kp + key * ks2 + dma_k[i]), (lds_void*)dk, 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vp + key * vs2 + dma_v[i]), (lds_void*)(dk + TILE), 16, 0, 0);
    }
  };

  // ---- this lane's query rows as B-operand fragments (rows past the end are 0)
  bf16x8 qf[R][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    const int row = wrow0 + 32 * rb + r32;
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc)
      qf[rb][kc] = as_bf16x8(row < nq ? load16(qp + (int64_t)row * p.q_stride[2] + 16 * kc + 8 * half)
                                      : u32x4{0, 0, 0, 0});
  }

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

  // ---- running state of this lane's R rows
  const float c2 = p.scale_log2;
  float m_run[R], l_run[R];   // base (base-2 units), float32 sum (LSE)
  f32x4 lsum[R];               // bf16 sum (normalises O), every register the row's sum
  // The bf16 sum runs on the matrix core: a P^T chunk read as the B operand
  // of v_mfma_f32_16x16x32_bf16 holds, in column n, keys 0-7 and 8-15 of rows
  // n and n+16, and this A operand is 1 where the key group belongs to the
  // lane's own row (v_dot2c would occupy the matrix pipe longer for the same
  // sum: 26.5 against 27.2 us on GPT-2's causal shape)
  bf16x8 lsel;
  {
    const __bf16 one = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? (__bf16)1.f : (__bf16)0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) lsel[e] = one;
  }
  f32x16 o[R][DBLK];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
    lsum[rb] = f32x4{};
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[rb][i] = f32x16{};
  }

  // tiles this wave needs: [lo_w, nt_w) (under the causal mask later tiles
  // lie in its future, under a window earlier ones lie behind it)
  const int nt_w = CAUSAL ? min(ntiles, (wrow0 + 32 * R - 1) / BC + 1 - jbase) : ntiles;
  const int lo_w = W >= 0 ? max(0, wrow0 - W) / BC - jbase : 0;

  // S^T of one 64-key tile (K in stage ST) for the R row blocks: each K
  // fragment read once, used R times
  auto scores = [&](int ST, f32x16 (&a)[R][2]) {
    const __bf16* ks = smem + ST * 2 * TILE;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) a[rb][0] = a[rb][1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks + koff[kc]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(ks + 32 * D + koff[kc]);
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        a[rb][0] = mfma32(k0, qf[rb][kc], a[rb][0]);
        a[rb][1] = mfma32(k1, qf[rb][kc], a[rb][1]);
      }
    }
  };

  // diagonal / ragged / window-edge tiles: -inf where the key is in the row's
  // future, past the end, or more than W behind the row
  auto mask = [&](int kv0, f32x16 (&a)[R][2]) {
    const bool win = W >= 0 && kv0 < wrow0 + 32 * R - 1 - W;
    if ((CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > nk) || win) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        const int row = wrow0 + 32 * rb + r32;
        const int kmin = win ? row - W : -1;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int k0 = kv0 + acc_key(jj, half), k1 = k0 + 32;
          a[rb][0][jj] = ((CAUSAL && k0 > row) || k0 >= nk || k0 < kmin) ? kNegInf : a[rb][0][jj];
          a[rb][1][jj] = ((CAUSAL && k1 > row) || k1 >= nk || k1 < kmin) ? kNegInf : a[rb][1][jj];
        }
      }
    }
  };

  // row maxima of a tile; the base moves (rescaling O and the sums) only when
  // some row's maximum grows by more than the threshold (wave-uniform, rare)
  auto move_base = [&](const f32x16 (&a)[R][2]) {
    float mt[R];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      float mx = fmaxf(a[rb][0][0], a[rb][1][0]);        // three-input max chain (v_max3_f32)
#pragma unroll
      for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, fmaxf(a[rb][0][jj], a[rb][1][jj]));
      mt[rb] = half_swap_max(mx) * c2;
      grow = grow || (mt[rb] > m_run[rb] + kRescaleThreshold);
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        const float m_new = fmaxf(m_run[rb], mt[rb]);
        const float alpha = fast_exp2(m_run[rb] - (m_new == kNegInf ? 0.f : m_new));
        l_run[rb] *= alpha;
        lsum[rb] *= alpha;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) o[rb][i] *= alpha;
        m_run[rb] = m_new;
      }
    }
  };

  // weights of a tile against the current base: float32 and bf16 row sums,
  // bf16 P^T chunks of 16 keys as B operands
  auto weights = [&](f32x16 (&a)[R][2], bf16x8 (&pb)[R][4]) {
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const float m_use = m_run[rb] == kNegInf ? 0.f : m_run[rb];
      float rs = 0.f;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const float p0 = fast_exp2(fmaf(a[rb][0][jj], c2, -m_use));
        const float p1 = fast_exp2(fmaf(a[rb][1][jj], c2, -m_use));
        a[rb][0][jj] = p0;
        a[rb][1][jj] = p1;
        rs += p0 + p1;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[rb][0][e] = (__bf16)a[rb][0][e];
        pb[rb][1][e] = (__bf16)a[rb][0][8 + e];
        pb[rb][2][e] = (__bf16)a[rb][1][e];
        pb[rb][3][e] = (__bf16)a[rb][1][8 + e];
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) lsum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pb[rb][c], lsum[rb], 0, 0, 0);
      l_run[rb] += half_swap_sum(rs);
    }
  };

  // O^T += V^T P^T (V in stage ST); V^T fragments by transposing reads, 4 keys
  // each, read once and used R times
  auto accumulate = [&](int ST, const bf16x8 (&pb)[R][4]) {
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
#pragma unroll
        for (int rb = 0; rb < R; ++rb) o[rb][db] = mfma32(a, pb[rb][c], o[rb][db]);
      }
    }
  };

  // Software pipeline over tiles. Iteration j holds tile j (V) and tile j+1
  // (K) in LDS while later tiles load: the scores of tile j+1 go to the
  // matrix cores while the exponentials of tile j run on the vector ALUs,
  // then O += V_j P_j overlaps the row maxima of tile j+1.
  f32x16 cur[R][2];                 // scores of tile j (the current tile)
  issue(0, 0);
  if (1 < ntiles) issue(1, 1);
  if (STAGES > 3 && 2 < ntiles) issue(2, 2);
  if (STAGES > 3 && 2 < ntiles) wait_vmcnt<2 * LPW>();   // tiles 0 and 1 landed, 2 may fly
  else wait_vmcnt<0>();
  __syncthreads();
  if (lo_w == 0 && 0 < nt_w) {
    scores(0, cur);
    mask(jbase * BC, cur);
    move_base(cur);
  }

  auto step = [&](int j, int SV) {          // SV = j % STAGES: stage of tile j
    if (j >= ntiles) return;
    const int SK = (SV + 1) % STAGES;        // stage of tile j+1
    if (j > 0) {                             // tile j+1 landed (later tiles may fly)
      if (STAGES > 3 && j + 2 < ntiles) wait_vmcnt<2 * LPW>();
      else wait_vmcnt<0>();
      __syncthreads();                       // ... for every wave; tile j-1's stage is free
    }
    if (j + STAGES - 1 < ntiles) issue(j + STAGES - 1, (SV + STAGES - 1) % STAGES);
    const bool act = j >= lo_w && j < nt_w, nxt = j + 1 >= lo_w && j + 1 < nt_w;
    bf16x8 pb[R][4];
    f32x16 nx[R][2];
    if (act && nxt) {
      scores(SK, nx);                        // matrix cores ...
      weights(cur, pb);                      // ... alongside the exponentials
      mask((jbase + j + 1) * BC, nx);
      accumulate(SV, pb);                    // matrix cores ...
      move_base(nx);                         // ... alongside the next maxima
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        cur[rb][0] = nx[rb][0];
        cur[rb][1] = nx[rb][1];
      }
    } else if (act) {                        // this wave's last tile
      weights(cur, pb);
      accumulate(SV, pb);
    } else if (nxt) {                        // this wave's first tile (behind a window)
      scores(SK, cur);
      mask((jbase + j + 1) * BC, cur);
      move_base(cur);
    }
  };

  for (int j = 0; j < ntiles; j += STAGES) {
    step(j, 0);
    step(j + 1, 1);
    step(j + 2, 2);
    if constexpr (STAGES > 3) step(j + 3, 3);
  }

  // ---- epilogue: O = acc / l (one division per row), LSE = ln 2 * (m + log2 l)
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    const int row = wrow0 + 32 * rb + r32;
    const float l_o = lsum[rb][0];
    const float inv_l = l_o > 0.f ? 1.f / l_o : 0.f;
    TOut* op = reinterpret_cast<TOut*>(p.o) + sv.o + (int64_t)row * p.o_stride[2];
    if constexpr (sizeof(TOut) == 2) {
      // lanes l and l ^ 32 hold 4-column halves of the same 8 columns of a
      // row: one swap per dword gives each lane 8 consecutive columns
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t w[2][2];
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int gq = 2 * m + c;
            bf16x2 a, bb;
            a[0] = (__bf16)(o[rb][db][4 * gq + 0] * inv_l); a[1] = (__bf16)(o[rb][db][4 * gq + 1] * inv_l);
            bb[0] = (__bf16)(o[rb][db][4 * gq + 2] * inv_l); bb[1] = (__bf16)(o[rb][db][4 * gq + 3] * inv_l);
            w[c][0] = __builtin_bit_cast(uint32_t, a);
            w[c][1] = __builtin_bit_cast(uint32_t, bb);
          }
          uint32_t got[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t send = half ? w[0][e] : w[1][e];
            const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
            got[e] = half ? r[0] : r[1];
          }
          const u32x4 out = half == 0 ? u32x4{w[0][0], w[0][1], got[0], got[1]} : u32x4{got[0], got[1], w[1][0], w[1][1]};
          if (row < nq) *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m + 8 * half) = out;
        }
    }
    if (row >= nq) continue;
    if constexpr (sizeof(TOut) == 4) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * half;
          const float v0 = o[rb][db][4 * gq + 0] * inv_l, v1 = o[rb][db][4 * gq + 1] * inv_l;
          const float v2 = o[rb][db][4 * gq + 2] * inv_l, v3 = o[rb][db][4 * gq + 3] * inv_l;
          *reinterpret_cast<f32x4*>(op + d) = f32x4{v0, v1, v2, v3};
        }
    }
    if (p.lse != nullptr && half == 0) {
      const float lse = l_run[rb] > 0.f ? (m_run[rb] + __log2f(l_run[rb])) * kLn2 : kNegInf;
      p.lse[sv.lse + row] = lse;
    }
  }
}


// Ping-pong variant for head_dim 128: eight waves in two groups of four (one
// wave of each group per SIMD). A wave's work is a chain of units separated by
// workgroup barriers:
//   G(j): S_{j+1}^T = K_{j+1} Q^T and O^T += V_j^T P_j^T (matrix cores),
//   S(j): mask, row maxima, exponentials and row sums of tile j (vector ALUs;
//         the sum of the bf16 weights goes to the matrix core from here),
// in the order G(-1) S(0) G(0) S(1) G(1) ... . Group 1 runs one unit behind
// group 0, so in every phase between two barriers one wave of each SIMD feeds
// the matrix core while the other runs the softmax, and the two swap at the
// next barrier.
//
// An item is 256 query rows of one head, or under the causal mask 256 / h
// rows of h heads that share a kv head (h up to 8, a power of two dividing
// the group): the waves' rows then span fewer keys, so fewer key tiles are
// streamed that only some of the waves use (at the diagonal, and at a
// window's far edge).
//
// A dense batch (or a packed batch of one sequence) runs on a persistent
// grid: one workgroup per compute unit, each with a fixed list of work
// items, and the K/V tiles of a workgroup's
// consecutive items form one stream through the ring. Stream tile g sits in
// stage g % STAGES; within its item (index t there) it is read in phases
// 2t .. 2t+3, and its stage is refilled with stream tile g+STAGES at phase
// 2t+4 (group 1) or 2t+5 (group 0), so near an item's end the ring already
// fills with the next item's first tiles. The next item's query rows go
// global -> LDS together with its first tile: an item starts with its Q and
// its first K/V tiles on chip, and no workgroup launch separates two items.
// A packed batch of several sequences keeps one item per workgroup and leaves
// the balancing of its mixed lengths to the hardware dispatcher.
template <int D, bool CAUSAL, typename TOut, int STAGES>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(const FwdParams p) {
  constexpr int NW = 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = BC * D;
  constexpr int ROWB = 2 * D;
  constexpr int NLD = TILE * 2 / 1024;
  constexpr int LPW = NLD / NW;              // 1-KB DMA writes per wave per K or V tile
  constexpr int QLPW = 32 * ROWB / 1024;     // 1-KB DMA writes per wave for its 32 query rows
  static_assert(D == 128, "a query row fills one LDS bank line");
  static_assert(NLD % NW == 0, "tile / wave mismatch");
  static_assert(STAGES == 3, "the unit rounds below are written out for a 3-stage ring");

  // [stage][K, V][TILE] ring, then [wave][32 rows][D] query rows whose 16-byte
  // chunks are XOR-ed with row % 16 (conflict-free ds_read_b128 of a column)
  __shared__ __attribute__((aligned(16))) __bf16 smem[STAGES * 2 * TILE + NW * 32 * D];
  __bf16* const qsm = smem + STAGES * 2 * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // the two waves that share a SIMD take different groups: each wave reads
  // its SIMD number and takes a ticket from that SIMD's LDS counter (kept in
  // the query area, which is free until the first query load)
  int grp;
  {
    int* const ticket = reinterpret_cast<int*>(qsm);
    if (tid < 4) ticket[tid] = 0;
    __syncthreads();
    const int simd = (__builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4)) & 3;   // HW_ID bits 5:4
    int tk = 0;
    if (lane == 0) tk = atomicAdd(&ticket[simd], 1);
    grp = __builtin_amdgcn_readfirstlane(tk) & 1;
    __syncthreads();
  }
  // Work items of this workgroup. Persistent grid (a dense batch, or a packed
  // batch of one sequence, whose items cost what a dense batch's do): the
  // workgroups of XCD x (blockIdx % 8,
  // the dispatcher's round-robin) share the contiguous range of the logical
  // order that work_item gives x, dealt out in a snake (round k left to right
  // for even k, right to left for odd k). Each (batch, kv head) row of the
  // logical order lists its query tiles heaviest first, with the query heads
  // (or head groups) of a kv head side by side, so two consecutive rounds give the workgroups
  // nearly the same causal cost (the same when a row holds whole pairs of
  // rounds and a round whole groups of heads). A packed sequence's real
  // length (the caller's longest length may overstate it) sets its item count
  // and query-tile count here, with that count's reciprocal.
  const bool persist = p.persist;
  int n_items = p.n_items, n_qt = p.n_qtiles;
  uint32_t qt_m = p.div_m[1];
  int qt_s = p.div_s[1];
  if (persist && p.cu_seqlens != nullptr) {
    const const_i32* cu = (const const_i32*)p.cu_seqlens;
    const int s0 = min(max(cu[0], 0), p.total);
    const int s1 = min(max(cu[1], s0), p.total);
    const int brw_l = 8 - p.hp_log2;
    n_qt = (s1 - s0 + (1 << brw_l) - 1) >> brw_l;
    n_items = (p.heads_q >> p.hp_log2) * n_qt;
    qt_s = n_qt <= 1 ? 0 : 32 - __builtin_clz((uint32_t)(n_qt - 1));
    qt_m = n_qt <= 1 ? 0u : (uint32_t)((((uint64_t)1 << (31 + qt_s)) + (uint64_t)n_qt - 1) / (uint64_t)n_qt);
  }
  // An item is 256 >> hp_log2 query rows of 1 << hp_log2 query heads of one
  // kv head: wave w takes head w >> rwl of them (rwl = 3 - hp_log2) and its
  // rows 32 (w % 2^rwl) on. With several heads per item the waves' rows span
  // fewer keys, so under the causal mask or a window fewer key tiles are
  // loaded that only some of the waves use.
  struct Item {
    int64_t q, k, v, o, lse;                 // element offsets of its sequence (q, o, lse: this wave's head)
    int nq, nk, w0, jbase, ntiles;           // w0: this wave's first query row
    bool valid;
  };
  // (called once per item; its inputs pass through an empty asm statement so
  // that none of its scalar arithmetic is hoisted out of the loops and kept
  // live in registers through them; the divisions are multiply-shifts by the
  // launcher's reciprocals)
  auto rdiv = [&](int n, int which) __attribute__((always_inline)) {
    const uint32_t m = which == 1 ? qt_m : p.div_m[which];
    const int sh = which == 1 ? qt_s : p.div_s[which];
    return m == 0 ? n : (int)(__umulhi((uint32_t)n, m) >> (sh - 1));
  };
  auto make_item = [&](int idx) __attribute__((always_inline)) {
    Item it{};
    int n = n_items, bid = blockIdx.x, nwg = gridDim.x, nqt = n_qt, hkv = p.heads_kv, hpl = p.hp_log2, wu = wave_u;
    asm volatile("" : "+s"(n), "+s"(bid), "+s"(nwg), "+s"(nqt), "+s"(hkv), "+s"(hpl), "+s"(wu), "+s"(idx));
    const int group = p.group >> hpl, rwl = 3 - hpl;
    int L;
    if (persist) {
      const int per = n >> 3, rem = n & 7, x = bid & 7;
      const int nslot = nwg >> 3, slot = bid >> 3;
      const int pos = idx * nslot + ((idx & 1) ? nslot - 1 - slot : slot);
      if (pos >= per + (x < rem ? 1 : 0)) return it;
      L = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + pos;
    } else {
      L = idx == 0 ? work_item(bid, nwg, p) : -1;
      if (L < 0) return it;                  // padding of the last XCD round
    }
    int d = rdiv(L, 0);
    const int g = L - d * group;
    L = d;
    d = rdiv(L, 1);
    const int t = L - d * nqt;
    L = d;
    const int b = rdiv(L, 2);
    const int kvh = L - b * hkv;
    const int hq = kvh * p.group + (g << hpl) + (wu >> rwl);     // this wave's query head
    const int qt = CAUSAL ? nqt - 1 - t : t;
    const SeqView sv = seq_view(p, b, hq, kvh);
    const int q0 = qt << (5 + rwl);
    if (q0 >= sv.nq) return it;              // a packed sequence shorter than the longest
    it.w0 = q0 + 32 * (wu & ((1 << rwl) - 1));
    it.q = sv.q; it.k = sv.k; it.v = sv.v; it.o = sv.o; it.lse = sv.lse;
    it.nq = sv.nq; it.nk = sv.nk;
    const int kv_end = CAUSAL ? min(it.nk, q0 + (32 << rwl)) : it.nk;
    // tiles wholly behind every row's window are never loaded
    it.jbase = (CAUSAL && p.window >= 0) ? max(0, q0 - p.window) / BC : 0;
    it.ntiles = (kv_end + BC - 1) / BC - it.jbase;
    it.valid = true;
    return it;
  };
  int idx = 0;
  const Item it0 = make_item(0);
  if (!it0.valid) return;                    // whole workgroup
  // the current item (its first K/V tile is stream tile c_t0)
  int c_t0 = 0, c_nt = it0.ntiles, c_nk = it0.nk, c_jb = it0.jbase, c_w0 = it0.w0, c_nq = it0.nq;
  int64_t c_o = it0.o, c_lse = it0.lse;

  const __bf16* __restrict__ qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* __restrict__ kg = reinterpret_cast<const __bf16*>(p.k);
  const __bf16* __restrict__ vg = reinterpret_cast<const __bf16*>(p.v);
  const int64_t ks2 = p.k_stride[2], vs2 = p.v_stride[2], qs2 = p.q_stride[2];
  const int W = CAUSAL ? p.window : -1;      // sliding window (row r sees keys r-W .. r)

  // DMA plan: this lane's 16-byte chunk of each 1-KB write, as a byte offset
  // inside one key tile, so a load is a scalar tile base plus a 32-bit offset
  int dma_row[LPW], dma_k[LPW], dma_v[LPW];
  uint32_t kofs[LPW], vofs[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int byte = (wave * LPW + i) * 1024 + lane * 16;
    const int r = byte / ROWB, pc = (byte % ROWB) / 16;
    dma_row[i] = r;
    dma_k[i] = 8 * (pc ^ kswz_t<D>(r));
    dma_v[i] = 8 * (pc ^ vswz_t<D>(r));
    kofs[i] = (uint32_t)(2 * (r * ks2 + dma_k[i]));
    vofs[i] = (uint32_t)(2 * (r * vs2 + dma_v[i]));
  }
  // this wave's 32 query rows of an item, from row qb on (nr rows are left
  // before the sequence end; later ones repeat the last), into its part of
  // the query area
  auto issue_q = [&](const __bf16* qb, int nr) __attribute__((always_inline)) {
    __bf16* dst = qsm + wave_u * 32 * D;
    int ln = lane;
    asm volatile("" : "+v"(ln));             // keeps the per-lane offsets out of the loops around (registers)
#pragma unroll
    for (int i = 0; i < QLPW; ++i) {
      const int rl = 4 * i + (ln >> 4);
      const int r = min(rl, nr - 1);
      const int ch = (ln & 15) ^ (rl & 15);
      __builtin_amdgcn_global_load_lds((const void*)(qb + (int64_t)r * qs2 + 8 * ch), (lds_void*)(dst + i * 512),
                                       16, 0, 0);
    }
  };

  // The issue cursor walks the stream: it points at the next K/V tile to
  // issue (ik, iv; irem keys left in its item from there on) and stops at
  // the end of the item after the current one (the query area holds one
  // item's rows ahead).
  int issued = 0;                            // stream tiles this wave has issued
  int iend = c_nt;                           // stream index where the cursor's item ends
  int ilim = 0;                              // and where it has to stop (set with the next item)
  const char* ik = reinterpret_cast<const char*>(kg + it0.k + (int64_t)it0.jbase * BC * ks2);
  const char* iv = reinterpret_cast<const char*>(vg + it0.v + (int64_t)it0.jbase * BC * vs2);
  int irem = it0.nk - it0.jbase * BC;
  issue_q(qg + it0.q + (int64_t)it0.w0 * qs2, it0.nq - it0.w0);
  // the next item (read once per item: these may live in spill lanes)
  Item nx;
  const char* nx_k;
  const char* nx_v;
  const __bf16* nx_q;
  int nx_nt, nx_rem, nx_qr;

  // Issue the next stream tile (stage ist = issued % STAGES); the first tile
  // of the next item takes that item's query rows with it.
  int ist = 0;
  auto issue_one = [&]() __attribute__((always_inline)) {
    if (issued == iend) {                    // on into the next item
      ik = nx_k;
      iv = nx_v;
      irem = nx_rem;
      iend += nx_nt;
      issue_q(nx_q, nx_qr);
    }
    __bf16* dst = smem + ist * 2 * TILE + wave_u * LPW * 512;
    if (irem >= BC) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        __builtin_amdgcn_global_load_lds((const void*)(ik + kofs[i]), (lds_void*)(dst + i * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(iv + vofs[i]), (lds_void*)(dst + TILE + i * 512), 16, 0, 0);
      }
    } else {                                 // ragged last tile: rows past the end repeat the last row
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int r = min(dma_row[i], irem - 1);
        const uint32_t ko = (uint32_t)(2 * (r * ks2 + dma_k[i])), vo = (uint32_t)(2 * (r * vs2 + dma_v[i]));
        __builtin_amdgcn_global_load_lds((const void*)(ik + ko), (lds_void*)(dst + i * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(iv + vo), (lds_void*)(dst + TILE + i * 512), 16, 0, 0);
      }
    }
    ik += 2 * BC * ks2;
    iv += 2 * BC * vs2;
    irem -= BC;
    ++issued;
    ist = ist == STAGES - 1 ? 0 : ist + 1;
  };
  // issue the stream up to tile `last`, within the current and the next item
  auto issue_upto = [&](int last) __attribute__((always_inline)) {
    const int lim = min(last + 1, ilim);
    while (issued < lim) issue_one();
  };
  // wait until this wave's loads of stream tile g of the current item (and
  // everything older) have landed: the loads younger than g are the later
  // tiles issued so far, plus the next item's query rows once the cursor has
  // moved into that item
  auto wait_for = [&](int g) __attribute__((always_inline)) {
    const int y = 2 * LPW * (issued - g - 1) + (issued > c_t0 + c_nt ? QLPW : 0);
    if (y >= 2 * LPW * 3 + QLPW) wait_vmcnt<2 * LPW * 3 + QLPW>();
    else if (y >= 2 * LPW * 2 + QLPW) wait_vmcnt<2 * LPW * 2 + QLPW>();
    else if (y >= 2 * LPW + QLPW) wait_vmcnt<2 * LPW + QLPW>();
    else if (y >= 2 * LPW * 2) wait_vmcnt<2 * LPW * 2>();
    else if (y >= 2 * LPW) wait_vmcnt<2 * LPW>();
    else wait_vmcnt<0>();
  };
  // workgroup barrier without the fence of __syncthreads (which would also
  // drain the loads still in flight for later tiles)
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

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
  // Sum of the bf16 weights that enter P V, on the matrix core (v_dot2c runs
  // on the matrix pipe too, so it would stall the other wave's MFMAs): a
  // P^T chunk read as the B operand of v_mfma_f32_16x16x32_bf16 holds, in
  // column n, keys 0-7 and 8-15 of rows n and n+16; the A operand below is 1
  // where the key group belongs to the row this lane's accumulator holds
  // (row lane % 32), so every register of lsum is that row's running sum.
  bf16x8 lsel;
  {
    const __bf16 one = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? (__bf16)1.f : (__bf16)0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) lsel[e] = one;
  }

  const float c2 = p.scale_log2;
  bf16x8 qf[KSTEPS];
  float m_run, l_run, m_use;                 // m_use: m_run, or 0 while no key has been seen
  f32x4 lsum;
  f32x16 o[DBLK];
  f32x16 sc[2];          // scores of the tile the next S unit works on
  bf16x8 pb[4];          // P^T of the tile the next G unit accumulates
  // per-item geometry of this wave
  int wrow0, row, nt_w, lo_w;

  auto scores = [&](int ST) __attribute__((always_inline)) {
    const __bf16* ks = smem + ST * 2 * TILE;
    sc[0] = sc[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks + koff[kc]);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(ks + 32 * D + koff[kc]);
      sc[0] = mfma32(k0, qf[kc], sc[0]);
      sc[1] = mfma32(k1, qf[kc], sc[1]);
    }
  };
  auto accumulate = [&](int ST) __attribute__((always_inline)) {
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
        o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[c], o[db]);
      }
    }
  };
  // Both halves of a G unit with the LDS fragment reads issued AHEAD steps
  // before the MFMA that consumes them (a scheduling barrier after each step
  // keeps that order): K for the 8 score k-steps, then V (two transposing
  // reads per PV MFMA) for the 16 PV MFMAs.
  auto gunit = [&](int SK, int SV) __attribute__((always_inline)) {
    constexpr int AHEAD = kAhead;
    const __bf16* ks = smem + SK * 2 * TILE;
    const __bf16* vs = smem + SV * 2 * TILE + TILE;
    bf16x8 kf[KSTEPS][2];
    bf16x4 vf[4 * DBLK][2];
    auto read_k = [&](int kc) __attribute__((always_inline)) {
      kf[kc][0] = *reinterpret_cast<const bf16x8*>(ks + koff[kc]);
      kf[kc][1] = *reinterpret_cast<const bf16x8*>(ks + 32 * D + koff[kc]);
    };
    // PV step i: key chunk i / DBLK, d block i % DBLK
    auto read_v = [&](int i) __attribute__((always_inline)) {
      const __bf16* va = vs + voff[i % DBLK] + 16 * (i / DBLK) * D;
      vf[i][0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va));
      vf[i][1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va + 4 * D));
    };
    // reads in consumption order: K k-steps 0..KSTEPS-1, then V steps 0..4*DBLK-1
    auto read = [&](int x) __attribute__((always_inline)) {
      if (x < KSTEPS) read_k(x);
      else if (x < KSTEPS + 4 * DBLK) read_v(x - KSTEPS);
    };
#pragma unroll
    for (int x = 0; x < AHEAD; ++x) read(x);
    sc[0] = sc[1] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) {
      __builtin_amdgcn_sched_barrier(0);
      read(kc + AHEAD);
      sc[0] = mfma32(kf[kc][0], qf[kc], sc[0]);
      sc[1] = mfma32(kf[kc][1], qf[kc], sc[1]);
    }
#pragma unroll
    for (int i = 0; i < 4 * DBLK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      read(KSTEPS + i + AHEAD);
      o[i % DBLK] = mfma32(__builtin_shufflevector(vf[i][0], vf[i][1], 0, 1, 2, 3, 4, 5, 6, 7), pb[i / DBLK],
                           o[i % DBLK]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto softmax = [&](int kv0) __attribute__((always_inline)) {
    const int nk = c_nk;
    const bool win = W >= 0 && kv0 < wrow0 + 31 - W;
    if ((CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > nk) || win) {
      const int kmin = win ? row - W : -1;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int k0 = kv0 + acc_key(jj, half), k1 = k0 + 32;
        sc[0][jj] = ((CAUSAL && k0 > row) || k0 >= nk || k0 < kmin) ? kNegInf : sc[0][jj];
        sc[1][jj] = ((CAUSAL && k1 > row) || k1 >= nk || k1 < kmin) ? kNegInf : sc[1][jj];
      }
    }
    // A single wave issues an independent VALU op about every 5 cycles but a
    // dependent one only every 10, so the row maximum and the row sum run as
    // four interleaved chains rather than one.
    float mq[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& a = sc[c >> 1];
      const int o8 = 8 * (c & 1);
      float m = fmaxf(fmaxf(a[o8], a[o8 + 1]), a[o8 + 2]);
      m = fmaxf(fmaxf(m, a[o8 + 3]), a[o8 + 4]);
      m = fmaxf(fmaxf(m, a[o8 + 5]), a[o8 + 6]);
      mq[c] = fmaxf(m, a[o8 + 7]);
    }
    const float mt = half_swap_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * c2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
      m_run = m_new;
      m_use = m_new == kNegInf ? 0.f : m_new;
    }
    float rq[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {          // P^T chunk c: keys 16c .. 16c+15 of the tile
        const float pr = fast_exp2(fmaf(sc[c >> 1][8 * (c & 1) + e], c2, -m_use));
        rq[c] = e == 0 ? pr : rq[c] + pr;
        pb[c][e] = (__bf16)pr;
      }
    }
    const float rs = (rq[0] + rq[1]) + (rq[2] + rq[3]);
    l_run += half_swap_sum(rs);
    // the bf16 weights' sum goes to the matrix core from the softmax unit, so
    // that both waves of a SIMD feed it in this phase (the other one is in
    // its matrix unit); same products, same order, same bits
#pragma unroll
    for (int c = 0; c < 4; ++c) lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lsel, pb[c], lsum, 0, 0, 0);
  };

  // Phases are numbered within the current item: at phase 2t+4 (group 1) or
  // 2t+5 (group 0) a wave issues its share of stream tile g+STAGES into the
  // stage of the item's tile t (stream tile g); before the barrier that
  // opens phase 2t, tile t must have landed.
  //   After an item's start, where the stream stands at least STAGES tiles
  // into the item (or at the end of the next one), each such step frees one
  // stage and the stream moves on by at most one tile. When tile t >= 2 is
  // waited for (end of phase 2t-1), the last step taken was that of tile
  // t-3, so no later tile is in flight: everything this wave has issued must
  // land. Tile 1 is waited for the same way at the end of phase 1 (tile 2,
  // issued at the item's start, lands with it). Tile 0 and the query rows
  // are waited for before the previous item's outputs are stored, or at the
  // first item's start.
  // ev_ph: this wave's next refill phase; permit: the last stream tile whose
  // stage is free by then
  int ev_ph, permit;
  auto phase_begin = [&](int ph) __attribute__((always_inline)) {
    if (ph == ev_ph) {
      ev_ph += 2;
      ++permit;
      if (issued <= permit && issued < ilim) issue_one();
    }
  };
  auto phase_end = [&](int ph, int nph) __attribute__((always_inline)) {
    if (ph + 1 >= nph) return;
    // tile (ph + 1) / 2 is read from the next phase on
    if ((ph & 1) && ph < 2 * c_nt - 1) wait_vmcnt<0>();
    barrier();
  };

  for (;;) {
    nx = make_item(idx + 1);
    nx_nt = nx.valid ? nx.ntiles : 0;
    ilim = iend + nx_nt;
    nx_k = reinterpret_cast<const char*>(kg + nx.k + (int64_t)nx.jbase * BC * ks2);
    nx_v = reinterpret_cast<const char*>(vg + nx.v + (int64_t)nx.jbase * BC * vs2);
    nx_rem = nx.nk - nx.jbase * BC;
    nx_q = qg + nx.q + (int64_t)nx.w0 * qs2;
    nx_qr = nx.nq - nx.w0;

    // Item start: its first tiles (and query rows) are issued, mostly during
    // the previous item already. The query rows are read before the stream
    // may run on into the next item, whose rows take their place.
    issue_upto(min(c_t0 + STAGES, c_t0 + c_nt) - 1);
    if (idx == 0) wait_for(c_t0);         // later items: waited for at the previous item's end
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));           // addresses made here, not kept from before the item loop
      const __bf16* qr = qsm + wave_u * 32 * D + (ln & 31) * D;
      const int c0 = (ln >> 5) ^ (ln & 15);
#pragma unroll
      for (int kc = 0; kc < KSTEPS; ++kc)
        qf[kc] = *reinterpret_cast<const bf16x8*>(qr + 8 * (c0 ^ (2 * kc)));
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    issue_upto(c_t0 + STAGES - 1);
    // The first item's first tile is published here; a later item's was
    // published by the barrier after the previous item's outputs. Without a
    // barrier here group 0 goes on to its first unit while group 1 finishes
    // this set-up (both groups still reach the same barriers).
    if (idx == 0) barrier();

    wrow0 = c_w0;
    asm volatile("" : "+v"(wrow0));
    row = wrow0 + r32;
    // Tiles this wave needs: [lo_w, nt_w). Without the mask that is every
    // tile, but the bound is still written in terms of the wave's first row
    // (equal to ntiles since wrow0 >= 0), and that row sits in a vector
    // register, a per-lane value to the compiler: a wave-uniform bound lets
    // it turn the unit loop into uniform branches whose register allocation
    // spills.
    nt_w = CAUSAL ? min(c_nt, (wrow0 + 31) / BC + 1 - c_jb)
                  : min(c_nt, (wrow0 + c_nk + BC - 1) / BC);
    lo_w = W >= 0 ? max(0, wrow0 - W) / BC - c_jb : 0;
    m_run = kNegInf;
    l_run = 0.f;
    m_use = 0.f;
    lsum = f32x4{};
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};

    const int nunits = 2 * c_nt + 1;   // G(-1), S(0), G(0), ..., S(nt-1), G(nt-1)
    const int nph = nunits + 1;
    ev_ph = grp == 0 ? 5 : 4;
    permit = c_t0 + STAGES - 1;
    if (grp == 1) {                          // group 1 idles through phase 0
      phase_begin(0);
      phase_end(0, nph);
    }
    // Unit u (r = its position in a round of 2 STAGES units; the stages it
    // reads are constants of r). Returns false past the last unit.
    auto unit = [&](int u, auto rc) __attribute__((always_inline)) -> bool {
      constexpr int r = decltype(rc)::value;
      if (u >= nunits) return false;
      const int ph = u + grp;
      phase_begin(ph);
      if constexpr (r & 1) {                          // S(j), j = (u - 1) / 2
        const int j = (u - 1) >> 1;
        if (j >= lo_w && j < nt_w) softmax((c_jb + j) * BC);
      } else {                                        // G(j), j = u / 2 - 1
        const int j = (u >> 1) - 1;
        constexpr int SK = (r / 2) % STAGES;          // stage of tile j + 1
        constexpr int SV = (r / 2 + STAGES - 1) % STAGES;     // stage of tile j
        if (j >= lo_w && j + 1 < nt_w) gunit(SK, SV);
        else {
          if (j + 1 >= lo_w && j + 1 < nt_w) scores(SK);
          if (j >= lo_w && j < nt_w) accumulate(SV);
        }
      }
      phase_end(ph, nph);
      return true;
    };
    // The item's tile t is stream tile c_t0 + t, in stage (c_t0 + t) % 3, so
    // its units start at position 2 (c_t0 % 3) of a round: the partial first
    // round is peeled off.
    const int rot = c_t0 % STAGES;
    int ub = 0;
    bool more = true;
    if (rot == 1) {
      more = unit(0, int_c<2>{}) && unit(1, int_c<3>{});
      ub = 2;
    }
    if (more && rot != 0) {
      more = unit(ub, int_c<4>{}) && unit(ub + 1, int_c<5>{});
      ub += 2;
    }
    if (more) {
      for (;; ub += 6) {
        if (!unit(ub + 0, int_c<0>{}) || !unit(ub + 1, int_c<1>{}) || !unit(ub + 2, int_c<2>{}) ||
            !unit(ub + 3, int_c<3>{}) || !unit(ub + 4, int_c<4>{}) || !unit(ub + 5, int_c<5>{}))
          break;
      }
    }
    if (grp == 0) phase_begin(nph - 1);              // group 0 idles through the last phase
    // The next item's first tile and query rows (issued at least two phases
    // ago; its stage held a tile that every wave has finished with) are
    // waited for before this item's outputs are stored: stores count in
    // vmcnt too, so a wait after them would wait for them. Only the next
    // item's second tile may be younger.
    if (nx_nt > 0) {
      issue_upto(c_t0 + c_nt);
      if (issued > c_t0 + c_nt + 1) wait_vmcnt<2 * LPW>();
      else wait_vmcnt<0>();
    }

    if constexpr (sizeof(TOut) == 2) {
      // bf16 out: lanes l and l ^ 32 hold 4-column halves of the same 8
      // columns of a row; one swap gives each lane 8 consecutive columns, so
      // a row goes out in 16-byte stores
      const float l_o = lsum[0];
      const float inv_l = l_o > 0.f ? 1.f / l_o : 0.f;
      TOut* op = reinterpret_cast<TOut*>(p.o) + c_o + (int64_t)row * p.o_stride[2];
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t w[2][2];                    // [chunk 2m, 2m+1][dword]: 4 bf16 of this lane
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int gq = 2 * m + c;
            bf16x2 a, bb;
            a[0] = (__bf16)(o[db][4 * gq + 0] * inv_l); a[1] = (__bf16)(o[db][4 * gq + 1] * inv_l);
            bb[0] = (__bf16)(o[db][4 * gq + 2] * inv_l); bb[1] = (__bf16)(o[db][4 * gq + 3] * inv_l);
            w[c][0] = __builtin_bit_cast(uint32_t, a);
            w[c][1] = __builtin_bit_cast(uint32_t, bb);
          }
          // half 0 sends chunk 2m+1 and keeps 2m; half 1 sends 2m and keeps 2m+1
          uint32_t got[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t send = half ? w[0][e] : w[1][e];
            const auto r = __builtin_amdgcn_permlane32_swap(send, send, false, false);
            got[e] = half ? r[0] : r[1];     // the partner lane's value
          }
          u32x4 out;
          if (half == 0) out = u32x4{w[0][0], w[0][1], got[0], got[1]};
          else out = u32x4{got[0], got[1], w[1][0], w[1][1]};
          if (row < c_nq) *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m + 8 * half) = out;
        }
    }
    if (row < c_nq) {
      if constexpr (sizeof(TOut) == 4) {
        const float l_o = lsum[0];
        const float inv_l = l_o > 0.f ? 1.f / l_o : 0.f;
        TOut* op = reinterpret_cast<TOut*>(p.o) + c_o + (int64_t)row * p.o_stride[2];
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * db + 8 * gq + 4 * half;
            const float v0 = o[db][4 * gq + 0] * inv_l, v1 = o[db][4 * gq + 1] * inv_l;
            const float v2 = o[db][4 * gq + 2] * inv_l, v3 = o[db][4 * gq + 3] * inv_l;
            *reinterpret_cast<f32x4*>(op + d) = f32x4{v0, v1, v2, v3};
          }
      }
      if (p.lse != nullptr && half == 0) {
        const float lse = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
        p.lse[c_lse + row] = lse;
      }
    }
    if (nx_nt == 0) break;                            // no next item
    barrier();                                        // the last phase's reads end; the next item's first tile is published
    ++idx;
    c_t0 += c_nt;
    c_nt = nx.ntiles; c_nk = nx.nk; c_jb = nx.jbase; c_w0 = nx.w0; c_nq = nx.nq;
    c_o = nx.o; c_lse = nx.lse;
  }
}


}  // namespace detail

namespace {

// Compute units of the current device (the persistent grid's size), looked
// up once per device. Concurrent first calls may both query the runtime; each
// stores the same value, and the relaxed atomics make that race-free.
inline int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, bool CAUSAL, typename TOut, int NW, int R, int STAGES>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  constexpr int BRW = 32 * R * NW;
  FwdParams q = p;
  q.n_qtiles = (p.seqlen_q + BRW - 1) / BRW;
  q.n_items = q.batch * q.heads_q * q.n_qtiles;
  q.cu_count = device_cus();
  const int64_t wgs = grid_for(q);
  hipLaunchKernelGGL((detail::fwd_bf16_kernel<D, CAUSAL, TOut, NW, R, STAGES>), dim3((unsigned)wgs), dim3(NW * 64),
                     0, stream, q);
  return hipGetLastError();
}

template <int D, bool CAUSAL, typename TOut, int STAGES>
hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  // Under the causal mask (and a window) an item takes up to 8 query heads of
  // a kv head with 256 / 8 rows each: all its waves then need the same key
  // tiles, where 256 rows of one head span 4 more tiles at the diagonal (and
  // 4 more at a window's far edge) that only some of the waves use.
  q.hp_log2 = 0;
  if (CAUSAL)
    while (q.hp_log2 < 3 && q.group % (2 << q.hp_log2) == 0) ++q.hp_log2;
  const int brw = 256 >> q.hp_log2;
  q.n_qtiles = (p.seqlen_q + brw - 1) / brw;
  q.n_items = q.batch * (q.heads_q >> q.hp_log2) * q.n_qtiles;
  fa_reciprocal(q.group >> q.hp_log2, &q.div_m[0], &q.div_s[0]);
  fa_reciprocal(q.n_qtiles, &q.div_m[1], &q.div_s[1]);
  fa_reciprocal(q.heads_kv, &q.div_m[2], &q.div_s[2]);
  // persistent (dense, or packed with one sequence): one workgroup per
  // compute unit (one fits, by its LDS), a whole number per XCD; packed: one
  // per work item
  q.persist = q.cu_seqlens == nullptr || q.batch == 1;
  const int64_t wgs = !q.persist
                          ? grid_for(q)
                          : std::min<int64_t>(std::max(8, device_cus() / 8 * 8), ((int64_t)q.n_items + 7) / 8 * 8);
  hipLaunchKernelGGL((detail::fwd_pp_kernel<D, CAUSAL, TOut, STAGES>), dim3((unsigned)wgs), dim3(512), 0, stream, q);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int NW, int R, int STAGES>
hipError_t launch_out(const FwdParams& p, hipStream_t stream) {
  return p.out_fp32 ? launch<D, CAUSAL, float, NW, R, STAGES>(p, stream)
                    : launch<D, CAUSAL, __bf16, NW, R, STAGES>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.in_fp32) return launch_fwd_f32(p, stream);
  if (p.head_dim == 64)
    return p.causal ? launch_out<64, true, 4, 1, 3>(p, stream) : launch_out<64, false, 4, 1, 3>(p, stream);
  if (p.causal)
    return p.out_fp32 ? launch_pp<128, true, float, kPpStages>(p, stream)
                      : launch_pp<128, true, __bf16, kPpStages>(p, stream);
  return p.out_fp32 ? launch_pp<128, false, float, kPpStages>(p, stream)
                    : launch_pp<128, false, __bf16, kPpStages>(p, stream);
}

}  // namespace fa
