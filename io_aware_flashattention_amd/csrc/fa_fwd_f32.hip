// Prefill attention forward for float32 inputs on gfx950 (the bf16 path is in
// fa_fwd.hip): exact softmax attention computed one 64-key tile at a time with
// a running row maximum and running row sum, so the N x N scores never leave
// the chip.
//
// The loop is the FlashAttention-2 order ("FlashAttention and GPU Data
// Movement", section 2 and the recurrence of section 3.1): a workgroup owns a
// 128-row query tile, streams K/V tiles through LDS, keeps an unnormalised
// float32 accumulator in registers, divides once at the end and writes O and
// the per-row log-sum-exp once. Under the causal mask, tiles wholly in the
// future are not loaded (the skip bound) and only tiles crossing the diagonal
// are masked, elementwise, before the row statistics see them (section 2.1).
//
// Mapping onto the CDNA4 compute unit (four 64-lane waves per workgroup, two
// workgroups per CU so one wave's softmax overlaps another's matrix work):
//   * wave w owns query rows q0+32w .. q0+32w+31; lane l owns row l % 32;
//   * S^T = K_tile Q^T on v_mfma_f32_32x32x16_bf16 (keys on M, rows on N);
//     K rows are fed in sigma order so the score accumulator is already the
//     B operand of O^T += V^T P^T: no register shuffles between the two;
//   * the softmax runs in base 2 with scale*log2(e) folded into one FMA per
//     score; a row's keys are split between lane l and lane l^32, joined with
//     one permlane32 swap for the max and one for the sum;
//   * K is staged as [key][d], V transposed as [d][key], both with XOR-swizzled
//     16-byte chunks, double-buffered: the next tile's global loads are in
//     flight while the current tile is computed.
// float32 inputs keep the same structure with every operand split into a
// bf16 high part and a bf16 remainder (x = hi + lo to about 16 significant
// bits); each product is hi*hi + hi*lo + lo*hi on the same bf16 matrix
// instructions, so float32 data is not truncated to 8 significant bits.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int BR = 128;   // query rows per workgroup
constexpr int BC = 64;    // keys per tile
constexpr int NT = 256;   // threads per workgroup

template <typename TIn> constexpr int min_blocks() { return sizeof(TIn) == 2 ? 2 : 1; }

template <int D, bool CAUSAL, typename TIn, typename TOut>
__global__ __launch_bounds__(NT, min_blocks<TIn>()) void fwd_kernel(const FwdParams p) {
  constexpr bool SPLIT = sizeof(TIn) == 4;   // float32 inputs: hi/lo bf16 planes
  constexpr int NP = SPLIT ? 2 : 1;          // LDS planes per operand
  constexpr int DCH = D / 8;                 // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;               // 32-row blocks of O^T
  constexpr int K_LOADS = BC * DCH / NT;     // K chunks per thread
  constexpr int V_ITEMS = (BC / 4) * DCH;    // (4 keys x 8 d) items per V tile
  constexpr int TILE = BC * D;               // elements per K or Vt tile
  using IO = In<TIn>;
  static_assert(K_LOADS >= 1 && BC * DCH % NT == 0, "tile / thread mismatch");

  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * NP * TILE];   // [stage][K planes | Vt planes]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int r32 = lane & 31;

  // ---- which (batch, head, query tile): XCD-aware, heavy causal tiles first
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

  const TIn* __restrict__ qp = reinterpret_cast<const TIn*>(p.q) + b * p.q_stride[0] + hq * p.q_stride[1];
  const TIn* __restrict__ kp = reinterpret_cast<const TIn*>(p.k) + b * p.k_stride[0] + kvh * p.k_stride[1];
  const TIn* __restrict__ vp = reinterpret_cast<const TIn*>(p.v) + b * p.v_stride[0] + kvh * p.v_stride[1];

  const int q0 = qt * BR;
  const int wrow0 = q0 + wave * 32;
  const int row = wrow0 + r32;
  const int nq = p.seqlen_q, nk = p.seqlen_k;

  // ---- this lane's query row as B-operand fragments (rows past the end are 0)
  bf16x8 qf[KSTEPS], ql[SPLIT ? KSTEPS : 1];
#pragma unroll
  for (int kc = 0; kc < KSTEPS; ++kc) {
    auto raw = row < nq ? IO::load(qp + (int64_t)row * p.q_stride[2] + 16 * kc + 8 * half) : IO::zero();
    if constexpr (SPLIT) {
      split_hi_lo(raw, qf[kc], ql[kc]);
    } else {
      qf[kc] = as_bf16x8(IO::pack(raw));
    }
  }

  const int kv_end = CAUSAL ? min(nk, q0 + BR) : nk;   // skip bound
  const int ntiles = (kv_end + BC - 1) / BC;

  // ---- global -> register staging of one K/V tile
  typename IO::Raw kreg[K_LOADS];
  typename IO::Raw vreg[4];
  const int v_item = tid;                       // one (4-key x 8-d) item per thread
  const int v_dc = v_item % DCH, v_kg = v_item / DCH;
  const bool v_on = V_ITEMS >= NT || v_item < V_ITEMS;

  auto load_tile = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + NT * i;
      const int key = c / DCH, ch = c % DCH;
      kreg[i] = (kv0 + key < nk) ? IO::load(kp + (int64_t)(kv0 + key) * p.k_stride[2] + 8 * ch) : IO::zero();
    }
    if (v_on) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kv0 + 4 * v_kg + i;
        vreg[i] = (key < nk) ? IO::load(vp + (int64_t)key * p.v_stride[2] + 8 * v_dc) : IO::zero();
      }
    }
  };

  auto store_tile = [&](int stage) {
    __bf16* ks = smem + stage * 2 * NP * TILE;     // K planes: hi [, lo]
    __bf16* vs = ks + NP * TILE;                   // Vt planes: hi [, lo]
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + NT * i;
      const int key = c / DCH, ch = c % DCH;
      const int at = key * D + 8 * (ch ^ kswz(key));
      if constexpr (SPLIT) {
        bf16x8 hi, lo;
        split_hi_lo(kreg[i], hi, lo);
        *reinterpret_cast<bf16x8*>(ks + at) = hi;
        *reinterpret_cast<bf16x8*>(ks + TILE + at) = lo;
      } else {
        *reinterpret_cast<u32x4*>(ks + at) = IO::pack(kreg[i]);
      }
    }
    if (v_on) {
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
        u32x4 w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (SPLIT) {
            bf16x8 hi, lo;
            split_hi_lo(vreg[i], hi, lo);
            w[i] = __builtin_bit_cast(u32x4, pl == 0 ? hi : lo);
          } else {
            w[i] = IO::pack(vreg[i]);
          }
        }
        // element e of keys 4kg..4kg+3 -> Vt[8*dc + e][4kg .. 4kg+3]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = (e & 1) * 16;
          const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xffffu, a1 = (w[1][e >> 1] >> sh) & 0xffffu;
          const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xffffu, a3 = (w[3][e >> 1] >> sh) & 0xffffu;
          const int d = 8 * v_dc + e;
          const int chunk = (v_kg >> 1) ^ vswz(d);
          *reinterpret_cast<u32x2*>(vs + pl * TILE + d * BC + 8 * chunk + 4 * (v_kg & 1)) =
              u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
        }
      }
    }
  };

  // ---- running state of this lane's row
  const float c2 = p.scale_log2;           // scale * log2(e): scores in base-2 units
  float m_run = kNegInf;                   // running max (base-2 units)
  float l_run = 0.f;                       // running sum of exp2(s - m_run)
  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * BC;
    const bool has_next = j + 1 < ntiles;
    if (has_next) load_tile(j + 1);

    // a wave whose rows all precede the tile's first key has nothing to do here
    const bool active = !CAUSAL || kv0 <= wrow0 + 31;
    if (active) {
      const __bf16* ks = smem + (j & 1) * 2 * NP * TILE;
      const __bf16* vs = ks + NP * TILE;

      // S^T for the 64 keys: two 32-key blocks
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const int key = 32 * kb + sigma32(r32);
#pragma unroll
        for (int kc = 0; kc < KSTEPS; ++kc) {
          const int at = key * D + 8 * ((2 * kc + half) ^ kswz(key));
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + at);
          if constexpr (SPLIT) {
            const bf16x8 al = *reinterpret_cast<const bf16x8*>(ks + TILE + at);
            s[kb] = mfma32(al, qf[kc], s[kb]);
            s[kb] = mfma32(a, ql[kc], s[kb]);
          }
          s[kb] = mfma32(a, qf[kc], s[kb]);
        }
      }

      // diagonal / ragged tiles: -inf where the key is in the row's future or past the end
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > nk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int key = kv0 + 32 * kb + acc_key(jj, half);
            const bool dead = (CAUSAL && key > row) || key >= nk;
            s[kb][jj] = dead ? kNegInf : s[kb][jj];
          }
      }

      // online softmax update for this row
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, s[kb][jj]);
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;   // no visible key yet
      const float alpha = fast_exp2(m_run - m_use);           // exp2(-inf) = 0 on the first tile
      m_run = m_new;

      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const float pv = fast_exp2(fmaf(s[kb][jj], c2, -m_use));
          s[kb][jj] = pv;
          rs += pv;
        }
      rs = half_swap_sum(rs);
      l_run = fmaf(l_run, alpha, rs);
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;

      // P^T chunks of 16 keys as bf16 B operands
      bf16x8 pb[4], pl[SPLIT ? 4 : 1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = s[c >> 1][8 * (c & 1) + e];
        pb[c] = to_bf16x8(f);
        if constexpr (SPLIT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] -= (float)pb[c][e];
          pl[c] = to_bf16x8(f);
        }
      }

      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int d = 32 * db + r32;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int at = d * BC + 8 * ((2 * c + half) ^ vswz(d));
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + at);
          if constexpr (SPLIT) {
            const bf16x8 al = *reinterpret_cast<const bf16x8*>(vs + TILE + at);
            o[db] = mfma32(al, pb[c], o[db]);
            o[db] = mfma32(a, pl[c], o[db]);
          }
          o[db] = mfma32(a, pb[c], o[db]);
        }
      }
    }

    if (has_next) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (one division per row), LSE = ln 2 * (m + log2 l)
  if (row < nq) {
    const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
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

template <int D, bool CAUSAL, typename TOut>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  q.n_qtiles = (p.seqlen_q + BR - 1) / BR;
  const int64_t wgs = (int64_t)q.batch * q.heads_q * q.n_qtiles;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, float, TOut>), dim3((unsigned)wgs), dim3(NT), 0, stream, q);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_out(const FwdParams& p, hipStream_t stream) {
  return p.out_fp32 ? launch<D, CAUSAL, float>(p, stream) : launch<D, CAUSAL, __bf16>(p, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.head_dim == 64) return p.causal ? launch_out<64, true>(p, stream) : launch_out<64, false>(p, stream);
  return p.causal ? launch_out<128, true>(p, stream) : launch_out<128, false>(p, stream);
}

}  // namespace fa
