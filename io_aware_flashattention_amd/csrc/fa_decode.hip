// Split-KV single-token decode for gfx950.
//
// With one query token per sequence the query-tile axis collapses to a single
// tile, so the key axis is the only long one: it is split across workgroups,
// every piece computes a partial output and its log-sum-exp, and a small
// second kernel merges the partials with the same rescaling identity the tile
// loop uses ("FlashAttention Explained: IO-Aware Attention, Tiling, Online
// Softmax and FP8 on Hopper", section "Decoding, Paged and Split-KV
// Variants"; "FlashAttention and GPU Data Movement", section 6.1).
//
// Work split (balanced by construction). The cache rows to read form one
// stream of T = Hkv * sum_b L_b tokens, slab after slab, slab = (sequence b,
// kv head). A fixed grid of W one-wave workgroups cuts it into W equal
// contiguous ranges of P tokens (P >= split_tokens). A wave streams its range
// and emits a partial (o, lse) for the G query heads of a slab each time it
// finishes its piece of that slab; the piece of slab s done by wave w is
// stored at index s + w, so at most B*Hkv + W partials exist. Every wave reads
// the same number of bytes, whatever the mix of sequence lengths.
//
// Per 32-key block the wave
//   * moves 8 KB of K and 8 KB of V global -> LDS with direct DMA loads into
//     a private ring of NST stages, NST-1 blocks ahead of the compute;
//   * computes S^T = K q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with
//     the G heads of the kv head on the N axis (bound by memory, not by the
//     matrix cores), K fragments by ds_read_b128 and V^T fragments by
//     transposing ds_read_b64_tr_b16, both through conflict-free swizzles;
//   * updates each head's running max and sums (one lane per head), with the
//     accumulator rescaled only when a maximum grows by more than 2^8; O is
//     normalised by the sum of the bf16-rounded weights, the log-sum-exp uses
//     the float32 sum.
//
// Paged cache (same section: keys and values are fetched through a block
// table). Token t of a sequence sits in slot t % page_size of the page the
// table names for logical block t / page_size. A 32-key block then touches at
// most three pages (page_size >= 16): the wave reads their table entries with
// scalar loads one block ahead of the DMA that needs them, so the lookup never
// waits on the vector-memory counter the DMA ring is paced by, and each lane
// picks its row's page and slot with a compare, not a division.
#include <atomic>

#include "fa_device.h"
#include "fa_launch.h"

#ifndef FA_DEC_NST
#define FA_DEC_NST 3          // ring stages per wave (NST-1 blocks in flight)
#endif
#ifndef FA_DEC_WPC
#define FA_DEC_WPC 3          // one-wave workgroups per CU (LDS-limited)
#endif

namespace fa {

namespace {

constexpr int KB = 32;                       // keys per block
constexpr int NST = FA_DEC_NST;
constexpr float kRescaleThreshold = 8.f;
static_assert(NST >= 2 && NST <= 4, "");

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// LDS swizzles of the 16-byte chunks of a K or V row (the bank model is
// described with the prefill kernel): 256-byte rows (D = 128) fill a bank
// line each, 128-byte rows (D = 64) share one between two rows
template <int D> __device__ __forceinline__ int kswz_d(int r) {
  return D == 128 ? (sigma32(r & 31) & 15) : ((r >> 1) & 7);
}
template <int D> __device__ __forceinline__ int vswz_d(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// Lengths and block-table entries are read at wave-uniform addresses through
// the constant address space, so they become scalar loads: they wait on the
// LDS/scalar counter, never on the vector-memory counter that paces the DMA.
typedef __attribute__((address_space(4))) const int32_t const_i32;

__device__ __forceinline__ int seq_len(const DecodeParams& p, int b) {
  return min(max(((const const_i32*)p.seqlens)[b], 0), p.max_seqlen);
}

// a wave-uniform 64-bit value computed in vector registers, moved to scalar ones
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Tokens per wave range, identical in both kernels: at least split_tokens, a
// multiple of the block, and W ranges cover all T tokens of the stream.
__device__ __forceinline__ int64_t range_tokens(const DecodeParams& p, int64_t T) {
  int64_t P = (T + p.n_waves - 1) / p.n_waves;
  P = P > p.split_tokens ? P : p.split_tokens;
  return (P + KB - 1) / KB * KB;
}

// Position in the token stream: slab (b, kvh), key position inside the slab
// (a multiple of the block, so blocks line up with pages), the piece's first
// key (keys of the first block before it belong to the previous range and
// are masked) and end of the piece (exclusive, inside the slab).
struct Cursor {
  int b, kvh, pos, start, end;
  int64_t slab_off;          // stream offset of the slab's first token
};

// Pages under one 32-key block of a paged cache: the table entries of the
// block's first three logical pages (raw, so that the scalar loads stay in
// flight until the DMA issue needs them), and the block's first and last key
// as slots counted from the start of the first page.
struct PageRun {
  int e0, e1, e2;
  int off, lim;
};

}  // namespace

namespace detail {

template <int D, typename TOut, bool PAGED>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int BLK = KB * D;                // bf16 elements per K (or V) block
  constexpr int NLD = BLK * 2 / 1024;        // 1-KB DMA writes per operand block (8 or 4)
  constexpr int RPW = 32 / NLD;              // block rows per write (4 or 8)
  constexpr int CPR = D / 8;                 // 16-byte chunks per row (16 or 8)
  __shared__ __attribute__((aligned(16))) __bf16 smem[NST * 2 * BLK];      // [stage][K, V][BLK]

  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int r32 = lane & 31;
  const int w = blockIdx.x;
  const int G = p.group;
  const int Hkv = p.heads_kv;

  // ---- plan: stream length and this wave's range [r0, r1). The lanes read
  // the lengths (clamped as seq_len does) and the wave combines them, rather
  // than one chain of scalar loads per batch.
  int64_t T = 0;
  for (int bb = lane; bb < p.batch; bb += 64) T += min(max(p.seqlens[bb], 0), p.max_seqlen);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) T += __shfl_xor(T, off);
  T = uniform64(T) * Hkv;
  const int64_t P = range_tokens(p, T);
  const int64_t r0 = (int64_t)w * P;
  if (r0 >= T) return;
  const int64_t r1 = r0 + P < T ? r0 + P : T;

  Cursor cur;                                // slab holding r0: the first batch whose tokens end past r0
  {
    int64_t off = 0;                         // stream offset of batch b's first token
    int b = 0;
    int64_t base = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
      const int bb = c0 + lane;
      const int64_t n = bb < p.batch ? (int64_t)min(max(p.seqlens[bb], 0), p.max_seqlen) * Hkv : 0;
      int64_t incl = n;                      // inclusive prefix over this chunk
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t t = __shfl_up(incl, d);
        incl += lane >= d ? t : 0;
      }
      const uint64_t hit = __builtin_amdgcn_ballot_w64(bb < p.batch && r0 < base + incl);
      if (hit != 0) {
        const int first = __builtin_ctzll(hit);
        b = c0 + first;
        off = base + __shfl(incl - n, first);
        break;
      }
      base += __shfl(incl, 63);
    }
    b = __builtin_amdgcn_readfirstlane(b);
    off = uniform64(off);
    const int L = seq_len(p, b);
    const int kvh = (int)((r0 - off) / L);
    cur.b = b;
    cur.kvh = kvh;
    cur.slab_off = off + (int64_t)kvh * L;
    cur.start = (int)(r0 - cur.slab_off);
    cur.pos = cur.start / KB * KB;
    cur.end = (int)min((int64_t)L, r1 - cur.slab_off);
  }
  // one block further along the range; false once it is exhausted
  auto advance = [&](Cursor& c) -> bool {
    c.pos += KB;
    if (c.pos < c.end) return true;
    if (c.slab_off + c.end >= r1) return false;
    int L = seq_len(p, c.b);
    c.slab_off += L;
    if (++c.kvh == Hkv) {                      // next non-empty sequence
      c.kvh = 0;
      do {
        ++c.b;
        L = seq_len(p, c.b);
      } while (L == 0);
    }
    c.pos = 0;
    c.start = 0;
    c.end = (int)min((int64_t)L, r1 - c.slab_off);
    return true;
  };

  // ---- DMA of one block: NLD 1-KB writes per operand, rows past the piece clamped
  const int drow = lane / CPR;                 // row of the lane's chunk, + RPW per write
  const int dchunk = lane % CPR;
  // byte offsets of the lane's K and V chunks in write i, from the block's
  // first row (whole blocks: contiguous, or page-aligned paged)
  // (32-bit: usable while 32 rows of the row or slot stride stay below 2^31 bytes)
  const bool lane_ok = p.kv_stride[2] < (int64_t(1) << 25);
  const bool fast_pages = PAGED && lane_ok && (p.page_size == 16 || p.page_size % KB == 0);
  uint32_t lane_k[NLD], lane_v[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int r = RPW * i + drow;
    lane_k[i] = (uint32_t)(2 * ((int64_t)r * p.kv_stride[2] + 8 * (dchunk ^ kswz_d<D>(r))));
    lane_v[i] = (uint32_t)(2 * ((int64_t)r * p.kv_stride[2] + 8 * (dchunk ^ vswz_d<D>(r))));
  }
  // Paged cache: table entries of the block at cursor c (scalar loads through
  // the constant address space; ids outside [0, num_pages) are clamped).
  auto pages_of = [&](const Cursor& c) {
    PageRun pr{};
    if constexpr (PAGED) {
      const int ps = p.page_size;
      const int pg0 = c.pos / ps;
      pr.off = c.pos - pg0 * ps;
      pr.lim = c.end - 1 - pg0 * ps;
      // pages past the piece's last key are not looked up (their entries may be stale)
      const int n1 = pr.lim >= ps ? 1 : 0, n2 = pr.lim >= 2 * ps ? 2 : n1;
      const const_i32* bt = (const const_i32*)p.block_table + (int64_t)c.b * p.max_blocks + pg0;
      pr.e0 = bt[0];
      pr.e1 = bt[n1];
      pr.e2 = bt[n2];
    }
    return pr;
  };
  auto issue = [&](const Cursor& c, int st, const PageRun& pr) {
    const __bf16* kp = reinterpret_cast<const __bf16*>(p.k);
    const __bf16* vp = reinterpret_cast<const __bf16*>(p.v);
    __bf16* dst = smem + st * 2 * BLK;
    if constexpr (PAGED) {
      if (fast_pages && c.pos + KB <= c.end) {
        // a whole, page-aligned block: rows 0-15 and 16-31 sit in pages e0 and
        // e1 (16-slot pages), or all in e0 from slot off (pages of 32k slots);
        // each load is a wave-uniform base plus the lane's precomputed offset.
        // A piece's last block takes the clamped path below: a masked key has
        // weight 0, but 0 times a never-written V slot can still be NaN.
        const int top = p.num_pages - 1;
        const int64_t hofs = (int64_t)c.kvh * p.kv_stride[1];
        const int rs = (int)p.kv_stride[2];
        const char* b0 = reinterpret_cast<const char*>(
            kp + (int64_t)min(max(pr.e0, 0), top) * p.kv_stride[0] + hofs + (p.page_size == 16 ? 0 : pr.off * rs));
        const char* b1 = p.page_size == 16
            ? reinterpret_cast<const char*>(kp + (int64_t)min(max(pr.e1, 0), top) * p.kv_stride[0] + hofs) - 32 * rs
            : b0;
        asm("" : "+s"(b0), "+s"(b1));
        const intptr_t dvk = reinterpret_cast<intptr_t>(vp) - reinterpret_cast<intptr_t>(kp);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const char* base = i < NLD / 2 ? b0 : b1;
          __builtin_amdgcn_global_load_lds((const void*)(base + lane_k[i]), (lds_void*)(dst + i * 512), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(base + dvk + lane_v[i]), (lds_void*)(dst + BLK + i * 512),
                                           16, 0, 0);
        }
        return;
      }
      // wave-uniform (page, kv head) bases of the block's pages; each lane then
      // picks its row's page with two compares and adds slot * row stride
      // (32-bit: page_size * stride < 2^31 is checked on the host)
      const int ps = p.page_size;
      const int top = p.num_pages - 1;
      const int64_t hofs = (int64_t)c.kvh * p.kv_stride[1];
      const __bf16* k0 = kp + (int64_t)min(max(pr.e0, 0), top) * p.kv_stride[0] + hofs;
      const __bf16* k1 = kp + (int64_t)min(max(pr.e1, 0), top) * p.kv_stride[0] + hofs;
      const __bf16* k2 = kp + (int64_t)min(max(pr.e2, 0), top) * p.kv_stride[0] + hofs;
      // opaque to the optimiser, which would otherwise select the raw entries
      // per lane and redo the clamp and the 64-bit products in vector registers
      asm("" : "+s"(k0), "+s"(k1), "+s"(k2));
      const intptr_t dvk = reinterpret_cast<intptr_t>(vp) - reinterpret_cast<intptr_t>(kp);
      const int rs = (int)p.kv_stride[2];
      const int o = pr.off + drow;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int r = RPW * i + drow;
        const int kr = min(o + RPW * i, pr.lim);           // slot counted from the first page
        const bool c1 = kr >= ps, c2 = kr >= 2 * ps;
        int slot = c1 ? kr - ps : kr;
        slot = c2 ? slot - ps : slot;
        const __bf16* row = (c2 ? k2 : c1 ? k1 : k0) + (uint32_t)(slot * rs);
        const __bf16* vrow = reinterpret_cast<const __bf16*>(reinterpret_cast<intptr_t>(row) + dvk);
        __builtin_amdgcn_global_load_lds((const void*)(row + 8 * (dchunk ^ kswz_d<D>(r))), (lds_void*)(dst + i * 512),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vrow + 8 * (dchunk ^ vswz_d<D>(r))),
                                         (lds_void*)(dst + BLK + i * 512), 16, 0, 0);
      }
    } else {
      if (lane_ok && c.pos + KB <= c.end) {    // a whole block: a uniform base plus the lane offsets
        const char* b0 = reinterpret_cast<const char*>(
            kp + (int64_t)c.b * p.kv_stride[0] + (int64_t)c.kvh * p.kv_stride[1] + (int64_t)c.pos * p.kv_stride[2]);
        asm("" : "+s"(b0));
        const intptr_t dvk = reinterpret_cast<intptr_t>(vp) - reinterpret_cast<intptr_t>(kp);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          __builtin_amdgcn_global_load_lds((const void*)(b0 + lane_k[i]), (lds_void*)(dst + i * 512), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(b0 + dvk + lane_v[i]), (lds_void*)(dst + BLK + i * 512), 16,
                                           0, 0);
        }
        return;
      }
      const int64_t base = (int64_t)c.b * p.kv_stride[0] + (int64_t)c.kvh * p.kv_stride[1];
      const int last = c.end - 1;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int r = RPW * i + drow;
        const int64_t row = base + (int64_t)min(c.pos + r, last) * p.kv_stride[2];
        __builtin_amdgcn_global_load_lds((const void*)(kp + row + 8 * (dchunk ^ kswz_d<D>(r))),
                                         (lds_void*)(dst + i * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vp + row + 8 * (dchunk ^ vswz_d<D>(r))),
                                         (lds_void*)(dst + BLK + i * 512), 16, 0, 0);
      }
    }
  };

  // ---- lane-constant fragment offsets (elements)
  int koff[KSTEPS];
  {
    const int r = sigma32(r32);
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc) koff[kc] = r * D + 8 * ((2 * kc + half) ^ kswz_d<D>(r));
  }
  int voff[DBLK];
  {
    const int gg = lane >> 4, i = lane & 15;
    const int r = 8 * (gg >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = 32 * db + 16 * (gg & 1) + 4 * (i & 3);
      voff[db] = r * D + 8 * ((col >> 3) ^ vswz_d<D>(r)) + (col & 7);
    }
  }

  const float c2 = p.scale_log2;
  bf16x8 qf[KSTEPS];
  int q_b = -1, q_kvh = -1;
  float m_run = kNegInf, l_run = 0.f, l_o = 0.f;
  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};

  // prologue: NST-1 blocks in flight
  Cursor dma = cur;
  PageRun dma_pages = pages_of(dma);
  bool dma_ok = true;
  int issued = 0;
  for (int s = 0; s < NST - 1 && dma_ok; ++s) {
    issue(dma, s, dma_pages);
    ++issued;
    dma_ok = advance(dma);
    if (dma_ok) dma_pages = pages_of(dma);
  }

  for (int blk = 0;; ++blk) {
    const int st = blk % NST;
    if (dma_ok) {                              // refill the stage block blk-1 used
      issue(dma, (blk + NST - 1) % NST, dma_pages);
      ++issued;
      dma_ok = advance(dma);
      if (dma_ok) dma_pages = pages_of(dma); // table entries for the next issue
    }
    const int ahead = issued - blk - 1;        // blocks allowed to stay in flight
    if (ahead >= 3) wait_vmcnt<6 * NLD>();
    else if (ahead == 2) wait_vmcnt<4 * NLD>();
    else if (ahead == 1) wait_vmcnt<2 * NLD>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);

    if (cur.b != q_b || cur.kvh != q_kvh) {    // this slab's queries as B operands
      q_b = cur.b;
      q_kvh = cur.kvh;
      const __bf16* qp = reinterpret_cast<const __bf16*>(p.q) + ((int64_t)q_b * p.heads_q + q_kvh * G + r32) * D;
#pragma unroll
      for (int kc = 0; kc < KSTEPS; ++kc)
        qf[kc] = as_bf16x8(r32 < G ? load16(qp + 16 * kc + 8 * half) : u32x4{0, 0, 0, 0});
    }

    const __bf16* ks = smem + st * 2 * BLK;
    const __bf16* vs = ks + BLK;
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kc = 0; kc < KSTEPS; ++kc)
      sc = mfma32(*reinterpret_cast<const bf16x8*>(ks + koff[kc]), qf[kc], sc);
    const int valid = cur.end - cur.pos;       // keys of this block inside the piece: [lo, valid)
    const int lo = cur.start - cur.pos;
    if (valid < KB || lo > 0) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int kk = acc_key(jj, half);
        sc[jj] = ((kk >= valid) | (kk < lo)) ? kNegInf : sc[jj];
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = fmaxf(mx, sc[jj]);
    const float mt = half_swap_max(mx) * c2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
      l_run *= alpha;
      l_o *= alpha;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const float pv = fast_exp2(fmaf(sc[jj], c2, -m_use));
      sc[jj] = pv;
      rs += pv;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[0][e] = (__bf16)sc[e];
      pb[1][e] = (__bf16)sc[8 + e];
    }
    float ro = 0.f;
    const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2 pr;
        pr[0] = pb[c][2 * e];
        pr[1] = pb[c][2 * e + 1];
        ro = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ro, false);
      }
    l_run += half_swap_sum(rs);
    l_o += half_swap_sum(ro);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const __bf16* va = vs + voff[db] + 16 * c * D;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(va + 4 * D));
        o[db] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[c], o[db]);
      }

    // end of a piece: its partial for the G heads goes to index slab + w
    if (cur.pos + KB >= cur.end) {
      const int slab = cur.b * Hkv + cur.kvh;
      if (r32 < G) {
        const int64_t part = (int64_t)(slab + w) * G + r32;
        const float inv = 1.f / l_o;           // l_o >= 1: the piece holds a key
        float* po = p.part_o + part * D;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int d = 32 * db + 8 * gq + 4 * half;
            *reinterpret_cast<f32x4*>(po + d) = f32x4{o[db][4 * gq] * inv, o[db][4 * gq + 1] * inv,
                                                      o[db][4 * gq + 2] * inv, o[db][4 * gq + 3] * inv};
          }
        if (half == 0) p.part_lse[part] = (m_run + __log2f(l_run)) * kLn2;
      }
      m_run = kNegInf;
      l_run = 0.f;
      l_o = 0.f;
#pragma unroll
      for (int i = 0; i < DBLK; ++i) o[i] = f32x16{};
    }
    wait_lgkm0();                              // this stage's reads are done before it is refilled
    __builtin_amdgcn_sched_barrier(0);
    if (!advance(cur)) break;
  }
}

// One wave per (b, query head): LSE = log sum_s exp(lse_s), O = sum_s
// exp(lse_s - LSE) o_s over the pieces s of the head's slab.
template <int D, typename TOut>
__global__ __launch_bounds__(256) void decode_merge_kernel(const DecodeParams p) {
  constexpr int EPL = D / 64;                  // output elements per lane (2 or 1)
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)p.batch * p.heads_q) return;
  const int b = (int)(row / p.heads_q);
  const int hq = (int)(row % p.heads_q);
  const int G = p.group;
  const int kvh = hq / G, g = hq % G;
  // stream length and this row's slab offset: the lanes read the lengths
  // (clamped as seq_len does) and the wave adds them up, rather than one
  // chain of scalar loads per batch
  int64_t T = 0, before = 0;
  for (int bb = lane; bb < p.batch; bb += 64) {
    const int64_t n = min(max(p.seqlens[bb], 0), p.max_seqlen);
    T += n;
    before += bb < b ? n : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    T += __shfl_xor(T, off);
    before += __shfl_xor(before, off);
  }
  T = uniform64(T) * p.heads_kv;
  before = uniform64(before);
  const int L = seq_len(p, b);
  TOut* op = reinterpret_cast<TOut*>(p.o) + row * D + EPL * lane;
  if (L == 0) {                                // no key: O = 0, LSE = -inf
#pragma unroll
    for (int e = 0; e < EPL; ++e) op[e] = (TOut)0.f;
    if (p.lse != nullptr && lane == 0) p.lse[row] = kNegInf;
    return;
  }
  const int64_t P = range_tokens(p, T);
  const int64_t slab_off = before * p.heads_kv + (int64_t)kvh * L;
  const int w0 = (int)(slab_off / P), w1 = (int)((slab_off + L - 1) / P);
  const int slab = b * p.heads_kv + kvh;
  float mx = kNegInf;
  for (int w = w0; w <= w1; ++w) mx = fmaxf(mx, p.part_lse[(int64_t)(slab + w) * G + g]);
  float den = 0.f, n[EPL] = {};
  for (int w = w0; w <= w1; ++w) {
    const int64_t part = (int64_t)(slab + w) * G + g;
    const float wt = __expf(p.part_lse[part] - mx);
    const float* v = p.part_o + part * D + EPL * lane;
    den += wt;
#pragma unroll
    for (int e = 0; e < EPL; ++e) n[e] = fmaf(wt, v[e], n[e]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int e = 0; e < EPL; ++e) op[e] = (TOut)(n[e] * inv);
  if (p.lse != nullptr && lane == 0) p.lse[row] = mx + __logf(den);
}

}  // namespace detail

namespace {

template <int D, typename TOut>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  if (p.block_table != nullptr)
    hipLaunchKernelGGL((detail::decode_split_kernel<D, TOut, true>), dim3((unsigned)p.n_waves), dim3(64), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((detail::decode_split_kernel<D, TOut, false>), dim3((unsigned)p.n_waves), dim3(64), 0, stream,
                       p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.batch * p.heads_q;
  hipLaunchKernelGGL((detail::decode_merge_kernel<D, TOut>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace

int decode_waves() { return 256 * FA_DEC_WPC; }

// Static workspace of fa_decode_noalloc: the split kernel's partials live in
// this file-scope device array instead of a caller's buffer. Every GPU the
// library runs on holds its own copy (at its own address) until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: the device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is passed on.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(void** ptr) {
  static std::atomic<uintptr_t> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  uintptr_t a = addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    a = reinterpret_cast<uintptr_t>(p);
    addr[dev].store(a, std::memory_order_release);     // a racing first call stores the same address
  }
  *ptr = reinterpret_cast<void*>(a);
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.head_dim == 64) return p.out_fp32 ? launch_t<64, float>(p, stream) : launch_t<64, __bf16>(p, stream);
  return p.out_fp32 ? launch_t<128, float>(p, stream) : launch_t<128, __bf16>(p, stream);
}

}  // namespace fa
