// FP8 (e4m3) prefill with incoherent processing, for head_dim 128 on gfx950
// ("FlashAttention Explained: IO-Aware Attention, Tiling, Online Softmax and
// FP8 on Hopper", section "FP8 Attention and Incoherent Processing").
//
// Quantiser. Q and K rows are multiplied by diag(s) H / sqrt(128) (random
// signs s, Sylvester Hadamard H; a fast Walsh-Hadamard transform: sixteen
// lanes hold a row, eight values each, butterflies of distance 1, 2, 4 inside
// a lane and 8 .. 64 across lanes by shuffles) and quantised to OCP e4m3 with
// one float32 scale per block of rows (128 query rows, 64 keys): codes =
// e4m3(x * 448 / amax), scale = amax / 448. V keeps its values and gets one
// scale per kv head; it is stored transposed, [d][key], with the keys of each
// 64-key tile permuted into the order in which one lane of the attention
// kernel holds its row's probabilities, so the P V operand is two 16-byte
// reads.
//
// Attention. The tile loop of the bf16 kernels on v_mfma_scale_f32_32x32x64
// _f8f6f4 (block scales fixed at 1): S^T = K Q^T for 64-key tiles as two
// 32-key blocks of two k-steps, the softmax in float32 with the tile's
// q-scale x k-scale folded into the one FMA per score, and O^T += V^T P^T
// with P quantised to e4m3 as 2^8 * 2^(x - m) against an integer base m that
// moves with the row maximum (one FMA and one exponential per score; every
// rescale is an exact power of two and every weight keeps three mantissa bits
// down to 2^-14 of the largest). O is divided by the sum of the quantised
// weights (one more, smaller MFMA against a lane-selected operand of ones)
// and multiplied by V's scale; the LSE uses the float32 sum. Each wave
// issues the score MFMAs of tile j+1 before the softmax of tile j, so the
// matrix cores run during
// the vector work; tiles arrive through a four-stage LDS ring.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

namespace {

constexpr int D8 = 128;      // head dim
constexpr int QB = 128;      // query rows per scale block (and per attention workgroup)
constexpr int KT = 64;       // keys per scale block and per tile
constexpr int ST8 = 4;       // K/V tile ring depth (two tiles in flight beyond the two in use)
constexpr int VROWS = 256;   // V rows per workgroup of the head maximum

#ifndef FA_FP8_WPE
#define FA_FP8_WPE 2         // waves per SIMD the attention kernel is register-limited to
#endif
#ifndef FA_FP8_NW
#define FA_FP8_NW 4          // waves (32 query rows each) per attention workgroup
#endif

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void8;
// per-tile scales are read at wave-uniform addresses through the constant
// address space (scalar loads), so they never wait on the DMA's counter
typedef __attribute__((address_space(4))) const float const_f32;

// two floats (already within +-448) to e4m3 bytes in the low or high half of w
template <bool HI>
__device__ __forceinline__ int pack2(float a, float b, int w) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, HI);
}
template <bool B> struct bool_c { static constexpr bool value = B; };
__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.f), 448.f); }

// position of key kappa (0..63) of a tile in the transposed V storage: the
// attention kernel's lane of half h holds, in byte b, the probability of key
// 8(b%16/4) + 4h + b%4 + 32(b/16); the storage puts that key at 32h + b
__device__ __forceinline__ int vpos(int kappa) {
  const int blk = kappa >> 5, r = kappa & 31;
  const int h = (r >> 2) & 1, bb = ((r >> 3) << 2) | (r & 3);
  return 32 * h + 16 * blk + bb;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) x = fmaxf(x, __shfl_xor(x, w, 64));
  return x;
}

}  // namespace

namespace detail {

// Rotate and quantise one block of ROWS rows of Q or K: grid (blocks, heads, batch).
template <int ROWS>
__global__ __launch_bounds__(256) void fp8_quant_qk_kernel(const Fp8QuantParams p, int which) {
  constexpr int PASSES = ROWS / 16;          // 16 rows per pass, 16 lanes per row
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 15, rsub = tid >> 4;   // lane's 8-value chunk, row within the pass
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = p.seqlen;
  if (which == 0 && blk == 0 && h == 0 && b == 0)     // V's maximum accumulates here next
    for (int i = tid; i < p.batch * p.heads_kv; i += 256) p.v_scale[i] = 0.f;
  const __bf16* src = reinterpret_cast<const __bf16*>(which == 0 ? p.q : p.k);
  const int64_t* st = which == 0 ? p.q_stride : p.kv_stride;
  const int heads = which == 0 ? p.heads_q : p.heads_kv;
  src += (int64_t)b * st[0] + (int64_t)h * st[1];

  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = p.signs != nullptr ? p.signs[8 * c + e] : 1.f;
  const float inv_sqrt_d = 0.08838834764831845f;

  float x[PASSES][8];
  float amax = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = blk * ROWS + ps * 16 + rsub;
    const bool ok = row < n;
    const bf16x8 v = as_bf16x8(ok ? load16(src + (int64_t)row * st[2] + 8 * c) : u32x4{0, 0, 0, 0});
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (float)v[e] * sg[e];
    if (p.signs != nullptr) {
      // butterflies inside the lane: distance 1, 2, 4
#pragma unroll
      for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & hh) == 0) {
            const float a = y[e], bb = y[e + hh];
            y[e] = a + bb;
            y[e + hh] = a - bb;
          }
      // across lanes: distance 8, 16, 32, 64 = lane distance 1, 2, 4, 8
#pragma unroll
      for (int lh = 1; lh < 16; lh <<= 1) {
        const bool upper = (c & lh) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float other = __shfl_xor(y[e], lh, 64);
          y[e] = upper ? other - y[e] : y[e] + other;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= inv_sqrt_d;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[ps][e] = ok ? y[e] : 0.f;
      amax = fmaxf(amax, fabsf(x[ps][e]));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float safe = amax > 0.f ? amax : 448.f;
  const float inv = 448.f / safe;
  float* scale = which == 0 ? p.q_scale : p.k_scale;
  const int nblk = (n + ROWS - 1) / ROWS;
  if (tid == 0) scale[((int64_t)b * heads + h) * nblk + blk] = safe / 448.f;
  uint8_t* dst = reinterpret_cast<uint8_t*>(which == 0 ? p.q8 : p.k8) + ((int64_t)b * heads + h) * n * D8;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int row = blk * ROWS + ps * 16 + rsub;
    if (row >= n) continue;
    int w0 = pack2<false>(clamp448(x[ps][0] * inv), clamp448(x[ps][1] * inv), 0);
    w0 = pack2<true>(clamp448(x[ps][2] * inv), clamp448(x[ps][3] * inv), w0);
    int w1 = pack2<false>(clamp448(x[ps][4] * inv), clamp448(x[ps][5] * inv), 0);
    w1 = pack2<true>(clamp448(x[ps][6] * inv), clamp448(x[ps][7] * inv), w1);
    *reinterpret_cast<u32x2*>(dst + (int64_t)row * D8 + 8 * c) = u32x2{(uint32_t)w0, (uint32_t)w1};
  }
}

// V has one scale per kv head, so its quantisation runs in three steps:
// the head's absolute maximum (fp8_v_amax_kernel, by atomics on the bit
// pattern of v_scale: non-negative floats order as unsigned integers; the
// first workgroup of the Q quantiser, earlier on the stream, zeroes v_scale),
// the codes (fp8_quant_v_kernel, one workgroup per 64-key tile), and the
// maximum turned into the scale (fp8_v_scale_kernel).
__global__ __launch_bounds__(256) void fp8_v_amax_kernel(const Fp8QuantParams p) {
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = tid & 15, rsub = tid >> 4;   // 16 lanes per row, 8 values each
  const int r0 = blockIdx.x * VROWS, h = blockIdx.y, b = blockIdx.z;
  const int n = p.seqlen;
  const __bf16* src = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride[0] + (int64_t)h * p.kv_stride[1];
  float amax = 0.f;
#pragma unroll 4
  for (int ps = 0; ps < VROWS / 16; ++ps) {
    const int row = r0 + ps * 16 + rsub;
    if (row < n) {
      const bf16x8 v = as_bf16x8(load16(src + (int64_t)row * p.kv_stride[2] + 8 * c));
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
    }
  }
  amax = wave_max(amax);
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  if (tid == 0) {
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax(reinterpret_cast<unsigned*>(p.v_scale) + (int64_t)b * p.heads_kv + h, __float_as_uint(amax));
  }
}

// One 64-key tile of one kv head of V into the transposed, key-permuted
// layout; v_scale holds the head's absolute maximum.
__global__ __launch_bounds__(256) void fp8_quant_v_kernel(const Fp8QuantParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[D8 * KT];     // [d][position]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * KT, h = blockIdx.y, b = blockIdx.z;
  const int n = p.seqlen, npad = (n + KT - 1) / KT * KT;
  const __bf16* src = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride[0] + (int64_t)h * p.kv_stride[1];
  const int c = tid & 15, rsub = tid >> 4;   // 16 lanes per row, 8 values each

  const float amax = p.v_scale[(int64_t)b * p.heads_kv + h];
  const float safe = amax > 0.f ? amax : 448.f;
  const float inv = 448.f / safe;

  uint8_t* dst = reinterpret_cast<uint8_t*>(p.v8t) + ((int64_t)b * p.heads_kv + h) * D8 * npad;
#pragma unroll
  for (int ps = 0; ps < KT / 16; ++ps) {
    const int kappa = ps * 16 + rsub, row = t0 + kappa;
    const bf16x8 v = as_bf16x8(row < n ? load16(src + (int64_t)row * p.kv_stride[2] + 8 * c) : u32x4{0, 0, 0, 0});
    const int pos = vpos(kappa);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int w = pack2<false>(clamp448((float)v[e] * inv), clamp448((float)v[e + 1] * inv), 0);
      tile[(8 * c + e) * KT + pos] = (uint8_t)(w & 0xff);
      tile[(8 * c + e + 1) * KT + pos] = (uint8_t)((w >> 8) & 0xff);
    }
  }
  __syncthreads();
  // 128 rows x 64 bytes out: 16 bytes per thread, two rounds
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i, d = idx >> 2, ch = idx & 3;
    *reinterpret_cast<u32x4*>(dst + (int64_t)d * npad + t0 + 16 * ch) =
        *reinterpret_cast<const u32x4*>(tile + d * KT + 16 * ch);
  }
}

__global__ __launch_bounds__(256) void fp8_v_scale_kernel(const Fp8QuantParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < p.batch * p.heads_kv) {
    const float amax = p.v_scale[i];
    p.v_scale[i] = (amax > 0.f ? amax : 448.f) / 448.f;
  }
}

// Attention on the quantised operands: FA_FP8_NW waves x 32 query rows per workgroup.
template <typename TOut>
__global__ __launch_bounds__(64 * FA_FP8_NW) __attribute__((amdgpu_waves_per_eu(FA_FP8_WPE, FA_FP8_WPE)))
void fwd_fp8_kernel(const Fp8FwdParams p) {
  constexpr int NW = FA_FP8_NW, BRW = 32 * NW, TILEB = KT * D8;   // bytes per K (or V^T) tile
  constexpr int LPW = 8 / NW;                // 1-KB DMA writes per wave per operand tile
  static_assert(8 % NW == 0, "");
  __shared__ __attribute__((aligned(16))) uint8_t smem[ST8 * 2 * TILEB];  // [stage][K, V^T][8 KB]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5, r32 = lane & 31;
  // one instance serves both masks: the flag is uniform, and the loop keeps one register allocation
  const bool causal = p.causal;
  const int n = p.seqlen, npad = (n + KT - 1) / KT * KT;
  const int nqt = (n + BRW - 1) / BRW;
  // Causal: in dispatch order every head's heaviest query tile first, then
  // every head's next one, so long workgroups start first and short ones
  // fill in behind them. When the kv groups come in whole rounds of 8, the
  // heads of one kv group go to one XCD (workgroups are dealt to the 8 XCDs
  // round-robin) and share its L2.
  int t, bh;
  if (causal) {
    const int nh = p.batch * p.heads_q, nkv = p.batch * p.heads_kv;
    t = blockIdx.x / nh;
    bh = blockIdx.x - t * nh;
    if (nkv % 8 == 0) {
      const int x = bh & 7, sl = bh >> 3;
      const int kg = x + 8 * (sl / p.group);
      bh = kg * p.group + sl % p.group;
    }
  } else {
    t = blockIdx.x % nqt;
    bh = blockIdx.x / nqt;
  }
  const int hq = bh % p.heads_q, b = bh / p.heads_q;
  const int kvh = hq / p.group;
  const int qt = causal ? nqt - 1 - t : t;   // heavy tiles first
  const int q0 = qt * BRW, wrow0 = q0 + wave * 32, row = wrow0 + r32;
  const int kv_end = causal ? min(n, q0 + BRW) : n;
  const int ntiles = (kv_end + KT - 1) / KT;
  const int nt_w = causal ? min(ntiles, (wrow0 + 31) / KT + 1) : ntiles;

  const uint8_t* kp = reinterpret_cast<const uint8_t*>(p.k8) + ((int64_t)b * p.heads_kv + kvh) * n * D8;
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(p.v8t) + ((int64_t)b * p.heads_kv + kvh) * D8 * npad;
  const const_f32* ksc = (const const_f32*)p.k_scale + ((int64_t)b * p.heads_kv + kvh) * (npad / KT);
  const float qs = p.q_scale[((int64_t)b * p.heads_q + hq) * ((n + QB - 1) / QB) + wrow0 / QB];
  const float vs = p.v_scale[(int64_t)b * p.heads_kv + kvh];

  // DMA: a tile is 8 K writes and 8 V^T writes of 1 KB; wave w issues LPW of each.
  // K: write i covers rows 8i..8i+7 (16-byte chunk lane%8 of row 8i + lane/8);
  // V^T: write i covers d rows 16i..16i+15 (chunk lane%4 of row 16i + lane/4).
  // The global chunk is XOR-swizzled by the row, so reads below XOR back.
  // The patterns keep the 16-lane row reads conflict-free on 64 banks x 4
  // bytes: K rows are 128 bytes (two per 256-byte bank line), so the 8 even
  // and the 8 odd rows of a read each need 8 distinct patterns: (kr / 2) % 8.
  // V^T rows are 64 bytes (four per line): rows d, d+4, d+8, d+12 need 4
  // distinct patterns: (d / 4) % 4.
  // lane offsets of its chunks from the tile's first key (K) and first position (V^T)
  int koff[LPW];
  int64_t voff[LPW];
#pragma unroll
  for (int i2 = 0; i2 < LPW; ++i2) {
    const int i = LPW * wave + i2;
    const int kr = 8 * i + (lane >> 3), kc = lane & 7;
    koff[i2] = kr * D8 + 16 * (kc ^ ((kr >> 1) & 7));
    const int d = 16 * i + (lane >> 2), vc = lane & 3;
    voff[i2] = (int64_t)d * npad + 16 * (vc ^ ((d >> 2) & 3));
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // LDS destinations stay scalar
  auto issue = [&](int tile, int stg) {
    const int kv0 = tile * KT;
    const uint8_t* vb = vp + kv0;            // V^T is zero-padded to npad positions: no clamp
    const bool whole = kv0 + KT <= n;        // else the last keys repeat key n-1
    const uint8_t* kb = kp + (int64_t)kv0 * D8;
#pragma unroll
    for (int i2 = 0; i2 < LPW; ++i2) {
      const int i = LPW * wave_u + i2;
      const uint8_t* ka = kb + koff[i2];
      if (!whole) {
        const int kr = 8 * i + (lane >> 3), kc = lane & 7;
        ka = kp + (int64_t)min(kv0 + kr, n - 1) * D8 + 16 * (kc ^ ((kr >> 1) & 7));
      }
      __builtin_amdgcn_global_load_lds((const void*)ka, (lds_void8*)(smem + stg * 2 * TILEB + i * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vb + voff[i2]),
                                       (lds_void8*)(smem + stg * 2 * TILEB + TILEB + i * 1024), 16, 0, 0);
    }
  };

  // this lane's query row as B operands: bytes 64 ks + 32 half .. +31
  i32x8 qf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q8) + (((int64_t)b * p.heads_q + hq) * n + row) * D8 + 64 * ks + 32 * half;
    const u32x4 a = row < n ? *reinterpret_cast<const u32x4*>(qp) : u32x4{0, 0, 0, 0};
    const u32x4 c = row < n ? *reinterpret_cast<const u32x4*>(qp + 16) : u32x4{0, 0, 0, 0};
    qf[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }
  // Weight sums on v_mfma_scale_f32_16x16x128_f8f6f4. Read as its B operand,
  // the P^T register of lane l (row l % 32, keys 32 (l / 32) ..) is column
  // l % 16 of k-group l / 16: groups 0 and 2 hold rows 0-15, groups 1 and 3
  // rows 16-31. The e4m3 A operand is 1.0 (0x38) where the parity of the
  // k-group matches bit 2 of the A row m = l % 16, else 0: output row m then
  // sums row (column) + 16 ((m / 4) & 1), so all four accumulator registers
  // of lane l (rows 4 (l / 16) .. +3) hold its own row's sum. The sum of a
  // tile's e4m3 weights (multiples of 2^-9 below 2^15) is exact in float32.
  const int sel1 = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;
  const i32x8 ones = {sel1, sel1, sel1, sel1, sel1, sel1, sel1, sel1};

  const float c2 = p.scale_log2 * qs;
  float m_run = kNegInf, l_run = 0.f;
  i32x8 pf = {};                             // this tile's e4m3 weights (B operand of O^T += V^T P^T)
  f32x16 o[4];
  f32x4 ls = f32x4{};                        // the last tile's sum of e4m3 weights, every register
  float l8 = 0.f;                            // sum of e4m3 weights of the earlier tiles
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};

  // S^T tile = K Q^T for the 64 keys of a tile: block blk holds keys 32 blk .. +31
  auto scores = [&](int tile, f32x16 (&s)[2]) {
    const uint8_t* ks_ = smem + (tile % ST8) * 2 * TILEB;
    // all four A fragments are read first, and the two accumulation chains
    // alternate, so no product waits for the one before it
    i32x8 af[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const int kr = 32 * blk + r32;       // key row of this lane's A fragment
        const int c0 = 4 * ks + 2 * half;
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks_ + kr * D8 + 16 * (c0 ^ ((kr >> 1) & 7)));
        const u32x4 c = *reinterpret_cast<const u32x4*>(ks_ + kr * D8 + 16 * ((c0 + 1) ^ ((kr >> 1) & 7)));
        af[ks][blk] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
      }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      s[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[0][blk], qf[0], f32x16{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
      s[blk] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[1][blk], qf[1], s[blk], 0, 0, 0, 127, 0, 127);
  };
  // every wave has waited for its own loads of tiles j and j+1; the barrier
  // publishes them and frees the stage of tile j-1 (its K was read two steps
  // ago, its V one step ago), which takes tile j+ST8-1
  auto sync_tile = [&](int j) {
    if (j + 2 < ntiles) __builtin_amdgcn_s_waitcnt((2 * LPW) | (7 << 4) | (15 << 8));   // tile j+2 may fly
    else __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (j + ST8 - 1 < ntiles) issue(j + ST8 - 1, (j + ST8 - 1) % ST8);
  };
  auto softmax_pv = [&](auto edge_c, int j, f32x16 (&sc)[2], float ce) {
    constexpr bool EDGE = decltype(edge_c)::value;   // the tile holds masked keys
    const uint8_t* vs_ = smem + (j % ST8) * 2 * TILEB + TILEB;
    const int kv0 = j * KT;
    // softmax: register jj of block blk holds key kv0 + 32 blk + 8(jj/4) + 4 half + jj%4.
    // The maximum is taken on the raw scores (the tile's scale ce is positive),
    // and one FMA per score both scales and subtracts the base; the base is
    // lowered by 8 so the weights come out as 2^8 * 2^(x - m), ready for e4m3.
    l8 += ls[0];                             // the previous tile's weights, at the current base
    // a key is visible when key <= lim; relative to this lane's first key of the tile
    const int rel = (causal ? min(row, n - 1) : n - 1) - kv0 - 4 * half;
    float x[2][16];
    float mq[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        x[blk][jj] = sc[blk][jj];
        if (EDGE) x[blk][jj] = 32 * blk + 8 * (jj >> 2) + (jj & 3) > rel ? kNegInf : x[blk][jj];
        mq[(2 * blk + (jj >> 3)) & 3] = fmaxf(mq[(2 * blk + (jj >> 3)) & 3], x[blk][jj]);
      }
    const float mt = half_swap_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * ce;
    if (__builtin_amdgcn_ballot_w64(mt > m_run)) {      // integer base: every rescale is a power of two
      const float m_new = mt > m_run ? ceilf(mt) : m_run;
      const float alpha = m_run == kNegInf ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
      l8 *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float mb = (m_run == kNegInf ? 0.f : m_run) - 8.f;
    float rq[4];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int bidx = 4 * w + e;                      // byte b: block b/16, register b%16
        pr[e] = fast_exp2(fmaf(x[bidx >> 4][bidx & 15], ce, -mb));    // <= 2^8
        rq[e] = w == 0 ? pr[e] : rq[e] + pr[e];
      }
      // both halves of the word are rewritten: the previous tile's word is only a placeholder
      pf[w] = pack2<true>(pr[2], pr[3], pack2<false>(pr[0], pr[1], pf[w]));
    }
    l_run += half_swap_sum((rq[0] + rq[1]) + (rq[2] + rq[3]));   // in units of 2^-8
    // O^T += V^T P^T: lane (d = 32 db + lane % 32, half) reads positions 32 half .. +31 of row d
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + r32, sw = (d >> 2) & 3;
      const u32x4 a = *reinterpret_cast<const u32x4*>(vs_ + d * KT + 16 * ((2 * half) ^ sw));
      const u32x4 c = *reinterpret_cast<const u32x4*>(vs_ + d * KT + 16 * ((2 * half + 1) ^ sw));
      const i32x8 af = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
      o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, pf, o[db], 0, 0, 0, 127, 0, 127);
    }
    ls = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf, f32x4{}, 0, 0, 0, 127, 0, 127);
  };

  // Software pipeline: step j issues the score MFMAs of tile j+1, which run on
  // the matrix cores while the vector unit takes tile j's softmax.
  for (int i = 0; i < ST8 - 1; ++i)
    if (i < ntiles) issue(i, i);
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  __syncthreads();
  f32x16 sa[2], sb[2];
  scores(0, sa);                             // every wave has at least one tile
  // the key scale of tile j is read one step ahead, so its scalar load is
  // not waited for at the start of the tile's softmax
  float ks_cur = ksc[0], ks_nxt = 0.f;
  auto step = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    sync_tile(j);
    if (j + 1 < nt_w) scores(j + 1, nxt);
    // this tile's scale (its load landed a step ago) is taken before the next
    // one is requested: scalar loads return out of order, so a wait for one
    // is a wait for all
    float ce = c2 * ks_cur;
    asm volatile("" : "+v"(ce));
    __builtin_amdgcn_sched_barrier(0);
    ks_nxt = ksc[min(j + 1, ntiles - 1)];   // lands during the softmax
    if (j < nt_w) {                          // later tiles are wholly in this wave's future
      const int kv0 = j * KT;
      if ((causal && kv0 + KT - 1 > wrow0) || kv0 + KT > n) softmax_pv(bool_c<true>{}, j, cur, ce);
      else softmax_pv(bool_c<false>{}, j, cur, ce);
    }
    ks_cur = ks_nxt;
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(j, sa, sb);
    if (j + 1 < ntiles) step(j + 1, sb, sa);
  }
  l8 += ls[0];

  const float inv_l = l8 > 0.f ? vs / l8 : 0.f;
  TOut* op = reinterpret_cast<TOut*>(p.o) + (((int64_t)b * p.heads_q + hq) * n + row) * D8;
  if constexpr (sizeof(TOut) == 2) {
    // lanes l and l ^ 32 hold 4-column halves of the same 8 columns of a row:
    // one swap per dword gives each lane 8 consecutive columns
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t w[2][2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int gq = 2 * m + c;
          bf16x2 a, bb;
          a[0] = (__bf16)(o[db][4 * gq] * inv_l); a[1] = (__bf16)(o[db][4 * gq + 1] * inv_l);
          bb[0] = (__bf16)(o[db][4 * gq + 2] * inv_l); bb[1] = (__bf16)(o[db][4 * gq + 3] * inv_l);
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
        if (row < n) *reinterpret_cast<u32x4*>(op + 32 * db + 16 * m + 8 * half) = out;
      }
  }
  if (row < n) {
    if constexpr (sizeof(TOut) == 4) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = 32 * db + 8 * gq + 4 * half;
          const float v0 = o[db][4 * gq] * inv_l, v1 = o[db][4 * gq + 1] * inv_l;
          const float v2 = o[db][4 * gq + 2] * inv_l, v3 = o[db][4 * gq + 3] * inv_l;
          *reinterpret_cast<f32x4*>(op + d) = f32x4{v0, v1, v2, v3};
        }
    }
    if (p.lse != nullptr && half == 0)
      p.lse[((int64_t)b * p.heads_q + hq) * n + row] = l_run > 0.f ? (m_run + __log2f(l_run) - 8.f) * kLn2 : kNegInf;
  }
}

}  // namespace detail

hipError_t launch_fp8_quant(const Fp8QuantParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((detail::fp8_quant_qk_kernel<QB>),
                     dim3((unsigned)((p.seqlen + QB - 1) / QB), (unsigned)p.heads_q, (unsigned)p.batch), dim3(256), 0,
                     stream, p, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((detail::fp8_quant_qk_kernel<KT>),
                     dim3((unsigned)((p.seqlen + KT - 1) / KT), (unsigned)p.heads_kv, (unsigned)p.batch), dim3(256), 0,
                     stream, p, 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(detail::fp8_v_amax_kernel,
                     dim3((unsigned)((p.seqlen + VROWS - 1) / VROWS), (unsigned)p.heads_kv, (unsigned)p.batch), dim3(256),
                     0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(detail::fp8_quant_v_kernel,
                     dim3((unsigned)((p.seqlen + KT - 1) / KT), (unsigned)p.heads_kv, (unsigned)p.batch), dim3(256), 0,
                     stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(detail::fp8_v_scale_kernel, dim3((unsigned)((p.batch * p.heads_kv + 255) / 256)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  const int64_t wgs = (int64_t)p.batch * p.heads_q * ((p.seqlen + 32 * FA_FP8_NW - 1) / (32 * FA_FP8_NW));
  if (p.out_fp32) hipLaunchKernelGGL((detail::fwd_fp8_kernel<float>), dim3((unsigned)wgs), dim3(64 * FA_FP8_NW), 0, stream, p);
  else hipLaunchKernelGGL((detail::fwd_fp8_kernel<__bf16>), dim3((unsigned)wgs), dim3(64 * FA_FP8_NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
