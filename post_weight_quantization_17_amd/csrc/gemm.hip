// Running a quantized layer on token batches: Y = act(X What^T).
//
// xuzou.cn reading card of the GPTQ paper, section 计算设置: the model is
// quantized one block at a time and the quantized block is run on the
// calibration tokens to produce the next block's inputs; section 方法适配
// (last paragraph): the quantized matrix is multiplied with dequantization on
// the fly. What = s (code - z) per group (astro-blog survey, section 1.2),
// held as fp16 to run: the fp32 product s (code - z), rounded to fp16.
//
// Two forms: the fused kernel below (no workspace; the weights are
// dequantized inside the product, tile by tile) and, further down, a
// two-pass form for large token batches that takes a caller workspace.
//
// Fused design (gfx950), one workgroup of 8 waves (two per SIMD) per 256-token x
// 128-weight-row output tile, K (d_in) in tiles of 64:
//  * X tiles [256 tokens][64] fp16 move straight from HBM into LDS
//    (global_load_lds, 16 bytes per lane) in three stages, the tile for
//    K step kt + 2 in flight while step kt runs; 16-byte chunk c of row r
//    sits at slot c ^ (r & 7), so the fragment reads of 32 consecutive rows
//    fall on distinct banks.
//  * d_in must be a multiple of 32; in a last K tile of 32 columns the
//    chunks past d_in re-read chunks 0-3 of the same tile, and the weights
//    they meet are zero (nothing past d_in is read).
//  * W tiles are cut from the packed words: the 256 units of a K tile (128
//    rows x 2 units of 32 codes; bits words of one row hold exactly 32
//    codes) are split in halves of 16 codes over waves 0-3 and 4-7; each
//    forms s (c - z) in fp32, rounds it to fp16 and stores the halfs into
//    the LDS tile [128 rows][64] (row pitch 72 halfs), double-buffered.
//  * Each wave computes 64 tokens x 64 rows with v_mfma_f32_32x32x16_f16
//    (2 x 2 tiles): A fragments are 8 consecutive K of one token, B
//    fragments 8 consecutive K of one weight row, both 16-byte LDS reads.
//  * Epilogue: optional ReLU on the fp32 sum, then round to fp16.
// fp16 x fp16 products are exact in fp32; the sums are fp32 (MFMA order).
#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int G_BM = 256;          // tokens per tile
constexpr int G_BN = 128;          // weight rows per tile
constexpr int G_BK = 64;           // K per tile
constexpr int G_P = G_BK + 8;      // LDS row pitch (halfs)
constexpr int G_THREADS = 512;      // 8 waves, two per SIMD
constexpr int G_XS = 3;            // X stages in LDS

// Code j (0..31) of a unit of BITS words: bits [BITS j, BITS j + BITS) of
// the unit's LSB-first stream.
template <int BITS, int J>
__device__ __forceinline__ uint32_t unit_field(const uint32_t (&w)[BITS]) {
  constexpr int p = BITS * J, wi = p / 32, off = p % 32;
  if constexpr (off + BITS <= 32) {
    return __builtin_amdgcn_ubfe(w[wi], off, BITS);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], off) & ((1u << BITS) - 1u);
  }
}

// fp16 bits of s (c - z): c - z formed exactly in fp32 (2^23 + c, minus
// 2^23 + z), the product rounded to fp32, then to fp16. The empty asm keeps
// the product a value of its own: fused into the conversion it would be
// rounded once.
__device__ __forceinline__ uint32_t dq_half(uint32_t c, float s, float zoff) {
  float k = __uint_as_float(0x4B000000u | c) - zoff;
  float prod = s * k;
  asm volatile("" : "+v"(prod));
  return uint32_t(__half_as_ushort(__float2half_rn(prod)));
}

template <int BITS, int J>
__device__ __forceinline__ uint32_t dq_pair(const uint32_t (&w)[BITS], float s, float zoff) {
  return dq_half(unit_field<BITS, J>(w), s, zoff) | (dq_half(unit_field<BITS, J + 1>(w), s, zoff) << 16);
}

// Codes H * 16 + 2 i, + 1 (i < 8) of a unit, as 8 pairs of fp16 bits.
template <int BITS, int H, int I = 0>
__device__ __forceinline__ void half_unit_pairs(const uint32_t (&w)[BITS], float s, float zoff, uint32_t (&h)[8]) {
  if constexpr (I < 8) {
    h[I] = dq_pair<BITS, 16 * H + 2 * I>(w, s, zoff);
    half_unit_pairs<BITS, H, I + 1>(w, s, zoff, h);
  }
}

template <int BITS>
__global__ void __launch_bounds__(G_THREADS, 1)
dequant_gemm_f16(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                 const int32_t* __restrict__ zeros, int d_out, int d_in, int nwords, int group, int ngroups,
                 const __half* __restrict__ X, int64_t n_tok, int64_t ldx, __half* __restrict__ Y, int64_t ldy,
                 int relu, int n_tiles_n, int n_tiles_m8) {
  // X: G_XS stages of [256 rows][128 bytes], 16-byte chunk c of row r at
  // slot c ^ (r & 7) (the fragment reads of 32 consecutive rows then spread
  // over the banks). W: two stages of the dequantized tile, row pitch G_P.
  __shared__ __attribute__((aligned(16))) unsigned char xs[G_XS][G_BM * 128];
  __shared__ __attribute__((aligned(16))) _Float16 ws0[G_BN * G_P];
  __shared__ __attribute__((aligned(16))) _Float16 ws1[G_BN * G_P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: tokens 64 wm .., rows 64 wn ..
  // Workgroups go to the 8 XCDs round-robin (b % 8). When the token tiles
  // split evenly, XCD x takes token tiles x, x + 8, ..., each across all
  // weight tiles in turn, so the X tile its CUs share stays in its own L2;
  // otherwise consecutive workgroups share the token tile.
  int tn;
  int64_t tm;
  const unsigned b = blockIdx.x;
  if (n_tiles_m8) {
    const unsigned j = b >> 3;
    tm = int64_t(j / unsigned(n_tiles_n)) * 8 + (b & 7);
    tn = int(j % unsigned(n_tiles_n));
  } else {
    tn = int(b % unsigned(n_tiles_n));
    tm = int64_t(b / unsigned(n_tiles_n));
  }
  const int64_t m0 = tm * G_BM;
  const int n0 = tn * G_BN;
  const int nkt = (d_in + G_BK - 1) / G_BK;  // d_in % 32 == 0: the last tile may hold 32 columns

  // Direct X loads: instruction i of wave w fills rows 8 (w + 8 i) .. + 7 of
  // a stage (1 KB); lane l brings row 8 (w + 8 i) + l / 8, logical chunk
  // (l % 8) ^ (row & 7), which lands in slot l % 8.
  constexpr int XL = G_BM * 128 / (16 * G_THREADS);  // direct loads per thread per tile
  const __half* xsrc[XL];
  int xchunk[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int r = 8 * (wave + 8 * i) + (lane >> 3);
    int64_t t = m0 + r;
    if (t >= n_tok) t = n_tok - 1;  // clamped rows are computed and never stored
    xchunk[i] = (lane & 7) ^ (r & 7);
    xsrc[i] = X + t * ldx + 8 * xchunk[i];
  }
  auto issue_x = [&](int kt, int st) {
    const int k0 = kt * G_BK;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      // In a last tile of 32 columns, chunks past d_in re-read chunks 0-3 of
      // the row (their weights are zero, so they add nothing).
      const int kc = k0 + 8 * xchunk[i] < d_in ? k0 : k0 - 32;
      __builtin_amdgcn_global_load_lds(xsrc[i] + kc,
                                       (__attribute__((address_space(3))) void*)(xs[st] + 1024 * (wave + 8 * i)), 16,
                                       0, 0);
    }
  };
  // Dequantization: the 256 units of a K tile (row wr, unit wu) are split in
  // halves of 16 codes; waves 0-3 take the first halves, waves 4-7 the second
  // (wave-uniform, so the bit offsets are compile-time constants).
  const int uidx = tid & 255, hh = wave >> 2;
  const int wr = uidx >> 1, wu = uidx & 1;
  const int wrow = n0 + wr < d_out ? n0 + wr : d_out - 1;
  const uint32_t* prow = packed + size_t(wrow) * nwords;
  const float* srow = scales + size_t(wrow) * ngroups;
  const int32_t* zrow = zeros + size_t(wrow) * ngroups;
  struct Unit {
    uint32_t w[BITS];
    float s, zoff;
  };
  auto load_unit = [&](int kt, Unit& u) {
    const int k0 = kt * G_BK;
    const bool in = k0 + 32 * wu < d_in;  // the second unit of a last 32-column tile is zero
    const int unit = (k0 >> 5) + (in ? wu : 0);
#pragma unroll
    for (int b = 0; b < BITS; ++b) u.w[b] = prow[unit * BITS + b];
    const int g = group > 0 ? (32 * unit) / group : 0;
    u.s = in ? srow[g] : 0.f;
    u.zoff = 8388608.f + float(zrow[g]);
  };
  auto store_unit = [&](const Unit& u, _Float16* wst) {
    uint32_t h[8];
    if (hh == 0)
      half_unit_pairs<BITS, 0>(u.w, u.s, u.zoff, h);
    else
      half_unit_pairs<BITS, 1>(u.w, u.s, u.zoff, h);
    _Float16* wd = wst + wr * G_P + 32 * wu + 16 * hh;
    *reinterpret_cast<uint4*>(wd) = make_uint4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<uint4*>(wd + 8) = make_uint4(h[4], h[5], h[6], h[7]);
  };

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{0};

  // fragment reads: lane l takes row l % 32 of its 32-row tile and logical
  // chunk l / 32 + 2 kk of the K tile (8 consecutive K)
  const int fr = lane & 31, fh = lane >> 5;
  auto mma = [&](int st, const _Float16* wst) {
    const unsigned char* xa = xs[st];
    const _Float16* wb = wst + (wn * 64 + fr) * G_P + 8 * fh;
#pragma unroll
    for (int kk = 0; kk < G_BK / 16; ++kk) {
      half8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + fr;
        a[i] = *reinterpret_cast<const half8*>(xa + r * 128 + 16 * ((fh + 2 * kk) ^ (r & 7)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const half8*>(wb + 32 * j * G_P + 16 * kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  // Schedule (per thread, VMEM ops in issue order): prologue W(0) X(0) W(1)
  // X(1); iteration kt issues W(kt+2) then X(kt+2) after its barrier. So at
  // iteration kt the XL most recent VMEM ops are X(kt+1)'s: vmcnt(XL) means
  // X(kt) (and W(kt+1)) have landed. Loads past the last tile re-load the
  // last tile (valid memory, never read), so the count is the same every time.
  static_assert(XL == 4, "the wait below encodes vmcnt(4)");
  Unit ua, ub;
  load_unit(0, ua);
  issue_x(0, 0);
  load_unit(nkt > 1 ? 1 : 0, ub);
  issue_x(nkt > 1 ? 1 : 0, 1 % G_XS);
  store_unit(ua, ws0);
  auto step = [&](int kt, Unit& use, Unit& next, _Float16* wcur, _Float16* wnext) {
    __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) expcnt(7) lgkmcnt(0): X(kt) landed, own LDS writes done
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int kn = kt + 2 < nkt ? kt + 2 : nkt - 1;
    load_unit(kn, next);
    issue_x(kn, (kt + 2) % G_XS);
    mma(kt % G_XS, wcur);
    store_unit(use, wnext);  // tile kt + 1 (a last duplicate is written and never read)
  };
  int kt = 0;
  for (; kt + 2 <= nkt; kt += 2) {
    step(kt, ub, ua, ws0, ws1);
    step(kt + 1, ua, ub, ws1, ws0);
  }
  if (kt < nkt) step(kt, ub, ua, ws0, ws1);
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no direct load outlives the workgroup's LDS

  // 32x32 result layout: lane l holds column l % 32 (a weight row) and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 (tokens) of register r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + 32 * j + fr;
      if (col >= d_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * fh + (r & 3);
        if (t >= n_tok) continue;
        float v = acc[i][j][r];
        if (relu) v = v > 0.f ? v : 0.f;
        Y[t * ldy + col] = __float2half_rn(v);
      }
    }
}


// An accumulator's value, read out of its AGPR where it is used. Left to
// itself the compiler copies all 256 accumulators to VGPRs at once after the
// main loop, which does not fit beside the live values.
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Buffer resource over [base, base + bytes): stores past the end are dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// ---------------------------------------------------------------------------
// Two-pass form for compute-bound batches (a caller workspace is given and
// d_in is a multiple of 128). The fused kernel above rebuilds each weight
// tile for every 256-token tile; with the 128 x 128 wave tiles the MFMA rate
// needs (one wave per SIMD) that rebuild does not hide behind the MFMAs, so
// here the weights are dequantized once per call. Both operands are laid out
// K-major in the workspace, so the product runs the Hessian's pipeline
// (direct-to-LDS loads, transposing LDS reads, one barrier per 32 K):
//   kmajor_transpose_f16:  X [n][d_in] -> XK [d_in][ldk]   (tokens >= n: 0)
//   dequant_kmajor_f16:    packed -> WK [d_in][ldw] = fp16(s (c - z))
//                          (rows >= d_out: 0), the same rounding as above
//   gemm_kmajor_f16:       Y[t][r] = act(sum_k XK[k][t] WK[k][r])
// ---------------------------------------------------------------------------
constexpr int K_T = 256;                   // tile edge (weight rows and tokens)
constexpr int K_BK = 32;                   // K per LDS stage
constexpr int K_NSTAGE = 4;
constexpr int K_PITCH = 1088;              // one slot pair: K rows k and k + 16, 512 bytes each, 64-byte pad
constexpr int K_PANEL = 16 * K_PITCH;
constexpr int K_STAGE = 2 * K_PANEL;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4v lds_short4;

// Two transposing reads (ds_read_b64_tr_b16): lanes 4r .. 4r + 3 of each
// 16-lane group fetch K row r of a 4 x 16 block; lane i receives column i's
// 4 values. Together: 8 K values of one column (MFMA operand layout).
__device__ __forceinline__ half8 kfrag(const unsigned char* lds, int off) {
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off + 4 * K_PITCH));
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(half8, v);
}

// 128 tokens x 64 channels per workgroup through LDS, 16-byte global reads
// and writes: XK[c][t] = X[t][c] for t < n, 0 for n <= t < ldk. Needs X
// 16-byte aligned with ldx % 8 == 0, d_in % 64 == 0 and ldk % 128 == 0.
__global__ void __launch_bounds__(256)
kmajor_transpose_f16(const __half* __restrict__ X, int64_t n, int d_in, int64_t ldx, __half* __restrict__ XK,
                     int64_t ldk) {
  __shared__ __attribute__((aligned(16))) unsigned short t[128][72];
  const int64_t t0 = int64_t(blockIdx.x) * 128;
  const int c0 = int(blockIdx.y) * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 256 * k, r = idx >> 3, q = idx & 7;  // token r, channels 8q .. 8q + 7
    const int64_t tok = t0 + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok < n) v = *reinterpret_cast<const uint4*>(X + tok * ldx + c0 + 8 * q);
    *reinterpret_cast<uint4*>(&t[r][8 * q]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = tid + 256 * k, c = idx & 63, p = idx >> 6;  // channel c, tokens 8p .. 8p + 7
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = uint32_t(t[8 * p + 2 * i][c]) | (uint32_t(t[8 * p + 2 * i + 1][c]) << 16);
    *reinterpret_cast<uint4*>(XK + int64_t(c0 + c) * ldk + t0 + 8 * p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// 64 weight rows x 64 codes per workgroup: WK[k][r] = fp16(s (c - z)), the
// fp32 product rounded to fp16 (dq_half above), 0 for d_out <= r < ldw.
template <int BITS>
__global__ void __launch_bounds__(256)
dequant_kmajor_f16(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                   const int32_t* __restrict__ zeros, int d_out, int d_in, int nwords, int units_per_group,
                   int ngroups, __half* __restrict__ WK, int ldw) {
  __shared__ unsigned short t[64][66];
  const int r0 = int(blockIdx.x) * 64, k0 = int(blockIdx.y) * 64;  // k0: two 32-code units
  const int tid = threadIdx.x;
  {
    // thread: row r0 + tid / 4, codes 16 (tid % 4) .. + 15 of the 64
    const int rr = tid >> 2, part = tid & 3;
    const int row = r0 + rr;
    const int unit = (k0 >> 5) + (part >> 1);
    unsigned short h[16];
    if (row < d_out && 32 * unit < d_in) {
      uint32_t w[BITS];
#pragma unroll
      for (int b = 0; b < BITS; ++b) w[b] = packed[size_t(row) * nwords + size_t(unit) * BITS + b];
      const int g = unit / units_per_group;
      const float sc = scales[size_t(row) * ngroups + g];
      const float zoff = 8388608.f + float(zeros[size_t(row) * ngroups + g]);
      uint32_t pr[8];
      if (part & 1) {
        pr[0] = dq_pair<BITS, 16>(w, sc, zoff); pr[1] = dq_pair<BITS, 18>(w, sc, zoff);
        pr[2] = dq_pair<BITS, 20>(w, sc, zoff); pr[3] = dq_pair<BITS, 22>(w, sc, zoff);
        pr[4] = dq_pair<BITS, 24>(w, sc, zoff); pr[5] = dq_pair<BITS, 26>(w, sc, zoff);
        pr[6] = dq_pair<BITS, 28>(w, sc, zoff); pr[7] = dq_pair<BITS, 30>(w, sc, zoff);
      } else {
        pr[0] = dq_pair<BITS, 0>(w, sc, zoff); pr[1] = dq_pair<BITS, 2>(w, sc, zoff);
        pr[2] = dq_pair<BITS, 4>(w, sc, zoff); pr[3] = dq_pair<BITS, 6>(w, sc, zoff);
        pr[4] = dq_pair<BITS, 8>(w, sc, zoff); pr[5] = dq_pair<BITS, 10>(w, sc, zoff);
        pr[6] = dq_pair<BITS, 12>(w, sc, zoff); pr[7] = dq_pair<BITS, 14>(w, sc, zoff);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[2 * e] = (unsigned short)(pr[e] & 0xffffu);
        h[2 * e + 1] = (unsigned short)(pr[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) h[e] = 0;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) t[rr][16 * part + e] = h[e];
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) {
    const int k = e >> 6, r = e & 63;  // code k, row r (rows contiguous)
    if (k0 + k < d_in && r0 + r < ldw) WK[int64_t(k0 + k) * ldw + r0 + r] = __ushort_as_half(t[r][k]);
  }
}

// Y[t][r] = act(sum_k XK[k][t] WK[k][r]) for one 256-row x 256-token tile per
// workgroup (4 waves, each 128 rows x 128 tokens on v_mfma_f32_32x32x16_f16),
// K in stages of 32 moved straight into LDS, four stages, one barrier per
// stage: the schedule of the Hessian's interior kernel, with the weight rows
// as its first panel and the tokens as its second. ldw, ldk are multiples of
// 256 (whole tiles; the padding holds zeros) and nk = d_in / 32 is a multiple
// of 4.
__global__ void __launch_bounds__(256, 1)
gemm_kmajor_f16(const __half* __restrict__ WK, int64_t ldw, const __half* __restrict__ XK, int64_t ldk, int nk,
                int d_out, int64_t n_tok, __half* __restrict__ Y, int64_t ldy, int relu, int vec_store,
                int n_tiles_n, int n_tiles_m8) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[K_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[K_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[K_STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds3[K_STAGE];

  // Work order. Workgroups go to the 8 XCDs round-robin (b % 8), 32 at a
  // time per XCD (one per CU). When the token tiles divide into 64, XCD x
  // takes token tiles x, x + 8, ... in blocks of 8, and walks each block
  // across the weight tiles 4 at a time: the 32 workgroups an XCD runs
  // together share 8 token panels and 4 weight panels in its L2 (12 panels
  // for 32 tiles, against 33 when one token tile meets 32 weight tiles).
  // Otherwise XCD x takes token tiles x, x + 8, ... each across all weight
  // tiles (as the fused kernel), or consecutive workgroups share a token tile.
  int tn;
  int64_t tm;
  const unsigned b = blockIdx.x;
  if (n_tiles_m8 == 2) {
    const unsigned j = b >> 3, x = b & 7, nt = unsigned(n_tiles_n);
    const unsigned tb = j / (8u * nt), rem = j % (8u * nt);  // token block, place in it
    const unsigned full = nt / 4u;                            // whole blocks of 4 weight tiles
    unsigned tl, wn;
    if (rem < 32u * full) {
      wn = (rem / 32u) * 4u + (rem % 4u);
      tl = tb * 8u + (rem % 32u) / 4u;
    } else {
      const unsigned w = nt - 4u * full, r2 = rem - 32u * full;  // the last, narrower block
      wn = 4u * full + r2 % w;
      tl = tb * 8u + r2 / w;
    }
    tm = int64_t(tl) * 8 + x;
    tn = int(wn);
  } else if (n_tiles_m8) {
    const unsigned j = b >> 3;
    tm = int64_t(j / unsigned(n_tiles_n)) * 8 + (b & 7);
    tn = int(j % unsigned(n_tiles_n));
  } else {
    tn = int(b % unsigned(n_tiles_n));
    tm = int64_t(b / unsigned(n_tiles_n));
  }
  const int I0 = tn * K_T;                 // weight rows
  const int64_t J0 = tm * K_T;             // tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Each wave issues 8 direct loads per stage: slot pairs wave + 4 (u % 4) of
  // the weight panel (u < 4) and of the token panel (u >= 4). A load fills
  // one slot pair: lanes 0-31 K row (pair), lanes 32-63 K row (pair + 16),
  // 8 columns per lane. Offsets are in elements from the stage's K base.
  uint32_t voff[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pair = wave + 4 * (u & 3);
    const int64_t ld = u < 4 ? ldw : ldk;
    const int64_t c0 = u < 4 ? int64_t(I0) : J0;
    voff[u] = uint32_t((pair + 16 * (lane >> 5)) * ld + 8 * (lane & 31));
    (void)c0;
  }
  const __half* wbase = WK + I0;
  const __half* xbase = XK + J0;
  auto issue = [&](int step, unsigned char* buf) {
    const __half* ws = wbase + int64_t(step) * K_BK * ldw;
    const __half* xs = xbase + int64_t(step) * K_BK * ldk;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pair = wave + 4 * (u & 3);
      unsigned char* l = buf + (u >> 2) * K_PANEL + pair * K_PITCH;
      __builtin_amdgcn_global_load_lds((u < 4 ? ws : xs) + voff[u], (__attribute__((address_space(3))) void*)l, 16,
                                       0, 0);
    }
  };

  // Per-lane base of the transposing fragment reads: 16-lane group g covers
  // 16 columns (16 * (g & 1) ..) for K rows 8 * (g >> 1) + [0, 4); within the
  // group lane 4r + q reads K row r, columns 4q .. 4q + 3.
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int lane_off = (8 * (g >> 1) + r) * K_PITCH + 2 * (16 * (g & 1) + 4 * q);
  const int a_base = lane_off + 2 * (wm * 128);
  const int b_base = K_PANEL + lane_off + 2 * (wn * 128);

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{0};

  half8 fa0[4], fb0[4], fa1[4], fb1[4];  // fragments: first / last 16 K of a stage
  auto read_frags = [&](const unsigned char* base, int kk, half8* fa, half8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = kfrag(base, a_base + 64 * i + 512 * kk);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = kfrag(base, b_base + 64 * j + 512 * kk);
  };
  auto mfma16 = [&](const half8* fa, const half8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // One stage s in two MFMA groups of 16 around one barrier (see the
  // Hessian's interior kernel): group A runs the first 16 K while the loads
  // of stage s + 3 and the reads of the last 16 K go out; after the barrier
  // (stage s + 1 landed for every wave, every wave done reading stage s - 1)
  // group B runs the last 16 K while the first 16 K of stage s + 1 are read.
  // Loads past the last stage re-load the last stage (valid memory, never
  // read), so the load count per stage, and with it the vmcnt, is constant.
  auto step = [&](int s, unsigned char* cur, unsigned char* next, unsigned char* later) {
    issue(s + 3 < nk ? s + 3 : nk - 1, later);
    read_frags(cur, 1, fa1, fb1);
    mfma16(fa0, fb0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // direct load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x4070);  // vmcnt(16) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(next, 0, fa0, fb0);
    mfma16(fa1, fb1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, lds0);
  issue(1 < nk ? 1 : nk - 1, lds1);
  issue(2 < nk ? 2 : nk - 1, lds2);
  __builtin_amdgcn_s_waitcnt(0x4070);  // stage 0 landed (vmcnt 16)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_frags(lds0, 0, fa0, fb0);
  for (int s = 0; s < nk; s += K_NSTAGE) {
    step(s, lds0, lds1, lds3);
    step(s + 1, lds1, lds2, lds0);
    step(s + 2, lds2, lds3, lds1);
    step(s + 3, lds3, lds0, lds2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0): no direct load outlives the workgroup's LDS

  // 32x32 result layout: lane l holds column l % 32 (a token) and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 (weight rows) of register r: each lane
  // stores 4 consecutive outputs of one token. Stores go through a buffer
  // resource over this tile's token rows (tokens past n_tok fall outside and
  // are dropped), so the epilogue has no per-lane branches.
  const int64_t rows_here = n_tok - J0 < K_T ? n_tok - J0 : K_T;
  const rsrc_t yr = make_rsrc(Y + J0 * ldy, uint32_t(rows_here * ldy * 2));
  const bool full = vec_store && I0 + K_T <= d_out;
  constexpr uint32_t OUT = 0x80000000u;  // an offset past the resource: dropped
  const int fr = lane & 31;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t rowoff = uint32_t(128 * wn + 32 * j + fr) * uint32_t(ldy) * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        __builtin_amdgcn_sched_barrier(0);
        const int col = I0 + 128 * wm + 32 * i + 8 * qq + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc_read(acc[i][j][4 * qq + e]);
          if (relu) v[e] = v[e] > 0.f ? v[e] : 0.f;
        }
        const __half2 lo = __float22half2_rn(make_float2(v[0], v[1]));
        const __half2 hi = __float22half2_rn(make_float2(v[2], v[3]));
        const uint32_t plo = *reinterpret_cast<const uint32_t*>(&lo), phi = *reinterpret_cast<const uint32_t*>(&hi);
        if (full) {
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{plo, phi}, yr, rowoff + 2u * uint32_t(col), 0, 0);
        } else {
          const uint32_t h[4] = {plo & 0xffffu, plo >> 16, phi & 0xffffu, phi >> 16};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)h[e], yr,
                                                  col + e < d_out ? rowoff + 2u * uint32_t(col + e) : OUT, 0, 0);
        }
      }
  }
}

}  // namespace
}  // namespace gptq

using namespace gptq;

namespace {
// Two-pass plan: padded leading dimensions and workspace bytes.
struct KPlan {
  int64_t ldw, ldk;
  size_t wk_bytes, xk_bytes, ws_bytes;
};
KPlan plan_kmajor(int64_t d_out, int64_t d_in, int64_t n_tokens) {
  KPlan p{};
  p.ldw = (d_out + K_T - 1) / K_T * K_T;
  p.ldk = (n_tokens + K_T - 1) / K_T * K_T;
  p.wk_bytes = align_up(size_t(d_in) * size_t(p.ldw) * 2, 256);
  p.xk_bytes = align_up(size_t(d_in) * size_t(p.ldk) * 2, 256);
  p.ws_bytes = p.wk_bytes + p.xk_bytes;
  return p;
}
// The two-pass form takes whole 128-K blocks and offsets that fit its
// 32-bit per-lane load offsets, 16-bit grid rows and 32-bit store offsets.
bool kmajor_ok(int64_t d_out, int64_t d_in, int64_t n_tokens, int64_t ldy) {
  const KPlan p = plan_kmajor(d_out, d_in, n_tokens);
  return d_in % (K_BK * K_NSTAGE) == 0 && d_in / 64 <= 65535 && p.ldw < (int64_t(1) << 26) &&
         p.ldk < (int64_t(1) << 26) && ldy <= (int64_t(1) << 21) &&
         (p.ldw / K_T) * (p.ldk / K_T) < (int64_t(1) << 31);
}
}  // namespace

extern "C" size_t gptq_dequant_gemm_workspace_size(int64_t d_out, int64_t d_in, int64_t n_tokens) {
  if (d_out < 1 || d_in < 1 || n_tokens < 0) return 0;
  return plan_kmajor(d_out, d_in, n_tokens).ws_bytes;
}

extern "C" int gptq_dequant_gemm(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_out,
                                 int64_t d_in, int bits, int64_t group_size, const void* X, int64_t n_tokens,
                                 int64_t ldx, void* Y, int64_t ldy, int relu, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (d_out < 1 || d_in < 1 || n_tokens < 0 || d_out > (int64_t(1) << 30) || d_in > (1 << 24)) return GPTQ_E_INVALID_ARG;
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 8)) return GPTQ_E_INVALID_ARG;
  if (group_size != -1 && group_size < 1) return GPTQ_E_INVALID_ARG;
  if (relu != 0 && relu != 1) return GPTQ_E_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  if (!packed || !scales || !zeros || !X || !Y || ldx < d_in || ldy < d_out) return GPTQ_E_INVALID_ARG;
  // K tiles of 64 columns (the last may hold 32), one group per 32-code
  // unit, 16-byte X rows.
  if (d_in % 32 != 0 || (group_size != -1 && group_size % G_BK != 0)) return GPTQ_E_UNSUPPORTED;
  if (ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0) return GPTQ_E_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (ws != nullptr) {
    const KPlan kp = plan_kmajor(d_out, d_in, n_tokens);
    if (ws_bytes < kp.ws_bytes) return GPTQ_E_WORKSPACE;
    if (kmajor_ok(d_out, d_in, n_tokens, ldy)) {
      const int nwords = int((d_in * bits + 31) / 32);
      const int ngroups = group_size == -1 ? 1 : int((d_in + group_size - 1) / group_size);
      const int upg = group_size == -1 ? (1 << 30) : int(group_size / 32);
      __half* WK = static_cast<__half*>(ws);
      __half* XK = reinterpret_cast<__half*>(static_cast<unsigned char*>(ws) + kp.wk_bytes);
      const dim3 gd(unsigned(kp.ldw / 64), unsigned((d_in + 63) / 64));
      switch (bits) {
        case 2:
          hipLaunchKernelGGL(dequant_kmajor_f16<2>, gd, dim3(256), 0, s, packed, scales, zeros, int(d_out), int(d_in),
                             nwords, upg, ngroups, WK, int(kp.ldw));
          break;
        case 3:
          hipLaunchKernelGGL(dequant_kmajor_f16<3>, gd, dim3(256), 0, s, packed, scales, zeros, int(d_out), int(d_in),
                             nwords, upg, ngroups, WK, int(kp.ldw));
          break;
        case 4:
          hipLaunchKernelGGL(dequant_kmajor_f16<4>, gd, dim3(256), 0, s, packed, scales, zeros, int(d_out), int(d_in),
                             nwords, upg, ngroups, WK, int(kp.ldw));
          break;
        default:
          hipLaunchKernelGGL(dequant_kmajor_f16<8>, gd, dim3(256), 0, s, packed, scales, zeros, int(d_out), int(d_in),
                             nwords, upg, ngroups, WK, int(kp.ldw));
          break;
      }
      if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
      hipLaunchKernelGGL(kmajor_transpose_f16, dim3(unsigned(kp.ldk / 128), unsigned(d_in / 64)), dim3(256), 0,
                         s, static_cast<const __half*>(X), n_tokens, int(d_in), ldx, XK, kp.ldk);
      if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
      const int64_t km = kp.ldk / K_T, kn = kp.ldw / K_T;
      const int vec = (reinterpret_cast<uintptr_t>(Y) % 8 == 0 && ldy % 4 == 0) ? 1 : 0;
      hipLaunchKernelGGL(gemm_kmajor_f16, dim3(unsigned(km * kn)), dim3(256), 0, s, WK, kp.ldw, XK, kp.ldk,
                         int(d_in / K_BK), int(d_out), n_tokens, static_cast<__half*>(Y), ldy, relu, vec, int(kn),
                         km % 64 == 0 ? 2 : (km % 8 == 0 ? 1 : 0));
      return launch_status();
    }
  }
  const int64_t tiles_m = (n_tokens + G_BM - 1) / G_BM, tiles_n = (d_out + G_BN - 1) / G_BN;
  if (tiles_m * tiles_n > (int64_t(1) << 31)) return GPTQ_E_INVALID_ARG;
  const int nwords = int((d_in * bits + 31) / 32);
  const int ngroups = group_size == -1 ? 1 : int((d_in + group_size - 1) / group_size);
  const dim3 grid(unsigned(tiles_m * tiles_n)), block(G_THREADS);
  const int m8 = tiles_m % 8 == 0 ? 1 : 0;
  const __half* x = static_cast<const __half*>(X);
  __half* y = static_cast<__half*>(Y);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(dequant_gemm_f16<2>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n), m8);
      break;
    case 3:
      hipLaunchKernelGGL(dequant_gemm_f16<3>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n), m8);
      break;
    case 4:
      hipLaunchKernelGGL(dequant_gemm_f16<4>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n), m8);
      break;
    default:
      hipLaunchKernelGGL(dequant_gemm_f16<8>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n), m8);
      break;
  }
  return launch_status();
}
