// Running a quantized layer on token batches: Y = act(X What^T).
//
// xuzou.cn reading card of the GPTQ paper, section 计算设置: the model is
// quantized one block at a time and the quantized block is run on the
// calibration tokens to produce the next block's inputs; section 方法适配
// (last paragraph): the quantized matrix is multiplied with dequantization on
// the fly. What = s (code - z) per group (astro-blog survey, section 1.2),
// held as fp16 to run: the fp32 product s (code - z), rounded to fp16.
//
// Design (gfx950), one workgroup of 8 waves (two per SIMD) per 256-token x
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

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" int gptq_dequant_gemm(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_out,
                                 int64_t d_in, int bits, int64_t group_size, const void* X, int64_t n_tokens,
                                 int64_t ldx, void* Y, int64_t ldy, int relu, void* stream) {
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
  const int64_t tiles_m = (n_tokens + G_BM - 1) / G_BM, tiles_n = (d_out + G_BN - 1) / G_BN;
  if (tiles_m * tiles_n > (int64_t(1) << 31)) return GPTQ_E_INVALID_ARG;
  const int nwords = int((d_in * bits + 31) / 32);
  const int ngroups = group_size == -1 ? 1 : int((d_in + group_size - 1) / group_size);
  const dim3 grid(unsigned(tiles_m * tiles_n)), block(G_THREADS);
  const int m8 = tiles_m % 8 == 0 ? 1 : 0;
  hipStream_t s = as_stream(stream);
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
