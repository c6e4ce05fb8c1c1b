// Running a quantized layer on token batches: Y = act(X What^T).
//
// xuzou.cn reading card of the GPTQ paper, section 计算设置: the model is
// quantized one block at a time and the quantized block is run on the
// calibration tokens to produce the next block's inputs; section 方法适配
// (last paragraph): the quantized matrix is multiplied with dequantization on
// the fly. What = s (code - z) per group (astro-blog survey, section 1.2),
// held as fp16 to run: the fp32 product s (code - z), rounded to fp16.
//
// Design (gfx950), one workgroup of 4 waves per 256-token x 128-weight-row
// output tile, K (d_in) in tiles of 64:
//  * X tiles [256 tokens][64] fp16 go through registers into LDS (row pitch
//    72 halfs, so the 16-byte fragment reads of 32 consecutive rows fall on
//    distinct banks).
//  * d_in must be a multiple of 32; a last K tile of 32 columns is padded
//    with zeros in LDS (nothing past d_in is read).
//  * W tiles are cut from the packed words: each thread takes one 32-code
//    unit (bits words of one row hold exactly 32 codes) per K tile, forms
//    s (c - z) in fp32, rounds it to fp16 and stores the 32 halfs into the
//    LDS tile [128 rows][64] (same pitch).
//  * Each wave computes 128 tokens x 64 rows with v_mfma_f32_32x32x16_f16
//    (4 x 2 tiles): A fragments are 8 consecutive K of one token, B
//    fragments 8 consecutive K of one weight row, both 16-byte LDS reads.
//  * Two LDS stages: the next K tile's global loads are issued before the
//    current tile's MFMAs and its dequantization runs beside them.
//  * Epilogue: optional ReLU on the fp32 sum, then round to fp16.
// fp16 x fp16 products are exact in fp32; the sums are fp32 (MFMA order).
#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int G_BM = 256;          // tokens per tile
constexpr int G_BN = 128;          // weight rows per tile
constexpr int G_BK = 64;           // K per tile
constexpr int G_P = G_BK + 8;      // LDS row pitch (halfs)
constexpr int G_THREADS = 256;

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

template <int BITS, int J = 0>
__device__ __forceinline__ void static_for_pairs(const uint32_t (&w)[BITS], float s, float zoff, uint32_t (&h)[16]) {
  if constexpr (J < 32) {
    h[J / 2] = dq_pair<BITS, J>(w, s, zoff);
    static_for_pairs<BITS, J + 2>(w, s, zoff, h);
  }
}

template <int BITS>
__global__ void __launch_bounds__(G_THREADS, 1)
dequant_gemm_f16(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                 const int32_t* __restrict__ zeros, int d_out, int d_in, int nwords, int group, int ngroups,
                 const __half* __restrict__ X, int64_t n_tok, int64_t ldx, __half* __restrict__ Y, int64_t ldy,
                 int relu, int n_tiles_n) {
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][G_BM * G_P];
  __shared__ __attribute__((aligned(16))) _Float16 ws[2][G_BN * G_P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // consecutive workgroups share the token tile and sweep the weight tiles
  const int tn = int(blockIdx.x % unsigned(n_tiles_n));
  const int64_t tm = int64_t(blockIdx.x / unsigned(n_tiles_n));
  const int64_t m0 = tm * G_BM;
  const int n0 = tn * G_BN;
  const int nkt = (d_in + G_BK - 1) / G_BK;  // d_in % 32 == 0: the last tile may hold 32 columns

  // X loads: 8 per thread per tile, lane group of 8 covers one row's 128 bytes.
  const int xr = tid >> 3, xc = (tid & 7) * 8;  // row (of 32) and K offset
  const __half* xrow[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int64_t t = m0 + xr + 32 * i;
    if (t >= n_tok) t = n_tok - 1;  // clamped rows are computed and never stored
    xrow[i] = X + t * ldx + xc;
  }
  // W unit: row wr of the tile, unit wu (codes 32 wu .. 32 wu + 31 of the K tile).
  const int wr = tid >> 1, wu = tid & 1;
  const int wrow = n0 + wr < d_out ? n0 + wr : d_out - 1;
  const uint32_t* prow = packed + size_t(wrow) * nwords;
  const float* srow = scales + size_t(wrow) * ngroups;
  const int32_t* zrow = zeros + size_t(wrow) * ngroups;

  uint4 xv[8];
  uint32_t pw[BITS];
  float sv = 0.f, zoff = 0.f;
  auto load_tile = [&](int kt) {
    const int k0 = kt * G_BK;
    // In a last tile of 32 columns, the second half of X and the second
    // unit are zeros (nothing past d_in is read); their products add 0.
    const bool x_in = k0 + xc < d_in, w_in = k0 + 32 * wu < d_in;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xv[i] = x_in ? *reinterpret_cast<const uint4*>(xrow[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    const int unit = (k0 >> 5) + wu;
#pragma unroll
    for (int b = 0; b < BITS; ++b) pw[b] = w_in ? prow[unit * BITS + b] : 0u;
    const int g = (group > 0 && w_in) ? (k0 + 32 * wu) / group : 0;
    sv = w_in ? srow[g] : 0.f;
    zoff = 8388608.f + (w_in ? float(zrow[g]) : 0.f);
  };
  auto store_tile = [&](int st) {
    _Float16* xd = xs[st];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(xd + (xr + 32 * i) * G_P + xc) = xv[i];
    uint32_t h[16];
    static_for_pairs<BITS>(pw, sv, zoff, h);
    _Float16* wd = ws[st] + wr * G_P + 32 * wu;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(wd + 8 * q) = make_uint4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx16{0};

  // fragment bases: lane l reads row l % 32 of its tile, K 8 (l / 32) ..
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) load_tile(kt + 1);
    const _Float16* xa = xs[st] + (wm * 128 + fr) * G_P + fk;
    const _Float16* wb = ws[st] + (wn * 64 + fr) * G_P + fk;
#pragma unroll
    for (int kk = 0; kk < G_BK / 16; ++kk) {
      half8 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const half8*>(xa + 32 * i * G_P + 16 * kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const half8*>(wb + 32 * j * G_P + 16 * kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_tile(st ^ 1);
    __syncthreads();
  }

  // 32x32 result layout: lane l holds column l % 32 (a weight row) and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 (tokens) of register r.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + 32 * j + fr;
      if (col >= d_out) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t t = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
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
  hipStream_t s = as_stream(stream);
  const __half* x = static_cast<const __half*>(X);
  __half* y = static_cast<__half*>(Y);
  switch (bits) {
    case 2:
      hipLaunchKernelGGL(dequant_gemm_f16<2>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n));
      break;
    case 3:
      hipLaunchKernelGGL(dequant_gemm_f16<3>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n));
      break;
    case 4:
      hipLaunchKernelGGL(dequant_gemm_f16<4>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n));
      break;
    default:
      hipLaunchKernelGGL(dequant_gemm_f16<8>, grid, block, 0, s, packed, scales, zeros, int(d_out), int(d_in), nwords,
                         int(group_size), ngroups, x, n_tokens, ldx, y, ldy, relu, int(tiles_n));
      break;
  }
  return launch_status();
}
