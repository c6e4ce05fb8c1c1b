// Use of the packed layer: quantized matrix x full-precision vectors.
//
// xuzou.cn reading card of the GPTQ paper, section 方法适配 (last paragraph)
// and section 瓶颈: batch-1 generation is dominated by matrix-vector
// products that are memory-bandwidth bound, so the inference kernel
// multiplies the quantized matrix by full-precision activations and
// dequantizes the weights on the fly, reading the low-bit words instead of
// fp16 weights. Dequantization: What = s (code - z) per group (astro-blog
// survey, section 1.2).
//
//   Y[b][r] = sum_c X[b][c] * s[r][g(c)] * (code[r][c] - z[r][g(c)])
//
// Design (gfx950). Three kernels:
//
// * dequant_matvec_pairs, for groups that are a multiple of 32 columns (or
//   one group per row) and 16-byte aligned activations: the 32-column unit
//   (BITS words) sits in one group, so it takes one scale and one zero.
//   The unit's 32 codes are taken as 16 pairs; a pair's two fields are cut
//   from one 32-bit window of the unit's bit stream, one field in each
//   16-bit half, and OR-ed under the fp16 exponent of 1024, which turns
//   each half into 1024 + (code << o) exactly; one packed fp16 FMA with the
//   power-of-two scale 2^-o and offset -1024 * 2^-o returns both codes as
//   fp16 values exactly, and one dot2 (fp16 pairs, fp32 accumulate)
//   multiplies them with the matching pair of activations. The pair plan
//   (which codes, which window, which offsets) depends only on BITS and
//   is fixed at compile time. A wave takes RB rows at once, so the
//   activation pairs and the unit's activation sum are built once for RB
//   rows; the next unit's loads are in flight while one unit is computed.
//   The zero is folded as s (sum c x - z sum x) per unit.
// * dequant_matmul_mfma, for 3 to 16 vectors per pass (d_col a multiple of
//   128, groups of 128-column multiples or one per row, aligned x): the
//   codes, cut with the same pair plan and already as code - z, are the B
//   operand of fp16 MFMAs, the activations the A operand (see below).
// * dequant_matvec_kernel, for every other case: one wave per row, codes
//   extracted one at a time and the fold taken per 8-column chunk.
//
// In both, each lane accumulates in fp32 and the 64 lanes are summed in a
// fixed order (xor butterfly), so the result is deterministic. The bytes
// read are the packed words, the scales and zeros, and X (shared by all
// rows, from L2).
#include <utility>

#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int MV_ROWS = 4;   // generic kernel: rows per workgroup, one wave each
constexpr int MV_WAVES = 4;  // pair kernel: waves per workgroup

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <int Q, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Q < N) {
    f(std::integral_constant<int, Q>{});
    static_for<Q + 1, N>(f);
  }
}

// Code j of a 32-code unit held in BITS words (bit p of the unit is bit
// p % 32 of word p / 32).
template <int BITS, int J>
__device__ __forceinline__ float unit_code(const uint32_t (&w)[BITS]) {
  constexpr int p = BITS * J, wi = p / 32, off = p % 32;
  uint32_t v = w[wi] >> off;
  if constexpr (off + BITS > 32) v |= w[wi + 1] << (32 - off);
  return float(v & ((1u << BITS) - 1u));
}

// Pair i (0..15) of a 32-code unit: codes lo and hi, and the first bit of the
// 32-bit window of the unit's bit stream both fields are cut from. In the
// window, code lo sits at bit o_lo and code hi at bit 16 + o_hi, both
// fields inside the 10 mantissa bits of their fp16 half.
template <int BITS>
struct PairPlan {
  static constexpr int lo(int i) {
    return BITS == 2 ? 16 * (i / 8) + i % 8 : BITS == 3 ? 8 * (i / 4) + i % 4 : BITS == 4 ? 8 * (i / 4) + i % 4
                                                                                           : 4 * (i / 2) + i % 2;
  }
  static constexpr int hi(int i) { return lo(i) + (BITS == 2 ? 8 : BITS == 8 ? 2 : 4); }
  static constexpr int win(int i) {
    return BITS == 2   ? 32 * (i / 8) + (i % 8 < 5 ? 0 : 10)
           : BITS == 3 ? 24 * (i / 4) + (i % 4 < 2 ? -4 : 2)
           : BITS == 4 ? 32 * (i / 4) + (i % 4 < 2 ? 0 : 8)
                       : 32 * (i / 2) + 8 * (i % 2);
  }
  static constexpr int o_lo(int i) { return BITS * lo(i) - win(i); }
  static constexpr int o_hi(int i) { return BITS * hi(i) - win(i) - 16; }
  static constexpr bool valid() {
    for (int i = 0; i < 16; ++i)
      if (o_lo(i) < 0 || o_lo(i) > 10 - BITS || o_hi(i) < 0 || o_hi(i) > 10 - BITS) return false;
    return true;
  }
};

// Bits [P, P + 32) of the unit (bit q is bit q % 32 of w[q / 32]); positions
// outside the unit read as zero.
template <int BITS, int P>
__device__ __forceinline__ uint32_t unit_window(const uint32_t (&w)[BITS]) {
  if constexpr (P < 0) {
    return w[0] << (-P);
  } else {
    constexpr int k = P / 32, sh = P % 32;
    if constexpr (sh == 0)
      return w[k];
    else if constexpr (k + 1 < BITS)
      return __builtin_amdgcn_alignbit(w[k + 1], w[k], sh);
    else
      return w[k] >> sh;
  }
}

// The pair masks and the fp16 exponent pattern, held in registers for the
// whole kernel: the mask in an SGPR, the exponent pattern in a VGPR, so
// that each pair's mask-and-merge is one v_and_or_b32 (a VOP3 instruction
// takes no literal operand on this target).
template <int BITS>
struct PairMasks {
  uint32_t m[16];
  uint32_t magic;
};

template <int BITS>
__device__ __forceinline__ constexpr uint32_t pair_mask(int i) {
  using PL = PairPlan<BITS>;
  return (((1u << BITS) - 1u) << PL::o_lo(i)) | (((1u << BITS) - 1u) << (16 + PL::o_hi(i)));
}

// First pair with the same mask as pair i (pairs that share a mask share a
// register).
template <int BITS>
__device__ __forceinline__ constexpr int mask_first(int i) {
  int j = 0;
  while (pair_mask<BITS>(j) != pair_mask<BITS>(i)) ++j;
  return j;
}

template <int BITS>
__device__ __forceinline__ PairMasks<BITS> pair_masks() {
  PairMasks<BITS> pm;
  static_for<0, 16>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (mask_first<BITS>(i) == i) {
      uint32_t v = pair_mask<BITS>(i);
      asm volatile("" : "+s"(v));
      pm.m[i] = v;
    } else {
      pm.m[i] = pm.m[mask_first<BITS>(i)];
    }
  });
  uint32_t g = 0x64006400u;
  asm volatile("" : "+v"(g));
  pm.magic = g;
  return pm;
}

// Sum over the unit of code * x, in fp32, with x given as the plan's pairs.
template <int BITS>
__device__ __forceinline__ float unit_dot(const uint32_t (&w)[BITS], const h2_t (&xp)[16], const PairMasks<BITS>& pm) {
  using PL = PairPlan<BITS>;
  static_assert(PL::valid(), "pair plan out of the fp16 mantissa");
  float dot = 0.f;
  static_for<0, 16>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    constexpr int olo = PL::o_lo(i), ohi = PL::o_hi(i);
    const uint32_t t = (unit_window<BITS, PL::win(i)>(w) & pm.m[i]) | pm.magic;  // 1024 + (code << o) per half
    const h2_t sc = {(_Float16)(1.0f / float(1 << olo)), (_Float16)(1.0f / float(1 << ohi))};
    const h2_t of = {(_Float16)(-1024.0f / float(1 << olo)), (_Float16)(-1024.0f / float(1 << ohi))};
    const h2_t c = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, t), sc, of);  // exact codes
    dot = __builtin_amdgcn_fdot2(c, xp[i], dot, false);
  });
  return dot;
}

// One unit's operands for RB rows and NB activation vectors.
template <int BITS, int RB, int NB>
struct PairLoads {
  uint32_t w[RB][BITS];
  float s[RB], z[RB];
  uint4 x[NB][4];
};

// Loads of unit u for the RB rows of row block rb (rows past d_row read row
// d_row - 1). With valid == false the loads still read unit u (valid
// memory) and the scales are set to zero, so the unit adds nothing.
template <int BITS, int RB, int NB>
__device__ __forceinline__ void pair_load(PairLoads<BITS, RB, NB>& L, int rb, int u, bool valid,
                                          const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                                          const int32_t* __restrict__ zeros, int d_row, int nwords, float inv_upg,
                                          int ngroups, const __half* __restrict__ x, int64_t ldx) {
  // (u + 0.5) / (group / 32) rounded down: the float error is far below the
  // distance 0.5 / (group / 32) to the nearest integer for units < 2^19.
  const int gi = min(int((float(u) + 0.5f) * inv_upg), ngroups - 1);
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int rr = min(rb * RB + r, d_row - 1);  // wave-uniform
    const uint32_t* pr = packed + size_t(rr) * nwords;
#pragma unroll
    for (int k = 0; k < BITS; ++k) L.w[r][k] = pr[u * BITS + k];
    const float sv = scales[size_t(rr) * ngroups + gi];
    L.s[r] = valid ? sv : 0.f;
    L.z[r] = float(zeros[size_t(rr) * ngroups + gi]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const uint4* xb = reinterpret_cast<const uint4*>(x + b * ldx + (u << 5));
#pragma unroll
    for (int q = 0; q < 4; ++q) L.x[b][q] = xb[q];
  }
}

template <int BITS, int RB, int NB>
__device__ __forceinline__ void pair_compute(const PairLoads<BITS, RB, NB>& L, const PairMasks<BITS>& pm,
                                             float (&acc)[RB][NB]) {
  using PL = PairPlan<BITS>;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    h2_t xn[16];  // natural pairs: xn[j] = (x[2j], x[2j + 1])
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xn[4 * q] = __builtin_bit_cast(h2_t, L.x[b][q].x);
      xn[4 * q + 1] = __builtin_bit_cast(h2_t, L.x[b][q].y);
      xn[4 * q + 2] = __builtin_bit_cast(h2_t, L.x[b][q].z);
      xn[4 * q + 3] = __builtin_bit_cast(h2_t, L.x[b][q].w);
    }
    h2_t xp[16];  // the plan's pairs: xp[i] = (x[lo(i)], x[hi(i)])
    float sx = 0.f;
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    static_for<0, 16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int a = PL::lo(i), c = PL::hi(i);
      xp[i] = __builtin_shufflevector(xn[a / 2], xn[c / 2], a % 2, 2 + c % 2);
      sx = __builtin_amdgcn_fdot2(xn[i], one, sx, false);
    });
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const float dot = unit_dot<BITS>(L.w[r], xp, pm);
      acc[r][b] = fmaf(L.s[r], fmaf(-L.z[r], sx, dot), acc[r][b]);
    }
  }
}

// Kernel arguments of the pair kernel.
struct PairArgs {
  const uint32_t* __restrict__ packed;
  const float* __restrict__ scales;
  const int32_t* __restrict__ zeros;
  int d_row, d_col, nwords;
  float inv_upg;
  int ngroups;
  const __half* __restrict__ x;
  int64_t ldx;
  float* __restrict__ y;
  int64_t ldy;
};

// End of row block rb: the partial last unit (d_col % 32 columns, on one
// lane; words past the row's last word and activations past d_col read
// zero), the lane sum in a fixed order, the store, and cleared sums.
template <int BITS, int RB, int NB>
__device__ __forceinline__ void pair_finish(const PairArgs& a, int rb, int lane, const PairMasks<BITS>& pm,
                                            float (&acc)[RB][NB]) {
  const int nfull = a.d_col >> 5;
  if ((a.d_col & 31) && lane == (nfull & 63)) {
    PairLoads<BITS, RB, NB> T;
    const int u = nfull;
    const int gi = min(int((float(u) + 0.5f) * a.inv_upg), a.ngroups - 1);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int rr = min(rb * RB + r, a.d_row - 1);
      const uint32_t* pr = a.packed + size_t(rr) * a.nwords;
#pragma unroll
      for (int k = 0; k < BITS; ++k) T.w[r][k] = (u * BITS + k < a.nwords) ? pr[u * BITS + k] : 0u;
      T.s[r] = a.scales[size_t(rr) * a.ngroups + gi];
      T.z[r] = float(a.zeros[size_t(rr) * a.ngroups + gi]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      uint32_t xw[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int c = (u << 5) + 2 * j;
        const uint32_t lo = c < a.d_col ? __half_as_ushort(a.x[b * a.ldx + c]) : 0u;
        const uint32_t hi = c + 1 < a.d_col ? __half_as_ushort(a.x[b * a.ldx + c + 1]) : 0u;
        xw[j] = lo | (hi << 16);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) T.x[b][q] = make_uint4(xw[4 * q], xw[4 * q + 1], xw[4 * q + 2], xw[4 * q + 3]);
    }
    pair_compute<BITS, RB, NB>(T, pm, acc);
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = acc[r][b];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
      if (lane == 0 && rb * RB + r < a.d_row) a.y[b * a.ldy + rb * RB + r] = v;
      acc[r][b] = 0.f;
    }
}

// One step of a wave's item stream: compute item (rb, j), held in Cur,
// while the next item's loads go to Nxt. The next loads are unconditional
// (after the wave's last item they re-read the current one), so no load
// sits under a branch. Returns whether there is a next item.
template <int BITS, int RB, int NB>
__device__ __forceinline__ bool pair_step(const PairArgs& a, PairLoads<BITS, RB, NB>& Cur,
                                          PairLoads<BITS, RB, NB>& Nxt, int& rb, int& j, int J, int nrb, int nwaves,
                                          int lane, const PairMasks<BITS>& pm, float (&acc)[RB][NB]) {
  const int nfull = a.d_col >> 5, last = nfull - 1;
  int rb2 = rb, j2 = j + 1;
  if (j2 == J) {
    j2 = 0;
    rb2 += nwaves;
  }
  const bool more = rb2 < nrb;
  const int rbl = more ? rb2 : rb, jl = more ? j2 : j;
  pair_load<BITS, RB, NB>(Nxt, rbl, min(lane + 64 * jl, last), lane + 64 * jl < nfull, a.packed, a.scales, a.zeros,
                          a.d_row, a.nwords, a.inv_upg, a.ngroups, a.x, a.ldx);
  pair_compute<BITS, RB, NB>(Cur, pm, acc);
  if (j == J - 1) pair_finish<BITS, RB, NB>(a, rb, lane, pm, acc);
  rb = rb2;
  j = j2;
  return more;
}

// Persistent waves: wave w takes row blocks (RB rows each) w, w + nwaves,
// ... and, in each, the 32-column units lane, lane + 64, ... of its rows.
// The (row block, unit slot) items of a wave form one stream whose next
// item's loads are in flight while the current item is computed, also
// across row blocks, so a wave starts cold once. Rows past d_row read row
// d_row - 1 and store nothing. Requires 16-byte aligned x rows
// (ldx % 8 == 0) and groups that are a multiple of 32 columns or one group
// per row.
template <int BITS, int RB, int NB>
__global__ void __launch_bounds__(256) dequant_matvec_pairs(const PairArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * MV_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = gridDim.x * MV_WAVES;
  const int nrb = (a.d_row + RB - 1) / RB;
  if (wave >= nrb) return;  // whole wave; the kernel has no barrier
  const int nfull = a.d_col >> 5;
  const int J = (nfull + 63) >> 6;  // unit slots per lane in a row block
  const PairMasks<BITS> pm = pair_masks<BITS>();
  float acc[RB][NB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
  if (J == 0) {  // d_col < 32: only the partial unit
    for (int rb = wave; rb < nrb; rb += nwaves) pair_finish<BITS, RB, NB>(a, rb, lane, pm, acc);
    return;
  }
  int rb = wave, j = 0;
  PairLoads<BITS, RB, NB> A, B;
  pair_load<BITS, RB, NB>(A, rb, min(lane, nfull - 1), lane < nfull, a.packed, a.scales, a.zeros, a.d_row, a.nwords,
                          a.inv_upg, a.ngroups, a.x, a.ldx);
  while (pair_step<BITS, RB, NB>(a, A, B, rb, j, J, nrb, nwaves, lane, pm, acc) &&
         pair_step<BITS, RB, NB>(a, B, A, rb, j, J, nrb, nwaves, lane, pm, acc)) {
  }
}

// ---------------------------------------------------------------------------
// MFMA form, for d_col % 128 == 0, groups of a multiple of 128 columns (or one
// group per row), 16-byte aligned x rows, up to 16 vectors per pass.
//
// A wave takes 16 rows; lane l handles row l % 16 and unit slot q = l / 16
// of each 128-column super-unit (4 units of 32 codes, one group). For each
// of the super-unit's 4 code chunks t, a lane's 4 code pairs (plan pairs
// 4t .. 4t+3 of its unit) become the 8 halves of the B operand of
// v_mfma_f32_16x16x32_f16, already as exact fp16 values code - z (the
// packed FMA's offset carries -1024 2^-o - z); the A operand is the same 4
// pairs of activations for vector l % 16, read from LDS, where the
// workgroup has staged them in pair order. So D[m][n] = sum over the
// super-unit of x_m (code - z)_n, and y[m][n] += s_n D[m][n] once per
// super-unit. The dot products run on the matrix core; the VALU only cuts
// and converts codes. Cutting and converting dominates either way, so for one
// or two vectors the pair kernel is faster (its loads read whole lines of one
// row); with more vectors this form takes 16 per pass against 2.
constexpr int MM_WAVES = 4;  // waves per workgroup, 16 rows each
constexpr int MM_CH = 8;     // super-units per LDS chunk: 8 x 4 KB of staged activations
constexpr int MM_MIN_BATCH = 3;  // one or two vectors: the pair kernel is faster (measured)

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

// The 4 code pairs of chunk t of a unit as the B operand (code - z, fp16).
template <int BITS, int T>
__device__ __forceinline__ half8 mm_codes(const uint32_t (&w)[BITS], const PairMasks<BITS>& pm, h2_t zz) {
  using PL = PairPlan<BITS>;
  h2_t c[4];
  static_for<0, 4>([&](auto pc) {
    constexpr int i = 4 * T + decltype(pc)::value;
    constexpr int olo = PL::o_lo(i), ohi = PL::o_hi(i);
    const uint32_t t = (unit_window<BITS, PL::win(i)>(w) & pm.m[i]) | pm.magic;  // 1024 + (code << o) per half
    const h2_t sc = {(_Float16)(1.0f / float(1 << olo)), (_Float16)(1.0f / float(1 << ohi))};
    const h2_t base = {(_Float16)(-1024.0f / float(1 << olo)), (_Float16)(-1024.0f / float(1 << ohi))};
    const h2_t of = base - zz;  // -1024 2^-o - z, exact in fp16
    c[decltype(pc)::value] = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, t), sc, of);  // code - z, exact
  });
  const h4_t lo = __builtin_shufflevector(c[0], c[1], 0, 1, 2, 3);
  const h4_t hi = __builtin_shufflevector(c[2], c[3], 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Staging of one LDS entry: the 4 activation pairs of chunk t of unit q of a
// super-unit for vector m, from the 8 activations that chunk needs (one
// 16-byte run, or two 8-byte runs for 2-bit codes), in plan order.
template <int BITS>
__device__ __forceinline__ uint4 mm_stage(const __half* __restrict__ xr, int col0, int t) {
  uint32_t a[4];
  if constexpr (BITS == 2) {
    const int base = col0 + 16 * (t >> 1) + 4 * (t & 1);
    const uint2 lo = *reinterpret_cast<const uint2*>(xr + base);
    const uint2 hi = *reinterpret_cast<const uint2*>(xr + base + 8);
    a[0] = lo.x;
    a[1] = lo.y;
    a[2] = hi.x;
    a[3] = hi.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + col0 + 8 * t);
    a[0] = v.x;
    a[1] = v.y;
    a[2] = v.z;
    a[3] = v.w;
  }
  // halves X0..X7 = a[0].lo, a[0].hi, a[1].lo, ...
  h2_t X[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) X[k] = __builtin_bit_cast(h2_t, a[k]);
  h2_t p[4];
  if constexpr (BITS == 8) {  // (X0, X2), (X1, X3), (X4, X6), (X5, X7)
    p[0] = __builtin_shufflevector(X[0], X[1], 0, 2);
    p[1] = __builtin_shufflevector(X[0], X[1], 1, 3);
    p[2] = __builtin_shufflevector(X[2], X[3], 0, 2);
    p[3] = __builtin_shufflevector(X[2], X[3], 1, 3);
  } else {  // (X0, X4), (X1, X5), (X2, X6), (X3, X7)
    p[0] = __builtin_shufflevector(X[0], X[2], 0, 2);
    p[1] = __builtin_shufflevector(X[0], X[2], 1, 3);
    p[2] = __builtin_shufflevector(X[1], X[3], 0, 2);
    p[3] = __builtin_shufflevector(X[1], X[3], 1, 3);
  }
  return make_uint4(__builtin_bit_cast(uint32_t, p[0]), __builtin_bit_cast(uint32_t, p[1]),
                    __builtin_bit_cast(uint32_t, p[2]), __builtin_bit_cast(uint32_t, p[3]));
}

// Rows past d_row read row d_row - 1 and store nothing; vectors past `batch`
// are staged as zeros and stored nowhere.
template <int BITS>
__global__ void __launch_bounds__(64 * MM_WAVES)
dequant_matmul_mfma(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                    const int32_t* __restrict__ zeros, int d_row, int d_col, int nwords, int group, int ngroups,
                    const __half* __restrict__ x, int64_t ldx, int batch, float* __restrict__ y, int64_t ldy) {
  __shared__ uint4 xs[MM_CH * 4 * 4 * 16];  // [super-unit][chunk t][unit q][vector m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int row = blockIdx.x * (16 * MM_WAVES) + wave * 16 + n;
  const int rrow = row < d_row ? row : d_row - 1;
  const uint32_t* __restrict__ pr = packed + size_t(rrow) * nwords;
  const float* __restrict__ sr = scales + size_t(rrow) * ngroups;
  const int32_t* __restrict__ zr = zeros + size_t(rrow) * ngroups;
  const PairMasks<BITS> pm = pair_masks<BITS>();
  const int nsu = d_col >> 7;
  const int su_per_group = group > 0 ? group >> 7 : nsu;  // super-units per group
  floatx4 Y = {0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nsu; c0 += MM_CH) {
    const int nch = nsu - c0 < MM_CH ? nsu - c0 : MM_CH;
    __syncthreads();  // the previous chunk's entries are no longer read
    for (int e = tid; e < nch * 256; e += 64 * MM_WAVES) {
      const int sl = e >> 8, t = (e >> 6) & 3, qq = (e >> 4) & 3, m = e & 15;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (m < batch) v = mm_stage<BITS>(x + m * ldx, 128 * (c0 + sl) + 32 * qq, t);
      xs[e] = v;
    }
    __syncthreads();
    uint32_t w[BITS], wn[BITS];
    const int u0 = 4 * c0 + q;
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = pr[u0 * BITS + k];
    for (int sl = 0; sl < nch; ++sl) {
      const int su = c0 + sl;
      // next super-unit's words (the last one re-read, unused), issued before this one is converted
      const int un = 4 * (sl + 1 < nch ? su + 1 : su) + q;
#pragma unroll
      for (int k = 0; k < BITS; ++k) wn[k] = pr[un * BITS + k];
      const int gi = su / su_per_group;
      const float sv = sr[gi];
      const _Float16 zh = (_Float16)float(zr[gi]);
      const h2_t zz = {zh, zh};
      floatx4 D = {0.f, 0.f, 0.f, 0.f};
      const uint4* xa = xs + (sl * 4) * 64 + q * 16 + n;  // entry (sl, t, q, m = n) at xa + 64 t
      static_for<0, 4>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        const half8 b = mm_codes<BITS, t>(w, pm, zz);
        const half8 a = __builtin_bit_cast(half8, xa[64 * t]);
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, D, 0, 0, 0);
      });
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[r] = fmaf(sv, D[r], Y[r]);
#pragma unroll
      for (int k = 0; k < BITS; ++k) w[k] = wn[k];
    }
  }
  // lane l holds y[m = 4 q + r][row]: D rows are the vectors, columns the rows
  if (row < d_row) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * q + r;
      if (m < batch) y[m * ldy + row] = Y[r];
    }
  }
}

template <int BITS, int NB, bool VECX>
__global__ void __launch_bounds__(256)
dequant_matvec_kernel(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                      const int32_t* __restrict__ zeros, int d_row, int d_col, int nwords, int group, int ngroups,
                      const __half* __restrict__ x, int64_t ldx, float* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * MV_ROWS + (threadIdx.x >> 6);
  if (row >= d_row) return;  // whole wave; the kernel has no barrier
  const uint32_t* __restrict__ pr = packed + size_t(row) * nwords;
  const float* __restrict__ sr = scales + size_t(row) * ngroups;
  const int32_t* __restrict__ zr = zeros + size_t(row) * ngroups;
  const int nunits = (d_col + 31) >> 5;
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  // Two units per lane per round, with the round's words, scales, zeros and
  // activations loaded before the first product, so a row costs one memory
  // round trip per round rather than one per unit. (The host passes at most
  // two vectors per launch; the chunk-by-chunk branch only serves wider
  // instantiations.)
  constexpr bool PREX = NB <= 2;
  constexpr int NX = PREX ? NB : 1;
  auto load_x = [&](int b, int cc, bool ok, float (&xo)[8]) {
    const __half* xb = x + b * ldx + cc;
    if (VECX && ok && cc + 8 <= d_col) {
      const uint4 raw = *reinterpret_cast<const uint4*>(xb);
      const __half2* hh = reinterpret_cast<const __half2*>(&raw);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xo[2 * i] = __low2float(hh[i]);
        xo[2 * i + 1] = __high2float(hh[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xo[i] = (ok && cc + i < d_col) ? __half2float(xb[i]) : 0.f;
    }
  };
  for (int u0 = lane; u0 < nunits; u0 += 128) {
    uint32_t w[2][BITS];
    float s[2][4], z[2][4];
    float xv[2][NX][4][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = u0 + 64 * h;
      const bool uok = u < nunits;
#pragma unroll
      for (int k = 0; k < BITS; ++k) {
        const int wi = u * BITS + k;
        w[h][k] = (uok && wi < nwords) ? pr[wi] : 0u;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int cc = (u << 5) + 8 * k;
        const bool ok = uok && cc < d_col;
        const int gi = ok ? (group > 0 ? cc / group : 0) : 0;
        s[h][k] = ok ? sr[gi] : 0.f;
        z[h][k] = ok ? float(zr[gi]) : 0.f;
        if constexpr (PREX) {
#pragma unroll
          for (int b = 0; b < NB; ++b) load_x(b, cc, ok, xv[h][b][k]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = u0 + 64 * h;
      static_for<0, 4>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        float code[8];
        static_for<0, 8>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          code[i] = unit_code<BITS, 8 * k + i>(w[h]);
        });
        const int cc = (u << 5) + 8 * k;
        const bool ok = u < nunits && cc < d_col;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float xo[8];
          if constexpr (PREX) {
#pragma unroll
            for (int i = 0; i < 8; ++i) xo[i] = xv[h][b][k][i];
          } else {
            load_x(b, cc, ok, xo);
          }
          float dot = 0.f, sx = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            dot = fmaf(code[i], xo[i], dot);
            sx += xo[i];
          }
          acc[b] = fmaf(s[h][k], fmaf(-z[h][k], sx, dot), acc[b]);
        }
      });
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float v = acc[b];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) y[b * ldy + row] = v;
  }
}

template <int BITS, int NB>
int launch_nb(bool vecx, const uint32_t* packed, const float* scales, const int32_t* zeros, int d_row, int d_col,
              int nwords, int group, int ngroups, const __half* x, int64_t ldx, float* y, int64_t ldy,
              hipStream_t s) {
  const dim3 grid(unsigned((d_row + MV_ROWS - 1) / MV_ROWS)), block(256);
  if (vecx)
    hipLaunchKernelGGL((dequant_matvec_kernel<BITS, NB, true>), grid, block, 0, s, packed, scales, zeros, d_row,
                       d_col, nwords, group, ngroups, x, ldx, y, ldy);
  else
    hipLaunchKernelGGL((dequant_matvec_kernel<BITS, NB, false>), grid, block, 0, s, packed, scales, zeros, d_row,
                       d_col, nwords, group, ngroups, x, ldx, y, ldy);
  return launch_status();
}

template <int BITS>
int launch_mfma(const uint32_t* packed, const float* scales, const int32_t* zeros, int d_row, int d_col, int nwords,
                int group, int ngroups, const __half* x, int64_t ldx, int batch, float* y, int64_t ldy, hipStream_t s) {
  const dim3 grid(unsigned((d_row + 16 * MM_WAVES - 1) / (16 * MM_WAVES))), block(64 * MM_WAVES);
  hipLaunchKernelGGL((dequant_matmul_mfma<BITS>), grid, block, 0, s, packed, scales, zeros, d_row, d_col, nwords, group,
                     ngroups, x, ldx, batch, y, ldy);
  return launch_status();
}

template <int BITS, int RB, int NB>
int launch_pairs_rb(const uint32_t* packed, const float* scales, const int32_t* zeros, int d_row, int d_col,
                    int nwords, float inv_upg, int ngroups, const __half* x, int64_t ldx, float* y, int64_t ldy,
                    hipStream_t s) {
  // Persistent grid: at most the waves the device holds at once, and, when
  // there are more row blocks than that, an equal count of row blocks for
  // every wave (k = ceil(row blocks / resident waves) each).
  static const int resident = [] {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dequant_matvec_pairs<BITS, RB, NB>, 64 * MV_WAVES, 0) !=
            hipSuccess || cus < 1 || per_cu < 1)
      return 0;
    return cus * per_cu * MV_WAVES;
  }();
  if (resident < 1) return GPTQ_E_HIP;
  const int nrb = (d_row + RB - 1) / RB;
  const int k = (nrb + resident - 1) / resident;
  const int waves = (nrb + k - 1) / k;
  const dim3 grid(unsigned((waves + MV_WAVES - 1) / MV_WAVES)), block(64 * MV_WAVES);
  const PairArgs a{packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy};
  hipLaunchKernelGGL((dequant_matvec_pairs<BITS, RB, NB>), grid, block, 0, s, a);
  return launch_status();
}

// Rows per wave: as many as keep at least 2048 waves (8 per CU) in the grid.
template <int BITS, int NB>
int launch_pairs_nb(const uint32_t* packed, const float* scales, const int32_t* zeros, int d_row, int d_col,
                    int nwords, float inv_upg, int ngroups, const __half* x, int64_t ldx, float* y, int64_t ldy,
                    hipStream_t s) {
  if (d_row >= 4 * 2048)
    return launch_pairs_rb<BITS, 4, NB>(packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy,
                                        s);
  if (d_row >= 2 * 2048)
    return launch_pairs_rb<BITS, 2, NB>(packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy,
                                        s);
  return launch_pairs_rb<BITS, 1, NB>(packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy, s);
}

template <int BITS>
int launch_bits(bool pairs, int nb, bool vecx, const uint32_t* packed, const float* scales, const int32_t* zeros,
                int d_row, int d_col, int nwords, int group, int ngroups, const __half* x, int64_t ldx, float* y,
                int64_t ldy, hipStream_t s) {
  if (pairs) {
    const float inv_upg = group > 0 ? 1.0f / float(group / 32) : 0.0f;
    if (nb == 2)
      return launch_pairs_nb<BITS, 2>(packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy,
                                      s);
    return launch_pairs_nb<BITS, 1>(packed, scales, zeros, d_row, d_col, nwords, inv_upg, ngroups, x, ldx, y, ldy, s);
  }
  if (nb == 2)
    return launch_nb<BITS, 2>(vecx, packed, scales, zeros, d_row, d_col, nwords, group, ngroups, x, ldx, y, ldy, s);
  return launch_nb<BITS, 1>(vecx, packed, scales, zeros, d_row, d_col, nwords, group, ngroups, x, ldx, y, ldy, s);
}

// What[r][c] = fp(s[r][g(c)] * (code[r][c] - z[r][g(c)])): the product in
// fp32 (code - z is an exact small integer), then rounded to the output type
// (round to nearest even). One workgroup per row (grid-stride over rows),
// threads along the row; every code is cut from at most two words of the
// row's stream, inside the row's words.
template <typename OT>
__global__ void __launch_bounds__(256)
dequantize_kernel(const uint32_t* __restrict__ packed, const float* __restrict__ scales,
                  const int32_t* __restrict__ zeros, int d_row, int d_col, int nwords, int bits, int group,
                  int ngroups, OT* __restrict__ out, int64_t ldo) {
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t r = blockIdx.x; r < d_row; r += gridDim.x) {
    const uint32_t* pr = packed + r * nwords;
    const float* sr = scales + r * ngroups;
    const int32_t* zr = zeros + r * ngroups;
    OT* orow = out + r * ldo;
    for (int c = threadIdx.x; c < d_col; c += blockDim.x) {
      const int64_t bit = int64_t(c) * bits;
      const int w = int(bit >> 5), off = int(bit & 31);
      uint32_t v = pr[w] >> off;
      if (off + bits > 32) v |= pr[w + 1] << (32 - off);  // word w + 1 holds the code's last bit: w + 1 < nwords
      v &= mask;
      const int g = group > 0 ? c / group : 0;
      float val = sr[g] * (float(v) - float(zr[g]));
      if constexpr (sizeof(OT) == 2) {
        // Keep the fp32 product a value of its own: fused into one
        // mixed-precision FMA with a +0 addend, the product would be rounded
        // once to fp16 and a -0 product would come out as +0.
        asm volatile("" : "+v"(val));
        orow[c] = __float2half_rn(val);
      } else {
        orow[c] = val;
      }
    }
  }
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" int gptq_dequant_matvec(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_row,
                                   int64_t d_col, int bits, int64_t group_size, const void* x, int64_t batch,
                                   int64_t ldx, float* y, void* stream) {
  if (d_row < 1 || d_col < 1 || batch < 1 || d_row > (int64_t(1) << 30) || d_col > (1 << 24)) return GPTQ_E_INVALID_ARG;
  if (!packed || !scales || !zeros || !x || !y || ldx < d_col) return GPTQ_E_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_E_INVALID_ARG;
  if (group_size != -1 && (group_size < 8 || group_size % 8 != 0)) return GPTQ_E_INVALID_ARG;
  const int nwords = int((d_col * bits + 31) / 32);
  const int ngroups = group_size == -1 ? 1 : int((d_col + group_size - 1) / group_size);
  const int grp = group_size == -1 ? 0 : int(group_size);
  const bool vecx = (ldx % 8 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  const bool pairs = vecx && (group_size == -1 || group_size % 32 == 0);
  // The MFMA form needs whole 128-column super-units inside one group; it
  // takes up to 16 vectors per pass, where the pair kernel takes 2.
  const bool mfma = vecx && d_col % 128 == 0 && (group_size == -1 || group_size % 128 == 0) && batch >= MM_MIN_BATCH;
  if (mfma) {
    hipStream_t s = as_stream(stream);
    const __half* xh = static_cast<const __half*>(x);
    for (int64_t b0 = 0; b0 < batch; b0 += 16) {
      const int nb = int(batch - b0 < 16 ? batch - b0 : 16);
      int st;
      switch (bits) {
        case 2:
          st = launch_mfma<2>(packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xh + b0 * ldx, ldx,
                              nb, y + b0 * d_row, d_row, s);
          break;
        case 3:
          st = launch_mfma<3>(packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xh + b0 * ldx, ldx,
                              nb, y + b0 * d_row, d_row, s);
          break;
        case 4:
          st = launch_mfma<4>(packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xh + b0 * ldx, ldx,
                              nb, y + b0 * d_row, d_row, s);
          break;
        default:
          st = launch_mfma<8>(packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xh + b0 * ldx, ldx,
                              nb, y + b0 * d_row, d_row, s);
          break;
      }
      if (st != GPTQ_OK) return st;
    }
    return GPTQ_OK;
  }
  hipStream_t s = as_stream(stream);
  const __half* xh = static_cast<const __half*>(x);
  for (int64_t b0 = 0; b0 < batch;) {
    const int64_t left = batch - b0;
    const int nb = left >= 2 ? 2 : 1;  // two vectors per pass keep every operand in registers
    const __half* xb = xh + b0 * ldx;
    float* yb = y + b0 * d_row;
    int st;
    switch (bits) {
      case 2:
        st = launch_bits<2>(pairs, nb, vecx, packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xb, ldx,
                            yb, d_row, s);
        break;
      case 3:
        st = launch_bits<3>(pairs, nb, vecx, packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xb, ldx,
                            yb, d_row, s);
        break;
      case 4:
        st = launch_bits<4>(pairs, nb, vecx, packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xb, ldx,
                            yb, d_row, s);
        break;
      default:
        st = launch_bits<8>(pairs, nb, vecx, packed, scales, zeros, int(d_row), int(d_col), nwords, grp, ngroups, xb, ldx,
                            yb, d_row, s);
        break;
    }
    if (st != GPTQ_OK) return st;
    b0 += nb;
  }
  return GPTQ_OK;
}

extern "C" int gptq_dequantize(const uint32_t* packed, const float* scales, const int32_t* zeros, int64_t d_row,
                               int64_t d_col, int bits, int64_t group_size, void* out, int out_dtype, int64_t ld_out,
                               void* stream) {
  if (d_row < 1 || d_col < 1 || d_row > (int64_t(1) << 30) || d_col > (1 << 24)) return GPTQ_E_INVALID_ARG;
  if (!packed || !scales || !zeros || !out || ld_out < d_col) return GPTQ_E_INVALID_ARG;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return GPTQ_E_INVALID_ARG;
  if (group_size != -1 && group_size < 1) return GPTQ_E_INVALID_ARG;
  if (out_dtype != GPTQ_F16 && out_dtype != GPTQ_F32) return GPTQ_E_INVALID_ARG;
  const int nwords = int((d_col * bits + 31) / 32);
  const int ngroups = group_size == -1 ? 1 : int((d_col + group_size - 1) / group_size);
  const int grp = group_size == -1 ? 0 : int(group_size);
  const unsigned grid = unsigned(d_row < 65536 ? d_row : 65536);
  hipStream_t s = as_stream(stream);
  if (out_dtype == GPTQ_F16)
    hipLaunchKernelGGL(dequantize_kernel<__half>, dim3(grid), dim3(256), 0, s, packed, scales, zeros, int(d_row),
                       int(d_col), nwords, bits, grp, ngroups, static_cast<__half*>(out), ld_out);
  else
    hipLaunchKernelGGL(dequantize_kernel<float>, dim3(grid), dim3(256), 0, s, packed, scales, zeros, int(d_row),
                       int(d_col), nwords, bits, grp, ngroups, static_cast<float*>(out), ld_out);
  return launch_status();
}
