// Stage 3 of the GPTQ layer path: the fixed-order column sweep.
//
// What is computed (aiqz.cc "GPTQ：一键量化大模型压缩", sections 误差补偿 and
// 分组方案; astro-blog LLM quantization survey, sections 1.2, 2.2, 2.3;
// xuzou.cn reading card of the GPTQ paper, section 方法适配): every row is
// swept over its columns in natural order; column q is rounded on its group's
// min-max grid, and its error, divided by U_qq, is spread over the row's
// later columns through row q of U (the upper Cholesky factor of H_d^-1).
// Blocks of 128 columns defer the update of all later columns to the end of
// the block, where it is one rank-128 product.
//
// Design (gfx950): rows are independent given U, so one persistent
// workgroup owns 16 rows for the whole sweep and needs no grid-wide
// synchronization. Per 128-column block it
//   1. stages U[blk, blk] (64 KB fp32) in LDS and 1/U_qq of each lane's
//      columns in registers;
//   2. runs the 128 sequential column steps with each row spread over one
//      16-lane DPP row (8 columns per lane, interleaved): the current value
//      of column q is broadcast from its owner lane with DPP row_newbcast,
//      every lane of the row takes the same rounding decision, and each lane
//      applies the rank-1 update to its own columns (U row q from LDS);
//   3. writes codes, packs the block's 32-bit words from an LDS copy of the
//      codes (128 * bits is a whole number of words), and stores the
//      negated errors -e = -err / U_qq in LDS (the update's A operand as it
//      is used: no negation and no wait on the LDS read beside the MFMAs);
//   4. applies W[rows, i2:] -= E U[blk, i2:] with v_mfma_f32_16x16x4f32 (the
//      workgroup's 16 rows are exactly one MFMA M tile; each lane's 4
//      consecutive output columns make W and U accesses 16-byte vectors),
//      in an fp32 working copy of W in the workspace.
// The first block reads the caller's W directly (no conversion pass).
// Group statistics for a group that starts at column q are taken from the
// current values when the sweep reaches q. The loss sum is kept in fp64.
#include <mutex>
#include <utility>

#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int QB = 128;        // block width
constexpr int QR = 16;         // rows per workgroup
constexpr int QT = 256;        // threads per workgroup
constexpr int QM = QB / 16;    // columns per lane per block
// Whole-tile layers at least this tall and this wide take 32 rows per
// workgroup. Measured: 49152 x 12288, 91.8 against 95-107 ms; 32768 x 8192,
// 31.3 against 28.5 ms; 12288 x 12288, 28.9 against 27.0 ms. It pays only where
// U (upper part 302 MB at d_col = 12288) does not stay in the last-level cache and
// there are enough rows for full rounds of one-per-CU workgroups.
constexpr int RG2_MIN_ROWS = 16384;
constexpr int RG2_MIN_COLS = 12288;
// Largest lazy-batch width (a multiple of QB) the sweep takes.
constexpr int LZ_MAX_B = 1024;
// Blocks per super-block of the 32-row and 8-wave whole-tile forms.
constexpr int SUPER_BLOCKS = 4;

template <int Q, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Q < N) {
    f(std::integral_constant<int, Q>{});
    static_for<Q + 1, N>(f);
  }
}

__device__ __forceinline__ float to_f(float v) { return v; }
__device__ __forceinline__ float to_f(__half v) { return __half2float(v); }

__device__ __forceinline__ floatx4 load4(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return floatx4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ floatx4 load4(const __half* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  const __half2 a = *reinterpret_cast<const __half2*>(&v.x);
  const __half2 b = *reinterpret_cast<const __half2*>(&v.y);
  return floatx4{__low2float(a), __high2float(a), __low2float(b), __high2float(b)};
}

// Buffer-resource loads: a uniform base and size in a 4-SGPR descriptor, a
// 32-bit per-lane byte offset in one VGPR and a uniform byte offset in an
// SGPR. The deferred update reads U this way, so no 64-bit per-lane address
// occupies registers while its loads are in flight (its deep ring of U
// loads needs the room). Every offset used stays inside the size given.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ floatx4 bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Grid of one group from its range [mn, mx] (which always includes 0).
// Min-max (astro-blog survey, 1.2; aiqz.cc, 分组方案): an all-zero group uses
// [-1, 1]; s = (xmax - xmin)/maxq, z = rint(-xmin/s).
// Symmetric (astro-blog survey, 1.2 with the aiqz.cc demo's scale): z = 0 on
// the signed grid, stored as unsigned codes with zero point zs = 2^(b-1);
// s = max|x| / qs, qs = 2^(b-1) - 1; an all-zero group uses max|x| = 1.
__device__ __forceinline__ void grid_params(float mn, float mx, float maxq, int sym, float qs, float zs, float& s,
                                            float& z, float& rs) {
  if (sym) {
    float amax = fmaxf(-mn, mx);
    if (amax == 0.f) amax = 1.f;
    s = amax / qs;
    z = zs;
  } else {
    if (mn == 0.f && mx == 0.f) {
      mn = -1.f;
      mx = 1.f;
    }
    s = (mx - mn) / maxq;
    z = rintf(-mn / s);
  }
  rs = 1.f / s;
}

// x / s rounded to nearest fp32 from rs = RN(1/s): q = RN(x rs) is within an
// ulp of x/s, the residual x - q s is exact in one fma, and one correction
// step q + (x - q s) rs gives the correctly rounded quotient (Markstein's
// division theorem), i.e. the same value as an IEEE division, in 3 ops.
__device__ __forceinline__ float div_rn(float x, float s, float rs) {
  const float q = x * rs;
  const float r = fmaf(-q, s, x);
  return fmaf(r, rs, q);
}

// Whole-tile form of a deferred update W[rows, n_lo:n_hi] -= E[:, ec0:ec0+K]
// U[k0:k0+K, n_lo:n_hi], K = 128 nkb, used when the layer needs no bounds
// test anywhere: d_col % 64 == 0, d_row a multiple of the workgroup's rows,
// W and U 16-byte aligned. The workgroup's rows are RG v_mfma_f32_16x16x4f32
// M tiles of 16 rows (Es the A operand) and U rows k0.. the B operand; wave w
// of the NW = 4 RG XW waves takes the 64-column chunks n_lo + 64 w + 64 NW c
// and applies all RG M tiles to each U operand it loads, so the U traffic per
// row falls with RG (XW > 1 only adds waves to this update). Each chunk of W
// is read once and written once per call, whatever K is. With no branches
// in the loop, the next chunk's W tiles (the accumulators' start values) and
// the U rows RING k-steps ahead, across chunk boundaries, stay in flight
// while the current chunk's MFMAs run.
template <typename WT, int RG, int XW, int EP>
__device__ __forceinline__ void trailing_update_whole(const WT* __restrict__ W, float* __restrict__ Wf,
                                                      const float* __restrict__ U, const float (*Es)[EP], int d_col,
                                                      int row0, int n_lo, int n_hi, int k0, int ec0, int nkb,
                                                      bool first) {
  constexpr int NW = 4 * RG * XW;  // waves per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int nb0 = n_lo + 64 * wave;
  const int nch = nb0 < n_hi ? (n_hi - nb0 + 64 * NW - 1) / (64 * NW) : 0;
  // U rows k0 .. k0 + 128 nkb as one buffer (byte offsets relative to row
  // k0); W and Wf through plain pointers, element offsets relative to the
  // workgroup's first row.
  const rsrc_t ur = make_rsrc(U + size_t(k0) * d_col, uint32_t(QB * nkb) * uint32_t(d_col) * 4u);
  const uint32_t col = uint32_t(nb0 + 4 * li);
  const uint32_t uv = (uint32_t(lk) * uint32_t(d_col) + col) * 4u;  // U row lk, column col
  const uint32_t ustep = 16u * uint32_t(d_col);                       // bytes per k-step (4 U rows)
  const uint32_t chb = 64u * NW * 4u;                                 // U bytes per chunk step
  const float* __restrict__ eb = &Es[li][ec0 + lk];  // A operand of k-step T: eb[16 g EP + 4 T]
  auto ldb = [&](int ch, int T) -> floatx4 { return bload4(ur, uv, uint32_t(ch) * chb + uint32_t(T) * ustep); };
  // (the workgroup's 16 RG rows span fewer than 2^32 elements: d_col <= 2^20)
  const WT* __restrict__ w0 = W + size_t(row0) * d_col;
  float* __restrict__ f0 = Wf + size_t(row0) * d_col;
  const uint32_t wv = uint32_t(4 * lk) * uint32_t(d_col) + col;  // element of row 4 lk, column col
  // rows 16 g + 4 lk + r of chunk ch: element wv + (16 g + r) d_col + 64 NW ch
  auto wso = [&](int g, int r, int ch) {
    return wv + uint32_t(16 * g + r) * uint32_t(d_col) + uint32_t(64 * NW * ch);
  };
  auto ldw = [&](int ch, floatx4 (&v)[RG][4]) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[g][r] = first ? load4(w0 + wso(g, r, ch)) : load4(f0 + wso(g, r, ch));
  };
  // U k-steps in flight. RG = 2 reads its A operands from LDS one k-step
  // ahead instead of keeping all 64 of them in registers. Measured at
  // 49152 x 12288 (32 rows, fp16 W): a ring of 8 k-steps, 61.2 ms; 16,
  // 62.8 ms (256 VGPRs, and the compiler moves accumulators between
  // registers); 4, 63.2 ms.
  constexpr int RING = 8;
  constexpr int KS4 = QB / 4;             // k-steps per 128 rows of U
  // Step t of a 32-step group uses slot t % RING, and the last RING steps of
  // a chunk prefetch the next chunk's first steps into their own slots: RING
  // must divide KS4.
  static_assert(KS4 % RING == 0, "the ring's slots must line up across chunks");
  floatx4 ring[RING];
  floatx4 wn[RG][4];
  if (nch > 0) {
#pragma unroll
    for (int t = 0; t < RING; ++t) ring[t] = ldb(0, t);
    ldw(0, wn);
  }
  for (int ch = 0; ch < nch; ++ch) {
    floatx4 acc[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t][r] = wn[g][r][t];
    const bool more = ch + 1 < nch;
    if (more) ldw(ch + 1, wn);
    float an[RG];  // RG = 2: the next k-step's A operands
    if constexpr (RG > 1) {
#pragma unroll
      for (int g = 0; g < RG; ++g) an[g] = eb[16 * g * EP];
    }
    // One group of KS4 k-steps (128 rows of U). In every group but the
    // chunk's last, all prefetches stay in this chunk.
    auto group = [&](int kb, bool last) {
#pragma unroll
      for (int t = 0; t < KS4; ++t) {
        const int T = KS4 * kb + t;
        const floatx4 b = ring[t % RING];
        if (!last || t + RING < KS4)
          ring[t % RING] = ldb(ch, T + RING);
        else if (more)
          ring[t % RING] = ldb(ch + 1, t + RING - KS4);
        if constexpr (RG == 1) {
          const float at = eb[4 * T];  // A operand: row li, k = 4T + lk
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[0][v] = __builtin_amdgcn_mfma_f32_16x16x4f32(at, b[v], acc[0][v], 0, 0, 0);
        } else {
          float a[RG];
#pragma unroll
          for (int g = 0; g < RG; ++g) a[g] = an[g];
          if (!last || t + 1 < KS4) {
#pragma unroll
            for (int g = 0; g < RG; ++g) an[g] = eb[16 * g * EP + 4 * (T + 1)];
          }
          asm volatile("" ::: "memory");  // each step's reads stay in their step (no hoisting)
#pragma unroll
          for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[g][v] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g], b[v], acc[g][v], 0, 0, 0);
        }
      }
    };
    for (int kb = 0; kb + 1 < nkb; ++kb) group(kb, false);
    group(nkb - 1, true);
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(f0 + wso(g, r, ch)) =
            make_float4(acc[g][0][r], acc[g][1][r], acc[g][2][r], acc[g][3][r]);
  }
}

// RG row groups of QR rows per workgroup (QT threads each), and XW times as
// many waves in the deferred update: with XW = 2 the waves beyond the row
// groups' 4 RG take part only in that update (and in the workgroup's
// barriers). RG > 1 and XW > 1 only for the whole-tile form.
//
// LZ = 2 selects a lazy-batch width B (`lazyb`) that is a multiple of QB, up
// to LZ_MAX_B, in the checked form: inside a B-column block each 128-column
// block's errors reach only the rest of the B-block; at the B-block's end the
// later columns receive all of its errors in one pass (the B-block's errors
// are kept in LDS). Widths that divide QB nest inside the 128-column block,
// whose in-block updates are eager in registers: a column past a B-column
// sub-block then receives the sub-block's errors one by one in column order,
// exactly as deferring them to the sub-block's end would apply them, so
// those widths run the LZ = 0 form. Each element sees the same fp32
// operations in the same order for every B, so every B gives the same
// results to the bit, as the method's exact lazy batches promise.
//
// SB > 1 (whole-tile form, B = QB, groups of at most QB columns) applies the
// same two-level deferral inside the kernel with SB-block super-blocks: the
// columns past a super-block receive its SB QB errors in one K = SB QB pass,
// so the fp32 working copy of those columns is read and written once per
// super-block instead of once per block. Each element still receives the
// errors block by block in column order (the MFMA chain over K runs in that
// order and W's fp32 value is exact in memory between blocks), so the
// results equal the SB = 1 form's to the bit. Group statistics of a group
// wider than QB would read columns past the block before the super-block's
// errors reach them, so such groups take SB = 1.
template <typename WT, bool WHOLE, int RG, int XW, int LZ = 0, int SB = 1>
__global__ void __launch_bounds__(QT * RG * XW, RG * XW == 1 && LZ == 0 ? 2 : 1)
gptq_sweep(const WT* __restrict__ W, float* __restrict__ Wf, const float* __restrict__ U, int d_row, int d_col,
           int bits, int sym, int group, int ngroups, int vec4, uint8_t* __restrict__ codes, float* __restrict__ scales,
           int32_t* __restrict__ zeros, uint32_t* __restrict__ packed, int nwords, float* __restrict__ row_loss,
           double* __restrict__ wg_loss, int lazyb) {
  static_assert(WHOLE || (RG == 1 && XW == 1), "the checked form takes one row group of 4 waves");
  static_assert(LZ == 0 || !WHOLE, "other lazy-batch widths take the checked form");
  static_assert(SB == 1 || (WHOLE && LZ == 0), "super-blocks only in the whole-tile form");
  constexpr int NT = QT * RG * XW, NR = QR * RG;       // threads and rows per workgroup
  constexpr int EW = LZ == 2 ? LZ_MAX_B : SB * QB;     // error columns kept in LDS
  __shared__ __attribute__((aligned(16))) float Ud[QB][QB];
  __shared__ float Es[NR][EW + 4];
  __shared__ uint8_t Cs[NR][QB];
  __shared__ double Lsum[NR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool rows_wave = wave < 4 * RG;  // wave-uniform: this wave carries rows
  const int rloc = rows_wave ? wave * 4 + (lane >> 4) : 0;
  const int sub = lane & 15;
  const int row0 = blockIdx.x * NR;
  const int row = row0 + rloc;
  const bool row_ok = rows_wave && row < d_row;
  const size_t rbase = size_t(row) * d_col;
  const float maxq = float((1 << bits) - 1);
  const float qs = float((1 << (bits - 1)) - 1), zs = float(1 << (bits - 1));

  float s = 1.f, z = 0.f, rs = 1.f;
  double lacc = 0.0;

  if (group < 0) {  // one group per row, from the original row
    float mn = 0.f, mx = 0.f;
    if (row_ok)
      for (int j = sub; j < d_col; j += 16) {
        const float v = to_f(W[rbase + j]);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
    mn = row16_min(mn);
    mx = row16_max(mx);
    grid_params(mn, mx, maxq, sym, qs, zs, s, z, rs);
    if (sub == 0 && row_ok) {
      scales[row] = s;
      zeros[row] = int(z);
    }
  }

  for (int i1 = 0; i1 < d_col; i1 += QB) {
    const int nvalid = d_col - i1 < QB ? d_col - i1 : QB;
    const bool first = (i1 == 0);
    // this block's first error column in Es
    const int kk0 = LZ == 2 ? i1 % lazyb : SB > 1 ? i1 % (SB * QB) : 0;

    // 1. U block (upper part; padded columns act as identity rows) and W block.
    if (vec4 && nvalid == QB) {
      // Full aligned block: 32 threads per row of 128 floats, NT / 32 rows
      // per pass, batches of 8 float4 loads in flight before their LDS
      // stores; the strict lower triangle is zeroed.
      constexpr int RP = NT / 32, NPT = QB / RP;  // rows per pass, rows per thread
      const int k0 = tid >> 5, j0 = (tid & 31) * 4;
      const float* src = U + size_t(i1 + k0) * d_col + i1 + j0;
#pragma unroll
      for (int half = 0; half < NPT / 8; ++half) {
        floatx4 uv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) uv[t] = load4(src + size_t(RP * (t + 8 * half)) * d_col);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int k = k0 + RP * (t + 8 * half);
          floatx4 v = uv[t];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = (j0 + u >= k) ? v[u] : 0.f;
          *reinterpret_cast<float4*>(&Ud[k][j0]) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    } else {
      for (int e = tid; e < QB * QB; e += NT) {
        const int k = e >> 7, j = e & (QB - 1);
        float v;
        if (k < nvalid && j < nvalid)
          v = j >= k ? U[size_t(i1 + k) * d_col + i1 + j] : 0.f;
        else
          v = (k == j) ? 1.f : 0.f;
        Ud[k][j] = v;
      }
    }
    float wr[QM];
#pragma unroll
    for (int m = 0; m < QM; ++m) {
      const int jl = 16 * m + sub;
      float v = 0.f;
      if (row_ok && jl < nvalid) v = first ? to_f(W[rbase + i1 + jl]) : Wf[rbase + i1 + jl];
      wr[m] = v;
    }
    __syncthreads();
    // 1/U_qq of the lane's own columns; step q broadcasts it from q's owner.
    float dv[QM];
#pragma unroll
    for (int m = 0; m < QM; ++m) dv[m] = 1.f / Ud[16 * m + sub][16 * m + sub];

    // 2. The 128 sequential column steps. Row q+1 of the U block is loaded
    //    while step q runs; the empty asm with a memory clobber keeps the
    //    steps in program order (no store merging or load hoisting across
    //    steps, which would lengthen live ranges).
    float uc[QM], un[QM];
#pragma unroll
    for (int mm = 0; mm < QM; ++mm) uc[mm] = Ud[0][16 * mm + sub];
    if (rows_wave) static_for<0, QB>([&](auto qc) {
      constexpr int q = decltype(qc)::value;
      constexpr int m = q / 16;
      constexpr int o = q % 16;
      if constexpr (q + 1 < QB) {
#pragma unroll
        for (int mm = (q + 1) / 16; mm < QM; ++mm) un[mm] = Ud[q + 1][16 * mm + sub];
      }
      const float dc = row_bcast<o>(dv[m]);
      if constexpr (o == 0) {
        if (group > 0 && q < nvalid && (i1 + q) % group == 0) {
          float mn = 0.f, mx = 0.f;
#pragma unroll
          for (int mm = m; mm < QM; ++mm) {
            const float v = (16 * mm + sub < q + group) ? wr[mm] : 0.f;
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
          }
          if (group > QB) {
            const int jend = i1 + group < d_col ? i1 + group : d_col;
            if (row_ok)
              for (int j = i1 + QB + sub; j < jend; j += 16) {
                const float v = first ? to_f(W[rbase + j]) : Wf[rbase + j];
                mn = fminf(mn, v);
                mx = fmaxf(mx, v);
              }
          }
          mn = row16_min(mn);
          mx = row16_max(mx);
          grid_params(mn, mx, maxq, sym, qs, zs, s, z, rs);
          if (sub == 0 && row_ok) {
            const int g = (i1 + q) / group;
            scales[size_t(row) * ngroups + g] = s;
            zeros[size_t(row) * ngroups + g] = int(z);
          }
        }
      }
      const float x = row_bcast<o>(wr[m]);
      float c = rintf(div_rn(x, s, rs)) + z;
      c = fminf(fmaxf(c, 0.f), maxq);
      const float err = fmaf(-s, c - z, x);  // x - s (c - z), rounded once
      const float e = err * dc;
#pragma unroll
      for (int mm = m; mm < QM; ++mm) wr[mm] = fmaf(-e, uc[mm], wr[mm]);
      lacc = fma(0.5 * double(e), double(e), lacc);
      asm volatile("" : "+v"(lacc));  // accumulate now, not deferred across steps
      // Every lane of the row holds the same code and error: all 16 store
      // the same value to the row's LDS slot, so no owner test is needed.
      Cs[rloc][q] = uint8_t(c);
      Es[rloc][kk0 + q] = -e;
      if constexpr (q + 1 < QB) {
#pragma unroll
        for (int mm = (q + 1) / 16; mm < QM; ++mm) uc[mm] = un[mm];
      }
      asm volatile("" ::: "memory");
    });

    // 3. Codes, packed words (the errors are already in Es).
    __syncthreads();
#pragma unroll
    for (int m = 0; m < QM; ++m) {
      const int jl = 16 * m + sub;
      if (row_ok && jl < nvalid) codes[rbase + i1 + jl] = Cs[rloc][jl];
    }
    {
      const int nwb = (nvalid * bits + 31) / 32;
      const int wbase = (i1 * bits) / 32;
      if (row_ok)
        for (int w = sub; w < nwb; w += 16)
          packed[size_t(row) * nwords + wbase + w] = pack_word(Cs[rloc], nvalid, bits, w);
    }

    // 4. Deferred update of the later columns: W[:, i2:] -= E U[blk, i2:].
    const int i2 = i1 + QB;
    if constexpr (WHOLE && SB == 1) {
      if (i2 < d_col) trailing_update_whole<WT, RG, XW, EW + 4>(W, Wf, U, Es, d_col, row0, i2, d_col, i1, 0, 1, first);
    } else if constexpr (WHOLE) {
      // Inside a super-block, this block's errors go to the rest of the
      // super-block; at its end, all of its errors go to the later columns.
      const int o1 = i1 - kk0;
      const int o2 = o1 + SB * QB < d_col ? o1 + SB * QB : d_col;
      if (i2 < o2)
        trailing_update_whole<WT, RG, XW, EW + 4>(W, Wf, U, Es, d_col, row0, i2, o2, i1, kk0, 1, first);
      else if (o2 < d_col)
        trailing_update_whole<WT, RG, XW, EW + 4>(W, Wf, U, Es, d_col, row0, o2, d_col, o1, 0, (o2 - o1) / QB,
                                                  o1 == 0);
    } else if (LZ == 2) {
      // Inside a B-block, this block's errors go to the rest of the B-block;
      // at its end, all of the B-block's errors go to the later columns (a
      // B-block followed by columns is always complete). At most one of the
      // two runs per block. Columns are bounded by n_hi, not d_col: those
      // past the B-block must not receive this block's errors yet.
      const int o1 = i1 - kk0;
      const int o2 = o1 + lazyb < d_col ? o1 + lazyb : d_col;
      const bool inner = i2 < o2;
      if (inner || o2 < d_col) {
        const int n_lo = inner ? i2 : o2, n_hi = inner ? o2 : d_col;
        const int k0 = inner ? i1 : o1;          // U row of the first error
        const int ec0 = inner ? kk0 : 0;         // Es column of the first error
        const int nsub = inner ? 1 : lazyb / QB;  // blocks of errors applied
        const bool fst = inner ? first : o1 == 0;
        const int li = lane & 15, lk = lane >> 4;
        for (int n0 = n_lo + 64 * wave; n0 < n_hi; n0 += 256) {
          const int col = n0 + 4 * li;
          const bool full = vec4 && (n0 + 64 <= n_hi);
          floatx4 acc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = row0 + 4 * lk + r;
            floatx4 v = {0.f, 0.f, 0.f, 0.f};
            if (rr < d_row) {
              const size_t off = size_t(rr) * d_col + col;
              if (full) {
                v = fst ? load4(W + off) : load4(Wf + off);
              } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                  if (col + t < n_hi) v[t] = fst ? to_f(W[off + t]) : Wf[off + t];
              }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t][r] = v[t];
          }
          const uint32_t ustep = uint32_t(4 * d_col);
          for (int sb = 0; sb < nsub; ++sb) {
            const float* ub = U + size_t(k0 + QB * sb + lk) * d_col + col;
            auto ldb = [&](int t) -> floatx4 {
              const float* p = ub + uint32_t(t) * ustep;
              floatx4 b = {0.f, 0.f, 0.f, 0.f};
              if (full) {
                b = load4(p);
              } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  if (col + u < n_hi) b[u] = p[u];
              }
              return b;
            };
            constexpr int RING = 8;
            floatx4 ring[RING];
#pragma unroll
            for (int t = 0; t < RING; ++t) ring[t] = ldb(t);
#pragma unroll
            for (int t = 0; t < QB / 4; ++t) {
              const float at = Es[li][ec0 + QB * sb + 4 * t + lk];  // A operand: row li, k = 128 sb + 4t + lk
              const floatx4 b = ring[t % RING];
              if (t + RING < QB / 4) ring[t % RING] = ldb(t + RING);
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(at, b[v], acc[v], 0, 0, 0);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rr = row0 + 4 * lk + r;
            if (rr >= d_row) continue;
            const size_t off = size_t(rr) * d_col + col;
            if (full) {
              *reinterpret_cast<float4*>(Wf + off) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (col + t < n_hi) Wf[off + t] = acc[t][r];
            }
          }
        }
      }
    } else if (i2 < d_col) {
      const int li = lane & 15, lk = lane >> 4;
      for (int n0 = i2 + 64 * wave; n0 < d_col; n0 += 256) {
        const int col = n0 + 4 * li;
        const bool full = vec4 && (n0 + 64 <= d_col);
        floatx4 acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = row0 + 4 * lk + r;
          floatx4 v = {0.f, 0.f, 0.f, 0.f};
          if (rr < d_row) {
            const size_t off = size_t(rr) * d_col + col;
            if (full) {
              v = first ? load4(W + off) : load4(Wf + off);
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (col + t < d_col) v[t] = first ? to_f(W[off + t]) : Wf[off + t];
            }
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t][r] = v[t];
        }
        // B operands U[i1 + 4t + lk][col .. col + 3] through a 16-deep
        // register ring: the load for step t + 16 is issued as step t retires.
        const float* ub = U + size_t(i1 + lk) * d_col + col;
        const uint32_t ustep = uint32_t(4 * d_col);
        auto ldb = [&](int t) -> floatx4 {
          const float* p = ub + uint32_t(t) * ustep;
          floatx4 b = {0.f, 0.f, 0.f, 0.f};
          if (full) {
            b = load4(p);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (col + u < d_col) b[u] = p[u];
          }
          return b;
        };
        constexpr int RING = 8;
        floatx4 ring[RING];
#pragma unroll
        for (int t = 0; t < RING; ++t) ring[t] = ldb(t);
#pragma unroll
        for (int t = 0; t < QB / 4; ++t) {
          const float at = Es[li][4 * t + lk];  // A operand: row li, k = 4t + lk
          const floatx4 b = ring[t % RING];
          if (t + RING < QB / 4) ring[t % RING] = ldb(t + RING);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_amdgcn_mfma_f32_16x16x4f32(at, b[v], acc[v], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = row0 + 4 * lk + r;
          if (rr >= d_row) continue;
          const size_t off = size_t(rr) * d_col + col;
          if (full) {
            *reinterpret_cast<float4*>(Wf + off) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
          } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (col + t < d_col) Wf[off + t] = acc[t][r];
          }
        }
      }
    }
    __syncthreads();
  }

  if (sub == 0 && rows_wave) {
    Lsum[rloc] = row_ok ? lacc : 0.0;
    if (row_ok && row_loss) row_loss[row] = float(lacc);
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int r = 0; r < NR; ++r) t += Lsum[r];
    wg_loss[blockIdx.x] = t;
  }
}

// Sum of the per-workgroup losses in a fixed order.
__global__ void __launch_bounds__(256) loss_final(const double* __restrict__ part, int n, double* __restrict__ loss) {
  __shared__ double sh[256];
  double t = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) t += part[i];
  sh[threadIdx.x] = t;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = sh[0];
}

__global__ void __launch_bounds__(256)
pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t d_row, int d_col, int bits, uint32_t* __restrict__ packed,
                  int nwords) {
  const int64_t n = d_row * nwords;
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / nwords;
    const int w = int(i % nwords);
    packed[i] = pack_word(codes + r * d_col, d_col, bits, w);
  }
}

inline bool bits_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 8; }

struct QuantWs {
  float* Wf;
  double* wg_loss;
  size_t bytes;
};

QuantWs carve_q(void* ws, int64_t d_row, int64_t d_col) {
  QuantWs w{};
  const size_t wf = align_up(size_t(d_row) * d_col * sizeof(float), 256);
  const int64_t nwg = (d_row + QR - 1) / QR;
  w.bytes = wf + align_up(size_t(nwg) * sizeof(double), 256);
  if (ws != nullptr) {  // sizes only when there is no workspace yet
    char* p = static_cast<char*>(ws);
    w.Wf = reinterpret_cast<float*>(p);
    w.wg_loss = reinterpret_cast<double*>(p + wf);
  }
  return w;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_quantize_layer_workspace_size(int64_t d_row, int64_t d_col, int bits, int64_t group_size,
                                                     int64_t block) {
  (void)bits;
  (void)group_size;
  (void)block;
  if (d_row < 1 || d_col < 1) return 0;
  return carve_q(nullptr, d_row, d_col).bytes;
}

namespace gptq {
namespace {

// Argument checks shared by both sweep entry points (nothing is touched
// before they pass).
int check_quantize_args(const void* W, int wdtype, int64_t d_row, int64_t d_col, const float* U, int bits,
                        int64_t group_size, int64_t block, int symmetric, const uint8_t* codes, const float* scales,
                        const int32_t* zeros, const uint32_t* packed, const double* loss) {
  if (d_row < 1 || d_col < 1 || d_row > (int64_t(1) << 30) || d_col > (1 << 20)) return GPTQ_E_INVALID_ARG;
  if (d_row * d_col > (int64_t(1) << 40)) return GPTQ_E_INVALID_ARG;
  if (!W || !U || !codes || !scales || !zeros || !packed || !loss) return GPTQ_E_INVALID_ARG;
  if (wdtype != GPTQ_F16 && wdtype != GPTQ_F32) return GPTQ_E_INVALID_ARG;
  if (!bits_ok(bits) || (symmetric != 0 && symmetric != 1)) return GPTQ_E_INVALID_ARG;
  if (block < 1) return GPTQ_E_INVALID_ARG;
  if (group_size != -1) {
    if (group_size < 1 || (block % group_size != 0 && group_size % block != 0)) return GPTQ_E_INVALID_ARG;
  }
  // lazy-batch widths: a power of two up to QB, or a multiple of QB up to LZ_MAX_B
  if (!(block <= QB && (block & (block - 1)) == 0) && !(block % QB == 0 && block <= LZ_MAX_B))
    return GPTQ_E_UNSUPPORTED;
  if (group_size != -1 && group_size % 16 != 0) return GPTQ_E_UNSUPPORTED;
  return GPTQ_OK;
}

// The sweep and the loss sum on stream s, with the working copy and loss
// partials at w (arguments already checked).
int launch_quantize(const void* W, int wdtype, int64_t d_row, int64_t d_col, const float* U, int bits,
                    int64_t group_size, int64_t block, int symmetric, uint8_t* codes, float* scales, int32_t* zeros,
                    uint32_t* packed, double* loss, float* row_loss, const QuantWs& w, hipStream_t s) {
  const int ngroups = group_size == -1 ? 1 : int((d_col + group_size - 1) / group_size);
  const int nwords = int((d_col * bits + 31) / 32);
  const int esz = wdtype == GPTQ_F16 ? 2 : 4;
  const int vec4 = (d_col % 4 == 0) && (reinterpret_cast<uintptr_t>(W) % (4 * esz) == 0) &&
                   (reinterpret_cast<uintptr_t>(U) % 16 == 0) ? 1 : 0;
  // Whole-tile layers (every chunk of the deferred update complete, every
  // workgroup's rows present) take the branch-free update; tall and wide ones
  // take 32 rows per workgroup, halving the U rows each row's update streams.
  // Lazy-batch widths above the block take the checked form with two-level
  // deferral; those that divide the block nest inside it (see gptq_sweep).
  // The 32-row and 8-wave forms hold one workgroup per CU and defer in
  // super-blocks of SUPER_BLOCKS blocks, which groups wider than the block
  // do not allow; such layers take the 4-wave 16-row form (two workgroups
  // per CU).
  const int lz = block > QB ? 2 : 0;
  const bool whole = lz == 0 && vec4 && d_col % 64 == 0 && d_row % QR == 0;
  const bool super = whole && (group_size == -1 || group_size <= QB);
  const int rg = (super && d_row % (2 * QR) == 0 && d_row >= RG2_MIN_ROWS && d_col >= RG2_MIN_COLS) ? 2 : 1;
  const unsigned nwg = unsigned((d_row + rg * QR - 1) / (rg * QR));
  // The other super-block layers take 16 rows and 8 waves per workgroup
  // (one workgroup per CU): the extra 4 waves work only in the deferred
  // update. Measured against two 4-wave workgroups per CU without
  // super-blocks: 12288 x 12288, 19.3 against 28.9 ms; 11008 x 4096, 2.84
  // against 2.90 ms.
  const int xw = (super && rg == 1) ? 2 : 1;
  if (wdtype == GPTQ_F16) {
    auto k = rg == 2 ? gptq_sweep<__half, true, 2, 1, 0, SUPER_BLOCKS>
             : xw == 2 ? gptq_sweep<__half, true, 1, 2, 0, SUPER_BLOCKS>
             : whole ? gptq_sweep<__half, true, 1, 1>
             : lz == 2 ? gptq_sweep<__half, false, 1, 1, 2>
                     : gptq_sweep<__half, false, 1, 1>;
    hipLaunchKernelGGL(k, dim3(nwg), dim3(rg * xw * QT), 0, s, static_cast<const __half*>(W), w.Wf, U, int(d_row),
                       int(d_col), bits, symmetric, int(group_size), ngroups, vec4, codes, scales, zeros, packed, nwords,
                       row_loss, w.wg_loss, int(block));
  } else {
    auto k = rg == 2 ? gptq_sweep<float, true, 2, 1, 0, SUPER_BLOCKS>
             : xw == 2 ? gptq_sweep<float, true, 1, 2, 0, SUPER_BLOCKS>
             : whole ? gptq_sweep<float, true, 1, 1>
             : lz == 2 ? gptq_sweep<float, false, 1, 1, 2>
                     : gptq_sweep<float, false, 1, 1>;
    hipLaunchKernelGGL(k, dim3(nwg), dim3(rg * xw * QT), 0, s, static_cast<const float*>(W), w.Wf, U, int(d_row),
                       int(d_col), bits, symmetric, int(group_size), ngroups, vec4, codes, scales, zeros, packed, nwords,
                       row_loss, w.wg_loss, int(block));
  }
  if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  hipLaunchKernelGGL(loss_final, dim3(1), dim3(256), 0, s, w.wg_loss, int(nwg), loss);
  return launch_status();
}

// Scratch of the allocation-free sweep entry point: the fp32 working copy
// of W (at most GPTQ_NOALLOC_MAX_WEIGHTS elements) followed by the
// per-workgroup loss partials (at most GPTQ_NOALLOC_MAX_ROWS / 16 doubles).
// Each GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, never a device
// address: its device address comes from hipGetSymbolAddress, per device.
constexpr size_t NOALLOC_WF_BYTES = size_t(GPTQ_NOALLOC_MAX_WEIGHTS) * sizeof(float);
constexpr size_t NOALLOC_BYTES = NOALLOC_WF_BYTES + 65536;
static_assert(NOALLOC_WF_BYTES % 256 == 0, "loss partials must start 256-byte aligned");
static_assert((GPTQ_NOALLOC_MAX_ROWS / QR) * sizeof(double) <= 65536, "loss partials must fit");
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on the current device, taken once per
// device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return GPTQ_E_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPTQ_E_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return GPTQ_OK;
}

}  // namespace
}  // namespace gptq

extern "C" int gptq_quantize_layer(const void* W, int wdtype, int64_t d_row, int64_t d_col, const float* U, int bits,
                                   int64_t group_size, int64_t block, int symmetric, uint8_t* codes, float* scales,
                                   int32_t* zeros, uint32_t* packed, double* loss, float* row_loss, void* ws,
                                   size_t ws_bytes, void* stream) {
  const int st = check_quantize_args(W, wdtype, d_row, d_col, U, bits, group_size, block, symmetric, codes, scales,
                                     zeros, packed, loss);
  if (st != GPTQ_OK) return st;
  const QuantWs w = carve_q(ws, d_row, d_col);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_E_WORKSPACE;
  return launch_quantize(W, wdtype, d_row, d_col, U, bits, group_size, block, symmetric, codes, scales, zeros, packed, loss,
                         row_loss, w, as_stream(stream));
}

extern "C" int gptq_quantize_layer_noalloc(const void* W, int wdtype, int64_t d_row, int64_t d_col, const float* U,
                                           int bits, int64_t group_size, int64_t block, int symmetric,
                                           uint8_t* codes, float* scales, int32_t* zeros, uint32_t* packed,
                                           double* loss, float* row_loss, void* stream) {
  const int st = check_quantize_args(W, wdtype, d_row, d_col, U, bits, group_size, block, symmetric, codes, scales,
                                     zeros, packed, loss);
  if (st != GPTQ_OK) return st;
  if (d_row > GPTQ_NOALLOC_MAX_ROWS || d_row * d_col > GPTQ_NOALLOC_MAX_WEIGHTS) return GPTQ_E_TOO_LARGE;
  hipStream_t s = as_stream(stream);
  if (s != nullptr) {  // the scratch used is the current device's: the stream must belong to it
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess) return GPTQ_E_HIP;
    if (cur != sdev) return GPTQ_E_INVALID_ARG;
  }
  void* base = nullptr;
  const int sa = scratch_address(&base);
  if (sa != GPTQ_OK) return sa;
  const QuantWs w = carve_q(base, d_row, d_col);
  if (w.bytes > NOALLOC_BYTES) return GPTQ_E_TOO_LARGE;
  // Nothing in the scratch must start at zero: every working-copy element
  // the sweep reads was written earlier in the same launch, and every loss
  // partial is written before loss_final reads it.
  return launch_quantize(W, wdtype, d_row, d_col, U, bits, group_size, block, symmetric, codes, scales, zeros, packed, loss,
                         row_loss, w, s);
}

extern "C" int gptq_pack_codes(const uint8_t* codes, int64_t d_row, int64_t d_col, int bits, uint32_t* packed,
                               void* stream) {
  if (d_row < 1 || d_col < 1 || d_col > (1 << 24) || !codes || !packed || !bits_ok(bits)) return GPTQ_E_INVALID_ARG;
  const int nwords = int((d_col * bits + 31) / 32);
  const int64_t n = d_row * nwords;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_codes_kernel, dim3(unsigned(blocks)), dim3(256), 0, as_stream(stream), codes, d_row,
                     int(d_col), bits, packed, nwords);
  return launch_status();
}

extern "C" const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "ok";
    case GPTQ_E_INVALID_ARG: return "invalid argument";
    case GPTQ_E_UNSUPPORTED: return "unsupported parameter";
    case GPTQ_E_WORKSPACE: return "workspace too small";
    case GPTQ_E_HIP: return "HIP launch or runtime error";
    case GPTQ_E_TOO_LARGE: return "layer larger than the allocation-free entry point's static scratch";
    default: return "unknown status";
  }
}

extern "C" const char* gptq_version(void) { return "0.1.0"; }
