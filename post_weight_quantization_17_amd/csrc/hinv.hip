// Stage 2 of the GPTQ layer path: U, the upper Cholesky factor of
// (H + lambda I)^-1, lambda = damp * mean(diag H).
//
// astro-blog LLM quantization survey, section 2.3 item 3, and the xuzou.cn
// reading card of the GPTQ paper, section 方法适配: the sweep's inverse
// Hessian rows are precomputed with a Cholesky factorization of the mildly
// damped Hessian, which the pages describe as more robust than updating an
// explicit inverse.
//
// Route taken here (same U, half the flops of "invert, then factor"):
// let J be the index reversal and A = J H_d J. With A = L L^T (L lower),
// H_d = V V^T for the upper V = J L J, and H_d^-1 = U^T U with U = V^-1 =
// J L^-1 J. The Cholesky factor with positive diagonal is unique, so this is
// the factor of H_d^-1 itself.
//
// L and X = L^-1 are computed together in fp64, one 128-column super-panel
// S = [s0, s1) of two 64-column blocks k0, k1 at a time:
//   step (one launch per super-panel): every workgroup factors both
//         diagonal blocks itself, X_k0 = chol(A_k0k0)^-1 and, after
//         A_k1k1 -= L_k1k0 L_k1k0^T with L_k1k0 = A_k1k0 X_k0^T,
//         X_k1 = chol(A_k1k1)^-1 (a pivot that is not positive sets `info`),
//         then computes its tiles of
//                  rows i >= s1:  L_iS, kept column-major in the panel buffer LT
//                  cols c < s1:   X_Sc = block row S of X
//   trail (once per super-panel, K = 128; the next super-panel's columns
//         take the previous super-panel too, K = 256):
//                  A_ij -= L_iS L_jS^T   for i >= j >= s1 (lower tiles)
//                  R_ic -= L_iS X_Sc     for i >= s1, c < s1
// R starts as the identity; block row k of R becomes block row k of X once
// its super-panel step has run. All products use the fp64 MFMA
// (v_mfma_f64_16x16x4f64). The trailing update, which holds almost all of
// the flops, reads the trailing matrix once per 128 columns instead of once
// per 64 and keeps 16 independent MFMA chains per wave.
#include <hip/hip_ext.h>

#include <mutex>
#include <utility>

#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int NB = 64;   // block (diagonal factorization) width
constexpr int KS = 128;  // super-panel width

template <int Q, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Q < N) {
    f(std::integral_constant<int, Q>{});
    static_for<Q + 1, N>(f);
  }
}

__device__ __forceinline__ doublex4 mfma64(double a, double b, doublex4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- setup
__global__ void __launch_bounds__(256)
hinv_lambda(const float* __restrict__ H, int d, double damp, double* __restrict__ lam,
            float* __restrict__ lambda_out, int32_t* __restrict__ info) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) s += double(H[int64_t(i) * d + i]);
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double l = damp * (part[0] / double(d));
    *lam = l;
    if (lambda_out) *lambda_out = float(l);
    *info = 0;
  }
}

// A[i][j] = H[d-1-j][d-1-i] + lambda [i == j] and R[i][j] = [i == j] for
// j <= i (reads H's lower triangle, which is the reversed matrix's lower
// triangle by symmetry), one 32x32 lower block per workgroup. The
// workgroups after the first nlow zero R on block rows [s0, s0 + 64) x
// columns [s0 + 64, s0 + 128) of each super-panel with two blocks: the only
// part of R above the diagonal that is read (by the trailing update, inside
// block rows S of X) before a super-panel step writes it. Nothing reads the
// rest of R above the diagonal.
__global__ void __launch_bounds__(256)
hinv_setup(const float* __restrict__ H, int d, const double* __restrict__ lam, double* __restrict__ A,
           double* __restrict__ R, int nlow) {
  __shared__ float t[32][33];
  if (int(blockIdx.x) >= nlow) {
    const int u = int(blockIdx.x) - nlow;
    const int i0 = (u >> 2) * KS + 32 * ((u >> 1) & 1), j0 = (u >> 2) * KS + NB + 32 * (u & 1);
    for (int e = threadIdx.x; e < 1024; e += 256) {
      const int i = i0 + (e >> 5), j = j0 + (e & 31);
      if (i < d && j < d) R[int64_t(i) * d + j] = 0.0;
    }
    return;
  }
  int b = blockIdx.x, bi = 0;
  while (b > bi) {
    b -= bi + 1;
    ++bi;
  }
  const int bj = b;  // bj <= bi
  const int i0 = bi * 32, j0 = bj * 32;
  const double l = *lam;
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int jj = e >> 5, ii = e & 31;
    const int i = i0 + ii, j = j0 + jj;
    t[jj][ii] = (i < d && j < d) ? H[int64_t(d - 1 - j) * d + (d - 1 - i)] : 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 1024; e += 256) {
    const int ii = e >> 5, jj = e & 31;
    const int i = i0 + ii, j = j0 + jj;
    if (i >= d || j >= d || j > i) continue;
    A[int64_t(i) * d + j] = double(t[jj][ii]) + (i == j ? l : 0.0);
    R[int64_t(i) * d + j] = i == j ? 1.0 : 0.0;
  }
}

// ------------------------------------------------------------ MFMA helpers
// v_mfma_f64_16x16x4f64 operands: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; result: lane l, register r holds row l / 16 + 4 r,
// column l % 16 of the 16x16 block.

// acc[t] += Aop * Bop for NBLK 16x16 blocks over k in [0, K), K a multiple
// of 4, with both operands in LDS: Aop(i, k) = As[k * pa + i] ("k-major",
// rows contiguous) or As[i * pa + k]; Bop(k, j) = Bs[k * pb + j].
// Block t covers rows ri[t] .. + 16, columns cj[t] .. + 16.
template <int NBLK, bool A_KMAJOR>
__device__ __forceinline__ void blocks_mma(doublex4 (&acc)[NBLK], const double* As, int pa, const double* Bs, int pb,
                                           const int (&ri)[NBLK], const int (&cj)[NBLK], int K) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = lane >> 4;
  for (int k = 0; k < K; k += 4) {
#pragma unroll
    for (int t = 0; t < NBLK; ++t) {
      const double a = A_KMAJOR ? As[(k + lk) * pa + ri[t] + lr] : As[(ri[t] + lr) * pa + k + lk];
      const double b = Bs[(k + lk) * pb + cj[t] + lr];
      acc[t] = mfma64(a, b, acc[t]);
    }
  }
}

// f(row, col, value) for every accumulator element of the blocks.
template <int NBLK, typename F>
__device__ __forceinline__ void blocks_for_each(doublex4 (&acc)[NBLK], const int (&ri)[NBLK], const int (&cj)[NBLK],
                                                F f) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int t = 0; t < NBLK; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) f(ri[t] + (lane >> 4) + 4 * r, cj[t] + (lane & 15), acc[t][r]);
}

template <int NBLK>
__device__ __forceinline__ void zero(doublex4 (&acc)[NBLK]) {
#pragma unroll
  for (int t = 0; t < NBLK; ++t) acc[t] = doublex4{0, 0, 0, 0};
}

// 1/x to within an ulp: hardware estimate plus two Newton steps.
__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  r = fma(r, fma(-x, r, 1.0), r);
  r = fma(r, fma(-x, r, 1.0), r);
  return r;
}

// ------------------------------------------------------------ super-panel step
// One launch per super-panel S = [s0, s1): block k0 = s0 (kb0 <= 64
// columns) and, when S is wider than 64, block k1 = s0 + 64 (kb1 <= 64
// columns; kb0 = 64 then). Every workgroup computes, with the same
// instructions on the same data, so that every copy is the same to the bit:
//   X_k0 = chol(A_k0k0)^-1,
//   L_k1k0 = A_k1k0 X_k0^T,
//   X_k1 = chol(A_k1k1 - L_k1k0 L_k1k0^T)^-1,
// and then its own tiles of both blocks:
//   rows i >= s1 (32 at a time):  L_ik0 = A_ik0 X_k0^T,
//                                 L_ik1 = (A_ik1 - L_ik0 L_k1k0^T) X_k1^T,
//                                 both column-major in the panel buffer LT
//                                 (LT[m * d + i] = L[i][s0 + m]);
//   columns c < s0 (32 at a time): X_k0c = X_k0 R_k0c,
//                                 X_k1c = X_k1 (R_k1c - L_k1k0 X_k0c), in R;
//   columns c in [s0, s0 + 64):   X_k1c = X_k1 (R_k1c - L_k1k0 X_k0c), with
//                                 X_k0c taken from X_k0 itself.
// Workgroup 0 also writes X_k0 and X_k1 into R's diagonal blocks and
// reports a pivot that is not positive. The copies of the two 64x64
// factorizations run side by side, so recomputing them costs the chain
// nothing: the super-panel needs one dependent launch, and the second
// block does not wait for the first block's panel to reach memory.
//
// The factorization is Gauss-Jordan on one symmetric 64x64 array v: step j
// eliminates column j with multipliers m_i = v_ij / v_jj (i > j). Columns
// c > j still hold the Schur complement (v_ic -= m_i v_jc); columns c < j
// hold the unit-lower inverse Y (v_ic -= m_i y_jc); column j itself becomes
// Y's column j (-m_i, and 1 on the diagonal). Row j of v therefore carries
// everything step j needs: y_jc left of the diagonal, the pivot, and the
// Schur row, which equals the Schur column by symmetry (m_i = v_ji / v_jj).
// After 64 steps X_kk = L^-1 has X_ic = y_ic / sqrt(pivot_i). Rows and
// columns past kb act as identity.
//
// Thread t owns the 4x4 block rows 4 (t / 16) .., columns 4 (t % 16) .. in
// registers for all 64 steps; the 16 threads that hold rows j and j+1 (one
// quarter of one wave) write them to LDS, double buffered, one barrier per
// two steps.
// LDS pitches (doubles) of 64-wide and 32-wide tiles. They are odd so that
// the 16 rows one quarter-wave reads in a row-major MFMA operand read (and
// the 16 columns a transposing store writes) fall in distinct banks: with a
// pitch of 68 those reads met 4 ways in a bank.
constexpr int PP = NB + 1;
constexpr int PQ = 32 + 1;
static_assert(NB * PQ >= 32 * PP, "the tile buffer holds 32 x 64 at pitch PP");
// Workgroups of one super-panel step. Each factors the diagonal blocks
// itself, so more workgroups take CU time from the trailing update running
// beside them; beyond this count a workgroup takes several tiles.
constexpr int STEP_MAX_WG = 128;

// v <- the factorization of the block whose lower part is in T (T[i][j],
// j <= i < kb); dr <- the pivots of the thread's rows. Two steps per
// barrier: the owners of rows j and j+1 (j even) publish both rows; every
// thread applies step j, derives row j+1 after step j at the positions it
// needs (its 4 rows, its 4 columns, the pivot pair) with the same
// arithmetic the owners use, and applies step j+1. A loop of 16 iterations
// of 4 unrolled steps keeps the body small enough to run from the
// instruction cache (each launch runs it once).
__device__ __forceinline__ void diag_factor(const double (*T)[PP], int kb, double (&v)[4][4], double (&dr)[4],
                                            double (*bv)[2][NB]) {
  const int tid = threadIdx.x;
  const int rb_ = 4 * (tid >> 4), cb_ = 4 * (tid & 15);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int i = rb_ + r, j = cb_ + c;
      const bool in = i < kb && j < kb;
      const double t = T[i > j ? i : j][i > j ? j : i];
      v[r][c] = in ? t : (i == j ? 1.0 : 0.0);
    }
#pragma unroll
  for (int r = 0; r < 4; ++r) dr[r] = 1.0;
#pragma nounroll
  for (int jb = 0; jb < NB; jb += 4) {
    static_for<0, 2>([&](auto hc) {
      constexpr int q0 = 2 * decltype(hc)::value;  // rows jb + q0, jb + q0 + 1
      constexpr int b = decltype(hc)::value;       // LDS buffer of this round
      const int j = jb + q0;
      const bool own_row = rb_ == jb, own_col = cb_ == jb;
      if (own_row) {
        *reinterpret_cast<double2*>(&bv[b][0][cb_]) = double2{v[q0][0], v[q0][1]};
        *reinterpret_cast<double2*>(&bv[b][0][cb_ + 2]) = double2{v[q0][2], v[q0][3]};
        *reinterpret_cast<double2*>(&bv[b][1][cb_]) = double2{v[q0 + 1][0], v[q0 + 1][1]};
        *reinterpret_cast<double2*>(&bv[b][1][cb_ + 2]) = double2{v[q0 + 1][2], v[q0 + 1][3]};
      }
      __syncthreads();
      const double pa = bv[b][0][j], pb = bv[b][0][j + 1], pc = bv[b][1][j + 1];
      double r0[4], c0[4], r1[4], c1[4];
      {
        const double2 a01 = *reinterpret_cast<const double2*>(&bv[b][0][rb_]);
        const double2 a23 = *reinterpret_cast<const double2*>(&bv[b][0][rb_ + 2]);
        const double2 b01 = *reinterpret_cast<const double2*>(&bv[b][0][cb_]);
        const double2 b23 = *reinterpret_cast<const double2*>(&bv[b][0][cb_ + 2]);
        const double2 e01 = *reinterpret_cast<const double2*>(&bv[b][1][rb_]);
        const double2 e23 = *reinterpret_cast<const double2*>(&bv[b][1][rb_ + 2]);
        const double2 f01 = *reinterpret_cast<const double2*>(&bv[b][1][cb_]);
        const double2 f23 = *reinterpret_cast<const double2*>(&bv[b][1][cb_ + 2]);
        r0[0] = a01.x, r0[1] = a01.y, r0[2] = a23.x, r0[3] = a23.y;
        c0[0] = b01.x, c0[1] = b01.y, c0[2] = b23.x, c0[3] = b23.y;
        r1[0] = e01.x, r1[1] = e01.y, r1[2] = e23.x, r1[3] = e23.y;
        c1[0] = f01.x, c1[1] = f01.y, c1[2] = f23.x, c1[3] = f23.y;
      }
      // step j
      const double rp = recip(pa);
      dr[q0] = own_row ? pa : dr[q0];
      double m[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = (rb_ + r > j) ? r0[r] * rp : 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const double nv = fma(-m[r], c0[c], v[r][c]);
          if (c == q0) {
            const double ycol = (r == q0 && own_row) ? 1.0 : -m[r];
            v[r][c] = own_col ? ycol : nv;
          } else {
            v[r][c] = nv;
          }
        }
      // row j+1 after step j: multiplier f = a(j+1, j) / a(j, j); column j
      // becomes Y's entry -f
      const double f = pb * rp;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        r1[t] = (rb_ + t == j) ? -f : fma(-f, r0[t], r1[t]);
        c1[t] = (cb_ + t == j) ? -f : fma(-f, c0[t], c1[t]);
      }
      const double pc1 = fma(-f, pb, pc);
      // step j+1
      const double rp1 = recip(pc1);
      dr[q0 + 1] = own_row ? pc1 : dr[q0 + 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) m[r] = (rb_ + r > j + 1) ? r1[r] * rp1 : 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const double nv = fma(-m[r], c1[c], v[r][c]);
          if (c == q0 + 1) {
            const double ycol = (r == q0 + 1 && own_row) ? 1.0 : -m[r];
            v[r][c] = own_col ? ycol : nv;
          } else {
            v[r][c] = nv;
          }
        }
    });
  }
}

struct StepArgs {
  const double* A;
  double* R;
  double* LT;
  int d, k0, kb0, kb1;
  int nrow, ncol, ntile;  // nrow row tiles, ncol column tiles below s0, then 2 more when kb1 > 0
};

// The tile's operands for block k0 (A_ik0 or R_k0c; nothing for the two
// column tiles inside the first block) and for block k1 (A_ik1 or R_k1c).
__device__ __forceinline__ void step_load(const StepArgs& g, int tb, double (&c0v)[8], double (&c1v)[8]) {
  const int tid = threadIdx.x, d = g.d, k1 = g.k0 + NB;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int e = tid + 256 * t;
    if (tb < g.nrow) {
      const int i0 = g.k0 + g.kb0 + g.kb1 + 32 * tb;
      const int ii = e >> 6, mm = e & 63;  // A[i0 + ii][k0 + mm], A[i0 + ii][k1 + mm]
      const bool ok0 = i0 + ii < d && mm < g.kb0;
      const bool ok1 = i0 + ii < d && mm < g.kb1;
      c0v[t] = g.A[ok0 ? int64_t(i0 + ii) * d + g.k0 + mm : 0];
      c0v[t] = ok0 ? c0v[t] : 0.0;
      c1v[t] = g.A[ok1 ? int64_t(i0 + ii) * d + k1 + mm : 0];
      c1v[t] = ok1 ? c1v[t] : 0.0;
    } else {
      const int c0 = 32 * (tb - g.nrow);
      const int ii = e >> 5, cc = e & 31;  // R[k0 + ii][c0 + cc], R[k1 + ii][c0 + cc]
      const bool ok0 = tb < g.nrow + g.ncol && ii < g.kb0;
      const bool ok1 = ii < g.kb1;
      c0v[t] = g.R[ok0 ? int64_t(g.k0 + ii) * d + c0 + cc : 0];
      c0v[t] = ok0 ? c0v[t] : 0.0;
      c1v[t] = g.R[ok1 ? int64_t(k1 + ii) * d + c0 + cc : 0];
      c1v[t] = ok1 ? c1v[t] : 0.0;
    }
  }
}

// One tile of both blocks, its operands in c0v / c1v. XT0, XT1 hold
// X_k0^T, X_k1^T; Lk[m][i] = L[k1 + i][k0 + m]. Begins after a barrier and
// ends with one.
__device__ __forceinline__ void step_tile(const StepArgs& g, int tb, const double (&c0v)[8], const double (&c1v)[8],
                                          const double (*XT0)[PP], const double (*XT1)[PP], const double (*Lk)[PP],
                                          double (*Lo)[PQ], double* Cs) {
  const int tid = threadIdx.x, wave = tid >> 6, d = g.d, k1 = g.k0 + NB;
  // Every product runs over all 64 k, a compile-time count the compiler
  // unrolls and pipelines: the operands are zero past kb0 / kb1 (the tile
  // loads zero-fill, X^T and L_k1k0 are zero outside the block).
  const bool two = g.kb1 > 0;
  doublex4 acc[2];
  if (tb < g.nrow) {
    // output 32 x 64 per block: wave w owns rows 0..31 of column block w
    const int i0 = g.k0 + g.kb0 + g.kb1 + 32 * tb;
    const int ri[2] = {0, 16};
    const int cj[2] = {16 * wave, 16 * wave};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = tid + 256 * t;
      Cs[(e >> 6) * PP + (e & 63)] = c0v[t];  // A_ik0
    }
    __syncthreads();
    zero(acc);
    blocks_mma<2, false>(acc, Cs, PP, &XT0[0][0], PP, ri, cj, NB);
    // transpose through LDS, then coalesced stores: Lo[m][i] = L_ik0
    blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { Lo[j][i] = s; });
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = tid + 256 * t, m = e >> 5, i = e & 31;
      if (m < g.kb0 && i0 + i < d) g.LT[int64_t(m) * d + i0 + i] = Lo[m][i];
    }
    if (two) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = tid + 256 * t;
        Cs[(e >> 6) * PP + (e & 63)] = c1v[t];  // A_ik1
      }
      __syncthreads();
      zero(acc);
      blocks_mma<2, true>(acc, &Lo[0][0], PQ, &Lk[0][0], PP, ri, cj, NB);
      blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { Cs[i * PP + j] -= s; });
      __syncthreads();
      zero(acc);
      blocks_mma<2, false>(acc, Cs, PP, &XT1[0][0], PP, ri, cj, NB);
      blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { Lo[j][i] = s; });  // L_ik1
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = tid + 256 * t, m = e >> 5, i = e & 31;
        if (m < g.kb1 && i0 + i < d) g.LT[int64_t(NB + m) * d + i0 + i] = Lo[m][i];
      }
    }
  } else {
    // output 64 x 32 per block: wave w owns row block w, both column blocks
    const int c0 = 32 * (tb - g.nrow);
    const int ri[2] = {16 * wave, 16 * wave};
    const int cj[2] = {0, 16};
    if (tb < g.nrow + g.ncol) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = tid + 256 * t;
        Cs[(e >> 5) * PQ + (e & 31)] = c0v[t];  // R_k0c
      }
      __syncthreads();
      // X_k0c = X_k0 C, the A operand X_k0[i][m] read k-major from X_k0^T
      zero(acc);
      blocks_mma<2, true>(acc, &XT0[0][0], PP, Cs, PQ, ri, cj, NB);
      blocks_for_each(acc, ri, cj, [&](int i, int j, double s) {
        Lo[i][j] = s;
        if (i < g.kb0) g.R[int64_t(g.k0 + i) * d + c0 + j] = s;
      });
    } else {
      // inside the first block: X_k0c is X_k0 itself (zero above its diagonal)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = tid + 256 * t, m = e >> 5, c = e & 31;
        Lo[m][c] = XT0[c0 - g.k0 + c][m];
      }
    }
    if (two) {
      __syncthreads();
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int e = tid + 256 * t;
        Cs[(e >> 5) * PQ + (e & 31)] = c1v[t];  // R_k1c
      }
      __syncthreads();
      zero(acc);
      blocks_mma<2, true>(acc, &Lk[0][0], PP, &Lo[0][0], PQ, ri, cj, NB);
      blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { Cs[i * PQ + j] -= s; });
      __syncthreads();
      zero(acc);
      blocks_mma<2, true>(acc, &XT1[0][0], PP, Cs, PQ, ri, cj, NB);
      blocks_for_each(acc, ri, cj, [&](int i, int j, double s) {
        if (i < g.kb1) g.R[int64_t(k1 + i) * d + c0 + j] = s;
      });
    }
  }
  __syncthreads();  // the next tile overwrites Lo and Cs
}

// X = D^-1/2 Y of one factorization (zero above the diagonal and past kb),
// stored transposed in XT; workgroup 0 also writes it into R's diagonal
// block at k and reports a pivot that is not positive (NaN included) as one
// plus its index in H. Every thread has read the factorization's input from
// XT before the factorization's first barrier.
__device__ __forceinline__ void diag_finish(const StepArgs& g, int k, int kb, const double (&v)[4][4],
                                            const double (&dr)[4], double (*XT)[PP], int* bad,
                                            int32_t* __restrict__ info) {
  const int tid = threadIdx.x;
  const int rb_ = 4 * (tid >> 4), cb_ = 4 * (tid & 15);
  if (blockIdx.x == 0) {
    if (tid == 0) *bad = NB;
    __syncthreads();
    if (cb_ == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (rb_ + r < kb && !(dr[r] > 0.0)) atomicMin(bad, rb_ + r);
    }
    __syncthreads();
    if (tid == 0 && *bad < NB) atomicCAS(reinterpret_cast<int*>(info), 0, 1 + (g.d - 1 - (k + *bad)));
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = rb_ + r;
    const double si = 1.0 / sqrt(dr[r]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = cb_ + c;
      const double x = (i < kb && j <= i) ? v[r][c] * si : 0.0;
      XT[j][i] = x;
      if (blockIdx.x == 0 && i < kb && j < kb) g.R[int64_t(k + i) * g.d + k + j] = x;
    }
  }
  __syncthreads();
}

// Grid: min(ntile, STEP_MAX_WG) workgroups (at least 1); workgroup b takes
// tiles b, b + grid, ...
__global__ void __launch_bounds__(256)
hinv_step(const StepArgs g, int32_t* __restrict__ info) {
  __shared__ double XT0[NB][PP];  // A_k0k0 during its factorization, then X_k0^T
  __shared__ double XT1[NB][PP];  // A_k1k1 during its factorization, then X_k1^T
  __shared__ double Lk[NB][PP];   // A_k1k0 (row-major), then Lk[m][i] = L[k1 + i][k0 + m]
  __shared__ double Lo[NB][PQ];   // the tile's L_ik0 (Lo[m][i]) or X_k0c (Lo[m][c])
  __shared__ double Cs[NB * PQ];  // the tile's C: 32 x 64 at pitch PP (rows) or 64 x 32 at pitch PQ (columns)
  __shared__ __attribute__((aligned(16))) double bv[2][2][NB];
  __shared__ int bad;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int d = g.d, k0 = g.k0, k1 = k0 + NB, kb0 = g.kb0, kb1 = g.kb1;
  constexpr int PER = NB * NB / 256;
  {
    double a00[PER], a10[PER], a11[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int e = tid + 256 * t, i = e >> 6, j = e & 63;
      const bool ok00 = i < kb0 && j <= i;
      const bool ok10 = i < kb1;
      const bool ok11 = i < kb1 && j <= i;
      a00[t] = g.A[ok00 ? int64_t(k0 + i) * d + k0 + j : int64_t(k0) * d + k0];
      a10[t] = g.A[ok10 ? int64_t(k1 + i) * d + k0 + j : int64_t(k0) * d + k0];
      a11[t] = g.A[ok11 ? int64_t(k1 + i) * d + k1 + j : int64_t(k0) * d + k0];
    }
#pragma unroll
    for (int t = 0; t < PER; ++t) {
      const int e = tid + 256 * t, i = e >> 6, j = e & 63;
      XT0[i][j] = (i < kb0 && j <= i) ? a00[t] : 0.0;
      Lk[i][j] = i < kb1 ? a10[t] : 0.0;
      XT1[i][j] = (i < kb1 && j <= i) ? a11[t] : 0.0;
    }
  }
  __syncthreads();
  double v[4][4], dr[4];
  diag_factor(XT0, kb0, v, dr, bv);
  diag_finish(g, k0, kb0, v, dr, XT0, &bad, info);
  if (kb1 > 0) {
    // L_k1k0 = A_k1k0 X_k0^T: wave w, rows 16 w .. + 16, all four column
    // blocks; Lk <- its transpose once every wave has read A_k1k0; then
    // A_k1k1 -= L_k1k0 L_k1k0^T.
    doublex4 acc[4];
    zero(acc);
    const int ri[4] = {16 * wave, 16 * wave, 16 * wave, 16 * wave};
    const int cj[4] = {0, 16, 32, 48};
    blocks_mma<4, false>(acc, &Lk[0][0], PP, &XT0[0][0], PP, ri, cj, NB);
    __syncthreads();
    blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { Lk[j][i] = s; });
    __syncthreads();
    zero(acc);
    blocks_mma<4, true>(acc, &Lk[0][0], PP, &Lk[0][0], PP, ri, cj, NB);
    blocks_for_each(acc, ri, cj, [&](int i, int j, double s) { XT1[i][j] -= s; });
    __syncthreads();
    diag_factor(XT1, kb1, v, dr, bv);
    diag_finish(g, k1, kb1, v, dr, XT1, &bad, info);
  }
  for (int tb = int(blockIdx.x); tb < g.ntile; tb += int(gridDim.x)) {
    double c0v[8], c1v[8];
    step_load(g, tb, c0v, c1v);
    step_tile(g, tb, c0v, c1v, XT0, XT1, Lk, Lo, Cs);
  }
}

// ---------------------------------------------------------- trailing step
// After the super-panel S = [s0, s1) (K = s1 - s0 = KS), with T x T tiles:
//   blocks [0, nA):   A tiles (lower part only):  A_ij -= L_iS L_jS^T
//                     either the lower triangle of tiles from (ra0, ra0), or
//                     a rectangle from (ra0, ca0)
//   blocks [nA, ..):  R tiles, rows from rr0, columns T tc < s1:
//                     R_ic -= L_iS X_Sc
// With p0 < s0 the tile first applies the earlier super-panel P = [p0, s0)
// from its own panel buffer LT0 (A_ij -= L_iP L_jP^T; R_ic -= L_iP X_Pc for
// tiles left of s0, since X_Pc is zero for c >= s0), accumulating both in the
// same registers: K = (s0 - p0) + (s1 - s0), in the order P then S.
// Each wave owns a (T/2) x (T/2) quarter (T = 128: 16 independent MFMA
// chains; T = 64, used when big tiles would leave CUs idle: 4 chains; T = 32,
// for the latency-bound look-ahead update: 1 chain). The operands (L_S
// column-major in LT; X_S as rows s0.. of R) pass through LDS in chunks of TK
// k (16 for the bulk update, 32 for the look-ahead); the next chunk's loads
// are in flight while the current one is multiplied. The accumulators start
// from the old tile, so it is read once and written once.
struct TrailSpec {
  int s0, s1;     // the super-panel whose columns are applied (K = s1 - s0)
  int ra0, naR;   // A part: first row (and, if tri, first column), tile rows
  int ca0, naC;   // A part: first column and tile columns of a rectangle; naC = 0: lower triangle
  int rr0, nrR;   // R part: first row, tile rows (columns: tiles 0 .. s1 / T)
  int p0;         // earlier super-panel [p0, s0) applied first; p0 = s0: none
};
template <int T, int TK>
__device__ __forceinline__ void trail_tile(double* __restrict__ A, double* __restrict__ R, const double* __restrict__ LT0,
                                           const double* __restrict__ LT, int d, const TrailSpec& sp, int tile,
                                           double (*As)[T + 4],
                                           double (*Bs)[T + 4]) {
  constexpr int BL = T / 32;           // 16x16 blocks per wave dimension
  constexpr int STEP = 256 / T;        // k rows loaded per pass
  constexpr int U = TK / STEP;         // loads per thread per chunk and operand
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int lr = lane & 15, lk = lane >> 4;
  const int s0 = sp.s0, s1 = sp.s1;
  const bool tri = sp.naC == 0;
  const int nA = tri ? sp.naR * (sp.naR + 1) / 2 : sp.naR * sp.naC;
  int b = tile;
  const bool apart = b < nA;
  int r0, c0;
  if (apart) {
    if (tri) {
      int ti = 0;
      while (b > ti) {
        b -= ti + 1;
        ++ti;
      }
      r0 = sp.ra0 + T * ti;
      c0 = sp.ra0 + T * b;
    } else {
      r0 = sp.ra0 + T * (b / sp.naC);
      c0 = sp.ca0 + T * (b % sp.naC);
      if (c0 > r0 + T - 1) return;  // entirely above the diagonal (whole workgroup)
    }
  } else {
    b -= nA;
    r0 = sp.rr0 + T * (b % sp.nrR);
    c0 = T * (b / sp.nrR);
  }
  double* __restrict__ M = apart ? A : R;
  // k runs over [0, K0) for the earlier super-panel (R tiles at or right of
  // s0 take none of it), then over [K0, K) for S
  const int K0 = (apart || c0 < s0) ? s0 - sp.p0 : 0;
  const int K = K0 + (s1 - s0);
  // chunk loads: thread t covers column t % T of k rows t / T + STEP u,
  // at per-thread bases plus a chunk offset that is the same for all threads
  const int li = tid % T, lk0 = tid / T;
  const int ga = r0 + li < d ? r0 + li : d - 1;
  const int gb = c0 + li < d ? c0 + li : d - 1;
  const double* __restrict__ srcA = LT0 + ga;
  const double* __restrict__ srcB = apart ? LT0 + gb : R + gb;
  const int64_t dLT = LT - LT0;
  auto chunk = [&](int kc, int64_t& oa, int64_t& ob) {
    if (kc < K0) {
      oa = int64_t(kc) * d;
      ob = apart ? oa : int64_t(sp.p0 + kc) * d;
    } else {
      oa = dLT + int64_t(kc - K0) * d;
      ob = apart ? oa : int64_t(s0 + kc - K0) * d;
    }
  };
  double la[U], lb[U];
  {
    int64_t oa, ob;
    chunk(0, oa, ob);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = int64_t(lk0 + STEP * u) * d;
      la[u] = srcA[oa + o];
      lb[u] = srcB[ob + o];
    }
  }
  // old tile into the accumulators (clamped addresses; rows past d and the
  // upper half of diagonal A tiles are computed but never stored)
  const int rw = r0 + (T / 2) * wr, cw = c0 + (T / 2) * wc;
  doublex4 acc[BL][BL];
#pragma unroll
  for (int ii = 0; ii < BL; ++ii)
#pragma unroll
    for (int jj = 0; jj < BL; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int gi = rw + ii * 16 + lk + 4 * r, gj = cw + jj * 16 + lr;
        gi = gi < d ? gi : d - 1;
        gj = gj < d ? gj : d - 1;
        acc[ii][jj][r] = M[int64_t(gi) * d + gj];
      }
  for (int kc = 0; kc < K; kc += TK) {
    __syncthreads();  // the previous chunk's products are done
#pragma unroll
    for (int u = 0; u < U; ++u) {
      As[lk0 + STEP * u][li] = -la[u];
      Bs[lk0 + STEP * u][li] = lb[u];
    }
    __syncthreads();
    if (kc + TK < K) {
      int64_t oa, ob;
      chunk(kc + TK, oa, ob);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t o = int64_t(lk0 + STEP * u) * d;
        la[u] = srcA[oa + o];
        lb[u] = srcB[ob + o];
      }
    }
#pragma unroll
    for (int k = 0; k < TK; k += 4) {
      double a[BL], bb[BL];
#pragma unroll
      for (int t = 0; t < BL; ++t) {
        a[t] = As[k + lk][(T / 2) * wr + 16 * t + lr];
        bb[t] = Bs[k + lk][(T / 2) * wc + 16 * t + lr];
      }
#pragma unroll
      for (int ii = 0; ii < BL; ++ii)
#pragma unroll
        for (int jj = 0; jj < BL; ++jj) acc[ii][jj] = mfma64(a[ii], bb[jj], acc[ii][jj]);
    }
  }
#pragma unroll
  for (int ii = 0; ii < BL; ++ii)
#pragma unroll
    for (int jj = 0; jj < BL; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = rw + ii * 16 + lk + 4 * r, gj = cw + jj * 16 + lr;
        const bool keep = gi < d && (apart ? gj <= gi : gj < s1);
        if (keep) M[int64_t(gi) * d + gj] = acc[ii][jj][r];
      }
}

// One tile per workgroup; TK = k per LDS chunk.
template <int T, int TK>
__global__ void __launch_bounds__(256, 2)
hinv_trail(double* __restrict__ A, double* __restrict__ R, const double* __restrict__ LT0,
           const double* __restrict__ LT, int d, TrailSpec sp) {
  __shared__ double As[TK][T + 4];  // As[k][i] = -L[r0 + i][s0 + k]
  __shared__ double Bs[TK][T + 4];  // Bs[k][j] = L[c0 + j][s0 + k] or X[s0 + k][c0 + j]
  trail_tile<T, TK>(A, R, LT0, LT, d, sp, blockIdx.x, As, Bs);
}

// U[i][j] = X[d-1-i][d-1-j] for i <= j, 0 below the diagonal.
__global__ void __launch_bounds__(256)
hinv_write_u(const double* __restrict__ R, int d, float* __restrict__ U) {
  const int64_t n = int64_t(d) * d;
  for (int64_t e = blockIdx.x * int64_t(256) + threadIdx.x; e < n; e += int64_t(gridDim.x) * 256) {
    const int i = int(e / d), j = int(e % d);
    U[e] = (i <= j) ? float(R[int64_t(d - 1 - i) * d + (d - 1 - j)]) : 0.f;
  }
}

// Panel buffers: super-panel p writes buffer p % NPANEL; the trailing
// updates of p and p + 1 read it (see the schedule at gptq_prepare_hinv).
constexpr int NPANEL = 7;

struct HinvWs {
  double *A, *R, *LT, *lam;
  size_t bytes;
};

HinvWs carve(void* ws, int64_t d) {
  HinvWs w{};
  const size_t mat = align_up(size_t(d) * d * sizeof(double), 256);
  const size_t panel = align_up(size_t(NPANEL) * KS * d * sizeof(double), 256);
  w.bytes = 2 * mat + panel + 256;
  if (ws != nullptr) {  // sizes only when there is no workspace yet
    char* p = static_cast<char*>(ws);
    w.A = reinterpret_cast<double*>(p);
    w.R = reinterpret_cast<double*>(p + mat);
    w.LT = reinterpret_cast<double*>(p + 2 * mat);
    w.lam = reinterpret_cast<double*>(p + 2 * mat + panel);
  }
  return w;
}

// Per-device auxiliary streams and events for the look-ahead (created once,
// kept until the process ends). Enqueueing a factorization holds a lock, so
// concurrent callers cannot interleave their event records.
struct AuxCtx {
  hipStream_t aux = nullptr, aux2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, join2 = nullptr, chain[NPANEL] = {}, strip2[NPANEL] = {},
             strip3[NPANEL] = {}, bulk[NPANEL] = {};
  bool ready = false;
};
std::mutex g_aux_mu;
AuxCtx g_aux[64];

AuxCtx* aux_context() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  AuxCtx& c = g_aux[dev];
  if (!c.ready) {
    if (hipStreamCreateWithFlags(&c.aux, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipStreamCreateWithFlags(&c.aux2, hipStreamNonBlocking) != hipSuccess) return nullptr;
    hipEvent_t* evs[3 + 4 * NPANEL] = {&c.fork, &c.join, &c.join2};
    for (int i = 0; i < NPANEL; ++i) {
      evs[3 + i] = &c.chain[i];
      evs[3 + NPANEL + i] = &c.strip2[i];
      evs[3 + 2 * NPANEL + i] = &c.strip3[i];
      evs[3 + 3 * NPANEL + i] = &c.bulk[i];
    }
    for (hipEvent_t* e : evs)
      if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess) return nullptr;
    c.ready = true;
  }
  return &c;
}

// bulk: the update beyond the next super-panel (throughput-bound: 128x128
// tiles while there are at least 4 per CU, 64x64 below that). The 128x128
// form moves 8 k per chunk: its LDS (17 KB) and registers (208) then leave
// room on a CU holding one of its workgroups for a super-panel step (136 KB,
// 288 registers) or a look-ahead workgroup, so the critical chain runs beside
// the bulk update instead of waiting for it to drain (with 16 k per chunk,
// 34 KB, the step fitted on no CU the bulk update occupied). d = 12288:
// factor 30.6 -> 29.0 ms.
// look-ahead: the next super-panel's strip (K = 256), on the critical path
// and bound by the latency of its dependent chunk loads: 32 k per chunk, and
// 32x32 tiles while 64x64 ones would not give every CU one. A non-null
// `done` is recorded by the launch itself, at the kernel's completion, which
// leaves no gap on the stream as a separate record does (if nothing is
// launched, it is recorded separately). Launch errors are left for
// hipGetLastError; the return value reports a failed separate record.
bool launch_trail(hipStream_t st, const HinvWs& w, const double* LT0, const double* LT, int d, TrailSpec sp,
                  bool bulk, hipEvent_t done = nullptr) {
  auto tiles = [&](int T, TrailSpec& q) -> int64_t {
    q = sp;
    const int rows = d - sp.ra0;
    q.naR = rows > 0 ? (rows + T - 1) / T : 0;
    if (sp.naC != 0) q.naC = (sp.naC + T - 1) / T;  // naC carries the column count in elements
    q.nrR = sp.nrR > 0 ? (sp.nrR + T - 1) / T : 0;  // nrR carries the row count in elements
    const int64_t nA = q.naC == 0 ? int64_t(q.naR) * (q.naR + 1) / 2 : int64_t(q.naR) * q.naC;
    return nA + int64_t(q.nrR) * (sp.s1 / T);
  };
  TrailSpec q;
  if (!bulk) {
    const int64_t n64 = tiles(64, q);
    if (n64 >= 256) {
      hipExtLaunchKernelGGL((hinv_trail<64, 32>), dim3(unsigned(n64)), dim3(256), 0, st, nullptr, done, 0, w.A, w.R,
                            static_cast<const double*>(LT0), static_cast<const double*>(LT), d, q);
      return true;
    }
    const int64_t n32 = tiles(32, q);
    if (n32 > 0) {
      hipExtLaunchKernelGGL((hinv_trail<32, 32>), dim3(unsigned(n32)), dim3(256), 0, st, nullptr, done, 0, w.A, w.R,
                            static_cast<const double*>(LT0), static_cast<const double*>(LT), d, q);
      return true;
    }
    return done == nullptr || hipEventRecord(done, st) == hipSuccess;
  }
  const int64_t n128 = tiles(128, q);
  if (n128 >= 4 * 256) {
    hipExtLaunchKernelGGL((hinv_trail<128, 8>), dim3(unsigned(n128)), dim3(256), 0, st, nullptr, done, 0, w.A, w.R,
                          static_cast<const double*>(LT0), static_cast<const double*>(LT), d, q);
    return true;
  }
  const int64_t n64 = tiles(64, q);
  if (n64 > 0) {
    hipExtLaunchKernelGGL((hinv_trail<64, 16>), dim3(unsigned(n64)), dim3(256), 0, st, nullptr, done, 0, w.A, w.R,
                          static_cast<const double*>(LT0), static_cast<const double*>(LT), d, q);
    return true;
  }
  return done == nullptr || hipEventRecord(done, st) == hipSuccess;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_prepare_hinv_workspace_size(int64_t d) {
  if (d < 1) return 0;
  return carve(nullptr, d).bytes;
}

// Schedule (S = the caller's stream, X and Y = the auxiliary streams).
// Strip q is super-panel q's columns of A (all rows below) and its rows of
// R. For each super-panel p = [s0, s1):
//   S: the super-panel step of p (writing the panel buffer LT[p % NPANEL])
//   S: "trail A": the super-panels that strip p + 1 still lacks, applied to it
//   X (and Y): after trail A, the rest of the trailing update, overlapping
//      the next super-panel steps on S
// Below PAIR_MIN_D ("single" form, X only): trail A applies p - 1 and p
// (K = 256; p alone for p = 0), and X applies p alone to strips p + 3 and
// beyond. Trail A of p waits for X's work of p - 2, the last other writer of
// strip p + 1.
// From PAIR_MIN_D on ("paired" form), the auxiliary streams work only at odd
// p and apply p - 1 and p together (K = 256), so each element of the
// trailing matrices is read and written once per two super-panels:
//   Y: strip p + 2 (event strip2), strip p + 3 (event strip3), then, once X
//      has finished the bulk update of p - 2 (event bulk), strips p + 4 and
//      p + 5 in one launch;
//   X: strips p + 6 and beyond (the bulk update, event bulk).
// X then runs the bulk updates back to back: nothing it waits for is behind
// its own previous launch, and S and Y do their work beside it. Trail A
// applies p - 1 and p for odd p and p alone for even p. It waits for Y's
// strip-(p + 1) update of p - 1 (strip2) for even p, and of p - 2 (strip3)
// for odd p. Each strip's updates form one chain: the bulk update of p - 6
// or p - 4 (X), Y's two-strip update of p - 4 or p - 2 (after that bulk
// update), Y's strip update of p - 2 or p (Y's order), trail A (its wait).
// A step waits, through this chain, for the bulk update that read the panel
// buffer it overwrites (seven buffers: step p + 7 overwrites p's).
// In both forms each auxiliary stream runs in order, so a wait also covers
// every kernel enqueued on that stream before the one waited for. Every
// strip receives every earlier super-panel exactly once before its step. U
// is the same to the bit in both forms: each element sees the same fp64
// MFMA sequence.
// Measured (factor alone): d = 12288, 27.9 ms; 29.0 ms when X itself did
// strips p + 2 to p + 5 between two bulk updates (one auxiliary stream);
// 30.6 ms with that and 16 k per chunk in the bulk update. d = 11008: 21.0,
// 21.9, 23.4 ms. d = 4096: 2.33 ms single, 2.43 ms paired (more launches per
// two super-panels).
constexpr int PAIR_MIN_D = 8192;
extern "C" int gptq_prepare_hinv(const float* H, int64_t d, double damp, float* U, float* lambda_out, int32_t* info,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (d < 1 || d > 65536 || H == nullptr || U == nullptr || info == nullptr) return GPTQ_E_INVALID_ARG;
  if (!(damp >= 0.0) || damp > 1e30) return GPTQ_E_INVALID_ARG;
  const HinvWs w = carve(ws, d);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_E_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int di = int(d);
  std::lock_guard<std::mutex> lock(g_aux_mu);
  AuxCtx* ctx = aux_context();

  hipStream_t x = ctx ? ctx->aux : s;
  hipStream_t y = ctx ? ctx->aux2 : s;
  // Under stream capture the events are recorded by hipEventRecord, whose
  // capture semantics are the documented ones; otherwise the launches of
  // trail A and of X's strip updates record their events themselves.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) return GPTQ_E_HIP;
  const bool by_launch = ctx && cap == hipStreamCaptureStatusNone;
  hipLaunchKernelGGL(hinv_lambda, dim3(1), dim3(256), 0, s, H, di, damp, w.lam, lambda_out, info);
  const int nb32 = (di + 31) / 32;
  const int nlow = nb32 * (nb32 + 1) / 2;
  int nup = 0;  // 4 upper 32x32 blocks per super-panel with two blocks
  for (int s0 = 0; s0 < di; s0 += KS)
    if ((di - s0 < KS ? di - s0 : KS) > NB) nup += 4;
  hipLaunchKernelGGL(hinv_setup, dim3(unsigned(nlow + nup)), dim3(256), 0, s, H, di, w.lam, w.A, w.R, nlow);
  if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  const bool paired = di >= PAIR_MIN_D;
  if (ctx) {
    if (hipEventRecord(ctx->fork, s) != hipSuccess || hipStreamWaitEvent(x, ctx->fork, 0) != hipSuccess)
      return GPTQ_E_HIP;
    if (paired && hipStreamWaitEvent(y, ctx->fork, 0) != hipSuccess) return GPTQ_E_HIP;
  }
  auto bound = [&](int a) { return a < di ? a : di; };
  // a trailing update on stream st, recording `ev` (by the launch when possible)
  auto update = [&](hipStream_t st, const double* LT0, const double* LT, TrailSpec sp, bool bulk,
                    hipEvent_t ev) -> bool {
    if (!launch_trail(st, w, LT0, LT, di, sp, bulk, by_launch ? ev : nullptr)) return false;
    if (launch_status() != GPTQ_OK) return false;
    return !ctx || by_launch || hipEventRecord(ev, st) == hipSuccess;
  };
  for (int p = 0, s0 = 0; s0 < di; ++p, s0 += KS) {
    const int s1 = bound(s0 + KS);
    double* LTw = w.LT + size_t(p % NPANEL) * KS * di;
    const int kb0 = s1 - s0 < NB ? s1 - s0 : NB;
    const int kb1 = s1 - s0 - kb0;
    const int nrow = (di - s1 + 31) / 32;
    const int ncol = s0 / 32;
    const int ntile = nrow + ncol + (kb1 > 0 ? 2 : 0);
    const int grid = ntile < 1 ? 1 : (ntile < STEP_MAX_WG ? ntile : STEP_MAX_WG);
    const StepArgs args{w.A, w.R, LTw, di, s0, kb0, kb1, nrow, ncol, ntile};
    hipLaunchKernelGGL(hinv_step, dim3(unsigned(grid)), dim3(256), 0, s, args, info);
    if (s1 < di) {
      const int s2 = bound(s1 + KS), s3 = bound(s2 + KS), s4 = bound(s3 + KS);
      const bool odd = (p & 1) != 0;
      const bool two = paired ? odd : p >= 1;  // trail A applies p - 1 too
      if (ctx && p >= 2) {
        hipEvent_t ev = (!paired || odd) ? ctx->strip3[(p - 2) % NPANEL] : ctx->strip2[(p - 1) % NPANEL];
        if (hipStreamWaitEvent(s, ev, 0) != hipSuccess) return GPTQ_E_HIP;
      }
      // trail A: columns [s1, s2) of A (all rows below), rows [s1, s2) of R
      const int p0 = two ? s0 - KS : s0;
      const double* LT0 = two ? w.LT + size_t((p - 1) % NPANEL) * KS * di : LTw;
      if (!launch_trail(s, w, LT0, LTw, di, TrailSpec{s0, s1, s1, 0, s1, s2 - s1, s1, s2 - s1, p0}, false,
                        by_launch ? ctx->chain[p % NPANEL] : nullptr))
        return GPTQ_E_HIP;
      if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
      if (ctx && !by_launch && hipEventRecord(ctx->chain[p % NPANEL], s) != hipSuccess) return GPTQ_E_HIP;
      if (!paired) {
        // X: p applied to strips p + 3 and beyond (A at and beyond s3, lower
        // triangle; R rows from s3), after trail A
        if (ctx && hipStreamWaitEvent(x, ctx->chain[p % NPANEL], 0) != hipSuccess) return GPTQ_E_HIP;
        if (s3 < di) launch_trail(x, w, LTw, LTw, di, TrailSpec{s0, s1, s3, 0, 0, 0, s3, di - s3, s0}, true);
        if (ctx && hipEventRecord(ctx->strip3[p % NPANEL], x) != hipSuccess) return GPTQ_E_HIP;
      } else if (odd && s2 < di) {
        // p - 1 and p applied to the rest of the trailing matrices, once
        // trail A is done: Y takes strips p + 2 and p + 3 (each a launch of
        // its own, as trail A of p + 1 and p + 2 wait for them), then strips
        // p + 4 and p + 5 after X's bulk update of p - 2 (their last other
        // writer); X takes the lower triangle of A from s6 and R's rows from
        // s6.
        const int s5 = bound(s4 + KS), s6 = bound(s5 + KS);
        hipEvent_t e2 = ctx ? ctx->strip2[p % NPANEL] : nullptr, e3 = ctx ? ctx->strip3[p % NPANEL] : nullptr;
        hipEvent_t eb = ctx ? ctx->bulk[p % NPANEL] : nullptr;
        if (ctx && hipStreamWaitEvent(y, ctx->chain[p % NPANEL], 0) != hipSuccess) return GPTQ_E_HIP;
        if (!update(y, LT0, LTw, TrailSpec{s0, s1, s2, 0, s2, s3 - s2, s2, s3 - s2, p0}, false, e2))
          return GPTQ_E_HIP;
        if (!update(y, LT0, LTw, TrailSpec{s0, s1, s3, 0, s3, s4 - s3, s3, s4 - s3, p0}, false, e3))
          return GPTQ_E_HIP;
        if (s4 < di) {
          if (ctx && p >= 3 && hipStreamWaitEvent(y, ctx->bulk[(p - 2) % NPANEL], 0) != hipSuccess)
            return GPTQ_E_HIP;
          launch_trail(y, w, LT0, LTw, di, TrailSpec{s0, s1, s4, 0, s4, s6 - s4, s4, s6 - s4, p0}, false);
        }
        if (ctx && hipStreamWaitEvent(x, ctx->chain[p % NPANEL], 0) != hipSuccess) return GPTQ_E_HIP;
        if (!update(x, LT0, LTw, TrailSpec{s0, s1, s6, 0, 0, 0, s6, di - s6, p0}, true, eb)) return GPTQ_E_HIP;
      }
    }
    if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  }
  if (ctx) {
    if (hipEventRecord(ctx->join, x) != hipSuccess || hipStreamWaitEvent(s, ctx->join, 0) != hipSuccess)
      return GPTQ_E_HIP;
    if (paired &&
        (hipEventRecord(ctx->join2, y) != hipSuccess || hipStreamWaitEvent(s, ctx->join2, 0) != hipSuccess))
      return GPTQ_E_HIP;
  }
  hipLaunchKernelGGL(hinv_write_u, dim3(2048), dim3(256), 0, s, w.R, di, U);
  return launch_status();
}
