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
// L and X = L^-1 are computed together by a right-looking blocked
// elimination in fp64 (panel width 64):
//   diag   (1 workgroup): L_kk = chol(A_kk) and X_kk = L_kk^-1 in LDS; a
//          pivot that is not positive sets `info`.
//   panel  (many):        L_ik = A_ik X_kk^T            for row blocks i > k
//                         X[k, :k] = X_kk R[k, :k]      (block row k of X)
//   update (many):        A_ij -= L_ik L_jk^T           (trailing lower part)
//                         R[i, :k+1] -= L_ik X[k, :k+1] (rows i > k)
// R starts as the identity; block row i of R becomes block row i of X once
// its own panel step runs. Each step's products are 64x64 tiles on the fp64
// MFMA (v_mfma_f64_16x16x4f64).
#include <utility>

#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int NB = 64;   // panel width
constexpr int LP = 68;   // LDS pitch (doubles) of 64-wide operand tiles

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

// A[i][j] = H[d-1-j][d-1-i] + lambda [i == j] for j <= i (reads H's lower
// triangle, which is the reversed matrix's lower triangle by symmetry);
// R = identity on and below the diagonal. One 32x32 lower block per group.
__global__ void __launch_bounds__(256)
hinv_setup(const float* __restrict__ H, int d, const double* __restrict__ lam, double* __restrict__ A,
           double* __restrict__ R) {
  __shared__ float t[32][33];
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
    const int64_t o = int64_t(i) * d + j;
    A[o] = double(t[jj][ii]) + (i == j ? l : 0.0);
    R[o] = (i == j) ? 1.0 : 0.0;
  }
}

// ------------------------------------------------------------ diag block
// Factor the kb x kb diagonal block at k0 and invert its factor. Schur form:
// step j eliminates column j with multipliers m_i = a_ij / a_jj, applied both
// to the trailing block (a_ic -= m_i a_cj, c in (j, i]) and to the unit-lower
// inverse Y (y_ic -= m_i y_jc, c <= j). Then L_ij = a_ij / sqrt(a_jj) and
// L^-1_ic = y_ic / sqrt(a_ii). Rows and columns past kb act as identity.
//
// Thread t owns row i = t / 4, columns c = t % 4 + 4 m (m < 16) of both a and
// y, in registers, for all 64 (fully unrolled) steps. Step j only exchanges
// column j of a and row j of y through LDS (double buffered: one barrier).
template <int Q, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Q < N) {
    f(std::integral_constant<int, Q>{});
    static_for<Q + 1, N>(f);
  }
}

__global__ void __launch_bounds__(256)
hinv_diag(double* __restrict__ A, double* __restrict__ R, int d, int k0, int kb, double* __restrict__ Lbuf,
          int32_t* __restrict__ info) {
  __shared__ double acol[2][NB];
  __shared__ double yrow[2][NB];
  __shared__ double dg[NB];
  const int tid = threadIdx.x;
  const int i_ = tid >> 2, c0_ = tid & 3;
  double av[NB / 4], yv[NB / 4];
  const int i = i_, c0 = c0_;
#pragma unroll
  for (int t = 0; t < NB / 4; ++t) {
    const int c = c0 + 4 * t;
    const bool in = i < kb && c <= i;
    const double v = A[in ? int64_t(k0 + i) * d + k0 + c : int64_t(k0) * d + k0];
    av[t] = in ? v : (i == c ? 1.0 : 0.0);
    yv[t] = (i == c) ? 1.0 : 0.0;
  }
  static_for<0, NB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int b = j & 1;
    // Fresh copies of the lane indices each step, so the compiler computes
    // this step's comparisons here instead of keeping all 64 steps' live.
    int i = i_, c0 = c0_;
    asm volatile("" : "+v"(i), "+v"(c0));
    if (c0 == (j & 3)) acol[b][i] = av[j >> 2];  // column j of a (all rows)
    if (i == j) {
#pragma unroll
      for (int t = 0; t < NB / 4; ++t) yrow[b][c0 + 4 * t] = yv[t];  // row j of y
    }
    __syncthreads();
    const double piv = acol[b][j];
    if (tid == 0) {
      dg[j] = piv;
      if (j < kb && !(piv > 0.0)) atomicCAS(reinterpret_cast<int*>(info), 0, 1 + (d - 1 - (k0 + j)));
    }
    const double m = i > j ? acol[b][i] / piv : 0.0;
    static_for<0, NB / 4>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const int c = c0 + 4 * t;
      if constexpr (4 * t > j) {
        av[t] = fma(-m, acol[b][c], av[t]);
      } else if constexpr (4 * t + 3 <= j) {
        yv[t] = fma(-m, yrow[b][c], yv[t]);
      } else {
        const bool up = c > j;
        const double o = up ? acol[b][c] : yrow[b][c];
        const double nv = fma(-m, o, up ? av[t] : yv[t]);
        av[t] = up ? nv : av[t];
        yv[t] = up ? yv[t] : nv;
      }
    });
    // Materialize this step's updates now (otherwise the compiler defers the
    // fma chains and keeps every step's operands live).
#pragma unroll
    for (int t = 0; t < NB / 4; ++t) asm volatile("" : "+v"(av[t]), "+v"(yv[t]));
  });
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NB / 4; ++t) {
    const int c = c0 + 4 * t;
    double x = 0.0;
    if (i < kb && c <= i) {
      const double sc = sqrt(dg[c]), si = sqrt(dg[i]);
      const double l = (c == i) ? si : av[t] / sc;
      x = yv[t] / si;
      A[int64_t(k0 + i) * d + k0 + c] = l;
      R[int64_t(k0 + i) * d + k0 + c] = x;
    }
    Lbuf[i * NB + c] = x;  // X_kk, zero outside the kb x kb lower triangle
  }
}

// ------------------------------------------------------ 64x64 tile products
// Each of the 4 waves owns a 32x32 quarter (2x2 MFMA 16x16 blocks).
// Ls[i][k] (pitch LP) is the left operand, Rs[k][j] (pitch LP) the right one;
// K is a multiple of 4 (zero padded).
__device__ __forceinline__ void tile_mma(const double (*Ls)[LP], const double (*Rs)[LP], int K, doublex4 acc[2][2]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  for (int k = 0; k < K; k += 4) {
    double av[2], bv[2];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) av[ii] = Ls[wr * 32 + ii * 16 + (lane & 15)][k + (lane >> 4)];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) bv[jj] = Rs[k + (lane >> 4)][wc * 32 + jj * 16 + (lane & 15)];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[ii][jj] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ii], bv[jj], acc[ii][jj], 0, 0, 0);
  }
}

// Visit the wave's accumulator elements: f(row, col, value) in tile coords.
// v_mfma_f64_16x16x4f64 result layout: lane l, register r holds row
// (l / 16) + 4 r, column l % 16 of the 16x16 block.
template <typename F>
__device__ __forceinline__ void tile_for_each(doublex4 acc[2][2], F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        f(wr * 32 + ii * 16 + (lane >> 4) + 4 * r, wc * 32 + jj * 16 + (lane & 15), acc[ii][jj][r]);
}

// ------------------------------------------------------------ panel step
// Blocks [0, nrow): L_ik for row block i = k1 + 64 b (in place in A).
// Blocks [nrow, nrow + ncol): X[k, c0:c0+64] = X_kk R[k, c0:c0+64], c0 < k0
// (in place in R).
__global__ void __launch_bounds__(256)
hinv_panel(double* __restrict__ A, double* __restrict__ R, int d, int k0, int kb, const double* __restrict__ Lbuf,
           int nrow) {
  __shared__ double Ls[NB][LP];
  __shared__ double Rs[NB][LP];
  const int tid = threadIdx.x;
  const int k1 = k0 + kb;
  const int Kp = (kb + 3) & ~3;
  doublex4 acc[2][2];
#pragma unroll
  for (int ii = 0; ii < 2; ++ii)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[ii][jj] = doublex4{0, 0, 0, 0};
  if (int(blockIdx.x) < nrow) {
    const int r0 = k1 + NB * blockIdx.x;
    // left: A[r0+i][k0+m]; right[m][j] = X_kk[j][m]
    double v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + 256 * t;
      const int i = e / NB, m = e % NB;
      const bool ok = r0 + i < d && m < kb;
      v[t] = A[ok ? int64_t(r0 + i) * d + k0 + m : 0];
      v[t] = ok ? v[t] : 0.0;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + 256 * t;
      const int i = e / NB, m = e % NB;
      Ls[i][m] = v[t];
      Rs[m][i] = Lbuf[i * NB + m];
    }
    __syncthreads();
    tile_mma(Ls, Rs, Kp, acc);
    tile_for_each(acc, [&](int i, int j, double v) {
      if (r0 + i < d && j < kb) A[int64_t(r0 + i) * d + k0 + j] = v;
    });
  } else {
    const int c0 = NB * (blockIdx.x - nrow);
    // left: X_kk[i][m]; right[m][c] = R[k0+m][c0+c]
    double v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + 256 * t;
      const int i = e / NB, c = e % NB;
      const bool ok = i < kb && c0 + c < k0;
      v[t] = R[ok ? int64_t(k0 + i) * d + c0 + c : 0];
      v[t] = ok ? v[t] : 0.0;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int e = tid + 256 * t;
      const int i = e / NB, c = e % NB;
      Ls[i][c] = Lbuf[i * NB + c];
      Rs[i][c] = v[t];
    }
    __syncthreads();
    tile_mma(Ls, Rs, Kp, acc);
    tile_for_each(acc, [&](int i, int c, double v) {
      if (i < kb && c0 + c < k0) R[int64_t(k0 + i) * d + c0 + c] = v;
    });
  }
}

// ----------------------------------------------------------- update step
// UT x UT output tiles (UT = 128 while the trailing matrix is large, 64 near
// the end where a few big tiles would only add latency), K = kb <= 64. Each
// of the 4 waves owns a (UT/2) x (UT/2) quarter of MFMA 16x16 blocks.
// Operands are staged with every load issued before the first LDS store.
constexpr int UP = 66;   // pitch (doubles) of the [UT][K] left operand

// Stages a UT-row x 64-col fp64 block of M (rows r0.., cols k0..) into LDS,
// Ls[r][k] (transpose = false) or Ls[k][r] (transpose = true). Elements with
// row >= rmax or col >= k0 + kmax read as zero; all loads use clamped
// in-bounds addresses and are issued before anything is stored.
template <int UT, bool TRANSPOSE, typename Dst>
__device__ __forceinline__ void stage_block(Dst Ls, const double* __restrict__ M, int d, int r0, int rmax, int k0,
                                            int kmax) {
  constexpr int PER = UT * 64 / 256;
  const int tid = threadIdx.x;
  double v[PER];
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + 256 * t;
    const int r = e >> 6, k = e & 63;
    const bool ok = (r0 + r < rmax) && (k < kmax);
    v[t] = M[ok ? int64_t(r0 + r) * d + k0 + k : 0];
    v[t] = ok ? v[t] : 0.0;
  }
#pragma unroll
  for (int t = 0; t < PER; ++t) {
    const int e = tid + 256 * t;
    const int r = e >> 6, k = e & 63;
    if (TRANSPOSE)
      Ls[k][r] = v[t];
    else
      Ls[r][k] = v[t];
  }
}

template <int UT, int RQ>
__device__ __forceinline__ void tileU_mma(const double (*Ls)[UP], const double (*Rs)[RQ], int K,
                                          doublex4 acc[UT / 32][UT / 32]) {
  constexpr int BL = UT / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  for (int k = 0; k < K; k += 4) {
    double av[BL], bv[BL];
#pragma unroll
    for (int ii = 0; ii < BL; ++ii) av[ii] = Ls[wr * (UT / 2) + ii * 16 + (lane & 15)][k + (lane >> 4)];
#pragma unroll
    for (int jj = 0; jj < BL; ++jj) bv[jj] = Rs[k + (lane >> 4)][wc * (UT / 2) + jj * 16 + (lane & 15)];
#pragma unroll
    for (int ii = 0; ii < BL; ++ii)
#pragma unroll
      for (int jj = 0; jj < BL; ++jj)
        acc[ii][jj] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ii], bv[jj], acc[ii][jj], 0, 0, 0);
  }
}

// M[tile element] -= acc for the elements `keep` selects. All loads are
// issued unconditionally (masked-off ones read M[0]) before any store, so
// the tile costs one memory round trip; only the stores are masked.
// v_mfma_f64_16x16x4f64 layout: lane l, register r -> row l/16 + 4r, col l%16.
template <int UT, typename Keep>
__device__ __forceinline__ void rmw_sub(double* __restrict__ M, int d, int r0, int c0,
                                        doublex4 acc[UT / 32][UT / 32], Keep keep) {
  constexpr int BL = UT / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  double old[BL][BL][4];
#pragma unroll
  for (int ii = 0; ii < BL; ++ii)
#pragma unroll
    for (int jj = 0; jj < BL; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = r0 + wr * (UT / 2) + ii * 16 + (lane >> 4) + 4 * r;
        const int gj = c0 + wc * (UT / 2) + jj * 16 + (lane & 15);
        old[ii][jj][r] = M[keep(gi, gj) ? int64_t(gi) * d + gj : 0];
      }
#pragma unroll
  for (int ii = 0; ii < BL; ++ii)
#pragma unroll
    for (int jj = 0; jj < BL; ++jj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gi = r0 + wr * (UT / 2) + ii * 16 + (lane >> 4) + 4 * r;
        const int gj = c0 + wc * (UT / 2) + jj * 16 + (lane & 15);
        if (keep(gi, gj)) M[int64_t(gi) * d + gj] = old[ii][jj][r] - acc[ii][jj][r];
      }
}

// Blocks [0, nA): lower UT-tiles (ti >= tj) of the trailing matrix at k1:
//   A_ij -= L_i L_j^T.
// Blocks [nA, nA + nT * nC): R[k1 + UT ti, UT tc] -= L_i X[k, UT tc].
template <int UT>
__global__ void __launch_bounds__(256)
hinv_update(double* __restrict__ A, double* __restrict__ R, int d, int k0, int kb, int nT, int nC) {
  constexpr int RQ = UT + 4;
  constexpr int BL = UT / 32;
  __shared__ double Ls[UT][UP];
  __shared__ double Rs[NB][RQ];
  const int k1 = k0 + kb;
  const int Kp = (kb + 3) & ~3;
  const int nA = nT * (nT + 1) / 2;
  int b = blockIdx.x;
  doublex4 acc[BL][BL];
#pragma unroll
  for (int ii = 0; ii < BL; ++ii)
#pragma unroll
    for (int jj = 0; jj < BL; ++jj) acc[ii][jj] = doublex4{0, 0, 0, 0};
  if (b < nA) {
    int ti = 0;
    while (b > ti) {
      b -= ti + 1;
      ++ti;
    }
    const int tj = b;
    const int r0 = k1 + UT * ti, c0 = k1 + UT * tj;
    stage_block<UT, false>(Ls, A, d, r0, d, k0, kb);
    stage_block<UT, true>(Rs, A, d, c0, d, k0, kb);  // Rs[m][j] = L[c0 + j][k0 + m]
    __syncthreads();
    tileU_mma<UT, RQ>(Ls, Rs, Kp, acc);
    rmw_sub<UT>(A, d, r0, c0, acc, [&](int gi, int gj) { return gi < d && gj <= gi; });
  } else {
    b -= nA;
    const int ti = b / nC, tc = b % nC;
    const int r0 = k1 + UT * ti, c0 = UT * tc;
    stage_block<UT, false>(Ls, A, d, r0, d, k0, kb);
    {
      // Rs[m][c] = X[k0 + m][c0 + c]; X is lower triangular inside the
      // diagonal block (R's upper part is never written, so it is masked).
      constexpr int PER = 64 * UT / 256;
      const int tid = threadIdx.x;
      double v[PER];
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int e = tid + 256 * t;  // 64 rows x UT cols
        const int m = e / UT, c = e % UT;
        const int g = c0 + c;
        const bool ok = m < kb && g < k1 && g <= k0 + m;
        v[t] = R[ok ? int64_t(k0 + m) * d + g : 0];
        v[t] = ok ? v[t] : 0.0;
      }
#pragma unroll
      for (int t = 0; t < PER; ++t) {
        const int e = tid + 256 * t;
        Rs[e / UT][e % UT] = v[t];
      }
    }
    __syncthreads();
    tileU_mma<UT, RQ>(Ls, Rs, Kp, acc);
    rmw_sub<UT>(R, d, r0, c0, acc, [&](int gi, int gj) { return gi < d && gj < k1; });
  }
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

struct HinvWs {
  double *A, *R, *lam, *Lbuf;
  size_t bytes;
};

HinvWs carve(void* ws, int64_t d) {
  HinvWs w{};
  const size_t mat = align_up(size_t(d) * d * sizeof(double), 256);
  char* p = static_cast<char*>(ws);
  w.A = reinterpret_cast<double*>(p);
  w.R = reinterpret_cast<double*>(p + mat);
  w.lam = reinterpret_cast<double*>(p + 2 * mat);
  w.Lbuf = reinterpret_cast<double*>(p + 2 * mat + 256);
  w.bytes = 2 * mat + 256 + align_up(NB * NB * sizeof(double), 256);
  return w;
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_prepare_hinv_workspace_size(int64_t d) {
  if (d < 1) return 0;
  return carve(nullptr, d).bytes;
}

extern "C" int gptq_prepare_hinv(const float* H, int64_t d, double damp, float* U, float* lambda_out, int32_t* info,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (d < 1 || d > 65536 || H == nullptr || U == nullptr || info == nullptr) return GPTQ_E_INVALID_ARG;
  if (!(damp >= 0.0) || damp > 1e30) return GPTQ_E_INVALID_ARG;
  const HinvWs w = carve(ws, d);
  if (ws == nullptr || ws_bytes < w.bytes) return GPTQ_E_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int di = int(d);
  hipLaunchKernelGGL(hinv_lambda, dim3(1), dim3(256), 0, s, H, di, damp, w.lam, lambda_out, info);
  const int nb32 = (di + 31) / 32;
  hipLaunchKernelGGL(hinv_setup, dim3(unsigned(nb32 * (nb32 + 1) / 2)), dim3(256), 0, s, H, di, w.lam, w.A, w.R);
  if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  for (int k0 = 0; k0 < di; k0 += NB) {
    const int kb = di - k0 < NB ? di - k0 : NB;
    const int k1 = k0 + kb;
    hipLaunchKernelGGL(hinv_diag, dim3(1), dim3(256), 0, s, w.A, w.R, di, k0, kb, w.Lbuf, info);
    const int nrow = (di - k1 + NB - 1) / NB;
    const int ncol = (k0 + NB - 1) / NB;
    if (nrow + ncol > 0)
      hipLaunchKernelGGL(hinv_panel, dim3(unsigned(nrow + ncol)), dim3(256), 0, s, w.A, w.R, di, k0, kb, w.Lbuf,
                         nrow);
    // 128-wide update tiles while they fill the GPU, 64-wide near the end.
    const int rem = di - k1;
    const int n128 = (rem + 127) / 128;
    if (n128 * (n128 + 1) / 2 >= 256) {
      const int nT = n128, nC = (k1 + 127) / 128;
      const int nblk = nT * (nT + 1) / 2 + nT * nC;
      hipLaunchKernelGGL(hinv_update<128>, dim3(unsigned(nblk)), dim3(256), 0, s, w.A, w.R, di, k0, kb, nT, nC);
    } else {
      const int nT = (rem + 63) / 64, nC = (k1 + 63) / 64;
      const int nblk = nT * (nT + 1) / 2 + nT * nC;
      if (nblk > 0)
        hipLaunchKernelGGL(hinv_update<64>, dim3(unsigned(nblk)), dim3(256), 0, s, w.A, w.R, di, k0, kb, nT, nC);
    }
    if (launch_status() != GPTQ_OK) return GPTQ_E_HIP;
  }
  hipLaunchKernelGGL(hinv_write_u, dim3(2048), dim3(256), 0, s, w.R, di, U);
  return launch_status();
}
