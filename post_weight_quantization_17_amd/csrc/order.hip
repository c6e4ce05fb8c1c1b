// Column orders: the act-order permutation and row/column gathers.
//
// mcipr.com "一文读懂GPTQ", section 四: the library configuration of the
// method has a desc_act flag (act-order). Reading: the columns are quantized
// in order of descending diag(H) (ties by ascending column index, NaN last,
// -0 equal to +0), i.e. the fixed-order method runs on W[:, p] and
// H[p][:, p], with groups consecutive in that order. The permutation is a
// counting rank (position of i = number of columns that come before it),
// so it needs no sort and no workspace: each workgroup compares 256 columns
// with a slice of the diagonal held in LDS and adds its counts with integer
// atomics (order-independent, so deterministic). The gathers move the
// weights, the Hessian, the codes or the activations into or out of that
// order; every index is checked against the source extent.
#include "gptq_common.h"

namespace gptq {
namespace {

constexpr int RANK_THREADS = 256;
constexpr int RANK_SLICE = 256;  // diagonal entries per workgroup: d/256 x d/256 workgroups

// Key of a total order in which a larger key comes first: NaN -> 0 (after
// every number), -0 -> +0, otherwise the float's bits mapped monotonically
// onto the unsigned integers (at least 1 for every non-NaN value).
__device__ __forceinline__ uint32_t order_key(float v) {
  if (v != v) return 0u;
  if (v == 0.0f) v = 0.0f;
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// rank[i] += #{ j in this workgroup's slice : key_j > key_i, or key_j == key_i and j < i }
__global__ void __launch_bounds__(RANK_THREADS)
act_order_rank(const float* __restrict__ H, int64_t d, int64_t ldh, int32_t* __restrict__ rank) {
  __shared__ uint32_t ks[RANK_SLICE];
  const int64_t j0 = int64_t(blockIdx.y) * RANK_SLICE;
  const int nj = int(d - j0 < RANK_SLICE ? d - j0 : RANK_SLICE);
  for (int t = threadIdx.x; t < nj; t += RANK_THREADS) ks[t] = order_key(H[(j0 + t) * (ldh + 1)]);
  __syncthreads();
  const int64_t i = int64_t(blockIdx.x) * RANK_THREADS + threadIdx.x;
  if (i >= d) return;  // no barrier follows
  const uint32_t ki = order_key(H[i * (ldh + 1)]);
  int cnt = 0;
  for (int t = 0; t < nj; ++t) {
    const uint32_t kj = ks[t];
    cnt += (kj > ki) || (kj == ki && j0 + t < i);
  }
  if (cnt) atomicAdd(&rank[i], cnt);
}

// perm[rank[i]] = i. The ranks of a strict total order are a permutation of
// 0 .. d-1, so every write is in range and every entry is written once.
__global__ void act_order_scatter(const int32_t* __restrict__ rank, int64_t d, int32_t* __restrict__ perm) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < d; i += int64_t(gridDim.x) * blockDim.x)
    perm[rank[i]] = int32_t(i);
}

// dst[i][q] = src[row_idx[i]][col_idx[q]] (identity where an index array is
// NULL); an index outside the source writes 0 and sets *info = 1. One
// workgroup per destination row (grid-stride over rows), threads along the
// row: coalesced writes, reads gathered inside one source row. Used for
// source rows longer than the LDS staging buffer.
template <typename T>
__global__ void __launch_bounds__(256)
gather_kernel(const T* __restrict__ src, int64_t src_rows, int64_t src_cols, int64_t lds,
              const int32_t* __restrict__ ridx, int64_t rows, const int32_t* __restrict__ cidx, int64_t cols,
              T* __restrict__ dst, int64_t ldd, int32_t* __restrict__ info) {
  for (int64_t i = blockIdx.x; i < rows; i += gridDim.x) {
    const int64_t si = ridx ? int64_t(ridx[i]) : i;
    const bool rok = si >= 0 && si < src_rows;
    const T* srow = src + (rok ? si : 0) * lds;
    T* drow = dst + i * ldd;
    for (int64_t q = threadIdx.x; q < cols; q += blockDim.x) {
      const int64_t sq = cidx ? int64_t(cidx[q]) : q;
      const bool ok = rok && sq >= 0 && sq < src_cols;
      drow[q] = ok ? srow[sq] : T(0);
      if (!ok && info) *info = 1;
    }
  }
}

constexpr int GATHER_LDS_MAX = 65536;  // bytes of one staged source row

// Same result as gather_kernel, for source rows of at most GATHER_LDS_MAX
// bytes: the source row is first copied into LDS with coalesced loads (16
// bytes per lane when VEC: every row 16-byte aligned), then gathered from
// LDS. The dynamic LDS size is the row length rounded up to 16 bytes. The
// row index, and so every branch around the barriers, is uniform across
// the workgroup.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256)
gather_lds_kernel(const T* __restrict__ src, int64_t src_rows, int64_t src_cols, int64_t lds,
                  const int32_t* __restrict__ ridx, int64_t rows, const int32_t* __restrict__ cidx, int64_t cols,
                  T* __restrict__ dst, int64_t ldd, int32_t* __restrict__ info) {
  extern __shared__ uint4 stage4[];
  T* stage = reinterpret_cast<T*>(stage4);
  constexpr int V = 16 / sizeof(T);
  const int nc = int(src_cols);
  for (int64_t i = blockIdx.x; i < rows; i += gridDim.x) {
    const int64_t si = ridx ? int64_t(ridx[i]) : i;
    const bool rok = si >= 0 && si < src_rows;
    if (rok) {
      const T* srow = src + si * lds;
      int t0 = 0;
      if (VEC) {
        const uint4* s4 = reinterpret_cast<const uint4*>(srow);
        const int nv = nc / V;
        for (int t = threadIdx.x; t < nv; t += blockDim.x) stage4[t] = s4[t];
        t0 = nv * V;
      }
      for (int t = t0 + threadIdx.x; t < nc; t += blockDim.x) stage[t] = srow[t];
    }
    __syncthreads();
    T* drow = dst + i * ldd;
    for (int64_t q = threadIdx.x; q < cols; q += blockDim.x) {
      const int64_t sq = cidx ? int64_t(cidx[q]) : q;
      const bool ok = rok && sq >= 0 && sq < src_cols;
      drow[q] = ok ? stage[sq] : T(0);
      if (!ok && info) *info = 1;
    }
    __syncthreads();  // the next row overwrites the stage
  }
}

template <typename T>
int launch_gather(const void* src, int64_t src_rows, int64_t src_cols, int64_t lds, const int32_t* ridx,
                  int64_t rows, const int32_t* cidx, int64_t cols, void* dst, int64_t ldd, int32_t* info,
                  hipStream_t s) {
  const unsigned grid = unsigned(rows < 65536 ? rows : 65536);
  const T* sp = static_cast<const T*>(src);
  T* dp = static_cast<T*>(dst);
  const int64_t row_bytes = src_cols * int64_t(sizeof(T));
  if (row_bytes <= GATHER_LDS_MAX) {
    const size_t smem = align_up(size_t(row_bytes), 16);
    const bool vec = reinterpret_cast<uintptr_t>(src) % 16 == 0 && (lds * int64_t(sizeof(T))) % 16 == 0;
    if (vec)
      hipLaunchKernelGGL((gather_lds_kernel<T, true>), dim3(grid), dim3(256), smem, s, sp, src_rows, src_cols, lds,
                         ridx, rows, cidx, cols, dp, ldd, info);
    else
      hipLaunchKernelGGL((gather_lds_kernel<T, false>), dim3(grid), dim3(256), smem, s, sp, src_rows, src_cols, lds,
                         ridx, rows, cidx, cols, dp, ldd, info);
  } else {
    hipLaunchKernelGGL((gather_kernel<T>), dim3(grid), dim3(256), 0, s, sp, src_rows, src_cols, lds, ridx, rows, cidx,
                       cols, dp, ldd, info);
  }
  return launch_status();
}

}  // namespace
}  // namespace gptq

using namespace gptq;

extern "C" int gptq_act_order_perm(const float* H, int64_t d, int64_t ldh, int32_t* perm, int32_t* invperm,
                                   void* stream) {
  if (d < 1 || d > int64_t(65535) * RANK_SLICE || ldh < d || !H || !perm || !invperm) return GPTQ_E_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  const unsigned fb = unsigned(d / 256 + 1 < 4096 ? d / 256 + 1 : 4096);
  hipLaunchKernelGGL(fill_i32, dim3(fb), dim3(256), 0, s, invperm, d, 0);
  int st = launch_status();
  if (st != GPTQ_OK) return st;
  const dim3 grid(unsigned((d + RANK_THREADS - 1) / RANK_THREADS), unsigned((d + RANK_SLICE - 1) / RANK_SLICE));
  hipLaunchKernelGGL(act_order_rank, grid, dim3(RANK_THREADS), 0, s, H, d, ldh, invperm);
  if ((st = launch_status()) != GPTQ_OK) return st;
  hipLaunchKernelGGL(act_order_scatter, dim3(fb), dim3(256), 0, s, invperm, d, perm);
  return launch_status();
}

extern "C" int gptq_gather(const void* src, int elem_bytes, int64_t src_rows, int64_t src_cols, int64_t ld_src,
                           const int32_t* row_idx, int64_t rows, const int32_t* col_idx, int64_t cols, void* dst,
                           int64_t ld_dst, int32_t* info, void* stream) {
  if (!src || !dst || src_rows < 1 || src_cols < 1 || rows < 1 || cols < 1) return GPTQ_E_INVALID_ARG;
  if (ld_src < src_cols || ld_dst < cols) return GPTQ_E_INVALID_ARG;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4) return GPTQ_E_INVALID_ARG;
  hipStream_t s = as_stream(stream);
  if (info) {
    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(64), 0, s, info, int64_t(1), 0);
    const int st = launch_status();
    if (st != GPTQ_OK) return st;
  }
  switch (elem_bytes) {
    case 1:
      return launch_gather<uint8_t>(src, src_rows, src_cols, ld_src, row_idx, rows, col_idx, cols, dst, ld_dst, info,
                                    s);
    case 2:
      return launch_gather<uint16_t>(src, src_rows, src_cols, ld_src, row_idx, rows, col_idx, cols, dst, ld_dst, info,
                                     s);
    default:
      return launch_gather<uint32_t>(src, src_rows, src_cols, ld_src, row_idx, rows, col_idx, cols, dst, ld_dst, info,
                                     s);
  }
}
