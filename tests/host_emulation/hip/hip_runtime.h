// Host emulation of the part of the HIP execution model that the sweep
// kernels use, for bounds-checked CPU runs of the library's own kernel
// source under AddressSanitizer (test infrastructure, never part of the
// library).
//
// Every workgroup runs as blockDim.x host threads; workgroups run one after
// another, so `__shared__` arrays become function-local statics. The
// cross-lane builtins (DPP moves and the fp32 16x16x4 MFMA) exchange values
// through a per-wave buffer behind a 64-thread barrier, so every lane of a
// wave must reach them together, as on the hardware. Global memory is the
// caller's host memory: an access outside an allocation is an ASan report.
#pragma once

#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <thread>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __align__(n) __attribute__((aligned(n)))

struct dim3 {
  uint32_t x, y, z;
  constexpr dim3(uint32_t x_ = 1, uint32_t y_ = 1, uint32_t z_ = 1) : x(x_), y(y_), z(z_) {}
};

struct alignas(16) float4 {
  float x, y, z, w;
};
struct alignas(8) uint2 {
  uint32_t x, y;
};
inline float4 make_float4(float x, float y, float z, float w) { return float4{x, y, z, w}; }

typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
typedef struct ihipStream_t* hipStream_t;

namespace simt {

typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct Wave {
  std::barrier<> bar{64};
  uint32_t u32[2][64];
  float a[2][64], b[2][64];
};

struct Workgroup {
  explicit Workgroup(unsigned n) : bar(n), waves((n + 63) / 64) {
    for (auto& w : waves) w = std::make_unique<Wave>();
  }
  std::barrier<> bar;
  std::vector<std::unique_ptr<Wave>> waves;
};

inline thread_local dim3 tid, bid;
inline thread_local Workgroup* wg = nullptr;
inline thread_local unsigned phase = 0;
inline dim3 grid_dim, block_dim;

inline Wave& my_wave() { return *wg->waves[tid.x / 64]; }
inline int my_lane() { return int(tid.x % 64); }

// Source lane of a DPP move within the 64-lane wave (the controls the
// kernels use: quad_perm, row_mirror, row_half_mirror, row_newbcast).
inline int dpp_source(int lane, int ctrl) {
  const int row = lane & ~15, r = lane & 15;
  if (ctrl >= 0 && ctrl <= 0xFF) return (lane & ~3) | ((ctrl >> (2 * (lane & 3))) & 3);
  if (ctrl == 0x140) return row + (15 - r);
  if (ctrl == 0x141) return row + ((r & 8) | (7 - (r & 7)));
  if (ctrl >= 0x150 && ctrl <= 0x15F) return row + (ctrl - 0x150);
  std::fprintf(stderr, "host emulation: DPP control 0x%x not modelled\n", ctrl);
  std::abort();
}

inline int dpp(int src, int ctrl, int row_mask, int bank_mask) {
  if (row_mask != 0xf || bank_mask != 0xf) {
    std::fprintf(stderr, "host emulation: DPP masks other than 0xf not modelled\n");
    std::abort();
  }
  Wave& w = my_wave();
  const int l = my_lane(), p = int(phase++ & 1);
  w.u32[p][l] = uint32_t(src);
  w.bar.arrive_and_wait();
  // Double-buffered: the next exchange writes the other buffer, and this
  // buffer is written again only after every lane has passed the next
  // barrier, i.e. after this read.
  return int(w.u32[p][dpp_source(l, ctrl)]);
}

// v_mfma_f32_16x16x4f32 (one 16x16 block, K = 4): lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16]; it returns D[4 (l / 16) + r][l % 16], r = 0..3.
inline floatx4_t mfma_16x16x4f32(float a, float b, floatx4_t c) {
  Wave& w = my_wave();
  const int l = my_lane(), p = int(phase++ & 1);
  w.a[p][l] = a;
  w.b[p][l] = b;
  w.bar.arrive_and_wait();
  const int j = l & 15, i0 = 4 * (l >> 4);
  floatx4_t d;
  for (int r = 0; r < 4; ++r) {
    float acc = c[r];
    for (int k = 0; k < 4; ++k) acc = std::fmaf(w.a[p][16 * k + i0 + r], w.b[p][16 * k + j], acc);
    d[r] = acc;
  }
  return d;
}

template <typename K, typename... A>
void launch(K kernel, dim3 grid, dim3 block, A... args) {
  if (grid.y != 1 || grid.z != 1 || block.y != 1 || block.z != 1 || block.x % 64 != 0 || block.x > 1024) {
    std::fprintf(stderr, "host emulation: launch shape not modelled\n");
    std::abort();
  }
  grid_dim = grid;
  block_dim = block;
  for (uint32_t b = 0; b < grid.x; ++b) {
    Workgroup g(block.x);
    std::vector<std::thread> th;
    th.reserve(block.x);
    for (uint32_t t = 0; t < block.x; ++t)
      th.emplace_back([&, t] {
        tid = dim3(t);
        bid = dim3(b);
        wg = &g;
        phase = 0;
        kernel(args...);
      });
    for (auto& x : th) x.join();
  }
}

}  // namespace simt

#define threadIdx (simt::tid)
#define blockIdx (simt::bid)
#define gridDim (simt::grid_dim)
#define blockDim (simt::block_dim)

inline void __syncthreads() { simt::wg->bar.arrive_and_wait(); }

inline float __int_as_float(int v) {
  float f;
  std::memcpy(&f, &v, 4);
  return f;
}
inline int __float_as_int(float f) {
  int v;
  std::memcpy(&v, &f, 4);
  return v;
}

// Raw buffer resources: a base, a size in bytes and the 32-bit offsets of
// each access. The kernels keep every access inside the size they give, so
// an access past it (which the hardware would drop or read as zero) is
// reported here as an error.
struct __amdgpu_buffer_rsrc_t {
  char* base;
  uint32_t bytes;
};
namespace simt {
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
inline char* buffer_at(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint32_t n) {
  const uint64_t off = uint64_t(voff) + uint64_t(soff);
  if (off + n > r.bytes) {
    std::fprintf(stderr, "host emulation: buffer access at byte %llu (+%u) past the resource's %u bytes\n",
                 (unsigned long long)off, n, r.bytes);
    std::abort();
  }
  return r.base + off;
}
template <typename V>
inline V buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  V v;
  std::memcpy(&v, buffer_at(r, voff, soff, sizeof(V)), sizeof(V));
  return v;
}
}  // namespace simt
inline __amdgpu_buffer_rsrc_t __builtin_amdgcn_make_buffer_rsrc(void* base, short stride, int bytes, int flags) {
  if (stride != 0) std::abort();
  (void)flags;
  return __amdgpu_buffer_rsrc_t{static_cast<char*>(base), uint32_t(bytes)};
}
#define __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, aux) simt::buffer_load<simt::u32x4_t>((r), (voff), (soff))
#define __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, aux) simt::buffer_load<simt::u32x2_t>((r), (voff), (soff))
#define __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, aux) \
  do {                                                                \
    const simt::u32x4_t v_ = (v);                                     \
    std::memcpy(simt::buffer_at((r), (voff), (soff), 16), &v_, 16);   \
  } while (0)

#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) simt::dpp((src), (ctrl), (rm), (bm))
#define __builtin_amdgcn_mov_dpp(src, ctrl, rm, bm, bc) simt::dpp((src), (ctrl), (rm), (bm))
#define __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, cbsz, abid, blgp) simt::mfma_16x16x4f32((a), (b), (c))

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) \
  simt::launch((kernel), dim3(grid), dim3(block), __VA_ARGS__)

inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
inline hipError_t hipStreamGetDevice(hipStream_t, int* d) {
  *d = 0;
  return hipSuccess;
}
#define HIP_SYMBOL(x) (&(x))
inline hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
  *p = const_cast<void*>(symbol);
  return hipSuccess;
}
