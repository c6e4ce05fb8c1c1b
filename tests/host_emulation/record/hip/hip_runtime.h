// Record-only stand-ins for the HIP runtime: kernel launches, event records
// and stream waits are logged in enqueue order and nothing runs (test
// infrastructure: the factor's two-stream schedule is checked from this log
// on the CPU; see hinv_schedule.cpp). Device code compiles against stubs
// that abort if ever called.
#pragma once

#include <any>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <tuple>
#include <type_traits>
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
inline dim3 threadIdx, blockIdx, gridDim, blockDim;

struct alignas(16) double2 {
  double x, y;
};
typedef enum hipError_t { hipSuccess = 0, hipErrorInvalidValue = 1 } hipError_t;
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
typedef enum hipStreamCaptureStatus {
  hipStreamCaptureStatusNone = 0,
  hipStreamCaptureStatusActive = 1
} hipStreamCaptureStatus;
constexpr unsigned hipStreamNonBlocking = 1;
constexpr unsigned hipEventDisableTiming = 2;

namespace rec {

[[noreturn]] inline void device_only() {
  std::fprintf(stderr, "record-only build: device code was called\n");
  std::abort();
}

struct Item {
  enum Kind { LAUNCH, RECORD, WAIT } kind;
  uintptr_t stream;
  const void* fn = nullptr;  // LAUNCH: the kernel
  std::any args;             // LAUNCH: std::tuple of the kernel's parameters
  uintptr_t event = 0;       // RECORD / WAIT
};
inline std::vector<Item> log;
inline uintptr_t next_id = 0x1000;
inline hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;

template <typename... P, typename... A>
void launch(void (*k)(P...), hipStream_t st, hipEvent_t stop, A&&... a) {
  Item it{Item::LAUNCH, reinterpret_cast<uintptr_t>(st)};
  it.fn = reinterpret_cast<const void*>(k);
  it.args = std::tuple<std::decay_t<P>...>(std::forward<A>(a)...);
  log.push_back(std::move(it));
  if (stop) log.push_back(Item{Item::RECORD, reinterpret_cast<uintptr_t>(st), nullptr, {}, reinterpret_cast<uintptr_t>(stop)});
}

}  // namespace rec

#define hipLaunchKernelGGL(kernel, grid, block, shmem, stream, ...) rec::launch((kernel), (stream), nullptr, __VA_ARGS__)
#define hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, stop, flags, ...) \
  rec::launch((kernel), (stream), (stop), __VA_ARGS__)

inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
inline hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned) {
  *s = reinterpret_cast<hipStream_t>(rec::next_id++);
  return hipSuccess;
}
inline hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = reinterpret_cast<hipEvent_t>(rec::next_id++);
  return hipSuccess;
}
inline hipError_t hipEventRecord(hipEvent_t e, hipStream_t s) {
  rec::log.push_back(rec::Item{rec::Item::RECORD, reinterpret_cast<uintptr_t>(s), nullptr, {}, reinterpret_cast<uintptr_t>(e)});
  return hipSuccess;
}
inline hipError_t hipStreamWaitEvent(hipStream_t s, hipEvent_t e, unsigned) {
  rec::log.push_back(rec::Item{rec::Item::WAIT, reinterpret_cast<uintptr_t>(s), nullptr, {}, reinterpret_cast<uintptr_t>(e)});
  return hipSuccess;
}
inline hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* c) {
  *c = rec::capture;
  return hipSuccess;
}

inline void __syncthreads() { rec::device_only(); }
template <typename T>
T atomicCAS(T*, T, T) { rec::device_only(); }
template <typename T>
T atomicMin(T*, T) { rec::device_only(); }

typedef double rec_doublex4 __attribute__((ext_vector_type(4)));
inline rec_doublex4 rec_mfma_f64(double, double, rec_doublex4) { rec::device_only(); }
inline double rec_rcp(double) { rec::device_only(); }
inline float rec_rcp(float) { rec::device_only(); }
#define __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, cbsz, abid, blgp) rec_mfma_f64((a), (b), (c))
#define __builtin_amdgcn_rcp(x) rec_rcp(x)
inline int rec_dpp(int) { rec::device_only(); }
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) rec_dpp(src)
#define __builtin_amdgcn_mov_dpp(src, ctrl, rm, bm, bc) rec_dpp(src)
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
