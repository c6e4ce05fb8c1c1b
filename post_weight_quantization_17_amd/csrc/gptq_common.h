// Shared definitions of the gfx950 GPTQ library: vector types for the MFMA
// builtins, launch-error mapping and small device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/gptq_mi355x.h"

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// Status of the last kernel launch on this thread, mapped to the ABI code.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GPTQ_OK : GPTQ_E_HIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Broadcast lane `src` of every 16-lane DPP row to the whole row
// (gfx90a+ DPP row_newbcast). SRC must be a compile-time constant.
template <int SRC>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + SRC, 0xf, 0xf, false));
}

// Butterfly reductions over the 16 lanes of a DPP row; every lane of the
// row receives the result.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, dpp_xor1(v));
  v = fminf(v, dpp_xor2(v));
  v = fminf(v, dpp_half_mirror(v));
  v = fminf(v, dpp_mirror(v));
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, dpp_half_mirror(v));
  v = fmaxf(v, dpp_mirror(v));
  return v;
}

// Word `w` of a row's LSB-first bitstream of b-bit codes: code j occupies
// stream bits [b j, b j + b); word w holds bits [32 w, 32 w + 32). Codes past
// `ncodes` count as zero; each code is masked to its low b bits.
template <typename CodePtr>
__device__ __forceinline__ uint32_t pack_word(CodePtr c, int ncodes, int bits, int w) {
  const int b0 = 32 * w;
  const int j0 = b0 / bits;
  int j1 = (b0 + 31) / bits;
  if (j1 > ncodes - 1) j1 = ncodes - 1;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t word = 0;
  for (int j = j0; j <= j1; ++j) {
    const int sh = j * bits - b0;
    const uint32_t v = uint32_t(c[j]) & mask;
    word |= sh >= 0 ? (v << sh) : (v >> (-sh));
  }
  return word;
}

}  // namespace gptq
