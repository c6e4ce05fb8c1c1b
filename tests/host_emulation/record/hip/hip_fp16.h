// Host stand-ins for the fp16 types and conversions the sweep kernels use
// (test infrastructure for the CPU runs).
#pragma once

struct __half {
  _Float16 x;
};
struct __half2 {
  __half x, y;
};
inline float __half2float(__half h) { return float(h.x); }
inline __half __float2half_rn(float f) { return __half{_Float16(f)}; }
inline float __low2float(__half2 a) { return float(a.x.x); }
inline float __high2float(__half2 a) { return float(a.y.x); }
