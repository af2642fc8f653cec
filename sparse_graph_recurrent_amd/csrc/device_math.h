// device_math.h -- float4 helpers and the tanh derivative shared by the
// recurrence kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace ckhip {
namespace {

__device__ __forceinline__ float4 f4(float x) { return make_float4(x, x, x, x); }
__device__ __forceinline__ float4 fma4(float w, float4 h, float4 acc) {
  acc.x = fmaf(w, h.x, acc.x);
  acc.y = fmaf(w, h.y, acc.y);
  acc.z = fmaf(w, h.z, acc.z);
  acc.w = fmaf(w, h.w, acc.w);
  return acc;
}
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 shfl4(float4 v, int src) {
  return make_float4(__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src));
}
__device__ __forceinline__ float4 shfl_xor4(float4 v, int m) {
  return make_float4(__shfl_xor(v.x, m), __shfl_xor(v.y, m), __shfl_xor(v.z, m),
                     __shfl_xor(v.w, m));
}
// fp64 accumulation of fp32 products (the per-microstep forward's row sums:
// one rounding to fp32 per row instead of one per added term)
__device__ __forceinline__ double4 d4(double x) { return make_double4(x, x, x, x); }
__device__ __forceinline__ double4 fma4d(float w, float4 h, double4 acc) {
  const double wd = (double)w;
  acc.x = fma(wd, (double)h.x, acc.x);
  acc.y = fma(wd, (double)h.y, acc.y);
  acc.z = fma(wd, (double)h.z, acc.z);
  acc.w = fma(wd, (double)h.w, acc.w);
  return acc;
}
__device__ __forceinline__ double4 add4d(double4 a, double4 b) {
  return make_double4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ double4 shfl4d(double4 v, int src) {
  return make_double4(__shfl(v.x, src), __shfl(v.y, src), __shfl(v.z, src), __shfl(v.w, src));
}
__device__ __forceinline__ double4 shfl_xor4d(double4 v, int m) {
  return make_double4(__shfl_xor(v.x, m), __shfl_xor(v.y, m), __shfl_xor(v.z, m),
                      __shfl_xor(v.w, m));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
// sech^2(a) = 4 e^{-2|a|} / (1 + e^{-2|a|})^2, from the pre-activation itself
// (not 1 - tanh^2, which cancels badly once |a| is a few units).
__device__ __forceinline__ float sech2f(float a) {
  float e = expf(-2.0f * fabsf(a));
  float d = 1.0f + e;
  return 4.0f * e / (d * d);
}

}  // namespace
}  // namespace ckhip
