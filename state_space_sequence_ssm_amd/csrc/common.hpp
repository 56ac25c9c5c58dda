// Shared device helpers for the gfx950 kernels of the Mamba-3 SSM core:
// bf16 <-> fp32 conversion, 16-byte vector loads, MFMA wrappers, wave scans.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kTwoPi = 6.283185307179586f;
constexpr float kInvTwoPi = 0.15915494309189535f;

// Element storage of an input tensor: float or bf16 (kept as uint16 bits).
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return static_cast<uint16_t>(pack_bf16x2(a, 0.f) & 0xffffu);
}

// Load/store of 16 bytes worth of elements as fp32 values.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int kElems = 4;
  __device__ static __forceinline__ void load(const float* p, float* out) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = v[i];
  }
};
template <>
struct Vec16<bf16_t> {
  static constexpr int kElems = 8;
  __device__ static __forceinline__ void load(const bf16_t* p, float* out) {
    u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};

template <typename T>
__device__ __forceinline__ float load_scalar(const T* p);
template <>
__device__ __forceinline__ float load_scalar<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_scalar<bf16_t>(const bf16_t* p) { return bf16_to_f32(p->bits); }

// Same, with the nontemporal hint (data read once).
template <typename T>
__device__ __forceinline__ float load_scalar_nt(const T* p);
template <>
__device__ __forceinline__ float load_scalar_nt<float>(const float* p) { return __builtin_nontemporal_load(p); }
template <>
__device__ __forceinline__ float load_scalar_nt<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(__builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p)));
}

template <typename T>
__device__ __forceinline__ void store_scalar(T* p, float v);
template <>
__device__ __forceinline__ void store_scalar<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_scalar<bf16_t>(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }

// Store 4 consecutive values in storage type T.
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2*>(p) = v;
}

// Inclusive prefix sum over lane segments of `width` lanes (power of two <= 64).
__device__ __forceinline__ float wave_inclusive_scan(float v, int width) {
  const int lane = threadIdx.x & 63;
  const int sl = lane & (width - 1);
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    if (d < width) {
      float o = __shfl_up(v, d, width);
      if (sl >= d) v += o;
    }
  }
  return v;
}

// Reduce an angle modulo 2*pi into [-pi, pi].
__device__ __forceinline__ float wrap_angle(float a) {
  return a - kTwoPi * rintf(a * kInvTwoPi);
}

}  // namespace m3
