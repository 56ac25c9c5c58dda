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

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e^-|z|): the positive step
// Delta from its raw value, without branches.  log1p(u), u in (0, 1], from
// the hardware log of w = fl(1 + u) scaled by u / (w - 1), which cancels the
// rounding of 1 + u (Goldberg's form; exact u when w rounds to 1).
__device__ __forceinline__ float softplus_f(float z) {
  const float u = __expf(-fabsf(z));
  const float w = 1.f + u;
  const float lp = w == 1.f ? u : __logf(w) * (u / (w - 1.f));
  return fmaxf(z, 0.f) + lp;
}

// Delta of one token with the prologue's options: softplus of raw + bias, or
// the value as given.  Tokens past the end (`valid` false) have Delta = 0.
__device__ __forceinline__ float delta_of(float raw, bool softplus, float bias, bool valid) {
  return !valid ? 0.f : (softplus ? softplus_f(raw + bias) : raw);
}

// Reduce an angle modulo 2*pi into [-pi, pi].
__device__ __forceinline__ float wrap_angle(float a) {
  return a - kTwoPi * rintf(a * kInvTwoPi);
}

// ---------------------------------------------------------------- MFMA and LDS fragments
// D (16 x 16, fp32) += A (16 x 32) B (32 x 16) on bf16 operands: lane (g =
// lane / 16, l16 = lane % 16) supplies row l16 of A and column l16 of B at
// eight k positions, and holds D[4 g + 0..3][l16] (gfx950 v_mfma_f32_16x16x32_bf16).
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 cat8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(v);
}
__device__ __forceinline__ u32x2 pack4(f32x4 v) { return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}; }
__device__ __forceinline__ f32x4 unpack4(u32x2 u) {
  return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
               __uint_as_float(u[1] & 0xffff0000u)};
}
// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  In each group of 16
// lanes, lane 4e + q reads 4 bf16 at its own address; afterwards lane i holds
// element i % 4 of lanes 4e + i / 4, e = 0..3.  With lane 4e + q pointing at
// columns c0 + 4q..+3 of row r_e of a row-major matrix, lane i receives column
// c0 + i of rows r_0..r_3: four k values of an MFMA operand column.
typedef short tr4_t __attribute__((ext_vector_type(4)));
// A uniform LDS element offset the compiler cannot relate to other offsets.
// Reads from two bases a constant distance apart are otherwise fused into one
// ds_read2_b64, which the LDS serves at half the rate of two single 8-byte
// reads (16 lanes per cycle on 32 banks instead of 32 lanes on 64 banks).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* p) {
  typedef __attribute__((address_space(3))) tr4_t* lds_tr4_ptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_tr4_ptr)(p)));
}
template <int CTRL, int ROWMASK, bool BOUND>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWMASK, 0xF, BOUND));
}
// Inclusive scan over aligned segments of W lanes (W a power of two, 8..64):
// row_shr 1/2/4/8 within rows of 16, then row_bcast 15 / 31 across rows.
template <int W>
__device__ __forceinline__ float seg_scan(float v) {
  const int sl = threadIdx.x & (W - 1);
  float t;
  t = dpp<0x111, 0xF, true>(v);
  v += (W >= 16 || sl >= 1) ? t : 0.f;
  t = dpp<0x112, 0xF, true>(v);
  v += (W >= 16 || sl >= 2) ? t : 0.f;
  t = dpp<0x114, 0xF, true>(v);
  v += (W >= 16 || sl >= 4) ? t : 0.f;
  if constexpr (W >= 16) v += dpp<0x118, 0xF, true>(v);
  if constexpr (W >= 32) v += dpp<0x142, 0xA, false>(v);
  if constexpr (W >= 64) v += dpp<0x143, 0xC, false>(v);
  return v;
}
// v plus the v of lane ^ 16 (add_x16) or lane ^ 32 (add_x32), in every lane:
// gfx950's permlane swaps hand lanes l & ~16 and l | 16 (or 32) their values
// on the vector ALU, where a lane shuffle is an LDS round trip.  Both lanes of
// a pair add in the same order, so they hold the same bits.
__device__ __forceinline__ float add_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over the 64 lanes of a wave, in every lane: the DPP scan's last lane (no
// LDS round trip, unlike a butterfly of lane shuffles).
__device__ __forceinline__ float wave_sum(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, seg_scan<64>(v)), 63));
}



// ---------------------------------------------------------------- buffer resources
// Loads and stores through a buffer resource spanning [base, base + bytes):
// an offset past the range reads 0 and drops the store, with no memory
// request.  Out-of-range offsets (kBad) instead of branches keep every wave's
// count of memory instructions the same, so the compiler's wait counts stay
// exact (a load issued early is not held up by later stores of unknown count).
constexpr uint32_t kBad = 0x7FFFFFF0u;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
// the same with the non-temporal cache policy (aux bit 1): data read or
// written once, kept from displacing reused lines
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}
__device__ __forceinline__ u32x2 bload8_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2);
}
__device__ __forceinline__ void bstore8_nt(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 2);
}
__device__ __forceinline__ void bstore16_nt(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 2);
}
__device__ __forceinline__ u32x2 bload8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ float bloadf(rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ f32x4 bloadf4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstoref(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

}  // namespace m3
