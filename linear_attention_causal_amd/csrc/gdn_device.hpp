// Device-side helpers shared by the gfx950 kernels of libgdn: activation
// storage types, wave64 reductions and the scalar nonlinearities of the
// Gated DeltaNet layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- storage

// Activations are either f32 or bf16 in memory; arithmetic is always f32.
template <typename Act> struct act_io;

template <> struct act_io<float> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, size_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  // four consecutive elements starting at a multiple of 4
  static __device__ __forceinline__ f32x4 load4(const void* p, size_t i) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(p) + i);
  }
  static __device__ __forceinline__ void store4(void* p, size_t i, f32x4 v) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p) + i) = v;
  }
  // Unconverted element, for loads whose conversion is deferred to the use.
  using raw_t = float;
  static __device__ __forceinline__ raw_t load_raw(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ float from_raw(raw_t r) { return r; }
  using raw4_t = f32x4;
  static __device__ __forceinline__ raw4_t load4_raw(const void* p, size_t i) { return load4(p, i); }
  static __device__ __forceinline__ f32x4 from_raw4(raw4_t r) { return r; }
  static constexpr int bytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Round to nearest even, as the hardware conversion does.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(unsigned short, h);
}

template <> struct act_io<__bf16> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return bf16_bits_to_f32(static_cast<const unsigned short*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, size_t i, float v) {
    static_cast<unsigned short*>(p)[i] = (unsigned short)f32_to_bf16_bits(v);
  }
  static __device__ __forceinline__ f32x4 load4(const void* p, size_t i) {
    uint2 u = *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(p) + i);
    f32x4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
  }
  static __device__ __forceinline__ void store4(void* p, size_t i, f32x4 v) {
    uint2 u;
    u.x = f32_to_bf16_bits(v.x) | (f32_to_bf16_bits(v.y) << 16);
    u.y = f32_to_bf16_bits(v.z) | (f32_to_bf16_bits(v.w) << 16);
    *reinterpret_cast<uint2*>(static_cast<unsigned short*>(p) + i) = u;
  }
  using raw_t = uint32_t;   // zero-extended bits
  static __device__ __forceinline__ raw_t load_raw(const void* p, size_t i) {
    return static_cast<const unsigned short*>(p)[i];
  }
  static __device__ __forceinline__ float from_raw(raw_t r) { return bf16_bits_to_f32(r); }
  using raw4_t = uint2;
  static __device__ __forceinline__ raw4_t load4_raw(const void* p, size_t i) {
    return *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(p) + i);
  }
  static __device__ __forceinline__ f32x4 from_raw4(raw4_t u) {
    f32x4 r;
    r.x = __uint_as_float(u.x << 16);
    r.y = __uint_as_float(u.x & 0xffff0000u);
    r.z = __uint_as_float(u.y << 16);
    r.w = __uint_as_float(u.y & 0xffff0000u);
    return r;
  }
  static constexpr int bytes = 2;
};

// Index of the calling wave in its workgroup, in a scalar register: role
// branches and operand-pointer selects on it stay uniform (scalar) instead of
// becoming per-lane selects that fetch kernel arguments with vector loads.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

// ---------------------------------------------------------------- math

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// x * sigmoid(x) with the hardware exp2 and reciprocal (a few ulp), for the
// bulk elementwise work of the chunked path.
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ float softplus(float x) {
  return x > 20.0f ? x : log1pf(expf(x));
}

// g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b)
__device__ __forceinline__ void gates(float A_log, float dt_bias, float a,
                                      float b, float& g, float& beta) {
  g = -expf(A_log) * softplus(a + dt_bias);
  beta = 1.0f / (1.0f + expf(-b));
}

// ---------------------------------------------------------------- wave64

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace gdn
