// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte register payload

// bf16 storage is handled as raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Element type traits: storage type and its conversion to fp32.
template <int DT> struct Elem;
template <> struct Elem<0> {  // fp32
  typedef float T;
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<1> {  // bf16 bits
  typedef uint16_t T;
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Load through a wave-uniform base and a 32-bit byte offset, which maps to
// the global_load form with an SGPR base, a VGPR offset and an immediate.
template <typename V>
__device__ __forceinline__ V ld_off(const void* __restrict__ base, uint32_t byte_off) {
  return *reinterpret_cast<const V*>(static_cast<const char*>(base) + byte_off);
}

// Two segments of tiles in one launch, mapped so that each XCD (workgroups
// are dealt round-robin over the 8 XCDs) works on contiguous logical tiles,
// which then share that XCD's L2: each XCD first takes an even share of
// segment 1's tiles (the longer ones, so they start early), then a
// contiguous range of segment 0's tiles.  The shares add up to the number of
// live workgroups (w < G0 + G1) the round-robin deal gives each XCD.
__device__ __forceinline__ void xcd_remap2(int w, int G0, int G1, int& seg, int& L) {
  constexpr int kXcd = 8;
  const int G = G0 + G1;
  const int x = w % kXcd, i = w / kXcd;
  const int q = G / kXcd, r = G % kXcd;
  const int q1 = G1 / kXcd, r1 = G1 % kXcd;
  const int s1 = q1 + (x < r1 ? 1 : 0);
  if (i < s1) {
    seg = 1;
    L = x * q1 + (x < r1 ? x : r1) + i;
  } else {
    seg = 0;
    L = (x * q + (x < r ? x : r)) - (x * q1 + (x < r1 ? x : r1)) + (i - s1);
  }
}

}  // namespace moe
