// Device helpers shared by the chunk kernels of the forward and backward passes
// (sequence ranges, block enumeration, packed transposed stores).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace chunk {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void seq_range(const SeqInfo& s, int n, int64_t& bos, int64_t& len) {
  if (s.cu) {
    bos = s.cu[n];
    len = s.cu[n + 1] - bos;
  } else {
    bos = static_cast<int64_t>(n) * s.T;
    len = s.T;
  }
}

// Lower-triangular 16x16 block (bi >= bj) of a 4x4 block grid, by index 0..9.
__device__ __forceinline__ void lower_block(int b, int& bi, int& bj) {
  bi = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
  bj = b - bi * (bi + 1) / 2;
}

// 16 bytes in four registers (a native vector type, so selects stay in registers)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t u4_word(const u32x4_t& v, int i) { return v[i]; }

// Element e of two row vectors a, b (16 bytes each), paired for a transposed
// store: {a[e], b[e]}.  Register-only (e is a compile-time index after unrolling).
template <typename E>
struct Pair;
template <>
struct Pair<uint16_t> {
  static __device__ __forceinline__ void store(uint16_t* dst, const u32x4_t& a, const u32x4_t& b, int e) {
    const uint32_t wa = u4_word(a, e >> 1), wb = u4_word(b, e >> 1);
    *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(wb, wa, (e & 1) ? 0x07060302u : 0x05040100u);
  }
};
template <>
struct Pair<float> {
  static __device__ __forceinline__ void store(float* dst, const u32x4_t& a, const u32x4_t& b, int e) {
    *reinterpret_cast<uint2*>(dst) = uint2{u4_word(a, e), u4_word(b, e)};
  }
};

template <typename E>
__device__ __forceinline__ void store4(E* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = float4{a, b, c, d};
}

template <typename Op>
__host__ __device__ constexpr int tsteps(int ri) {  // k-steps covering T row block ri
  return (16 * (ri + 1) + Op::KSTEP - 1) / Op::KSTEP;
}

// Buffer resource over `bytes` bytes at `base` (gfx9 raw buffer: stride 0, 32-bit
// data format).  Stores at offsets past `bytes` are dropped by the hardware's
// range check, which lets a loop store conditionally without branching; with
// bytes = 0 every store is dropped and `base` is never dereferenced.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
typedef uint32_t u32x2v_t __attribute__((vector_size(8)));
typedef uint32_t u32x4v_t __attribute__((vector_size(16)));
template <typename E>
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int off, float a, float b, float c,
                                              float d);
template <>
__device__ __forceinline__ void buffer_store4<uint16_t>(__amdgpu_buffer_rsrc_t r, int off, float a, float b,
                                                        float c, float d) {
  const u32x2v_t v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
template <>
__device__ __forceinline__ void buffer_store4<float>(__amdgpu_buffer_rsrc_t r, int off, float a, float b,
                                                     float c, float d) {
  const u32x4v_t v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buffer_store1(__amdgpu_buffer_rsrc_t r, int off, float a) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, off, 0, 0);
}
// One value as an element of type E (bf16 rounded to nearest even, or fp32) at byte
// offset `off`.
template <typename E>
__device__ __forceinline__ void buffer_store1e(__amdgpu_buffer_rsrc_t r, int off, float a) {
  if constexpr (sizeof(E) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(a), r, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, off, 0, 0);
}

}  // namespace chunk
}  // namespace gdn
