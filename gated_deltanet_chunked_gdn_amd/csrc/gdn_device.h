// Device-side building blocks for the gfx950 kernels of libgdn: number
// conversions, MFMA operand fragments and 16x16 tile products.
//
// MFMA conventions used throughout (CDNA3/CDNA4 matrix-core register layout for
// the 16x16 output shapes):
//   * the 16x16 fp32 accumulator of a wave64 holds C[4*(lane/16) + r][lane%16]
//     in element r (r = 0..3) of lane `lane`;
//   * an A operand fragment of v_mfma_f32_16x16x32_bf16 is A[lane%16][8*(lane/16) + 0..7]
//     and a B fragment is B[8*(lane/16) + 0..7][lane%16];
//   * v_mfma_f32_16x16x4_f32 takes A[lane%16][lane/16] and B[lane/16][lane%16].
// Both operands are therefore read the same way from LDS when the A operand is
// stored row-major (M x K) and the B operand is stored transposed (N x K), the
// reduction index contiguous: `frag(buf, ld, lane, k0)` reads row lane%16 from
// column k0 + (lane/16) * KPL on.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values packed into one dword, `a` in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ----------------------------------------------------------------------------------
// Operand policies.  `elem` is what operand tiles hold in LDS.
// ----------------------------------------------------------------------------------
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

struct OpBf16 {
  using elem = uint16_t;
  using frag_t = bf16x8_t;
  static constexpr int KSTEP = 32;  // reduction depth of one MFMA
  static constexpr int KPL = 8;     // reduction elements per lane
  static __device__ __forceinline__ elem cvt(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ float widen(elem x) { return bf16_to_f32(x); }
  // Fragment of row (lane % 16) of `buf`, reduction columns k0 + 8 (lane / 16) + 0..7.
  static __device__ __forceinline__ frag_t frag(const elem* buf, int ld, int lane, int k0) {
    const uint4 u = *reinterpret_cast<const uint4*>(buf + (lane & 15) * ld + k0 + (lane >> 4) * 8);
    return __builtin_bit_cast(bf16x8_t, u);
  }
  // The same fragment read from memory where `row` already points at this lane's row.
  static __device__ __forceinline__ frag_t frag_row(const elem* row, int lane, int k0) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + k0 + (lane >> 4) * 8);
    return __builtin_bit_cast(bf16x8_t, u);
  }
  // Fragment of the transpose of a row-major LDS buffer: element m of lane `lane`
  // is buf[k0 + 8 (lane / 16) + m][lane % 16].  Two ds_read_b64_tr_b16: within each
  // 16-lane group, lane s supplies row k0 + 8 g + s / 4 (+4), columns 4 (s % 4) .. +3,
  // and lane i receives column i of the four rows.
  static __device__ __forceinline__ frag_t frag_tr(const elem* buf, int ld, int lane, int k0) {
    const int s = lane & 15;
    const elem* p0 = buf + (k0 + 8 * (lane >> 4) + (s >> 2)) * ld + 4 * (s & 3);
    const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
    const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + 4 * ld));
    typedef short i16x8_t __attribute__((ext_vector_type(8)));
    const i16x8_t ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, ab);
  }
  // Multiply element m of a fragment by s[k0 + 8 (lane / 16) + m] and re-round.
  static __device__ __forceinline__ frag_t scale(frag_t f, const float* s, int lane, int k0) {
    uint4 u = __builtin_bit_cast(uint4, f);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const float* sc = s + k0 + (lane >> 4) * 8;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float lo = __uint_as_float(w[m] << 16) * sc[2 * m];
      const float hi = __uint_as_float(w[m] & 0xffff0000u) * sc[2 * m + 1];
      w[m] = pack_bf16x2(lo, hi);
    }
    return __builtin_bit_cast(bf16x8_t, uint4{w[0], w[1], w[2], w[3]});
  }
  static __device__ __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

struct OpF32 {
  using elem = float;
  using frag_t = float;
  static constexpr int KSTEP = 4;
  static constexpr int KPL = 1;
  static __device__ __forceinline__ elem cvt(float x) { return x; }
  static __device__ __forceinline__ float widen(elem x) { return x; }
  static __device__ __forceinline__ frag_t frag(const elem* buf, int ld, int lane, int k0) {
    return buf[(lane & 15) * ld + k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ frag_t frag_row(const elem* row, int lane, int k0) {
    return row[k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ frag_t frag_tr(const elem* buf, int ld, int lane, int k0) {
    return buf[(k0 + (lane >> 4)) * ld + (lane & 15)];
  }
  static __device__ __forceinline__ frag_t scale(frag_t f, const float* s, int lane, int k0) {
    return f * s[k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ f32x4_t mma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// acc += A(16 x K) * B(K x 16): A row-major at `a` (leading dim lda), B stored
// transposed (16 x K) at `bt` (leading dim ldb); K a multiple of Op::KSTEP.
template <typename Op, int K>
__device__ __forceinline__ void tile_mma(f32x4_t& acc, const typename Op::elem* a, int lda,
                                         const typename Op::elem* bt, int ldb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += Op::KSTEP)
    acc = Op::mma(Op::frag(a, lda, lane, k0), Op::frag(bt, ldb, lane, k0), acc);
}

// fp32 tile product with a row-major B (used by the triangular solve):
// acc += A(16 x K) * B(K x 16), both fp32 row-major.
template <int K>
__device__ __forceinline__ void tile_mma_f32_rowmajor(f32x4_t& acc, const float* a, int lda,
                                                      const float* b, int ldb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(lane & 15) * lda + k0 + (lane >> 4)],
                                               b[(k0 + (lane >> 4)) * ldb + (lane & 15)], acc,
                                               0, 0, 0);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Load/store of io-dtype values.
template <typename IO>
struct IoT;
template <>
struct IoT<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};
template <>
struct IoT<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float x) { *p = x; }
};

// Lane shift within rows of 16 lanes / row broadcasts (DPP; gfx9 encodings).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: a shift-and-add
// scan inside each row of 16 lanes, then the row totals are carried across rows
// by the row_bcast:15 / row_bcast:31 broadcasts.  Lanes whose DPP source lies
// outside the row (or whose row is masked off) add 0.
__device__ __forceinline__ float wave_inclusive_scan(float x, int /*lane*/) {
  x += dpp_f32<0x111, 0xf>(x);  // row_shr:1
  x += dpp_f32<0x112, 0xf>(x);  // row_shr:2
  x += dpp_f32<0x114, 0xf>(x);  // row_shr:4
  x += dpp_f32<0x118, 0xf>(x);  // row_shr:8
  x += dpp_f32<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_f32<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

}  // namespace gdn
