// Output epilogue of the chunked gated delta rule on gfx950: per (token, head),
//   y = o / sqrt(mean(o^2) + eps) * weight * silu(z)
// ("Research Sprint Day 2", "Building some intuition", step 7: normalise per head,
// then gate with silu(z)), in fp32 and rounded once to the io dtype.
//
// HBM-bound elementwise work: a group of lanes holds one row of Dv values (one
// 16-byte vector of o and of z per lane), the sum of squares is reduced across the
// group with lane shuffles, and the row is written once.
#include <hip/hip_runtime.h>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

template <typename E, int DV>
__global__ __launch_bounds__(256) void epilogue_kernel(EpilogueParams p) {
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));  // elements per 16-byte vector
  constexpr int LPR = DV / EPV;                          // lanes per row (a power of two, <= 64)
  constexpr int RPB = 256 / LPR;                         // rows per block
  const int tid = threadIdx.x, sub = tid % LPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + tid / LPR;
  const bool live = row < p.rows;
  const int64_t off = (live ? row : 0) * DV + sub * EPV;
  u32x4_t ov = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
  if (live) {
    ov = *reinterpret_cast<const u32x4_t*>(static_cast<const E*>(p.o) + off);
    zv = *reinterpret_cast<const u32x4_t*>(static_cast<const E*>(p.z) + off);
  }
  float of[EPV], zf[EPV];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    if constexpr (sizeof(E) == 2) {
      of[e] = __uint_as_float((e & 1) ? (ov[e >> 1] & 0xffff0000u) : (ov[e >> 1] << 16));
      zf[e] = __uint_as_float((e & 1) ? (zv[e >> 1] & 0xffff0000u) : (zv[e >> 1] << 16));
    } else {
      of[e] = __uint_as_float(ov[e]);
      zf[e] = __uint_as_float(zv[e]);
    }
    ss = fmaf(of[e], of[e], ss);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float inv = 1.f / sqrtf(ss / static_cast<float>(DV) + p.eps);
  if (!live) return;
  float wf[EPV];
#pragma unroll
  for (int x = 0; x < EPV / 4; ++x) {
    const float4 w4 = p.weight ? *reinterpret_cast<const float4*>(p.weight + sub * EPV + 4 * x)
                               : float4{1.f, 1.f, 1.f, 1.f};
    wf[4 * x] = w4.x; wf[4 * x + 1] = w4.y; wf[4 * x + 2] = w4.z; wf[4 * x + 3] = w4.w;
  }
  E yo[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    const float w = wf[e];
    const float silu = zf[e] / (1.f + __expf(-zf[e]));
    const float y = of[e] * inv * w * silu;
    if constexpr (sizeof(E) == 2)
      yo[e] = f32_to_bf16(y);
    else
      yo[e] = y;
  }
  *reinterpret_cast<u32x4_t*>(static_cast<E*>(p.y) + off) = *reinterpret_cast<const u32x4_t*>(yo);
}

template <typename E, int DV>
hipError_t launch_t(const EpilogueParams& p, hipStream_t s) {
  constexpr int LPR = DV / (16 / static_cast<int>(sizeof(E)));
  constexpr int RPB = 256 / LPR;
  const int64_t blocks = (p.rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((epilogue_kernel<E, DV>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const EpilogueParams& p, int Dv, hipStream_t s) {
  switch (Dv) {
    case 16: return launch_t<E, 16>(p, s);
    case 32: return launch_t<E, 32>(p, s);
    case 64: return launch_t<E, 64>(p, s);
    case 128: return launch_t<E, 128>(p, s);
    case 256: return launch_t<E, 256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_epilogue(const EpilogueParams& p, int Dv, bool bf16, hipStream_t s) {
  return bf16 ? launch_e<uint16_t>(p, Dv, s) : launch_e<float>(p, Dv, s);
}

}  // namespace gdn
