// Fused input prologue of the chunked gated delta rule on gfx950: the
// L2-normalised q and k (fp32 norms, then one rounding to the io dtype), beta and
// the log-decay g, in one pass over HBM.
//
//   q_out = q / max(||q||, 1e-30),  k_out = k / max(||k||, 1e-30)
//       (normalise in FP32, then cast: fla issue #1550 page, "Proposed scope")
//   beta  = sigmoid(b)  (x 2 with negative eigenvalues allowed)
//   g     = -exp(A_log[h]) softplus(a + dt_bias[h])  or  -5 sigmoid(a)
//       ("Research Sprint Day 2", "Building some intuition", the gate steps),
//       or the first form per key channel (the KDA gate layout of the cuLA
//       issue #126 page: a, g shaped like q, dt_bias per head and channel)
//
// The work is HBM-bound elementwise: each row of d_k values is read by a group of
// lanes (one 16-byte vector per lane), its sum of squares reduced across the group
// with lane shuffles, and written back once; the first lane of each group also
// forms the gates of its (token, head); with per-channel gates every lane forms
// those of its channels.  Rows of q and k are handled by the same lanes.
#include <hip/hip_runtime.h>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

__device__ __forceinline__ float sigmoidf_(float x) { return 1.f / (1.f + __expf(-x)); }
// softplus(x) = log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|)), without overflow
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }

template <typename E, int DK, bool CHAN>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueParams p) {
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));  // elements per 16-byte vector
  constexpr int LPR = DK / EPV;                          // lanes per row
  constexpr int RPB = 256 / LPR;                         // rows per block
  const int tid = threadIdx.x, sub = tid % LPR;
  const int64_t th = static_cast<int64_t>(blockIdx.x) * RPB + tid / LPR;  // token-head
  const bool live = th < p.rows;
  const int64_t off = (live ? th : 0) * DK + sub * EPV;
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  // every lane loads (rows past the end re-read row 0): no branch around a load
  const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(q + off);
  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(k + off);
  f32x4_t ca[EPV / 4], cb[EPV / 4];  // per-channel gates: a and dt_bias of this lane's channels
  if constexpr (CHAN) {
    const int h0 = static_cast<int>((live ? th : 0) % p.H);
#pragma unroll
    for (int u = 0; u < EPV / 4; ++u) {
      ca[u] = *reinterpret_cast<const f32x4_t*>(p.a + off + 4 * u);
      cb[u] = *reinterpret_cast<const f32x4_t*>(p.dt_bias + h0 * DK + sub * EPV + 4 * u);
    }
  }
  float qf[EPV], kf[EPV];
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int e = 0; e < EPV; ++e) {
    if constexpr (sizeof(E) == 2) {
      const uint32_t wq = qv[e >> 1], wk = kv[e >> 1];
      qf[e] = __uint_as_float((e & 1) ? (wq & 0xffff0000u) : (wq << 16));
      kf[e] = __uint_as_float((e & 1) ? (wk & 0xffff0000u) : (wk << 16));
    } else {
      qf[e] = __uint_as_float(qv[e]);
      kf[e] = __uint_as_float(kv[e]);
    }
    sq = fmaf(qf[e], qf[e], sq);
    sk = fmaf(kf[e], kf[e], sk);
  }
  // sums over the LPR lanes of the row (LPR is a power of two and divides 64)
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    sq += __shfl_xor(sq, m, 64);
    sk += __shfl_xor(sk, m, 64);
  }
  const float nq = fmaxf(sqrtf(sq), 1e-30f), nk = fmaxf(sqrtf(sk), 1e-30f);
  if (live) {
    E qo[EPV], ko[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if constexpr (sizeof(E) == 2) {
        qo[e] = f32_to_bf16(qf[e] / nq);
        ko[e] = f32_to_bf16(kf[e] / nk);
      } else {
        qo[e] = qf[e] / nq;
        ko[e] = kf[e] / nk;
      }
    }
    *reinterpret_cast<u32x4_t*>(static_cast<E*>(p.q_out) + off) = *reinterpret_cast<const u32x4_t*>(qo);
    *reinterpret_cast<u32x4_t*>(static_cast<E*>(p.k_out) + off) = *reinterpret_cast<const u32x4_t*>(ko);
    const int h = static_cast<int>(th % p.H);
    if (sub == 0) {
      const float bs = sigmoidf_(p.b[th]);
      p.beta[th] = p.allow_neg ? 2.f * bs : bs;
      if constexpr (!CHAN) {
        const float a = p.a[th];
        p.g[th] = p.gate_kind == 0 ? -__expf(p.A_log[h]) * softplusf_(a + p.dt_bias[h]) : -5.f * sigmoidf_(a);
      }
    }
    if constexpr (CHAN) {
      const float ea = -__expf(p.A_log[h]);
#pragma unroll
      for (int u = 0; u < EPV / 4; ++u) {
        f32x4_t gv;
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = ea * softplusf_(ca[u][e] + cb[u][e]);
        *reinterpret_cast<f32x4_t*>(p.g + off + 4 * u) = gv;
      }
    }
  }
}

template <typename E, int DK>
hipError_t launch_t(const PrologueParams& p, hipStream_t s) {
  constexpr int LPR = DK / (16 / static_cast<int>(sizeof(E)));
  constexpr int RPB = 256 / LPR;
  const int64_t blocks = (p.rows + RPB - 1) / RPB;
  if (blocks == 0) return hipSuccess;
  if (p.gate_kind == 2)
    hipLaunchKernelGGL((prologue_kernel<E, DK, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((prologue_kernel<E, DK, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) return Dk == 64 ? launch_t<uint16_t, 64>(p, s) : launch_t<uint16_t, 128>(p, s);
  return Dk == 64 ? launch_t<float, 64>(p, s) : launch_t<float, 128>(p, s);
}

}  // namespace gdn
