// Token-by-token gated delta rule in IEEE fp32: the GPU's full-length second
// reference ("fused recurrent operator" of the fla issue #1550 page,
// "Reproduction and evidence"), forward and reverse mode.  Not the fast path.
//
// One workgroup of 256 threads per (sequence, head); thread j < Dv owns column j
// of the d_k x d_v state in registers (columns never mix: the update of
// "Research Sprint Day 1", section "The GDN update").  Per token:
//   S <- a S,  r = S^T k,  e = beta (v - r),  S <- S + k e^T,  o = scale S^T q
// i.e. the fused single-outer-product form of "Research Sprint Day 2",
// section "FLOPs per token".  Token data is staged in LDS in blocks.
//
// Reverse mode: a forward sweep stores the state at the start of every block of
// kRecBlock tokens (workspace); blocks are then visited last to first, each
// replayed forward from its checkpoint into a per-(sequence, head) replay
// buffer, then walked backwards.  Gradients that sum over columns (dq, dk,
// dbeta, dg) are reduced through LDS in a fixed order, so results are
// deterministic.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kFwdBlock = 16;

__device__ __forceinline__ void seq_range(const SeqInfo& s, int n, int64_t& bos, int64_t& len) {
  if (s.cu) {
    bos = s.cu[n];
    len = s.cu[n + 1] - bos;
  } else {
    bos = static_cast<int64_t>(n) * s.T;
    len = s.T;
  }
}

template <int DK, typename E>
__global__ __launch_bounds__(256) void recurrent_fwd_kernel(RecParams p) {
  __shared__ float ks[kFwdBlock][DK];
  __shared__ float qs[kFwdBlock][DK];
  __shared__ float vs[kFwdBlock][256];
  __shared__ float as[kFwdBlock], bs[kFwdBlock];
  const int j = threadIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int H = p.H, Dv = p.Dv;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  E* o = static_cast<E*>(p.o);
  const bool col = j < Dv;

  float s[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i)
    s[i] = (col && p.S0) ? p.S0[((static_cast<int64_t>(n) * H + h) * DK + i) * Dv + j] : 0.f;

  for (int64_t t0 = 0; t0 < len; t0 += kFwdBlock) {
    const int nv = static_cast<int>(len - t0 < kFwdBlock ? len - t0 : kFwdBlock);
    __syncthreads();
    for (int x = j; x < kFwdBlock * DK; x += 256) {
      const int tt = x / DK, i = x % DK;
      const bool ok = tt < nv;
      ks[tt][i] = ok ? IoT<E>::ld(k + ((bos + t0 + tt) * H + h) * DK + i) : 0.f;
      qs[tt][i] = ok ? IoT<E>::ld(q + ((bos + t0 + tt) * H + h) * DK + i) : 0.f;
    }
    for (int x = j; x < kFwdBlock * Dv; x += 256) {
      const int tt = x / Dv, c = x % Dv;
      vs[tt][c] = tt < nv ? IoT<E>::ld(v + ((bos + t0 + tt) * H + h) * Dv + c) : 0.f;
    }
    if (j < kFwdBlock) {
      as[j] = j < nv ? expf(p.g[(bos + t0 + j) * H + h]) : 1.f;
      bs[j] = j < nv ? p.beta[(bos + t0 + j) * H + h] : 0.f;
    }
    __syncthreads();
    if (col) {
      for (int tt = 0; tt < nv; ++tt) {
        const float a = as[tt];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          s[i] *= a;
          r = fmaf(s[i], ks[tt][i], r);
        }
        const float e = bs[tt] * (vs[tt][j] - r);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          s[i] = fmaf(ks[tt][i], e, s[i]);
          acc = fmaf(s[i], qs[tt][i], acc);
        }
        IoT<E>::st(o + ((bos + t0 + tt) * H + h) * Dv + j, p.scale * acc);
      }
    }
  }
  if (col && p.S_final) {
#pragma unroll
    for (int i = 0; i < DK; ++i)
      p.S_final[((static_cast<int64_t>(n) * H + h) * DK + i) * Dv + j] = s[i];
  }
}

template <int DK, typename E>
__global__ __launch_bounds__(256) void recurrent_bwd_kernel(RecParams p) {
  constexpr int RB = kRecBlock;
  extern __shared__ __align__(16) float smem[];
  const int Dv = p.Dv, H = p.H;
  const int ldr = Dv + 1;
  float* red = smem;                     // [2 * DK][Dv + 1]: per-column partials of dq, dk
  float* ks = red + 2 * DK * ldr;        // [RB][DK]
  float* qs = ks + RB * DK;              // [RB][DK]
  float* as = qs + RB * DK;              // [RB]
  float* bs = as + RB;                   // [RB]
  float* wred = bs + RB;                 // [4][2]
  const int j = threadIdx.x, lane = j & 63, wave = j >> 6, h = blockIdx.y, n = blockIdx.z;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  const E* dO = static_cast<const E*>(p.dO);
  const bool col = j < Dv;
  const int64_t nh = static_cast<int64_t>(n) * H + h;
  float* ckpt = p.ws + nh * p.ckpt_stride;                                     // [nblk][DK][Dv]
  float* replay = p.ws + static_cast<int64_t>(p.N) * H * p.ckpt_stride +
                  nh * static_cast<int64_t>(RB) * DK * Dv;                     // [RB][DK][Dv]
  const int nblk = static_cast<int>((len + RB - 1) / RB);

  auto stage = [&](int64_t t0, int nv) {
    __syncthreads();
    for (int x = j; x < RB * DK; x += 256) {
      const int tt = x / DK, i = x % DK;
      const bool ok = tt < nv;
      ks[x] = ok ? IoT<E>::ld(k + ((bos + t0 + tt) * H + h) * DK + i) : 0.f;
      qs[x] = ok ? IoT<E>::ld(q + ((bos + t0 + tt) * H + h) * DK + i) : 0.f;
    }
    if (j < RB) {
      as[j] = j < nv ? expf(p.g[(bos + t0 + j) * H + h]) : 1.f;
      bs[j] = j < nv ? p.beta[(bos + t0 + j) * H + h] : 0.f;
    }
    __syncthreads();
  };

  // ---- forward sweep: checkpoints at block starts ----
  float s[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) s[i] = (col && p.S0) ? p.S0[(nh * DK + i) * Dv + j] : 0.f;
  for (int b = 0; b < nblk; ++b) {
    const int64_t t0 = static_cast<int64_t>(b) * RB;
    const int nv = static_cast<int>(len - t0 < RB ? len - t0 : RB);
    if (col) {
#pragma unroll
      for (int i = 0; i < DK; ++i) ckpt[(static_cast<int64_t>(b) * DK + i) * Dv + j] = s[i];
    }
    stage(t0, nv);
    if (col) {
      for (int tt = 0; tt < nv; ++tt) {
        const float a = as[tt];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          s[i] *= a;
          r = fmaf(s[i], ks[tt * DK + i], r);
        }
        const float e = bs[tt] * (IoT<E>::ld(v + ((bos + t0 + tt) * H + h) * Dv + j) - r);
#pragma unroll
        for (int i = 0; i < DK; ++i) s[i] = fmaf(ks[tt * DK + i], e, s[i]);
      }
    }
  }

  // ---- reverse sweep ----
  float dS[DK];
#pragma unroll
  for (int i = 0; i < DK; ++i) dS[i] = (col && p.dS_final) ? p.dS_final[(nh * DK + i) * Dv + j] : 0.f;
  for (int b = nblk - 1; b >= 0; --b) {
    const int64_t t0 = static_cast<int64_t>(b) * RB;
    const int nv = static_cast<int>(len - t0 < RB ? len - t0 : RB);
    stage(t0, nv);
    if (col) {  // replay the block, keeping S_{t-1} of every token
#pragma unroll
      for (int i = 0; i < DK; ++i) s[i] = ckpt[(static_cast<int64_t>(b) * DK + i) * Dv + j];
      for (int tt = 0; tt < nv; ++tt) {
        const float a = as[tt];
#pragma unroll
        for (int i = 0; i < DK; ++i) replay[(static_cast<int64_t>(tt) * DK + i) * Dv + j] = s[i];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          s[i] *= a;
          r = fmaf(s[i], ks[tt * DK + i], r);
        }
        const float e = bs[tt] * (IoT<E>::ld(v + ((bos + t0 + tt) * H + h) * Dv + j) - r);
#pragma unroll
        for (int i = 0; i < DK; ++i) s[i] = fmaf(ks[tt * DK + i], e, s[i]);
      }
    }
    for (int tt = nv - 1; tt >= 0; --tt) {
      const int64_t row = bos + t0 + tt;
      float db = 0.f, dga = 0.f;
      if (col) {
        const float a = as[tt], bb = bs[tt];
        const float vj = IoT<E>::ld(v + (row * H + h) * Dv + j);
        const float doj = IoT<E>::ld(dO + (row * H + h) * Dv + j);
        const float* kt = ks + tt * DK;
        const float* qt = qs + tt * DK;
        float sp[DK];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          sp[i] = a * replay[(static_cast<int64_t>(tt) * DK + i) * Dv + j];
          r = fmaf(sp[i], kt[i], r);
        }
        const float e = bb * (vj - r);
        // o_t = scale S_t^T q_t
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          dS[i] = fmaf(p.scale * qt[i], doj, dS[i]);
          red[i * ldr + j] = p.scale * fmaf(kt[i], e, sp[i]) * doj;
        }
        // S_t = S' + k e^T
        float de = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) de = fmaf(dS[i], kt[i], de);
        db = de * (vj - r);
        IoT<E>::st(static_cast<E*>(p.dv) + (row * H + h) * Dv + j, bb * de);
        const float dr = -bb * de;
        // r = S'^T k ; S' = a S_{t-1}
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          red[(DK + i) * ldr + j] = fmaf(sp[i], dr, dS[i] * e);
          dS[i] = fmaf(kt[i], dr, dS[i]);
        }
#pragma unroll
        for (int i = 0; i < DK; ++i) {
          dga = fmaf(dS[i], sp[i], dga);  // a <dS', S_{t-1}> = <dS', S'>
          dS[i] *= a;
        }
      }
      db = wave_sum(db);
      dga = wave_sum(dga);
      if (lane == 0) {
        wred[wave * 2 + 0] = db;
        wred[wave * 2 + 1] = dga;
      }
      __syncthreads();
      if (j < 2 * DK) {
        float acc = 0.f;
        for (int c = 0; c < Dv; ++c) acc += red[j * ldr + c];
        E* dst = j < DK ? static_cast<E*>(p.dq) + (row * H + h) * DK + j
                        : static_cast<E*>(p.dk) + (row * H + h) * DK + (j - DK);
        IoT<E>::st(dst, acc);
      }
      if (j == 0) {
        p.dbeta[row * H + h] = ((wred[0] + wred[2]) + wred[4]) + wred[6];
        p.dg[row * H + h] = ((wred[1] + wred[3]) + wred[5]) + wred[7];
      }
      __syncthreads();
    }
  }
  if (col && p.dS0) {
#pragma unroll
    for (int i = 0; i < DK; ++i) p.dS0[(nh * DK + i) * Dv + j] = dS[i];
  }
}

template <int DK, typename E>
hipError_t launch_rec_t(const RecParams& p, hipStream_t s) {
  dim3 grid(1, p.H, p.N);
  hipLaunchKernelGGL((recurrent_fwd_kernel<DK, E>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.dO) return e;
  const size_t smem = (2 * DK * (p.Dv + 1) + 2 * kRecBlock * DK + 2 * kRecBlock + 8) * sizeof(float);
  auto kern = recurrent_bwd_kernel<DK, E>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256), smem, s, p);
  return hipGetLastError();
}

}  // namespace

size_t recurrent_bwd_ws_floats(int N, int H, int Dk, int Dv, int64_t max_len) {
  const int64_t nblk = (max_len + kRecBlock - 1) / kRecBlock;
  const int64_t ckpt = nblk * Dk * Dv;
  return static_cast<size_t>(N) * H * (ckpt + static_cast<int64_t>(kRecBlock) * Dk * Dv);
}

hipError_t launch_recurrent(const RecParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_rec_t<64, uint16_t>(p, s);
    if (Dk == 128) return launch_rec_t<128, uint16_t>(p, s);
  } else {
    if (Dk == 64) return launch_rec_t<64, float>(p, s);
    if (Dk == 128) return launch_rec_t<128, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
