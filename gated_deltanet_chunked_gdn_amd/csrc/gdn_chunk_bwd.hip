// Chunked backward pass of the gated delta rule on gfx950.
//
// Gradients of L = <o, dO> + <S_final, dS_final> (the six gradients of the
// "Research Sprint Day 1" page, "Results", plus dS0).  With the chunk algebra of
// the forward (gamma, Gamma, D, T, W, U, E, P and K~ = diag(exp(gamma_n - gamma)) K
// for one chunk of n <= 64 tokens, state S_c before it) and dOs = scale dO, the
// reverse mode of one chunk, given dS_{c+1}, is
//   dE  = K~ dS_{c+1} + P^T dOs
//   dS_c = Gamma_n dS_{c+1} + (diag(Gamma) Q)^T dOs - W^T dE        [state pass]
//        = Gamma_n dS_{c+1} + Q^T diag(Gamma) dOs - K^T diag(beta Gamma) T^T dE
//   dK~ = E dS_{c+1}^T,  dQ = diag(Gamma) dOs S_c^T + (dP o D) K,  dP = lower(dOs E^T)
//   dW  = -dE S_c^T,  dT = dE (diag(beta) V)^T + dW (diag(beta Gamma) K)^T
//   dA  = strict_lower(-T^T dT T^T),  dV = diag(beta) T^T dE
//   dK  = diag(exp(gamma_n - gamma)) dK~ + (dP o D)^T Q + (dKK + dKK^T) K
//         + diag(beta Gamma) T^T dW,   dKK = dA o beta_i D
//   dbeta, dgamma: the row sums of the terms above that carry beta, Gamma or D;
//   dg = reverse cumsum of dgamma within the chunk (gamma = cumsum g).
//
// Kernels (the forward states come from the forward state kernel run with a
// per-chunk state output):
//   chunk_dstate_kernel: one workgroup per (sequence, head, 16-column tile of
//     d_v), sequential over the chunks in reverse; holds the d_k x 16 slice of
//     dS in fp32 MFMA accumulators, stores dS_{c+1} of every chunk and dS0.  The
//     operands of chunk c - 1 are loaded while chunk c is processed; W is never
//     formed (the second form of the state pass above).
//   chunk_grad_kernel: one workgroup per (chunk, head, sequence), fully
//     parallel; loops over d_v in tiles for every product that reduces over d_v
//     (fp32 accumulators held across tiles), then the 64 x 64 and 64 x d_k
//     stages, and writes dq, dk, dv, dg, dbeta.  Per-token sums are taken per
//     wave and added in a fixed order, so the results are deterministic.
//
// Every product is a 16x16-block MFMA product whose operands are read from LDS,
// either with the reduction index contiguous or, for an operand stored the other
// way round, with transposing reads (ds_read_b64_tr_b16), so each tile is staged
// in one orientation only; a block is computed either as X or as X^T so that its
// store to LDS or HBM is contiguous along the 4 accumulator rows of a lane.  Precision as in the forward: bf16 io -> bf16 MFMA operands,
// fp32 accumulation, fp32 states, decays, sums and dS; fp32 io -> fp32 MFMA.
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

// 16-byte load through a buffer resource; offsets past its range read zeros.
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// An offset every buffer range check rejects.
constexpr int kNoLoadB = 0x7ffffff0;
// Four consecutive elements of type E (bf16 or fp32) at byte offset `off`, widened to fp32.
template <typename E>
__device__ __forceinline__ float4 bload4e(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (sizeof(E) == 2) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return float4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                  __uint_as_float(u[1] & 0xffff0000u)};
  } else {
    return __builtin_bit_cast(float4, bload16(r, off));
  }
}

template <typename E>
__device__ __forceinline__ u32x4_t ld16(const E* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
template <typename E>
__device__ __forceinline__ void st16(E* p, const u32x4_t& v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// Element e of a 16-byte vector, widened to fp32.
template <typename E>
__device__ __forceinline__ float wide_elem(const u32x4_t& v, int e);
template <>
__device__ __forceinline__ float wide_elem<uint16_t>(const u32x4_t& v, int e) {
  return __uint_as_float((e & 1) ? (v[e >> 1] & 0xffff0000u) : (v[e >> 1] << 16));
}
template <>
__device__ __forceinline__ float wide_elem<float>(const u32x4_t& v, int e) {
  return __uint_as_float(v[e]);
}

// Four consecutive io elements (8- or 16-byte aligned) widened to fp32, one LDS read.
template <typename E>
__device__ __forceinline__ f32x4_t wide4(const E* p);
template <>
__device__ __forceinline__ f32x4_t wide4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
template <>
__device__ __forceinline__ f32x4_t wide4<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}

// Store a 16x16 accumulator block C (C[4 (lane/16) + r][lane % 16] in element r)
// transposed, dst[(lane % 16) * ld + 4 (lane/16) + r]: contiguous per lane.
template <typename E>
__device__ __forceinline__ void store_t(E* dst, int ld, const f32x4_t& c, int lane) {
  store4<E>(dst + (lane & 15) * ld + 4 * (lane >> 4), c[0], c[1], c[2], c[3]);
}

// Sum over the four 16-lane groups: lanes l, l+16, l+32, l+48 all end with the total.
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
// Sum over the 16 lanes of a group: every lane of the group ends with the total.
__device__ __forceinline__ float sum_in_group(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}

// acc += A(16 x K) * B(K x 16) with A given transposed: At row-major (K x 16 block
// at `at`, leading dim lda), B stored transposed (16 x K) at `bt`.  The A operand is
// read with a transposing LDS read, so no transposed copy of At is staged.
template <typename Op, int K>
__device__ __forceinline__ void tile_mma_ta(f32x4_t& acc, const typename Op::elem* at, int lda,
                                            const typename Op::elem* bt, int ldb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += Op::KSTEP)
    acc = Op::mma(Op::frag_tr(at, lda, lane, k0), Op::frag(bt, ldb, lane, k0), acc);
}

template <int DK, typename Op>
__device__ __forceinline__ void stage_gates(const BwdParams& p, int64_t row0, int nv, int h, int lane,
                                            float* gam, float* Gam, float* dec, float* bet,
                                            float* bg) {
  // gamma by an in-register scan (log2 units); padded rows: g = 0, beta = 0
  const bool ok = lane < nv;
  const float gv = ok ? p.g[(row0 + lane) * p.H + h] : 0.f;
  const float bv = ok ? p.beta[(row0 + lane) * p.H + h] : 0.f;
  const float g2 = wave_inclusive_scan(gv * kLog2e, lane);
  const float gl2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), 63));
  const float G = exp2f(g2);
  gam[lane] = g2;
  Gam[lane] = G;
  dec[lane] = exp2f(gl2 - g2);
  if (bet) bet[lane] = bv;
  bg[lane] = bv * G;
}

// ===================================================================================
// Reverse state-gradient pass
// ===================================================================================
template <int DK, typename Op>
struct DStateSmem {
  using E = typename Op::elem;
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;   // rows of length d_k
  static constexpr int LDC = 64 + PADE;   // rows of length 64
  static constexpr int LDB = 128 + PADE;  // rows of length 128
  E Ks[64 * LDK];   // K rows
  E Qs[64 * LDK];   // Q rows
  E Tm[64 * LDC];   // T rows
  E Pr[64 * LDC];   // P rows (from the preparation kernel)
  E dB[2][16 * LDB];   // [ dOs^T | dE^T ] of each of the two tiles
  E dU[2][16 * LDB];   // [ (diag(Gamma) dOs)^T | (-diag(beta Gamma) T^T dE)^T ] of each tile
  E dSt[2][16 * LDK];  // dS^T of each tile
  float Gam[64], dec[64], bg[64];
};

// Two 16-column tiles of d_v per workgroup: waves 0-3 take the first, waves 4-7 the
// second, and all eight stage the chunk's K, Q, T and P once for both.
template <int DK, typename Op>
__global__ __launch_bounds__(512) void chunk_dstate_kernel(BwdParams p) {
  using E = typename Op::elem;
  using SM = DStateSmem<DK, Op>;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDB = SM::LDB, KS = Op::KSTEP;
  constexpr int EPV = 16 / sizeof(E);
  constexpr int SRB = DK / 64;  // 16-row blocks of dS per wave
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const E* __restrict__ q = static_cast<const E*>(p.q);
  const E* __restrict__ k = static_cast<const E*>(p.k);
  const E* __restrict__ dO = static_cast<const E*>(p.dO);
  const E* __restrict__ prw = static_cast<const E*>(p.prws);
  const E* __restrict__ tws = static_cast<const E*>(p.tws);

  const int H = p.H, Dv = p.Dv, NT = Dv / 16, NP = (NT + 1) / 2;
  const int NB = gridDim.x, L = blockIdx.x;
  const int vb = (NB % 8 == 0) ? (L % 8) * (NB / 8) + L / 8 : L;  // tiles of a head share an XCD
  const int tp = vb % NP, nh = vb / NP, h = nh % H, n = nh / H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wt = w >> 2, wl = w & 3;  // this wave's tile of the pair, its wave within the tile
  const int tile = 2 * tp + wt;
  const bool tile_ok = tile < NT;     // (an odd count of tiles leaves the last pair's second empty)
  const int j0 = (tile_ok ? tile : NT - 1) * 16;
  E* const dB = sm.dB[wt];
  E* const dU = sm.dU[wt];
  E* const dSt = sm.dSt[wt];
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int nch = static_cast<int>((len + 63) / 64);
  const int64_t slot0 = bos / 64 + n;
  const int64_t nhS = (static_cast<int64_t>(n) * H + h) * DK;

  f32x4_t dS[SRB];
#pragma unroll
  for (int sr = 0; sr < SRB; ++sr) {
    const int i = 16 * (wl * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = p.dS_final ? p.dS_final[(nhS + i + r) * Dv + j0 + j] : 0.f;
    dS[sr] = f32x4_t{x[0], x[1], x[2], x[3]};
    store4<E>(dSt + j * LDK + i, x[0], x[1], x[2], x[3]);
  }

  // The global operands of chunk c - 1 (K, Q, T, dOs, the gates) are loaded into
  // registers while chunk c is processed, and staged into LDS at the start of
  // the next step: the load latency hides behind the products.
  constexpr int NSV = 64 * (DK / EPV) / 512;  // K (and Q) vectors per thread
  constexpr int NTV = 64 * 64 / EPV / 512;    // T vectors per thread
  static_assert(NSV * 512 == 64 * (DK / EPV) && NTV * 512 == 64 * 64 / EPV, "whole vectors per thread");
  // Loads go through buffer resources bounded to the chunk's valid rows, so rows
  // past its end read as zeros without a branch or a select (either would make
  // the wave wait for every load in flight at that point), and the lane offsets
  // are 32-bit and the same for every chunk.
  constexpr int ES = static_cast<int>(sizeof(E));
  struct Pre {
    u32x4_t kv[NSV], qv[NSV], tv[NTV], pv[NTV];
    u32x4_t dor;  // four dO values of this wave's tile, row (tid % 256) / 4 (raw io elements)
    float gv, bv;
  };
  auto load_pre = [&](Pre& pr, int c) {
    const int64_t c0 = static_cast<int64_t>(c) * 64, row0 = bos + c0;
    const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
    const int rowk = ((nv - 1) * H * DK + DK) * ES;
    const auto rk = buffer_rsrc(k + (row0 * H + h) * DK, rowk);
    const auto rq = buffer_rsrc(q + (row0 * H + h) * DK, rowk);
#pragma unroll
    for (int i = 0; i < NSV; ++i) {
      const int x = tid + 512 * i, t = x / (DK / EPV), cv = (x % (DK / EPV)) * EPV;
      pr.kv[i] = bload16(rk, (t * H * DK + cv) * ES);
      pr.qv[i] = bload16(rq, (t * H * DK + cv) * ES);
    }
    const auto rt = buffer_rsrc(tws + ((slot0 + c) * H + h) * 4096, 4096 * ES);
    const auto rp = buffer_rsrc(prw + ((slot0 + c) * H + h) * 4096, 4096 * ES);
#pragma unroll
    for (int i = 0; i < NTV; ++i) {
      const int x = tid + 512 * i, t = x / (64 / EPV), cv = (x % (64 / EPV)) * EPV;
      pr.tv[i] = bload16(rt, (t * 64 + cv) * ES);
      pr.pv[i] = bload16(rp, (t * 64 + cv) * ES);
    }
    {
      const int t = (tid & 255) >> 2, cq = (tid & 3) * 4;
      const auto ro = buffer_rsrc(dO + (row0 * H + h) * Dv + j0, ((nv - 1) * H * Dv + 16) * ES);
      if constexpr (sizeof(E) == 2) {
        const auto u = __builtin_amdgcn_raw_buffer_load_b64(ro, (t * H * Dv + cq) * ES, 0, 0);
        pr.dor = u32x4_t{u[0], u[1], 0u, 0u};
      } else {
        pr.dor = bload16(ro, (t * H * Dv + cq) * ES);
      }
    }
    {  // every wave loads the gates (zeros past the chunk's end)
      const int gb = ((nv - 1) * H + 1) * 4;
      pr.gv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.g + row0 * H + h, gb), lane * H * 4, 0, 0));
      pr.bv = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(p.beta + row0 * H + h, gb), lane * H * 4, 0, 0));
    }
  };
  auto stage_pre = [&](const Pre& pr) {
#pragma unroll
    for (int i = 0; i < NSV; ++i) {
      const int x = tid + 512 * i, t = x / (DK / EPV), cv = (x % (DK / EPV)) * EPV;
      st16(sm.Ks + t * LDK + cv, pr.kv[i]);
      st16(sm.Qs + t * LDK + cv, pr.qv[i]);
    }
#pragma unroll
    for (int i = 0; i < NTV; ++i) {
      const int x = tid + 512 * i, t = x / (64 / EPV), cv = (x % (64 / EPV)) * EPV;
      st16(sm.Tm + t * LDC + cv, pr.tv[i]);
      st16(sm.Pr + t * LDC + cv, pr.pv[i]);
    }
    // gamma by an in-register scan (log2 units), in every wave; wave 0 stores the
    // decays (padded rows: g = 0, beta = 0)
    const float g2 = wave_inclusive_scan(pr.gv * kLog2e, lane);
    const float G = exp2f(g2);
    if (w == 0) {
      const float gl2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), 63));
      sm.Gam[lane] = G;
      sm.dec[lane] = exp2f(gl2 - g2);
      sm.bg[lane] = pr.bv * G;
    }
    {
      const int t = (tid & 255) >> 2, cq = (tid & 3) * 4;
      const float Gt = __shfl(G, t, 64);
      float dov[4];
      if constexpr (sizeof(E) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dov[e] = __uint_as_float((e & 1) ? (pr.dor[e >> 1] & 0xffff0000u) : (pr.dor[e >> 1] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dov[e] = __uint_as_float(pr.dor[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = dov[e];
        dB[(cq + e) * LDB + t] = Op::cvt(p.scale * x);
        dU[(cq + e) * LDB + t] = Op::cvt(p.scale * Gt * x);
      }
    }
  };
  Pre pre;
  if (nch > 0) load_pre(pre, nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    {  // dS_{c+1}, the gradient of the state after chunk c
      const auto rd = buffer_rsrc(static_cast<E*>(p.dstates) + ((slot0 + c) * H + h) * static_cast<int64_t>(DK) * Dv,
                                  tile_ok ? DK * Dv * static_cast<int>(sizeof(E)) : 0);
#pragma unroll
      for (int sr = 0; sr < SRB; ++sr) {
        const int i = 16 * (wl * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          buffer_store1e<E>(rd, ((i + r) * Dv + j0 + j) * static_cast<int>(sizeof(E)), dS[sr][r]);
      }
    }
    // ---- stage K, Q, T, P (rows), dOs^T of this tile and the gates; load chunk c - 1 ----
    stage_pre(pre);
    if (c > 0) load_pre(pre, c - 1);
    __syncthreads();

    // ---- dE = diag(decay) K dS + P^T dOs, token block wl of this wave's tile ----
    {
      f32x4_t acc = zero4();
      tile_mma<Op, DK>(acc, sm.Ks + 16 * wl * LDK, LDK, dSt, LDK, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= sm.dec[16 * wl + 4 * (lane >> 4) + r];
      for (int ks = (16 * wl) / KS; ks < 64 / KS; ++ks)
        acc = Op::mma(Op::frag_tr(sm.Pr + 16 * wl, LDC, lane, ks * KS), Op::frag(dB, LDB, lane, ks * KS), acc);
      store_t<E>(dB + 64 + 16 * wl, LDB, acc, lane);
    }
    __syncthreads();

    // ---- F = T^T dE (token block wl; T is lower triangular), scaled to -beta Gamma F ----
    // (-W^T dE = K^T diag(-beta Gamma) T^T dE, so W itself is never formed)
    {
      f32x4_t acc = zero4();
      for (int ks = (16 * wl) / KS; ks < 64 / KS; ++ks)
        acc = Op::mma(Op::frag_tr(sm.Tm + 16 * wl, LDC, lane, ks * KS), Op::frag(dB + 64, LDB, lane, ks * KS), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= -sm.bg[16 * wl + 4 * (lane >> 4) + r];
      store_t<E>(dU + 64 + 16 * wl, LDB, acc, lane);
    }
    __syncthreads();

    // ---- dS <- Gamma_n dS + [Q^T | K^T] [diag(Gamma) dOs ; -diag(beta Gamma) F] ----
    {
      const float gn = sm.Gam[63];
#pragma unroll
      for (int sr = 0; sr < SRB; ++sr) {
        const int rb = wl * SRB + sr;
        f32x4_t acc = dS[sr] * gn;
#pragma unroll
        for (int ks = 0; ks < 64 / KS; ++ks)
          acc = Op::mma(Op::frag_tr(sm.Qs + 16 * rb, LDK, lane, ks * KS), Op::frag(dU, LDB, lane, ks * KS), acc);
#pragma unroll
        for (int ks = 0; ks < 64 / KS; ++ks)
          acc = Op::mma(Op::frag_tr(sm.Ks + 16 * rb, LDK, lane, ks * KS), Op::frag(dU + 64, LDB, lane, ks * KS),
                        acc);
        dS[sr] = acc;
        store_t<E>(dSt + 16 * rb, LDK, acc, lane);
      }
    }
    __syncthreads();
  }
  if (p.dS0 && tile_ok) {
#pragma unroll
    for (int sr = 0; sr < SRB; ++sr) {
      const int i = 16 * (wl * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dS0[(nhS + i + r) * Dv + j0 + j] = dS[sr][r];
    }
  }
}

// ===================================================================================
// Per-chunk gradients
// ===================================================================================
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// LDS plan (element offsets; E = io element type).  Persistent: K rows, T.  Every
// transposed operand (of K, Q, T, V, dOs, S, dS, dE, dW, dQK and dKK) is read with
// transposing LDS reads from the one stored orientation.
// Region U is reused: first the pre-chunk products and the d_v tiles, then the
// 64 x 64 / 64 x d_k stages.
template <int DK, typename Op>
struct GradLayout {
  using E = typename Op::elem;
  static constexpr int DVT = sizeof(E) == 2 ? 32 : 16;  // d_v tile (one bf16 MFMA depth)
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE, LDC = 64 + PADE, LDV = DVT + PADE;
  static constexpr int nK = 64 * LDK, nC = 64 * LDC, nV = 64 * LDV, nS = DK * LDV;
  static constexpr int oKs = 0, oTm = oKs + nK, oU = oTm + nC;
  // pre-chunk and d_v tiles
  static constexpr int aWn = 0, aPr = aWn + nK, aTile = aPr + nC;
  static constexpr int aVr = aTile, aSr = aVr + nV, adSr = aSr + nS, adOr = adSr + nS;
  static constexpr int aEr = adOr + nV, adEr = aEr + nV, aEnd = adEr + nV;
  // 64 x 64 and 64 x d_k stages: dQK^T, dKK^T, dW rows (then Q rows), dT^T, X^T
  static constexpr int bQKt = 0, bKKt = bQKt + nC, bWr = bKKt + nC, bQr = bWr;
  static constexpr int bTb = bWr + nK, bXt = bTb + nC, bEnd = bXt + nC;
  static constexpr int nU = cmax(aEnd, bEnd);
  static constexpr int nElem = oU + nU;
  static constexpr int fOff = (nElem * static_cast<int>(sizeof(E)) + 15) / 16 * 16;
  // fp32 arrays: gam, Gam, dec, bet, bg [64]; pb, pg [8][64]; pn, sdot [8]
  static constexpr int nFloat = 5 * 64 + 2 * 8 * 64 + 16;
  static constexpr size_t bytes = static_cast<size_t>(fOff) + nFloat * 4;
};

// With bf16 operands at d_k = 64 the kernel is held to 128 registers so that two
// workgroups share a CU (a few registers spill; measured faster than one
// workgroup per CU without spills).
template <int DK, typename Op>
__global__ __launch_bounds__(512)
__attribute__((amdgpu_waves_per_eu(DK == 64 && sizeof(typename Op::elem) == 2 ? 4 : 1))) void chunk_grad_kernel(
    BwdParams p) {
  using E = typename Op::elem;
  using GL = GradLayout<DK, Op>;
  constexpr int LDK = GL::LDK, LDC = GL::LDC, LDV = GL::LDV, DVT = GL::DVT, KS = Op::KSTEP;
  constexpr int EPV = 16 / sizeof(E);
  constexpr int NKS = DK / 32;  // 64 x d_k blocks per wave (4 * DK / 16 over 8 waves)
  constexpr int NBT = DVT / 16 * 4;  // (d_v, token) blocks of one tile
  extern __shared__ __align__(16) char smem_raw[];
  E* const base = reinterpret_cast<E*>(smem_raw);
  E* const Ks = base + GL::oKs;
  E* const Tm = base + GL::oTm;
  E* const U = base + GL::oU;
  float* const fl = reinterpret_cast<float*>(smem_raw + GL::fOff);
  float* const gam = fl;
  float* const Gam = fl + 64;
  float* const dec = fl + 128;
  float* const bet = fl + 192;
  float* const bg = fl + 256;
  float* const pb = fl + 320;        // [8][64] per-wave partial dbeta
  float* const pg = fl + 320 + 512;  // [8][64] per-wave partial dgamma
  float* const pn = fl + 320 + 1024;      // [8] per-wave partial dgamma_n
  float* const sdot = fl + 320 + 1024 + 8;  // [8] per-wave <dS_{c+1}, S_c>

  const E* __restrict__ q = static_cast<const E*>(p.q);
  const E* __restrict__ k = static_cast<const E*>(p.k);
  const E* __restrict__ v = static_cast<const E*>(p.v);
  const E* __restrict__ dO = static_cast<const E*>(p.dO);
  const E* __restrict__ prw = static_cast<const E*>(p.prws);
  const E* __restrict__ tws = static_cast<const E*>(p.tws);
  E* __restrict__ dq = static_cast<E*>(p.dq);
  E* __restrict__ dk = static_cast<E*>(p.dk);
  E* __restrict__ dvo = static_cast<E*>(p.dv);

  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int H = p.H, Dv = p.Dv;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t c0 = static_cast<int64_t>(c) * 64;
  if (c0 >= len) return;
  const int64_t row0 = bos + c0;
  const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
  const int64_t slot = bos / 64 + n + c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const E* Sg = static_cast<const E*>(p.states) + (slot * H + h) * static_cast<int64_t>(DK) * Dv;
  const E* dSg = static_cast<const E*>(p.dstates) + (slot * H + h) * static_cast<int64_t>(DK) * Dv;

  // Global operands of one d_v tile (V and dO rows, S_c and dS_{c+1}), loaded into
  // registers one tile ahead of their use.
  constexpr int NVX = (64 * (DVT / EPV) + 511) / 512;
  constexpr int NSX = (DK * (DVT / 4) + 511) / 512;
  struct TileLd {
    u32x4_t vv[NVX], ov[NVX];
    float4 sv[NSX], dv[NSX];
  };
  TileLd tl;
  // Buffer resources bounded to the chunk's valid rows and the state slots: rows
  // past the chunk's end and columns past d_v read as zeros (and are never
  // stored), with 32-bit offsets instead of per-lane 64-bit addresses.
  const int rowb = ((nv - 1) * H * Dv + Dv) * static_cast<int>(sizeof(E));
  const auto rv = buffer_rsrc(v + (row0 * H + h) * Dv, rowb);
  const auto rdo = buffer_rsrc(dO + (row0 * H + h) * Dv, rowb);
  const auto rdv = buffer_rsrc(dvo + (row0 * H + h) * Dv, rowb);
  const auto rs = buffer_rsrc(Sg, DK * Dv * static_cast<int>(sizeof(E)));
  const int rowk = ((nv - 1) * H * DK + DK) * static_cast<int>(sizeof(E));
  const auto rq = buffer_rsrc(q + (row0 * H + h) * DK, rowk);
  const auto rk = buffer_rsrc(k + (row0 * H + h) * DK, rowk);
  const auto rdq = buffer_rsrc(dq + (row0 * H + h) * DK, rowk);
  const auto rdk = buffer_rsrc(dk + (row0 * H + h) * DK, rowk);
  const auto rds = buffer_rsrc(dSg, DK * Dv * static_cast<int>(sizeof(E)));
  auto load_tile = [&](TileLd& L, int v0) {
#pragma unroll
    for (int ix = 0; ix < NVX; ++ix) {
      const int x = tid + 512 * ix, t = x / (DVT / EPV), cv = (x % (DVT / EPV)) * EPV;
      const int off = x < 64 * (DVT / EPV) && v0 + cv < Dv ? (t * H * Dv + v0 + cv) * static_cast<int>(sizeof(E))
                                                             : kNoLoadB;
      L.vv[ix] = bload16(rv, off);
      L.ov[ix] = bload16(rdo, off);
    }
#pragma unroll
    for (int ix = 0; ix < NSX; ++ix) {
      const int x = tid + 512 * ix, i = x / (DVT / 4), cv = (x % (DVT / 4)) * 4;
      const int off = x < DK * (DVT / 4) && v0 + cv < Dv ? (i * Dv + v0 + cv) * static_cast<int>(sizeof(E)) : kNoLoadB;
      L.sv[ix] = bload4e<E>(rs, off);
      L.dv[ix] = bload4e<E>(rds, off);
    }
  };

  // ---------------- stage K, T, P (rows); gates ----------------
  E* const Wn = U + GL::aWn;
  E* const Pr = U + GL::aPr;
  {
    for (int x = tid; x < 64 * (DK / EPV); x += 512) {
      const int t = x / (DK / EPV), cv = (x % (DK / EPV)) * EPV;
      const u32x4_t kv = bload16(rk, (t * H * DK + cv) * static_cast<int>(sizeof(E)));
      st16(Ks + t * LDK + cv, kv);
    }
    const E* T = tws + (slot * H + h) * 4096;
    const E* P = prw + (slot * H + h) * 4096;
    for (int x = tid; x < 64 * 64 / EPV; x += 512) {
      const int t = x / (64 / EPV), cv = (x % (64 / EPV)) * EPV;
      const u32x4_t tv = ld16(T + t * 64 + cv), pv = ld16(P + t * 64 + cv);
      st16(Tm + t * LDC + cv, tv);
      st16(Pr + t * LDC + cv, pv);
    }
    for (int x = tid; x < 2 * 8 * 64 + 16; x += 512) pb[x] = 0.f;  // pb, pg, pn, sdot
    if (w == 0) stage_gates<DK, Op>(p, row0, nv, h, lane, gam, Gam, dec, bet, bg);
    load_tile(tl, 0);  // the first d_v tile's operands, while the pre-tile products run
    __syncthreads();

    // -W (rows t) from W^T = K^T (T diag(beta Gamma))^T; blocks (a: d_k, b: tokens)
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int idx = w + 8 * s, a = idx >> 2, b = idx & 3;
      f32x4_t acc = zero4();
      for (int ks = 0; ks < (16 * (b + 1) + KS - 1) / KS; ++ks)
        acc = Op::mma(Op::frag_tr(Ks + 16 * a, LDK, lane, ks * KS),
                      Op::scale(Op::frag(Tm + 16 * b * LDC, LDC, lane, ks * KS), bg, lane, ks * KS), acc);
      store_t<E>(Wn + 16 * b * LDK + 16 * a, LDK, -acc, lane);
    }
  }
  // Lower 16x16 blocks (bi >= bj) owned by this wave: blk w, and 8 + w for w < 2.
  const int nlow = w < 2 ? 2 : 1;
  int lbi[2], lbj[2];
  lower_block(w, lbi[0], lbj[0]);
  lower_block(w < 2 ? 8 + w : w, lbi[1], lbj[1]);
  __syncthreads();

  // ---------------- d_v tiles ----------------
  f32x4_t dKtT[NKS], dQ6T[NKS], dWT[NKS], dP[2], dT1T[2];
#pragma unroll
  for (int s = 0; s < NKS; ++s) dKtT[s] = dQ6T[s] = dWT[s] = zero4();
  dP[0] = dP[1] = dT1T[0] = dT1T[1] = zero4();
  float sdot_acc = 0.f;
  E* const Vr = U + GL::aVr;
  E* const Sr = U + GL::aSr;
  E* const dSr = U + GL::adSr;
  E* const dOr = U + GL::adOr;
  E* const Er = U + GL::aEr;
  E* const dEr = U + GL::adEr;
  auto stage_tile = [&](const TileLd& L, int v0) {
#pragma unroll
    for (int ix = 0; ix < NVX; ++ix) {
      const int x = tid + 512 * ix, t = x / (DVT / EPV), cv = (x % (DVT / EPV)) * EPV;
      if (x < 64 * (DVT / EPV)) {
        st16(Vr + t * LDV + cv, L.vv[ix]);
        E os[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) os[e] = Op::cvt(p.scale * wide_elem<E>(L.ov[ix], e));
        st16(dOr + t * LDV + cv, *reinterpret_cast<const u32x4_t*>(os));
      }
    }
#pragma unroll
    for (int ix = 0; ix < NSX; ++ix) {
      const int x = tid + 512 * ix, i = x / (DVT / 4), cv = (x % (DVT / 4)) * 4;
      if (x < DK * (DVT / 4)) {
        const float4 sv = L.sv[ix], dv4 = L.dv[ix];
        sdot_acc += sv.x * dv4.x + sv.y * dv4.y + sv.z * dv4.z + sv.w * dv4.w;
        store4<E>(Sr + i * LDV + cv, sv.x, sv.y, sv.z, sv.w);
        store4<E>(dSr + i * LDV + cv, dv4.x, dv4.y, dv4.z, dv4.w);
      }
    }
  };
  for (int v0 = 0; v0 < Dv; v0 += DVT) {
    // stage V and dOs (rows and transposed), S_c and dS_{c+1} (rows and transposed);
    // load the next tile meanwhile
    stage_tile(tl, v0);
    if (v0 + DVT < Dv) load_tile(tl, v0 + DVT);
    __syncthreads();
    // E^T and dE^T, block (bdv, bt) per wave
    if (w < NBT) {
      const int bdv = w >> 2, bt = w & 3;
      f32x4_t e = zero4();
      for (int ks = 0; ks < (16 * (bt + 1) + KS - 1) / KS; ++ks)
        e = Op::mma(Op::frag_tr(Vr + 16 * bdv, LDV, lane, ks * KS),
                    Op::scale(Op::frag(Tm + 16 * bt * LDC, LDC, lane, ks * KS), bet, lane, ks * KS), e);
      tile_mma_ta<Op, DK>(e, Sr + 16 * bdv, LDV, Wn + 16 * bt * LDK, LDK, lane);
      store_t<E>(Er + 16 * bt * LDV + 16 * bdv, LDV, e, lane);
      f32x4_t de = zero4();
      tile_mma_ta<Op, DK>(de, dSr + 16 * bdv, LDV, Ks + 16 * bt * LDK, LDK, lane);
      const float dc = dec[16 * bt + (lane & 15)];
      de = de * dc;
      for (int ks = (16 * bt) / KS; ks < 64 / KS; ++ks)
        de = Op::mma(Op::frag_tr(dOr + 16 * bdv, LDV, lane, ks * KS),
                     Op::frag_tr(Pr + 16 * bt, LDC, lane, ks * KS), de);
      store_t<E>(dEr + 16 * bt * LDV + 16 * bdv, LDV, de, lane);
    }
    __syncthreads();
    // accumulate the d_v reductions
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int idx = w + 8 * s, a = idx >> 2, b = idx & 3;
      tile_mma<Op, DVT>(dKtT[s], dSr + 16 * a * LDV, LDV, Er + 16 * b * LDV, LDV, lane);
      tile_mma<Op, DVT>(dQ6T[s], Sr + 16 * a * LDV, LDV, dOr + 16 * b * LDV, LDV, lane);
      tile_mma<Op, DVT>(dWT[s], Sr + 16 * a * LDV, LDV, dEr + 16 * b * LDV, LDV, lane);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nlow) {
        const int bi = lbi[s], bj = lbj[s];
        tile_mma<Op, DVT>(dP[s], dOr + 16 * bi * LDV, LDV, Er + 16 * bj * LDV, LDV, lane);
        tile_mma<Op, DVT>(dT1T[s], Vr + 16 * bj * LDV, LDV, dEr + 16 * bi * LDV, LDV, lane);
      }
    }
    // dV^T block = (T^T dE)^T; dv = beta dVb; dbeta += rowsum(dVb o V)
    if (w < NBT) {
      const int bdv = w >> 2, bt = w & 3;
      f32x4_t acc = zero4();
      for (int ks = (16 * bt) / KS; ks < 64 / KS; ++ks)
        acc = Op::mma(Op::frag_tr(dEr + 16 * bdv, LDV, lane, ks * KS),
                      Op::frag_tr(Tm + 16 * bt, LDC, lane, ks * KS), acc);
      const int t = 16 * bt + (lane & 15), cl = 16 * bdv + 4 * (lane >> 4);
      const float bt_ = bet[t];
      float part = 0.f;
      const f32x4_t vrow = wide4<E>(Vr + t * LDV + cl);
#pragma unroll
      for (int r = 0; r < 4; ++r) part += acc[r] * vrow[r];
      part = sum_groups(part);
      if (lane < 16) pb[w * 64 + t] += part;
      buffer_store4<E>(rdv, v0 + cl < Dv ? (t * H * Dv + v0 + cl) * static_cast<int>(sizeof(E)) : kNoLoadB,
                       bt_ * acc[0], bt_ * acc[1], bt_ * acc[2], bt_ * acc[3]);
    }
    __syncthreads();
  }
  sdot_acc = wave_sum(sdot_acc);
  if (lane == 0) sdot[w] = sdot_acc;

  {
    // Lane-derived values are formed again from here on (through an opaque copy
    // of the thread index), so that no address computed before the d_v loop stays
    // live across it: kept live, they cost more registers than the 128 this
    // kernel is held to, and their spill traffic outweighed the recomputation.
    int tid_o = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid_o));
    const int tid = tid_o, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // ---------------- 64 x 64 and 64 x d_k stages ----------------
    E* const dQKt = U + GL::bQKt;
    E* const dKKt = U + GL::bKKt;
    E* const dWr = U + GL::bWr;
    E* const Qr = U + GL::bQr;
    E* const dTb = U + GL::bTb;
    E* const Xt = U + GL::bXt;
    // Q rows for the last stage (its operand Q^T, read transposed), loaded now and
    // staged once dW is no longer needed (rows past the chunk's end read zeros).
    constexpr int NQV = 64 * (DK / EPV) / 512;
    u32x4_t qpre[NQV];
  #pragma unroll
    for (int i = 0; i < NQV; ++i) {
      const int x = tid + 512 * i, t = x / (DK / EPV), cv = (x % (DK / EPV)) * EPV;
      qpre[i] = bload16(rq, (t * H * DK + cv) * static_cast<int>(sizeof(E)));
    }
    // dW rows; dQK = dP o D (stored transposed)
  #pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int idx = w + 8 * s, a = idx >> 2, b = idx & 3;
      store_t<E>(dWr + 16 * b * LDK + 16 * a, LDK, -dWT[s], lane);  // dW^T block (a, b)
    }
    {  // zero the 16x16 blocks no owner writes: above the diagonal in dT^T, below it
       // in dQK^T and dKK^T (16-byte stores)
      constexpr int VR = 16 / EPV, NZ = 3 * 6 * 16 * VR;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      for (int x = tid; x < NZ; x += 512) {
        const int arr = x / (6 * 16 * VR), rem = x % (6 * 16 * VR);
        const int blk = rem / (16 * VR), rr = (rem / VR) % 16, cv = (rem % VR) * EPV;
        const int bu = blk < 3 ? 0 : (blk < 5 ? 1 : 2), bl = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
        E* const base = arr == 0 ? dTb : (arr == 1 ? dQKt : dKKt);
        const int rb = arr == 0 ? bu : bl, cb = arr == 0 ? bl : bu;
        st16(base + (16 * rb + rr) * LDC + 16 * cb + cv, z);
      }
    }
  #pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nlow) {
        const int bi = lbi[s], bj = lbj[s];
        const int i0 = 16 * bi + 4 * (lane >> 4), j = 16 * bj + (lane & 15);
        f32x4_t dqk;
  #pragma unroll
        for (int r = 0; r < 4; ++r)
          dqk[r] = i0 + r >= j ? dP[s][r] * exp2f(fminf(gam[i0 + r] - gam[j], 0.f)) : 0.f;
        store_t<E>(dQKt + 16 * bj * LDC + 16 * bi, LDC, dqk, lane);
      }
    }
    __syncthreads();
    // dT^T = diag(beta) dT1^T + diag(beta Gamma) (K dW^T), strictly lower part of dT.
    // dKb^T = dW^T T (the last use of dW; kept in registers for the final stage).
  #pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nlow) {
        const int bi = lbi[s], bj = lbj[s];
        f32x4_t acc = zero4();
        tile_mma<Op, DK>(acc, Ks + 16 * bj * LDK, LDK, dWr + 16 * bi * LDK, LDK, lane);
        const int j0 = 16 * bj + 4 * (lane >> 4), i = 16 * bi + (lane & 15);
        f32x4_t dt;
  #pragma unroll
        for (int r = 0; r < 4; ++r)
          dt[r] = i > j0 + r ? bet[j0 + r] * dT1T[s][r] + bg[j0 + r] * acc[r] : 0.f;
        store_t<E>(dTb + 16 * bi * LDC + 16 * bj, LDC, dt, lane);
      }
    }
    f32x4_t dKbT[NKS];
  #pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int idx = w + 8 * s, a = idx >> 2, b = idx & 3;
      dKbT[s] = zero4();
      for (int ks = (16 * b) / KS; ks < 64 / KS; ++ks)
        dKbT[s] = Op::mma(Op::frag_tr(dWr + 16 * a, LDK, lane, ks * KS),
                          Op::frag_tr(Tm + 16 * b, LDC, lane, ks * KS), dKbT[s]);
    }
    __syncthreads();
    // X = dT T^T (all 16 blocks, two per wave), stored transposed.  The Q rows go
    // where dW was.
  #pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int idx = w + 8 * s, bk = idx >> 2, bj = idx & 3;
      f32x4_t acc = zero4();
      const int kb = bk < bj ? bk : bj;
      for (int ks = 0; ks < (16 * (kb + 1) + KS - 1) / KS; ++ks)
        acc = Op::mma(Op::frag(dTb + 16 * bk * LDC, LDC, lane, ks * KS),
                      Op::frag(Tm + 16 * bj * LDC, LDC, lane, ks * KS), acc);
      store_t<E>(Xt + 16 * bj * LDC + 16 * bk, LDC, acc, lane);
    }
  #pragma unroll
    for (int i = 0; i < NQV; ++i) {
      const int x = tid + 512 * i, t = x / (DK / EPV), cv = (x % (DK / EPV)) * EPV;
      st16(Qr + t * LDK + cv, qpre[i]);
    }
    __syncthreads();
    // dA = strict_lower(-T^T X); QK and KK formed again; dbeta, dKK (stored
    // transposed), dD = dP o QK; dDD row and column sums.
  #pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s < nlow) {
        const int bi = lbi[s], bj = lbj[s];
        f32x4_t qk = zero4(), kkb = zero4();
        tile_mma<Op, DK>(qk, Qr + 16 * bi * LDK, LDK, Ks + 16 * bj * LDK, LDK, lane);
        tile_mma<Op, DK>(kkb, Ks + 16 * bi * LDK, LDK, Ks + 16 * bj * LDK, LDK, lane);
        f32x4_t acc = zero4();
        for (int ks = (16 * bi) / KS; ks < 64 / KS; ++ks)
          acc = Op::mma(Op::frag_tr(Tm + 16 * bi, LDC, lane, ks * KS),
                        Op::frag(Xt + 16 * bj * LDC, LDC, lane, ks * KS), acc);
        const int i0 = 16 * bi + 4 * (lane >> 4), j = 16 * bj + (lane & 15);
        f32x4_t dkk, dd;
        float rows[4], colp = 0.f;
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + r;
          const bool lo = i > j;
          const float d = i >= j ? exp2f(fminf(gam[i] - gam[j], 0.f)) : 0.f;
          const float da = lo ? -acc[r] : 0.f;
          const float b_i = bet[i];
          const float kk = kkb[r];
          rows[r] = da * kk * d;                 // dbeta_i
          dkk[r] = da * b_i * d;                 // dKK
          const float dd0 = i >= j ? dP[s][r] * qk[r] : 0.f;  // dD = dP o QK
          dd[r] = (dd0 + da * b_i * kk) * d;     // dD o D
          colp += dd[r];
        }
        store_t<E>(dKKt + 16 * bj * LDC + 16 * bi, LDC, dkk, lane);
        // row sums over the 16 lanes of a group; column sums over the four groups
        float rs[4], rd[4];
  #pragma unroll
        for (int r = 0; r < 4; ++r) {
          rs[r] = sum_in_group(rows[r]);
          rd[r] = sum_in_group(dd[r]);
        }
        colp = sum_groups(colp);
        if ((lane & 15) == 0) {
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            pb[w * 64 + i0 + r] += rs[r];
            pg[w * 64 + i0 + r] += rd[r];
          }
        }
        if (lane < 16) pg[w * 64 + j] -= colp;
      }
    }
    __syncthreads();
    // dq^T, dk^T blocks (a: d_k, b: tokens) and the per-token terms they carry
    float pn_acc = 0.f;
  #pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int idx = w + 8 * s, a = idx >> 2, b = idx & 3;
      const int t = 16 * b + (lane & 15), d0 = 16 * a + 4 * (lane >> 4);
      // dq^T = Gamma o (dOs S_c^T)^T + K^T dQK^T
      const f32x4_t q6 = dQ6T[s] * Gam[t];
      f32x4_t dqa = q6;
      for (int ks = 0; ks < (16 * (b + 1) + KS - 1) / KS; ++ks)
        dqa = Op::mma(Op::frag_tr(Ks + 16 * a, LDK, lane, ks * KS),
                      Op::frag_tr(dQKt + 16 * b, LDC, lane, ks * KS), dqa);
      // dk^T = decay o dK~^T + Q^T dQK + K^T (dKK + dKK^T) + (beta Gamma) o dKb^T;
      // dKK is strictly lower, so only token blocks >= b of dKK and <= b of dKK^T
      // reach column block b
      f32x4_t dka = zero4();
      for (int ks = (16 * b) / KS; ks < 64 / KS; ++ks)
        dka = Op::mma(Op::frag_tr(Qr + 16 * a, LDK, lane, ks * KS),
                      Op::frag(dQKt + 16 * b * LDC, LDC, lane, ks * KS), dka);
      for (int ks = (16 * b) / KS; ks < 64 / KS; ++ks)
        dka = Op::mma(Op::frag_tr(Ks + 16 * a, LDK, lane, ks * KS),
                      Op::frag(dKKt + 16 * b * LDC, LDC, lane, ks * KS), dka);
      for (int ks = 0; ks < (16 * (b + 1) + KS - 1) / KS; ++ks)
        dka = Op::mma(Op::frag_tr(Ks + 16 * a, LDK, lane, ks * KS),
                      Op::frag_tr(dKKt + 16 * b, LDC, lane, ks * KS), dka);
      const float dct = dec[t], bgt = bg[t];
      float qd = 0.f, rk = 0.f, tj = 0.f;
      const f32x4_t krow = wide4<E>(Ks + t * LDK + d0), qrow = wide4<E>(Qr + t * LDK + d0);
  #pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float kv = krow[r];
        qd += qrow[r] * q6[r];
        rk += dKbT[s][r] * kv;
        tj += dKtT[s][r] * dct * kv;
        dka[r] += dct * dKtT[s][r] + bgt * dKbT[s][r];
      }
      qd = sum_groups(qd);
      rk = sum_groups(rk);
      tj = sum_groups(tj);
      if (lane < 16) {
        pg[w * 64 + t] += qd + bet[t] * Gam[t] * rk - tj;
        pb[w * 64 + t] += Gam[t] * rk;
        pn_acc += tj;
      }
      {
        const int off = (t * H * DK + d0) * static_cast<int>(sizeof(E));
        buffer_store4<E>(rdq, off, dqa[0], dqa[1], dqa[2], dqa[3]);
        buffer_store4<E>(rdk, off, dka[0], dka[1], dka[2], dka[3]);
      }
    }
    pn_acc = wave_sum(pn_acc);
    if (lane == 0) pn[w] = pn_acc;
    __syncthreads();
    if (w == 0) {
      float db = 0.f, dgm = 0.f;
  #pragma unroll
      for (int x = 0; x < 8; ++x) {
        db += pb[x * 64 + lane];
        dgm += pg[x * 64 + lane];
      }
      if (lane == 63) {
        float sd = 0.f, sn = 0.f;
  #pragma unroll
        for (int x = 0; x < 8; ++x) {
          sd += sdot[x];
          sn += pn[x];
        }
        dgm += Gam[63] * sd + sn;
      }
      // dg_t = sum of dgamma_u over u >= t: a forward scan of the reversed lanes
      const float rev = __shfl(dgm, 63 - lane, 64);
      const float sc = wave_inclusive_scan(rev, lane);
      const float dgt = __shfl(sc, 63 - lane, 64);
      if (lane < nv) {
        p.dg[(row0 + lane) * H + h] = dgt;
        p.dbeta[(row0 + lane) * H + h] = db;
      }
    }
  }
}

template <int DK, typename Op>
hipError_t launch_bwd_t(const BwdParams& b, hipStream_t s) {
  constexpr size_t ds_smem = sizeof(DStateSmem<DK, Op>);
  constexpr size_t gr_smem = GradLayout<DK, Op>::bytes;
  static_assert(ds_smem <= 160 * 1024 && gr_smem <= 160 * 1024, "LDS budget exceeded");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_dstate_kernel<DK, Op>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(ds_smem));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_grad_kernel<DK, Op>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(gr_smem));
  if (e != hipSuccess) return e;
  auto dstate = chunk_dstate_kernel<DK, Op>;
  auto grad = chunk_grad_kernel<DK, Op>;
  hipLaunchKernelGGL(dstate, dim3(b.N * b.H * ((b.Dv / 16 + 1) / 2)), dim3(512), ds_smem, s, b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (b.max_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(grad, dim3(b.max_chunks, b.H, b.N), dim3(512), gr_smem, s, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bwd(const BwdParams& b, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_bwd_t<64, OpBf16>(b, s);
    if (Dk == 128) return launch_bwd_t<128, OpBf16>(b, s);
  } else {
    if (Dk == 64) return launch_bwd_t<64, OpF32>(b, s);
    if (Dk == 128) return launch_bwd_t<128, OpF32>(b, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
