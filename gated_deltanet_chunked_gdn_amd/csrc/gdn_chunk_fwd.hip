// Chunked forward pass of the gated delta rule on gfx950.
//
// One workgroup (4 waves) owns one (sequence, head, 16-column tile of d_v) and
// walks the sequence's chunks of 64 tokens in order.  Column j of the state
// only ever mixes with column j of v (k, alpha and beta are shared by every
// column: the update of "Research Sprint Day 1", section "The GDN update"), so
// the tiles of a head are independent and need no communication.  The
// workgroup keeps its d_k x 16 slice of S in fp32 MFMA accumulators for the
// whole sequence; HBM sees each input once and each output once.
//
// Per chunk (n <= 64 tokens; padded rows carry k = q = v = 0, g = 0, beta = 0,
// which leaves every result unchanged):
//   gamma = cumsum(g)  (one wave-wide scan), Gamma = exp(gamma)         [cumsum of g
//          rather than a product of alpha: "Research Sprint Day 2", gates step 5]
//   A = strict_lower(diag(beta) (K K^T) o D),  D_ij = exp(gamma_i - gamma_j)
//   P = lower_incl((Q K^T) o D)                                  [causal QK score]
//   T = (I + A)^-1, fp32: 16x16 diagonal blocks by forward substitution, the
//       off-diagonal blocks by T_ij = -T_ii sum_k A_ik T_kj with fp32 MFMA
//                                                     [triangular inverse/solve]
//   R = diag(beta) (V - diag(Gamma) K S),  E = T R     [the errors e_t, i.e. the
//                                                      WY value tensor minus W S]
//   O = scale (diag(Gamma) Q S + P E)
//   S <- Gamma_n S + (diag(exp(gamma_n - gamma)) K)^T E
// (intermediates named as in the fla issue #1550 page, "Intermediate rounding
// diagnosis").  Exponents are never positive, so decays underflow to zero
// harmlessly and nothing is divided by a decay.
//
// Precision: the bf16 instantiation feeds bf16 operands to
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation; S, gamma, the decays, A and
// the solve stay fp32, and T, P, R, E and the state operand are rounded to bf16
// only as MFMA inputs.  The fp32 instantiation runs every product on
// v_mfma_f32_16x16x4_f32 (IEEE fp32 products and sums).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DT, typename Op>
struct FwdSmem {
  using E = typename Op::elem;
  // Row strides chosen so that the 16 rows one MFMA fragment read touches fall
  // in distinct LDS banks (row pitch = 4 banks mod 64).
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;  // rows of length d_k
  static constexpr int LDC = 64 + PADE;  // rows of length 64 (one chunk)
  static constexpr int LDF = 64 + 4;     // fp32 rows of length 64
  static constexpr int LDM = 20;         // per-wave 16x16 fp32 scratch
  E Ks[64 * LDK];    // K, token-major
  E Qs[64 * LDK];    // Q, token-major
  E KtT[DK * LDC];   // (diag(exp(gamma_n - gamma)) K)^T, d_k-major
  E Tm[64 * LDC];    // T as an MFMA operand
  E Pm[64 * LDC];    // P as an MFMA operand
  E St[DT * LDK];    // S^T (tile columns x d_k) as an MFMA operand
  E Rt[DT * LDC];    // R^T
  E Et[DT * LDC];    // E^T
  float Af[64 * LDF];
  float Tf[64 * LDF];
  float Mt[4 * 16 * LDM];
  float Vs[64 * DT];
  float gam[64], Gam[64], dec[64], bet[64];
};

// Lower-triangular 16x16 block (bi >= bj) of a 4x4 block grid, by index 0..9.
__device__ __forceinline__ void lower_block(int b, int& bi, int& bj) {
  bi = b < 1 ? 0 : b < 3 ? 1 : b < 6 ? 2 : 3;
  bj = b - bi * (bi + 1) / 2;
}

template <int DK, typename Op>
__device__ __forceinline__ void load_rows(typename Op::elem* dst, int ld,
                                          const typename Op::elem* src, int64_t row0, int nv,
                                          int H, int h, int tid) {
  using E = typename Op::elem;
  constexpr int EPV = 16 / sizeof(E);  // elements per 16-byte vector
  constexpr int VPR = DK / EPV;        // vectors per row
#pragma unroll
  for (int x = tid; x < 64 * VPR; x += 256) {
    const int t = x / VPR, c = x % VPR;
    uint4 val = {0u, 0u, 0u, 0u};
    if (t < nv) val = *reinterpret_cast<const uint4*>(src + ((row0 + t) * H + h) * DK + c * EPV);
    *reinterpret_cast<uint4*>(dst + t * ld + c * EPV) = val;
  }
}

template <int DK, int DT, typename Op>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(FwdParams p) {
  using E = typename Op::elem;
  using SM = FwdSmem<DK, DT, Op>;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDF = SM::LDF, LDM = SM::LDM;
  constexpr int SRB = DK / 64;  // 16-row blocks of S per wave
  constexpr int NCB = DT / 16;  // 16-column blocks per tile
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = blockIdx.x * DT, h = blockIdx.y, n = blockIdx.z;
  const int H = p.H, Dv = p.Dv;
  int64_t bos, len;
  if (p.seq.cu) {
    bos = p.seq.cu[n];
    len = p.seq.cu[n + 1] - bos;
  } else {
    bos = static_cast<int64_t>(n) * p.seq.T;
    len = p.seq.T;
  }
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  E* o = static_cast<E*>(p.o);

  // Blocks above the diagonal of T and P are never written: zero them once.
  for (int x = tid; x < 64 * LDC; x += 256) {
    sm.Tm[x] = Op::cvt(0.f);
    sm.Pm[x] = Op::cvt(0.f);
  }

  f32x4_t Sacc[SRB][NCB];
#pragma unroll
  for (int s = 0; s < SRB; ++s)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * (wave * SRB + s) + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
        const float x = p.S0 ? p.S0[((static_cast<int64_t>(n) * H + h) * DK + i) * Dv + j0 + j] : 0.f;
        Sacc[s][cb][r] = x;
        sm.St[j * LDK + i] = Op::cvt(x);
      }
  __syncthreads();

  for (int64_t c0 = 0; c0 < len; c0 += 64) {
    const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
    const int64_t row0 = bos + c0;

    // ---- load the chunk; gamma by a wave-wide scan ----
    if (wave == 0) {
      const float gv = lane < nv ? p.g[(row0 + lane) * H + h] : 0.f;
      const float gm = wave_inclusive_scan(gv, lane);
      const float gl = __shfl(gm, 63, 64);
      sm.gam[lane] = gm;
      sm.Gam[lane] = expf(gm);
      sm.dec[lane] = expf(gl - gm);
    } else if (wave == 1) {
      sm.bet[lane] = lane < nv ? p.beta[(row0 + lane) * H + h] : 0.f;
    }
    load_rows<DK, Op>(sm.Ks, LDK, k, row0, nv, H, h, tid);
    load_rows<DK, Op>(sm.Qs, LDK, q, row0, nv, H, h, tid);
    for (int x = tid; x < 64 * DT; x += 256) {
      const int t = x / DT, j = x % DT;
      sm.Vs[x] = t < nv ? Op::widen(v[((row0 + t) * H + h) * Dv + j0 + j]) : 0.f;
    }
    __syncthreads();

    // ---- decayed keys (transposed), A and P ----
    for (int x = tid; x < DK * 64; x += 256) {
      const int i = x >> 6, t = x & 63;
      sm.KtT[i * LDC + t] = Op::cvt(Op::widen(sm.Ks[t * LDK + i]) * sm.dec[t]);
    }
    for (int blk = wave; blk < 20; blk += 4) {
      const bool qk = blk >= 10;
      int bi, bj;
      lower_block(qk ? blk - 10 : blk, bi, bj);
      f32x4_t acc = zero4();
      tile_mma<Op, DK>(acc, (qk ? sm.Qs : sm.Ks) + 16 * bi * LDK, LDK, sm.Ks + 16 * bj * LDK, LDK,
                       lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * bi + 4 * (lane >> 4) + r, j = 16 * bj + (lane & 15);
        const float d = expf(fminf(sm.gam[i] - sm.gam[j], 0.f));
        if (qk)
          sm.Pm[i * LDC + j] = Op::cvt(i >= j ? acc[r] * d : 0.f);
        else
          sm.Af[i * LDF + j] = i > j ? sm.bet[i] * acc[r] * d : 0.f;
      }
    }
    __syncthreads();

    // ---- T = (I + A)^-1 ----
    if (lane < 16) {  // wave w inverts diagonal block w; lane = column
      const int w = wave, c = lane;
      float tcol[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s += sm.Af[(16 * w + r) * LDF + 16 * w + m] * tcol[m];
        tcol[r] = r == c ? 1.f : (r < c ? 0.f : -s);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tf[(16 * w + r) * LDF + 16 * w + c] = tcol[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {  // block diagonals below the main one
      const bool act = wave < 4 - d;
      const int bj = wave, bi = wave + d;
      float* Mt = sm.Mt + wave * 16 * LDM;
      if (act) {
        f32x4_t m = zero4();
        for (int kb = bj; kb < bi; ++kb)
          tile_mma_f32_rowmajor<16>(m, sm.Af + 16 * bi * LDF + 16 * kb, LDF,
                                    sm.Tf + 16 * kb * LDF + 16 * bj, LDF, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) Mt[(4 * (lane >> 4) + r) * LDM + (lane & 15)] = m[r];
      }
      __syncthreads();
      if (act) {
        f32x4_t x = zero4();
        tile_mma_f32_rowmajor<16>(x, sm.Tf + 16 * bi * LDF + 16 * bi, LDF, Mt, LDM, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.Tf[(16 * bi + 4 * (lane >> 4) + r) * LDF + 16 * bj + (lane & 15)] = -x[r];
      }
      __syncthreads();
    }
    for (int x = tid; x < 64 * 64; x += 256) {
      const int i = x >> 6, j = x & 63;
      if ((j >> 4) <= (i >> 4)) sm.Tm[i * LDC + j] = Op::cvt(sm.Tf[i * LDF + j]);
    }
    __syncthreads();

    // ---- the state chain: R, E, O, S ----
    f32x4_t Y[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4_t xk = zero4(), yq = zero4();
      tile_mma<Op, DK>(xk, sm.Ks + 16 * wave * LDK, LDK, sm.St + 16 * cb * LDK, LDK, lane);
      tile_mma<Op, DK>(yq, sm.Qs + 16 * wave * LDK, LDK, sm.St + 16 * cb * LDK, LDK, lane);
      Y[cb] = yq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
        sm.Rt[j * LDC + t] = Op::cvt(sm.bet[t] * (sm.Vs[t * DT + j] - sm.Gam[t] * xk[r]));
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4_t e = zero4();
      tile_mma<Op, 64>(e, sm.Tm + 16 * wave * LDC, LDC, sm.Rt + 16 * cb * LDC, LDC, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
        sm.Et[j * LDC + t] = Op::cvt(e[r]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4_t pe = zero4();
      tile_mma<Op, 64>(pe, sm.Pm + 16 * wave * LDC, LDC, sm.Et + 16 * cb * LDC, LDC, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
        if (t < nv)
          o[((row0 + t) * H + h) * Dv + j0 + j] =
              Op::cvt(p.scale * (sm.Gam[t] * Y[cb][r] + pe[r]));
      }
    }
    const float gl = sm.Gam[63];
#pragma unroll
    for (int s = 0; s < SRB; ++s)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int sb = wave * SRB + s;
        f32x4_t acc = Sacc[s][cb] * gl;
        tile_mma<Op, 64>(acc, sm.KtT + 16 * sb * LDC, LDC, sm.Et + 16 * cb * LDC, LDC, lane);
        Sacc[s][cb] = acc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * sb + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
          sm.St[j * LDK + i] = Op::cvt(acc[r]);
        }
      }
    __syncthreads();
  }

  if (p.S_final) {
#pragma unroll
    for (int s = 0; s < SRB; ++s)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * (wave * SRB + s) + 4 * (lane >> 4) + r, j = 16 * cb + (lane & 15);
          p.S_final[((static_cast<int64_t>(n) * H + h) * DK + i) * Dv + j0 + j] = Sacc[s][cb][r];
        }
  }
}

template <int DK, int DT, typename Op>
hipError_t launch_fwd_t(const FwdParams& p, int N, hipStream_t s) {
  constexpr size_t smem = sizeof(FwdSmem<DK, DT, Op>);
  static_assert(smem <= 160 * 1024, "LDS budget of one gfx950 CU exceeded");
  auto kern = chunk_fwd_kernel<DK, DT, Op>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(smem));
  if (e != hipSuccess) return e;
  dim3 grid(p.Dv / DT, p.H, N);
  hipLaunchKernelGGL(kern, grid, dim3(256), smem, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd(const FwdParams& p, int N, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_fwd_t<64, 16, OpBf16>(p, N, s);
    if (Dk == 128) return launch_fwd_t<128, 16, OpBf16>(p, N, s);
  } else {
    if (Dk == 64) return launch_fwd_t<64, 16, OpF32>(p, N, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
