// Chunked forward pass of the gated delta rule on gfx950: two kernels.
//
// Chunk algebra (chunks of 64 tokens; n <= 64 valid rows, padded rows carry
// k = q = v = 0, g = 0, beta = 0 and change nothing).  With S the state before
// the chunk (d_k x d_v), the update of "Research Sprint Day 1", section "The GDN
// update", applied to every token of the chunk gives
//   gamma = cumsum(g), Gamma = exp(gamma), D_ij = exp(gamma_i - gamma_j)  (j <= i)
//       [cumsum of g instead of a product of alpha: "Research Sprint Day 2",
//        "Building some intuition", gates step 5]
//   A = strict_lower(diag(beta) (K K^T) o D),  T = (I + A)^-1   [triangular inverse]
//   E = U - W S with the WY tensors U = T diag(beta) V, W = T diag(beta Gamma) K
//     = (T diag(beta)) (V - diag(Gamma) K S)      (the chunk's errors e_t)
//   P = lower_incl((Q K^T) o D)                                 [causal QK score]
//   O = scale (diag(Gamma) Q S + P E)
//   S <- Gamma_n S + K^T diag(exp(gamma_n - gamma)) E
// (intermediates named as on the fla issue #1550 page, "Intermediate rounding
// diagnosis").  Only exponents <= 0 are formed, so decays underflow to zero
// harmlessly and nothing is divided by a decay.
//
// Kernel 1, chunk_prep_kernel: one workgroup per (chunk, head, sequence), fully
//   parallel.  gamma and the decays, A and P with MFMA, T = (I + A)^-1 in fp32
//   (16x16 diagonal blocks by forward substitution, the blocks below by
//   T_ij = -T_ii sum_k A_ik T_kj with fp32 MFMA); stores T diag(beta) (lower
//   blocks only), P (in MFMA operand order), the decays, and for the backward T.
// Kernel 2, chunk_state_kernel: one workgroup per (segment, sequence, head,
//   16-column tile of d_v); column j of S only mixes with column j of v, so
//   tiles are independent.  Eight waves in two roles:
//     state waves (0-3) hold the d_k x 16 fp32 slice of S in MFMA accumulators
//       and run chunk c: R = V - diag(Gamma) K S, E = (T diag(beta)) R, the
//       state update; they touch only LDS;
//     output waves (4-7) load chunk c + 2 along whole rows, stage chunk c + 1
//       into LDS and form the output of chunk c.
//   Three workgroup barriers per chunk.  The tiles of one head share an XCD (and
//   its L2), so each input byte comes from HBM once per head.
//
// Precision: bf16 io feeds bf16 MFMA operands (v_mfma_f32_16x16x32_bf16) with
// fp32 accumulation; S, gamma, the decays, A and the inverse are fp32; T
// diag(beta), P, R, E and the state operand are rounded to bf16 only as MFMA
// inputs.  fp32 io runs every product on v_mfma_f32_16x16x4_f32 (IEEE fp32).
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buffer_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// An offset that every buffer range check rejects: the load returns zeros and
// moves no data.
constexpr int kNoLoad = 0x7ffffff0;

// One io element at byte offset `off`, widened to fp32 (bf16 widens exactly).
template <typename IO>
__device__ __forceinline__ float io_load1(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (sizeof(IO) == 2)
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0)) << 16);
  else
    return buffer_load1(r, off);
}
// 16 bytes of io elements into `dst` of compute element type E: a plain copy when
// the types agree, else 8 bf16 widened to 8 fp32 (two 16-byte stores).
template <typename E, typename IO>
__device__ __forceinline__ void io_stage16(E* dst, const u32x4_t& x) {
  if constexpr (sizeof(E) == sizeof(IO)) {
    *reinterpret_cast<u32x4_t*>(dst) = x;
  } else {
    static_assert(sizeof(E) == 4 && sizeof(IO) == 2, "bf16 io widened to fp32");
    const u32x4_t lo = {x[0] << 16, x[0] & 0xffff0000u, x[1] << 16, x[1] & 0xffff0000u};
    const u32x4_t hi = {x[2] << 16, x[2] & 0xffff0000u, x[3] << 16, x[3] & 0xffff0000u};
    *reinterpret_cast<u32x4_t*>(dst) = lo;
    *reinterpret_cast<u32x4_t*>(dst + 4) = hi;
  }
}

// Row block, row and column of element e of a packed lower-block matrix.
__device__ __forceinline__ void lpack_pos(int e, int& i, int& j) {
  const int rb = e < lpack_base(1) ? 0 : e < lpack_base(2) ? 1 : e < lpack_base(3) ? 2 : 3;
  const int w = 16 * (rb + 1), rel = e - lpack_base(rb);
  i = 16 * rb + rel / w;
  j = rel % w;
}

// ===================================================================================
// Kernel 1: per-chunk T = (I + A)^-1, T diag(beta), P and the decays
// ===================================================================================
template <int DK, typename Op>
struct PrepSmem {
  using E = typename Op::elem;
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;
  static constexpr int LDF = 64 + 4;
  static constexpr int LDM = 20;
  static constexpr size_t kBytes = 64 * LDK * sizeof(E);                      // K rows
  static constexpr size_t tBytes = (64 * LDF + 4 * 16 * LDM) * sizeof(float);  // T, block temps
  static constexpr size_t uBytes = kBytes > tBytes ? kBytes : tBytes;
  alignas(16) char U[uBytes];  // K rows, then (once A and P are formed) T and the block temps
  float Af[64 * LDF];
  float gam[64], bet[64];
};

// IO: element type of q and k in memory (the compute type, or bf16 widened to
// fp32 for fp32 products on bf16 inputs).
template <int DK, typename Op, typename IO>
__global__ __launch_bounds__(256) void chunk_prep_kernel(FwdParams p) {
  using E = typename Op::elem;
  using F = typename Op::frag_t;
  using SM = PrepSmem<DK, Op>;
  constexpr int LDK = SM::LDK, LDF = SM::LDF, LDM = SM::LDM, KS = Op::KSTEP;
  constexpr int EPV = 16 / sizeof(E);
  constexpr int NKK = DK / KS;
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  E* const Ks = reinterpret_cast<E*>(sm.U);
  float* const Tf = reinterpret_cast<float*>(sm.U);
  float* const Mts = Tf + 64 * LDF;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, H = p.H;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t c0 = static_cast<int64_t>(c) * 64;
  if (c0 >= len) return;  // uniform over the workgroup
  const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
  const int64_t row0 = bos + c0;
  const int64_t slot = bos / 64 + n + c;
  const IO* __restrict__ k = static_cast<const IO*>(p.k);
  const IO* __restrict__ q = static_cast<const IO*>(p.q);
  const bool want_p = p.pws != nullptr || p.prws != nullptr;
  // Each wave forms the A blocks of row block `wave` and the P blocks of row block
  // 3 - wave: five 16x16 blocks per wave.
  const int ai = wave, pi = 3 - wave;

  // Every load is issued up front, through buffer resources bounded to the
  // chunk's valid rows (padded rows read as zeros): Q rows of row block pi as
  // MFMA fragments, K rows, g and beta.  No load sits inside a branch and every
  // loaded value is used by every wave: a load in a branch, or one sunk into
  // the only branch that uses it, is waited for where that branch ends.
  const int s_e = static_cast<int>(sizeof(IO));
  const int rows_bytes = ((nv - 1) * H * DK + DK) * s_e;
  F qf[NKK];
  {
    // without P the resource covers no bytes: the loads return zeros and read nothing
    const auto rq = buffer_rsrc(q + (row0 * H + h) * DK, want_p ? rows_bytes : 0);
    const int t = 16 * pi + (lane & 15);
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) {
      const int off = (t * H * DK + ks * KS + (lane >> 4) * Op::KPL) * s_e;
      if constexpr (sizeof(E) == 2)
        qf[ks] = __builtin_bit_cast(F, buffer_load16(rq, off));
      else
        qf[ks] = io_load1<IO>(rq, off);
    }
  }
  constexpr int EPVI = 16 / static_cast<int>(sizeof(IO));  // io elements per 16-byte vector
  constexpr int VPR = DK / EPVI;
  constexpr int NKV = 64 * VPR / 256;
  const auto rk = buffer_rsrc(k + (row0 * H + h) * DK, rows_bytes);
  u32x4_t kv[NKV];
#pragma unroll
  for (int x = 0; x < NKV; ++x) {
    const int vi = x * 256 + tid, t = vi / VPR, cc = vi % VPR;
    kv[x] = buffer_load16(rk, (t * H * DK + cc * EPVI) * s_e);
  }
  const auto rg = buffer_rsrc(p.g + row0 * H + h, ((nv - 1) * H + 1) * 4);
  const auto rb = buffer_rsrc(p.beta + row0 * H + h, ((nv - 1) * H + 1) * 4);
  const float gv = buffer_load1(rg, lane * H * 4) * kLog2e;
  const float bv = buffer_load1(rb, lane * H * 4);
#pragma unroll
  for (int x = 0; x < NKV; ++x) {
    const int vi = x * 256 + tid, t = vi / VPR, cc = vi % VPR;
    io_stage16<E, IO>(Ks + t * LDK + cc * EPVI, kv[x]);
  }
  {
    // every wave scans g and writes beta (identical values); wave 0 also stores the decays
    const float g2 = wave_inclusive_scan(gv, lane);  // gamma * log2(e)
    sm.gam[lane] = g2;
    sm.bet[lane] = bv;
    if (wave == 0 && p.gws) {  // Gamma and the decays to the chunk end, for the state pass
      const float gl2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), 63));
      float* gr = p.gws + (slot * H + h) * 128;
      gr[lane] = exp2f(g2);
      gr[64 + lane] = exp2f(gl2 - g2);
    }
  }
  __syncthreads();

  // A = strict_lower(diag(beta) (K K^T) o D) (fp32, row block ai), and
  // P = lower_incl((Q K^T) o D) (row block pi), formed as P^T blocks and stored
  // straight to the workspace in MFMA operand order: fragment (pi, ks) holds, in
  // lane 16 g + t, the KPL entries P[16 pi + t][ks KSTEP + g KPL ..], so that a
  // plain load of 64 consecutive lanes yields the operand (the blocks above the
  // diagonal as zeros); for the backward, row-major instead.
  {
    // K fragments of row block ai (the A operand of the A blocks), and the gates
    // each lane needs, read once
    const int lr = lane & 15, lg = lane >> 4;
    F ka[NKK];
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) ka[ks] = Op::frag(Ks + 16 * ai * LDK, LDK, lane, ks * KS);
    const float4 gA = *reinterpret_cast<const float4*>(sm.gam + 16 * ai + 4 * lg);  // rows i of A
    const float4 bA = *reinterpret_cast<const float4*>(sm.bet + 16 * ai + 4 * lg);
    const float gAr[4] = {gA.x, gA.y, gA.z, gA.w}, bAr[4] = {bA.x, bA.y, bA.z, bA.w};
    const float gP = sm.gam[16 * pi + lr];  // row i of P
    constexpr int NTS = 64 / KS, KPL = Op::KPL;
    E* P = p.pws ? static_cast<E*>(p.pws) + (slot * H + h) * 4096 + pi * NTS * 64 * KPL : nullptr;
    E* Prow = p.prws ? static_cast<E*>(p.prws) + (slot * H + h) * 4096 : nullptr;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
      if (!want_p && bj > ai) continue;
      F kb[NKK];  // K fragments of row block bj: B operand of A block (ai, bj), A operand of P^T block (bj, pi)
      if (bj <= ai || bj <= pi) {
#pragma unroll
        for (int ks = 0; ks < NKK; ++ks) kb[ks] = Op::frag(Ks + 16 * bj * LDK, LDK, lane, ks * KS);
      }
      if (bj <= ai) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKK; ++ks) acc = Op::mma(ka[ks], kb[ks], acc);
        const int j = 16 * bj + lr;
        const float gj = sm.gam[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * ai + 4 * lg + r;
          const float x = bAr[r] * acc[r] * __builtin_amdgcn_exp2f(fminf(gAr[r] - gj, 0.f));
          sm.Af[i * LDF + j] = i > j ? x : 0.f;
        }
      }
      if (want_p) {
        // block (pi, bj) of P, as P^T: C[j][i] = K_j . Q_i; stored in operand
        // order (the blocks above the diagonal as zeros)
        f32x4_t acc = zero4();
        if (bj <= pi) {
#pragma unroll
          for (int ks = 0; ks < NKK; ++ks) acc = Op::mma(kb[ks], qf[ks], acc);
        }
        const int i = 16 * pi + lr, jb = 16 * bj + 4 * lg;
        const float4 gj = *reinterpret_cast<const float4*>(sm.gam + jb);
        const float gjr[4] = {gj.x, gj.y, gj.z, gj.w};
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[r] * __builtin_amdgcn_exp2f(fminf(gP - gjr[r], 0.f));
          pv[r] = jb + r <= i ? x : 0.f;
        }
        // row-major for the backward (every block, zeros above the diagonal)
        if (Prow) store4<E>(Prow + i * 64 + jb, pv[0], pv[1], pv[2], pv[3]);
        // (fragments entirely above the diagonal are never read and not stored)
        if (P && (jb / KS) * KS < 16 * (pi + 1)) {
          if constexpr (KPL == 8) {  // the four columns are consecutive entries of one lane
            store4<E>(P + ((jb / KS) * 64 + 16 * ((jb % KS) / KPL) + lr) * KPL + jb % KPL, pv[0], pv[1], pv[2], pv[3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) P[((jb + r) / KS) * 64 + 16 * ((jb + r) % KS) + lr] = Op::cvt(pv[r]);
          }
        }
      }
    }
  }
  __syncthreads();  // A complete; K rows no longer needed (their space becomes T)

  // T = (I + A)^-1: diagonal blocks by forward substitution (wave w, lane = column)
  if (lane < 16) {
    const int w = wave, cc = lane;
    float tcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s += sm.Af[(16 * w + r) * LDF + 16 * w + m] * tcol[m];
      tcol[r] = r == cc ? 1.f : (r < cc ? 0.f : -s);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tf[(16 * w + r) * LDF + 16 * w + cc] = tcol[r];
  }
  __syncthreads();
  // then the block diagonals below: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  for (int d = 1; d < 4; ++d) {
    const bool act = wave < 4 - d;
    const int bj = wave, bi = wave + d;
    float* Mt = Mts + wave * 16 * LDM;
    if (act) {
      f32x4_t m = zero4();
      for (int kb = bj; kb < bi; ++kb)
        tile_mma_f32_rowmajor<16>(m, sm.Af + 16 * bi * LDF + 16 * kb, LDF, Tf + 16 * kb * LDF + 16 * bj, LDF, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Mt[(4 * (lane >> 4) + r) * LDM + (lane & 15)] = m[r];
    }
    __syncthreads();
    if (act) {
      f32x4_t x = zero4();
      tile_mma_f32_rowmajor<16>(x, Tf + 16 * bi * LDF + 16 * bi, LDF, Mt, LDM, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Tf[(16 * bi + 4 * (lane >> 4) + r) * LDF + 16 * bj + (lane & 15)] = -x[r];
    }
    __syncthreads();
  }

  // T diag(beta), packed (the entries above the diagonal inside the diagonal
  // blocks are exact zeros), and T row-major for the backward
  const int64_t sh = slot * H + h;
  if (p.tbws) {
    E* dst = static_cast<E*>(p.tbws) + sh * kTbSlot;
    if constexpr (sizeof(E) == 2) {
      // bf16: six operand fragments (row block mb, reduction step s <= mb / 2); lane
      // (m, g) holds row 32 (mb / 2) + 8 (m / 4) + 4 (mb % 2) + m % 4 (the row order of
      // the state pass's accumulators), columns 32 s + 8 g + 0..7
      for (int x = tid; x < 6 * 64; x += 256) {
        const int f = x >> 6, ln = x & 63, m = ln & 15, g = ln >> 4;
        const int mb = f < 2 ? f : 2 + (f - 2) / 2, s = f < 2 ? 0 : (f - 2) % 2;
        const int i = 32 * (mb >> 1) + 8 * (m >> 2) + 4 * (mb & 1) + (m & 3), jb = 32 * s + 8 * g;
        E vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = jb + e;
          vals[e] = Op::cvt((j >> 4) <= (i >> 4) ? Tf[i * LDF + j] * sm.bet[j] : 0.f);
        }
        *reinterpret_cast<uint4*>(dst + x * 8) = *reinterpret_cast<const uint4*>(vals);
      }
    } else {
      for (int x = tid; x < kLPack / EPV; x += 256) {
        int i, jb;
        lpack_pos(x * EPV, i, jb);
        E vals[EPV];
#pragma unroll
        for (int m = 0; m < EPV; ++m) vals[m] = Op::cvt(Tf[i * LDF + jb + m] * sm.bet[jb + m]);
        *reinterpret_cast<uint4*>(dst + x * EPV) = *reinterpret_cast<const uint4*>(vals);
      }
    }
  }
  if (p.tws) {
    E* dst = static_cast<E*>(p.tws) + sh * 4096;
    constexpr int VPT = 64 / EPV;
    for (int x = tid; x < 64 * VPT; x += 256) {
      const int i = x / VPT, jb = (x % VPT) * EPV;
      E vals[EPV];
#pragma unroll
      for (int m = 0; m < EPV; ++m) {
        const int j = jb + m;
        vals[m] = Op::cvt((j >> 4) <= (i >> 4) ? Tf[i * LDF + j] : 0.f);
      }
      *reinterpret_cast<uint4*>(dst + i * 64 + jb) = *reinterpret_cast<const uint4*>(vals);
    }
  }
}

// ===================================================================================
// Kernel 2: the state pass with output
// ===================================================================================
// LDS of one workgroup: the per-chunk operands of the state waves in two ring
// slots (the chunk in use and the next one, being staged) and the hand-off
// buffers between the roles.
template <int DK, typename Op>
struct StateSmem {
  using E = typename Op::elem;
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;  // rows of length d_k
  static constexpr int LDC = 64 + PADE;  // rows of length 64 (one chunk)
  static constexpr int LDR = 16 + PADE;  // rows of length 16 (one tile)
  alignas(16) E Ks[2][64 * LDK];   // K rows (rows of padded tokens are zero)
  alignas(16) E Tb[2][64 * LDC];   // T diag(beta); the blocks above the diagonal stay zero
  alignas(16) E Vs[2][64 * 16];    // the v tile
  alignas(16) float Gs[2][128];    // Gamma and exp(gamma_n - gamma)
  alignas(16) E Sb[16 * LDK];      // S^T of this tile as an MFMA operand, [j][d_k]
  alignas(16) E Rr[64 * LDR];      // R = V - diag(Gamma) K S, [t][j]
  alignas(16) E Et[16 * LDC];      // E^T
  alignas(16) E Ett[16 * LDC];     // (diag(exp(gamma_n - gamma)) E)^T
  alignas(16) float Ys[64 * 20];   // Y = Q S (fp32), [t][j]
};

// Four consecutive io values, widened when used.
template <typename E>
struct Raw4;
template <>
struct Raw4<uint16_t> {
  uint2 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float operator[](int r) const {
    const uint32_t w = r < 2 ? u.x : u.y;
    return __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct Raw4<float> {
  float4 u;
  __device__ __forceinline__ void load(const float* p) { u = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float operator[](int r) const {
    return r == 0 ? u.x : r == 1 ? u.y : r == 2 ? u.z : u.w;
  }
};

// STATES: also store S_c before every chunk (the backward's forward half).
// OUT: compute and store the output (stores are further masked per segment).
template <int DK, typename Op, typename IO, bool STATES, bool OUT>
__global__ __launch_bounds__(512) void chunk_state_kernel(FwdParams p) {
  using E = typename Op::elem;
  using F = typename Op::frag_t;
  using SM = StateSmem<DK, Op>;
  constexpr int LDK = SM::LDK, LDC = SM::LDC, LDR = SM::LDR;
  constexpr int KS = Op::KSTEP;
  constexpr int NKK = DK / KS;  // k-steps over d_k
  constexpr int NTS = 64 / KS;  // k-steps over one chunk
  constexpr int DPW = DK / 64;  // 16-row blocks of S per state wave
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const IO* __restrict__ q = static_cast<const IO*>(p.q);
  const IO* __restrict__ k = static_cast<const IO*>(p.k);
  const IO* __restrict__ v = static_cast<const IO*>(p.v);
  const E* __restrict__ tbw = static_cast<const E*>(p.tbws);
  const E* __restrict__ pw = static_cast<const E*>(p.pws);
  const float* __restrict__ gw = p.gws;
  IO* __restrict__ o = static_cast<IO*>(p.o);
  constexpr int SIO = static_cast<int>(sizeof(IO));

  const int H = p.H, Dv = p.Dv, NC = p.ncol, NT = NC / 16;
  // XCD-aware block order: consecutive virtual blocks (the tiles of one head)
  // land on the same XCD, which the hardware picks as blockIdx % 8.
  const int NB = gridDim.x, L = blockIdx.x;
  const int vb = (NB % 8 == 0) ? (L % 8) * (NB / 8) + L / 8 : L;
  const int tile = vb % NT, nh = (vb / NT) % (p.N * H), h = nh % H, n = nh / H;
  const int seg = p.seg_base + vb / NT / (p.N * H);
  const int j0 = tile * 16;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  // this block's chunks: segment `seg` of the sequence (all of it when G == 1)
  const int nch_all = static_cast<int>((len + 63) / 64);
  const int seg_len = (nch_all + p.G - 1) / p.G;
  const int cb = min(seg * seg_len, nch_all);
  const int nch = min(cb + seg_len, nch_all) - cb;
  const int64_t slot0 = bos / 64 + n + cb;
  const bool store_o = p.write_o == kOutAll || (p.write_o == kOutSeg0 && seg == 0);
  const bool use_v = !p.zero_u;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int wr = w & 3, lr = lane & 15, lg = lane >> 4;
  const int tc = 16 * wr + lr;  // this lane's token row / column
  const bool state_wave = w < 4;
  const int64_t nhS = (static_cast<int64_t>(n) * H + h) * DK;
  const int64_t segS = (static_cast<int64_t>(seg) * p.N * H + nh) * DK;  // [G][N][H][DK][NC] buffers

  auto chunk_rows = [&](int c) {  // valid rows of chunk c
    const int64_t c0 = static_cast<int64_t>(cb + c) * 64;
    return static_cast<int>(len - c0 < 64 ? len - c0 : 64);
  };
  auto clampc = [&](int c) { return c < nch ? c : nch - 1; };

  f32x4_t Sacc[DPW];
  if (state_wave) {
#pragma unroll
    for (int x = 0; x < DPW; ++x) {
      const int i = 16 * (wr * DPW + x) + 4 * lg;
      float s4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (p.start_mode == kStartCarry)
          s4[r] = p.carry[(segS + i + r) * NC + j0 + lr];
        else if (p.start_mode == kStartIdentity)
          s4[r] = i + r == j0 + lr ? 1.f : 0.f;
        else if (p.start_mode == kStartS0 && seg == 0 && p.S0)
          s4[r] = p.S0[(nhS + i + r) * Dv + j0 + lr];
        else
          s4[r] = 0.f;
      }
      Sacc[x] = f32x4_t{s4[0], s4[1], s4[2], s4[3]};
      store4<E>(sm.Sb + lr * LDK + i, s4[0], s4[1], s4[2], s4[3]);
    }
  }
  auto write_state = [&](void) {
    const bool to_final = p.final_to_sfinal && seg == p.G - 1;
    if (to_final ? p.S_final != nullptr : p.seg_out != nullptr) {
#pragma unroll
      for (int x = 0; x < DPW; ++x) {
        const int i = 16 * (wr * DPW + x) + 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (to_final)
            p.S_final[(nhS + i + r) * Dv + j0 + lr] = Sacc[x][r];
          else
            p.seg_out[(segS + i + r) * NC + j0 + lr] = Sacc[x][r];
        }
      }
    }
  };
  if (nch == 0) {  // empty segment (uniform over the workgroup): the state passes through
    if (state_wave) write_state();
    return;
  }
  // The chunk loop is unrolled by two (the ring slots) and has no tail branch:
  // steps past the last chunk run on clamped data and change nothing.
  // Straight-line bodies let the compiler wait for exactly the loads each step
  // consumes.
  const int nsteps = (nch + 1) / 2 * 2;

  // Q and P rows tc of a chunk straight into MFMA operand fragments: Q from the
  // chunk's rows, P in the operand order the prep kernel stores (fragment ks only
  // where it meets the blocks on or below the diagonal).  Padded rows read as zeros.
  auto frag_load = [](__amdgpu_buffer_rsrc_t r, int off) -> F {
    if constexpr (sizeof(E) == 2)
      return __builtin_bit_cast(F, buffer_load16(r, off));
    else
      return buffer_load1(r, off);
  };
  auto load_q = [&](F (&f)[NKK], int c) {
    const int nv = chunk_rows(c);
    const int64_t row0 = bos + static_cast<int64_t>(cb + c) * 64;
    const auto rq = buffer_rsrc(q + (row0 * H + h) * DK, ((nv - 1) * H * DK + DK) * SIO);
#pragma unroll
    for (int ks = 0; ks < NKK; ++ks) {
      const int off = (tc * H * DK + ks * KS + lg * Op::KPL) * SIO;
      if constexpr (sizeof(E) == 2)
        f[ks] = __builtin_bit_cast(F, buffer_load16(rq, off));
      else
        f[ks] = io_load1<IO>(rq, off);
    }
  };
  auto load_p = [&](F (&f)[NTS], int c) {
    const auto rp = buffer_rsrc(pw + ((slot0 + c) * H + h) * 4096, 4096 * static_cast<int>(sizeof(E)));
#pragma unroll
    for (int ks = 0; ks < NTS; ++ks)
      f[ks] = frag_load(rp, ks * KS < 16 * (wr + 1) ? ((wr * NTS + ks) * 64 + lane) * Op::KPL * static_cast<int>(sizeof(E))
                                                    : kNoLoad);
  };

  if (state_wave) {
    // ============ state waves: the recurrence and the output of their 16 tokens ============
    // In step c: phase 1 forms Z^T = S^T K^T and Y^T = S^T Q^T from the same S^T
    // fragments (Y goes to the loader waves, which form the output), then R;
    // phase 2 E = (T diag(beta)) R; phase 3 the state update, and loads Q of
    // chunk c + 2 (phase 3 is the one with the least memory traffic).  Only the
    // Q loads touch memory.
    F qf[2][NKK];
    if (OUT) {
      load_q(qf[0], 0);
      load_q(qf[1], clampc(1));
    }
    __syncthreads();  // chunk 0 staged
    int c0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = c0 + u;
        const bool active = c < nch;
        const E* Ks = sm.Ks[u];
        const float* Gs = sm.Gs[u];
        // phase 1
        if (STATES) {  // S_c, the state before chunk c, kept for the backward
          const auto rs = buffer_rsrc(static_cast<float*>(p.states) +
                                          ((slot0 + clampc(c)) * H + h) * static_cast<int64_t>(DK) * Dv,
                                      active ? DK * Dv * 4 : 0);
#pragma unroll
          for (int x = 0; x < DPW; ++x) {
            const int i = 16 * (wr * DPW + x) + 4 * lg;
#pragma unroll
            for (int r = 0; r < 4; ++r) buffer_store1(rs, ((i + r) * Dv + j0 + lr) * 4, Sacc[x][r]);
          }
        }
        F sa[NKK];
#pragma unroll
        for (int ks = 0; ks < NKK; ++ks) sa[ks] = Op::frag(sm.Sb, LDK, lane, ks * KS);
        f32x4_t z = zero4(), yacc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKK; ++ks) {
          z = Op::mma(sa[ks], Op::frag(Ks + 16 * wr * LDK, LDK, lane, ks * KS), z);
          if (OUT) yacc = Op::mma(sa[ks], qf[u][ks], yacc);
        }
        if (OUT) *reinterpret_cast<f32x4_t*>(sm.Ys + tc * 20 + 4 * lg) = yacc;
        Raw4<E> vv;
        vv.load(sm.Vs[u] + tc * 16 + 4 * lg);
        const float gt = Gs[tc];
        const bool real = tc < chunk_rows(clampc(c));
        float rr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rr[r] = real ? (use_v ? vv[r] : 0.f) - gt * z[r] : 0.f;
        store4<E>(sm.Rr + tc * LDR + 4 * lg, rr[0], rr[1], rr[2], rr[3]);
        __syncthreads();
        // phase 2: E = (T diag(beta)) R
        f32x4_t e = zero4();
#pragma unroll
        for (int ks = 0; ks < NTS; ++ks)
          e = Op::mma(Op::frag(sm.Tb[u] + 16 * wr * LDC, LDC, lane, ks * KS), Op::frag_tr(sm.Rr, LDR, lane, ks * KS), e);
        const int t0 = 16 * wr + 4 * lg;
        const float4 dc = *reinterpret_cast<const float4*>(Gs + 64 + t0);
        store4<E>(sm.Et + lr * LDC + t0, e[0], e[1], e[2], e[3]);
        store4<E>(sm.Ett + lr * LDC + t0, e[0] * dc.x, e[1] * dc.y, e[2] * dc.z, e[3] * dc.w);
        __syncthreads();
        // phase 3: S <- Gamma_n S + K^T (decayed E)
        const float gn = Gs[63];
        F ef[NTS];
#pragma unroll
        for (int ks = 0; ks < NTS; ++ks) ef[ks] = Op::frag(sm.Ett, LDC, lane, ks * KS);
#pragma unroll
        for (int x = 0; x < DPW; ++x) {
          const int db = wr * DPW + x;
          f32x4_t acc = Sacc[x] * gn;
#pragma unroll
          for (int ks = 0; ks < NTS; ++ks) acc = Op::mma(Op::frag_tr(Ks + 16 * db, LDK, lane, ks * KS), ef[ks], acc);
          Sacc[x] = active ? acc : Sacc[x];
        }
#pragma unroll
        for (int x = 0; x < DPW; ++x)
          store4<E>(sm.Sb + lr * LDK + 16 * (wr * DPW + x) + 4 * lg, Sacc[x][0], Sacc[x][1], Sacc[x][2], Sacc[x][3]);
        if (OUT) load_q(qf[u], clampc(c + 2));
        __syncthreads();
      }
      c0 += 2;
    } while (c0 < nsteps);
    write_state();
  } else {
    // ============ loader waves: the LDS ring, and the output ============
    // In step c (the state waves on chunk c): phase 1 stages K, v and the decays
    // of chunk c + 1 and refills the freed registers with K of chunk c + 3; phase
    // 2 stages T diag(beta) of chunk c + 1 and loads the rest of chunk c + 3;
    // phase 3 forms the output of chunk c (O^T = scale (Gamma o Y^T + E^T P^T), Y
    // from the state waves) and loads P of chunk c + 2 straight into the operand
    // fragments it has just used.  Every load thus has two steps to arrive, with
    // two register sets.  Loads run along
    // whole rows (consecutive lanes read consecutive 16-byte vectors), in groups
    // spread over the phases so that the texture-address unit (about one 1 KB
    // wave load per 16 cycles) works through them behind the compute; buffer
    // resources bound them to the chunk's valid rows (rows of padded tokens read
    // as zeros), and lanes past the end of a short array load nothing (kNoLoad)
    // and write nothing.
    const int ot = tid - 256;
    constexpr int EPV = 16 / static_cast<int>(sizeof(E));
    constexpr int EPVI = 16 / SIO;                    // io elements per 16-byte vector
    constexpr int KVR = DK / EPVI;                    // 16-byte vectors per K row (io)
    constexpr int NKV = 64 * KVR / 256;               // K vectors per loader thread
    constexpr int VVR = SIO;                          // 16-byte vectors per v-tile row (io)
    constexpr int TVN = kLPack / EPV;                 // vectors of a packed T diag(beta)
    constexpr int NTV = (TVN + 255) / 256;
    struct LoadSet {
      u32x4_t kv[NKV];  // K: vector x * 256 + ot is row (x * 256 + ot) / KVR
      u32x4_t tv[NTV];  // T diag(beta): packed vector x * 256 + ot (< TVN)
      u32x4_t vv;       // the v tile: vector ot (< 64 VVR)
      u32x4_t gv;       // decays: floats 4 ot .. 4 ot + 3 (ot < 32)
    };
    LoadSet ls[2];
    auto load_k = [&](LoadSet& s, int c) {
      const int nv = chunk_rows(c);
      const int64_t row0 = bos + static_cast<int64_t>(cb + c) * 64;
      const auto rk = buffer_rsrc(k + (row0 * H + h) * DK, ((nv - 1) * H * DK + DK) * SIO);
#pragma unroll
      for (int x = 0; x < NKV; ++x) {
        const int vi = x * 256 + ot, t = vi / KVR, cv = (vi % KVR) * EPVI;
        s.kv[x] = buffer_load16(rk, (t * H * DK + cv) * SIO);
      }
    };
    auto load_rest = [&](LoadSet& s, int c) {  // T diag(beta), the v tile, the decays
      const int nv = chunk_rows(c);
      const int64_t row0 = bos + static_cast<int64_t>(cb + c) * 64;
      const int64_t sh = (slot0 + c) * H + h;
      const auto rt = buffer_rsrc(tbw + sh * kTbSlot, kLPack * static_cast<int>(sizeof(E)));
#pragma unroll
      for (int x = 0; x < NTV; ++x) s.tv[x] = buffer_load16(rt, (x * 256 + ot) * 16);
      // (a pass without V still loads, from columns clamped into the row, and discards them)
      const auto rv = buffer_rsrc(v + (row0 * H + h) * Dv, ((nv - 1) * H * Dv + Dv) * SIO);
      const int t = ot / VVR, cpos = (ot % VVR) * EPVI;
      s.vv = buffer_load16(rv, ot < 64 * VVR ? (t * H * Dv + min(j0 + cpos, Dv - EPVI)) * SIO : kNoLoad);
      s.gv = buffer_load16(buffer_rsrc(gw + sh * 128, 512), ot * 16);
    };
    auto stage_t = [&](const LoadSet& s, int sl) {
#pragma unroll
      for (int x = 0; x < NTV; ++x) {
        int i, jb;
        lpack_pos(min(x * 256 + ot, TVN - 1) * EPV, i, jb);
        if (x * 256 + ot < TVN) *reinterpret_cast<u32x4_t*>(sm.Tb[sl] + i * LDC + jb) = s.tv[x];
      }
    };
    auto stage_kvg = [&](const LoadSet& s, int sl) {
#pragma unroll
      for (int x = 0; x < NKV; ++x) {
        const int vi = x * 256 + ot, t = vi / KVR, cv = (vi % KVR) * EPVI;
        io_stage16<E, IO>(sm.Ks[sl] + t * LDK + cv, s.kv[x]);
      }
      if (ot < 64 * VVR) io_stage16<E, IO>(sm.Vs[sl] + (ot / VVR) * 16 + (ot % VVR) * EPVI, s.vv);
      if (ot < 32) *reinterpret_cast<u32x4_t*>(sm.Gs[sl] + 4 * ot) = s.gv;
    };

    // prologue: the blocks above the diagonal of both T diag(beta) slots are zero
    // for good; chunk 0 staged, chunk 1 loading
    {
      constexpr int VPT = 64 / EPV;
      const u32x4_t zv = {0u, 0u, 0u, 0u};
      for (int x = ot; x < 2 * 64 * VPT; x += 256) {
        const int sl = x / (64 * VPT), rem = x % (64 * VPT), i = rem / VPT, jv = (rem % VPT) * EPV;
        if ((jv >> 4) > (i >> 4)) *reinterpret_cast<u32x4_t*>(sm.Tb[sl] + i * LDC + jv) = zv;
      }
    }
    F pf[2][NTS];
    load_k(ls[0], 0);
    load_rest(ls[0], 0);
    load_k(ls[1], clampc(1));
    load_rest(ls[1], clampc(1));
    if (OUT) load_p(pf[0], 0);
    stage_t(ls[0], 0);
    stage_kvg(ls[0], 0);
    load_k(ls[0], clampc(2));
    load_rest(ls[0], clampc(2));
    if (OUT) load_p(pf[1], clampc(1));
    __syncthreads();
    int c0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = c0 + u;
        // phase 1
        stage_kvg(ls[u ^ 1], u ^ 1);
        load_k(ls[u ^ 1], clampc(c + 3));
        __syncthreads();
        // phase 2
        stage_t(ls[u ^ 1], u ^ 1);
        load_rest(ls[u ^ 1], clampc(c + 3));
        __syncthreads();
        // phase 3
        if (OUT) {  // O^T = scale (Gamma o Y^T + E^T P^T), columns j, token tc
          f32x4_t oacc = zero4();
#pragma unroll
          for (int ks = 0; ks < NTS; ++ks) oacc = Op::mma(Op::frag(sm.Et, LDC, lane, ks * KS), pf[u][ks], oacc);
          const f32x4_t yacc = *reinterpret_cast<const f32x4_t*>(sm.Ys + tc * 20 + 4 * lg);
          const float gt = sm.Gs[u][tc];
          // rows of padded tokens and steps past the last chunk fall outside the range
          const int cc = clampc(c), nv = chunk_rows(cc);
          const auto ro = buffer_rsrc(o + ((bos + static_cast<int64_t>(cb + cc) * 64) * H + h) * Dv + j0,
                                      store_o && c < nch ? ((nv - 1) * H * Dv + 16) * SIO : 0);
          buffer_store4<IO>(ro, (tc * H * Dv + 4 * lg) * SIO,
                           p.scale * (gt * yacc[0] + oacc[0]), p.scale * (gt * yacc[1] + oacc[1]),
                           p.scale * (gt * yacc[2] + oacc[2]), p.scale * (gt * yacc[3] + oacc[3]));
          load_p(pf[u], clampc(c + 2));
        }
        __syncthreads();
      }
      c0 += 2;
    } while (c0 < nsteps);
  }
}

// Segment carries (sequential in the segment index, parallel over sequences,
// heads and 16-column tiles): start(1) = end(0), and
// start(sigma + 1) = M_sigma start(sigma) + b_sigma for sigma = 1 .. G-2, in fp32,
// with a fixed summation order.  One block of 256 threads per 16-column tile.
template <int DK>
__global__ __launch_bounds__(256) void seg_carry_kernel(CarryParams c) {
  __shared__ float cur[DK][17];
  const int NT = c.Dv / 16;
  const int tile = blockIdx.x % NT, nh = blockIdx.x / NT;
  const int j0 = tile * 16, tid = threadIdx.x, jj = tid & 15, i0 = tid >> 4;
  const int64_t NHD = static_cast<int64_t>(c.N) * c.H * DK;
  auto at = [&](int sigma, int i) {  // element offset in a [G][N][H][DK][Dv] buffer
    return (sigma * NHD + static_cast<int64_t>(nh) * DK + i) * c.Dv + j0 + jj;
  };
  for (int i = i0; i < DK; i += 16) {
    const float x = c.ends[at(0, i)];
    cur[i][jj] = x;
    c.starts[at(1, i)] = x;
  }
  __syncthreads();
  for (int sg = 1; sg + 1 < c.G; ++sg) {
    float nxt[DK / 16];
    const float* M = c.maps + (sg * NHD + static_cast<int64_t>(nh) * DK) * DK;  // [G][N][H][DK][DK]
#pragma unroll
    for (int r = 0; r < DK / 16; ++r) {
      const int i = i0 + 16 * r;
      float acc = c.ends[at(sg, i)];
      for (int k = 0; k < DK; ++k) acc = fmaf(M[static_cast<int64_t>(i) * DK + k], cur[k][jj], acc);
      nxt[r] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < DK / 16; ++r) {
      const int i = i0 + 16 * r;
      cur[i][jj] = nxt[r];
      c.starts[at(sg + 1, i)] = nxt[r];
    }
    __syncthreads();
  }
}

template <typename K>
hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes));
}

template <int DK, typename Op, typename IO>
hipError_t launch_prep(const FwdParams& p, hipStream_t s) {
  constexpr size_t smem = sizeof(PrepSmem<DK, Op>);
  static_assert(smem <= 160 * 1024, "LDS budget exceeded");
  auto prep = chunk_prep_kernel<DK, Op, IO>;
  hipError_t e = allow_lds(prep, smem);
  if (e != hipSuccess || p.max_chunks == 0) return e;
  hipLaunchKernelGGL(prep, dim3(p.max_chunks, p.H, p.N), dim3(256), smem, s, p);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int cu_count() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    counts[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return counts[dev];
}

template <int DK, typename Op, typename IO, bool STATES, bool OUT>
hipError_t launch_state(const FwdParams& q, hipStream_t s) {
  if constexpr (std::is_same<Op, OpBf16>::value) {
    return launch_state_chain(q, DK, STATES, OUT, s);
  } else {
    constexpr size_t need = sizeof(StateSmem<DK, Op>);
    static_assert(need <= 160 * 1024, "LDS budget exceeded");
    // A grid with fewer than two workgroups per compute unit asks for more than
    // half of a CU's 160 KB of LDS, so that no CU holds two of them while another
    // stays idle; larger grids pack two per CU where they fit.
    const int blocks = q.nseg * q.N * q.H * (q.ncol / 16);
    const size_t smem = blocks < 2 * cu_count() && need < 82 * 1024 ? 82 * 1024 : need;
    auto state = chunk_state_kernel<DK, Op, IO, STATES, OUT>;
    hipError_t e = allow_lds(state, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(state, dim3(blocks), dim3(512), smem, s, q);
    return hipGetLastError();
  }
}

template <int DK, typename Op, typename IO>
hipError_t launch_states_t(const FwdParams& p, hipStream_t s) {
  hipError_t e = launch_prep<DK, Op, IO>(p, s);
  if (e != hipSuccess) return e;
  FwdParams q = p;
  q.G = 1; q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = kOutNone;
  q.zero_u = 0; q.ncol = p.Dv; q.carry = nullptr; q.seg_out = nullptr; q.final_to_sfinal = 0;
  q.S_final = nullptr;
  return launch_state<DK, Op, IO, true, false>(q, s);
}

// Forward that keeps what the backward needs: the preparation writes T, T
// diag(beta), the decays, P in operand order (for the output) and P row-major
// (for the backward); the state pass writes o, S_final and the state before every
// chunk.
template <int DK, typename Op, typename IO>
hipError_t launch_save_t(const FwdParams& p, hipStream_t s) {
  hipError_t e = launch_prep<DK, Op, IO>(p, s);
  if (e != hipSuccess) return e;
  FwdParams q = p;
  q.G = 1; q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = kOutAll;
  q.zero_u = 0; q.ncol = p.Dv; q.carry = nullptr; q.seg_out = nullptr; q.final_to_sfinal = 1;
  return launch_state<DK, Op, IO, true, true>(q, s);
}

template <int DK, typename Op, typename IO>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  hipError_t e = launch_prep<DK, Op, IO>(p, s);
  if (e != hipSuccess) return e;
  FwdParams q = p;
  q.ncol = p.Dv;
  q.zero_u = 0;
  q.carry = nullptr;
  if (p.G == 1) {
    q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = kOutAll;
    q.seg_out = nullptr; q.final_to_sfinal = 1;
    return launch_state<DK, Op, IO, false, true>(q, s);
  }
  // G segments per sequence: (1) segment 0 from S0 with its outputs, and the
  // segments 1 .. G-2 from zero (their offsets b); (2) the transition maps M of
  // segments 1 .. G-2 (the same pass with V = 0, started from the identity);
  // (3) the carries; (4) segments 1 .. G-1 again from their carried start states.
  const size_t ends_floats = static_cast<size_t>(p.G) * p.N * p.H * DK * p.Dv;
  float* ends = p.seg_ws;
  float* starts = ends + ends_floats;
  float* maps = starts + ends_floats;
  q.seg_base = 0; q.nseg = p.G - 1; q.start_mode = kStartS0; q.write_o = kOutSeg0;
  q.seg_out = ends; q.final_to_sfinal = 0;
  if ((e = launch_state<DK, Op, IO, false, true>(q, s)) != hipSuccess) return e;
  if (p.G > 2) {
    FwdParams m = q;
    m.ncol = DK; m.seg_base = 1; m.nseg = p.G - 2; m.start_mode = kStartIdentity;
    m.write_o = kOutNone; m.zero_u = 1; m.seg_out = maps;
    if ((e = launch_state<DK, Op, IO, false, false>(m, s)) != hipSuccess) return e;
  }
  CarryParams c{ends, maps, starts, p.G, p.N, p.H, DK, p.Dv};
  hipLaunchKernelGGL(seg_carry_kernel<DK>, dim3(p.N * p.H * (p.Dv / 16)), dim3(256), 0, s, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  q.seg_base = 1; q.nseg = p.G - 1; q.start_mode = kStartCarry; q.write_o = kOutAll;
  q.carry = starts; q.seg_out = nullptr; q.final_to_sfinal = 1;
  return launch_state<DK, Op, IO, false, true>(q, s);
}

}  // namespace

hipError_t launch_chunk_fwd_states(const FwdParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_states_t<64, OpBf16, uint16_t>(p, s);
    if (Dk == 128) return launch_states_t<128, OpBf16, uint16_t>(p, s);
  } else {
    if (Dk == 64) return launch_states_t<64, OpF32, float>(p, s);
    if (Dk == 128) return launch_states_t<128, OpF32, float>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd_save(const FwdParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_save_t<64, OpBf16, uint16_t>(p, s);
    if (Dk == 128) return launch_save_t<128, OpBf16, uint16_t>(p, s);
  } else {
    if (Dk == 64) return launch_save_t<64, OpF32, float>(p, s);
    if (Dk == 128) return launch_save_t<128, OpF32, float>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_segment_carry(const float* ends, const float* maps, float* starts, int G, int N, int H, int Dk,
                                int Dv, hipStream_t s) {
  CarryParams c{ends, maps, starts, G, N, H, Dk, Dv};
  if (Dk == 128)
    hipLaunchKernelGGL(seg_carry_kernel<128>, dim3(N * H * (Dv / 16)), dim3(256), 0, s, c);
  else if (Dk == 64)
    hipLaunchKernelGGL(seg_carry_kernel<64>, dim3(N * H * (Dv / 16)), dim3(256), 0, s, c);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const FwdParams& p, int Dk, bool bf16, bool fp32_products, hipStream_t s) {
  if (bf16 && !fp32_products) {
    if (Dk == 64) return launch_fwd_t<64, OpBf16, uint16_t>(p, s);
    if (Dk == 128) return launch_fwd_t<128, OpBf16, uint16_t>(p, s);
  } else if (bf16) {  // bf16 inputs and output, every product in IEEE fp32
    if (Dk == 64) return launch_fwd_t<64, OpF32, uint16_t>(p, s);
    if (Dk == 128) return launch_fwd_t<128, OpF32, uint16_t>(p, s);
  } else {
    if (Dk == 64) return launch_fwd_t<64, OpF32, float>(p, s);
    if (Dk == 128) return launch_fwd_t<128, OpF32, float>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
