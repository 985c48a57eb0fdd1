// Backward of the chunked gated delta rule with one decay per key channel (the
// KDA gate layout of the cuLA issue #126 page, "Minimal public reproduction").
//
// Forward per chunk of n <= 64 rows (gdn_kda.hip), gamma = cumsum(g) per channel,
// Gamma = exp(gamma), Kd = K o Gamma, Qd = Q o Gamma, Kb = K o exp(gamma_n - gamma),
// A = diag(beta) Ab with Ab_ij = sum_c k_ic k_jc exp(gamma_ic - gamma_jc) (j < i),
// T = (I + A)^-1, P_ij = sum_c q_ic k_jc exp(gamma_ic - gamma_jc) (j <= i):
//   R = V - Kd S,  E = T diag(beta) R,  O = scale (Qd S + P E),
//   S' = diag(Gamma_n) S + Kb^T E.
// Reverse mode, with dS' the gradient of the state after the chunk and
// dOs = scale dO:
//   dE = P^T dOs + Kb dS',  G = T^T dE,  F = diag(beta) G (= dV),
//   dS = diag(Gamma_n) dS' + Qd^T dOs - Kd^T F              (state-gradient pass)
//   dbeta = rowsum(G o R) + rowsum(dA o Ab),  dA = -G E^T (j < i),  dP = dOs E^T (j <= i),
//   dKd = -F S^T,  dQd = dOs S^T,  dKb = E dS'^T,  dGamma_n = rowsum(dS' o S),
// then through the decays: for M_ij = sum_c x_ic y_jc exp(gamma_ic - gamma_jc),
//   dx_ic = sum_j dM_ij y_jc exp(gamma_ic - gamma_jc),
//   dy_jc = sum_i dM_ij x_ic exp(gamma_ic - gamma_jc),  dgamma += x o dx - y o dy
// (M = P: x = q, y = k; M = Ab: x = y = k, dM = diag(beta) dA), and
//   dq = dQd o Gamma + dx_P,  dk = dKd o Gamma + dKb o exp(gamma_n - gamma) + ...,
//   dgamma += dKd o Kd + dQd o Qd - dKb o Kb,  dgamma_n = Gamma_n o dGamma_n + colsum(dKb o Kb),
//   dg_s = sum_{i >= s} dgamma_i + dgamma_n  (the reverse cumulative sum of the chunk).
// Every exponent formed is <= 0, so any decay strength is safe.
//
// Two kernels:
//   kda_dstate_kernel -- one workgroup per (sequence, head, 16 value columns);
//                        walks the chunks last to first on the forward's
//                        records, storing dS' of every chunk (fp32).  Its
//                        products take the records' operand type (bf16 MFMA
//                        with fp32 accumulation for bf16 io, fp32 for fp32 io).
//   kda_grad_kernel   -- one workgroup per (chunk, head, sequence), fully
//                        parallel, fp32 throughout (fp32 MFMA): the products
//                        above over 16-column tiles of d_v, then the decay
//                        terms pair by pair and the cumulative sum.
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_kda_common.h"

namespace gdn {
namespace {

using chunk::seq_range;

// N consecutive values (N a multiple of 8, 16-byte aligned) widened to fp32:
// 16-byte loads.
template <int N>
__device__ __forceinline__ void ld_row(const uint16_t* p, float (&out)[N]) {
#pragma unroll
  for (int u = 0; u < N / 8; ++u) {
    const uint4 x = *reinterpret_cast<const uint4*>(p + 8 * u);
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[8 * u + 2 * e] = __uint_as_float(w4[e] << 16);
      out[8 * u + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
    }
  }
}
template <int N>
__device__ __forceinline__ void ld_row(const float* p, float (&out)[N]) {
#pragma unroll
  for (int u = 0; u < N / 4; ++u) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + 4 * u);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * u + e] = x[e];
  }
}

// ---------------------------------------------------------------------------
// State-gradient pass.  LDS, in elements of the MFMA operand type EL: the chunk's
// record with rows padded by 16 bytes, then the B-operand tiles stored transposed
// (16 rows of the value tile, reduction index contiguous), then Gamma_n (fp32).
template <int DK, typename EL>
struct DsLds {
  static constexpr int PAD = 16 / static_cast<int>(sizeof(EL));
  static constexpr int L64 = 64 + PAD, LK = DK + PAD;
  static constexpr int kTb = 0;                  // [64][L64] T diag(beta)
  static constexpr int kP = kTb + 64 * L64;      // [64][L64] P
  static constexpr int kKG = kP + 64 * L64;      // [64][LK] K o Gamma
  static constexpr int kQG = kKG + 64 * LK;      // [64][LK] Q o Gamma
  static constexpr int kKDt = kQG + 64 * LK;     // [DK][L64] decayed keys, transposed
  static constexpr int kDoT = kKDt + DK * L64;   // [16][L64] (scale dO)^T
  static constexpr int kDsT = kDoT + 16 * L64;   // [16][LK] dS'^T
  static constexpr int kDeT = kDsT + 16 * LK;    // [16][L64] dE^T
  static constexpr int kFT = kDeT + 16 * L64;    // [16][L64] -F^T
  static constexpr int kElems = kFT + 16 * L64;
  static constexpr int kGnByte = (kElems * static_cast<int>(sizeof(EL)) + 15) / 16 * 16;
  static constexpr int kBytes = kGnByte + DK * 4;
};

// C tile (lane: rows 4 (lane / 16) + r of column lane % 16) stored transposed:
// dst[lane % 16][4 (lane / 16) + r], four consecutive elements.
template <typename EL>
__device__ __forceinline__ void store_ct(EL* dst, int ld, const f32x4_t& c, int lane) {
  chunk::store4<EL>(dst + (lane & 15) * ld + 4 * (lane >> 4), c[0], c[1], c[2], c[3]);
}

// Four waves: wave w forms rows 16 w .. 16 w + 15 of dE and F and holds the
// state-gradient rows 16 (w + 4 b) + 4 (lane / 16) + r in fp32 accumulators.
// The products take the record's operands as stored (bf16 for bf16 io, fp32 for
// fp32 io), transposed ones through transposing LDS reads; dE, F and dS' are
// rounded to that type as operands.  The next chunk's record and dO tile are
// loaded into registers while a chunk is processed.
template <int DK, typename E>
__global__ __launch_bounds__(256) void kda_dstate_kernel(KdaBwdParams p) {
  using Op = std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>;
  using EL = typename Op::elem;
  using R = kda::Rec<DK, EL>;
  using L = DsLds<DK, EL>;
  constexpr int KS = Op::KSTEP;
  constexpr int RB = DK / 64;                                  // state row blocks per wave
  constexpr int EPV = 16 / static_cast<int>(sizeof(EL));       // record elements per vector
  constexpr int NV = R::kGnByte / 16 / 256;                    // record vectors per thread
  constexpr int U64 = 4096 / EPV / 256;                        // vectors of one 64 x 64 matrix
  constexpr int UDK = 64 * DK / EPV / 256;                     // vectors of one 64 x DK matrix
  static_assert(NV == 2 * U64 + 3 * UDK, "record layout");
  constexpr int VPR = 16 * static_cast<int>(sizeof(E)) / 16;  // dO vectors per tile row
  constexpr int EPVIO = 16 / static_cast<int>(sizeof(E));
  extern __shared__ __align__(16) char sds[];
  EL* const sm = reinterpret_cast<EL*>(sds);
  float* const gn = reinterpret_cast<float*>(sds + L::kGnByte);
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  const int ntile = p.Dv / 16;
  const int nb = gridDim.x, Lb = blockIdx.x;
  const int vb = (nb % 8 == 0) ? (Lb % 8) * (nb / 8) + Lb / 8 : Lb;  // tiles of a head share an XCD
  const int tile = vb % ntile, nh = vb / ntile, h = nh % p.H, n = nh / p.H;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int nch = static_cast<int>((len + 63) / 64);
  const int Dv = p.Dv, c0 = tile * 16 + col;
  const E* dO = static_cast<const E*>(p.dO);
  const int64_t slot0 = bos / 64 + n;
  const char* const rec0 = static_cast<const char*>(p.rec) + (slot0 * p.H + h) * static_cast<int64_t>(R::kBytes);
  const int64_t rec_step = static_cast<int64_t>(p.H) * R::kBytes;

  f32x4_t dS[RB];
  const int64_t sbase = (static_cast<int64_t>(n) * p.H + h) * DK;
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dS[b][r] = p.dS_final ? p.dS_final[(sbase + 16 * (w + 4 * b) + 4 * g4 + r) * Dv + c0] : 0.f;

  // prefetch: the record of chunk c (its five matrices as 16-byte vectors tid + 256 u,
  // and Gamma_n) and the dO tile (rows past the sequence read as zeros through a
  // buffer resource bounded to the chunk's rows)
  f32x4_t pr[NV];
  f32x4_t pg = zero4();
  f32x4_t pd = zero4();
  const int drow = tid / VPR < 64 ? tid / VPR : 63, dpart = tid % VPR;
  auto prefetch = [&](int c) {
    const char* rc = rec0 + c * rec_step;
#pragma unroll
    for (int u = 0; u < NV; ++u) pr[u] = *reinterpret_cast<const f32x4_t*>(rc + 16 * (tid + 256 * u));
    pg = *reinterpret_cast<const f32x4_t*>(rc + R::kGnByte + 16 * (tid < DK / 4 ? tid : 0));
    const int64_t r0 = 64LL * c;
    const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
    const auto rd = chunk::buffer_rsrc(dO + ((bos + r0) * p.H + h) * Dv + tile * 16,
                                       static_cast<int>(((nr - 1) * p.H * Dv + 16) * sizeof(E)));
    pd = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                         rd, (drow * p.H * Dv + dpart * EPVIO) * static_cast<int>(sizeof(E)), 0, 0));
  };
  if (nch > 0) prefetch(nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    __syncthreads();  // every read of the previous chunk's LDS is done
    // the record into padded rows (each u lies in one matrix)
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      EL* dstp;
      if (u < 2 * U64) {
        const int f = EPV * (tid + 256 * (u < U64 ? u : u - U64));
        dstp = sm + (u < U64 ? L::kTb : L::kP) + (f / 64) * L::L64 + f % 64;
      } else if (u < 2 * U64 + 2 * UDK) {
        const int f = EPV * (tid + 256 * (u < 2 * U64 + UDK ? u - 2 * U64 : u - 2 * U64 - UDK));
        dstp = sm + (u < 2 * U64 + UDK ? L::kKG : L::kQG) + (f / DK) * L::LK + f % DK;
      } else {
        const int f = EPV * (tid + 256 * (u - 2 * U64 - 2 * UDK));
        dstp = sm + L::kKDt + (f / 64) * L::L64 + f % 64;
      }
      *reinterpret_cast<f32x4_t*>(dstp) = pr[u];
    }
    if (tid < DK / 4) *reinterpret_cast<f32x4_t*>(gn + 4 * tid) = pg;
    // (scale dO)^T: row j of the tile supplies column j
    if (tid < 64 * VPR) {
      float x[EPVIO];
      if constexpr (sizeof(E) == 2) {
        const uint32_t* u = reinterpret_cast<const uint32_t*>(&pd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = __uint_as_float(u[e] << 16);
          x[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = pd[e];
      }
#pragma unroll
      for (int e = 0; e < EPVIO; ++e) sm[L::kDoT + (dpart * EPVIO + e) * L::L64 + drow] = Op::cvt(p.scale * x[e]);
    }
    // dS' (the gradient after chunk c): to the per-chunk buffer (operand type) and,
    // transposed, to LDS
    EL* const dsg = static_cast<EL*>(p.dstates) + ((slot0 + c) * p.H + h) * static_cast<int64_t>(DK) * Dv;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rb = w + 4 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) dsg[(16 * rb + 4 * g4 + r) * Dv + c0] = Op::cvt(dS[b][r]);
      store_ct<EL>(sm + L::kDsT + 16 * rb, L::LK, dS[b], lane);
    }
    __syncthreads();
    if (c > 0) prefetch(c - 1);
    // dE = P^T dOs + Kb dS' (rows 16 w ..)
    {
      f32x4_t acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += KS)
        acc = Op::mma(Op::frag_tr(sm + L::kP + 16 * w, L::L64, lane, k0), Op::frag(sm + L::kDoT, L::L64, lane, k0), acc);
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += KS)
        acc = Op::mma(Op::frag_tr(sm + L::kKDt + 16 * w, L::L64, lane, k0), Op::frag(sm + L::kDsT, L::LK, lane, k0),
                      acc);
      store_ct<EL>(sm + L::kDeT + 16 * w, L::L64, acc, lane);
    }
    __syncthreads();
    // -F = -(T diag(beta))^T dE
    {
      f32x4_t acc = zero4();
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += KS)
        acc = Op::mma(Op::frag_tr(sm + L::kTb + 16 * w, L::L64, lane, k0), Op::frag(sm + L::kDeT, L::L64, lane, k0),
                      acc);
      store_ct<EL>(sm + L::kFT + 16 * w, L::L64, -acc, lane);
    }
    __syncthreads();
    // dS <- diag(Gamma_n) dS' + Qd^T dOs - Kd^T F
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rb = w + 4 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[b][r] *= gn[16 * rb + 4 * g4 + r];
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += KS)
        dS[b] = Op::mma(Op::frag_tr(sm + L::kQG + 16 * rb, L::LK, lane, k0), Op::frag(sm + L::kDoT, L::L64, lane, k0),
                        dS[b]);
#pragma unroll
      for (int k0 = 0; k0 < 64; k0 += KS)
        dS[b] = Op::mma(Op::frag_tr(sm + L::kKG + 16 * rb, L::LK, lane, k0), Op::frag(sm + L::kFT, L::L64, lane, k0),
                        dS[b]);
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dS0[(sbase + 16 * (w + 4 * b) + 4 * g4 + r) * Dv + c0] = dS[b][r];
  }
}

// Largest decay of one channel from the first row of a 16-row block to its middle
// row, or from there to its last row (log2 units), for which the gradient kernel
// forms the diagonal blocks' pair sums through the middle row.
constexpr float kMaxBlockDropBwd = 100.f;

// ---------------------------------------------------------------------------
// Gradient kernel.  Phase V (the d_v tiles) keeps its operands in the MFMA
// operand type EL (bf16 for bf16 io, fp32 for fp32 io) with rows padded by 16
// bytes; the tiles are TW = 32 (bf16: one MFMA depth) or 16 (fp32) columns of d_v.
template <int DK, typename EL>
struct GradVLds {
  static constexpr int ES = static_cast<int>(sizeof(EL));
  static constexpr int PAD = 16 / ES;
  static constexpr int TW = ES == 2 ? 32 : 16;
  static constexpr int LT = TW + PAD, LKE = DK + PAD, L64E = 64 + PAD;
  static constexpr int kSt = 0;                         // [DK][LT] S tile
  static constexpr int kDst = kSt + DK * LT * ES;       // [DK][LT] dS' tile
  static constexpr int kV = kDst + DK * LT * ES;        // [64][LT] V tile
  static constexpr int kDo = kV + 64 * LT * ES;         // [64][LT] scale dO tile
  static constexpr int kR = kDo + 64 * LT * ES;         // [64][LT] R
  static constexpr int kE = kR + 64 * LT * ES;          // [64][LT] E
  static constexpr int kDe = kE + 64 * LT * ES;         // [64][LT] dE
  static constexpr int kG = kDe + 64 * LT * ES;         // [64][LT] G = T^T dE
  static constexpr int kDv = kG + 64 * LT * ES;         // [64][LT] dv = diag(beta) G (io type = EL)
  static constexpr int kBe = kDv + 64 * LT * ES;        // [64] beta (fp32)
  static constexpr int kKd = kBe + 64 * 4;              // [64][LKE] K o Gamma
  static constexpr int kKb = kKd + 64 * LKE * ES;       // [64][LKE] K o exp(gamma_n - gamma)
  static constexpr int kT = kKb + 64 * LKE * ES;        // [64][L64E] T
  static constexpr int kP = kT + 64 * L64E * ES;        // [64][L64E] P (zero above the diagonal)
  static constexpr int kBytes = kP + 64 * L64E * ES;
  static_assert(kBe % 16 == 0 && kKd % 16 == 0 && kT % 16 == 0, "16-byte aligned rows");
};

// The later phases, in floats (rows of d_k + 4, and 84 for dA and dP: read both
// along rows and down columns).
template <int DK>
struct GradLds {
  static constexpr int LK = DK + 4;
  static constexpr int LY = 84;
  static constexpr int kDA = 0;                   // [64][LY] dA = -G E^T
  static constexpr int kDP = kDA + 64 * LY;       // [64][LY] dP = dOs E^T
  static constexpr int kQ = kDP + 64 * LY;        // [64][LK] q
  static constexpr int kK = kQ + 64 * LK;         // [64][LK] k
  static constexpr int kGam = kK + 64 * LK;       // [64][LK] gamma (log2 units)
  static constexpr int kBe2 = kGam + 64 * LK;     // [64] beta
  static constexpr int kEndY = kBe2 + 64;
  static constexpr int kDbA = kEndY;              // [64] sum_{j < i} dA_ij Ab_ij (read in phase Z)
  static constexpr int kSteep = kDbA + 64;        // flag: some block decays by more than 2^kMaxBlockDropBwd
  static constexpr int kDgn = kSteep + 4;         // [DK] sum over d_v of dS' o S (read in phase Z)
  static constexpr int kFloats = kDgn + DK;
  static_assert(3 * 64 * LK + DK <= kDbA, "phase X and Z arrays below the dbeta partials");
  static_assert(kFloats * 4 <= 160 * 1024, "LDS budget exceeded");
};
template <int DK, typename EL>
constexpr size_t grad_smem_bytes() {
  return GradVLds<DK, EL>::kBytes > GradLds<DK>::kFloats * 4 ? GradVLds<DK, EL>::kBytes
                                                             : GradLds<DK>::kFloats * 4;
}

// Eight waves.  Phase V: per TW-column tile of d_v, waves 0-3 form R then E and
// waves 4-7 dE then G (one 16-row block each), then every wave accumulates its
// share of dA, dP (two 16x16 tiles each) and G S^T, dQd, dKb (DK / 32 tiles each).
// Phase X/Y: wave w < DK / 16 owns channels 16 w .. 16 w + 15 (lane: one channel,
// 16 rows) for the elementwise terms and the pair sums: pairs inside the diagonal
// 16x16 blocks one exponential each, pairs across blocks as fp32 MFMA products of
// rows decayed to a reference row between the blocks.  Phase Z: thread (i, cg) =
// (tid / 8, tid % 8) stores row i's channels cg DK/8 .., thread c < DK forms
// channel c's reverse cumulative sum.
template <int DK, typename E>
__global__ __launch_bounds__(512) void kda_grad_kernel(KdaBwdParams p) {
  using Op = std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>;
  using EL = typename Op::elem;
  using V = GradVLds<DK, EL>;
  using L = GradLds<DK>;
  constexpr int LK = L::LK, LY = L::LY;
  constexpr int TW = V::TW, LT = V::LT, LKE = V::LKE, L64E = V::L64E, KS = Op::KSTEP;
  constexpr int CPT = DK / 8;         // channels per thread in the row phases
  constexpr int NK = DK / 32;         // G S^T / dQd / dKb tiles per wave
  constexpr int NB = TW / 16;         // 16-column blocks of a tile
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));    // io elements per vector
  constexpr int VPR = TW / EPV;                            // io vectors per tile row
  constexpr int EPS = 16 / static_cast<int>(sizeof(EL));   // state elements per vector
  constexpr int SPR = TW / EPS;                            // state vectors per tile row
  constexpr int NSV = (DK * SPR + 511) / 512;              // state vectors per thread
  static_assert(VPR * 64 <= 512 && (NSV == 1 || NSV * 512 == DK * SPR), "tile loads");
  static_assert(sizeof(E) == sizeof(EL), "dv is staged in the operand type, which is the io type");
  extern __shared__ __align__(16) float sg[];
  char* const sv = reinterpret_cast<char*>(sg);
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 15, g4 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t r0 = 64LL * c;
  if (r0 >= len) return;
  const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
  const int H = p.H, Dv = p.Dv;
  const int64_t slot = bos / 64 + n + c;
  const float* const aux = p.aux + (slot * H + h) * static_cast<int64_t>(kda::Aux::kFloats);
  const EL* const Sg = static_cast<const EL*>(p.states) + (slot * H + h) * static_cast<int64_t>(DK) * Dv;
  const EL* const dSg = static_cast<const EL*>(p.dstates) + (slot * H + h) * static_cast<int64_t>(DK) * Dv;
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  const E* dO = static_cast<const E*>(p.dO);
  const int ri = tid >> 3, cg = tid & 7;   // row phases: row ri, channels cg CPT ..
  const int rowc = ri < nr ? ri : nr - 1;  // rows past the chunk load its last row and are zeroed

  EL* const st = reinterpret_cast<EL*>(sv + V::kSt);
  EL* const dst = reinterpret_cast<EL*>(sv + V::kDst);
  EL* const vt = reinterpret_cast<EL*>(sv + V::kV);
  EL* const dot = reinterpret_cast<EL*>(sv + V::kDo);
  EL* const rt = reinterpret_cast<EL*>(sv + V::kR);
  EL* const et = reinterpret_cast<EL*>(sv + V::kE);
  EL* const det = reinterpret_cast<EL*>(sv + V::kDe);
  EL* const gt = reinterpret_cast<EL*>(sv + V::kG);
  EL* const dvt = reinterpret_cast<EL*>(sv + V::kDv);
  float* const be = reinterpret_cast<float*>(sv + V::kBe);
  EL* const kd = reinterpret_cast<EL*>(sv + V::kKd);
  EL* const kb = reinterpret_cast<EL*>(sv + V::kKb);
  EL* const tm = reinterpret_cast<EL*>(sv + V::kT);
  EL* const pm = reinterpret_cast<EL*>(sv + V::kP);

  // ---- stage 0: gamma, K o Gamma, K o exp(gamma_n - gamma), T, P, beta --------
  // (k and gamma pass through fp32 scratch at the start of LDS first)
  {
    float* const ksc = sg;               // [64][LK]
    float* const gsc = sg + 64 * LK;     // [64][LK]
    const int64_t off = ((bos + r0 + rowc) * H + h) * DK + cg * CPT;
    float kv[CPT], gv[CPT];
    ld_row<CPT>(k + off, kv);
    ld_row<CPT>(p.g + off, gv);
    f32x4_t tv[2], pv4[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      tv[u] = *reinterpret_cast<const f32x4_t*>(aux + kda::Aux::kT + 4 * (tid + 512 * u));
      pv4[u] = *reinterpret_cast<const f32x4_t*>(aux + kda::Aux::kP + 4 * (tid + 512 * u));
    }
    const float bt = p.beta[(bos + r0 + (lane < nr ? lane : nr - 1)) * H + h];
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      ksc[ri * LK + cg * CPT + e] = ri < nr ? kv[e] : 0.f;
      gsc[ri * LK + cg * CPT + e] = ri < nr ? gv[e] * chunk::kLog2e : 0.f;
    }
    __syncthreads();
    if (tid < DK) {  // cumulative sum of channel tid over the chunk, in place (log2 units)
      float acc = 0.f;
      for (int i = 0; i < 64; ++i) {
        acc += gsc[i * LK + tid];
        gsc[i * LK + tid] = acc;
      }
    }
    __syncthreads();
    float gl[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      kv[e] = ksc[ri * LK + cg * CPT + e];
      gv[e] = gsc[ri * LK + cg * CPT + e];
      gl[e] = gsc[63 * LK + cg * CPT + e];
    }
    __syncthreads();  // the scratch is dead from here on
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      kd[ri * LKE + cg * CPT + e] = Op::cvt(kv[e] * __builtin_amdgcn_exp2f(gv[e]));
      kb[ri * LKE + cg * CPT + e] = Op::cvt(kv[e] * __builtin_amdgcn_exp2f(gl[e] - gv[e]));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vx = tid + 512 * u, i = vx >> 4, j0 = 4 * (vx & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tm[i * L64E + j0 + e] = Op::cvt(tv[u][e]);
        pm[i * L64E + j0 + e] = Op::cvt(j0 + e <= i ? pv4[u][e] : 0.f);
      }
    }
    if (tid < 64) be[tid] = tid < nr ? bt : 0.f;
  }

  // ---- phase V: the d_v tiles ----------------------------------------------
  f32x4_t aA[2], aP[2], aKd[NK], aQd[NK], aKb[NK];
#pragma unroll
  for (int x = 0; x < 2; ++x) aA[x] = aP[x] = zero4();
#pragma unroll
  for (int x = 0; x < NK; ++x) aKd[x] = aQd[x] = aKb[x] = zero4();
  float dbv = 0.f;       // tid < 64: sum over d_v of G o R for row tid
  float dgp[NSV];        // sum over d_v of dS' o S, this thread's part of rows tid / SPR + (512 / SPR) u
#pragma unroll
  for (int u = 0; u < NSV; ++u) dgp[u] = 0.f;

  // tile prefetch: S and dS' rows (operand-type vectors), V and dO rows (io
  // vectors, bounded to the chunk's rows: past them the loads read zeros)
  const bool iol = tid < 64 * VPR;
  const int iorow = iol ? tid / VPR : 0, iopart = tid % VPR;
  const int vbytes = static_cast<int>(((nr - 1) * H * Dv + Dv) * sizeof(E));
  const auto rv = chunk::buffer_rsrc(v + ((bos + r0) * H + h) * Dv, vbytes);
  const auto rdo = chunk::buffer_rsrc(dO + ((bos + r0) * H + h) * Dv, vbytes);
  f32x4_t ps[NSV], pds[NSV], pv = zero4(), pdo = zero4();
  // (d_v a multiple of 16: the last bf16 tile may hold 16 valid columns; the
  // vectors past d_v load column v0 again and are staged as zeros)
  auto prefetch = [&](int t) {
    const int v0 = TW * t;
#pragma unroll
    for (int u = 0; u < NSV; ++u) {
      const int x = tid + 512 * u, row = x < DK * SPR ? x / SPR : 0, part = x % SPR;
      const int cv = v0 + EPS * part < Dv ? v0 + EPS * part : v0;
      ps[u] = *reinterpret_cast<const f32x4_t*>(Sg + row * Dv + cv);
      pds[u] = *reinterpret_cast<const f32x4_t*>(dSg + row * Dv + cv);
    }
    const int cv = v0 + iopart * EPV < Dv ? v0 + iopart * EPV : v0;
    const int off = (iorow * H * Dv + cv) * static_cast<int>(sizeof(E));
    pv = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    pdo = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
  };
  // EPV io values of a vector to EL in LDS, times mul
  auto io_to_lds = [&](EL* dstp, const f32x4_t& x, float mul) {
    if constexpr (sizeof(E) == 2) {
      const uint32_t* u = reinterpret_cast<const uint32_t*>(&x);
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = mul * __uint_as_float(u[e] << 16);
        f[2 * e + 1] = mul * __uint_as_float(u[e] & 0xffff0000u);
      }
      *reinterpret_cast<uint4*>(dstp) = uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                              pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
    } else {
      *reinterpret_cast<f32x4_t*>(dstp) = x * mul;
    }
  };
  const int ntile = (Dv + TW - 1) / TW;
  prefetch(0);
  for (int t = 0; t < ntile; ++t) {
    const int v0 = TW * t;
    __syncthreads();  // the previous tile's reads are done (and stage 0's writes visible)
#pragma unroll
    for (int u = 0; u < NSV; ++u) {
      const int x = tid + 512 * u, row = x / SPR, part = x % SPR;
      if (x >= DK * SPR) continue;
      const f32x4_t z = zero4();
      const bool okc = v0 + EPS * part < Dv;
      const f32x4_t a = okc ? ps[u] : z, b = okc ? pds[u] : z;
      *reinterpret_cast<f32x4_t*>(st + row * LT + EPS * part) = a;   // EPS operand values, as stored
      *reinterpret_cast<f32x4_t*>(dst + row * LT + EPS * part) = b;
      if constexpr (sizeof(EL) == 2) {
        const uint32_t* ua = reinterpret_cast<const uint32_t*>(&a);
        const uint32_t* ub = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dgp[u] = fmaf(__uint_as_float(ua[e] << 16), __uint_as_float(ub[e] << 16), dgp[u]);
          dgp[u] = fmaf(__uint_as_float(ua[e] & 0xffff0000u), __uint_as_float(ub[e] & 0xffff0000u), dgp[u]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dgp[u] = fmaf(a[e], b[e], dgp[u]);
      }
    }
    if (iol) {
      const bool okc = v0 + iopart * EPV < Dv;
      io_to_lds(vt + iorow * LT + iopart * EPV, okc ? pv : zero4(), 1.f);
      io_to_lds(dot + iorow * LT + iopart * EPV, okc ? pdo : zero4(), p.scale);
    }
    __syncthreads();
    if (t + 1 < ntile) prefetch(t + 1);
    if (w < 4) {  // R = V - Kd S (rows 16 w ..)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KS)
          acc = Op::mma(Op::frag(kd + 16 * w * LKE, LKE, lane, k0), Op::frag_tr(st + 16 * nb, LT, lane, k0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * w + 4 * g4 + r;
          rt[row * LT + 16 * nb + col] = Op::cvt(Op::widen(vt[row * LT + 16 * nb + col]) - acc[r]);
        }
      }
    } else {  // dE = P^T dOs + Kb dS' (rows 16 (w - 4) ..)
      const int w4 = w - 4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += KS)
          acc = Op::mma(Op::frag_tr(pm + 16 * w4, L64E, lane, k0), Op::frag_tr(dot + 16 * nb, LT, lane, k0), acc);
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KS)
          acc = Op::mma(Op::frag(kb + 16 * w4 * LKE, LKE, lane, k0), Op::frag_tr(dst + 16 * nb, LT, lane, k0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) det[(16 * w4 + 4 * g4 + r) * LT + 16 * nb + col] = Op::cvt(acc[r]);
      }
    }
    __syncthreads();
    if (w < 4) {  // E = T diag(beta) R
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += KS)
          acc = Op::mma(Op::scale(Op::frag(tm + 16 * w * L64E, L64E, lane, k0), be, lane, k0),
                        Op::frag_tr(rt + 16 * nb, LT, lane, k0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) et[(16 * w + 4 * g4 + r) * LT + 16 * nb + col] = Op::cvt(acc[r]);
      }
    } else {  // G = T^T dE; dv = diag(beta) G (to LDS, stored below)
      const int w4 = w - 4;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 64; k0 += KS)
          acc = Op::mma(Op::frag_tr(tm + 16 * w4, L64E, lane, k0), Op::frag_tr(det + 16 * nb, LT, lane, k0), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * w4 + 4 * g4 + r;
          gt[row * LT + 16 * nb + col] = Op::cvt(acc[r]);
          dvt[row * LT + 16 * nb + col] = Op::cvt(be[row] * acc[r]);
        }
      }
    }
    __syncthreads();
    // dv rows out of LDS as 16-byte vectors (rows and columns past the chunk and d_v stay)
    if (tid < 64 * VPR) {
      const int row = tid / VPR, part = tid % VPR;
      if (row < nr && v0 + part * EPV < Dv)
        *reinterpret_cast<uint4*>(static_cast<E*>(p.dv) + ((bos + r0 + row) * H + h) * Dv + v0 + part * EPV) =
            *reinterpret_cast<const uint4*>(dvt + row * LT + part * EPV);
    }
    // accumulations over this tile's TW columns
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ta = 2 * w + x, ti = ta >> 2, tj = ta & 3;
#pragma unroll
      for (int k0 = 0; k0 < TW; k0 += KS) {
        const auto fe = Op::frag(et + 16 * tj * LT, LT, lane, k0);
        aA[x] = Op::mma(Op::frag(gt + 16 * ti * LT, LT, lane, k0), fe, aA[x]);
        aP[x] = Op::mma(Op::frag(dot + 16 * ti * LT, LT, lane, k0), fe, aP[x]);
      }
    }
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int tk = NK * w + x, ti = tk / (DK / 16), tc = tk % (DK / 16);
#pragma unroll
      for (int k0 = 0; k0 < TW; k0 += KS) {
        const auto fs = Op::frag(st + 16 * tc * LT, LT, lane, k0);
        aKd[x] = Op::mma(Op::frag(gt + 16 * ti * LT, LT, lane, k0), fs, aKd[x]);
        aQd[x] = Op::mma(Op::frag(dot + 16 * ti * LT, LT, lane, k0), fs, aQd[x]);
        aKb[x] = Op::mma(Op::frag(et + 16 * ti * LT, LT, lane, k0), Op::frag(dst + 16 * tc * LT, LT, lane, k0),
                         aKb[x]);
      }
    }
    if (tid < 64) {
#pragma unroll
      for (int j = 0; j < TW; ++j) dbv = fmaf(Op::widen(gt[tid * LT + j]), Op::widen(rt[tid * LT + j]), dbv);
    }
  }
  // dKd = -diag(beta) G S^T: the rows' beta, read before the tile memory is reused
  float bkd[4];
  {
    const int ti = (NK * w) / (DK / 16);  // the same row block for every x of this wave
#pragma unroll
    for (int r = 0; r < 4; ++r) bkd[r] = be[16 * ti + 4 * g4 + r];
  }
  // the SPR lanes of a state row hold its dS' o S partial sums
#pragma unroll
  for (int u = 0; u < NSV; ++u) {
#pragma unroll
    for (int sh = 1; sh < SPR; sh <<= 1) dgp[u] += __shfl_xor(dgp[u], sh, 64);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NSV; ++u) {
    const int x = tid + 512 * u;
    if (x < DK * SPR && x % SPR == 0) sg[L::kDgn + x / SPR] = dgp[u];
  }

  // ---- phase X: dKd = -F S^T, dQd = dOs S^T, dKb = E dS'^T to their owners ----
  // From here on wave w < DK / 16 owns channel c = 16 w + lane % 16 and rows
  // 16 b + 4 (lane / 16) + r (b, r < 4): the element layout of an MFMA result
  // tile, so the pair products below land on their owners.
  constexpr int NCB = DK / 16;
  const bool cw = w < NCB;
  const int ch = 16 * (cw ? w : 0) + col;
  float xKd[4][4], xQd[4][4], xKb[4][4];
  {
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int tk = NK * w + x, ti = tk / (DK / 16), tc = tk % (DK / 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ti + 4 * g4 + r, cc = 16 * tc + col;
        sg[row * LK + cc] = -bkd[r] * aKd[x][r];
        sg[64 * LK + row * LK + cc] = aQd[x][r];
        sg[2 * 64 * LK + row * LK + cc] = aKb[x][r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * b + 4 * g4 + r;
        xKd[b][r] = sg[row * LK + ch];
        xQd[b][r] = sg[64 * LK + row * LK + ch];
        xKb[b][r] = sg[2 * 64 * LK + row * LK + ch];
      }
    __syncthreads();
  }

  // ---- phase Y: dA, dP, q, k, gamma; elementwise terms and pair sums ----------
  float* const dA = sg + L::kDA;
  float* const dP = sg + L::kDP;
  float* const qs = sg + L::kQ;
  float* const ks = sg + L::kK;
  float* const gs = sg + L::kGam;
  float* const be2 = sg + L::kBe2;
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int ta = 2 * w + x, ti = ta >> 2, tj = ta & 3;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g4 + r, j = 16 * tj + col;
      dA[i * LY + j] = -aA[x][r];
      dP[i * LY + j] = aP[x][r];
    }
  }
  f32x4_t abr0, abr1;  // Ab row ri, columns 8 cg .. 8 cg + 7
  {
    const int64_t off = ((bos + r0 + rowc) * H + h) * DK + cg * CPT;
    float qv[CPT], kv[CPT], gv[CPT];
    ld_row<CPT>(q + off, qv);
    ld_row<CPT>(k + off, kv);
    ld_row<CPT>(p.g + off, gv);
    const float bt = p.beta[(bos + r0 + (lane < nr ? lane : nr - 1)) * H + h];
    abr0 = *reinterpret_cast<const f32x4_t*>(aux + kda::Aux::kAb + ri * 64 + 8 * cg);
    abr1 = *reinterpret_cast<const f32x4_t*>(aux + kda::Aux::kAb + ri * 64 + 8 * cg + 4);
    const bool ok = ri < nr;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      qs[ri * LK + cg * CPT + e] = ok ? qv[e] : 0.f;
      ks[ri * LK + cg * CPT + e] = ok ? kv[e] : 0.f;
      gs[ri * LK + cg * CPT + e] = ok ? gv[e] * chunk::kLog2e : 0.f;
    }
    if (tid < 64) be2[tid] = tid < nr ? bt : 0.f;
    if (tid == 0) sg[L::kSteep] = 0.f;
  }
  __syncthreads();
  if (tid < DK) {  // gamma, and the largest decay of channel tid across one half of a 16-row block
    float acc = 0.f, first = 0.f, mid = 0.f, drop = 0.f;
    for (int i = 0; i < 64; ++i) {
      acc += gs[i * LK + tid];
      gs[i * LK + tid] = acc;
      if (i % 16 == 0) first = acc;
      if (i % 16 == 8) {
        mid = acc;
        drop = fmaxf(drop, first - mid);
      }
      if (i % 16 == 15) drop = fmaxf(drop, mid - acc);
    }
    if (drop > kMaxBlockDropBwd) sg[L::kSteep] = 1.f;  // (every writer stores the same value)
  }
  __syncthreads();
  const bool steep = sg[L::kSteep] != 0.f;  // uniform over the workgroup
  // dbeta's second term, sum_{j < i} dA_ij Ab_ij: eight threads per row i, eight
  // columns each, added across the eight lanes (the rest comes in phase Z)
  {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = 8 * cg + e, j1 = j0 + 4;
      part += j0 < ri ? dA[ri * LY + j0] * abr0[e] : 0.f;
      part += j1 < ri ? dA[ri * LY + j1] * abr1[e] : 0.f;
    }
    part += __shfl_xor(part, 1, 64);
    part += __shfl_xor(part, 2, 64);
    part += __shfl_xor(part, 4, 64);
    if (cg == 0) sg[L::kDbA + ri] = part;
  }
  const float gnl = tid < DK ? gs[63 * LK + tid] : 0.f;  // gamma_n of channel tid (phase Z)
  float dq[4][4], dk[4][4], dgam[4][4];
  float xsum = 0.f;  // this lane's rows of sum_i (dKb o Kb)_i, channel ch
  if (cw) {
    const float gn = gs[63 * LK + ch];
    // the elementwise terms of K o Gamma, Q o Gamma and the decayed keys
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * b + 4 * g4 + r;
        const float gi = gs[i * LK + ch], ki = ks[i * LK + ch], qi = qs[i * LK + ch];
        const float G = __builtin_amdgcn_exp2f(gi), eb = __builtin_amdgcn_exp2f(gn - gi);
        const float xx = xKb[b][r] * ki * eb;
        dq[b][r] = xQd[b][r] * G;
        dk[b][r] = xKd[b][r] * G + xKb[b][r] * eb;
        dgam[b][r] = (xKd[b][r] * ki + xQd[b][r] * qi) * G - xx;
        xsum += xx;
      }
    // Pair products through a reference row, on fp32 MFMA.  Row side (results on
    // the rows i of block bi, sums over the rows j of block bj):
    //   sum_j M_ij y_j exp(gamma_i - gamma_j) = exp(gamma_i - gamma_a) sum_j M_ij (y_j exp(gamma_a - gamma_j));
    // column side (results on the rows j of block bj, sums over the rows i of bi):
    //   sum_i M_ij x_i exp(gamma_i - gamma_j) = exp(gamma_c - gamma_j) sum_i M_ij (x_i exp(gamma_i - gamma_c)).
    // Across blocks (bj < bi) a = 16 bj + 15 and c = 16 bi, so every factor is <= 1.
    // Inside a diagonal block (bi = bj = b) a = c = 16 b + 8, the middle row: every
    // factor lies between 2^-D and 2^D, D the larger decay from the block's first
    // row to its middle row and from there to its last, which the steep flag bounds
    // by kMaxBlockDropBwd (log2 units); steeper chunks take the pairs one by one below.
    auto pairs = [&](int bi, int bj, int ra, int rc, bool diag) __attribute__((always_inline)) {
      const float ga = gs[ra * LK + ch], gc = gs[rc * LK + ch];
      f32x4_t p1 = zero4(), p2 = zero4(), p3 = zero4(), p4 = zero4();
      const int im = 16 * bi + col;   // A row of the row side
      const int jm = 16 * bj + col;   // A row of the column side
      const float bim = be2[im];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int j = 16 * bj + 4 * st + g4;  // row side: k index
        const int i = 16 * bi + 4 * st + g4;  // column side: k index
        const float kr = ks[j * LK + ch] * __builtin_amdgcn_exp2f(ga - gs[j * LK + ch]);
        float a1 = dP[im * LY + j], a2 = bim * dA[im * LY + j];
        float a3 = dP[i * LY + jm], a4 = be2[i] * dA[i * LY + jm];
        if (diag) {
          a1 = j <= im ? a1 : 0.f;
          a2 = j < im ? a2 : 0.f;
          a3 = i >= jm ? a3 : 0.f;
          a4 = i > jm ? a4 : 0.f;
        }
        const float ec = __builtin_amdgcn_exp2f(gs[i * LK + ch] - gc);
        p1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, kr, p1, 0, 0, 0);
        p2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, kr, p2, 0, 0, 0);
        p3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, qs[i * LK + ch] * ec, p3, 0, 0, 0);
        p4 = __builtin_amdgcn_mfma_f32_16x16x4f32(a4, ks[i * LK + ch] * ec, p4, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * bi + 4 * g4 + r, j = 16 * bj + 4 * g4 + r;
        const float fi = __builtin_amdgcn_exp2f(gs[i * LK + ch] - ga);
        const float fj = __builtin_amdgcn_exp2f(gc - gs[j * LK + ch]);
        const float ki = ks[i * LK + ch], qi = qs[i * LK + ch], kj = ks[j * LK + ch];
        dq[bi][r] += fi * p1[r];
        dk[bi][r] += fi * p2[r];
        dgam[bi][r] += fi * (qi * p1[r] + ki * p2[r]);
        const float cs = fj * (p3[r] + p4[r]);
        dk[bj][r] += cs;
        dgam[bj][r] -= kj * cs;
      }
    };
    // (written out: every block index must be a compile-time constant, so that
    // the per-block accumulators stay in registers)
    pairs(1, 0, 15, 16, false);
    pairs(2, 0, 15, 32, false);
    pairs(3, 0, 15, 48, false);
    pairs(2, 1, 31, 32, false);
    pairs(3, 1, 31, 48, false);
    pairs(3, 2, 47, 48, false);
    if (!steep) {
      pairs(0, 0, 8, 8, true);
      pairs(1, 1, 24, 24, true);
      pairs(2, 2, 40, 40, true);
      pairs(3, 3, 56, 56, true);
    } else {
      // pairs inside the diagonal blocks one by one, one exponential each:
      // exp(gamma_i - gamma_j) for j <= i (row side), exp(gamma_j - gamma_i) for j >= i
      auto one_by_one = [&](int b) __attribute__((always_inline)) {
        float gi[4], aq[4], ak1[4], bp[4], ba[4], bir[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gi[r] = gs[(16 * b + 4 * g4 + r) * LK + ch];
          bir[r] = be2[16 * b + 4 * g4 + r];
          aq[r] = ak1[r] = bp[r] = ba[r] = 0.f;
        }
        for (int jj = 0; jj < 16; ++jj) {
          const int j = 16 * b + jj;
          const float kj = ks[j * LK + ch], qj = qs[j * LK + ch], gj = gs[j * LK + ch], bj = be2[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * b + 4 * g4 + r;
            const float e = __builtin_amdgcn_exp2f(-fabsf(gi[r] - gj));
            const float pij = dP[i * LY + j], aij = dA[i * LY + j];
            const float pji = dP[j * LY + i], aji = dA[j * LY + i];
            aq[r] = fmaf(j <= i ? pij : 0.f, kj * e, aq[r]);
            ak1[r] = fmaf(j < i ? bir[r] * aij : 0.f, kj * e, ak1[r]);
            bp[r] = fmaf(j >= i ? pji : 0.f, qj * e, bp[r]);
            ba[r] = fmaf(j > i ? bj * aji : 0.f, kj * e, ba[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * b + 4 * g4 + r;
          const float ki = ks[i * LK + ch], qi = qs[i * LK + ch];
          dq[b][r] += aq[r];
          dk[b][r] += ak1[r] + bp[r] + ba[r];
          dgam[b][r] += qi * aq[r] + ki * (ak1[r] - bp[r] - ba[r]);
        }
      };
      one_by_one(0);
      one_by_one(1);
      one_by_one(2);
      one_by_one(3);
    }
  }
  __syncthreads();

  // ---- phase Z: dq, dk stores; dg = reverse cumulative sum of dgamma, plus dgamma_n ----
  float* const dqs = sg;               // [64][LK]
  float* const dks = sg + 64 * LK;     // [64][LK]
  float* const dgs = sg + 2 * 64 * LK; // [64][LK] dgamma
  float* const xs = sg + 3 * 64 * LK;  // [DK] sum over the rows of dKb o Kb
  // the four lanes of a channel (lane % 16 equal) hold its 64 rows between them
  xsum += __shfl_xor(xsum, 16, 64);
  xsum += __shfl_xor(xsum, 32, 64);
  if (cw) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * b + 4 * g4 + r;
        dqs[i * LK + ch] = dq[b][r];
        dks[i * LK + ch] = dk[b][r];
        dgs[i * LK + ch] = dgam[b][r];
      }
    if (g4 == 0) xs[ch] = xsum;
  }
  __syncthreads();
  if (ri < nr) {
    E* const dqo = static_cast<E*>(p.dq) + ((bos + r0 + ri) * H + h) * DK + cg * CPT;
    E* const dko = static_cast<E*>(p.dk) + ((bos + r0 + ri) * H + h) * DK + cg * CPT;
#pragma unroll
    for (int e0 = 0; e0 < CPT; e0 += 8) {
      float a8[8], b8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a8[e] = dqs[ri * LK + cg * CPT + e0 + e];
        b8[e] = dks[ri * LK + cg * CPT + e0 + e];
      }
      if constexpr (sizeof(E) == 2) {
        *reinterpret_cast<uint4*>(dqo + e0) = uint4{pack_bf16x2(a8[0], a8[1]), pack_bf16x2(a8[2], a8[3]),
                                                    pack_bf16x2(a8[4], a8[5]), pack_bf16x2(a8[6], a8[7])};
        *reinterpret_cast<uint4*>(dko + e0) = uint4{pack_bf16x2(b8[0], b8[1]), pack_bf16x2(b8[2], b8[3]),
                                                    pack_bf16x2(b8[4], b8[5]), pack_bf16x2(b8[6], b8[7])};
      } else {
        *reinterpret_cast<f32x4_t*>(dqo + e0) = f32x4_t{a8[0], a8[1], a8[2], a8[3]};
        *reinterpret_cast<f32x4_t*>(dqo + e0 + 4) = f32x4_t{a8[4], a8[5], a8[6], a8[7]};
        *reinterpret_cast<f32x4_t*>(dko + e0) = f32x4_t{b8[0], b8[1], b8[2], b8[3]};
        *reinterpret_cast<f32x4_t*>(dko + e0 + 4) = f32x4_t{b8[4], b8[5], b8[6], b8[7]};
      }
    }
  }
  // dbeta (rows tid < 64): sum over d_v of G o R, plus the Ab term
  if (tid < nr) p.dbeta[(bos + r0 + tid) * H + h] = dbv + sg[L::kDbA + tid];
  if (tid < DK) {
    float acc = __builtin_amdgcn_exp2f(gnl) * sg[L::kDgn + tid] + xs[tid];
    for (int s2 = 63; s2 >= 0; --s2) {
      acc += dgs[s2 * LK + tid];
      if (s2 < nr) p.dg[((bos + r0 + s2) * H + h) * DK + tid] = acc;
    }
  }
}

template <int DK, typename E>
hipError_t launch_kda_bwd_t(const KdaBwdParams& p, hipStream_t s) {
  using EL = typename std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>::elem;
  constexpr size_t ds_smem = DsLds<DK, EL>::kBytes;
  constexpr size_t gr_smem = grad_smem_bytes<DK, EL>();
  static_assert(gr_smem <= 160 * 1024, "LDS budget exceeded");
  static_assert(ds_smem <= 160 * 1024, "LDS budget exceeded");
  auto ds = kda_dstate_kernel<DK, E>;
  auto gr = kda_grad_kernel<DK, E>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(ds), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(ds_smem));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(gr), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(gr_smem));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ds, dim3(p.N * p.H * (p.Dv / 16)), dim3(256), ds_smem, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.max_chunks > 0) {
    hipLaunchKernelGGL(gr, dim3(p.max_chunks, p.H, p.N), dim3(512), gr_smem, s, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_kda_bwd(const KdaBwdParams& p, int Dk, bool bf16, hipStream_t s) {
  if (Dk == 128) return bf16 ? launch_kda_bwd_t<128, uint16_t>(p, s) : launch_kda_bwd_t<128, float>(p, s);
  if (Dk == 64) return bf16 ? launch_kda_bwd_t<64, uint16_t>(p, s) : launch_kda_bwd_t<64, float>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
