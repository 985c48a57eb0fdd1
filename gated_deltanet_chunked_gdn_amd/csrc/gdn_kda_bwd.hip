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
// Two kernels, both fp32 throughout (fp32 MFMA, 16x16x4):
//   kda_dstate_kernel -- one workgroup per (sequence, head, 16 value columns);
//                        walks the chunks last to first on the forward's
//                        records, storing dS' of every chunk.
//   kda_grad_kernel   -- one workgroup per (chunk, head, sequence), fully
//                        parallel: the products above over 16-column tiles of
//                        d_v, then the decay terms pair by pair and the
//                        cumulative sum.
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_kda_common.h"

namespace gdn {
namespace {

using chunk::seq_range;

__device__ __forceinline__ float ldf(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ldf(const float* p) { return *p; }

// acc += A(16 x K) B(K x 16) on fp32 MFMA.  `a` points at A(m, kq) and `b` at
// B(kq, n) for this lane (m = n = lane % 16, kq = lane / 16); SA and SB are the
// strides between consecutive k.  Up to four independent accumulation chains.
template <int K, int SA, int SB, typename TA>
__device__ __forceinline__ void mm(f32x4_t& acc, const TA* a, const float* b, float ascale = 1.f) {
  constexpr int NS = K / 4;
  constexpr int NA = NS < 4 ? NS : 4;
  static_assert(NS * 4 == K, "K must be a multiple of 4");
  f32x4_t x[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) x[j] = zero4();
#pragma unroll
  for (int st = 0; st < NS; ++st)
    x[st % NA] = __builtin_amdgcn_mfma_f32_16x16x4f32(ascale * ldf(a + 4 * st * SA), b[4 * st * SB], x[st % NA],
                                                      0, 0, 0);
#pragma unroll
  for (int j = 0; j < NA; ++j) acc += x[j];
}

// ---------------------------------------------------------------------------
// State-gradient pass.  LDS (bytes): the chunk's record as stored, then fp32
// tiles with rows of 20 floats.
template <int DK, typename EL>
struct DsLds {
  using R = kda::Rec<DK, EL>;
  static constexpr int LT = 20;
  static constexpr int kRec = 0;                    // record matrices and Gamma_n, as in global memory
  static constexpr int kDo = R::kBytes;             // float [64][LT]: scale dO, rows past the chunk zero
  static constexpr int kDs = kDo + 64 * LT * 4;     // float [DK][LT]: dS'
  static constexpr int kDe = kDs + DK * LT * 4;     // float [64][LT]: dE
  static constexpr int kF = kDe + 64 * LT * 4;      // float [64][LT]: F
  static constexpr int kBytes = kF + 64 * LT * 4;
};

// Four waves: wave w forms rows 16 w .. 16 w + 15 of dE and F and holds the
// state-gradient rows 16 (w + 4 b) + 4 (lane / 16) + r in accumulators.  The next
// chunk's record and dO tile are loaded into registers while a chunk is
// processed and written to LDS at the top of the next step.
template <int DK, typename E>
__global__ __launch_bounds__(256) void kda_dstate_kernel(KdaBwdParams p) {
  using EL = std::conditional_t<sizeof(E) == 2, uint16_t, float>;
  using R = kda::Rec<DK, EL>;
  using L = DsLds<DK, EL>;
  constexpr int LT = L::LT;
  constexpr int RB = DK / 64;                      // state row blocks per wave
  constexpr int NVEC = R::kBytes / 16;             // record vectors
  constexpr int NU = (NVEC + 255) / 256;           // record vectors per thread
  constexpr int VPR = 16 * static_cast<int>(sizeof(E)) / 16;  // dO vectors per tile row
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));
  extern __shared__ __align__(16) char sds[];
  const EL* const rs = reinterpret_cast<const EL*>(sds + L::kRec);
  const float* const gn = reinterpret_cast<const float*>(sds + R::kGnByte);
  float* const dos = reinterpret_cast<float*>(sds + L::kDo);
  float* const dss = reinterpret_cast<float*>(sds + L::kDs);
  float* const des = reinterpret_cast<float*>(sds + L::kDe);
  float* const fs = reinterpret_cast<float*>(sds + L::kF);
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g4 = lane >> 4, kq = g4;
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

  // prefetch: the record of chunk c and the dO tile (rows past the sequence read
  // as zeros through a buffer resource bounded to the chunk's rows)
  f32x4_t pr[NU];
  f32x4_t pd = zero4();
  const int drow = tid / VPR < 64 ? tid / VPR : 63, dpart = tid % VPR;
  auto prefetch = [&](int c) {
    const char* rc = rec0 + c * rec_step;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int x = tid + 256 * u;
      pr[u] = *reinterpret_cast<const f32x4_t*>(rc + 16 * (x < NVEC ? x : NVEC - 1));
    }
    const int64_t r0 = 64LL * c;
    const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
    const auto rd = chunk::buffer_rsrc(dO + ((bos + r0) * p.H + h) * Dv + tile * 16,
                                       static_cast<int>(((nr - 1) * p.H * Dv + 16) * sizeof(E)));
    pd = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                         rd, (drow * p.H * Dv + dpart * EPV) * static_cast<int>(sizeof(E)), 0, 0));
  };
  if (nch > 0) prefetch(nch - 1);

  for (int c = nch - 1; c >= 0; --c) {
    __syncthreads();  // every read of the previous chunk's LDS is done
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int x = tid + 256 * u;
      if (x < NVEC) *reinterpret_cast<f32x4_t*>(sds + L::kRec + 16 * x) = pr[u];
    }
    if (tid < 64 * VPR) {
      float* dst = dos + drow * LT + dpart * EPV;
      if constexpr (sizeof(E) == 2) {
        const uint32_t* u = reinterpret_cast<const uint32_t*>(&pd);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[2 * e] = p.scale * __uint_as_float(u[e] << 16);
          dst[2 * e + 1] = p.scale * __uint_as_float(u[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = p.scale * pd[e];
      }
    }
    // dS' (the gradient after chunk c) to LDS and to the per-chunk buffer
    float* const dsg = p.dstates + ((slot0 + c) * p.H + h) * static_cast<int64_t>(DK) * Dv;
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (w + 4 * b) + 4 * g4 + r;
        dss[row * LT + col] = dS[b][r];
        dsg[row * Dv + c0] = dS[b][r];
      }
    __syncthreads();
    if (c > 0) prefetch(c - 1);
    // dE = P^T dOs + Kb dS' (rows 16 w ..)
    {
      f32x4_t acc = zero4();
      mm<64, 64, LT>(acc, rs + R::kP + kq * 64 + 16 * w + col, dos + kq * LT + col);
      mm<DK, 64, LT>(acc, rs + R::kKDt + kq * 64 + 16 * w + col, dss + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) des[(16 * w + 4 * g4 + r) * LT + col] = acc[r];
    }
    __syncthreads();
    // F = (T diag(beta))^T dE
    {
      f32x4_t acc = zero4();
      mm<64, 64, LT>(acc, rs + R::kTb + kq * 64 + 16 * w + col, des + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) fs[(16 * w + 4 * g4 + r) * LT + col] = acc[r];
    }
    __syncthreads();
    // dS <- diag(Gamma_n) dS' + Qd^T dOs - Kd^T F
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rb = w + 4 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[b][r] *= gn[16 * rb + 4 * g4 + r];
      mm<64, DK, LT>(dS[b], rs + R::kQG + kq * DK + 16 * rb + col, dos + kq * LT + col);
      f32x4_t kf = zero4();
      mm<64, DK, LT>(kf, rs + R::kKG + kq * DK + 16 * rb + col, fs + kq * LT + col);
      dS[b] -= kf;
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) p.dS0[(sbase + 16 * (w + 4 * b) + 4 * g4 + r) * Dv + c0] = dS[b][r];
  }
}

// ---------------------------------------------------------------------------
// Gradient kernel.  LDS in floats; rows of d_k + 4 (LK), 68 (L64) and 20 (LT)
// floats.  Phase V (the d_v tiles) uses the first layout, the later phases reuse
// the same memory.
template <int DK>
struct GradLds {
  static constexpr int LK = DK + 4, L64 = 68, LT = 20;
  // phase V: the per-tile arrays first (within 64 KiB: immediate LDS offsets)
  static constexpr int kSt = 0;                   // [DK][LT] S tile
  static constexpr int kDst = kSt + DK * LT;      // [DK][LT] dS' tile
  static constexpr int kV = kDst + DK * LT;       // [64][LT] V tile
  static constexpr int kDo = kV + 64 * LT;        // [64][LT] scale dO tile
  static constexpr int kR = kDo + 64 * LT;        // [64][LT] R
  static constexpr int kBR = kR + 64 * LT;        // [64][LT] diag(beta) R
  static constexpr int kE = kBR + 64 * LT;        // [64][LT] E
  static constexpr int kDe = kE + 64 * LT;        // [64][LT] dE
  static constexpr int kG = kDe + 64 * LT;        // [64][LT] G = T^T dE
  static constexpr int kBe = kG + 64 * LT;        // [64] beta
  static constexpr int kKd = kBe + 64;            // [64][LK] K o Gamma
  static constexpr int kKb = kKd + 64 * LK;       // [64][LK] K o exp(gamma_n - gamma)
  static constexpr int kT = kKb + 64 * LK;        // [64][L64] T
  static constexpr int kP = kT + 64 * L64;        // [64][L64] P (zero above the diagonal)
  static constexpr int kEndV = kP + 64 * L64;
  // phase Y
  static constexpr int kDA = 0;                   // [64][L64] dA = -G E^T
  static constexpr int kDP = kDA + 64 * L64;      // [64][L64] dP = dOs E^T
  static constexpr int kQ = kDP + 64 * L64;       // [64][LK] q
  static constexpr int kK = kQ + 64 * LK;         // [64][LK] k
  static constexpr int kGam = kK + 64 * LK;       // [64][LK] gamma (log2 units)
  static constexpr int kBe2 = kGam + 64 * LK;     // [64] beta
  static constexpr int kEndY = kBe2 + 64;
  static constexpr int kFloats = kEndV > kEndY ? kEndV : kEndY;
  static_assert(kBe * 4 <= 65536, "tile arrays within the immediate-offset range");
  static_assert(3 * 64 * LK <= kFloats, "phase X dump must fit");
  static_assert(kFloats * 4 <= 160 * 1024, "LDS budget exceeded");
};

// Eight waves.  Phase V: per 16-column tile of d_v, waves 0-3 form R then E and
// waves 4-7 dE then G (one 16-row block each), then every wave accumulates its
// share of dA, dP (two 16x16 tiles each) and dKd, dQd, dKb (DK / 32 tiles each).
// Phase X/Y: thread (i, cg) = (tid / 8, tid % 8) owns row i, channels
// cg DK/8 .. + DK/8, for the elementwise terms and the pair sums.  Phase Z: thread
// c < DK forms channel c's reverse cumulative sum.
template <int DK, typename E>
__global__ __launch_bounds__(512) void kda_grad_kernel(KdaBwdParams p) {
  using L = GradLds<DK>;
  constexpr int LK = L::LK, L64 = L::L64, LT = L::LT;
  constexpr int CPT = DK / 8;         // channels per thread in the row phases
  constexpr int NK = DK / 32;         // dKd / dQd / dKb tiles per wave
  constexpr int VPR = 16 * static_cast<int>(sizeof(E)) / 16;  // io vectors per tile row
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));
  extern __shared__ __align__(16) float sg[];
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, col = lane & 15, g4 = lane >> 4, kq = g4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t r0 = 64LL * c;
  if (r0 >= len) return;
  const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
  const int H = p.H, Dv = p.Dv;
  const int64_t slot = bos / 64 + n + c;
  const float* const aux = p.aux + (slot * H + h) * static_cast<int64_t>(kda::Aux::kFloats);
  const float* const Sg = p.states + (slot * H + h) * static_cast<int64_t>(DK) * Dv;
  const float* const dSg = p.dstates + (slot * H + h) * static_cast<int64_t>(DK) * Dv;
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  const E* dO = static_cast<const E*>(p.dO);
  const int ri = tid >> 3, cg = tid & 7;   // row phases: row ri, channels cg CPT ..
  const int rowc = ri < nr ? ri : nr - 1;  // rows past the chunk load its last row and are zeroed

  // ---- stage 0: gamma, K o Gamma, K o exp(gamma_n - gamma), T, P, beta --------
  float* const kd = sg + L::kKd;
  float* const kb = sg + L::kKb;
  {
    const int64_t off = ((bos + r0 + rowc) * H + h) * DK + cg * CPT;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const float kv = IoT<E>::ld(k + off + e), gv = p.g[off + e];
      kd[ri * LK + cg * CPT + e] = ri < nr ? kv : 0.f;
      kb[ri * LK + cg * CPT + e] = ri < nr ? gv * chunk::kLog2e : 0.f;
    }
    for (int x = tid; x < 64 * 64; x += 512) {
      const int i = x >> 6, j = x & 63;
      sg[L::kT + i * L64 + j] = aux[kda::Aux::kT + x];
      sg[L::kP + i * L64 + j] = j <= i ? aux[kda::Aux::kP + x] : 0.f;
    }
    if (tid < 64) sg[L::kBe + tid] = tid < nr ? p.beta[(bos + r0 + tid) * H + h] : 0.f;
  }
  __syncthreads();
  if (tid < DK) {  // cumulative sum of channel tid over the chunk, in place (log2 units)
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) {
      acc += kb[i * LK + tid];
      kb[i * LK + tid] = acc;
    }
  }
  __syncthreads();
  {
    float kv[CPT], gv[CPT], gl[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      kv[e] = kd[ri * LK + cg * CPT + e];
      gv[e] = kb[ri * LK + cg * CPT + e];
      gl[e] = kb[63 * LK + cg * CPT + e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      kd[ri * LK + cg * CPT + e] = kv[e] * __builtin_amdgcn_exp2f(gv[e]);
      kb[ri * LK + cg * CPT + e] = kv[e] * __builtin_amdgcn_exp2f(gl[e] - gv[e]);
    }
  }

  // ---- phase V: the d_v tiles ----------------------------------------------
  float* const st = sg + L::kSt;
  float* const dst = sg + L::kDst;
  float* const vt = sg + L::kV;
  float* const dot = sg + L::kDo;
  float* const rt = sg + L::kR;
  float* const brt = sg + L::kBR;
  float* const et = sg + L::kE;
  float* const det = sg + L::kDe;
  float* const gt = sg + L::kG;
  const float* const be = sg + L::kBe;
  f32x4_t aA[2], aP[2], aKd[NK], aQd[NK], aKb[NK];
#pragma unroll
  for (int x = 0; x < 2; ++x) aA[x] = aP[x] = zero4();
#pragma unroll
  for (int x = 0; x < NK; ++x) aKd[x] = aQd[x] = aKb[x] = zero4();
  float dbv = 0.f;   // tid < 64: sum over d_v of G o R for row tid
  float dgn = 0.f;   // tid < DK: sum over d_v of dS' o S for channel tid

  // tile prefetch: S and dS' rows (four floats per vector), V and dO rows (io
  // vectors, bounded to the chunk's rows: past them the loads read zeros)
  const bool sl = tid < DK * 4;
  const int srow = sl ? tid >> 2 : 0, spart = tid & 3;
  const bool iol = tid < 64 * VPR;
  const int iorow = iol ? tid / VPR : 0, iopart = tid % VPR;
  const int vbytes = static_cast<int>(((nr - 1) * H * Dv + Dv) * sizeof(E));
  const auto rv = chunk::buffer_rsrc(v + ((bos + r0) * H + h) * Dv, vbytes);
  const auto rdo = chunk::buffer_rsrc(dO + ((bos + r0) * H + h) * Dv, vbytes);
  f32x4_t ps = zero4(), pds = zero4(), pv = zero4(), pdo = zero4();
  auto prefetch = [&](int t) {
    const int v0 = 16 * t;
    ps = *reinterpret_cast<const f32x4_t*>(Sg + srow * Dv + v0 + 4 * spart);
    pds = *reinterpret_cast<const f32x4_t*>(dSg + srow * Dv + v0 + 4 * spart);
    const int off = (iorow * H * Dv + v0 + iopart * EPV) * static_cast<int>(sizeof(E));
    pv = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    pdo = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
  };
  auto io_to_lds = [&](float* dstp, const f32x4_t& x, float mul) {
    if constexpr (sizeof(E) == 2) {
      const uint32_t* u = reinterpret_cast<const uint32_t*>(&x);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dstp[2 * e] = mul * __uint_as_float(u[e] << 16);
        dstp[2 * e + 1] = mul * __uint_as_float(u[e] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dstp[e] = mul * x[e];
    }
  };
  const int ntile = Dv / 16;
  prefetch(0);
  for (int t = 0; t < ntile; ++t) {
    const int v0 = 16 * t;
    __syncthreads();  // the previous tile's reads are done (and stage 0's writes visible)
    if (sl) {
      *reinterpret_cast<f32x4_t*>(st + srow * LT + 4 * spart) = ps;
      *reinterpret_cast<f32x4_t*>(dst + srow * LT + 4 * spart) = pds;
    }
    if (iol) {
      io_to_lds(vt + iorow * LT + iopart * EPV, pv, 1.f);
      io_to_lds(dot + iorow * LT + iopart * EPV, pdo, p.scale);
    }
    __syncthreads();
    if (t + 1 < ntile) prefetch(t + 1);
    if (w < 4) {  // R = V - Kd S and diag(beta) R (rows 16 w ..)
      f32x4_t acc = zero4();
      mm<DK, 1, LT>(acc, kd + (16 * w + col) * LK + kq, st + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g4 + r;
        const float rv2 = vt[row * LT + col] - acc[r];
        rt[row * LT + col] = rv2;
        brt[row * LT + col] = be[row] * rv2;
      }
    } else {  // dE = P^T dOs + Kb dS' (rows 16 (w - 4) ..)
      const int w4 = w - 4;
      f32x4_t acc = zero4();
      mm<64, L64, LT>(acc, sg + L::kP + kq * L64 + 16 * w4 + col, dot + kq * LT + col);
      mm<DK, 1, LT>(acc, kb + (16 * w4 + col) * LK + kq, dst + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) det[(16 * w4 + 4 * g4 + r) * LT + col] = acc[r];
    }
    __syncthreads();
    if (w < 4) {  // E = T diag(beta) R
      f32x4_t acc = zero4();
      mm<64, 1, LT>(acc, sg + L::kT + (16 * w + col) * L64 + kq, brt + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) et[(16 * w + 4 * g4 + r) * LT + col] = acc[r];
    } else {  // G = T^T dE; dv = diag(beta) G
      const int w4 = w - 4;
      f32x4_t acc = zero4();
      mm<64, L64, LT>(acc, sg + L::kT + kq * L64 + 16 * w4 + col, det + kq * LT + col);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w4 + 4 * g4 + r;
        gt[row * LT + col] = acc[r];
        if (row < nr) IoT<E>::st(static_cast<E*>(p.dv) + ((bos + r0 + row) * H + h) * Dv + v0 + col, be[row] * acc[r]);
      }
    }
    __syncthreads();
    // accumulations over this tile's 16 columns
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ta = 2 * w + x, ti = ta >> 2, tj = ta & 3;
      mm<16, 1, 1>(aA[x], gt + (16 * ti + col) * LT + kq, et + (16 * tj + col) * LT + kq);
      mm<16, 1, 1>(aP[x], dot + (16 * ti + col) * LT + kq, et + (16 * tj + col) * LT + kq);
    }
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int tk = NK * w + x, ti = tk / (DK / 16), tc = tk % (DK / 16);
      mm<16, 1, 1>(aKd[x], gt + (16 * ti + col) * LT + kq, st + (16 * tc + col) * LT + kq, be[16 * ti + col]);
      mm<16, 1, 1>(aQd[x], dot + (16 * ti + col) * LT + kq, st + (16 * tc + col) * LT + kq);
      mm<16, 1, 1>(aKb[x], et + (16 * ti + col) * LT + kq, dst + (16 * tc + col) * LT + kq);
    }
    if (tid < 64) {
#pragma unroll
      for (int j = 0; j < 16; ++j) dbv = fmaf(gt[tid * LT + j], rt[tid * LT + j], dbv);
    }
    if (tid < DK) {
#pragma unroll
      for (int j = 0; j < 16; ++j) dgn = fmaf(dst[tid * LT + j], st[tid * LT + j], dgn);
    }
  }
  __syncthreads();

  // ---- phase X: dKd = -F S^T, dQd = dOs S^T, dKb = E dS'^T to the row threads --
  float xKd[CPT], xQd[CPT], xKb[CPT];
  {
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int tk = NK * w + x, ti = tk / (DK / 16), tc = tk % (DK / 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ti + 4 * g4 + r, ch = 16 * tc + col;
        sg[row * LK + ch] = -aKd[x][r];
        sg[64 * LK + row * LK + ch] = aQd[x][r];
        sg[2 * 64 * LK + row * LK + ch] = aKb[x][r];
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const int ch = cg * CPT + e;
      xKd[e] = sg[ri * LK + ch];
      xQd[e] = sg[64 * LK + ri * LK + ch];
      xKb[e] = sg[2 * 64 * LK + ri * LK + ch];
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
      dA[i * L64 + j] = -aA[x][r];
      dP[i * L64 + j] = aP[x][r];
    }
  }
  {
    const int64_t off = ((bos + r0 + rowc) * H + h) * DK + cg * CPT;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      const bool ok = ri < nr;
      qs[ri * LK + cg * CPT + e] = ok ? IoT<E>::ld(q + off + e) : 0.f;
      ks[ri * LK + cg * CPT + e] = ok ? IoT<E>::ld(k + off + e) : 0.f;
      gs[ri * LK + cg * CPT + e] = ok ? p.g[off + e] * chunk::kLog2e : 0.f;
    }
    if (tid < 64) be2[tid] = tid < nr ? p.beta[(bos + r0 + tid) * H + h] : 0.f;
  }
  __syncthreads();
  if (tid < DK) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) {
      acc += gs[i * LK + tid];
      gs[i * LK + tid] = acc;
    }
  }
  __syncthreads();
  // dbeta (rows tid < 64): sum over d_v of G o R, plus sum_{j < i} dA_ij Ab_ij
  if (tid < 64) {
    float acc = dbv;
    for (int j = 0; j < tid; ++j) acc = fmaf(dA[tid * L64 + j], aux[kda::Aux::kAb + tid * 64 + j], acc);
    if (tid < nr) p.dbeta[(bos + r0 + tid) * H + h] = acc;
  }
  const float gnl = tid < DK ? gs[63 * LK + tid] : 0.f;  // gamma_n of channel tid (phase Z)
  float dgam[CPT], xx[CPT];
  {
    const float bi = be2[ri];
    E* const dqo = static_cast<E*>(p.dq) + ((bos + r0 + ri) * H + h) * DK + cg * CPT;
    E* const dko = static_cast<E*>(p.dk) + ((bos + r0 + ri) * H + h) * DK + cg * CPT;
    // eight channels at a time
#pragma unroll
    for (int e0 = 0; e0 < CPT; e0 += 8) {
      const int cb = cg * CPT + e0;
      float gi[8], kv[8], qv[8], dq8[8], dk8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gi[e] = gs[ri * LK + cb + e];
        kv[e] = ks[ri * LK + cb + e];
        qv[e] = qs[ri * LK + cb + e];
        const float gn = gs[63 * LK + cb + e];
        const float G = __builtin_amdgcn_exp2f(gi[e]), eb = __builtin_amdgcn_exp2f(gn - gi[e]);
        dq8[e] = xQd[e0 + e] * G;
        dk8[e] = xKd[e0 + e] * G + xKb[e0 + e] * eb;
        xx[e0 + e] = xKb[e0 + e] * kv[e] * eb;
        dgam[e0 + e] = (xKd[e0 + e] * kv[e] + xQd[e0 + e] * qv[e]) * G - xx[e0 + e];
      }
      // row side: j <= i
      float aq[8], ak[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) aq[e] = ak[e] = 0.f;
      for (int j = 0; j <= ri; ++j) {
        const float pij = dP[ri * L64 + j];
        const float aij = j < ri ? bi * dA[ri * L64 + j] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = ks[j * LK + cb + e] * __builtin_amdgcn_exp2f(gi[e] - gs[j * LK + cb + e]);
          aq[e] = fmaf(pij, t, aq[e]);
          ak[e] = fmaf(aij, t, ak[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dq8[e] += aq[e];
        dk8[e] += ak[e];
        dgam[e0 + e] += qv[e] * aq[e] + kv[e] * ak[e];
      }
      // column side: i' >= i
      float bp[8], ba[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bp[e] = ba[e] = 0.f;
      for (int i2 = ri; i2 < 64; ++i2) {
        const float pji = dP[i2 * L64 + ri];
        const float aji = i2 > ri ? be2[i2] * dA[i2 * L64 + ri] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = __builtin_amdgcn_exp2f(gs[i2 * LK + cb + e] - gi[e]);
          bp[e] = fmaf(pji, qs[i2 * LK + cb + e] * d, bp[e]);
          ba[e] = fmaf(aji, ks[i2 * LK + cb + e] * d, ba[e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dk8[e] += bp[e] + ba[e];
        dgam[e0 + e] -= kv[e] * (bp[e] + ba[e]);
      }
      if (ri < nr) {
        if constexpr (sizeof(E) == 2) {
          *reinterpret_cast<uint4*>(dqo + e0) = uint4{pack_bf16x2(dq8[0], dq8[1]), pack_bf16x2(dq8[2], dq8[3]),
                                                      pack_bf16x2(dq8[4], dq8[5]), pack_bf16x2(dq8[6], dq8[7])};
          *reinterpret_cast<uint4*>(dko + e0) = uint4{pack_bf16x2(dk8[0], dk8[1]), pack_bf16x2(dk8[2], dk8[3]),
                                                      pack_bf16x2(dk8[4], dk8[5]), pack_bf16x2(dk8[6], dk8[7])};
        } else {
          *reinterpret_cast<f32x4_t*>(dqo + e0) = f32x4_t{dq8[0], dq8[1], dq8[2], dq8[3]};
          *reinterpret_cast<f32x4_t*>(dqo + e0 + 4) = f32x4_t{dq8[4], dq8[5], dq8[6], dq8[7]};
          *reinterpret_cast<f32x4_t*>(dko + e0) = f32x4_t{dk8[0], dk8[1], dk8[2], dk8[3]};
          *reinterpret_cast<f32x4_t*>(dko + e0 + 4) = f32x4_t{dk8[4], dk8[5], dk8[6], dk8[7]};
        }
      }
    }
  }
  __syncthreads();

  // ---- phase Z: dg = reverse cumulative sum of dgamma, plus dgamma_n -----------
  float* const dgs = sg;             // [64][LK] dgamma
  float* const xs = sg + 64 * LK;    // [64][LK] dKb o Kb
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    dgs[ri * LK + cg * CPT + e] = dgam[e];
    xs[ri * LK + cg * CPT + e] = xx[e];
  }
  __syncthreads();
  if (tid < DK) {
    float acc = __builtin_amdgcn_exp2f(gnl) * dgn;
    for (int i = 0; i < 64; ++i) acc += xs[i * LK + tid];
    for (int s = 63; s >= 0; --s) {
      acc += dgs[s * LK + tid];
      if (s < nr) p.dg[((bos + r0 + s) * H + h) * DK + tid] = acc;
    }
  }
}

template <int DK, typename E>
hipError_t launch_kda_bwd_t(const KdaBwdParams& p, hipStream_t s) {
  using EL = std::conditional_t<sizeof(E) == 2, uint16_t, float>;
  constexpr size_t ds_smem = DsLds<DK, EL>::kBytes;
  constexpr size_t gr_smem = GradLds<DK>::kFloats * sizeof(float);
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
