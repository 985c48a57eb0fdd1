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
//   W = T diag(beta Gamma) K,  U = T diag(beta) V                [WY tensors w, u]
//   E = U - W S                 (the chunk's errors e_t: the "write" of the update)
//   P = lower_incl((Q K^T) o D)                                 [causal QK score]
//   O = scale (diag(Gamma) Q S + P E)
//   S <- Gamma_n S + K^T diag(exp(gamma_n - gamma)) E
// (intermediates named as on the fla issue #1550 page, "Intermediate rounding
// diagnosis").  Only exponents <= 0 are formed, so decays underflow to zero
// harmlessly and nothing is divided by a decay.
//
// Kernel 1, chunk_prep_kernel: one workgroup per (chunk, head, sequence), fully
//   parallel.  Computes A with MFMA and T = (I + A)^-1 in fp32 in LDS (16x16
//   diagonal blocks by forward substitution, the blocks below by
//   T_ij = -T_ii sum_k A_ik T_kj with fp32 MFMA), stores T (upper blocks zero)
//   in the workspace.
// Kernel 2, chunk_state_kernel: one workgroup per (sequence, head, 16-column
//   tile of d_v); column j of S only mixes with column j of v, so tiles are
//   independent.  Eight waves in two roles, pipelined one chunk apart:
//     producers (waves 4-7) turn chunk c+1 into W, U, P, K^T and the decays,
//       reading q/k/v/g/beta/T straight from HBM (one chunk of prefetch);
//     consumers (waves 0-3) hold the d_k x 16 fp32 slice of S in MFMA
//       accumulators and run chunk c: E = U - W S, O, and the state update.
//   Two workgroup barriers per chunk; the producer/consumer hand-off is
//   double-buffered where a buffer is read across the mid-chunk barrier.
//   Blocks are mapped so that the tiles of one head share an XCD (and its L2).
//
// Precision: bf16 io feeds bf16 MFMA operands (v_mfma_f32_16x16x32_bf16) with
// fp32 accumulation; S, gamma, the decays, A and the solve are fp32; T, W, U,
// P, E and the state operand are rounded to bf16 only as MFMA inputs.  fp32 io
// runs every product on v_mfma_f32_16x16x4_f32 (IEEE fp32).
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

// ===================================================================================
// Kernel 1: per-chunk T = (I + A)^-1
// ===================================================================================
template <int DK, typename Op>
struct PrepSmem {
  using E = typename Op::elem;
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;
  static constexpr int LDF = 64 + 4;
  static constexpr int LDM = 20;
  E Ks[64 * LDK];
  float Af[64 * LDF];
  float Tf[64 * LDF];
  float Mt[4 * 16 * LDM];
  float gam[64], bet[64];
};

template <int DK, typename Op>
__global__ __launch_bounds__(256) void chunk_prep_kernel(FwdParams p) {
  using E = typename Op::elem;
  using SM = PrepSmem<DK, Op>;
  constexpr int LDK = SM::LDK, LDF = SM::LDF, LDM = SM::LDM;
  constexpr int EPV = 16 / sizeof(E);
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, H = p.H;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t c0 = static_cast<int64_t>(c) * 64;
  if (c0 >= len) return;  // uniform over the workgroup
  const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
  const int64_t row0 = bos + c0;
  const int64_t slot = bos / 64 + n + c;
  E* Tout = static_cast<E*>(p.tws) + (slot * H + h) * 4096;
  const E* k = static_cast<const E*>(p.k);

  if (wave == 0) {
    const float gv = lane < nv ? p.g[(row0 + lane) * H + h] * kLog2e : 0.f;
    sm.gam[lane] = wave_inclusive_scan(gv, lane);  // gamma * log2(e)
  } else if (wave == 1) {
    sm.bet[lane] = lane < nv ? p.beta[(row0 + lane) * H + h] : 0.f;
  }
  constexpr int VPR = DK / EPV;
  for (int x = tid; x < 64 * VPR; x += 256) {
    const int t = x / VPR, cc = x % VPR;
    uint4 val = {0u, 0u, 0u, 0u};
    if (t < nv) val = *reinterpret_cast<const uint4*>(k + ((row0 + t) * H + h) * DK + cc * EPV);
    *reinterpret_cast<uint4*>(sm.Ks + t * LDK + cc * EPV) = val;
  }
  __syncthreads();

  // A = strict_lower(diag(beta) (K K^T) o D), fp32
  for (int b = wave; b < 10; b += 4) {
    int bi, bj;
    lower_block(b, bi, bj);
    f32x4_t acc = zero4();
    tile_mma<Op, DK>(acc, sm.Ks + 16 * bi * LDK, LDK, sm.Ks + 16 * bj * LDK, LDK, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * bi + 4 * (lane >> 4) + r, j = 16 * bj + (lane & 15);
      const float d = exp2f(fminf(sm.gam[i] - sm.gam[j], 0.f));
      sm.Af[i * LDF + j] = i > j ? sm.bet[i] * acc[r] * d : 0.f;
    }
  }
  __syncthreads();

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
    for (int r = 0; r < 16; ++r) sm.Tf[(16 * w + r) * LDF + 16 * w + cc] = tcol[r];
  }
  __syncthreads();
  // then the block diagonals below: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  for (int d = 1; d < 4; ++d) {
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

  // store T row-major, blocks above the diagonal as zeros
  constexpr int VPT = 64 / EPV;
  for (int x = tid; x < 64 * VPT; x += 256) {
    const int i = x / VPT, jb = (x % VPT) * EPV;
    E vals[EPV];
#pragma unroll
    for (int m = 0; m < EPV; ++m) {
      const int j = jb + m;
      vals[m] = Op::cvt((j >> 4) <= (i >> 4) ? sm.Tf[i * LDF + j] : 0.f);
    }
    *reinterpret_cast<uint4*>(Tout + i * 64 + jb) = *reinterpret_cast<const uint4*>(vals);
  }
}

// ===================================================================================
// Kernel 2: the state pass with output, producer/consumer waves
// ===================================================================================
template <int DK, typename Op>
struct StateSmem {
  using E = typename Op::elem;
  static constexpr int PADE = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LDK = DK + PADE;  // rows of length d_k
  static constexpr int LDC = 64 + PADE;  // rows of length 64 (one chunk)
  // producer -> consumer
  E Ws[64 * LDK];           // W, token-major (consumers read it before the mid barrier)
  E Pm[64 * LDC];           // P, row-major; upper blocks stay zero
  E Kt[2][DK * LDC];        // K^T, d_k-major (consumers read it after the mid barrier)
  float Us[4 * 64 * 4];     // U in the consumers' accumulator order [row block][lane][r]
  float Gam[2][64];         // exp(gamma)
  float Dec[2][64];         // exp(gamma_n - gamma)
  // producer private
  E Ks[64 * LDK];           // K, token-major
  E Qs[2][64 * LDK];        // Q, token-major: staged by the consumers one chunk ahead
  E Vt[16 * LDC];           // V tile transposed
  E Tm[64 * LDC];           // T of the chunk being prepared (row-major, upper blocks zero)
  float gam[64], bg[64], bet[64];
  // consumer private
  E St[16 * LDK];           // S^T (16 columns x d_k)
  E Et[16 * LDC];           // E^T
  E Ett[16 * LDC];          // (diag(exp(gamma_n - gamma)) E)^T
};

template <int DK, typename Op>
__global__ __launch_bounds__(512) void chunk_state_kernel(FwdParams p) {
  using E = typename Op::elem;
  using F = typename Op::frag_t;
  using SM = StateSmem<DK, Op>;
  constexpr int LDK = SM::LDK, LDC = SM::LDC;
  constexpr int KS = Op::KSTEP;
  constexpr int NKQ = DK / KS;               // k-steps over d_k
  constexpr int SRB = DK / 64;               // 16-row blocks of S per consumer wave
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));
  constexpr int EPT = DK / 8;                // k/q elements per producer thread per token
  constexpr int UPT = EPT / EPV;             // 16-byte vectors per token
  constexpr int NVS = 16 / EPV;              // 16-byte vectors per row of a v tile
  static_assert(EPT % EPV == 0, "thread slice must be whole vectors");
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool consumer = wave < 4;
  const int w = wave & 3;
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
  const bool write_o = p.write_o == kOutAll || (p.write_o == kOutSeg0 && seg == 0);
  const bool use_v = !p.zero_u;
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);
  const E* v = static_cast<const E*>(p.v);
  const E* tws = static_cast<const E*>(p.tws);
  E* o = static_cast<E*>(p.o);
  const int64_t nhS = (static_cast<int64_t>(n) * H + h) * DK;
  const int64_t segS = (static_cast<int64_t>(seg) * p.N * H + nh) * DK;  // [G][N][H][DK][NC] buffers

  // upper blocks of P are never written
  for (int x = tid; x < 64 * LDC; x += 512) {
    const int i = x / LDC, j = x % LDC;
    if ((j >> 4) > (i >> 4)) sm.Pm[x] = Op::cvt(0.f);
  }

  if (consumer) {
    // ===================== consumers: the state recurrence =====================
    // Besides the recurrence of chunk s-1, the consumers stage Q of chunk s
    // (first half) and compute its causal score P (second half).
    f32x4_t Sacc[SRB];
    const int tp = tid & 31, ds = tid >> 5;
    u32x4_t qreg[2 * UPT];
    auto load_q = [&](int c) {  // rows of Q of chunk c (clamped into the sequence)
      const int64_t c0 = static_cast<int64_t>(cb + c) * 64;
      const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const E* qr = q + ((bos + c0 + min(2 * tp + tt, nv - 1)) * H + h) * DK + ds * EPT;
#pragma unroll
        for (int u = 0; u < UPT; ++u) qreg[tt * UPT + u] = *reinterpret_cast<const u32x4_t*>(qr + u * EPV);
      }
    };
    if (nch > 0 && write_o) load_q(0);
#pragma unroll
    for (int sr = 0; sr < SRB; ++sr) {
      const int i = 16 * (w * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (p.start_mode == kStartCarry)
          x[r] = p.carry[(segS + i + r) * NC + j0 + j];
        else if (p.start_mode == kStartIdentity)
          x[r] = i + r == j0 + j ? 1.f : 0.f;
        else if (p.start_mode == kStartS0 && seg == 0 && p.S0)
          x[r] = p.S0[(nhS + i + r) * Dv + j0 + j];
        else
          x[r] = 0.f;
      }
      Sacc[sr] = f32x4_t{x[0], x[1], x[2], x[3]};
      store4<E>(sm.St + j * LDK + i, x[0], x[1], x[2], x[3]);
    }
    __syncthreads();
    for (int s = 0; s <= nch; ++s) {
      f32x4_t yacc = zero4();
      F pf[tsteps<Op>(3)];
      float gam_o = 0.f, gam_n = 0.f;
      const int c = s - 1, b = c & 1;
      if (s < nch && write_o) {  // stage Q of chunk s, padded rows as zeros; prefetch the next
        const int64_t cs0 = static_cast<int64_t>(cb + s) * 64;
        const int nv = static_cast<int>(len - cs0 < 64 ? len - cs0 : 64);
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * tp + tt;
#pragma unroll
          for (int u = 0; u < UPT; ++u)
            *reinterpret_cast<u32x4_t*>(sm.Qs[s & 1] + t * LDK + ds * EPT + u * EPV) =
                t < nv ? qreg[tt * UPT + u] : z;
        }
        load_q(s + 1 < nch ? s + 1 : s);
      }
      if (s >= 1) {
        if (p.states) {  // S_c, the state before chunk c, kept for the backward
          float* dst = p.states + ((slot0 + c) * H + h) * static_cast<int64_t>(DK) * Dv;
#pragma unroll
          for (int sr = 0; sr < SRB; ++sr) {
            const int i = 16 * (w * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[static_cast<int64_t>(i + r) * Dv + j0 + j] = Sacc[sr][r];
          }
        }
        // X = W S (rows of this wave), Y^T = S^T Q^T
        f32x4_t xacc = zero4();
#pragma unroll
        for (int ks = 0; ks < NKQ; ++ks) {
          const F st = Op::frag(sm.St, LDK, lane, ks * KS);
          xacc = Op::mma(Op::frag(sm.Ws + 16 * w * LDK, LDK, lane, ks * KS), st, xacc);
          if (write_o) yacc = Op::mma(st, Op::frag(sm.Qs[b] + 16 * w * LDK, LDK, lane, ks * KS), yacc);
        }
        // E = U - X; E^T and the decayed E^T go to LDS for every consumer
        const float4 u = use_v ? *reinterpret_cast<const float4*>(sm.Us + (w * 64 + lane) * 4)
                               : float4{0.f, 0.f, 0.f, 0.f};
        const float uu[4] = {u.x, u.y, u.z, u.w};
        const int t0 = 16 * w + 4 * (lane >> 4), j = lane & 15;
        float e[4], ed[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = uu[r] - xacc[r];
          ed[r] = e[r] * sm.Dec[b][t0 + r];
        }
        store4<E>(sm.Et + j * LDC + t0, e[0], e[1], e[2], e[3]);
        store4<E>(sm.Ett + j * LDC + t0, ed[0], ed[1], ed[2], ed[3]);
        // this wave's rows of P and the decays it needs after the barrier
#pragma unroll
        for (int ks = 0; ks < tsteps<Op>(3); ++ks)
          pf[ks] = write_o && ks < tsteps<Op>(w) ? Op::frag(sm.Pm + 16 * w * LDC, LDC, lane, ks * KS) : F{};
        gam_o = sm.Gam[b][16 * w + (lane & 15)];
        gam_n = sm.Gam[b][63];
      }
      __syncthreads();
      if (s >= 1) {
        const int64_t c0 = static_cast<int64_t>(cb + c) * 64;
        const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
        // O^T = E^T P^T + Y^T scaled by Gamma  (rows j, columns t)
        f32x4_t oacc = zero4();
#pragma unroll
        for (int ks = 0; ks < tsteps<Op>(3); ++ks)
          oacc = Op::mma(Op::frag(sm.Et, LDC, lane, ks * KS), pf[ks], oacc);
        const int t = 16 * w + (lane & 15), jj = 4 * (lane >> 4);
        if (write_o && t < nv) {
          E* dst = o + ((bos + c0 + t) * H + h) * Dv + j0 + jj;
          store4<E>(dst, p.scale * (gam_o * yacc[0] + oacc[0]), p.scale * (gam_o * yacc[1] + oacc[1]),
                    p.scale * (gam_o * yacc[2] + oacc[2]), p.scale * (gam_o * yacc[3] + oacc[3]));
        }
        // S <- Gamma_n S + K^T (decayed E)
#pragma unroll
        for (int sr = 0; sr < SRB; ++sr) {
          const int sb = w * SRB + sr;
          f32x4_t acc = Sacc[sr] * gam_n;
#pragma unroll
          for (int ks = 0; ks < 64 / KS; ++ks)
            acc = Op::mma(Op::frag(sm.Kt[b] + 16 * sb * LDC, LDC, lane, ks * KS),
                          Op::frag(sm.Ett, LDC, lane, ks * KS), acc);
          Sacc[sr] = acc;
          store4<E>(sm.St + (lane & 15) * LDK + 16 * sb + 4 * (lane >> 4), acc[0], acc[1], acc[2], acc[3]);
        }
      }
      if (s < nch && write_o) {
        // P = lower_incl(Q K^T o D) of chunk s, computed transposed so rows of P
        // store contiguously.  Blocks (bi, bj) by wave:
        //   0: (0,0) (1,0) (1,1)   1: (2,0) (2,1) (2,2)   2: (3,0) (3,1)   3: (3,2) (3,3)
        const int bq = s & 1;
        auto pblock = [&](int bi, int bj) {
          f32x4_t acc = zero4();
          tile_mma<Op, DK>(acc, sm.Ks + 16 * bj * LDK, LDK, sm.Qs[bq] + 16 * bi * LDK, LDK, lane);
          const int i = 16 * bi + (lane & 15), jb = 16 * bj + 4 * (lane >> 4);
          const float gi = sm.gam[i];
          const float4 gj = *reinterpret_cast<const float4*>(sm.gam + jb);
          const float gjj[4] = {gj.x, gj.y, gj.z, gj.w};
          float pv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float d = exp2f(fminf(gi - gjj[r], 0.f));
            pv[r] = jb + r <= i ? acc[r] * d : 0.f;
          }
          store4<E>(sm.Pm + i * LDC + jb, pv[0], pv[1], pv[2], pv[3]);
        };
        if (w == 0) {
          pblock(0, 0); pblock(1, 0); pblock(1, 1);
        } else if (w == 1) {
          pblock(2, 0); pblock(2, 1); pblock(2, 2);
        } else if (w == 2) {
          pblock(3, 0); pblock(3, 1);
        } else {
          pblock(3, 2); pblock(3, 3);
        }
      }
      __syncthreads();
    }
    const bool to_final = p.final_to_sfinal && seg == p.G - 1;
    if (to_final ? p.S_final != nullptr : p.seg_out != nullptr) {
#pragma unroll
      for (int sr = 0; sr < SRB; ++sr) {
        const int i = 16 * (w * SRB + sr) + 4 * (lane >> 4), j = lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (to_final)
            p.S_final[(nhS + i + r) * Dv + j0 + j] = Sacc[sr][r];
          else
            p.seg_out[(segS + i + r) * NC + j0 + j] = Sacc[sr][r];
        }
      }
    }
  } else {
    // ===================== producers: chunk c+1 while consumers run chunk c =====================
    // Prefetches are issued one chunk ahead and unconditionally (rows clamped
    // into the sequence, padded rows zeroed when used), so the compiler can wait
    // for exactly the loads it needs.
    const int ptid = tid - 256, tp = ptid & 31, ds = ptid >> 5;
    u32x4_t kreg[2 * UPT], vreg[2];
    float greg = 0.f, breg = 0.f;
    // W and U work split by row blocks of T: waves 0, 1 take row blocks {0, 3},
    // waves 2, 3 take {1, 2} (three k-steps each), each wave half of W's columns.
    constexpr int TS = tsteps<Op>(3);
    constexpr int TPT = 64 * 64 / 256 / EPV;  // 16-byte vectors of T per producer thread
    u32x4_t treg[TPT];
    auto for_rowblocks = [&](auto&& fn) {  // fn(integral_constant<R0>, integral_constant<R1>)
      if (w < 2)
        fn(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
      else
        fn(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    };
    auto load_chunk = [&](int c) {  // raw rows of chunk c and its T into registers
      const int64_t c0 = static_cast<int64_t>(cb + c) * 64;
      const int64_t row0 = bos + c0;
      const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = min(2 * tp + tt, nv - 1);
        const E* kr = k + ((row0 + t) * H + h) * DK + ds * EPT;
#pragma unroll
        for (int u = 0; u < UPT; ++u) kreg[tt * UPT + u] = *reinterpret_cast<const u32x4_t*>(kr + u * EPV);
        if (use_v && w < NVS / 2)  // wave-uniform: the threads that store the v tile
          vreg[tt] = *reinterpret_cast<const u32x4_t*>(v + ((row0 + t) * H + h) * Dv + j0 + ds * EPV);
      }
      if (w == 0) {
        const int tl = min(lane, nv - 1);
        greg = p.g[(row0 + tl) * H + h];
        breg = p.beta[(row0 + tl) * H + h];
      }
      const E* T = tws + ((slot0 + c) * H + h) * 4096 + ptid * TPT * EPV;
#pragma unroll
      for (int x = 0; x < TPT; ++x) treg[x] = *reinterpret_cast<const u32x4_t*>(T + x * EPV);
    };
    // One pipeline step: stage chunk s in LDS (first half), then build its W, U
    // and P (second half).  Every prefetched register is consumed in the first
    // half, before the next chunk's loads are issued into it, so the loads stay
    // in flight across a whole step.
    auto step = [&](int s) {
      const int b = s & 1;
      if (s < nch) {
        const int64_t c0 = static_cast<int64_t>(cb + s) * 64;
        const int nv = static_cast<int>(len - c0 < 64 ? len - c0 : 64);
        const u32x4_t z = {0u, 0u, 0u, 0u};
        // rows of chunk s: K, Q token-major; K^T; V^T (padded rows as zeros)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * tp + tt;
          const bool ok = t < nv;
#pragma unroll
          for (int u = 0; u < UPT; ++u) {
            kreg[tt * UPT + u] = ok ? kreg[tt * UPT + u] : z;
            *reinterpret_cast<u32x4_t*>(sm.Ks + t * LDK + ds * EPT + u * EPV) = kreg[tt * UPT + u];
          }
          vreg[tt] = ok ? vreg[tt] : z;
        }
        {
          E* kt = sm.Kt[b] + (ds * EPT) * LDC + 2 * tp;
#pragma unroll
          for (int e = 0; e < EPT; ++e)
            Pair<E>::store(kt + e * LDC, kreg[e / EPV], kreg[UPT + e / EPV], e % EPV);
        }
        if (ptid < 32 * NVS) {
          E* vt = sm.Vt + (ds * EPV) * LDC + 2 * tp;
#pragma unroll
          for (int e = 0; e < EPV; ++e) Pair<E>::store(vt + e * LDC, vreg[0], vreg[1], e);
        }
#pragma unroll
        for (int x = 0; x < TPT; ++x) {
          const int e0 = (ptid * TPT + x) * EPV;  // element of the 64 x 64 T
          *reinterpret_cast<u32x4_t*>(sm.Tm + (e0 / 64) * LDC + e0 % 64) = treg[x];
        }
        if (w == 0) {
          // gamma by an in-register scan; decays as exp2 of log2(e)-scaled values
          const bool ok = lane < nv;
          const float g2 = wave_inclusive_scan(ok ? greg * kLog2e : 0.f, lane);
          const float gl2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2), 63));
          const float G = exp2f(g2);
          const float bt = ok ? breg : 0.f;
          sm.gam[lane] = g2;
          sm.Gam[b][lane] = G;
          sm.Dec[b][lane] = exp2f(gl2 - g2);
          sm.bet[lane] = bt;
          sm.bg[lane] = bt * G;
        }
        load_chunk(s + 1 < nch ? s + 1 : s);
      }
      __syncthreads();
      if (s < nch) {
        // W^T = K^T (T diag(beta Gamma))^T, transposed so rows of W store contiguously;
        // U = T diag(beta) V for one row block, in the consumers' accumulator order
        for_rowblocks([&](auto R0, auto R1) {
          constexpr int rb[2] = {decltype(R0)::value, decltype(R1)::value};
          constexpr int NCW = DK / 32;  // 16-column blocks of W per wave
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int ri = rb[x];
            F tw[TS];
#pragma unroll
            for (int ks = 0; ks < tsteps<Op>(rb[x]); ++ks)
              tw[ks] = Op::scale(Op::frag(sm.Tm + 16 * rb[x] * LDC, LDC, lane, ks * KS), sm.bg, lane, ks * KS);
#pragma unroll
            for (int cj = 0; cj < NCW; ++cj) {
              const int cw = (w & 1) * NCW + cj;
              f32x4_t acc = zero4();
#pragma unroll
              for (int ks = 0; ks < tsteps<Op>(rb[x]); ++ks)
                acc = Op::mma(Op::frag(sm.Kt[b] + 16 * cw * LDC, LDC, lane, ks * KS), tw[ks], acc);
              store4<E>(sm.Ws + (16 * ri + (lane & 15)) * LDK + 16 * cw + 4 * (lane >> 4), acc[0],
                        acc[1], acc[2], acc[3]);
            }
          }
          if (!use_v) return;  // transition maps: U = 0, read as zeros by the consumers
          const int x = w & 1;
          const int ri = x ? rb[1] : rb[0];
          f32x4_t acc = zero4();
          if (x == 0) {
#pragma unroll
            for (int ks = 0; ks < tsteps<Op>(rb[0]); ++ks)
              acc = Op::mma(Op::scale(Op::frag(sm.Tm + 16 * rb[0] * LDC, LDC, lane, ks * KS), sm.bet, lane, ks * KS),
                            Op::frag(sm.Vt, LDC, lane, ks * KS), acc);
          } else {
#pragma unroll
            for (int ks = 0; ks < tsteps<Op>(rb[1]); ++ks)
              acc = Op::mma(Op::scale(Op::frag(sm.Tm + 16 * rb[1] * LDC, LDC, lane, ks * KS), sm.bet, lane, ks * KS),
                            Op::frag(sm.Vt, LDC, lane, ks * KS), acc);
          }
          *reinterpret_cast<float4*>(sm.Us + (ri * 64 + lane) * 4) = float4{acc[0], acc[1], acc[2], acc[3]};
        });
      }
      __syncthreads();
    };
    if (nch > 0) load_chunk(0);
    __syncthreads();
    for (int s = 0; s <= nch; ++s) step(s);
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

template <int DK, typename Op>
hipError_t set_fwd_attributes() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_prep_kernel<DK, Op>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(sizeof(PrepSmem<DK, Op>)));
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_state_kernel<DK, Op>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(sizeof(StateSmem<DK, Op>)));
}

template <int DK, typename Op>
hipError_t launch_states_t(const FwdParams& p, hipStream_t s) {
  hipError_t e = set_fwd_attributes<DK, Op>();
  if (e != hipSuccess) return e;
  if (p.max_chunks == 0) return hipSuccess;
  auto prep = chunk_prep_kernel<DK, Op>;
  auto state = chunk_state_kernel<DK, Op>;
  constexpr size_t prep_smem = sizeof(PrepSmem<DK, Op>);
  constexpr size_t state_smem = sizeof(StateSmem<DK, Op>);
  hipLaunchKernelGGL(prep, dim3(p.max_chunks, p.H, p.N), dim3(256), prep_smem, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  FwdParams q = p;
  q.G = 1; q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = kOutNone;
  q.zero_u = 0; q.ncol = p.Dv; q.carry = nullptr; q.seg_out = nullptr; q.final_to_sfinal = 0;
  q.S_final = nullptr;
  hipLaunchKernelGGL(state, dim3(p.N * p.H * (p.Dv / 16)), dim3(512), state_smem, s, q);
  return hipGetLastError();
}

template <int DK, typename Op>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  constexpr size_t prep_smem = sizeof(PrepSmem<DK, Op>);
  constexpr size_t state_smem = sizeof(StateSmem<DK, Op>);
  static_assert(prep_smem <= 160 * 1024 && state_smem <= 160 * 1024, "LDS budget exceeded");
  auto prep = chunk_prep_kernel<DK, Op>;
  auto state = chunk_state_kernel<DK, Op>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(prep_smem));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(state),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(state_smem));
  if (e != hipSuccess) return e;
  if (p.max_chunks > 0) {
    hipLaunchKernelGGL(prep, dim3(p.max_chunks, p.H, p.N), dim3(256), prep_smem, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto run_state = [&](const FwdParams& q) {
    hipLaunchKernelGGL(state, dim3(q.nseg * q.N * q.H * (q.ncol / 16)), dim3(512), state_smem, s, q);
    return hipGetLastError();
  };
  FwdParams q = p;
  q.ncol = p.Dv;
  q.zero_u = 0;
  q.carry = nullptr;
  if (p.G == 1) {
    q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = kOutAll;
    q.seg_out = nullptr; q.final_to_sfinal = 1;
    return run_state(q);
  }
  // G segments per sequence: (1) segment 0 from S0 with its outputs, and the
  // segments 1 .. G-2 from zero (their offsets b); (2) the transition maps M of
  // segments 1 .. G-2 (the same pass with U = 0, started from the identity);
  // (3) the carries; (4) segments 1 .. G-1 again from their carried start states.
  const size_t ends_floats = static_cast<size_t>(p.G) * p.N * p.H * DK * p.Dv;
  float* ends = p.seg_ws;
  float* starts = ends + ends_floats;
  float* maps = starts + ends_floats;
  q.seg_base = 0; q.nseg = p.G - 1; q.start_mode = kStartS0; q.write_o = kOutSeg0;
  q.seg_out = ends; q.final_to_sfinal = 0;
  if ((e = run_state(q)) != hipSuccess) return e;
  if (p.G > 2) {
    FwdParams m = q;
    m.ncol = DK; m.seg_base = 1; m.nseg = p.G - 2; m.start_mode = kStartIdentity;
    m.write_o = kOutNone; m.zero_u = 1; m.seg_out = maps;
    if ((e = run_state(m)) != hipSuccess) return e;
  }
  CarryParams c{ends, maps, starts, p.G, p.N, p.H, DK, p.Dv};
  hipLaunchKernelGGL(seg_carry_kernel<DK>, dim3(p.N * p.H * (p.Dv / 16)), dim3(256), 0, s, c);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  q.seg_base = 1; q.nseg = p.G - 1; q.start_mode = kStartCarry; q.write_o = kOutAll;
  q.carry = starts; q.seg_out = nullptr; q.final_to_sfinal = 1;
  return run_state(q);
}

}  // namespace

hipError_t launch_chunk_fwd_states(const FwdParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_states_t<64, OpBf16>(p, s);
    if (Dk == 128) return launch_states_t<128, OpBf16>(p, s);
  } else {
    if (Dk == 64) return launch_states_t<64, OpF32>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const FwdParams& p, int Dk, bool bf16, hipStream_t s) {
  if (bf16) {
    if (Dk == 64) return launch_fwd_t<64, OpBf16>(p, s);
    if (Dk == 128) return launch_fwd_t<128, OpBf16>(p, s);
  } else {
    if (Dk == 64) return launch_fwd_t<64, OpF32>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
