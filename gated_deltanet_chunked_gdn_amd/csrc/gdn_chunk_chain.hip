// State pass of the chunked forward for bf16 io on gfx950: the whole per-chunk
// recurrence of one 16-column tile of the state runs in one wave, in registers.
//
// Per chunk (64 tokens; rows of padded tokens carry k = v = 0 and change nothing),
// with S the state before the chunk (d_k x d_v; "Research Sprint Day 1", section
// "The GDN update", applied token by token, gates as cumulative log decays per the
// "Research Sprint Day 2" page, "Building some intuition"):
//   Z = K S,  R = V - diag(Gamma) Z,  E = (T diag(beta)) R       (the chunk's errors)
//   S <- Gamma_n S + K^T diag(exp(gamma_n - gamma)) E
//   O = scale (diag(Gamma) Q S + P E)
// T diag(beta), P and the decays come from the per-chunk preparation kernel.
//
// Register layout.  A 16x16 fp32 MFMA accumulator holds, in lane (j, g) = (lane %
// 16, lane / 16), rows 4g + r (r = 0..3) of column j, and a B operand of
// v_mfma_f32_16x16x32_bf16 holds reduction rows 8g + 0..7 of column j.  Pairing
// the 16-row blocks 2s and 2s + 1 and giving row 4g + r of block b the index
//   tau(b, g, r) = 32 (b / 2) + 8 g + 4 (b % 2) + r
// makes the two accumulators of a pair exactly the B operand of reduction step s
// (indices 32 s + 8 g + 0..7, in order).  So every product's result feeds the next
// one without leaving the registers: S (rows of d_k in tau order) -> Z, R, E (token
// rows in tau order) -> the state update, whose A operand K^T is read with its rows
// in tau order by ds_read_b64_tr_b16 from the K rows staged in LDS.  Operands read
// from memory absorb the order: the Z operand reads K rows tau(mb, m), T diag(beta)
// is stored by the preparation kernel as operand fragments with rows in tau order.
//
// Waves of a workgroup (one workgroup per (segment, sequence, head, 16-column tile)):
//   waves 0-1 (state): the recurrence of chunk c, split by halves of d_k: wave h
//                      holds rows [d_k h / 2, d_k (h + 1) / 2) of the tile of S,
//                      forms its partial Z, and the two partials are summed through
//                      LDS; both waves then form R and E, and each updates its half
//                      of S.  They hand S_c and E_c to wave 2;
//   waves 2-3 (output): O of chunk c - 1 as O^T = scale (Gamma o (S^T Q^T) + E^T P^T),
//                      token row blocks 0-1 and 2-3, with Q and P loaded from memory
//                      straight into operand fragments;
//   waves 4-5:         stage K, the v tile (transposed, fp32), T diag(beta) and the
//                      decays of chunk c + 1 into the LDS ring and load chunk c + 3.
// A pass without outputs (the backward's state pass, the segment maps) has four
// waves, the state and staging waves, and no hand-off buffers.
// Two workgroup barriers per chunk: X (the partial Z exchanged) and Y (end of step);
// the output and staging work is spread over both intervals.  (Waves are placed on
// the SIMDs round robin: each state wave shares its SIMD with a staging wave.)
#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace chunk;

__device__ __forceinline__ int tau(int b, int g, int r) { return 32 * (b >> 1) + 8 * g + 4 * (b & 1) + r; }

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load1(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// An offset every buffer range check rejects: the load returns zeros.
constexpr int kNoLoad = 0x7ffffff0;

// Two accumulators (blocks 2s, 2s + 1) as one bf16 operand fragment (RNE).
__device__ __forceinline__ bf16x8_t pack_pair(const f32x4_t& a, const f32x4_t& b) {
  const uint4 u{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ f32x4_t mma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K rows in LDS, swizzled: row t holds its 16-byte pieces u (8 bf16 each) at piece
// u ^ ksw(t), chosen so that the row-fragment reads of Z (one piece of the 16 rows
// tau(mb, m) per 16-lane group) and the transposed reads of the update (4
// consecutive rows x 4 pieces per 16-lane group) each touch distinct 16-byte bank
// groups: with 16 pieces per row ksw(t) = 4 (t % 4) + (t / 8) % 4; with 8 pieces
// (rows of 128 bytes, two rows per bank cycle) ksw(t) = 4 ((t / 2) % 2) + (t / 8) % 4.
template <int DK>
__device__ __forceinline__ int ksw(int t) {
  if constexpr (DK == 128) return 4 * (t & 3) + ((t >> 3) & 3);
  else return 4 * ((t >> 1) & 1) + ((t >> 3) & 3);
}
// bf16 offset of piece u (0 .. DK / 8 - 1) of row t
template <int DK>
__device__ __forceinline__ int kpos(int t, int u) { return t * DK + 8 * (u ^ ksw<DK>(t)); }

// LDS of the state pass; without outputs (OUT false) there are no output waves and
// no hand-off buffers for them.
template <int DK, bool OUT>
struct ChainSmem {
  static constexpr int LDV = 64 + 4;  // rows of the transposed v tile
  static constexpr int NKS = DK / 32;
  alignas(16) uint16_t Ks[2][64 * DK];          // K rows, swizzled pieces (kpos)
  alignas(16) float Vt[2][16 * LDV];            // the v tile, transposed (fp32)
  alignas(16) float Gs[2][128];                 // Gamma, exp(gamma_n - gamma)
  alignas(16) bf16x8_t Tb[2][6][64];            // T diag(beta) operand fragments
  alignas(16) bf16x8_t hand[OUT ? 3 : 1][OUT ? NKS : 1][OUT ? 64 : 1];  // S_c operand fragments (ring of 3:
                                                // S_c is written in step c - 1, read in step c + 1)
  alignas(16) f32x4_t handE[OUT ? 2 : 1][OUT ? 4 : 1][OUT ? 64 : 1];    // E_c (fp32, accumulator layout)
  alignas(16) f32x4_t zx[2][4][64];             // partial Z of each state wave
};

// At d_k = 64 the register budget is held to 128 so that two workgroups share a
// CU (grids of many heads run several workgroups per CU); at d_k = 128 the chain
// needs ~170 registers and the train shapes run one workgroup per CU anyway.
template <int DK, bool STATES, bool OUT>
__global__ __launch_bounds__(384) __attribute__((amdgpu_waves_per_eu(DK == 64 ? 4 : 1))) void chunk_chain_kernel(
    FwdParams p) {
  using SM = ChainSmem<DK, OUT>;
  constexpr int LDV = SM::LDV;
  constexpr int NKS = DK / 32;  // reduction steps over d_k
  constexpr int HS = NKS / 2;   // ... over the half of d_k a state wave holds
  constexpr int HB = DK / 32;   // 16-row blocks of S per state wave
  extern __shared__ __align__(16) char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ k = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ v = static_cast<const uint16_t*>(p.v);
  const uint16_t* __restrict__ tbw = static_cast<const uint16_t*>(p.tbws);
  const uint16_t* __restrict__ pw = static_cast<const uint16_t*>(p.pws);
  const float* __restrict__ gw = p.gws;
  uint16_t* __restrict__ o = static_cast<uint16_t*>(p.o);

  const int H = p.H, Dv = p.Dv, NC = p.ncol, NT = NC / 16;
  // XCD-aware order: the workgroups of one head land on one XCD (blockIdx % 8),
  // whose L2 then serves their shared per-chunk reads.
  const int NB = gridDim.x, L = blockIdx.x;
  const int vb = (NB % 8 == 0) ? (L % 8) * (NB / 8) + L / 8 : L;
  const int tile = vb % NT, nh = (vb / NT) % (p.N * H), h = nh % H, n = nh / H;
  const int seg = p.seg_base + vb / NT / (p.N * H);
  const int j0 = tile * 16;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int nch_all = static_cast<int>((len + 63) / 64);
  const int seg_len = (nch_all + p.G - 1) / p.G;
  const int cb = min(seg * seg_len, nch_all);
  const int nch = min(cb + seg_len, nch_all) - cb;
  const int64_t slot0 = bos / 64 + n + cb;
  const bool store_o = p.write_o == kOutAll || (p.write_o == kOutSeg0 && seg == 0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t nhS = (static_cast<int64_t>(n) * H + h) * DK;
  const int64_t segS = (static_cast<int64_t>(seg) * p.N * H + nh) * DK;

  auto chunk_rows = [&](int c) {
    const int64_t c0 = static_cast<int64_t>(cb + c) * 64;
    return static_cast<int>(len - c0 < 64 ? len - c0 : 64);
  };
  auto clampc = [&](int c) { return c < nch ? c : nch - 1; };
  auto row0_of = [&](int c) { return bos + static_cast<int64_t>(cb + c) * 64; };
  const int nsteps = (nch + 1) / 2 * 2;

  if (w < 2) {
    // ================= state waves: half hh of d_k =================
    const int hh = w;
    // S: blocks hh HB .. hh HB + HB - 1 of the d_k x 16 fp32 tile (rows in tau order)
    f32x4_t S[HB];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = tau(hh * HB + i, lg, r), j = j0 + lr;
        float x;
        if (p.start_mode == kStartCarry)
          x = p.carry[(segS + d) * NC + j];
        else if (p.start_mode == kStartIdentity)
          x = d == j ? 1.f : 0.f;
        else if (p.start_mode == kStartS0 && seg == 0 && p.S0)
          x = p.S0[(nhS + d) * Dv + j];
        else
          x = 0.f;
        S[i][r] = x;
      }
    }
    auto write_state = [&]() {
      const bool to_final = p.final_to_sfinal && seg == p.G - 1;
      if (to_final ? p.S_final != nullptr : p.seg_out != nullptr) {
#pragma unroll
        for (int i = 0; i < HB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int d = tau(hh * HB + i, lg, r), j = j0 + lr;
            if (to_final)
              p.S_final[(nhS + d) * Dv + j] = S[i][r];
            else
              p.seg_out[(segS + d) * NC + j] = S[i][r];
          }
      }
    };
    if (nch == 0) {
      write_state();
      return;
    }
    // Sf[i]: the B operand of reduction step hh HS + i (rows 32 s + 8 g + 0..7)
    bf16x8_t Sf[HS];
#pragma unroll
    for (int i = 0; i < HS; ++i) {
      Sf[i] = pack_pair(S[2 * i], S[2 * i + 1]);
      if (OUT) sm.hand[0][hh * HS + i][lane] = Sf[i];
    }
    __syncthreads();  // chunk 0 staged
    int c0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = c0 + u;
        const bool active = c < nch;  // (only the optional state stores look at it)
        const uint16_t* Ks = sm.Ks[u];
        const float* Gs = sm.Gs[u];
        if (STATES) {  // S_c, the state before chunk c, for the backward (bf16: its operand type there)
          const auto rs = buffer_rsrc(static_cast<uint16_t*>(p.states) +
                                          ((slot0 + clampc(c)) * H + h) * static_cast<int64_t>(DK) * Dv,
                                      active ? DK * Dv * 2 : 0);
#pragma unroll
          for (int i = 0; i < HB; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              buffer_store1e<uint16_t>(rs, (tau(hh * HB + i, lg, r) * Dv + j0 + lr) * 2, S[i][r]);
        }
        // ---- interval A: partial Z = K[:, half] S[half] (token rows in tau order) ----
        bf16x8_t ka[HS][4];
#pragma unroll
        for (int i = 0; i < HS; ++i)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            ka[i][mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                         Ks + kpos<DK>(tau(mb, lr >> 2, lr & 3), 4 * (hh * HS + i) + lg)));
        f32x4_t Zp[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int i = 0; i < HS; ++i)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) Zp[mb] = mma(ka[i][mb], Sf[i], Zp[mb]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) sm.zx[hh][mb][lane] = Zp[mb];
        // (a step past the last chunk finds its decays staged as zero and Gamma_n
        // as 1, and leaves S unchanged)
        const float gn = Gs[63];
#pragma unroll
        for (int i = 0; i < HB; ++i) S[i] = S[i] * gn;
        __syncthreads();  // X: both partials of Z written
        // ---- interval B: R, E, and the update of this half of S ----
        // LDS reads go out in batches of at most 15 (the depth the LDS wait
        // counter can name), each ahead of the products that use it: the
        // partials of Z and T diag(beta); the v tile and Gamma; the decays to the
        // chunk end and the K^T fragments of the update (rows in tau order, via
        // ds_read_b64_tr_b16: lane s of each 16-lane group supplies token row
        // 8 g + s / 4 (+ 4) of the step and the four columns 32 (b / 2) + 8 (s % 4) +
        // 4 (b % 2) + 0..3, i.e. half b % 2 of piece 4 (b / 2) + s % 4).
        f32x4_t zp0[4], zp1[4];
        bf16x8_t tb[6];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          zp0[mb] = sm.zx[0][mb][lane];
          zp1[mb] = sm.zx[1][mb][lane];
        }
#pragma unroll
        for (int f = 0; f < 6; ++f) tb[f] = sm.Tb[u][f][lane];
        __builtin_amdgcn_sched_barrier(0);
        float4 v4[4], g4[4], d4[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int t0 = tau(mb, lg, 0);
          v4[mb] = *reinterpret_cast<const float4*>(sm.Vt[u] + lr * LDV + t0);
          g4[mb] = *reinterpret_cast<const float4*>(Gs + t0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the same sum, in the same order, in both waves
        f32x4_t Z[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) Z[mb] = zp0[mb] + zp1[mb];
        // R = V - diag(Gamma) Z (the v tile reads as zeros in a pass without V)
        auto r_of = [&](int mb) {
          const float vv[4] = {v4[mb].x, v4[mb].y, v4[mb].z, v4[mb].w};
          const float gg[4] = {g4[mb].x, g4[mb].y, g4[mb].z, g4[mb].w};
          f32x4_t r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = vv[e] - gg[e] * Z[mb][e];
          return r;
        };
        const bf16x8_t Rf0 = pack_pair(r_of(0), r_of(1));
        // E = (T diag(beta)) R (the blocks above the diagonal skipped)
        f32x4_t E[4];
        E[0] = mma(tb[0], Rf0, zero4());
        E[1] = mma(tb[1], Rf0, zero4());
        E[2] = mma(tb[2], Rf0, zero4());
        E[3] = mma(tb[4], Rf0, zero4());
        const bf16x8_t Rf1 = pack_pair(r_of(2), r_of(3));
        E[2] = mma(tb[3], Rf1, E[2]);
        E[3] = mma(tb[5], Rf1, E[3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) d4[mb] = *reinterpret_cast<const float4*>(Gs + 64 + tau(mb, lg, 0));
        bf16x8_t kt[2][HB];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < HB; ++i) {
            const int b = hh * HB + i;
            const int t = 32 * s + 8 * lg + (lr >> 2), pc = 4 * (b >> 1) + (lr & 3);
            const uint16_t* p0 = Ks + kpos<DK>(t, pc) + 4 * (b & 1);
            const uint16_t* p1 = Ks + kpos<DK>(t + 4, pc) + 4 * (b & 1);
            const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0));
            const i16x4_t bb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p1));
            kt[s][i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        __builtin_amdgcn_sched_barrier(0);
        // decayed E as the B operand of the update; E (fp32) to the output wave
        auto ed_of = [&](int mb) { return E[mb] * f32x4_t{d4[mb].x, d4[mb].y, d4[mb].z, d4[mb].w}; };
        const bf16x8_t Edf0 = pack_pair(ed_of(0), ed_of(1));
        if (OUT && hh == 0) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) sm.handE[u][mb][lane] = E[mb];
        }
        // S <- Gamma_n S + K^T (decayed E) on this half: HB independent chains
#pragma unroll
        for (int i = 0; i < HB; ++i) S[i] = mma(kt[0][i], Edf0, S[i]);
        const bf16x8_t Edf1 = pack_pair(ed_of(2), ed_of(3));
#pragma unroll
        for (int i = 0; i < HB; ++i) S[i] = mma(kt[1][i], Edf1, S[i]);
#pragma unroll
        for (int i = 0; i < HS; ++i) {
          Sf[i] = pack_pair(S[2 * i], S[2 * i + 1]);
          if (OUT) sm.hand[(c + 1) % 3][hh * HS + i][lane] = Sf[i];  // S_{c+1}, for the output wave
        }
        __syncthreads();  // Y: end of step
      }
      c0 += 2;
    } while (c0 < nsteps);
    write_state();
  } else if (OUT && w < 4) {
    if constexpr (OUT) {  // (compiled only where the pass has outputs)
      // ================= output waves: token row blocks 2 ow, 2 ow + 1 =================
      if (nch == 0) return;
      const int ow = w - 2;
      // Q rows 16 nb + j (B operand of S^T Q^T), P rows 16 nb + j in the operand
      // order the preparation kernel stores (fragment (nb, s) of 64 lanes), Gamma.
      struct OutSet {
        bf16x8_t qf[2][NKS];
        bf16x8_t pf[2][2];  // [block][reduction step], step 1 only for blocks 2-3
        float gq[2];
      };
      OutSet os[2];
      auto load_q = [&](OutSet& st, int c) {
        if (!OUT) return;
        const int nv = chunk_rows(c);
        const int64_t row0 = row0_of(c);
        const auto rq = buffer_rsrc(q + (row0 * H + h) * DK, ((nv - 1) * H * DK + DK) * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int s = 0; s < NKS; ++s)
            st.qf[i][s] = __builtin_bit_cast(
                bf16x8_t, buf_load16(rq, ((16 * (2 * ow + i) + lr) * H * DK + 32 * s + 8 * lg) * 2));
      };
      auto load_p = [&](OutSet& st, int c) {
        if (!OUT) return;
        const int64_t sh = (slot0 + c) * H + h;
        const auto rp = buffer_rsrc(pw + sh * 4096, 4096 * 2);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            if (s == 0 || ow == 1)
              st.pf[i][s] = __builtin_bit_cast(bf16x8_t, buf_load16(rp, (((2 * ow + i) * 2 + s) * 64 + lane) * 16));
        const auto rg = buffer_rsrc(gw + sh * 128, 256);
#pragma unroll
        for (int i = 0; i < 2; ++i) st.gq[i] = buf_load1(rg, (16 * (2 * ow + i) + lr) * 4);
      };
      // Output of chunk c in two parts: Y^T = S_c^T Q^T (interval A of step c + 1),
      // then E_c^T P^T and the store (interval B of step c + 1).
      f32x4_t y[2];
      auto part_y = [&](int c, const OutSet& st) {
        bf16x8_t sf[NKS];
#pragma unroll
        for (int s = 0; s < NKS; ++s) sf[s] = sm.hand[c % 3][s][lane];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          y[i] = zero4();
#pragma unroll
          for (int s = 0; s < NKS; ++s) y[i] = mma(sf[s], st.qf[i][s], y[i]);
        }
      };
      auto part_pe = [&](int c, int ue, OutSet& st) {
        const bf16x8_t ef0 = pack_pair(sm.handE[ue][0][lane], sm.handE[ue][1][lane]);
        bf16x8_t ef1 = ef0;
        if (ow == 1) ef1 = pack_pair(sm.handE[ue][2][lane], sm.handE[ue][3][lane]);
        const int cc = clampc(c), nv = chunk_rows(cc);
        const auto ro = buffer_rsrc(o + (row0_of(cc) * H + h) * Dv + j0,
                                    store_o && c < nch ? ((nv - 1) * H * Dv + 16) * 2 : 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f32x4_t pe = mma(ef0, st.pf[i][0], zero4());
          if (ow == 1) pe = mma(ef1, st.pf[i][1], pe);
          const float gt = st.gq[i];
          buffer_store4<uint16_t>(ro, ((16 * (2 * ow + i) + lr) * H * Dv + 4 * lg) * 2,
                                  p.scale * (gt * y[i][0] + pe[0]), p.scale * (gt * y[i][1] + pe[1]),
                                  p.scale * (gt * y[i][2] + pe[2]), p.scale * (gt * y[i][3] + pe[3]));
        }
      };
      load_q(os[0], 0);
      load_p(os[0], 0);
      load_q(os[1], clampc(1));
      load_p(os[1], clampc(1));
      __syncthreads();
      int c0 = 0;
      do {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = c0 + u;
          // interval A of step c: Y^T of chunk c - 1, then Q of chunk c + 1
          if (OUT && c > 0) {
            part_y(c - 1, os[u ^ 1]);
            load_q(os[u ^ 1], clampc(c + 1));
          }
          __syncthreads();  // X
          // interval B: the rest of chunk c - 1's output, then P and Gamma of chunk c + 1
          if (OUT && c > 0) {
            part_pe(c - 1, u ^ 1, os[u ^ 1]);
            load_p(os[u ^ 1], clampc(c + 1));
          }
          __syncthreads();  // Y: S_c and E_c handed over
        }
        c0 += 2;
      } while (c0 < nsteps);
      if (OUT) {  // the last step's chunk
        part_y(nsteps - 1, os[1]);
        part_pe(nsteps - 1, 1, os[1]);
      }
    }
  } else {
    // ================= loader waves =================
    if (nch == 0) return;
    const int lt = tid - (OUT ? 256 : 128);  // 0..127
    constexpr int KVR = DK / 8;             // 16-byte vectors per K row
    constexpr int NKV = 64 * KVR / 128;     // K vectors per loader thread
    struct LoadSet {
      u32x4_t kv[NKV];
      u32x4_t tv[3];  // T diag(beta) fragments: 16-byte vectors lt, lt + 128, lt + 256
      u32x4_t vv;     // v tile: row lt / 2, columns j0 + 8 (lt % 2) .. + 7
      u32x4_t gv;     // decays: floats 4 lt .. 4 lt + 3 (lt < 32)
      bool past;      // a step past the last chunk
    };
    LoadSet ls[2];
    const bool use_v = !p.zero_u;
    auto load_k = [&](LoadSet& s, int cu) {
      const int c = clampc(cu);
      const int nv = chunk_rows(c);
      const int64_t row0 = row0_of(c);
      const auto rk = buffer_rsrc(k + (row0 * H + h) * DK, ((nv - 1) * H * DK + DK) * 2);
#pragma unroll
      for (int x = 0; x < NKV; ++x) {
        const int vi = x * 128 + lt, t = vi / KVR, cv = (vi % KVR) * 8;
        s.kv[x] = buf_load16(rk, (t * H * DK + cv) * 2);
      }
    };
    auto load_rest = [&](LoadSet& s, int cu) {
      const int c = clampc(cu);
      s.past = cu >= nch;
      const int nv = chunk_rows(c);
      const int64_t row0 = row0_of(c);
      // (a pass without V loads nothing: the range is empty and the tile reads as zeros)
      const auto rv = buffer_rsrc(v + (row0 * H + h) * Dv, use_v ? ((nv - 1) * H * Dv + Dv) * 2 : 0);
      s.vv = buf_load16(rv, ((lt >> 1) * H * Dv + min(j0 + 8 * (lt & 1), Dv - 8)) * 2);
      const int64_t sh = (slot0 + c) * H + h;
      const auto rt = buffer_rsrc(tbw + sh * kTbSlot, 6 * 1024);
#pragma unroll
      for (int x = 0; x < 3; ++x) s.tv[x] = buf_load16(rt, (x * 128 + lt) * 16);
      const auto rg = buffer_rsrc(gw + sh * 128, 512);
      s.gv = buf_load16(rg, lt < 32 ? lt * 16 : kNoLoad);
    };
    auto stage_k = [&](const LoadSet& s, int sl) {
#pragma unroll
      for (int x = 0; x < NKV; ++x) {
        const int vi = x * 128 + lt, t = vi / KVR;
        *reinterpret_cast<u32x4_t*>(sm.Ks[sl] + kpos<DK>(t, vi % KVR)) = s.kv[x];
      }
    };
    auto stage_rest = [&](const LoadSet& s, int sl) {
      const int t = lt >> 1, cbase = 8 * (lt & 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wd = s.vv[e >> 1];
        sm.Vt[sl][(cbase + e) * LDV + t] = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
      }
#pragma unroll
      for (int x = 0; x < 3; ++x) {
        const int vi = x * 128 + lt;
        sm.Tb[sl][vi >> 6][vi & 63] = __builtin_bit_cast(bf16x8_t, s.tv[x]);
      }
      if (lt < 32) {
        // past the last chunk: no decay of E and Gamma_n = 1, so S stays unchanged
        u32x4_t gv = s.gv;
        if (s.past && lt >= 16) gv = u32x4_t{0u, 0u, 0u, 0u};
        if (s.past && lt == 15) gv[3] = __float_as_uint(1.f);
        *reinterpret_cast<u32x4_t*>(sm.Gs[sl] + 4 * lt) = gv;
      }
    };
    load_k(ls[0], 0);
    load_rest(ls[0], 0);
    load_k(ls[1], 1);
    load_rest(ls[1], 1);
    stage_k(ls[0], 0);
    stage_rest(ls[0], 0);
    load_k(ls[0], 2);
    load_rest(ls[0], 2);
    __syncthreads();
    int c0 = 0;
    do {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = c0 + u;
        // interval A of step c: K of chunk c + 1 staged; interval B: the v tile,
        // T diag(beta) and the decays staged, then chunk c + 3 loaded
        stage_k(ls[u ^ 1], u ^ 1);
        __syncthreads();  // X
        stage_rest(ls[u ^ 1], u ^ 1);
        load_k(ls[u ^ 1], c + 3);
        load_rest(ls[u ^ 1], c + 3);
        __syncthreads();  // Y
      }
      c0 += 2;
    } while (c0 < nsteps);
  }
}

int cu_count_chain() {
  static int counts[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (counts[dev] == 0) {
    int n = 0;
    counts[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return counts[dev];
}

template <int DK, bool STATES, bool OUT>
hipError_t launch_chain_t(const FwdParams& q, hipStream_t s) {
  constexpr size_t need = sizeof(ChainSmem<DK, OUT>);
  static_assert(DK == 64 || DK == 128, "K swizzle defined for 8 or 16 pieces per row");
  static_assert(need <= 160 * 1024, "LDS budget exceeded");
  // A grid with fewer than two workgroups per compute unit asks for more than half
  // of a CU's LDS so that no CU holds two while another idles.
  const int blocks = q.nseg * q.N * q.H * (q.ncol / 16);
  const size_t smem = blocks < 2 * cu_count_chain() && need < 82 * 1024 ? 82 * 1024 : need;
  auto kern = chunk_chain_kernel<DK, STATES, OUT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  // (without outputs: the two state waves and the two loader waves only)
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(OUT ? 384 : 256), smem, s, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_chain(const FwdParams& p, int Dk, bool states, bool out, hipStream_t s) {
  if (Dk == 128) {
    if (states) return out ? launch_chain_t<128, true, true>(p, s) : launch_chain_t<128, true, false>(p, s);
    return out ? launch_chain_t<128, false, true>(p, s) : launch_chain_t<128, false, false>(p, s);
  }
  if (Dk == 64) {
    if (states) return out ? launch_chain_t<64, true, true>(p, s) : launch_chain_t<64, true, false>(p, s);
    return out ? launch_chain_t<64, false, true>(p, s) : launch_chain_t<64, false, false>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
