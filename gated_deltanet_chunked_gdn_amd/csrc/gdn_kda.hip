// Chunked gated delta rule with one decay per key channel (the KDA gate layout
// of the cuLA issue #126 page, "Minimal public reproduction": g shaped like q).
//
// Per token, a = exp(g_t) (length Dk):  S <- diag(a) S,  e = beta (v - S^T k),
// S <- S + k e^T,  o = scale S^T q  (the update of "Research Sprint Day 1",
// "The GDN update", with a diagonal forget factor).  Over a chunk of n <= 64
// rows, with gamma = cumsum(g) per channel (the log-space accumulation the
// Day-2 page, "Building some intuition", gates step 5, prefers) and Gamma = exp(gamma):
//   A_ij = beta_i sum_c k_ic k_jc exp(gamma_ic - gamma_jc)   (j < i)
//   P_ij = sum_c q_ic k_jc exp(gamma_ic - gamma_jc)           (j <= i)
//   E = (I + A)^-1 diag(beta) (V - (K o Gamma) S)
//   O = scale ((Q o Gamma) S + P E)
//   S <- diag(Gamma_n) S + (K o exp(gamma_n - gamma))^T E
// Every exponent above is <= 0 (g <= 0, j <= i), so nothing overflows however
// strong the decay.  The per-channel factor cannot be pulled out of K K^T as one
// rank-one mask, but for rows i > r >= j it splits as exp(gamma_ic - gamma_rc)
// exp(gamma_rc - gamma_jc) with both exponents <= 0.
//
// Two kernels.  Decays, A, the inverse and the state are fp32; the chunk record
// is stored in the io element type, so that the state pass multiplies bf16
// operands with fp32 accumulation for bf16 io and runs IEEE fp32 products for
// fp32 io.
//   kda_prep_kernel  -- one workgroup per (chunk, head, sequence); writes the
//                       chunk's record: T diag(beta), P, K o Gamma, Q o Gamma,
//                       (K o exp(gamma_n - gamma))^T and Gamma_n.  A and P below
//                       the diagonal blocks are fp32 MFMA products of rows decayed
//                       to a reference row between the two blocks.
//   kda_state_kernel -- one workgroup per (sequence, head, 16 value columns);
//                       walks the chunks in order with its state tile in fp32
//                       MFMA accumulators; four of its eight waves load the next
//                       chunks' records meanwhile.
#include <type_traits>

#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_kda_common.h"

namespace gdn {
namespace {

using chunk::seq_range;
using chunk::u32x4_t;

template <int DK, typename EL>
using KdaRec = kda::Rec<DK, EL>;

// LDS of the prep kernel (bytes): K and Q rows in the io element type, gamma in
// fp32, A in fp32 (beta on its unused diagonal), all rows unpadded and swizzled
// in 16-byte units so that the 16 rows an MFMA fragment reads sit in distinct
// banks.  Once the record's K, Q and decay parts are written, the K, Q and
// gamma rows are dead and the solve's T and block products reuse their space.  For bf16
// io this is 80 KiB: two workgroups per CU.
template <int DK, typename E>
struct PrepLds {
  static constexpr int kK = 0;                                    // E [64][DK]
  static constexpr int kQ = kK + 64 * DK * static_cast<int>(sizeof(E));
  static constexpr int kG = kQ + 64 * DK * static_cast<int>(sizeof(E));  // float [64][DK]
  static constexpr int kA = kG + 64 * DK * 4;                     // float [64][64]
  static constexpr int kBytes = kA + 64 * 64 * 4;
  static constexpr int kT = 0;                                    // float [64][65], over K, Q, gamma
  static constexpr int kM = kT + 64 * 65 * 4;                     // float [4][16][17]
  static_assert(kM + 4 * 16 * 17 * 4 <= kA, "the solve's buffers must fit over K, Q and gamma");
};
// Swizzled column of channel ch in row i: 16-byte units (EPV elements) XOR-ed
// with the row's low bits.
template <int DK, int EPV>
__device__ __forceinline__ int swz(int i, int ch) {
  return ch ^ ((EPV * (i & 15)) & (DK - 1));
}

template <int DK, typename E>
constexpr size_t prep_smem_bytes() {
  return PrepLds<DK, E>::kBytes;
}

template <typename E>
__device__ __forceinline__ f32x4_t ld4f(const E* p);  // four consecutive io elements, widened
template <>
__device__ __forceinline__ f32x4_t ld4f<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
}
template <>
__device__ __forceinline__ f32x4_t ld4f<float>(const float* p) {
  return *reinterpret_cast<const f32x4_t*>(p);
}

// The diagonal 16x16 blocks of A and P factor through their middle row m = 16 b + 8:
// exp(gamma_i - gamma_j) = exp(gamma_i - gamma_m) exp(gamma_m - gamma_j) for any
// rows i, j of the block, each factor between 2^-D and 2^D, D the larger of the
// block's decays from its first row to m and from m to its last row.  While no
// channel has D above kMaxBlockDrop in any diagonal block (log2 units), both
// factors and their products with the keys and queries stay far inside fp32 and
// the blocks are MFMA products like the others; a chunk with a steeper block takes
// the exact pair-by-pair sums instead.  (Entries above the diagonal, which these
// products also form, can reach 2^(2 D) and are never kept.)  The flag lives in an
// unused entry above A's diagonal.
constexpr float kMaxBlockDrop = 100.f;
constexpr int kSteepAt = 63;  // A's entry (0, 63)

// Eight values to eight consecutive operand elements (16-byte aligned): one
// 16-byte store for bf16 (round to nearest even), two for fp32.
template <typename EL>
__device__ __forceinline__ void store8(EL* dst, const float (&v)[8]) {
  if constexpr (sizeof(EL) == 2) {
    const uint4 u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    *reinterpret_cast<uint4*>(dst) = u;
  } else {
    *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

template <int DK, typename E>
__global__ __launch_bounds__(512) void kda_prep_kernel(KdaParams p) {
  using Op = std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>;
  using EL = typename Op::elem;
  using R = KdaRec<DK, EL>;
  using PL = PrepLds<DK, E>;
  constexpr int EPV = 16 / static_cast<int>(sizeof(E));  // io elements per 16 bytes
  extern __shared__ __align__(16) char smp[];
  E* const ks = reinterpret_cast<E*>(smp + PL::kK);      // [64][DK] keys (swizzled)
  E* const qs = reinterpret_cast<E*>(smp + PL::kQ);      // [64][DK] queries (swizzled)
  float* const gs = reinterpret_cast<float*>(smp + PL::kG);  // [64][DK] g, then gamma log2(e) (swizzled by 4)
  float* const As = reinterpret_cast<float*>(smp + PL::kA);  // [64][64] A; beta_i at (i, i)
  float* const Ts = reinterpret_cast<float*>(smp + PL::kT);  // [64][65] T = (I + A)^-1 (after the outputs)
  float* const Ms = reinterpret_cast<float*>(smp + PL::kM);  // [4][16][17] block products of the solve
  auto kidx = [](int i, int ch) { return i * DK + swz<DK, EPV>(i, ch); };
  auto gidx = [](int i, int ch) { return i * DK + swz<DK, 4>(i, ch); };
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t r0 = 64LL * c;
  if (r0 >= len) return;
  const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
  const int64_t slot = bos / 64 + n + c;
  char* const recb = static_cast<char*>(p.ws) + (slot * p.H + h) * static_cast<int64_t>(R::kBytes);
  EL* const rec = reinterpret_cast<EL*>(recb);
  float* const aux = p.aux ? p.aux + (slot * p.H + h) * static_cast<int64_t>(kda::Aux::kFloats) : nullptr;
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);

  // Every load of the chunk is issued before the first store (eight channels per
  // vector; native vector types).  Rows past the chunk's end load its last row
  // (no branch around a load) and are stored as zero keys, queries and g, so
  // gamma stays at the last row's value and those rows contribute nothing.
  {
    constexpr int VPR = DK / 8;          // eight-channel vectors per row
    constexpr int NV = 64 * VPR / 512;   // vectors per thread
    constexpr int W = sizeof(E) / 2;     // 16-byte words per eight io elements
    u32x4_t kr[NV][W], qr[NV][W], gr[NV][2];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + 512 * u, i = x / VPR, ch = 8 * (x % VPR);
      const int64_t off = ((bos + r0 + (i < nr ? i : nr - 1)) * p.H + h) * DK + ch;
#pragma unroll
      for (int wd = 0; wd < W; ++wd) {
        kr[u][wd] = *reinterpret_cast<const u32x4_t*>(k + off + wd * EPV);
        qr[u][wd] = *reinterpret_cast<const u32x4_t*>(q + off + wd * EPV);
      }
      gr[u][0] = *reinterpret_cast<const u32x4_t*>(p.g + off);
      gr[u][1] = *reinterpret_cast<const u32x4_t*>(p.g + off + 4);
    }
    const float bv = p.beta[(bos + r0 + (lane < nr ? lane : nr - 1)) * p.H + h];
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + 512 * u, i = x / VPR, ch = 8 * (x % VPR);
      const bool ok = i < nr;
#pragma unroll
      for (int wd = 0; wd < W; ++wd) {
        *reinterpret_cast<u32x4_t*>(ks + kidx(i, ch + wd * EPV)) = ok ? kr[u][wd] : z;
        *reinterpret_cast<u32x4_t*>(qs + kidx(i, ch + wd * EPV)) = ok ? qr[u][wd] : z;
      }
      *reinterpret_cast<u32x4_t*>(gs + gidx(i, ch)) = ok ? gr[u][0] : z;
      *reinterpret_cast<u32x4_t*>(gs + gidx(i, ch + 4)) = ok ? gr[u][1] : z;
    }
    if (tid < 64) As[tid * 64 + tid] = tid < nr ? bv : 0.f;
    if (tid == 0) As[kSteepAt] = 0.f;
  }
  __syncthreads();
  if (tid < DK) {  // channel tid: its 64 values are read at once, summed in registers (log2 units)
    float col[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) col[i] = gs[gidx(i, tid)] * chunk::kLog2e;
    float acc = 0.f, first = 0.f, mid = 0.f, drop = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      acc += col[i];
      gs[gidx(i, tid)] = acc;
      if (i % 16 == 0) first = acc;
      if (i % 16 == 8) {
        mid = acc;
        drop = fmaxf(drop, first - mid);
      }
      if (i % 16 == 15) drop = fmaxf(drop, mid - acc);
    }
    if (drop > kMaxBlockDrop) As[kSteepAt] = 1.f;  // (every writer stores the same value)
  }
  __syncthreads();
  const bool steep = As[kSteepAt] != 0.f;  // uniform over the workgroup

  // A and P.  Below the 16x16 diagonal blocks, block (bi, bj) factors through the
  // last row r = 16 bj + 15 of block bj: exp(gamma_i - gamma_j) =
  // exp(gamma_i - gamma_r) exp(gamma_r - gamma_j) channel by channel, both factors
  // <= 1 (j <= r < i), so A and P there are fp32 MFMA products of decayed rows;
  // waves 0-5 take one such block each.  A lane reads four consecutive channels of
  // its rows at once and feeds them to four products (in the product of k-step
  // (k0, e) the lanes of group g hold channel k0 + 4 g + e, in both operands).
  // The diagonal blocks go the same way through their middle row (waves 6 and 7,
  // two blocks each) unless the chunk is steep; then they are summed pair by pair,
  // one exponential per channel: every thread takes one of the first 512 pairs
  // whole and an eighth of a channel range of one of the last 32, whose sixteen
  // parts are added within a DPP row.
  // rows ia (A operand) and jb (B operand) of this lane, both decayed to row rr
  auto decayed_product = [&](int ia, int jb, int rr, f32x4_t& accA, f32x4_t& accP, int kb = 0, int ke = DK) {
    accA = zero4();
    accP = zero4();
#pragma unroll 2
    for (int k0 = kb; k0 < ke; k0 += 16) {
      const int ch = k0 + 4 * (lane >> 4);
      const f32x4_t gr = *reinterpret_cast<const f32x4_t*>(gs + gidx(rr, ch));
      const f32x4_t gi = *reinterpret_cast<const f32x4_t*>(gs + gidx(ia, ch));
      const f32x4_t gj = *reinterpret_cast<const f32x4_t*>(gs + gidx(jb, ch));
      const f32x4_t ki = ld4f<E>(ks + kidx(ia, ch)), qi = ld4f<E>(qs + kidx(ia, ch)), kj = ld4f<E>(ks + kidx(jb, ch));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ei = __builtin_amdgcn_exp2f(gi[e] - gr[e]);
        const float bk = kj[e] * __builtin_amdgcn_exp2f(gr[e] - gj[e]);
        accA = __builtin_amdgcn_mfma_f32_16x16x4f32(ki[e] * ei, bk, accA, 0, 0, 0);
        accP = __builtin_amdgcn_mfma_f32_16x16x4f32(qi[e] * ei, bk, accP, 0, 0, 0);
      }
    }
  };
  // A diagonal block's results: A below the diagonal (beta_i on it), P on and below it.
  auto store_diag = [&](int b, const f32x4_t& accA, const f32x4_t& accP) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int i = 16 * b + 4 * (lane >> 4) + q4, j = 16 * b + (lane & 15);
      if (j < i) As[i * 64 + j] = As[i * 64 + i] * accA[q4];
      if (j <= i) rec[R::kP + i * 64 + j] = Op::cvt(accP[q4]);
      if (aux) {
        aux[kda::Aux::kAb + i * 64 + j] = j < i ? accA[q4] : 0.f;
        aux[kda::Aux::kP + i * 64 + j] = j <= i ? accP[q4] : 0.f;
      }
    }
  };
  // The MFMA work per SIMD (wave w runs on SIMD w % 4) is balanced at two and a
  // half blocks: waves 0-5 take one block below the diagonal blocks each, wave 6
  // diagonal block 0 and wave 7 block 2 whole, and blocks 1 and 3 are split by
  // channel halves between waves 6 / 4 and 7 / 5.  The second halves' sums wait in
  // A's unused upper blocks ((0,1), (0,2) for block 1; (1,2), (1,3) for block 3)
  // until the barrier below, after which waves 6 and 7 add them to their own.
  f32x4_t hA = zero4(), hP = zero4();  // waves 6, 7: first half of block 1 / 3
  if (wave < 6) {
    const int bi = wave < 3 ? wave + 1 : wave < 5 ? wave - 1 : 3;  // (1,0) (2,0) (3,0) (2,1) (3,1) (3,2)
    const int bj = wave < 3 ? 0 : wave < 5 ? 1 : 2;
    f32x4_t accA, accP;
    decayed_product(16 * bi + (lane & 15), 16 * bj + (lane & 15), 16 * bj + 15, accA, accP);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int i = 16 * bi + 4 * (lane >> 4) + q4, j = 16 * bj + (lane & 15);
      As[i * 64 + j] = As[i * 64 + i] * accA[q4];
      rec[R::kP + i * 64 + j] = Op::cvt(accP[q4]);
      if (aux) {
        aux[kda::Aux::kAb + i * 64 + j] = accA[q4];
        aux[kda::Aux::kP + i * 64 + j] = accP[q4];
      }
    }
    if (wave >= 4 && !steep) {  // second channel half of diagonal block 1 (wave 4) or 3 (wave 5)
      const int b = wave == 4 ? 1 : 3, rb = wave == 4 ? 0 : 1;
      decayed_product(16 * b + (lane & 15), 16 * b + (lane & 15), 16 * b + 8, accA, accP, DK / 2, DK);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = 16 * rb + 4 * (lane >> 4) + q4, cc = lane & 15;
        As[r * 64 + 16 * (rb + 1) + cc] = accA[q4];
        As[r * 64 + 16 * (rb + 2) + cc] = accP[q4];
      }
    }
  } else if (!steep) {
    const int b0 = 2 * (wave - 6), b1 = b0 + 1;  // whole block b0, first half of block b1
    f32x4_t accA, accP;
    decayed_product(16 * b0 + (lane & 15), 16 * b0 + (lane & 15), 16 * b0 + 8, accA, accP);
    store_diag(b0, accA, accP);
    decayed_product(16 * b1 + (lane & 15), 16 * b1 + (lane & 15), 16 * b1 + 8, hA, hP, 0, DK / 2);
  }
  if (!steep) {
    __syncthreads();  // the second halves of blocks 1 and 3 are in A's upper blocks
    if (wave >= 6) {
      const int b1 = 2 * (wave - 6) + 1, rb = wave - 6;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r = 16 * rb + 4 * (lane >> 4) + q4, cc = lane & 15;
        hA[q4] += As[r * 64 + 16 * (rb + 1) + cc];
        hP[q4] += As[r * 64 + 16 * (rb + 2) + cc];
      }
      store_diag(b1, hA, hP);
    }
  }
  if (steep) {
    // pair tl of diagonal block b: row il, column jl <= il inside the block
    auto pair_of = [](int t, int& i, int& j) {
      const int b = t / 136, tl = t % 136;
      int il = static_cast<int>((sqrtf(8.f * tl + 1.f) - 1.f) * 0.5f);
      if (il * (il + 1) / 2 > tl) --il;
      if ((il + 1) * (il + 2) / 2 <= tl) ++il;
      i = 16 * b + il;
      j = 16 * b + tl - il * (il + 1) / 2;
    };
    // channels [c0, c0 + NCH) of pair (i, j): A and P sums
    auto pair_sums = [&](int i, int j, int c0, int nch, float& a, float& sc) {
      a = 0.f;
      sc = 0.f;
#pragma unroll 4
      for (int ch = c0; ch < c0 + nch; ch += 4) {
        const f32x4_t k4i = ld4f<E>(ks + kidx(i, ch));
        const f32x4_t k4j = ld4f<E>(ks + kidx(j, ch));
        const f32x4_t q4i = ld4f<E>(qs + kidx(i, ch));
        const f32x4_t g4i = *reinterpret_cast<const f32x4_t*>(gs + gidx(i, ch));
        const f32x4_t g4j = *reinterpret_cast<const f32x4_t*>(gs + gidx(j, ch));
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const float kd = k4j[x] * __builtin_amdgcn_exp2f(g4i[x] - g4j[x]);
          a = fmaf(k4i[x], kd, a);
          sc = fmaf(q4i[x], kd, sc);
        }
      }
    };
    // waves 6-7 (no MFMA block) take pairs 0..127, waves 0-5 pairs 128..511
    int i, j;
    float a, sc;
    pair_of(tid >= 384 ? tid - 384 : tid + 128, i, j);
    pair_sums(i, j, 0, DK, a, sc);
    if (j < i) As[i * 64 + j] = As[i * 64 + i] * a;
    rec[R::kP + i * 64 + j] = Op::cvt(sc);
    if (aux) {
      aux[kda::Aux::kAb + i * 64 + j] = a;
      aux[kda::Aux::kP + i * 64 + j] = sc;
    }
    // pairs 512..543: sixteen threads (one DPP row) per pair, DK / 16 channels each
    pair_of(512 + (tid >> 4), i, j);
    pair_sums(i, j, (DK / 16) * (tid & 15), DK / 16, a, sc);
    a += dpp_f32<0x111, 0xf>(a);  // row_shr:1 .. 8: lane 15 of the row ends with the row's sum
    sc += dpp_f32<0x111, 0xf>(sc);
    a += dpp_f32<0x112, 0xf>(a);
    sc += dpp_f32<0x112, 0xf>(sc);
    a += dpp_f32<0x114, 0xf>(a);
    sc += dpp_f32<0x114, 0xf>(sc);
    a += dpp_f32<0x118, 0xf>(a);
    sc += dpp_f32<0x118, 0xf>(sc);
    if ((tid & 15) == 15) {
      if (j < i) As[i * 64 + j] = As[i * 64 + i] * a;
      rec[R::kP + i * 64 + j] = Op::cvt(sc);
      if (aux) {
        aux[kda::Aux::kAb + i * 64 + j] = a;
        aux[kda::Aux::kP + i * 64 + j] = sc;
      }
    }
  }
  // P above the diagonal: eight zeros per 16-byte store where all eight columns
  // lie above it, single zeros in the group that holds the diagonal
  {
    const int i = tid >> 3, jb = 8 * (tid & 7);
    if (jb > i) {
      const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store8<EL>(rec + R::kP + i * 64 + jb, z);
    } else if (jb + 7 > i) {
      for (int j = i + 1; j < jb + 8; ++j) rec[R::kP + i * 64 + j] = Op::cvt(0.f);
    }
  }

  // the record's K o Gamma, Q o Gamma, decayed keys and Gamma_n (K, Q and gamma
  // are dead afterwards: T and the block products take their place)
  {
    const int rl = nr - 1;
    // eight consecutive channels of one row per thread and pass
    for (int x = tid; x < 8 * DK; x += 512) {
      const int i = x / (DK / 8), ch = 8 * (x % (DK / 8));
      const f32x4_t k0 = ld4f<E>(ks + kidx(i, ch)), k1 = ld4f<E>(ks + kidx(i, ch + 4));
      const f32x4_t q0 = ld4f<E>(qs + kidx(i, ch)), q1 = ld4f<E>(qs + kidx(i, ch + 4));
      const f32x4_t g0 = *reinterpret_cast<const f32x4_t*>(gs + gidx(i, ch));
      const f32x4_t g1 = *reinterpret_cast<const f32x4_t*>(gs + gidx(i, ch + 4));
      float kv[8], qv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float e0 = __builtin_amdgcn_exp2f(g0[e]), e1 = __builtin_amdgcn_exp2f(g1[e]);
        kv[e] = k0[e] * e0;
        kv[e + 4] = k1[e] * e1;
        qv[e] = q0[e] * e0;
        qv[e + 4] = q1[e] * e1;
      }
      store8<EL>(rec + R::kKG + i * DK + ch, kv);
      store8<EL>(rec + R::kQG + i * DK + ch, qv);
    }
    // decayed keys, transposed: eight consecutive rows of one channel per thread and pass
    for (int x = tid; x < 8 * DK; x += 512) {
      const int ch = x >> 3, i0 = 8 * (x & 7);
      const float gl = gs[gidx(rl, ch)];
      float dv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dv[e] = IoT<E>::ld(ks + kidx(i0 + e, ch)) * __builtin_amdgcn_exp2f(gl - gs[gidx(i0 + e, ch)]);
      store8<EL>(rec + R::kKDt + ch * 64 + i0, dv);
    }
    if (tid < DK) reinterpret_cast<float*>(recb + R::kGnByte)[tid] = __builtin_amdgcn_exp2f(gs[gidx(rl, tid)]);
  }
  __syncthreads();
  for (int x = tid; x < 64 * 64; x += 512) {
    const int i = x / 64, j = x % 64;
    if (j / 16 > i / 16) Ts[i * 65 + j] = 0.f;  // T is zero above its diagonal blocks
  }

  // T = (I + A)^-1: the 16x16 diagonal blocks by forward substitution (wave w
  // inverts block w, one column per lane), then the blocks below, band by band:
  // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj (fp32 MFMA)
  if (wave < 4 && lane < 16) {
    const int b = wave, cc = lane;
    float tcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc = fmaf(As[(16 * b + r) * 64 + 16 * b + m], tcol[m], acc);
      tcol[r] = r == cc ? 1.f : (r < cc ? 0.f : -acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Ts[(16 * b + r) * 65 + 16 * b + cc] = tcol[r];
  }
  __syncthreads();
  for (int d = 1; d < 4; ++d) {
    const bool act = wave < 4 - d;
    const int bj = wave, bi = wave + d;
    float* Mt = Ms + wave * 16 * 17;
    if (act) {
      f32x4_t m = zero4();
      for (int kb = bj; kb < bi; ++kb)
        tile_mma_f32_rowmajor<16>(m, As + 16 * bi * 64 + 16 * kb, 64, Ts + 16 * kb * 65 + 16 * bj, 65, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Mt[(4 * (lane >> 4) + r) * 17 + (lane & 15)] = m[r];
    }
    __syncthreads();
    if (act) {
      f32x4_t x = zero4();
      tile_mma_f32_rowmajor<16>(x, Ts + 16 * bi * 65 + 16 * bi, 65, Mt, 17, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[(16 * bi + 4 * (lane >> 4) + r) * 65 + 16 * bj + (lane & 15)] = -x[r];
    }
    __syncthreads();
  }

  for (int x = tid; x < 64 * 64; x += 512) {
    const int i = x / 64, j = x % 64;
    rec[R::kTb + x] = Op::cvt(Ts[i * 65 + j] * As[j * 64 + j]);
    if (aux) aux[kda::Aux::kT + x] = Ts[i * 65 + j];
  }
}

// acc += A(16 x K) B(K x 16) (A row-major, B stored transposed, as tile_mma),
// the k-steps dealt round-robin to up to four accumulators so that independent
// chains are in flight instead of one dependent chain.
template <typename Op, int K>
__device__ __forceinline__ void tile_mma_split(f32x4_t& acc, const typename Op::elem* a, int lda,
                                               const typename Op::elem* bt, int ldb, int lane) {
  constexpr int NS = K / Op::KSTEP;
  constexpr int NA = NS < 4 ? NS : 4;
  static_assert(NS * Op::KSTEP == K, "K must be a multiple of the MFMA depth");
  f32x4_t x[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) x[j] = zero4();
#pragma unroll
  for (int st = 0; st < NS; ++st)
    x[st % NA] = Op::mma(Op::frag(a, lda, lane, st * Op::KSTEP), Op::frag(bt, ldb, lane, st * Op::KSTEP), x[st % NA]);
  f32x4_t t = x[0];
#pragma unroll
  for (int j = 1; j < NA; ++j) t += x[j];
  acc += t;
}

// LDS of the state kernel, in elements of the operand type EL (row strides keep
// 16-byte aligned rows), then Gamma_n as DK floats.
template <int DK, typename EL>
struct StateLds {
  static constexpr int PAD = 16 / static_cast<int>(sizeof(EL));
  static constexpr int LK = DK + PAD;  // rows of K o Gamma, Q o Gamma and the transposed state
  static constexpr int L64 = 64 + PAD; // rows of 64-wide matrices
  static constexpr int kKG = 0;
  static constexpr int kQG = kKG + 64 * LK;
  static constexpr int kKDt = kQG + 64 * LK;
  static constexpr int kTb = kKDt + DK * L64;
  static constexpr int kP = kTb + 64 * L64;
  static constexpr int kSt = kP + 64 * L64;   // [16][LK]: S^T of the tile
  static constexpr int kRt = kSt + 16 * LK;   // [16][L64]: (V - (K o Gamma) S)^T
  static constexpr int kEt = kRt + 16 * L64;  // [16][L64]: E^T
  static constexpr int LV = 16 + PAD;         // rows of the v tile
  static constexpr int kVs = kEt + 16 * L64;  // [64][LV]: the chunk's v tile (io element type)
  static constexpr int kElems = kVs + 64 * LV;
  static constexpr int kGnByte = (kElems * static_cast<int>(sizeof(EL)) + 15) / 16 * 16;
  static constexpr int kBytes = kGnByte + DK * 4;
};

// One chunk record in registers: the five matrices (contiguous at the start of
// the record) as 16-byte vectors tid + 256 u, and Gamma_n[tid].  Every matrix
// spans a multiple of 256 vectors, so each u belongs to one matrix at compile
// time.  (A native vector type: arrays of HIP's float4 struct are kept in
// scratch memory when they live across a barrier.)
template <int DK, typename EL>
struct Stager {
  using L = StateLds<DK, EL>;
  using R = KdaRec<DK, EL>;
  static constexpr int EPV = 16 / static_cast<int>(sizeof(EL));   // elements per vector
  static constexpr int NV = R::kGnByte / 16 / 256;
  static constexpr int kUP = 4096 / EPV / 256;                     // first u of P
  static constexpr int kUKG = 2 * kUP;                             // first u of K o Gamma
  static constexpr int kUQG = kUKG + 64 * DK / EPV / 256;          // first u of Q o Gamma
  static constexpr int kUKD = kUQG + 64 * DK / EPV / 256;          // first u of the decayed keys
  static_assert(kUKD + 64 * DK / EPV / 256 == NV, "record layout");

  static __device__ __forceinline__ void load(f32x4_t (&r)[NV], float& gn, const char* rec, int tid) {
#pragma unroll
    for (int u = 0; u < NV; ++u) r[u] = *reinterpret_cast<const f32x4_t*>(rec + 16 * (tid + 256 * u));
    // every lane loads (lanes past DK re-read entry 0): a branch around the load
    // would make the wave wait for all of its loads right here
    gn = reinterpret_cast<const float*>(rec + R::kGnByte)[tid < DK ? tid : 0];
  }
  static __device__ __forceinline__ void store(const f32x4_t (&r)[NV], float gn, char* smb, int tid) {
    EL* const sm = reinterpret_cast<EL*>(smb);
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      EL* dst;
      if (u < kUKG) {  // T diag(beta) or P: 64-wide rows
        const int f = EPV * (tid + 256 * (u < kUP ? u : u - kUP));
        dst = sm + (u < kUP ? L::kTb : L::kP) + (f / 64) * L::L64 + f % 64;
      } else if (u < kUKD) {  // K o Gamma or Q o Gamma: DK-wide rows
        const int f = EPV * (tid + 256 * (u < kUQG ? u - kUKG : u - kUQG));
        dst = sm + (u < kUQG ? L::kKG : L::kQG) + (f / DK) * L::LK + f % DK;
      } else {  // decayed keys, transposed: DK rows of 64
        const int f = EPV * (tid + 256 * (u - kUKD));
        dst = sm + L::kKDt + (f / 64) * L::L64 + f % 64;
      }
      *reinterpret_cast<f32x4_t*>(dst) = r[u];
    }
    if (tid < DK) reinterpret_cast<float*>(smb + L::kGnByte)[tid] = gn;
  }
};

// Eight waves: waves 0-3 compute (wave w owns rows 16 w .. 16 w + 15 of the
// chunk and state row blocks w, w + 4), waves 4-7 keep the records of the next
// two chunks (one for fp32 records) in registers while the current one is
// computed and write each to LDS at the top of its step.  The state stays fp32 in accumulators; for bf16 io the
// products take bf16 operands (the record, S, R and E rounded to bf16) with
// fp32 accumulation, for fp32 io every product is IEEE fp32.
template <int DK, typename E>
__global__ __launch_bounds__(512) void kda_state_kernel(KdaParams p) {
  using Op = std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>;
  using EL = typename Op::elem;
  using R = KdaRec<DK, EL>;
  using L = StateLds<DK, EL>;
  using St8 = Stager<DK, EL>;
  constexpr int RB = DK / 64;  // state row blocks per compute wave
  extern __shared__ __align__(16) char smb[];
  EL* const sm = reinterpret_cast<EL*>(smb);
  const float* const gn_s = reinterpret_cast<const float*>(smb + L::kGnByte);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool loader = tid >= 256;
  const int lt = tid - 256;
  const int col = lane & 15, g4 = lane >> 4;
  const int NC = p.ncol, ntile = NC / 16;
  const int nb = gridDim.x;
  const int Lb = blockIdx.x;
  const int vb = (nb % 8 == 0) ? (Lb % 8) * (nb / 8) + Lb / 8 : Lb;  // tiles of a head share an XCD
  const int tile = vb % ntile, nh = (vb / ntile) % (p.N * p.H), h = nh % p.H, n = nh / p.H;
  const int seg = p.seg_base + vb / ntile / (p.N * p.H);
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  // this workgroup's segment: chunks [cb, cb + nch) of the sequence
  const int nch_all = static_cast<int>((len + 63) / 64);
  const int seg_len = (nch_all + p.G - 1) / p.G;
  const int cb = min(seg * seg_len, nch_all);
  const int nch = min(cb + seg_len, nch_all) - cb;
  const bool store_o = p.write_o == kOutAll || (p.write_o == kOutSeg0 && seg == 0);
  const int Dv = p.Dv;
  const int c0 = tile * 16 + col;
  const E* v = static_cast<const E*>(p.v);
  E* o = static_cast<E*>(p.o);
  EL* St = sm + L::kSt;
  EL* Rt = sm + L::kRt;
  EL* Et = sm + L::kEt;
  const char* rec0 =
      static_cast<const char*>(p.ws) + ((bos / 64 + n + cb) * p.H + h) * static_cast<int64_t>(R::kBytes);
  const int64_t rec_step = static_cast<int64_t>(p.H) * R::kBytes;  // next chunk slot, same head

  // The two roles run separate loops with the same four barriers per chunk, so
  // the loaders' prefetch registers and the compute waves' operands never have
  // to be allocated side by side.
  if (loader) {
    // the chunk's v tile (64 rows x 16 columns) travels with its record: one
    // 16-byte vector per loader lane, through a buffer resource bounded to the
    // chunk's valid rows (rows past the sequence, and every row of a pass without
    // V, read as zeros; lanes past the tile load row 63 again and keep nothing)
    constexpr int VPR = 16 * static_cast<int>(sizeof(E)) / 16;  // vectors per tile row
    constexpr int EPV = 16 / static_cast<int>(sizeof(E));
    const int vrow = lt / VPR < 64 ? lt / VPR : 63, vcol = (lt % VPR) * EPV;
    const bool vlane = lt < 64 * VPR;
    auto load_vt = [&](int c) {
      const int64_t r0 = 64LL * (cb + c);
      const int nv = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
      const auto rv = chunk::buffer_rsrc(v + ((bos + r0) * p.H + h) * Dv + tile * 16,
                                  p.zero_u ? 0 : static_cast<int>(((nv - 1) * p.H * Dv + 16) * sizeof(E)));
      return __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, (vrow * p.H * Dv + vcol) * static_cast<int>(sizeof(E)), 0, 0));
    };
    auto store_vt = [&](const f32x4_t& x, int) {
      if (vlane) *reinterpret_cast<f32x4_t*>(sm + L::kVs + vrow * L::LV + vcol) = x;
    };
    if constexpr (St8::NV <= 16) {
      // two records in flight: chunk c + 2 is requested as chunk c is staged
      f32x4_t pa[St8::NV], pb[St8::NV];
      f32x4_t va = {0.f, 0.f, 0.f, 0.f}, vb2 = {0.f, 0.f, 0.f, 0.f};
      float ga = 0.f, gb = 0.f;
      if (nch > 0) {
        St8::load(pa, ga, rec0, lt);
        va = load_vt(0);
      }
      if (nch > 1) {
        St8::load(pb, gb, rec0 + rec_step, lt);
        vb2 = load_vt(1);
      }
      for (int c = 0; c < nch; c += 2) {
        __syncthreads();  // the previous chunk's reads of the staged record are done
        St8::store(pa, ga, smb, lt);
        store_vt(va, c);
        __syncthreads();
        if (c + 2 < nch) {
          St8::load(pa, ga, rec0 + (c + 2) * rec_step, lt);
          va = load_vt(c + 2);
        }
        __syncthreads();
        __syncthreads();
        if (c + 1 < nch) {
          __syncthreads();
          St8::store(pb, gb, smb, lt);
          store_vt(vb2, c + 1);
          __syncthreads();
          if (c + 3 < nch) {
            St8::load(pb, gb, rec0 + (c + 3) * rec_step, lt);
            vb2 = load_vt(c + 3);
          }
          __syncthreads();
          __syncthreads();
        }
      }
    } else {
      // fp32 records (twice the registers): one record in flight
      f32x4_t pa[St8::NV];
      f32x4_t va = {0.f, 0.f, 0.f, 0.f};
      float ga = 0.f;
      if (nch > 0) {
        St8::load(pa, ga, rec0, lt);
        va = load_vt(0);
      }
      for (int c = 0; c < nch; ++c) {
        __syncthreads();
        St8::store(pa, ga, smb, lt);
        store_vt(va, c);
        __syncthreads();
        if (c + 1 < nch) {
          St8::load(pa, ga, rec0 + (c + 1) * rec_step, lt);
          va = load_vt(c + 1);
        }
        __syncthreads();
        __syncthreads();
      }
    }
    return;
  }

  // compute waves: state rows 16 rb + 4 g4 + r, rb = w + 4 b, in accumulators
  f32x4_t S[RB];
  const int64_t sbase = (static_cast<int64_t>(n) * p.H + h) * DK;
  const int64_t segS = (static_cast<int64_t>(seg) * p.N * p.H + nh) * DK;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (w + 4 * b) + 4 * g4 + r;
      float x = 0.f;
      if (p.start_mode == kStartCarry)
        x = p.carry[(segS + row) * NC + c0];
      else if (p.start_mode == kStartIdentity)
        x = row == c0 ? 1.f : 0.f;
      else if (p.start_mode == kStartS0 && seg == 0 && p.S0)
        x = p.S0[(sbase + row) * Dv + c0];
      S[b][r] = x;
    }
  }
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) St[col * L::LK + 16 * (w + 4 * b) + 4 * g4 + r] = Op::cvt(S[b][r]);
  for (int c = 0; c < nch; ++c) {
    const int64_t r0 = 64LL * (cb + c);
    const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
    if (p.states) {  // the state before the chunk, for the backward (one segment; operand type)
      EL* const sc = static_cast<EL*>(p.states) + ((bos / 64 + n + cb + c) * p.H + h) * static_cast<int64_t>(DK) * Dv;
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[(16 * (w + 4 * b) + 4 * g4 + r) * Dv + c0] = Op::cvt(S[b][r]);
    }
    __syncthreads();
    __syncthreads();  // the record and the v tile of chunk c are in LDS
    float vcur[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) vcur[r] = IoT<EL>::ld(sm + L::kVs + (16 * w + 4 * g4 + r) * L::LV + col);
    // R = V - (K o Gamma) S and (Q o Gamma) S for rows 16 w .. 16 w + 15
    f32x4_t qsacc = zero4();
    {
      f32x4_t ks = zero4();
      tile_mma_split<Op, DK>(ks, sm + L::kKG + 16 * w * L::LK, L::LK, St, L::LK, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Rt[col * L::L64 + 16 * w + 4 * g4 + r] = Op::cvt(vcur[r] - ks[r]);
      tile_mma_split<Op, DK>(qsacc, sm + L::kQG + 16 * w * L::LK, L::LK, St, L::LK, lane);
    }
    __syncthreads();
    // E = T diag(beta) R
    {
      f32x4_t e = zero4();
      tile_mma_split<Op, 64>(e, sm + L::kTb + 16 * w * L::L64, L::L64, Rt, L::L64, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Et[col * L::L64 + 16 * w + 4 * g4 + r] = Op::cvt(e[r]);
    }
    __syncthreads();
    // O = scale ((Q o Gamma) S + P E)
    tile_mma_split<Op, 64>(qsacc, sm + L::kP + 16 * w * L::L64, L::L64, Et, L::L64, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * w + 4 * g4 + r;
      if (store_o && row < nr) IoT<E>::st(o + ((bos + r0 + row) * p.H + h) * Dv + c0, p.scale * qsacc[r]);
    }
    // S <- diag(Gamma_n) S + (K o exp(gamma_n - gamma))^T E
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rb = w + 4 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[b][r] *= gn_s[16 * rb + 4 * g4 + r];
      tile_mma_split<Op, 64>(S[b], sm + L::kKDt + 16 * rb * L::L64, L::L64, Et, L::L64, lane);
    }
    // every compute wave has finished reading St (before the previous barrier),
    // so the new state can replace it now
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) St[col * L::LK + 16 * (w + 4 * b) + 4 * g4 + r] = Op::cvt(S[b][r]);
  }

  const bool to_final = p.final_to_sfinal && seg == p.G - 1;
  if (to_final ? p.S_final != nullptr : p.seg_out != nullptr) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * (w + 4 * b) + 4 * g4 + r;
        if (to_final)
          p.S_final[(sbase + row) * Dv + c0] = S[b][r];
        else
          p.seg_out[(segS + row) * NC + c0] = S[b][r];
      }
  }
}

template <int DK, typename E>
hipError_t launch_kda_t(const KdaParams& p, hipStream_t s) {
  using EL = typename std::conditional_t<sizeof(E) == 2, OpBf16, OpF32>::elem;
  static_assert(StateLds<DK, EL>::kBytes <= 160 * 1024, "LDS budget exceeded");
  static_assert(prep_smem_bytes<DK, E>() <= 160 * 1024, "LDS budget exceeded");
  constexpr size_t prep_smem = prep_smem_bytes<DK, E>();
  constexpr size_t state_smem = StateLds<DK, EL>::kBytes;
  auto prep = kda_prep_kernel<DK, E>;
  auto state = kda_state_kernel<DK, E>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(prep_smem));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(state), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(state_smem));
  if (e != hipSuccess) return e;
  if (p.max_chunks > 0) {
    hipLaunchKernelGGL(prep, dim3(p.max_chunks, p.H, p.N), dim3(512), prep_smem, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto run = [&](const KdaParams& q) {
    hipLaunchKernelGGL(state, dim3(q.nseg * q.N * q.H * (q.ncol / 16)), dim3(512), state_smem, s, q);
    return hipGetLastError();
  };
  KdaParams q = p;
  q.ncol = p.Dv;
  q.zero_u = 0;
  q.carry = nullptr;
  if (p.G == 1) {
    q.seg_base = 0; q.nseg = 1; q.start_mode = kStartS0; q.write_o = p.o ? kOutAll : kOutNone;
    q.seg_out = nullptr; q.final_to_sfinal = 1;
    return run(q);
  }
  // G segments per sequence, as for the scalar-gate pass: (1) segment 0 from S0
  // with its outputs and segments 1 .. G-2 from zero (their offsets b); (2) the
  // transition maps M of segments 1 .. G-2 (V = 0, started from the identity);
  // (3) the carries, composed in fp32; (4) segments 1 .. G-1 again from them.
  const size_t ends_floats = static_cast<size_t>(p.G) * p.N * p.H * DK * p.Dv;
  float* ends = p.seg_ws;
  float* starts = ends + ends_floats;
  float* maps = starts + ends_floats;
  q.seg_base = 0; q.nseg = p.G - 1; q.start_mode = kStartS0; q.write_o = kOutSeg0;
  q.seg_out = ends; q.final_to_sfinal = 0;
  if ((e = run(q)) != hipSuccess) return e;
  if (p.G > 2) {
    KdaParams m = q;
    m.ncol = DK; m.seg_base = 1; m.nseg = p.G - 2; m.start_mode = kStartIdentity;
    m.write_o = kOutNone; m.zero_u = 1; m.seg_out = maps;
    if ((e = run(m)) != hipSuccess) return e;
  }
  if ((e = launch_segment_carry(ends, maps, starts, p.G, p.N, p.H, DK, p.Dv, s)) != hipSuccess) return e;
  q.seg_base = 1; q.nseg = p.G - 1; q.start_mode = kStartCarry; q.write_o = kOutAll;
  q.carry = starts; q.seg_out = nullptr; q.final_to_sfinal = 1;
  return run(q);
}

}  // namespace

hipError_t launch_kda_fwd(const KdaParams& p, int Dk, bool bf16, hipStream_t s) {
  if (Dk == 128) return bf16 ? launch_kda_t<128, uint16_t>(p, s) : launch_kda_t<128, float>(p, s);
  if (Dk == 64) return bf16 ? launch_kda_t<64, uint16_t>(p, s) : launch_kda_t<64, float>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
