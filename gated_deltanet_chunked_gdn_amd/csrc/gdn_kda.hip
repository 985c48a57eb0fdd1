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
// strong the decay; the per-channel factor cannot be pulled out of K K^T as a
// rank-one mask, which is why A and P are summed channel by channel.
//
// Two kernels, all arithmetic in fp32 (io dtype only at the loads and the o store):
//   kda_prep_kernel  -- one workgroup per (chunk, head, sequence); writes the
//                       chunk's record: T diag(beta), P, K o Gamma, Q o Gamma,
//                       (K o exp(gamma_n - gamma))^T and Gamma_n.
//   kda_state_kernel -- one workgroup per (sequence, head, 16 value columns);
//                       walks the chunks in order with its state tile in fp32
//                       MFMA accumulators (v_mfma_f32_16x16x4_f32); four of its
//                       eight waves load the next chunk's record meanwhile.
#include "gdn_chunk_common.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using chunk::seq_range;

// Offsets (floats) inside one (chunk slot, head) record.
template <int DK>
struct KdaRec {
  static constexpr int kTb = 0;               // T diag(beta), 64 x 64, zero above the diagonal
  static constexpr int kP = 4096;             // P, 64 x 64, zero above the diagonal
  static constexpr int kKG = 8192;            // K o Gamma, 64 x DK
  static constexpr int kQG = kKG + 64 * DK;   // Q o Gamma, 64 x DK
  static constexpr int kKDt = kQG + 64 * DK;  // (K o exp(gamma_n - gamma))^T, DK x 64
  static constexpr int kGn = kKDt + 64 * DK;  // Gamma_n, DK
  static constexpr int kSize = kGn + DK;
};

// Eight consecutive io elements: raw load, widening store of eight floats to LDS.
template <typename E>
struct Vec8;
template <>
struct Vec8<uint16_t> {
  using raw = uint4;
  static __device__ __forceinline__ raw load(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  static __device__ __forceinline__ raw zero() { return uint4{0u, 0u, 0u, 0u}; }
  static __device__ __forceinline__ void store(float* dst, const raw& u) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float f[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f[2 * m] = __uint_as_float(w[m] << 16);
      f[2 * m + 1] = __uint_as_float(w[m] & 0xffff0000u);
    }
    *reinterpret_cast<float4*>(dst) = float4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<float4*>(dst + 4) = float4{f[4], f[5], f[6], f[7]};
  }
};
template <>
struct Vec8<float> {
  struct raw {
    float4 a, b;
  };
  static __device__ __forceinline__ raw load(const float* p) {
    return raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ raw zero() { return raw{float4{0.f, 0.f, 0.f, 0.f}, float4{0.f, 0.f, 0.f, 0.f}}; }
  static __device__ __forceinline__ void store(float* dst, const raw& u) {
    *reinterpret_cast<float4*>(dst) = u.a;
    *reinterpret_cast<float4*>(dst + 4) = u.b;
  }
};

template <int DK>
constexpr size_t prep_smem_bytes() {
  return (3 * 64 * (DK + 4) + 2 * 64 * 65 + 4 * 16 * 17 + 64) * sizeof(float);
}

template <int DK, typename E>
__global__ __launch_bounds__(256) void kda_prep_kernel(KdaParams p) {
  using R = KdaRec<DK>;
  constexpr int LD = DK + 4;  // 16-byte rows: four channels per LDS read
  extern __shared__ __align__(16) float sm[];
  float* ks = sm;             // [64][LD] keys
  float* qs = ks + 64 * LD;   // [64][LD] queries
  float* gs = qs + 64 * LD;   // [64][LD] g, then gamma = cumsum(g)
  float* As = gs + 64 * LD;   // [64][65] A (strictly lower)
  float* Ts = As + 64 * 65;   // [64][65] T = (I + A)^-1
  float* Ms = Ts + 64 * 65;   // [4][16][17] block products of the solve
  float* bs = Ms + 4 * 16 * 17;  // [64] beta
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int64_t r0 = 64LL * c;
  if (r0 >= len) return;
  const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
  const int64_t slot = bos / 64 + n + c;
  float* rec = p.ws + (slot * p.H + h) * static_cast<int64_t>(R::kSize);
  const E* q = static_cast<const E*>(p.q);
  const E* k = static_cast<const E*>(p.k);

  // rows past the chunk's end hold zero keys and queries and g = 0, so gamma
  // stays at the last row's value and those rows contribute nothing.  Eight
  // channels per load; every load of the thread is issued before the first store.
  {
    constexpr int VPR = DK / 8;             // vectors per row
    constexpr int NV = 64 * VPR / 256;      // vectors per thread
    typename Vec8<E>::raw kr[NV], qr[NV];
    float4 ga[NV], gb[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + 256 * u, i = x / VPR, ch = 8 * (x % VPR);
      const int64_t off = ((bos + r0 + i) * p.H + h) * DK + ch;
      if (i < nr) {
        kr[u] = Vec8<E>::load(k + off);
        qr[u] = Vec8<E>::load(q + off);
        ga[u] = *reinterpret_cast<const float4*>(p.g + off);
        gb[u] = *reinterpret_cast<const float4*>(p.g + off + 4);
      } else {
        kr[u] = Vec8<E>::zero();
        qr[u] = Vec8<E>::zero();
        ga[u] = gb[u] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int x = tid + 256 * u, i = x / VPR, ch = 8 * (x % VPR);
      Vec8<E>::store(ks + i * LD + ch, kr[u]);
      Vec8<E>::store(qs + i * LD + ch, qr[u]);
      *reinterpret_cast<float4*>(gs + i * LD + ch) = ga[u];
      *reinterpret_cast<float4*>(gs + i * LD + ch + 4) = gb[u];
    }
  }
  if (tid < 64) bs[tid] = tid < nr ? p.beta[(bos + r0 + tid) * p.H + h] : 0.f;
  __syncthreads();
  if (tid < DK) {
    float acc = 0.f;
    for (int i = 0; i < 64; ++i) {
      acc += gs[i * LD + tid];
      gs[i * LD + tid] = acc;
    }
  }
  __syncthreads();

  // A and P over the 2080 pairs j <= i, one pair per thread at a time
  for (int pi = tid; pi < 64 * 65 / 2; pi += 256) {
    int i = static_cast<int>((sqrtf(8.f * pi + 1.f) - 1.f) * 0.5f);
    if (i * (i + 1) / 2 > pi) --i;
    if ((i + 1) * (i + 2) / 2 <= pi) ++i;
    const int j = pi - i * (i + 1) / 2;
    const float* ki = ks + i * LD;
    const float* kj = ks + j * LD;
    const float* qi = qs + i * LD;
    const float* gi = gs + i * LD;
    const float* gj = gs + j * LD;
    float a = 0.f, s = 0.f;
#pragma unroll 4
    for (int ch = 0; ch < DK; ch += 4) {
      const float4 k4i = *reinterpret_cast<const float4*>(ki + ch);
      const float4 k4j = *reinterpret_cast<const float4*>(kj + ch);
      const float4 q4i = *reinterpret_cast<const float4*>(qi + ch);
      const float4 g4i = *reinterpret_cast<const float4*>(gi + ch);
      const float4 g4j = *reinterpret_cast<const float4*>(gj + ch);
      const float d0 = k4j.x * __expf(g4i.x - g4j.x), d1 = k4j.y * __expf(g4i.y - g4j.y);
      const float d2 = k4j.z * __expf(g4i.z - g4j.z), d3 = k4j.w * __expf(g4i.w - g4j.w);
      a = fmaf(k4i.x, d0, fmaf(k4i.y, d1, fmaf(k4i.z, d2, fmaf(k4i.w, d3, a))));
      s = fmaf(q4i.x, d0, fmaf(q4i.y, d1, fmaf(q4i.z, d2, fmaf(q4i.w, d3, s))));
    }
    As[i * 65 + j] = j < i ? bs[i] * a : 0.f;
    rec[R::kP + i * 64 + j] = s;
  }
  for (int x = tid; x < 64 * 64; x += 256) {
    const int i = x / 64, j = x % 64;
    if (j > i) rec[R::kP + x] = 0.f;
    if (j / 16 > i / 16) Ts[i * 65 + j] = 0.f;  // T is zero above its diagonal blocks
  }
  __syncthreads();

  // T = (I + A)^-1: the 16x16 diagonal blocks by forward substitution (wave w
  // inverts block w, one column per lane), then the blocks below, band by band:
  // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj (fp32 MFMA)
  if (lane < 16) {
    const int b = wave, cc = lane;
    float tcol[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) acc = fmaf(As[(16 * b + r) * 65 + 16 * b + m], tcol[m], acc);
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
        tile_mma_f32_rowmajor<16>(m, As + 16 * bi * 65 + 16 * kb, 65, Ts + 16 * kb * 65 + 16 * bj, 65, lane);
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

  for (int x = tid; x < 64 * 64; x += 256) {
    const int i = x / 64, j = x % 64;
    rec[R::kTb + x] = Ts[i * 65 + j] * bs[j];
  }
  const float* gn = gs + (nr - 1) * LD;
  for (int x = tid; x < 64 * DK; x += 256) {
    const int i = x / DK, ch = x % DK;
    const float e = __expf(gs[i * LD + ch]);
    rec[R::kKG + x] = ks[i * LD + ch] * e;
    rec[R::kQG + x] = qs[i * LD + ch] * e;
  }
  for (int x = tid; x < 64 * DK; x += 256) {
    const int ch = x / 64, i = x % 64;
    rec[R::kKDt + x] = ks[i * LD + ch] * __expf(gn[ch] - gs[i * LD + ch]);
  }
  if (tid < DK) rec[R::kGn + tid] = __expf(gn[tid]);
}

// LDS of the state kernel (floats): row strides keep 16-byte aligned rows.
template <int DK>
struct StateLds {
  static constexpr int LK = DK + 4;  // rows of K o Gamma, Q o Gamma and the transposed state
  static constexpr int L64 = 68;     // rows of 64-wide matrices
  static constexpr int kKG = 0;
  static constexpr int kQG = kKG + 64 * LK;
  static constexpr int kKDt = kQG + 64 * LK;
  static constexpr int kTb = kKDt + DK * L64;
  static constexpr int kP = kTb + 64 * L64;
  static constexpr int kSt = kP + 64 * L64;   // [16][LK]: S^T of the tile
  static constexpr int kRt = kSt + 16 * LK;   // [16][L64]: (V - (K o Gamma) S)^T
  static constexpr int kEt = kRt + 16 * L64;  // [16][L64]: E^T
  static constexpr int kGn = kEt + 16 * L64;  // [DK]
  static constexpr int kFloats = kGn + DK;
};

// One chunk record in registers: the matrices (T diag(beta), P, K o Gamma,
// Q o Gamma, the decayed keys; contiguous in the record) as 16-byte vectors
// tid + 256 u, and Gamma_n[tid].  Region boundaries are multiples of 256
// vectors, so each u belongs to one matrix at compile time.  (A native vector
// type: arrays of HIP's float4 struct are kept in scratch memory when they live
// across a barrier.)
template <int DK>
struct Stager {
  using L = StateLds<DK>;
  static constexpr int NV = (8192 + 3 * 64 * DK) / 4 / 256;
  static constexpr int kUP = 4096 / 4 / 256;                // first u of P
  static constexpr int kUKG = 8192 / 4 / 256;               // first u of K o Gamma
  static constexpr int kUQG = kUKG + 64 * DK / 4 / 256;     // first u of Q o Gamma
  static constexpr int kUKD = kUQG + 64 * DK / 4 / 256;     // first u of the decayed keys

  static __device__ __forceinline__ void load(f32x4_t (&r)[NV], float& gn, const float* rec, int tid) {
#pragma unroll
    for (int u = 0; u < NV; ++u) r[u] = *reinterpret_cast<const f32x4_t*>(rec + 4 * (tid + 256 * u));
    gn = tid < DK ? rec[8192 + 3 * 64 * DK + tid] : 0.f;
  }
  static __device__ __forceinline__ void store(const f32x4_t (&r)[NV], float gn, float* sm, int tid) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float* dst;
      if (u < kUKG) {  // T diag(beta) or P: 64-wide rows
        const int f = 4 * (tid + 256 * (u < kUP ? u : u - kUP));
        dst = sm + (u < kUP ? L::kTb : L::kP) + (f / 64) * L::L64 + f % 64;
      } else if (u < kUKD) {  // K o Gamma or Q o Gamma: DK-wide rows
        const int f = 4 * (tid + 256 * (u < kUQG ? u - kUKG : u - kUQG));
        dst = sm + (u < kUQG ? L::kKG : L::kQG) + (f / DK) * L::LK + f % DK;
      } else {  // decayed keys, transposed: DK rows of 64
        const int f = 4 * (tid + 256 * (u - kUKD));
        dst = sm + L::kKDt + (f / 64) * L::L64 + f % 64;
      }
      *reinterpret_cast<f32x4_t*>(dst) = r[u];
    }
    if (tid < DK) sm[L::kGn + tid] = gn;
  }
};

// Eight waves: waves 0-3 compute (wave w owns rows 16 w .. 16 w + 15 of the
// chunk and state row blocks w, w + 4), waves 4-7 load the next chunk's record
// into registers while the current one is computed and write it to LDS at the
// top of the next step.
template <int DK, typename E>
__global__ __launch_bounds__(512) void kda_state_kernel(KdaParams p) {
  using R = KdaRec<DK>;
  using L = StateLds<DK>;
  using St8 = Stager<DK>;
  constexpr int RB = DK / 64;  // state row blocks per compute wave
  extern __shared__ __align__(16) float sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool loader = tid >= 256;
  const int lt = tid - 256;
  const int col = lane & 15, g4 = lane >> 4;
  const int ntile = p.Dv / 16;
  const int nb = p.N * p.H * ntile;
  const int Lb = blockIdx.x;
  const int vb = (nb % 8 == 0) ? (Lb % 8) * (nb / 8) + Lb / 8 : Lb;  // tiles of a head share an XCD
  const int tile = vb % ntile, nh = vb / ntile, h = nh % p.H, n = nh / p.H;
  int64_t bos, len;
  seq_range(p.seq, n, bos, len);
  const int nch = static_cast<int>((len + 63) / 64);
  const int Dv = p.Dv;
  const int c0 = tile * 16 + col;
  const E* v = static_cast<const E*>(p.v);
  E* o = static_cast<E*>(p.o);
  float* St = sm + L::kSt;
  float* Rt = sm + L::kRt;
  float* Et = sm + L::kEt;
  const float* rec0 = p.ws + ((bos / 64 + n) * p.H + h) * static_cast<int64_t>(R::kSize);
  const int64_t rec_step = static_cast<int64_t>(p.H) * R::kSize;  // next chunk slot, same head

  // The two roles run separate loops with the same four barriers per chunk, so
  // the loaders' prefetch registers and the compute waves' operands never have
  // to be allocated side by side.
  if (loader) {
    f32x4_t pre[St8::NV];
    float pre_gn = 0.f;
    if (nch > 0) St8::load(pre, pre_gn, rec0, lt);
    for (int c = 0; c < nch; ++c) {
      __syncthreads();  // the previous chunk's reads of the staged record are done
      St8::store(pre, pre_gn, sm, lt);
      __syncthreads();
      if (c + 1 < nch) St8::load(pre, pre_gn, rec0 + (c + 1) * rec_step, lt);
      __syncthreads();
      __syncthreads();
    }
    return;
  }

  // compute waves: state rows 16 rb + 4 g4 + r, rb = w + 4 b, in accumulators
  f32x4_t S[RB];
  const int64_t sbase = (static_cast<int64_t>(n) * p.H + h) * DK;
#pragma unroll
  for (int b = 0; b < RB; ++b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (w + 4 * b) + 4 * g4 + r;
      S[b][r] = p.S0 ? p.S0[(sbase + row) * Dv + c0] : 0.f;
      St[col * L::LK + row] = S[b][r];
    }
  }
  for (int c = 0; c < nch; ++c) {
    const int64_t r0 = 64LL * c;
    const int nr = static_cast<int>(len - r0 < 64 ? len - r0 : 64);
    __syncthreads();
    __syncthreads();  // the record of chunk c is in LDS
    {
      // R = V - (K o Gamma) S for rows 16 w .. 16 w + 15
      f32x4_t ks = zero4();
      tile_mma<OpF32, DK>(ks, sm + L::kKG + 16 * w * L::LK, L::LK, St, L::LK, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g4 + r;
        const float vv = row < nr ? IoT<E>::ld(v + ((bos + r0 + row) * p.H + h) * Dv + c0) : 0.f;
        Rt[col * L::L64 + row] = vv - ks[r];
      }
    }
    __syncthreads();
    // E = T diag(beta) R, then (Q o Gamma) S while E is published
    f32x4_t qsacc = zero4();
    {
      f32x4_t e = zero4();
      tile_mma<OpF32, 64>(e, sm + L::kTb + 16 * w * L::L64, L::L64, Rt, L::L64, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) Et[col * L::L64 + 16 * w + 4 * g4 + r] = e[r];
      tile_mma<OpF32, DK>(qsacc, sm + L::kQG + 16 * w * L::LK, L::LK, St, L::LK, lane);
    }
    __syncthreads();
    // O = scale ((Q o Gamma) S + P E)
    tile_mma<OpF32, 64>(qsacc, sm + L::kP + 16 * w * L::L64, L::L64, Et, L::L64, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * w + 4 * g4 + r;
      if (row < nr) IoT<E>::st(o + ((bos + r0 + row) * p.H + h) * Dv + c0, p.scale * qsacc[r]);
    }
    // S <- diag(Gamma_n) S + (K o exp(gamma_n - gamma))^T E
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int rb = w + 4 * b;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[b][r] *= sm[L::kGn + 16 * rb + 4 * g4 + r];
      tile_mma<OpF32, 64>(S[b], sm + L::kKDt + 16 * rb * L::L64, L::L64, Et, L::L64, lane);
    }
    // every compute wave has finished reading St (before the previous barrier),
    // so the new state can replace it now
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) St[col * L::LK + 16 * (w + 4 * b) + 4 * g4 + r] = S[b][r];
  }

  if (p.S_final) {
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.S_final[(sbase + 16 * (w + 4 * b) + 4 * g4 + r) * Dv + c0] = S[b][r];
  }
}

template <int DK, typename E>
hipError_t launch_kda_t(const KdaParams& p, hipStream_t s) {
  static_assert(StateLds<DK>::kFloats * sizeof(float) <= 160 * 1024, "LDS budget exceeded");
  static_assert(prep_smem_bytes<DK>() <= 160 * 1024, "LDS budget exceeded");
  constexpr size_t prep_smem = prep_smem_bytes<DK>();
  constexpr size_t state_smem = StateLds<DK>::kFloats * sizeof(float);
  auto prep = kda_prep_kernel<DK, E>;
  auto state = kda_state_kernel<DK, E>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(prep_smem));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(state), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(state_smem));
  if (e != hipSuccess) return e;
  if (p.max_chunks > 0) {
    hipLaunchKernelGGL(prep, dim3(p.max_chunks, p.H, p.N), dim3(256), prep_smem, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(state, dim3(p.N * p.H * (p.Dv / 16)), dim3(512), state_smem, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_fwd(const KdaParams& p, int Dk, bool bf16, hipStream_t s) {
  if (Dk == 128) return bf16 ? launch_kda_t<128, uint16_t>(p, s) : launch_kda_t<128, float>(p, s);
  if (Dk == 64) return bf16 ? launch_kda_t<64, uint16_t>(p, s) : launch_kda_t<64, float>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
