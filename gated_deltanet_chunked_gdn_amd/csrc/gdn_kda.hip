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
//                       MFMA accumulators (v_mfma_f32_16x16x4_f32).
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

template <int DK>
constexpr size_t prep_smem_bytes() {
  return (3 * 64 * (DK + 1) + 2 * 64 * 65 + 64) * sizeof(float);
}

template <int DK, typename E>
__global__ __launch_bounds__(256) void kda_prep_kernel(KdaParams p) {
  using R = KdaRec<DK>;
  constexpr int LD = DK + 1;  // odd stride: rows read by consecutive lanes hit distinct banks
  extern __shared__ __align__(16) float sm[];
  float* ks = sm;             // [64][LD] keys
  float* qs = ks + 64 * LD;   // [64][LD] queries
  float* gs = qs + 64 * LD;   // [64][LD] g, then gamma = cumsum(g)
  float* As = gs + 64 * LD;   // [64][65] A (strictly lower)
  float* Ts = As + 64 * 65;   // [64][65] T = (I + A)^-1
  float* bs = Ts + 64 * 65;   // [64] beta
  const int c = blockIdx.x, h = blockIdx.y, n = blockIdx.z, tid = threadIdx.x;
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
  // stays at the last row's value and those rows contribute nothing
  for (int x = tid; x < 64 * DK; x += 256) {
    const int i = x / DK, ch = x % DK;
    const bool ok = i < nr;
    const int64_t off = ((bos + r0 + i) * p.H + h) * DK + ch;
    ks[i * LD + ch] = ok ? IoT<E>::ld(k + off) : 0.f;
    qs[i * LD + ch] = ok ? IoT<E>::ld(q + off) : 0.f;
    gs[i * LD + ch] = ok ? p.g[off] : 0.f;
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
#pragma unroll 8
    for (int ch = 0; ch < DK; ++ch) {
      const float kd = kj[ch] * __expf(gi[ch] - gj[ch]);
      a = fmaf(ki[ch], kd, a);
      s = fmaf(qi[ch], kd, s);
    }
    As[i * 65 + j] = j < i ? bs[i] * a : 0.f;
    rec[R::kP + i * 64 + j] = s;
  }
  for (int x = tid; x < 64 * 64; x += 256) {
    const int i = x / 64, j = x % 64;
    if (j > i) rec[R::kP + x] = 0.f;
  }
  __syncthreads();

  // T = (I + A)^-1 by forward substitution, one column per lane of wave 0
  if (tid < 64) {
    const int col = tid;
    for (int i = 0; i < 64; ++i) {
      float t = i == col ? 1.f : 0.f;
      if (i > col) {
        for (int j = col; j < i; ++j) t = fmaf(-As[i * 65 + j], Ts[j * 65 + col], t);
      }
      Ts[i * 65 + col] = t;
    }
  }
  __syncthreads();

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

// Copy `rows` rows of `cols` floats (cols % 4 == 0) from a dense global matrix
// into LDS rows of stride ld.
__device__ __forceinline__ void stage(float* dst, int ld, const float* src, int rows, int cols, int tid) {
  const int per_row = cols / 4;
  for (int x = tid; x < rows * per_row; x += 256) {
    const int r = x / per_row, c4 = x % per_row;
    *reinterpret_cast<float4*>(dst + r * ld + 4 * c4) = *reinterpret_cast<const float4*>(src + r * cols + 4 * c4);
  }
}

template <int DK, typename E>
__global__ __launch_bounds__(256) void kda_state_kernel(KdaParams p) {
  using R = KdaRec<DK>;
  using L = StateLds<DK>;
  constexpr int RB = DK / 64;  // state row blocks per wave
  extern __shared__ __align__(16) float sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

  // state rows 16 rb + 4 g4 + r, rb = w + 4 b, in accumulators
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
    const int64_t slot = bos / 64 + n + c;
    const float* rec = p.ws + (slot * p.H + h) * static_cast<int64_t>(R::kSize);
    __syncthreads();  // the previous chunk's reads of the staged record are done
    stage(sm + L::kKG, L::LK, rec + R::kKG, 64, DK, tid);
    stage(sm + L::kQG, L::LK, rec + R::kQG, 64, DK, tid);
    stage(sm + L::kKDt, L::L64, rec + R::kKDt, DK, 64, tid);
    stage(sm + L::kTb, L::L64, rec + R::kTb, 64, 64, tid);
    stage(sm + L::kP, L::L64, rec + R::kP, 64, 64, tid);
    if (tid < DK) sm[L::kGn + tid] = rec[R::kGn + tid];
    __syncthreads();

    // R = V - (K o Gamma) S and (Q o Gamma) S for rows 16 w .. 16 w + 15
    f32x4_t ks = zero4(), qsacc = zero4();
    tile_mma<OpF32, DK>(ks, sm + L::kKG + 16 * w * L::LK, L::LK, St, L::LK, lane);
    tile_mma<OpF32, DK>(qsacc, sm + L::kQG + 16 * w * L::LK, L::LK, St, L::LK, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * w + 4 * g4 + r;
      const float vv = row < nr ? IoT<E>::ld(v + ((bos + r0 + row) * p.H + h) * Dv + c0) : 0.f;
      Rt[col * L::L64 + row] = vv - ks[r];
    }
    __syncthreads();

    // E = T diag(beta) R
    f32x4_t e = zero4();
    tile_mma<OpF32, 64>(e, sm + L::kTb + 16 * w * L::L64, L::L64, Rt, L::L64, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) Et[col * L::L64 + 16 * w + 4 * g4 + r] = e[r];
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
    // every wave has finished reading St (the first barrier of this chunk), so
    // the new state can replace it now
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
  hipLaunchKernelGGL(state, dim3(p.N * p.H * (p.Dv / 16)), dim3(256), state_smem, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_fwd(const KdaParams& p, int Dk, bool bf16, hipStream_t s) {
  if (Dk == 128) return bf16 ? launch_kda_t<128, uint16_t>(p, s) : launch_kda_t<128, float>(p, s);
  if (Dk == 64) return bf16 ? launch_kda_t<64, uint16_t>(p, s) : launch_kda_t<64, float>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace gdn
