// C ABI of libgdn: argument validation, workspace sizing and dispatch.
// Every check runs on the host before the first launch (see include/gdn.h).
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "gdn_internal.h"
#include "gdn_kda_common.h"

namespace {

struct Range {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
};

Range span(const void* p, size_t bytes) {
  Range r;
  if (p && bytes) {
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + bytes;
  }
  return r;
}

bool overlap(const Range& a, const Range& b) {
  return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Checked {
  int64_t tokens = 0;    // B * T
  int64_t max_len = 0;   // longest sequence
  int32_t N = 0;
  bool bf16 = false;
  size_t io = 4;         // bytes per io element
  bool fp32_products = false;  // IEEE fp32 products (fp32 io, or GDN_PRECISION_FP32)
  size_t ce = 4;         // bytes per element of the per-chunk records (the product operand type)
};

enum class Kind { ChunkFwd, ChunkBwd, RecFwd, RecBwd, KdaFwd, KdaBwd };

gdn_status check_problem(const gdn_problem* p, Kind kind, Checked* c) {
  if (!p) return GDN_ERR_NULL;
  if (p->io_dtype != GDN_FP32 && p->io_dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (p->B < 0 || p->T < 0 || p->H <= 0 || p->Dk <= 0 || p->Dv <= 0 || p->num_seqs < 0)
    return GDN_ERR_SHAPE;
  if (p->Dk != 64 && p->Dk != 128) return GDN_ERR_UNSUPPORTED;
  if (p->Dv % 16 != 0 || p->Dv < 16 || p->Dv > 256) return GDN_ERR_UNSUPPORTED;
  if (p->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (p->precision != GDN_PRECISION_IO && p->precision != GDN_PRECISION_FP32) return GDN_ERR_UNSUPPORTED;
  const bool fp32_policy_bf16 = p->precision == GDN_PRECISION_FP32 && p->io_dtype == GDN_BF16;
  if (fp32_policy_bf16 && (kind == Kind::ChunkBwd || kind == Kind::KdaFwd || kind == Kind::KdaBwd))
    return GDN_ERR_UNSUPPORTED;
  const bool chunked = kind == Kind::ChunkFwd || kind == Kind::ChunkBwd;
  if (chunked) {
    const int G = p->num_segments;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return GDN_ERR_UNSUPPORTED;
    if (kind == Kind::ChunkBwd && G != 1) return GDN_ERR_UNSUPPORTED;
    // one chunk of one head's rows is addressed with 32-bit byte offsets
    if (static_cast<int64_t>(64) * p->H * std::max(p->Dk, p->Dv) * 4 > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  }
  if (kind == Kind::KdaFwd) {
    const int G = p->num_segments;
    if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return GDN_ERR_UNSUPPORTED;
    // one state-kernel launch has up to G * N * H * (max(Dk, Dv) / 16) blocks
    if (static_cast<int64_t>(G) * p->num_seqs * p->H * (std::max(p->Dk, p->Dv) / 16) > INT32_MAX)
      return GDN_ERR_UNSUPPORTED;
  }
  if (kind == Kind::KdaBwd) {
    if (p->num_segments != 1) return GDN_ERR_UNSUPPORTED;
    // one chunk of one head's rows is addressed with 32-bit byte offsets
    if (static_cast<int64_t>(64) * p->H * std::max(p->Dk, p->Dv) * 4 > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(p->num_seqs) * p->H * (p->Dv / 16) > INT32_MAX) return GDN_ERR_UNSUPPORTED;
  }
  if (kind == Kind::RecBwd && static_cast<size_t>(2) * p->Dk * (p->Dv + 1) * 4 +
                                      (2 * gdn::kRecBlock * p->Dk + 2 * gdn::kRecBlock + 8) * 4 >
                                  160 * 1024)
    return GDN_ERR_UNSUPPORTED;

  const bool packed = p->cu_seqlens_host || p->cu_seqlens_dev;
  if (packed) {
    if (!p->cu_seqlens_host || !p->cu_seqlens_dev) return GDN_ERR_NULL;
    if (p->B != 1) return GDN_ERR_SHAPE;
    const int32_t* cu = p->cu_seqlens_host;
    if (cu[0] != 0 || cu[p->num_seqs] != p->T) return GDN_ERR_SEQLENS;
    int64_t mx = 0;
    for (int32_t n = 0; n < p->num_seqs; ++n) {
      if (cu[n + 1] < cu[n]) return GDN_ERR_SEQLENS;
      mx = std::max<int64_t>(mx, cu[n + 1] - cu[n]);
    }
    c->max_len = mx;
  } else {
    if (p->num_seqs != p->B) return GDN_ERR_SHAPE;
    c->max_len = p->T;
  }
  if (p->num_seqs > 65535 || p->H > 65535) return GDN_ERR_UNSUPPORTED;
  // one state-kernel launch has num_segments * N * H * (Dv / 16) blocks
  if (static_cast<int64_t>(chunked && p->num_segments > 1 ? p->num_segments : 1) * p->num_seqs * p->H *
          (p->Dv / 16) > INT32_MAX)
    return GDN_ERR_UNSUPPORTED;
  c->tokens = static_cast<int64_t>(p->B) * p->T;
  c->N = p->num_seqs;
  c->bf16 = p->io_dtype == GDN_BF16;
  c->io = c->bf16 ? 2 : 4;
  c->fp32_products = !c->bf16 || p->precision == GDN_PRECISION_FP32;
  c->ce = c->fp32_products ? 4 : 2;
  return GDN_OK;
}

size_t t_slot_bytes(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * 64 * 64 * c.ce;
  return (b + 255) / 256 * 256;
}

size_t packed_slot_bytes(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * gdn::kTbSlot * c.ce;
  return (b + 255) / 256 * 256;
}

size_t gate_slot_bytes(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * 128 * sizeof(float);
  return (b + 255) / 256 * 256;
}

// Per-chunk states and state gradients of the backward, in the products' operand
// type (bf16 for bf16 products, fp32 for fp32 products: every use of them in the
// gradient kernel is as an operand of that type).
size_t state_slot_bytes(const gdn_problem* p, const Checked& c) {
  return static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * p->Dk * p->Dv * c.ce;
}

size_t kda_rec_region(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * gdn::kda_rec_bytes(p->Dk, c.bf16);
  return (b + 255) / 256 * 256;
}

// The KDA backward's fp32 copies of T, Ab and P, and its per-chunk states and state
// gradients in the operand type.
size_t kda_aux_region(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * gdn::kda::Aux::kFloats * 4;
  return (b + 255) / 256 * 256;
}
size_t kda_state_region(const gdn_problem* p, const Checked& c) {
  const size_t b = static_cast<size_t>(gdn::chunk_slots(c.tokens, c.N)) * p->H * p->Dk * p->Dv * c.ce;
  return (b + 255) / 256 * 256;
}

size_t workspace_bytes(const gdn_problem* p, Kind kind, const Checked& c) {
  if (kind == Kind::RecBwd)
    return gdn::recurrent_bwd_ws_floats(c.N, p->H, p->Dk, p->Dv, c.max_len) * sizeof(float);
  if (kind == Kind::ChunkFwd) {
    if (c.N == 0) return 0;
    // per (chunk slot, head): T diag(beta) (lower 16x16 blocks packed, io element
    // type), the causal score P (64 x 64 in MFMA operand order) and the chunk's
    // decays (128 fp32); then (num_segments > 1) the fp32 segment end states,
    // start states and maps
    return packed_slot_bytes(p, c) + t_slot_bytes(p, c) + gate_slot_bytes(p, c) +
           gdn::segment_ws_bytes(p->num_segments, c.N, p->H, p->Dk, p->Dv);
  }
  if (kind == Kind::KdaFwd) {
    if (c.N == 0) return 0;
    // one record per (chunk slot, head), then (num_segments > 1) the fp32 segment
    // end states, start states and maps
    return kda_rec_region(p, c) + gdn::segment_ws_bytes(p->num_segments, c.N, p->H, p->Dk, p->Dv);
  }
  if (kind == Kind::KdaBwd) {
    if (c.N == 0) return 0;
    // the forward's records, then T, Ab and P in fp32, then the state before and
    // the state gradient after every chunk (operand type)
    return kda_rec_region(p, c) + kda_aux_region(p, c) + 2 * kda_state_region(p, c);
  }
  if (kind == Kind::ChunkBwd) {
    if (c.N == 0) return 0;
    // T (64 x 64), T diag(beta) (packed), the decays and P (64 x 64) per (chunk
    // slot, head), then the state before and the state gradient after every chunk,
    // [slot][H][Dk][Dv] each in the operand type
    return 2 * t_slot_bytes(p, c) + packed_slot_bytes(p, c) + gate_slot_bytes(p, c) + 2 * state_slot_bytes(p, c);
  }
  return 0;
}

// The backward's buffer: per (chunk slot, head) T, T diag(beta) (packed), the
// decays and P row-major; the state before and the state gradient after every
// chunk (operand type); then (for the forward that keeps them) P in operand order.
struct BwdLayout {
  char* tws;
  char* tbws;
  float* gws;
  char* prws;
  char* states;
  char* dstates;
  char* pws;
};
BwdLayout bwd_layout(const gdn_problem* p, const Checked& c, void* ws) {
  char* const b = static_cast<char*>(ws);
  const size_t tb = t_slot_bytes(p, c), pb = packed_slot_bytes(p, c), gb = gate_slot_bytes(p, c);
  const size_t sb = state_slot_bytes(p, c);
  BwdLayout l;
  l.tws = b;
  l.tbws = b + tb;
  l.gws = reinterpret_cast<float*>(b + tb + pb);
  l.prws = b + tb + pb + gb;
  l.states = l.prws + tb;
  l.dstates = l.prws + tb + sb;
  l.pws = l.prws + tb + 2 * sb;
  return l;
}
size_t saved_bytes_needed(const gdn_problem* p, const Checked& c) {
  return c.N == 0 ? 0 : workspace_bytes(p, Kind::ChunkBwd, c) + t_slot_bytes(p, c);
}

struct Tensor {
  const void* ptr;
  size_t bytes;
  size_t align;
  bool required;
};

// Checks NULL / alignment of every tensor and that no output overlaps another
// tensor.  `ins` are read-only, `outs` are written.
gdn_status check_tensors(const std::vector<Tensor>& ins, const std::vector<Tensor>& outs) {
  for (const auto* set : {&ins, &outs})
    for (const Tensor& t : *set) {
      if (!t.ptr) {
        if (t.required && t.bytes) return GDN_ERR_NULL;
        continue;
      }
      if (!aligned(t.ptr, t.align)) return GDN_ERR_ALIGN;
    }
  for (size_t i = 0; i < outs.size(); ++i) {
    const Range ro = span(outs[i].ptr, outs[i].bytes);
    for (const Tensor& t : ins)
      if (overlap(ro, span(t.ptr, t.bytes))) return GDN_ERR_ALIAS;
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlap(ro, span(outs[j].ptr, outs[j].bytes))) return GDN_ERR_ALIAS;
  }
  return GDN_OK;
}

gdn::SeqInfo seq_info(const gdn_problem* p) { return gdn::SeqInfo{p->cu_seqlens_dev, p->T}; }

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

}  // namespace

namespace gdn {

gdn_status check_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* S0, const void* o, const float* S_final,
                           size_t* ws_need) {
  Checked c;
  gdn_status st = check_problem(p, Kind::ChunkFwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, ng * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false}},
                     {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false}});
  if (st != GDN_OK) return st;
  *ws_need = workspace_bytes(p, Kind::ChunkFwd, c);
  return GDN_OK;
}

}  // namespace gdn

extern "C" {

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int32_t s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "required pointer is NULL";
    case GDN_ERR_SHAPE: return "size out of range or inconsistent";
    case GDN_ERR_DTYPE: return "io_dtype is not a gdn_dtype";
    case GDN_ERR_UNSUPPORTED: return "unsupported Dk, Dv, chunk, num_segments, precision or pass";
    case GDN_ERR_WORKSPACE: return "workspace NULL or too small";
    case GDN_ERR_ALIAS: return "an output overlaps another tensor";
    case GDN_ERR_HIP: return "HIP launch failed";
    case GDN_ERR_SEQLENS: return "cu_seqlens not a non-decreasing 0..T sequence";
    case GDN_ERR_ALIGN: return "tensor pointer misaligned";
    case GDN_ERR_SCRATCH: return "problem needs more workspace than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

gdn_status gdn_workspace_size(const gdn_problem* p, int32_t pass, size_t* bytes) {
  if (!bytes) return GDN_ERR_NULL;
  Kind kind;
  switch (pass) {
    case GDN_PASS_CHUNK_FWD: kind = Kind::ChunkFwd; break;
    case GDN_PASS_CHUNK_BWD: kind = Kind::ChunkBwd; break;
    case GDN_PASS_RECURRENT_FWD: kind = Kind::RecFwd; break;
    case GDN_PASS_RECURRENT_BWD: kind = Kind::RecBwd; break;
    case GDN_PASS_KDA_FWD: kind = Kind::KdaFwd; break;
    case GDN_PASS_CHUNK_SAVED: kind = Kind::ChunkBwd; break;
    case GDN_PASS_KDA_BWD: kind = Kind::KdaBwd; break;
    case GDN_PASS_KDA_SAVED: kind = Kind::KdaBwd; break;
    default: return GDN_ERR_UNSUPPORTED;
  }
  Checked c;
  const gdn_status st = check_problem(p, kind, &c);
  if (st != GDN_OK) return st;
  *bytes = pass == GDN_PASS_CHUNK_SAVED ? saved_bytes_needed(p, c) : workspace_bytes(p, kind, c);
  return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* S0, void* o,
                         float* S_final, void* workspace, size_t ws_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::ChunkFwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, ng * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false}},
                     {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false},
                      {workspace, ws_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::ChunkFwd, c);
  if (need && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  gdn::FwdParams fp{};
  fp.q = q; fp.k = k; fp.v = v; fp.g = g; fp.beta = beta; fp.S0 = S0; fp.o = o;
  fp.S_final = S_final; fp.seq = seq_info(p);
  fp.tws = nullptr;
  char* const wsb = static_cast<char*>(workspace);
  const size_t pb = packed_slot_bytes(p, c);
  fp.tbws = wsb;
  fp.pws = wsb + pb;
  fp.gws = reinterpret_cast<float*>(wsb + pb + t_slot_bytes(p, c));
  fp.N = c.N; fp.H = p->H; fp.Dv = p->Dv;
  fp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  fp.scale = p->scale;
  fp.G = p->num_segments;
  fp.seg_ws = fp.G > 1 ? reinterpret_cast<float*>(wsb + pb + t_slot_bytes(p, c) + gate_slot_bytes(p, c)) : nullptr;
  return hip_status(gdn::launch_chunk_fwd(fp, p->Dk, c.bf16, c.fp32_products, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_kda_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* S0, void* o,
                             float* S_final, void* workspace, size_t ws_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::KdaFwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, nk * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false}},
                     {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false},
                      {workspace, ws_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::KdaFwd, c);
  if (need && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  gdn::KdaParams kp{};
  kp.q = q; kp.k = k; kp.v = v; kp.g = g; kp.beta = beta; kp.S0 = S0; kp.o = o; kp.S_final = S_final;
  kp.ws = workspace;
  kp.seq = seq_info(p);
  kp.N = c.N; kp.H = p->H; kp.Dv = p->Dv;
  kp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  kp.scale = p->scale;
  kp.G = p->num_segments;
  kp.seg_ws = kp.G > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kda_rec_region(p, c)) : nullptr;
  return hip_status(gdn::launch_kda_fwd(kp, p->Dk, c.bf16, static_cast<hipStream_t>(stream)));
}

// The per-channel-decay backward's buffer: the forward's records, fp32 T, Ab and P,
// and the state before and its gradient after every chunk (operand type).
struct KdaBwdLayout {
  void* rec;
  float* aux;
  char* states;
  char* dstates;
};
KdaBwdLayout kda_bwd_layout(const gdn_problem* p, const Checked& c, void* ws) {
  char* const b = static_cast<char*>(ws);
  const size_t rb = kda_rec_region(p, c), ab = kda_aux_region(p, c), sb = kda_state_region(p, c);
  return KdaBwdLayout{ws, reinterpret_cast<float*>(b + rb), b + rb + ab, b + rb + ab + sb};
}

// The forward part of the per-channel-decay backward: records, fp32 T, Ab and P, the
// state before every chunk; o and S_final too when given.
gdn_status kda_fwd_keep(const gdn_problem* p, const Checked& c, const KdaBwdLayout& l, const void* q,
                        const void* k, const void* v, const float* g, const float* beta, const float* S0,
                        void* o, float* S_final, hipStream_t s) {
  gdn::KdaParams kp{};
  kp.q = q; kp.k = k; kp.v = v; kp.g = g; kp.beta = beta; kp.S0 = S0; kp.o = o; kp.S_final = S_final;
  kp.ws = l.rec;
  kp.seq = seq_info(p);
  kp.N = c.N; kp.H = p->H; kp.Dv = p->Dv;
  kp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  kp.scale = p->scale;
  kp.G = 1;
  kp.aux = l.aux;
  kp.states = l.states;
  return hip_status(gdn::launch_kda_fwd(kp, p->Dk, c.bf16, s));
}

// The reverse passes of the per-channel-decay backward on a filled buffer.
gdn_status kda_bwd_from(const gdn_problem* p, const Checked& c, const KdaBwdLayout& l, const void* q,
                        const void* k, const void* v, const float* g, const float* beta, const void* dO,
                        const float* dS_final, void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dS0,
                        hipStream_t s) {
  gdn::KdaBwdParams bp{};
  bp.q = q; bp.k = k; bp.v = v; bp.g = g; bp.beta = beta; bp.dO = dO; bp.dS_final = dS_final;
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta; bp.dS0 = dS0;
  bp.rec = l.rec; bp.aux = l.aux; bp.states = l.states; bp.dstates = l.dstates;
  bp.seq = seq_info(p);
  bp.N = c.N; bp.H = p->H; bp.Dv = p->Dv;
  bp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  bp.scale = p->scale;
  return hip_status(gdn::launch_kda_bwd(bp, p->Dk, c.bf16, s));
}

gdn_status gdn_kda_chunk_bwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* S0, const void* dO,
                             const float* dS_final, void* dq, void* dk, void* dv, float* dg,
                             float* dbeta, float* dS0, void* workspace, size_t ws_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::KdaBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, nk * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false},
                      {dO, nv * c.io, 16, true}, {dS_final, ns * 4, 4, false}},
                     {{dq, nk * c.io, 16, true}, {dk, nk * c.io, 16, true}, {dv, nv * c.io, 16, true},
                      {dg, nk * 4, 4, true}, {dbeta, ng * 4, 4, true}, {dS0, ns * 4, 4, false},
                      {workspace, ws_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::KdaBwd, c);
  if (need && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const KdaBwdLayout l = kda_bwd_layout(p, c, workspace);
  st = kda_fwd_keep(p, c, l, q, k, v, g, beta, S0, nullptr, nullptr, s);
  if (st != GDN_OK) return st;
  return kda_bwd_from(p, c, l, q, k, v, g, beta, dO, dS_final, dq, dk, dv, dg, dbeta, dS0, s);
}

gdn_status gdn_kda_chunk_fwd_save(const gdn_problem* p, const void* q, const void* k, const void* v,
                                  const float* g, const float* beta, const float* S0, void* o,
                                  float* S_final, void* saved, size_t saved_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::KdaBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, nk * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false}},
                     {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false},
                      {saved, saved_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::KdaBwd, c);
  if (need && (!saved || saved_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  return kda_fwd_keep(p, c, kda_bwd_layout(p, c, saved), q, k, v, g, beta, S0, o, S_final,
                      static_cast<hipStream_t>(stream));
}

gdn_status gdn_kda_chunk_bwd_saved(const gdn_problem* p, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, const void* dO, const float* dS_final,
                                   void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dS0,
                                   void* saved, size_t saved_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::KdaBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, nk * 4, 4, true}, {beta, ng * 4, 4, true},
                      {dO, nv * c.io, 16, true}, {dS_final, ns * 4, 4, false}},
                     {{dq, nk * c.io, 16, true}, {dk, nk * c.io, 16, true}, {dv, nv * c.io, 16, true},
                      {dg, nk * 4, 4, true}, {dbeta, ng * 4, 4, true}, {dS0, ns * 4, 4, false},
                      {saved, saved_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::KdaBwd, c);
  if (need && (!saved || saved_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  return kda_bwd_from(p, c, kda_bwd_layout(p, c, saved), q, k, v, g, beta, dO, dS_final, dq, dk, dv, dg, dbeta,
                      dS0, static_cast<hipStream_t>(stream));
}

// The reverse passes of the backward on a filled buffer.
gdn_status launch_bwd_from(const gdn_problem* p, const Checked& c, const BwdLayout& l, const void* q,
                           const void* k, const void* v, const float* g, const float* beta, const void* dO,
                           const float* dS_final, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                           float* dS0, hipStream_t s) {
  gdn::BwdParams bp{};
  bp.q = q; bp.k = k; bp.v = v; bp.g = g; bp.beta = beta; bp.dO = dO; bp.dS_final = dS_final;
  bp.dq = dq; bp.dk = dk; bp.dv = dv; bp.dg = dg; bp.dbeta = dbeta; bp.dS0 = dS0;
  bp.tws = l.tws; bp.prws = l.prws; bp.states = l.states; bp.dstates = l.dstates; bp.seq = seq_info(p);
  bp.N = c.N; bp.H = p->H; bp.Dv = p->Dv;
  bp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  bp.scale = p->scale;
  return hip_status(gdn::launch_chunk_bwd(bp, p->Dk, c.bf16, s));
}

gdn_status gdn_chunk_bwd(const gdn_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* S0, const void* dO,
                         const float* dS_final, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* dS0, void* workspace, size_t ws_bytes,
                         void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::ChunkBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, ng * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false},
                      {dO, nv * c.io, 16, true}, {dS_final, ns * 4, 4, false}},
                     {{dq, nk * c.io, 16, true}, {dk, nk * c.io, 16, true}, {dv, nv * c.io, 16, true},
                      {dg, ng * 4, 4, true}, {dbeta, ng * 4, 4, true}, {dS0, ns * 4, 4, false},
                      {workspace, ws_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, Kind::ChunkBwd, c);
  if (need && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const BwdLayout l = bwd_layout(p, c, workspace);
  gdn::FwdParams fp{};
  fp.q = q; fp.k = k; fp.v = v; fp.g = g; fp.beta = beta; fp.S0 = S0;
  fp.tws = l.tws; fp.tbws = l.tbws; fp.pws = nullptr; fp.gws = l.gws; fp.prws = l.prws;
  fp.states = l.states; fp.seq = seq_info(p);
  fp.N = c.N; fp.H = p->H; fp.Dv = p->Dv;
  fp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  fp.scale = p->scale;
  fp.G = 1;
  st = hip_status(gdn::launch_chunk_fwd_states(fp, p->Dk, c.bf16, s));
  if (st != GDN_OK) return st;
  return launch_bwd_from(p, c, l, q, k, v, g, beta, dO, dS_final, dq, dk, dv, dg, dbeta, dS0, s);
}

gdn_status gdn_chunk_fwd_save(const gdn_problem* p, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* S0, void* o,
                              float* S_final, void* saved, size_t saved_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::ChunkBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, ng * 4, 4, true}, {beta, ng * 4, 4, true}, {S0, ns * 4, 4, false}},
                     {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false},
                      {saved, saved_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = saved_bytes_needed(p, c);
  if (need && (!saved || saved_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  const BwdLayout l = bwd_layout(p, c, saved);
  gdn::FwdParams fp{};
  fp.q = q; fp.k = k; fp.v = v; fp.g = g; fp.beta = beta; fp.S0 = S0; fp.o = o; fp.S_final = S_final;
  fp.tws = l.tws; fp.tbws = l.tbws; fp.pws = l.pws; fp.gws = l.gws; fp.prws = l.prws;
  fp.states = l.states; fp.seq = seq_info(p);
  fp.N = c.N; fp.H = p->H; fp.Dv = p->Dv;
  fp.max_chunks = static_cast<int32_t>((c.max_len + 63) / 64);
  fp.scale = p->scale;
  fp.G = 1;
  return hip_status(gdn::launch_chunk_fwd_save(fp, p->Dk, c.bf16, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_chunk_bwd_saved(const gdn_problem* p, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const void* dO, const float* dS_final,
                               void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dS0,
                               void* saved, size_t saved_bytes, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::ChunkBwd, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {v, nv * c.io, 16, true},
                      {g, ng * 4, 4, true}, {beta, ng * 4, 4, true},
                      {dO, nv * c.io, 16, true}, {dS_final, ns * 4, 4, false}},
                     {{dq, nk * c.io, 16, true}, {dk, nk * c.io, 16, true}, {dv, nv * c.io, 16, true},
                      {dg, ng * 4, 4, true}, {dbeta, ng * 4, 4, true}, {dS0, ns * 4, 4, false},
                      {saved, saved_bytes, 16, false}});
  if (st != GDN_OK) return st;
  const size_t need = saved_bytes_needed(p, c);
  if (need && (!saved || saved_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  return launch_bwd_from(p, c, bwd_layout(p, c, saved), q, k, v, g, beta, dO, dS_final, dq, dk, dv, dg, dbeta,
                         dS0, static_cast<hipStream_t>(stream));
}

gdn_status gdn_recurrent_ref(const gdn_problem* p, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const float* S0, void* o,
                             float* S_final, const void* dO, const float* dS_final, void* dq,
                             void* dk, void* dv, float* dg, float* dbeta, float* dS0,
                             void* workspace, size_t ws_bytes, void* stream) {
  const bool bwd = dO != nullptr;
  const Kind kind = bwd ? Kind::RecBwd : Kind::RecFwd;
  Checked c;
  gdn_status st = check_problem(p, kind, &c);
  if (st != GDN_OK) return st;
  const size_t nk = c.tokens * p->H * p->Dk, nv = c.tokens * p->H * p->Dv, ng = c.tokens * p->H;
  const size_t ns = static_cast<size_t>(c.N) * p->H * p->Dk * p->Dv;
  std::vector<Tensor> ins = {{q, nk * c.io, 16, true},   {k, nk * c.io, 16, true},
                             {v, nv * c.io, 16, true},   {g, ng * 4, 4, true},
                             {beta, ng * 4, 4, true},    {S0, ns * 4, 4, false}};
  std::vector<Tensor> outs = {{o, nv * c.io, 16, true}, {S_final, ns * 4, 4, false},
                              {workspace, ws_bytes, 16, false}};
  if (bwd) {
    ins.push_back({dO, nv * c.io, 16, true});
    ins.push_back({dS_final, ns * 4, 4, false});
    outs.push_back({dq, nk * c.io, 16, true});
    outs.push_back({dk, nk * c.io, 16, true});
    outs.push_back({dv, nv * c.io, 16, true});
    outs.push_back({dg, ng * 4, 4, true});
    outs.push_back({dbeta, ng * 4, 4, true});
    outs.push_back({dS0, ns * 4, 4, false});
  }
  st = check_tensors(ins, outs);
  if (st != GDN_OK) return st;
  const size_t need = workspace_bytes(p, kind, c);
  if (need && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
  if (c.N == 0) return GDN_OK;
  gdn::RecParams rp{};
  rp.q = q; rp.k = k; rp.v = v; rp.g = g; rp.beta = beta; rp.S0 = S0; rp.o = o;
  rp.S_final = S_final; rp.dO = dO; rp.dS_final = dS_final; rp.dq = dq; rp.dk = dk; rp.dv = dv;
  rp.dg = dg; rp.dbeta = dbeta; rp.dS0 = dS0;
  rp.ws = static_cast<float*>(workspace);
  rp.ckpt_stride = ((c.max_len + gdn::kRecBlock - 1) / gdn::kRecBlock) * p->Dk * p->Dv;
  rp.seq = seq_info(p);
  rp.N = c.N; rp.H = p->H; rp.Dv = p->Dv; rp.scale = p->scale;
  return hip_status(gdn::launch_recurrent(rp, p->Dk, c.bf16, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prologue(const gdn_problem* p, const void* q, const void* k, const float* a, const float* b,
                        const float* A_log, const float* dt_bias, int32_t gate_kind, int32_t allow_neg_eigval,
                        void* q_out, void* k_out, float* g, float* beta, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::RecFwd, &c);
  if (st != GDN_OK) return st;
  if (gate_kind != GDN_GATE_GDN && gate_kind != GDN_GATE_BOUNDED5 && gate_kind != GDN_GATE_GDN_CHANNEL)
    return GDN_ERR_UNSUPPORTED;
  const size_t nk = c.tokens * p->H * p->Dk, ng = c.tokens * p->H;
  const bool chan = gate_kind == GDN_GATE_GDN_CHANNEL;
  const bool gdn_gate = gate_kind != GDN_GATE_BOUNDED5;
  const size_t na = chan ? nk : ng;                                      // a and g elements
  const size_t nbias = static_cast<size_t>(p->H) * (chan ? p->Dk : 1);  // dt_bias elements
  st = check_tensors({{q, nk * c.io, 16, true}, {k, nk * c.io, 16, true}, {a, na * 4, chan ? 16u : 4u, true},
                      {b, ng * 4, 4, true}, {A_log, static_cast<size_t>(p->H) * 4, 4, gdn_gate},
                      {dt_bias, nbias * 4, chan ? 16u : 4u, gdn_gate}},
                     {{q_out, nk * c.io, 16, true}, {k_out, nk * c.io, 16, true}, {g, na * 4, chan ? 16u : 4u, true},
                      {beta, ng * 4, 4, true}});
  if (st != GDN_OK) return st;
  if (ng == 0) return GDN_OK;
  gdn::PrologueParams pp{};
  pp.q = q; pp.k = k; pp.a = a; pp.b = b; pp.A_log = A_log; pp.dt_bias = dt_bias;
  pp.q_out = q_out; pp.k_out = k_out; pp.g = g; pp.beta = beta;
  pp.rows = static_cast<int64_t>(ng); pp.H = p->H; pp.gate_kind = gate_kind; pp.allow_neg = allow_neg_eigval != 0;
  return hip_status(gdn::launch_prologue(pp, p->Dk, c.bf16, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_epilogue(const gdn_problem* p, const void* o, const void* z, const float* weight, float eps,
                        void* y, void* stream) {
  Checked c;
  gdn_status st = check_problem(p, Kind::RecFwd, &c);
  if (st != GDN_OK) return st;
  if ((p->Dv & (p->Dv - 1)) != 0) return GDN_ERR_UNSUPPORTED;
  const size_t nv = c.tokens * p->H * p->Dv;
  st = check_tensors({{o, nv * c.io, 16, true}, {z, nv * c.io, 16, true},
                      {weight, static_cast<size_t>(p->Dv) * 4, 16, false}},
                     {{y, nv * c.io, 16, true}});
  if (st != GDN_OK) return st;
  if (nv == 0) return GDN_OK;
  gdn::EpilogueParams ep{};
  ep.o = o; ep.z = z; ep.weight = weight; ep.y = y;
  ep.rows = static_cast<int64_t>(c.tokens) * p->H; ep.eps = eps;
  return hip_status(gdn::launch_epilogue(ep, p->Dv, c.bf16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
