// Host-visible kernel parameter blocks and launchers of libgdn (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// gdn_chunk_fwd's host checks of the problem and of every tensor except the
// workspace (include/gdn.h); on success *ws_need is the workspace it needs.
gdn_status check_chunk_fwd(const gdn_problem* p, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* S0, const void* o, const float* S_final,
                           size_t* ws_need);

// Sequence n covers packed rows [bos, bos + len): from cu (device) when given,
// else the dense batch row n * T .. n * T + T.
struct SeqInfo {
  const int32_t* cu;  // device offsets or nullptr
  int32_t T;          // dense sequence length (unused when cu != nullptr)
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* S0;  // [N, H, Dk, Dv] or nullptr
  void* o;
  float* S_final;   // [N, H, Dk, Dv] or nullptr
  void* tws;        // per-chunk T = (I + A)^-1 (io element type, 64 x 64 per slot), or nullptr
  void* tbws;       // per-chunk T diag(beta), lower blocks packed (kLPack io elements per slot)
  void* pws;        // per-chunk P = lower_incl((Q K^T) o D) in MFMA operand order (4096 io
                    // elements per slot: fragment (row block, k-step) of 64 lanes each), or nullptr
  float* gws;       // per-chunk Gamma and exp(gamma_n - gamma), [slot][H][128] fp32
  void* prws;       // per-chunk P row-major for the backward (64 x 64 io elements per slot,
                    // zeros above the diagonal), or nullptr
  SeqInfo seq;
  int32_t N, H, Dv;
  int32_t max_chunks;  // chunks of the longest sequence
  float scale;
  // Segment split: every sequence is cut into G runs of whole chunks; segment
  // sigma covers chunks [sigma L, min((sigma + 1) L, nch)), L = ceil(nch / G).
  // One launch of the state kernel covers segments seg_base .. seg_base + nseg - 1.
  int32_t G, seg_base, nseg;
  int32_t start_mode;  // kStartS0 / kStartZero / kStartIdentity / kStartCarry
  int32_t write_o;     // kOutNone / kOutAll / kOutSeg0
  int32_t zero_u;      // U = 0: propagate transition maps instead of states
  int32_t ncol;        // state columns: Dv, or Dk for transition maps
  const float* carry;  // [G][N][H][Dk][ncol] start states (kStartCarry)
  float* seg_out;      // [G][N][H][Dk][ncol] end states, or nullptr
  int32_t final_to_sfinal;  // segment G - 1 writes S_final (layout [N][H][Dk][Dv])
  float* seg_ws;       // G > 1: ends, starts ([G][N][H][Dk][Dv] each), maps ([G][N][H][Dk][Dk])
  void* states;        // or nullptr: S_c before every chunk, [chunk slot][H][Dk][Dv] in the
                       // operand type (bf16 for bf16 products, fp32 for fp32 products)
};

enum : int32_t { kStartS0 = 0, kStartZero = 1, kStartIdentity = 2, kStartCarry = 3 };
enum : int32_t { kOutNone = 0, kOutAll = 1, kOutSeg0 = 2 };

struct CarryParams {
  const float* ends;   // [G][N][H][Dk][Dv]: end state of each segment run from its own start
  const float* maps;   // [G][N][H][Dk][Dk]: transition map of each segment
  float* starts;       // [G][N][H][Dk][Dv]: start states, written for sigma = 1 .. G - 1
  int32_t G, N, H, Dk, Dv;
};

// Chunk slots of the T workspace.  Chunk c of sequence n (first row bos) uses
// slot bos / 64 + n + c; slots of different sequences never overlap because a
// sequence of len rows has at most floor((bos + len) / 64) - floor(bos / 64) + 1
// chunks.  Total slots: floor(total_rows / 64) + N + 1.
inline int64_t chunk_slots(int64_t total_rows, int64_t N) { return total_rows / 64 + N + 1; }

// A 64 x 64 matrix that is zero above its 16x16 block diagonal, stored packed:
// row block rb (16 rows of 16 (rb + 1) entries, row-major) at element 128 rb (rb + 1).
constexpr int kLPack = 2560;
__host__ __device__ constexpr int lpack_base(int rb) { return 128 * rb * (rb + 1); }
// Elements of the per-chunk T diag(beta) record: the packed lower blocks (fp32 io),
// or, for bf16 io, six MFMA operand fragments of 64 lanes x 8 entries: fragment
// (row block mb, reduction step s), s <= mb / 2, lane (m, g) = (lane % 16, lane / 16)
// holding row 32 (mb / 2) + 8 (m / 4) + 4 (mb % 2) + m % 4, columns 32 s + 8 g + 0..7.
constexpr int kTbSlot = 3072;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const void* dO;
  const float* dS_final;  // or nullptr (zero)
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dS0;             // or nullptr (not wanted)
  const void* tws;        // T of every chunk slot (io element type, 64 x 64)
  const void* prws;       // P of every chunk slot, row-major (io element type, 64 x 64)
  const void* states;     // S_c before every chunk, [slot][H][Dk][Dv], operand type (as FwdParams)
  void* dstates;          // dS_{c+1} after every chunk, [slot][H][Dk][Dv], operand type
  SeqInfo seq;
  int32_t N, H, Dv;
  int32_t max_chunks;
  float scale;
};

struct RecParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* S0;
  void* o;
  float* S_final;
  const void* dO;        // nullptr: forward only
  const float* dS_final;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* dbeta;
  float* dS0;
  float* ws;             // workspace (backward: checkpoints and replay buffers)
  int64_t ckpt_stride;   // floats of checkpoints per (sequence, head)
  SeqInfo seq;
  int32_t N, H, Dv;
  float scale;
};

constexpr int kRecBlock = 16;  // tokens per replay block of the recurrent backward

struct PrologueParams {
  const void* q;
  const void* k;
  const float* a;
  const float* b;
  const float* A_log;    // [H] (gate_kind 0)
  const float* dt_bias;  // [H] (gate_kind 0)
  void* q_out;
  void* k_out;
  float* g;
  float* beta;
  int64_t rows;          // B * T * H token-heads
  int32_t H;
  int32_t gate_kind;     // 0: -exp(A_log) softplus(a + dt_bias); 1: -5 sigmoid(a);
                         // 2: form 0 per key channel (a, g [rows][Dk], dt_bias [H][Dk])
  int32_t allow_neg;     // beta = 2 sigmoid(b)
};

// Launchers; return hipSuccess or the launch error.  `dk`/`dv` are the head sizes,
// `bf16` selects the io dtype.
// fp32_products: IEEE fp32 products for bf16 io (the inputs widened exactly, o rounded once)
hipError_t launch_chunk_fwd(const FwdParams& p, int Dk, bool bf16, bool fp32_products, hipStream_t s);
// The bf16 state pass (one launch): `states` stores S_c before every chunk, `out`
// forms the output.  Reads the bf16 T diag(beta) fragments, P and the decays.
hipError_t launch_state_chain(const FwdParams& p, int Dk, bool states, bool out, hipStream_t s);
// T, T diag(beta) and the decays of every chunk slot, and the per-chunk states
// (no outputs): the forward half of the chunked backward.  Uses p.tws, p.tbws,
// p.gws and p.states; G must be 1.
hipError_t launch_chunk_fwd_states(const FwdParams& p, int Dk, bool bf16, hipStream_t s);
// Forward with o and S_final that also keeps the backward's records (T, T
// diag(beta), decays, P row-major in prws; P in operand order in pws) and the
// state before every chunk (states).
hipError_t launch_chunk_fwd_save(const FwdParams& p, int Dk, bool bf16, hipStream_t s);
// Bytes of forward workspace beyond the per-chunk records for G segments (0 for G = 1).
inline size_t segment_ws_bytes(int G, int N, int H, int Dk, int Dv) {
  if (G <= 1) return 0;
  const size_t nh = static_cast<size_t>(G) * N * H * Dk;
  return (2 * nh * Dv + nh * Dk) * sizeof(float);
}
// Reverse state-gradient pass and per-chunk gradients; needs b.tws and b.states
// filled by launch_chunk_fwd_states.
hipError_t launch_chunk_bwd(const BwdParams& b, int Dk, bool bf16, hipStream_t s);
hipError_t launch_recurrent(const RecParams& p, int Dk, bool bf16, hipStream_t s);
hipError_t launch_prologue(const PrologueParams& p, int Dk, bool bf16, hipStream_t s);

struct EpilogueParams {
  const void* o;
  const void* z;
  const float* weight;  // [Dv] or nullptr (ones)
  void* y;
  int64_t rows;         // B * T * H token-heads
  float eps;
};
hipError_t launch_epilogue(const EpilogueParams& p, int Dv, bool bf16, hipStream_t s);

// Chunked forward with one log-decay per key channel (g shaped like q).
struct KdaParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;        // [rows][H][Dk]
  const float* beta;     // [rows][H]
  const float* S0;       // [N, H, Dk, Dv] or nullptr
  void* o;
  float* S_final;        // [N, H, Dk, Dv] or nullptr
  void* ws;              // one record of kda_rec_bytes(Dk, bf16) bytes per (chunk slot, head)
  SeqInfo seq;
  int32_t N, H, Dv;
  int32_t max_chunks;
  float scale;
  // Segment split, as FwdParams: segment sigma covers chunks [sigma L, min((sigma +
  // 1) L, nch)), L = ceil(nch / G); one launch covers segments seg_base ..
  // seg_base + nseg - 1.
  int32_t G, seg_base, nseg;
  int32_t start_mode;       // kStartS0 / kStartZero / kStartIdentity / kStartCarry
  int32_t write_o;          // kOutNone / kOutAll / kOutSeg0
  int32_t zero_u;           // V = 0: propagate transition maps instead of states
  int32_t ncol;             // state columns: Dv, or Dk for transition maps
  const float* carry;       // [G][N][H][Dk][ncol] start states (kStartCarry)
  float* seg_out;           // [G][N][H][Dk][ncol] end states, or nullptr
  int32_t final_to_sfinal;  // segment G - 1 writes S_final
  float* seg_ws;            // G > 1: end states, start states, maps (segment_ws_bytes)
  // For the backward (nullptr otherwise): the prep kernel also writes T, Ab and P
  // in fp32 (kda::Aux floats per (chunk slot, head)); the state kernel writes the
  // state before every chunk, [slot][H][Dk][Dv] in the operand type (bf16 for bf16
  // io, fp32 for fp32 io).
  float* aux;
  void* states;
};
// Per (chunk slot, head): T diag(beta) and P (64 x 64 each), K o Gamma, Q o Gamma
// and (K o exp(gamma_n - gamma))^T (64 x Dk each) in the io element type (the
// MFMA operand type), then Gamma_n (Dk fp32).
inline size_t kda_rec_bytes(int Dk, bool bf16) {
  return (8192 + 3 * 64 * static_cast<size_t>(Dk)) * (bf16 ? 2 : 4) + 4 * static_cast<size_t>(Dk);
}
hipError_t launch_kda_fwd(const KdaParams& p, int Dk, bool bf16, hipStream_t s);
// Backward of the per-key-channel-decay pass on records, aux matrices and per-chunk
// states already written (launch_kda_fwd with aux and states set): the reverse
// state-gradient pass (dS after every chunk into dstates; dS0) and the per-chunk
// gradient kernel.
struct KdaBwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const void* dO;
  const float* dS_final;  // [N, H, Dk, Dv] or nullptr (zero)
  void* dq;
  void* dk;
  void* dv;
  float* dg;              // [rows][H][Dk]
  float* dbeta;           // [rows][H]
  float* dS0;             // [N, H, Dk, Dv] or nullptr
  const void* rec;        // the forward's records
  const float* aux;
  const void* states;     // [slot][H][Dk][Dv], operand type (as KdaParams::states)
  void* dstates;          // dS after every chunk, [slot][H][Dk][Dv], operand type
  SeqInfo seq;
  int32_t N, H, Dv;
  int32_t max_chunks;
  float scale;
};
hipError_t launch_kda_bwd(const KdaBwdParams& p, int Dk, bool bf16, hipStream_t s);
// Start states of segments 1 .. G - 1 composed in fp32 from the segments' end
// states b (ends, from zero; segment 0 from S0) and transition maps M (maps):
// starts[s + 1] = M_s starts[s] + b_s, starts[1] = ends[0].  Layouts [G][N][H][Dk][Dv]
// and [G][N][H][Dk][Dk].
hipError_t launch_segment_carry(const float* ends, const float* maps, float* starts, int G, int N, int H, int Dk,
                                int Dv, hipStream_t s);
size_t recurrent_bwd_ws_floats(int N, int H, int Dk, int Dv, int64_t max_len);

}  // namespace gdn
