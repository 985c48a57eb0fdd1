// Drives the host side of the C ABI (gdn_abi.cpp, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against launcher stand-ins): status strings, workspace
// sizes over a grid of problems up to the documented limits, and every entry point
// with invalid arguments (each must fail before any launch) and with valid-looking
// ones (which reach the stand-in launchers and report GDN_ERR_HIP).  Pointers are
// fake device addresses: the shim never dereferences them.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "gdn.h"

extern int g_launches;

namespace {

int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

gdn_problem problem(int B, int T, int H, int Dk, int Dv, int io = GDN_BF16, int G = 1) {
  gdn_problem p{};
  p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.num_seqs = B;
  p.io_dtype = io; p.scale = 1.0f; p.chunk = 64; p.num_segments = G; p.precision = GDN_PRECISION_IO;
  return p;
}

// 14 fake, 16-byte aligned device addresses 1 GiB apart
void* fake(int i) { return reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000000000ull) + (static_cast<uintptr_t>(i) << 30)); }
float* ffake(int i) { return static_cast<float*>(fake(i)); }

}  // namespace

int main() {
  EXPECT(gdn_abi_version() == GDN_ABI_VERSION);
  for (int s = -3; s < 16; ++s) EXPECT(gdn_status_str(s) != nullptr);

  // workspace sizes: every pass over a grid of shapes, dtypes, segment counts and policies
  size_t bytes = 0;
  EXPECT(gdn_workspace_size(nullptr, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_NULL);
  gdn_problem p0 = problem(1, 64, 1, 64, 64);
  EXPECT(gdn_workspace_size(&p0, GDN_PASS_CHUNK_FWD, nullptr) == GDN_ERR_NULL);
  EXPECT(gdn_workspace_size(&p0, 99, &bytes) == GDN_ERR_UNSUPPORTED);
  const int Ts[] = {0, 1, 63, 64, 65, 1000, 65536};
  const int Hs[] = {1, 3, 64};
  const int Ds[] = {16, 48, 64, 80, 128, 256, 512};
  const int Gs[] = {1, 2, 3, 16};
  long ok = 0, rejected = 0;
  for (int pass = 0; pass <= 6; ++pass)
    for (int T : Ts)
      for (int H : Hs)
        for (int Dk : Ds)
          for (int Dv : Ds)
            for (int io : {static_cast<int>(GDN_FP32), static_cast<int>(GDN_BF16), 7})
              for (int G : Gs)
                for (int prec : {0, 1, 5}) {
                  gdn_problem p = problem(2, T, H, Dk, Dv, io, G);
                  p.precision = prec;
                  const gdn_status st = gdn_workspace_size(&p, pass, &bytes);
                  if (st == GDN_OK) ++ok; else ++rejected;
                }
  EXPECT(ok > 0 && rejected > 0);
  // limits: sizes that would overflow 32-bit offsets or grid dimensions are refused
  {
    gdn_problem p = problem(1, 64, 70000, 128, 128);
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_UNSUPPORTED);
    p = problem(-1, 64, 1, 64, 64);
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_SHAPE);
    p = problem(1, 64, 1, 64, 64);
    p.chunk = 32;
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_UNSUPPORTED);
  }

  // packed sequences: valid and invalid host offsets
  {
    const int32_t cu_ok[] = {0, 0, 37, 200};
    const int32_t cu_bad[] = {0, 50, 40, 200};
    const int32_t cu_end[] = {0, 10, 20, 199};
    gdn_problem p = problem(1, 200, 3, 64, 64);
    p.num_seqs = 3;
    p.cu_seqlens_host = cu_ok;
    p.cu_seqlens_dev = reinterpret_cast<const int32_t*>(fake(20));
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_OK);
    p.cu_seqlens_host = cu_bad;
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_SEQLENS);
    p.cu_seqlens_host = cu_end;
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_ERR_SEQLENS);
    p.cu_seqlens_host = cu_ok;
    p.cu_seqlens_dev = nullptr;
    EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) != GDN_OK);
  }

  const int launches0 = g_launches;
  gdn_problem p = problem(2, 300, 3, 128, 64);
  // forward: a NULL input, an overlap, a misalignment, a short workspace: no launch
  EXPECT(gdn_workspace_size(&p, GDN_PASS_CHUNK_FWD, &bytes) == GDN_OK);
  EXPECT(gdn_chunk_fwd(&p, nullptr, fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6), fake(7),
                       bytes, nullptr) == GDN_ERR_NULL);
  EXPECT(gdn_chunk_fwd(&p, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr,
                       static_cast<char*>(fake(0)) + 4096, ffake(6), fake(7), bytes, nullptr) == GDN_ERR_ALIAS);
  EXPECT(gdn_chunk_fwd(&p, static_cast<char*>(fake(0)) + 2, fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5),
                       ffake(6), fake(7), bytes, nullptr) == GDN_ERR_ALIGN);
  EXPECT(gdn_chunk_fwd(&p, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6), fake(7),
                       bytes - 1, nullptr) == GDN_ERR_WORKSPACE);
  EXPECT(g_launches == launches0);
  // ... and valid-looking calls reach the launchers
  EXPECT(gdn_chunk_fwd(&p, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6), fake(7),
                       bytes, nullptr) == GDN_ERR_HIP);
  for (int G : {2, 4, 16}) {
    gdn_problem pg = problem(2, 300, 3, 128, 64, GDN_BF16, G);
    size_t b = 0;
    EXPECT(gdn_workspace_size(&pg, GDN_PASS_CHUNK_FWD, &b) == GDN_OK);
    EXPECT(gdn_chunk_fwd(&pg, fake(0), fake(1), fake(2), ffake(3), ffake(4), ffake(8), fake(5), ffake(6), fake(7),
                         b, nullptr) == GDN_ERR_HIP);
    EXPECT(gdn_kda_chunk_fwd(&pg, fake(0), fake(1), fake(2), ffake(3), ffake(4), ffake(8), fake(5), ffake(6),
                             fake(7), 1ull << 29, nullptr) != GDN_OK);
  }
  // backward and the retained-state pair
  gdn_problem pb = problem(2, 300, 3, 64, 128);
  size_t bw = 0, sv = 0;
  EXPECT(gdn_workspace_size(&pb, GDN_PASS_CHUNK_BWD, &bw) == GDN_OK);
  EXPECT(gdn_workspace_size(&pb, GDN_PASS_CHUNK_SAVED, &sv) == GDN_OK && sv > bw);
  EXPECT(gdn_chunk_bwd(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), nullptr, fake(6),
                       fake(7), fake(8), ffake(9), ffake(10), nullptr, fake(11), bw, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_chunk_bwd(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), nullptr, fake(6),
                       fake(7), fake(8), ffake(9), ffake(10), nullptr, fake(11), bw - 16, nullptr) == GDN_ERR_WORKSPACE);
  EXPECT(gdn_chunk_fwd_save(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6), fake(7),
                            sv, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_chunk_bwd_saved(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), fake(5), nullptr, fake(6), fake(7),
                             fake(8), ffake(9), ffake(10), ffake(12), fake(11), sv, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_chunk_bwd_saved(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), fake(5), nullptr, fake(6), fake(7),
                             fake(8), ffake(9), ffake(10), ffake(12), fake(2), sv, nullptr) == GDN_ERR_ALIAS);
  // per-channel-decay backward: g and dg span Dk floats per token-head
  size_t kw = 0;
  EXPECT(gdn_workspace_size(&pb, GDN_PASS_KDA_BWD, &kw) == GDN_OK && kw > 0);
  EXPECT(gdn_kda_chunk_bwd(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), nullptr, fake(6),
                           fake(7), fake(8), ffake(9), ffake(10), nullptr, fake(11), kw, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_kda_chunk_bwd(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), nullptr, fake(6),
                           fake(7), fake(8), ffake(9), ffake(10), nullptr, fake(11), kw - 16, nullptr) ==
         GDN_ERR_WORKSPACE);
  size_t ks = 0;
  EXPECT(gdn_workspace_size(&pb, GDN_PASS_KDA_SAVED, &ks) == GDN_OK && ks == kw);
  EXPECT(gdn_kda_chunk_fwd_save(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6),
                                fake(7), ks, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_kda_chunk_bwd_saved(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), fake(5), nullptr, fake(6),
                                 fake(7), fake(8), ffake(9), ffake(10), ffake(12), fake(11), ks, nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_kda_chunk_bwd_saved(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), fake(5), nullptr, fake(6),
                                 fake(7), fake(8), ffake(9), ffake(10), ffake(12), fake(2), ks, nullptr) ==
         GDN_ERR_ALIAS);
  gdn_problem pk2 = problem(2, 300, 3, 64, 128, GDN_BF16, 2);
  EXPECT(gdn_kda_chunk_bwd(&pk2, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), nullptr, fake(6),
                           fake(7), fake(8), ffake(9), ffake(10), nullptr, fake(11), kw, nullptr) ==
         GDN_ERR_UNSUPPORTED);
  // recurrent reference, prologue, epilogue
  size_t rw = 0;
  EXPECT(gdn_workspace_size(&pb, GDN_PASS_RECURRENT_BWD, &rw) == GDN_OK);
  EXPECT(gdn_recurrent_ref(&pb, fake(0), fake(1), fake(2), ffake(3), ffake(4), nullptr, fake(5), ffake(6), fake(7),
                           nullptr, fake(8), fake(9), fake(10), ffake(11), ffake(12), nullptr, fake(13), rw,
                           nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_prologue(&pb, fake(0), fake(1), ffake(2), ffake(3), ffake(4), ffake(5), 0, 0, fake(6), fake(7),
                      ffake(8), ffake(9), nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_prologue(&pb, fake(0), fake(1), ffake(2), ffake(3), ffake(4), ffake(5), 99, 0, fake(6), fake(7),
                      ffake(8), ffake(9), nullptr) != GDN_OK);
  EXPECT(gdn_epilogue(&pb, fake(0), fake(1), ffake(2), 1e-6f, fake(3), nullptr) == GDN_ERR_HIP);
  EXPECT(gdn_epilogue(&pb, fake(0), fake(1), ffake(2), 1e-6f, fake(0), nullptr) == GDN_ERR_ALIAS);
  // empty problem: nothing to launch
  gdn_problem pe = problem(0, 0, 3, 64, 64);
  EXPECT(gdn_workspace_size(&pe, GDN_PASS_CHUNK_FWD, &bytes) == GDN_OK && bytes == 0);

  std::printf("%s: %ld sizes accepted, %ld refused, %d launches, %d failures\n", failures ? "FAILED" : "ok", ok,
              rejected, g_launches - launches0, failures);
  return failures ? 1 : 0;
}
