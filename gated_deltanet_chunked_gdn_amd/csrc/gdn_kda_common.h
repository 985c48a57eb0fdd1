// Layouts shared by the per-key-channel-decay forward and backward kernels.
#pragma once
#include <stdint.h>

namespace gdn {
namespace kda {

// One (chunk slot, head) record written by the preparation kernel: five matrices
// in the MFMA operand type EL (bf16 for bf16 io, fp32 for fp32 io; element
// offsets below), then Gamma_n as DK floats at byte kGnByte.
template <int DK, typename EL>
struct Rec {
  static constexpr int kTb = 0;               // T diag(beta), 64 x 64, zero above the diagonal
  static constexpr int kP = 4096;             // P, 64 x 64, zero above the diagonal
  static constexpr int kKG = 8192;            // K o Gamma, 64 x DK
  static constexpr int kQG = kKG + 64 * DK;   // Q o Gamma, 64 x DK
  static constexpr int kKDt = kQG + 64 * DK;  // (K o exp(gamma_n - gamma))^T, DK x 64
  static constexpr int kElems = kKDt + 64 * DK;
  static constexpr int kGnByte = kElems * static_cast<int>(sizeof(EL));
  static constexpr int kBytes = kGnByte + DK * 4;
  static_assert(kGnByte % 4096 == 0 && kBytes % 16 == 0, "record alignment");
};

// fp32 matrices the preparation kernel also keeps for the backward, per (chunk
// slot, head): T = (I + A)^-1 (zero above the diagonal), the undecayed-beta key
// products Ab (A = diag(beta) Ab; meaningful below the diagonal only) and P
// (meaningful on and below the diagonal only).
struct Aux {
  static constexpr int kT = 0;
  static constexpr int kAb = 4096;
  static constexpr int kP = 8192;
  static constexpr int kFloats = 3 * 4096;
};

}  // namespace kda
}  // namespace gdn
