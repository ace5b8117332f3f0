// ckda_record.h -- the per-(chunk, head) record that the chunk-local kernel
// writes to the forward workspace and the state-passing kernel reads.
//
// With b the in-chunk cumulative log-gate, P the in-chunk sign product,
// qf = P q, kf = P k, X = I + Diag(beta) A (A, M the strictly lower / lower
// intra-chunk key-key and query-key products, see chunk.hip):
//
//   W   = X^{-1} Diag(beta) (kf e^b)          [64][DK]  token-major
//   Qh  = qf e^b                               [64][DK]  token-major
//   KbT = (P_L kf e^{b_L - b})^T               [DK][64]  channel-major
//   M   (lower triangle, zero above the diagonal inside the 32x32 diagonal
//        blocks; blocks (0..31, 32..63) are never read)
//                                              [64][64]  row = output token
//   d   = P_L e^{b_L}                          [DK]      float32
//   u   = X^{-1} Diag(beta) V                  [64][DV]  float32, stored as
//         16x16 tiles (J, vt) in the MFMA C/D lane layout: element
//         (16J + 4g + i, 16vt + n) at ((J*DV/16 + vt)*64 + 16g + n)*4 + i
//
// so that one chunk's state step is
//   U = u - W S,   O = Qh S + M U,   S <- Diag(d) S + KbT U.
//
// Storage: bf16 inputs keep W, Qh, KbT and M as two bf16 planes (hi, then lo
// = bf16(x - hi)); fp32 inputs store every matrix as one fp32 plane.  (W in
// one bf16 rounding is enough while the gates decay, but where they do not,
// e.g. beta = 2 and |alpha| = 1, its rounding error is carried by the state
// from chunk to chunk and grows with the sequence.)  Every block is a whole
// number of 16-byte units.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace ckda {

template <int DK, int DV, bool F32>
struct Record {
    static constexpr int ES = F32 ? 4 : 2;   // bytes per element and plane
    static constexpr int NP = F32 ? 1 : 2;   // planes of W, Qh, KbT, M
    static constexpr int W_ROW = DK * ES;    // bytes per row
    static constexpr int Q_ROW = DK * ES;
    static constexpr int K_ROW = 64 * ES;
    static constexpr int M_ROW = 64 * ES;
    static constexpr size_t OFF_W = 0;
    static constexpr size_t W_PLANE = 64 * W_ROW;
    static constexpr size_t OFF_Q = OFF_W + NP * W_PLANE;
    static constexpr size_t Q_PLANE = 64 * Q_ROW;
    static constexpr size_t OFF_K = OFF_Q + NP * Q_PLANE;
    static constexpr size_t K_PLANE = static_cast<size_t>(DK) * K_ROW;
    static constexpr size_t OFF_M = OFF_K + NP * K_PLANE;
    static constexpr size_t M_PLANE = 64 * M_ROW;
    static constexpr size_t OFF_D = OFF_M + NP * M_PLANE;
    static constexpr size_t OFF_U = OFF_D + DK * 4;
    static constexpr size_t STAGED = OFF_U;   // W .. d: staged whole by the state kernel
    static constexpr size_t BYTES = OFF_U + static_cast<size_t>(64) * DV * 4;
    static_assert(OFF_U % 16 == 0 && BYTES % 16 == 0, "16-byte units");
};

// chunk slot of chunk j of document d (varlen): floor(cu[d]/64) + d + j.
// Slots are distinct across documents and below ceil(T_total/64) + N.
__host__ __device__ inline int varlen_slot(int cu_d, int d, int j) { return cu_d / 64 + d + j; }

}  // namespace ckda
