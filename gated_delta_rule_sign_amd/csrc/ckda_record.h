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
//   flag                                       uint32, then padding to 256 bytes
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
    // one 32-bit word: nonzero when the chunk's gates leave the anchored
    // factoring's range and the record comes from the exact path (chunk.hip).
    // The record is then padded to a multiple of 256 bytes, so every record
    // starts on a cache-line boundary: a record that straddles lines turns
    // its stores into partial-line writes.
    static constexpr size_t OFF_FLAG = OFF_U + static_cast<size_t>(64) * DV * 4;
    static constexpr size_t BYTES = (OFF_FLAG + 4 + 255) / 256 * 256;
    static_assert(OFF_U % 16 == 0 && OFF_FLAG % 16 == 0, "16-byte units");
};

// The record of the backward's reverse (state-gradient) pass: the same chunk
// quantities, transposed, since the adjoint of the state step
//   dU = scale M^T dO + KbT^T G,   G <- Diag(d) G + scale Qh^T dO - W^T dU
// (G = dL/dS at the chunk end, true frame) contracts every matrix over its
// other index.  Each A operand is then read along a contiguous K:
//   KB  = KbT^T = P_L kf e^{b_L - b}           [64][DK]  token-major
//   QT  = Qh^T                                 [DK][64]  channel-major
//   WT  = W^T                                  [DK][64]  channel-major
//   MT  = M^T (row = column token i; zero left of the diagonal and in the
//         blocks (16..31, 0..15), (48..63, 32..47) that 32-token steps read)
//                                              [64][64]
//   d   = P_L e^{b_L}                          [DK]      float32
//   flag                                       uint32, padding to 256 bytes
// Storage as in Record (hi/lo bf16 planes for bf16 inputs, fp32 otherwise).
template <int DK, int DV, bool F32>
struct RevRecord {
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NP = F32 ? 1 : 2;
    static constexpr int KB_ROW = DK * ES;
    static constexpr int QT_ROW = 64 * ES;
    static constexpr int WT_ROW = 64 * ES;
    static constexpr int MT_ROW = 64 * ES;
    static constexpr size_t OFF_KB = 0;
    static constexpr size_t KB_PLANE = 64 * KB_ROW;
    static constexpr size_t OFF_QT = OFF_KB + NP * KB_PLANE;
    static constexpr size_t QT_PLANE = static_cast<size_t>(DK) * QT_ROW;
    static constexpr size_t OFF_WT = OFF_QT + NP * QT_PLANE;
    static constexpr size_t WT_PLANE = static_cast<size_t>(DK) * WT_ROW;
    static constexpr size_t OFF_MT = OFF_WT + NP * WT_PLANE;
    static constexpr size_t MT_PLANE = 64 * MT_ROW;
    static constexpr size_t OFF_D = OFF_MT + NP * MT_PLANE;
    static constexpr size_t OFF_FLAG = OFF_D + DK * 4;
    static constexpr size_t BYTES = (OFF_FLAG + 4 + 255) / 256 * 256;
    static_assert(OFF_D % 16 == 0 && OFF_FLAG % 16 == 0, "16-byte units");
};

// What the backward's first chunk-parallel gradient phase hands to its second,
// per (chunk slot, head): dA = Diag(beta) strict_lower(dX) and
// dM = scale lower(dO U^T) ([64][64], row = output token; zero above the
// diagonal, also in the blocks (0..15, 16..31), (32..47, 48..63)), and U
// ([64][DV] token-major).  Storage as in Record.
template <int DK, int DV, bool F32>
struct GradOut {
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int NP = F32 ? 1 : 2;
    static constexpr int A_ROW = 64 * ES;
    static constexpr int U_ROW = DV * ES;
    static constexpr size_t A_PLANE = 64 * A_ROW;
    static constexpr size_t U_PLANE = 64 * U_ROW;
    static constexpr size_t OFF_DA = 0;
    static constexpr size_t OFF_DM = OFF_DA + NP * A_PLANE;
    static constexpr size_t OFF_U = OFF_DM + NP * A_PLANE;
    static constexpr size_t BYTES = (OFF_U + NP * U_PLANE + 255) / 256 * 256;
};

// chunk slot of chunk j of document d (varlen): floor(cu[d]/64) + d + j.
// Slots are distinct across documents and below ceil(T_total/64) + N.
__host__ __device__ inline int varlen_slot(int cu_d, int d, int j) { return cu_d / 64 + d + j; }

}  // namespace ckda
