// ckda_chunk.h -- the chunk-local kernel body shared by the chunked forward
// (chunk.hip), the backward's reverse-record pass (chunk_rev.hip) and its
// first chunk-parallel gradient phase (chunk_grad.hip); each of those files
// instantiates one mode, so the three compile in parallel.
//
// Method: the KDA-style WY/UT chunk-wise form of the recurrence (Complex KDA
// paper page, section 2 "Linear RNNs": DeltaNet/KDA admit WY-based
// chunk-wise implementations; section 1: the kernels are a small change to
// KDA's), with the signed gate carried as log-magnitude plus a running sign
// product pushed onto q and k ("complex-kda-1.3B-100B" model card).  Per
// chunk of 64 tokens, in the chunk-local folded frame (the sign product
// restarts at +1 at every chunk):
//
//   b_r = sum_{i<=r} g_i,  P_r = prod_{i<=r} s_i,  qf = P q,  kf = P k
//   A_ri = sum_c kf_rc kf_ic e^{b_rc - b_ic}  (i < r),  M_ri likewise with qf_r (i <= r)
//   X = I + Diag(beta) A
//
// Everything here is independent of the state, so this kernel runs one
// workgroup per (chunk, head) over the whole input at once and writes the
// record described in ckda_record.h (W, u, Qh, KbT, M, d); the state-passing
// kernel (state.hip) then only runs the S-dependent products per chunk.
//
// Workgroup: 4 * DK/CG waves (CG = min(DK, 64) channels per wave).  Wave w
// owns token tile R = w % 4 (tokens 16R..16R+15) and channel group w / 4;
// lane (n, g) holds token 16R + n and channels c0 + 0..7 of every 32-channel
// step, which is exactly the B-operand layout of v_mfma_f32_16x16x32: the
// row operands of the A/M products never leave registers.
//  1. per-channel inclusive scans over the tile's 16 tokens (DPP row scans),
//     tile totals exchanged through LDS;
//  2. exponentials, anchored at b of token 15 (tokens 0..31) or token 47
//     (tokens 32..63): row operands kf e^{b - m}, qf e^{b - m} (registers),
//     column operand kf e^{m - b} (LDS); the cross-half block uses
//     kf e^{m1 - b} for its half-0 columns, so every factor is bounded by the
//     decay over half a chunk;
//  3. A^T / M^T tiles on the matrix cores (split precision for bf16 inputs,
//     fp32 matrix cores for fp32 inputs);
//  4. inverses of the four 16x16 diagonal blocks of X, then the block
//     forward substitution X [W | u] = Diag(beta) [kf e^b | V] on 16x16x16
//     matrix-core products, one 16-column tile per wave at a time.
#pragma once
#include <type_traits>

#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"
#include "ckda_record.h"
#include "ckda_sync.h"

namespace ckda {

template <int DK>
struct ChunkShape {
    static constexpr int CG = DK < 64 ? DK : 64;   // channels per wave
    static constexpr int NCG = DK / CG;            // channel groups
    static constexpr int NW = 4 * NCG;             // waves
    static constexpr int KSW = CG / 32;            // 32-channel steps per wave
    static constexpr int NE = 8 * KSW;             // elements per lane
    static_assert(NCG <= 2, "at most two channel groups");
    static constexpr int PC = DK + 8;              // column-operand pitch (elements)
    static constexpr int PY = 16 + 4;              // diagonal-inverse pitch
    // LDS (bytes).  Phase A: totals, beta, column operands, partial tiles;
    // phase B (after the A/M tiles) reuses the column-operand space: the row
    // operand kf e^{b - m} over colk, the diagonal blocks, off-diagonal blocks
    // and diagonal inverses over colkf.
    static constexpr int L_TOTB = 0;                          // float [4][DK]
    static constexpr int L_TOTP = L_TOTB + 4 * DK * 4;        // uint32 [4][DK/4]
    static constexpr int L_BETA = L_TOTP + 4 * (DK / 4) * 4;  // float [64]
    static constexpr int L_NRM = L_BETA + 64 * 4;             // float2 [NCG][64]: sum k^2, sum q^2
    static constexpr int L_FLAG = L_NRM + NCG * 64 * 8;       // uint32 [16]: per-wave envelope flags
    static constexpr int L_COLK = L_FLAG + 64;                // operand [64][PC]
    static constexpr int L_COLKF = L_COLK + 64 * PC * 4;      // operand [32][PC]
    static constexpr int L_PART = L_COLKF + 32 * PC * 4;      // f32x4 [20][64]
    static constexpr int SZ_PART = NCG > 1 ? 20 * 64 * 16 : 0;
    static constexpr int L_RK = L_COLK;                       // operand [64][PC]: kf e^{b - m}
    static constexpr int L_LDIAG = L_COLKF;                   // float [4][16][17]
    static constexpr int L_LOFF = L_LDIAG + 4 * 16 * 17 * 4;  // operand [6*64][4]
    static constexpr int L_Y = L_LOFF + 6 * 64 * 4 * 4;       // operand [64][PY]
    static constexpr int L_BEND = L_Y + 64 * PY * 4;
    static_assert(SZ_PART == 0 || L_BEND <= L_PART, "phase B must not reach the partial tiles");
    static constexpr int LDS = (L_PART + SZ_PART) > L_BEND ? (L_PART + SZ_PART) : L_BEND;
    static_assert(LDS <= 80 * 1024, "two workgroups per CU");
    static_assert((L_COLK % 16) == 0 && (L_COLKF % 16) == 0 && (L_PART % 16) == 0 && (L_LDIAG % 16) == 0 &&
                  (L_LOFF % 16) == 0 && (L_Y % 16) == 0, "align");
    // exact path (phase A only): kf and b (log2 units) of every token as fp32
    // rows of XP floats, over the operand and partial-tile areas
    static constexpr int XP = DK + 8;
    static constexpr int L_XK = L_COLK;
    static constexpr int L_XB = L_XK + 64 * XP * 4;
    static constexpr int L_XEND = L_XB + 64 * XP * 4;
    static constexpr int LDS_EX = L_XEND > LDS ? L_XEND : LDS;
    static_assert(LDS_EX <= 80 * 1024 && (L_XB % 16) == 0, "two workgroups per CU");
};

// LDS of the backward's first gradient phase, after the chunk-local prologue
// (kModeGrad): Xi = X^{-1} and its transpose over the diagonal-inverse and
// partial-tile areas, then U and Y ([64][DV], token-major) for the
// contractions over the value channels, over the Ke rows and Xi when each wave
// holds one value tile (OVL) and after them otherwise; per-value-tile partial
// sums of the beta gradient last.
template <int DK, int DV>
struct GradShape {
    using SH = ChunkShape<DK>;
    static constexpr int VPW = (DV / 16 + SH::NW - 1) / SH::NW;   // value tiles per wave
    static constexpr bool OVL = VPW == 1;
    static constexpr int PX = 64 + 8;                 // Xi pitch (elements)
    static constexpr int PU = DV + 8;                 // U, Y pitch
    static constexpr int L_XI = SH::L_COLKF;
    static constexpr int L_XIT = L_XI + 64 * PX * 4;
    static constexpr int L_XEND = L_XIT + 64 * PX * 4;
    static constexpr int L_UT = OVL ? SH::L_COLK : L_XEND;
    static constexpr int L_YT = L_UT + 64 * PU * 4;
    static constexpr int L_UEND = L_YT + 64 * PU * 4;
    static constexpr int L_DBR = L_UEND > L_XEND ? L_UEND : L_XEND;   // float [DV/16][64]
    static constexpr int L_END = L_DBR + (DV / 16) * 64 * 4;
    static constexpr int LDS0 = L_END > SH::LDS ? L_END : SH::LDS;
    static constexpr int LDS = LDS0 > SH::LDS_EX ? LDS0 : SH::LDS_EX;
    static_assert(LDS <= 160 * 1024 && (L_XIT % 16) == 0 && (L_UT % 16) == 0 && (L_YT % 16) == 0 &&
                  (L_DBR % 16) == 0, "LDS");
    static_assert(!OVL || L_UEND <= L_DBR, "layout");
};

// Largest |in-tile prefix of the log-gate| (log2 units) the anchored
// factoring takes.  With g <= 0 every anchored exponent x = b - m of a token
// is bounded by its 16-token tile's total, so the row and column factors e^x,
// e^-x stay within [2^-96, 2^96], and a product term flushed below fp32's
// normal range is at most 2^-30 of the entries it feeds.  A chunk beyond it in
// any channel (or with any g > 0) is redone by the exact path.
constexpr float kEnvelope = 96.f;

constexpr int kModeFwd = 0, kModeRev = 1, kModeGrad = 2;

// off-diagonal 16x16 block index of (J, K), K < J
__device__ __forceinline__ int loff_index(int J, int K) { return (J * (J - 1)) / 2 + K; }
// lower 16x16 block (R, I), I <= R
__device__ __forceinline__ int tri_index(int R, int I) { return (R * (R + 1)) / 2 + I; }

struct ChunkParams {
    const void *q, *k, *v;
    const float* g;
    const int8_t* s;
    const float* beta;
    unsigned char* ws;
    const int32_t* cu;   // varlen document starts (device), or nullptr
    int T, H, ndocs;
    int gate_map;        // g, beta hold pre-activations (CKDA_GATE_MAP); s unused
    // compact envelope flags, one word per (slot, head) record, or nullptr
    // (then each record keeps its own); written by the fast pass, read by
    // the exact pass
    uint32_t* flags;
    // kModeGrad: the backward's first gradient phase
    const float* h_ckpt;      // chunk-start states (true frame)
    const float* dU;          // dL/dU per (slot, head), C/D tiles (reverse pass)
    const void* dout;         // dO
    float* dv;                // dL/dV out
    float* dbeta;             // dL/dbeta out
    unsigned char* gout;      // dA, dM, U per (slot, head), gout_bytes apart
    size_t gout_bytes;
    float scale;
};

// The backward's first chunk-parallel gradient phase, after the chunk-local
// prologue of chunk_body (kModeGrad: b, P, kf, qf; A; the diagonal inverses
// and off-diagonal blocks of X = I + Diag(beta) A in LDS; Ke = kf e^b in the
// row-operand area).  With S0 the chunk-start state (true frame), dU from the
// reverse pass and R = V - Ke S0 (the WY/UT chunk form; Complex KDA paper
// page, section 2 "Linear RNNs"):
//   Xi = X^{-1},  U = Xi Diag(beta) R,  Y = Xi^T dU,  dV = Diag(beta) Y,
//   dX = -Y U^T,  dA = Diag(beta) strict_lower(dX),  dM = scale lower(dO U^T),
//   dbeta_r = sum_v Y_rv R_rv + sum_{i<r} dX_ri A_ri.
// dV and dbeta are final; dA, dM and U go to the second phase (GradOut).
// Waves: the four Xi column tiles on waves 0..3; then each wave one (or, with
// four waves and DV = 128, two) 16-column value tile for the products with S0,
// Xi and dU; then waves 0..3 the dX rows of token tile R = w and waves 4..7
// (or the same waves after them) dM.
template <typename Tin, int DK, int DV, typename Subst, int VPW_>
__device__ __forceinline__ void grad_phase1(const ChunkParams& p, const int slot, const int h, const int tok0,
                                            const int L, unsigned char* smem, Subst& substitute,
                                            const f32x4 (&accA)[4], const uint32_t (&vpre)[VPW_][4][4])
{
    using SH = ChunkShape<DK>;
    using GS = GradShape<DK, DV>;
    constexpr bool F32 = sizeof(Tin) == 4;
    using PR = Prec<F32>;
    using GO = GradOut<DK, DV, F32>;
    constexpr int NW = SH::NW, VPW = GS::VPW, RT = DK / 16, KS = RT / 2;
    static_assert(VPW == VPW_, "value tiles per wave");
    const int H = p.H;
    const int tid = static_cast<int>(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, n = l & 15, gq = l >> 4;
    const float* const beta_s = reinterpret_cast<const float*>(smem + SH::L_BETA);
    const LdsMat rkm{smem + SH::L_RK, SH::PC, 64 * SH::PC};   // Ke
    const LdsMat xim{smem + GS::L_XI, GS::PX, 64 * GS::PX};
    const LdsMat xitm{smem + GS::L_XIT, GS::PX, 64 * GS::PX};
    const LdsMat utm{smem + GS::L_UT, GS::PU, 64 * GS::PU};
    const LdsMat ytm{smem + GS::L_YT, GS::PU, 64 * GS::PU};
    float* const dbr = reinterpret_cast<float*>(smem + GS::L_DBR);
    const size_t ch = static_cast<size_t>(slot) * H + h;

    // ---- Xi = X^{-1}, column tile w (rows 16J + 4g + i of column 16w + n)
    f32x4 Xt[4];
    if (w < 4) {
        float rhs[4][4];
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) rhs[J][i] = (16 * J + 4 * gq + i == 16 * w + n) ? 1.f : 0.f;
        substitute(rhs, Xt, false);
    }
    lds_sync();   // the inverses and off-diagonal blocks are consumed
    if (w < 4) {
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            PR::store4(xitm, 16 * w + n, 16 * J + 4 * gq, Xt[J]);   // Xi^T row 16w + n
#pragma unroll
            for (int j = 0; j < 4; ++j) PR::store1(xim, 16 * J + 4 * gq + j, 16 * w + n, Xt[J][j]);
        }
    }
    lds_sync();

    // ---- per value tile: S0 products, U, Y, dV and beta's R-term
    size_t ck;   // checkpoint: equal-length [B][H][NT][DK][DV], varlen [slot][H][DK][DV]
    if (p.cu) {
        ck = ch;
    } else {
        const int nch = (p.T + 63) / 64;
        const int b = slot / nch, j = slot - b * nch;
        ck = (static_cast<size_t>(b) * H + h) * nch + j;
    }
    const float* const S0 = p.h_ckpt + ck * DK * DV;
    const f32x4* const dUp = reinterpret_cast<const f32x4*>(p.dU + ch * 64 * DV);
    f32x4 Uk[VPW][4], Yk[VPW][4];
#pragma unroll
    for (int vi = 0; vi < VPW; ++vi) {
        const int vt = w + NW * vi;
        if (vt < DV / 16) {
            const int col = 16 * vt + n;
            // the S0 column slice as B operands: 32 channels per step (rows
            // 32ks + 4g + i and 32ks + 16 + 4g + i, the A side's K order)
            typename PR::F8 Sb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                f32x4 a, b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = S0[static_cast<size_t>(32 * ks + 4 * gq + i) * DV + col];
                    b[i] = S0[static_cast<size_t>(32 * ks + 16 + 4 * gq + i) * DV + col];
                }
                Sb[ks] = PR::regs8(a, b);
            }
            f32x4 X[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                X[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    X[J] = PR::mma8(PR::load4x2(rkm, 16 * J + n, 32 * ks + 4 * gq, 32 * ks + 16 + 4 * gq), Sb[ks], X[J]);
            }
            f32x4 Rr[4], Rp[4];
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 16 * J + 4 * gq + i;
                    const float vv = __uint_as_float(F32 ? vpre[vi][J][i] : (vpre[vi][J][i] << 16));
                    Rr[J][i] = (tt < L ? vv : 0.f) - X[J][i];
                    Rp[J][i] = beta_s[tt] * Rr[J][i];
                }
            const typename PR::F8 Rb[2] = {PR::regs8(Rp[0], Rp[1]), PR::regs8(Rp[2], Rp[3])};
            f32x4 du[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) du[J] = dUp[(J * (DV / 16) + vt) * 64 + l];
            const typename PR::F8 Db[2] = {PR::regs8(du[0], du[1]), PR::regs8(du[2], du[3])};
            f32x4 U[4], Y[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                U[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                Y[J] = U[J];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    U[J] = PR::mma8(PR::load4x2(xim, 16 * J + n, 32 * kt + 4 * gq, 32 * kt + 16 + 4 * gq), Rb[kt], U[J]);
                    Y[J] = PR::mma8(PR::load4x2(xitm, 16 * J + n, 32 * kt + 4 * gq, 32 * kt + 16 + 4 * gq), Db[kt], Y[J]);
                }
            }
            const __amdgpu_buffer_rsrc_t vrc =
                buffer_rsrc(p.dv + (static_cast<size_t>(tok0) * H + h) * DV, static_cast<uint32_t>(L * H * DV * 4));
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 16 * J + 4 * gq + i;
                    buffer_store_f32(vrc, static_cast<uint32_t>((tt * H * DV + col) * 4), beta_s[tt] * Y[J][i]);
                    const float x = row_scan_add(Y[J][i] * Rr[J][i]);   // lane 15: the tile's 16 columns
                    if (n == 15) dbr[vt * 64 + tt] = x;
                }
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                Uk[vi][J] = U[J];
                Yk[vi][J] = Y[J];
            }
            if constexpr (!GS::OVL) {
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        PR::store1(utm, 16 * J + 4 * gq + i, col, U[J][i]);
                        PR::store1(ytm, 16 * J + 4 * gq + i, col, Y[J][i]);
                    }
            }
        }
    }
    if constexpr (GS::OVL) {
        lds_sync();   // Ke and Xi are consumed: U and Y go over them
#pragma unroll
        for (int vi = 0; vi < VPW; ++vi) {
            const int vt = w + NW * vi;
            if (vt < DV / 16) {
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        PR::store1(utm, 16 * J + 4 * gq + i, 16 * vt + n, Uk[vi][J][i]);
                        PR::store1(ytm, 16 * J + 4 * gq + i, 16 * vt + n, Yk[vi][J][i]);
                    }
            }
        }
    }
    lds_sync();   // U, Y and the beta partial sums in LDS

    // ---- dX and dM: tile (I, R) of C[i][r] = sum_v U[i][v] B[r][v], B = Y
    // (dX = -C^T) or dO (dM = scale C^T); lane (n, g) ends with row
    // r = 16R + n, columns 16I + 4g .. +3, the layout of A's tiles
    unsigned char* const go = p.gout + ch * p.gout_bytes;
    const Tin* const dO = static_cast<const Tin*>(p.dout);
    auto dofrag = [&](int R, int k) -> typename PR::F8 {   // B fragment of dO rows 16R .. 16R+15
        const int tt = 16 * R + n;
        const size_t base = (static_cast<size_t>(tok0 + min(tt, L - 1)) * H + h) * DV + 32 * k + 4 * gq;
        typename PR::F8 f;
        if constexpr (F32) {
            f.a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(dO) + base);
            f.b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(dO) + base + 16);
            if (tt >= L) f.a = f.b = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
            u32x2 a = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(dO) + base);
            u32x2 b = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(dO) + base + 16);
            if (tt >= L) a = b = u32x2{0u, 0u};
            f.hi = __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
            f.lo = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});   // bf16 inputs: dO is exact in one plane
        }
        return f;
    };
#pragma unroll
    for (int pass = 0; pass < (NW == 8 ? 1 : 2); ++pass) {
        const bool isM = NW == 8 ? (w >= 4) : (pass == 1);
        const int R = w & 3;
        f32x4 acc[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) acc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < DV / 32; ++k) {
            const typename PR::F8 bf = isM ? dofrag(R, k)
                                           : PR::load4x2(ytm, 16 * R + n, 32 * k + 4 * gq, 32 * k + 16 + 4 * gq);
#pragma unroll
            for (int I = 0; I < 4; ++I)
                if (I <= R)
                    acc[I] = PR::mma8(PR::load4x2(utm, 16 * I + n, 32 * k + 4 * gq, 32 * k + 16 + 4 * gq), bf, acc[I]);
        }
        const int r = 16 * R + n;
        const float br = beta_s[r];
        float aterm = 0.f;
        unsigned char* const dst = go + (isM ? GO::OFF_DM : GO::OFF_DA);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 16 * I + 4 * gq + j;
                    if (isM) {
                        o[j] = i <= r ? p.scale * acc[I][j] : 0.f;
                    } else {
                        const float dx = -acc[I][j];
                        aterm += i < r ? dx * accA[I][j] : 0.f;
                        o[j] = i < r ? br * dx : 0.f;
                    }
                }
                PR::gstore4(dst, GO::A_PLANE, GO::A_ROW, r, 16 * I + 4 * gq, o);
            }
        }
        if ((R & 1) == 0)   // blocks (0,1), (2,3): read by the second phase's 32-token steps
            PR::gstore4(dst, GO::A_PLANE, GO::A_ROW, r, 16 * (R + 1) + 4 * gq, f32x4{0.f, 0.f, 0.f, 0.f});
        if (!isM) {
            aterm += __shfl_xor(aterm, 16, 64);
            aterm += __shfl_xor(aterm, 32, 64);
            if (gq == 0 && r < L) {
                float db = aterm;
#pragma unroll
                for (int vt = 0; vt < DV / 16; ++vt) db += dbr[vt * 64 + r];
                if (p.gate_map) {   // dL/dy of the beta pre-activation
                    const float bb = beta_s[r];
                    db *= bb * (1.f - 0.5f * bb);
                }
                p.dbeta[static_cast<size_t>(tok0 + r) * H + h] = db;
            }
        }
    }
    // ---- U for the second phase (token-major planes, no padding)
    constexpr int UPR = DV * GO::ES / 16;
    for (int u = tid; u < GO::NP * 64 * UPR; u += NW * 64) {
        const int pl = u / (64 * UPR), rr = (u / UPR) % 64, cu = u % UPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + GS::L_UT + (pl * 64 + rr) * GS::PU * GO::ES + cu * 16);
        *reinterpret_cast<u32x4*>(go + GO::OFF_U + pl * GO::U_PLANE + static_cast<size_t>(rr) * GO::U_ROW + cu * 16) = v;
    }
}

// One (chunk slot, head).  HG: one gate per (token, head) (g, s [.., H]),
// broadcast over the channels; NQK: q and k normalised per (token, head) over
// the key channels.  EX = false: the anchored fast path, which writes the
// record's flag and leaves the record to the exact path when the chunk's
// gates leave the anchors' range; EX = true: the exact path (A and M entry by
// entry), run only on flagged chunks.
//
// MODE: kModeFwd writes the forward's record; kModeRev the backward's
// reverse-pass record (RevRecord: KbT^T, Qh^T, W^T, M^T, d), skipping u and
// its substitution; kModeGrad writes no record and hands the chunk's A, the
// diagonal inverses and Ke = kf e^b over to the backward's first
// chunk-parallel gradient phase (grad.hip).
template <typename Tin, int DK, int DV, bool HG, bool NQK, bool EX, int MODE, bool GM>
__device__ __forceinline__ void chunk_body(const ChunkParams& p, const int slot, const int h, unsigned char* smem)
{
    using SH = ChunkShape<DK>;
    constexpr bool F32 = sizeof(Tin) == 4;
    constexpr bool REV = MODE == kModeRev, GRAD = MODE == kModeGrad;
    using PR = Prec<F32>;
    using RC = std::conditional_t<REV || GRAD, RevRecord<DK, DV, F32>, Record<DK, DV, F32>>;
    constexpr int NW = SH::NW, KSW = SH::KSW, NE = SH::NE, CG = SH::CG, PC = SH::PC;

    const int H = p.H;
    int tok0, L;
    if (p.cu) {
        // the document whose slot range holds this slot (slot bases increase with d)
        int lo = 0, hi = p.ndocs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (varlen_slot(p.cu[mid], mid, 0) <= slot) lo = mid; else hi = mid - 1;
        }
        const int j = slot - varlen_slot(p.cu[lo], lo, 0);
        const int len = p.cu[lo + 1] - p.cu[lo];
        if (64 * j >= len) {             // unused slot (whole workgroup)
            if (MODE == kModeRev && threadIdx.x == 0) p.flags[static_cast<size_t>(slot) * H + h] = 0u;
            return;
        }
        tok0 = p.cu[lo] + 64 * j;
        L = min(64, len - 64 * j);
    } else {
        const int nch = (p.T + 63) / 64;
        const int b = slot / nch, j = slot - b * nch;
        tok0 = b * p.T + 64 * j;
        L = min(64, p.T - 64 * j);
    }
    unsigned char* const rec = p.ws + (static_cast<size_t>(slot) * H + h) * RC::BYTES;
    const Tin* __restrict__ q = static_cast<const Tin*>(p.q);
    const Tin* __restrict__ k = static_cast<const Tin*>(p.k);
    const Tin* __restrict__ v = static_cast<const Tin*>(p.v);

    // (the exact kernel runs this body in a loop: an opaque thread index keeps
    // the lane-derived addresses from being hoisted out of it into registers)
    const int tid = EX ? opaque_tid() : static_cast<int>(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = w & 3;            // token tile of the prep and of the A/M rows
    const int cgi = w >> 2;         // channel group
    const int l = tid & 63, n = l & 15, gq = l >> 4;
    const int t = 16 * R + n;
    const bool valid = t < L;

    float* const totb = reinterpret_cast<float*>(smem + SH::L_TOTB);
    uint32_t* const totp = reinterpret_cast<uint32_t*>(smem + SH::L_TOTP);
    float* const beta_s = reinterpret_cast<float*>(smem + SH::L_BETA);
    const LdsMat colk{smem + SH::L_COLK, PC, 64 * PC};
    const LdsMat colkf{smem + SH::L_COLKF, PC, 32 * PC};

    // ---- inputs: the lane's token, channels c0 .. c0+7 of each step -------
    Raw8<Tin> q8[KSW], k8[KSW];
    float bs[NE];
    uint32_t par[2 * KSW];   // sign bytes; bit 7 of byte e set <=> s = -1
    {
        // padding tokens (t >= L) read the chunk's last token and are then
        // replaced by g = 0, s = +1, q = k = 0, beta = 0 (unconditional loads)
        const size_t trow = static_cast<size_t>(tok0 + min(t, L - 1)) * H + h;
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            const int c0 = CG * cgi + 32 * ks + 8 * gq;
            const size_t base = trow * DK + c0;
            q8[ks].load(q + base);
            k8[ks].load(k + base);
            if constexpr (HG) {
                const float gx = p.g[trow];
                const float gt = GM ? gate_map_g(gx) : gx;
                const uint32_t sb = GM ? (gx < 0.f ? 0xFFu : 0x01u) : static_cast<uint8_t>(p.s[trow]);
                const uint32_t sw = sb * 0x01010101u;
#pragma unroll
                for (int e = 0; e < 8; ++e) bs[8 * ks + e] = gt;
                par[2 * ks] = sw;
                par[2 * ks + 1] = sw;
            } else {
                float4 a = reinterpret_cast<const float4*>(p.g + base)[0];
                float4 b = reinterpret_cast<const float4*>(p.g + base)[1];
                uint2 sv;
                if constexpr (GM) {   // signs from the pre-activations, then the map
                    auto sb = [](float x, int sh) { return (x < 0.f ? 0xFFu : 0x01u) << sh; };
                    sv.x = sb(a.x, 0) | sb(a.y, 8) | sb(a.z, 16) | sb(a.w, 24);
                    sv.y = sb(b.x, 0) | sb(b.y, 8) | sb(b.z, 16) | sb(b.w, 24);
                    a = make_float4(gate_map_g(a.x), gate_map_g(a.y), gate_map_g(a.z), gate_map_g(a.w));
                    b = make_float4(gate_map_g(b.x), gate_map_g(b.y), gate_map_g(b.z), gate_map_g(b.w));
                } else {
                    sv = *reinterpret_cast<const uint2*>(p.s + base);
                }
                bs[8 * ks + 0] = a.x; bs[8 * ks + 1] = a.y; bs[8 * ks + 2] = a.z; bs[8 * ks + 3] = a.w;
                bs[8 * ks + 4] = b.x; bs[8 * ks + 5] = b.y; bs[8 * ks + 6] = b.z; bs[8 * ks + 7] = b.w;
                par[2 * ks] = sv.x;
                par[2 * ks + 1] = sv.y;
            }
            if (!valid) {
                q8[ks].zero();
                k8[ks].zero();
#pragma unroll
                for (int e = 0; e < 8; ++e) bs[8 * ks + e] = 0.f;
                par[2 * ks] = 0x01010101u;
                par[2 * ks + 1] = 0x01010101u;
            }
        }
        const float bt = GM ? gate_map_beta(p.beta[trow]) : p.beta[trow];
        if (cgi == 0 && gq == 0) beta_s[t] = valid ? bt : 0.f;
    }
    float2* const nrm = reinterpret_cast<float2*>(smem + SH::L_NRM);
    if constexpr (NQK) {   // sums of squares of the token's k and q: lanes, then channel groups
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kv = k8[ks].get(e), qv = q8[ks].get(e);
                sk += kv * kv;
                sq += qv * qv;
            }
        sk += __shfl_xor(sk, 16, 64);
        sk += __shfl_xor(sk, 32, 64);
        sq += __shfl_xor(sq, 16, 64);
        sq += __shfl_xor(sq, 32, 64);
        if (gq == 0) nrm[cgi * 64 + t] = make_float2(sk, sq);
    }
    bool outside = false;   // g > 0 anywhere in the lane's elements
    if constexpr (!EX) {
#pragma unroll
        for (int i = 0; i < (HG ? 1 : NE); ++i) outside |= bs[i] > 0.f;
    }
    // ---- 1. in-tile scans (log2 units), tile totals to LDS -----------------
    if constexpr (HG) {   // every channel carries the head's gate: one scan per lane
        const float b1 = row_scan_add(bs[0] * kLog2e);
        const uint32_t p1 = row_scan_xor(par[0]);
#pragma unroll
        for (int i = 0; i < NE; ++i) bs[i] = b1;
#pragma unroll
        for (int i = 0; i < 2 * KSW; ++i) par[i] = p1;
    } else {
#pragma unroll
        for (int i = 0; i < NE; ++i) bs[i] = row_scan_add(bs[i] * kLog2e);
#pragma unroll
        for (int i = 0; i < 2 * KSW; ++i) par[i] = row_scan_xor(par[i]);
    }
    if constexpr (!EX) {   // envelope of the anchored factoring, one flag per wave
#pragma unroll
        for (int i = 0; i < NE; ++i) outside |= !(fabsf(bs[i]) <= kEnvelope);
        const unsigned long long any = __ballot(outside);
        if (l == 0) reinterpret_cast<uint32_t*>(smem + SH::L_FLAG)[w] = any != 0ull ? 1u : 0u;
    }
    if (n == 15) {
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            const int c0 = CG * cgi + 32 * ks + 8 * gq;
            float4* dst = reinterpret_cast<float4*>(totb + R * DK + c0);
            dst[0] = make_float4(bs[8 * ks + 0], bs[8 * ks + 1], bs[8 * ks + 2], bs[8 * ks + 3]);
            dst[1] = make_float4(bs[8 * ks + 4], bs[8 * ks + 5], bs[8 * ks + 6], bs[8 * ks + 7]);
            *reinterpret_cast<uint2*>(totp + R * (DK / 4) + c0 / 4) = make_uint2(par[2 * ks], par[2 * ks + 1]);
        }
    }
    lds_sync();
    if constexpr (!EX) {   // the flag decides for the whole workgroup
        const uint32_t* fw = reinterpret_cast<const uint32_t*>(smem + SH::L_FLAG);
        uint32_t f = 0;
#pragma unroll
        for (int x = 0; x < NW; ++x) f |= fw[x];
        if (tid == 0 && !GRAD) {   // (the gradient phase reads the reverse pass's flags)
            if (p.flags) p.flags[static_cast<size_t>(slot) * H + h] = f;
            *reinterpret_cast<uint32_t*>(rec + RC::OFF_FLAG) = f;
        }
        if (f) return;
    }

    // ---- 2. exponentials and operands -------------------------------------
    float ik = 1.f, iq = 1.f;   // 1 / ||k||, 1 / ||q|| (a zero vector stays zero)
    if constexpr (NQK) {
        float2 a = nrm[t];
        if (SH::NCG > 1) {
            const float2 b2 = nrm[64 + t];
            a.x += b2.x;
            a.y += b2.y;
        }
        ik = inv_norm(a.x);
        iq = inv_norm(a.y);
    }
    typename PR::F8 rkB[KSW], rqB[KSW];   // row operands (B side of the A/M tiles)
    float qfr[KSW][8];                    // exact path: the token's qf
    float* const xk = reinterpret_cast<float*>(smem + SH::L_XK);
    float* const xb = reinterpret_cast<float*>(smem + SH::L_XB);
    constexpr int XP = SH::XP;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CG * cgi + 32 * ks + 8 * gq;
        // anchors per channel (log2 units): b at token 15 (m0) and 47 (m1),
        // and the sum over the earlier tiles of this wave's token tile
        float b[8], mh[8], m1[8], bL[8];   // bL: b at the chunk's last token (REV)
        if constexpr (HG) {   // equal across channels: one value per lane (the rest folds away)
            const float t0 = totb[c0], t1 = totb[DK + c0], t2 = totb[2 * DK + c0];
            const float pre = (R > 0 ? t0 : 0.f) + (R > 1 ? t1 : 0.f) + (R > 2 ? t2 : 0.f);
            const float m1v = t0 + t1 + t2, mhv = R < 2 ? t0 : m1v, bv = bs[8 * ks] + pre;
            const float bLv = REV ? m1v + totb[3 * DK + c0] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                b[e] = bv;
                m1[e] = m1v;
                mh[e] = mhv;
                bL[e] = bLv;
            }
        } else {
            float4 Tt[4][2];
#pragma unroll
            for (int x = 0; x < (REV ? 4 : 3); ++x) {
                Tt[x][0] = reinterpret_cast<const float4*>(totb + x * DK + c0)[0];
                Tt[x][1] = reinterpret_cast<const float4*>(totb + x * DK + c0)[1];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                auto pick = [&](const float4 (&v2)[2]) {
                    const float4 vv = v2[e >> 2];
                    return (e & 3) == 0 ? vv.x : (e & 3) == 1 ? vv.y : (e & 3) == 2 ? vv.z : vv.w;
                };
                const float t0 = pick(Tt[0]), t1 = pick(Tt[1]), t2 = pick(Tt[2]);
                b[e] = bs[8 * ks + e] + ((R > 0 ? t0 : 0.f) + (R > 1 ? t1 : 0.f) + (R > 2 ? t2 : 0.f));
                m1[e] = t0 + t1 + t2;
                mh[e] = R < 2 ? t0 : m1[e];
                bL[e] = REV ? m1[e] + pick(Tt[3]) : 0.f;
            }
        }
        // sign-folded q and k (running product over the earlier tiles and this one)
        float kf[8], qf[8];
        {
            uint32_t pw0 = par[2 * ks], pw1 = par[2 * ks + 1];
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                if (x < R) {
                    const uint2 pv = *reinterpret_cast<const uint2*>(totp + x * (DK / 4) + c0 / 4);
                    pw0 ^= pv.x;
                    pw1 ^= pv.y;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sgn = HG ? ((pw0 << 24) & 0x80000000u)   // all bytes equal
                                        : ((((e >> 2) ? pw1 : pw0) << (24 - 8 * (e & 3))) & 0x80000000u);
                kf[e] = __uint_as_float(__float_as_uint(NQK ? k8[ks].get(e) * ik : k8[ks].get(e)) ^ sgn);
                qf[e] = __uint_as_float(__float_as_uint(NQK ? q8[ks].get(e) * iq : q8[ks].get(e)) ^ sgn);
            }
        }
        CKDA_FENCE();
        float x[8];
        if constexpr (!EX) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = fminf(fmaxf(b[e] - mh[e], -126.f), 126.f);
            {   // column operand kf e^{m - b}
                float ck[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ck[e] = kf[e] * __builtin_amdgcn_exp2f(-x[e]);
                PR::store8(colk, t, c0, ck);
            }
            if (R < 2) {   // its cross-half version kf e^{m1 - b} for the half-1 rows
                float ckf[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ckf[e] = kf[e] * __builtin_amdgcn_exp2f(fminf(m1[e] - b[e], 126.f));
                PR::store8(colkf, t, c0, ckf);
            }
        } else {   // kf and b of the token, unscaled, for the entry-by-entry products
            float4* pk = reinterpret_cast<float4*>(xk + t * XP + c0);
            float4* pb = reinterpret_cast<float4*>(xb + t * XP + c0);
            pk[0] = make_float4(kf[0], kf[1], kf[2], kf[3]);
            pk[1] = make_float4(kf[4], kf[5], kf[6], kf[7]);
            pb[0] = make_float4(b[0], b[1], b[2], b[3]);
            pb[1] = make_float4(b[4], b[5], b[6], b[7]);
#pragma unroll
            for (int e = 0; e < 8; ++e) qfr[ks][e] = qf[e];
        }
        CKDA_FENCE();
        float e0[8];   // e^b
        {   // Qh = qf e^b to the record; d = P_L e^{b_L} from token 63
            float qh[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                e0[e] = __builtin_amdgcn_exp2f(fminf(b[e], 126.f));
                qh[e] = qf[e] * e0[e];
            }
            if constexpr (GRAD) {
                // no record
            } else if constexpr (REV) {
                PR::template gstore_col<8>(rec + RC::OFF_QT, RC::QT_PLANE, RC::QT_ROW, c0, t, qh);
                // KB = P_L kf e^{b_L - b}: the exponent is <= 0 (g <= 0), so no anchor
                uint2 pl = *reinterpret_cast<const uint2*>(totp + c0 / 4);
#pragma unroll
                for (int x = 1; x < 4; ++x) {
                    const uint2 pv = *reinterpret_cast<const uint2*>(totp + x * (DK / 4) + c0 / 4);
                    pl.x ^= pv.x;
                    pl.y ^= pv.y;
                }
                float kb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sg = HG ? ((pl.x << 24) & 0x80000000u)
                                           : ((((e >> 2) ? pl.y : pl.x) << (24 - 8 * (e & 3))) & 0x80000000u);
                    const float v = kf[e] * __builtin_amdgcn_exp2f(fminf(bL[e] - b[e], 126.f));
                    kb[e] = __uint_as_float(__float_as_uint(v) ^ sg);
                }
                PR::gstore8(rec + RC::OFF_KB, RC::KB_PLANE, RC::KB_ROW, t, c0, kb);
            } else {
                PR::gstore8(rec + RC::OFF_Q, RC::Q_PLANE, RC::Q_ROW, t, c0, qh);
            }
            if (!GRAD && t == 63) {   // the sign of P_L: kf and k differ exactly in it (also for k = +-0)
                float dd[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sg = (__float_as_uint(kf[e]) ^ __float_as_uint(k8[ks].get(e))) & 0x80000000u;
                    dd[e] = __uint_as_float(__float_as_uint(e0[e]) ^ sg);
                }
                float4* dp = reinterpret_cast<float4*>(rec + RC::OFF_D + 4 * c0);
                dp[0] = make_float4(dd[0], dd[1], dd[2], dd[3]);
                dp[1] = make_float4(dd[4], dd[5], dd[6], dd[7]);
            }
        }
        CKDA_FENCE();
        if constexpr (!EX) {   // row operands kf e^{b - m}, qf e^{b - m} (registers)
            float rk[8], rq[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float e1 = __builtin_amdgcn_exp2f(x[e]);
                rk[e] = kf[e] * e1;
                rq[e] = qf[e] * e1;
            }
            rkB[ks] = PR::regs8(f32x4{rk[0], rk[1], rk[2], rk[3]}, f32x4{rk[4], rk[5], rk[6], rk[7]});
            rqB[ks] = PR::regs8(f32x4{rq[0], rq[1], rq[2], rq[3]}, f32x4{rq[4], rq[5], rq[6], rq[7]});
        }
    }
    lds_sync();

    // ---- KbT = (P_L kf e^{b_L - b})^T from the column operand --------------
    // task = (channel c, 8-token group tg); the column operand of a half is
    // kf e^{m - b}, so KbT = that times P_L e^{b_L - m}
    if constexpr (MODE == kModeFwd) {
        for (int task = tid; task < DK * 8; task += NW * 64) {
            // four lanes on the 8-token groups of one channel row (64
            // contiguous bytes per plane), sixteen channels per wave
            const int c = (task / 4) % DK, tg = 4 * (task / (4 * DK)) + task % 4;
            const float B0 = totb[c], B1 = totb[DK + c], B2 = totb[2 * DK + c], B3 = totb[3 * DK + c];
            const float m = (tg >= 4) ? (B0 + B1 + B2) : B0;
            const uint32_t pw = totp[c / 4] ^ totp[DK / 4 + c / 4] ^ totp[DK / 2 + c / 4] ^ totp[3 * (DK / 4) + c / 4];
            const uint32_t sgn = (pw << (24 - 8 * (c & 3))) & 0x80000000u;
            float x[8];
            if constexpr (!EX) {
                const float f = __uint_as_float(
                    __float_as_uint(__builtin_amdgcn_exp2f(fminf(B0 + B1 + B2 + B3 - m, 126.f))) ^ sgn);
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = f * PR::get1(colk, 8 * tg + j, c);
            } else {   // kf e^{b_L - b} with the exponent taken whole
                const float bL = B0 + B1 + B2 + B3;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tt = 8 * tg + j;
                    const float v = xk[tt * XP + c] * __builtin_amdgcn_exp2f(fminf(bL - xb[tt * XP + c], 126.f));
                    x[j] = __uint_as_float(__float_as_uint(v) ^ sgn);
                }
            }
            PR::gstore8(rec + RC::OFF_K, RC::K_PLANE, RC::K_ROW, c, 8 * tg, x);
        }
    }

    // ---- 3. A^T / M^T tiles (I, R), I <= R, over this wave's channels -------
    // lane (n, g) ends with row 16R + n, columns 16I + 4g .. +3 of A and M
    f32x4 accA[4], accM[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        accA[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        accM[I] = accA[I];
    }
    if constexpr (!EX) {
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            const int c0 = CG * cgi + 32 * ks + 8 * gq;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I <= R) {
                    const bool cross = (R >= 2) && (I < 2);
                    const typename PR::F8 a = PR::load8(cross ? colkf : colk, 16 * I + n, c0);
                    accA[I] = PR::mma8(a, rkB[ks], accA[I]);
                    if (!GRAD) accM[I] = PR::mma8(a, rqB[ks], accM[I]);   // (the gradient phase needs A only)
                }
            }
        }
    } else {
        // exact path: the row token t against tokens 16I .. 16I + 15, each
        // entry sum_c kf_tc kf_ic e^{b_tc - b_ic} (and qf_tc for M) with the
        // exponent taken whole, over the lane's channels; then summed over
        // the four lanes that hold the row's other channel octets.  Entries
        // above the diagonal come out as garbage and are masked below.  Eight
        // columns at a time: lane (n, g) keeps columns 16I + 4g .. +3 (the
        // C/D layout), so half hj serves the lanes with g = 2hj, 2hj + 1.
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
#pragma unroll
                for (int hj = 0; hj < 2; ++hj) {
                    float pa[8], pm[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        pa[j] = 0.f;
                        pm[j] = 0.f;
                    }
#pragma unroll
                    for (int ks = 0; ks < KSW; ++ks) {
                        const int c0 = CG * cgi + 32 * ks + 8 * gq;
                        float kr[8], br[8];
                        {
                            const float4* pk = reinterpret_cast<const float4*>(xk + t * XP + c0);
                            const float4* pb = reinterpret_cast<const float4*>(xb + t * XP + c0);
                            const float4 k0 = pk[0], k1 = pk[1], b0 = pb[0], b1 = pb[1];
                            kr[0] = k0.x; kr[1] = k0.y; kr[2] = k0.z; kr[3] = k0.w;
                            kr[4] = k1.x; kr[5] = k1.y; kr[6] = k1.z; kr[7] = k1.w;
                            br[0] = b0.x; br[1] = b0.y; br[2] = b0.z; br[3] = b0.w;
                            br[4] = b1.x; br[5] = b1.y; br[6] = b1.z; br[7] = b1.w;
                        }
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int i = 16 * I + 8 * hj + j;
                            const float4* pk = reinterpret_cast<const float4*>(xk + i * XP + c0);
                            const float4* pb = reinterpret_cast<const float4*>(xb + i * XP + c0);
                            const float4 k0 = pk[0], k1 = pk[1], b0 = pb[0], b1 = pb[1];
                            const float ki[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                            const float bi[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const float u = ki[e] * __builtin_amdgcn_exp2f(fminf(br[e] - bi[e], 126.f));
                                pa[j] = fmaf(kr[e], u, pa[j]);
                                pm[j] = fmaf(qfr[ks][e], u, pm[j]);
                            }
                            CKDA_FENCE();   // one column's loads in flight at a time
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        pa[j] += __shfl_xor(pa[j], 16, 64);
                        pa[j] += __shfl_xor(pa[j], 32, 64);
                        pm[j] += __shfl_xor(pm[j], 16, 64);
                        pm[j] += __shfl_xor(pm[j], 32, 64);
                    }
                    if ((gq >> 1) == hj) {
                        const int o = 4 * (gq & 1);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            accA[I][jj] = o ? pa[4 + jj] : pa[jj];
                            accM[I][jj] = o ? pm[4 + jj] : pm[jj];
                        }
                    }
                }
            }
        }
        // kf e^b itself: the right-hand side of W, with no anchor
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            const int c0 = CG * cgi + 32 * ks + 8 * gq;
            float rk[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                rk[e] = xk[t * XP + c0 + e] * __builtin_amdgcn_exp2f(fminf(xb[t * XP + c0 + e], 126.f));
            rkB[ks] = PR::regs8(f32x4{rk[0], rk[1], rk[2], rk[3]}, f32x4{rk[4], rk[5], rk[6], rk[7]});
        }
        lds_sync();   // the partial-tile area overlaps kf and b
    }
    f32x4* const part = reinterpret_cast<f32x4*>(smem + SH::L_PART);
    if (SH::NCG > 1 && cgi == 1) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                part[tri_index(R, I) * 64 + l] = accA[I];
                if (!GRAD) part[(10 + tri_index(R, I)) * 64 + l] = accM[I];
            }
        }
    }
    lds_sync();

    // V for this wave's value tiles of the substitution.  Vector memory
    // loads and stores retire in order, so these loads go out before the M
    // stores below (and long after the Qh / KbT stores), and their latency
    // hides behind the diagonal inverses; each value keeps its own register
    // until use (combining two loads would wait for both here).  Lane (n, g)
    // holds rows 16J + 4g + i of column 16vt + n (the C/D layout).
    constexpr int VPW = (DV / 16 + NW - 1) / NW;   // value tiles per wave
    uint32_t vpre[VPW][4][4];
    // (addresses are clamped into the chunk so every load is unconditional:
    // a guarded load becomes a branch that waits for its result in place)
#pragma unroll
    for (int vi = 0; vi < (REV ? 0 : VPW); ++vi) {
        const int vtc = min(w + NW * vi, DV / 16 - 1);
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * J + 4 * gq + i;
                const size_t idx = (static_cast<size_t>(tok0 + min(tt, L - 1)) * H + h) * DV + 16 * vtc + n;
                vpre[vi][J][i] = F32 ? __float_as_uint(reinterpret_cast<const float*>(v)[idx])
                                     : static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(v)[idx]);
            }
    }
    // ---- 4. row operand kf e^{b - m} to LDS (over colk) for the right-hand
    // sides; M to the record; -beta A blocks and diagonals to LDS (over colkf)
    const LdsMat rkm{smem + SH::L_RK, PC, 64 * PC};
    const LdsMat loffm{smem + SH::L_LOFF, 4, 6 * 64 * 4};
    const LdsMat ym{smem + SH::L_Y, SH::PY, 64 * SH::PY};
    float* const ldiag = reinterpret_cast<float*>(smem + SH::L_LDIAG);
    if constexpr (GRAD && !EX) {   // Ke = kf e^b = (kf e^{b - m}) e^m for the gradient phase
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) {
            const int c0 = CG * cgi + 32 * ks + 8 * gq;
            float ke[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float m0 = totb[c0 + e];
                const float m = R < 2 ? m0 : m0 + totb[DK + c0 + e] + totb[2 * DK + c0 + e];
                ke[e] = PR::get8(rkB[ks], e) * __builtin_amdgcn_exp2f(fminf(m, 126.f));
            }
            PR::store8(rkm, t, c0, ke);
        }
    } else {   // (the exact path's rkB is kf e^b already)
#pragma unroll
        for (int ks = 0; ks < KSW; ++ks) PR::store8f(rkm, t, CG * cgi + 32 * ks + 8 * gq, rkB[ks]);
    }
    if (cgi == 0) {
        const int r = 16 * R + n;
        const float br = beta_s[r];
        if (!GRAD && (R & 1) == 0) {   // blocks (0,1), (2,3): read by the 32-token steps of the state pass
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            if constexpr (REV) {   // M^T: rows 16(R+1) + 4g .. +3, column r
                const float z4[4] = {0.f, 0.f, 0.f, 0.f};
                PR::template gstore_col<4>(rec + RC::OFF_MT, RC::MT_PLANE, RC::MT_ROW, 16 * (R + 1) + 4 * gq, r, z4);
            } else if constexpr (MODE == kModeFwd) {
                PR::gstore4(rec + RC::OFF_M, RC::M_PLANE, RC::M_ROW, r, 16 * (R + 1) + 4 * gq, zero);
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                f32x4 a = accA[I], m = accM[I];
                if (SH::NCG > 1) {
                    a += part[tri_index(R, I) * 64 + l];
                    if (!GRAD) m += part[(10 + tri_index(R, I)) * 64 + l];
                }
                accA[I] = a;   // the whole of A's tile (the gradient phase reads it)
                f32x4 mv;
#pragma unroll
                for (int j = 0; j < 4; ++j) mv[j] = (I < R || 4 * gq + j <= n) ? m[j] : 0.f;
                if constexpr (GRAD) {
                    // no record
                } else if constexpr (REV) {
                    const float m4[4] = {mv[0], mv[1], mv[2], mv[3]};
                    PR::template gstore_col<4>(rec + RC::OFF_MT, RC::MT_PLANE, RC::MT_ROW, 16 * I + 4 * gq, r, m4);
                } else {
                    PR::gstore4(rec + RC::OFF_M, RC::M_PLANE, RC::M_ROW, r, 16 * I + 4 * gq, mv);
                }
                if (I == R) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        ldiag[(R * 16 + n) * 17 + 4 * gq + j] = (4 * gq + j < n) ? br * a[j] : 0.f;
                } else {
                    f32x4 nv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) nv[j] = -br * a[j];
                    PR::store4(loffm, loff_index(R, I) * 64 + l, 0, nv);
                }
            }
        }
    }
    lds_sync();

    // ---- inverses of the diagonal blocks I + Ldiag_J (wave 0: J = g, column n)
    if (w == 0) {
        const int J = gq, cc = n;
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == cc) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= ldiag[(J * 16 + r) * 17 + i] * y[i];
            y[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) PR::store1(ym, J * 16 + r, cc, y[r]);
    }
    lds_sync();

    // ---- block forward substitution, one 16-column tile of [W | u] at a time
    // wave w: channel tiles w, w + NW, ... of W and value tiles w, w + NW, ... of u
    {
        // X Z = Diag(beta) rhs (with_beta), or X Z = rhs, for one 16-column tile
        auto substitute = [&](const float (&rhs)[4][4], f32x4 (&X)[4], bool with_beta = true) {
            typename PR::F4 Xb[4];
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                f32x4 z;
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = with_beta ? beta_s[16 * J + 4 * gq + i] * rhs[J][i] : rhs[J][i];
#pragma unroll
                for (int K = 0; K < J; ++K) z = PR::mma4(PR::load4(loffm, loff_index(J, K) * 64 + l, 0), Xb[K], z);
                X[J] = PR::mma4(PR::load4(ym, 16 * J + n, 4 * gq), PR::regs4(z), zero);
                Xb[J] = PR::regs4(X[J]);
            }
        };
        if constexpr (GRAD) {
            grad_phase1<Tin, DK, DV>(p, slot, h, tok0, L, smem, substitute, accA, vpre);
            return;
        }
#pragma unroll
        for (int vi = 0; vi < (REV ? 0 : VPW); ++vi) {   // (the reverse record has no u)
            const int vt = w + NW * vi;
            if (vt < DV / 16) {
                float rhs[4][4];
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = __uint_as_float(F32 ? vpre[vi][J][i] : (vpre[vi][J][i] << 16));
                        rhs[J][i] = (16 * J + 4 * gq + i < L) ? x : 0.f;   // padding rows of V are zero
                    }
                f32x4 X[4];
                substitute(rhs, X);
                if constexpr (MODE == kModeFwd) {
#pragma unroll
                    for (int J = 0; J < 4; ++J)
                        *reinterpret_cast<f32x4*>(rec + RC::OFF_U + ((J * (DV / 16) + vt) * 64 + l) * 16) = X[J];
                }
            }
        }
        for (int ct = w; ct < DK / 16; ct += NW) {
            // kf e^b = (kf e^{b - m}) e^m, m the anchor of the token's half
            const int c = 16 * ct + n;
            const float m0 = totb[c], m1 = m0 + totb[DK + c] + totb[2 * DK + c];
            const float em0 = EX ? 1.f : __builtin_amdgcn_exp2f(fminf(m0, 126.f));
            const float em1 = EX ? 1.f : __builtin_amdgcn_exp2f(fminf(m1, 126.f));
            float rhs[4][4];
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) rhs[J][i] = PR::get1(rkm, 16 * J + 4 * gq + i, c) * (J < 2 ? em0 : em1);
            f32x4 X[4];
            substitute(rhs, X);
            if constexpr (REV) {   // W^T: row 16ct + n, columns 16J + 4g .. +3
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    PR::gstore4(rec + RC::OFF_WT, RC::WT_PLANE, RC::WT_ROW, 16 * ct + n, 16 * J + 4 * gq, X[J]);
            } else if constexpr (MODE == kModeFwd) {
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int i = 0; i < 4; i += 2)
                        PR::gstore2c(rec + RC::OFF_W, RC::W_PLANE, RC::W_ROW, 16 * J + 4 * gq + i, 16 * ct + n,
                                     X[J][i], X[J][i + 1]);
            }
        }
    }
}

// one workgroup per (chunk slot, head); second bound: waves per SIMD (two
// 8-wave workgroups per CU -> 4, at most 128 VGPRs)
template <typename Tin, int DK, int DV, bool HG, bool NQK, int MODE, bool GM>
__global__ void __launch_bounds__(ChunkShape<DK>::NW * 64, 4) ckda_chunk_kernel(ChunkParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    // heads fastest: neighbouring workgroups share token rows
    chunk_body<Tin, DK, DV, HG, NQK, false, MODE, GM>(p, blockIdx.x / p.H, blockIdx.x % p.H, smem);
}

// The exact path over the records the fast kernel flagged: workgroup x looks
// at chunk-heads x*per .. x*per + per - 1 (per <= 64; record index = slot * H
// + head), whose flags one wave-wide load gathers, and redoes the flagged ones
// in turn.  With nothing flagged the launch reads one word per chunk-head.
template <typename Tin, int DK, int DV, bool HG, bool NQK, int MODE, bool GM>
__global__ void __launch_bounds__(ChunkShape<DK>::NW * 64, 4) ckda_chunk_exact_kernel(ChunkParams p, int nch, int per)
{
    using RC = std::conditional_t<MODE != kModeFwd, RevRecord<DK, DV, sizeof(Tin) == 4>, Record<DK, DV, sizeof(Tin) == 4>>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int c0 = blockIdx.x * per;
    const int l = threadIdx.x & 63;
    bool f = false;
    if (l < per && c0 + l < nch)
        f = (p.flags ? p.flags[c0 + l]
                     : *reinterpret_cast<const uint32_t*>(p.ws + static_cast<size_t>(c0 + l) * RC::BYTES + RC::OFF_FLAG)) != 0u;
    unsigned long long mask = __ballot(f);   // the same in every wave
    while (mask != 0ull) {
        const int j = __builtin_ctzll(mask);
        mask &= mask - 1ull;
        const int ch = c0 + j;
        chunk_body<Tin, DK, DV, HG, NQK, true, MODE, GM>(p, ch / p.H, ch % p.H, smem);
        lds_sync();   // before the next chunk-head reuses LDS
    }
}

template <typename Tin, int DK, int DV, bool HG, bool NQK, int MODE, bool GM>
static hipError_t launch_chunk_g(const ChunkParams& p, int nslots, hipStream_t stream) {
    using SH = ChunkShape<DK>;
    constexpr int LDS = MODE == kModeGrad ? GradShape<DK, DV>::LDS : SH::LDS;
    constexpr int LDS_EX = MODE == kModeGrad ? GradShape<DK, DV>::LDS : SH::LDS_EX;
    const long long grid = static_cast<long long>(nslots) * p.H;
    if (grid == 0) return hipSuccess;
    auto kern = ckda_chunk_kernel<Tin, DK, DV, HG, NQK, MODE, GM>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(SH::NW * 64), LDS, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // exact path: about 512 workgroups (two per CU), each over up to 64 chunk-heads
    auto kx = ckda_chunk_exact_kernel<Tin, DK, DV, HG, NQK, MODE, GM>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kx), hipFuncAttributeMaxDynamicSharedMemorySize, LDS_EX);
    if (e != hipSuccess) return e;
    const int per = static_cast<int>(grid > 512 * 64LL ? 64 : (grid + 511) / 512);
    const long long gx = (grid + per - 1) / per;
    hipLaunchKernelGGL(kx, dim3(static_cast<unsigned>(gx)), dim3(SH::NW * 64), LDS_EX, stream, p,
                       static_cast<int>(grid), per);
    return hipGetLastError();
}

// the optional gate map as a template parameter: the plain kernels carry none
// of its code
template <typename Tin, int DK, int DV, bool HG, bool NQK, int MODE>
static hipError_t launch_chunk_t(const ChunkParams& p, int nslots, hipStream_t stream) {
    return p.gate_map ? launch_chunk_g<Tin, DK, DV, HG, NQK, MODE, true>(p, nslots, stream)
                      : launch_chunk_g<Tin, DK, DV, HG, NQK, MODE, false>(p, nslots, stream);
}

template <typename Tin, int MODE>
static hipError_t launch_chunk_dt(const ChunkParams& p, const FwdArgs& A, int nslots, hipStream_t stream) {
#define CKDA_CHUNK(DK_, DV_)                                                                            \
    if (A.DK == DK_ && A.DV == DV_) {                                                                   \
        if (A.qk_norm)                                                                                  \
            return A.head_gate ? launch_chunk_t<Tin, DK_, DV_, true, true, MODE>(p, nslots, stream)     \
                               : launch_chunk_t<Tin, DK_, DV_, false, true, MODE>(p, nslots, stream);   \
        return A.head_gate ? launch_chunk_t<Tin, DK_, DV_, true, false, MODE>(p, nslots, stream)        \
                           : launch_chunk_t<Tin, DK_, DV_, false, false, MODE>(p, nslots, stream);      \
    }
    CKDA_CHUNK(32, 32) CKDA_CHUNK(32, 64) CKDA_CHUNK(32, 128)
    CKDA_CHUNK(64, 32) CKDA_CHUNK(64, 64) CKDA_CHUNK(64, 128)
    CKDA_CHUNK(128, 32) CKDA_CHUNK(128, 64) CKDA_CHUNK(128, 128)
#undef CKDA_CHUNK
    return hipErrorInvalidValue;
}

inline ChunkParams chunk_params(const FwdArgs& A) {
    ChunkParams p{};
    p.q = A.q; p.k = A.k; p.v = A.v; p.g = A.g; p.s = A.s; p.beta = A.beta;
    p.ws = static_cast<unsigned char*>(A.ws); p.cu = A.cu; p.T = A.T; p.H = A.H; p.ndocs = A.ndocs;
    p.gate_map = A.gate_map ? 1 : 0;
    return p;
}

}  // namespace ckda
