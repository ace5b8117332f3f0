// grad.hip -- the backward's second chunk-parallel gradient phase: dq, dk, dg.
//
// The backward is the plain reverse-mode derivative of the chunk form the
// forward computes (WY/UT chunk form of the recurrence, Complex KDA paper
// page, section 2 "Linear RNNs"; the sign folding of the signed gate as on the
// "complex-kda-1.3B-100B" model card).  Per chunk of 64 tokens, in the
// chunk-local folded frame, with b the in-chunk cumulative log-gate, P the
// in-chunk sign product, kf = P k, qf = P q, Gamma_ti = e^{b_t - b_i} per
// channel, and
//   Ke = kf e^b,  Qh = qf e^b,  KB = P_L kf e^{b_L - b},  d = P_L e^{b_L},
//   A_ti = sum_c kf_t kf_i Gamma_ti (i < t),  M_ti = sum_c qf_t kf_i Gamma_ti (i <= t),
// this phase takes S0 (the chunk-start state), G (dL/dS at the chunk's end,
// from the reverse pass), dO, and from the first phase dV = dL/dV,
// U, dA = dL/dA and dM = dL/dM, and forms
//   dQh = scale dO S0^T,  dKe = -dV S0^T,  dKB = U G^T,
//   dkf = sum_i dA_ti kf_i Gamma_ti + sum_t (dA_ti kf_t + dM_ti qf_t) Gamma_ti
//         + dKe e^b + P_L dKB e^{b_L - b},
//   dqf = sum_i dM_ti kf_i Gamma_ti + dQh e^b,
//   db  = kf (row part of dkf) + qf (row part of dqf) - kf (column part of dkf)
//         + Ke dKe + Qh dQh - KB dKB,
//   plus, at the chunk's last token (b_L, through KB and d):
//         sum_t KB dKB + d sum_v G S0,
//   dg_t = sum_{r >= t} db_r,  dq = P dqf,  dk = P dkf
// (and through the per-head L2 normalisation of q and k where it is on).
//
// Layout: one workgroup per (chunk slot, head), DK / 16 waves; wave w owns
// key channels 16w .. 16w+15 and lane (n, g) holds channel 16w + n at tokens
// 16J + 4g + i (J, i = 0..3): the C/D layout of a [token][channel] product.
// The value contractions with S0 and G take dO, dV, U rows as A operands and
// S0, G rows as B operands; the token contractions through dA and dM take the
// lane's own kf, qf (times the anchored exponentials) as B operands, so every
// product lands where the token's scans, the sign and the reverse cumulative
// sum for dg already are.  Gamma is factored through anchors at tokens 15 and
// 47, as in the chunk-local forward; chunks outside that envelope (flagged by
// the reverse-record pass) are skipped here and redone by the exact variant,
// which forms the Gamma-weighted sums entry by entry.
#include <type_traits>

#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"
#include "ckda_record.h"
#include "ckda_sync.h"

namespace ckda {

template <int DK, int DV, bool EX, int CW = DK>
struct Grad2Shape {
    static constexpr int NW = CW / 16;   // waves: one 16-channel tile each
    static constexpr int PA = 64 + 8;    // dA, dM pitch (elements)
    static constexpr int PV = DV + 8;    // dV, U pitch
    // phase a: dV and U, the A operands over the value channels
    static constexpr int L_DV = 0;
    static constexpr int L_U = L_DV + 64 * PV * 4;
    static constexpr int L_AEND = L_U + 64 * PV * 4;
    // phase b (over phase a): dA and dM as stored, and (fast variant) their
    // transposes; the exact variant holds kf, qf, b of every (token, channel)
    static constexpr int L_DA = 0;
    static constexpr int L_DM = L_DA + 64 * PA * 4;
    static constexpr int L_DAT = L_DM + 64 * PA * 4;
    static constexpr int L_DMT = L_DAT + 64 * PA * 4;
    static constexpr int L_X = L_DAT;                    // float [3][64][DK]: kf, qf, b (exact)
    static constexpr int L_XLO = L_X + 3 * 64 * DK * 4;  // bf16 [64][DK]: b's low part (exact)
    static constexpr int L_BEND = EX ? L_XLO + 64 * DK * 2 : L_DMT + 64 * PA * 4;
    // per-token partial sums over each wave's channels: float [2][NW][64]
    static constexpr int L_RED = L_AEND > L_BEND ? L_AEND : L_BEND;
    static constexpr int L_INV = L_RED + 2 * NW * 64 * 4;   // float [2][64]: 1/||k||, 1/||q||
    static constexpr int L_SUM = L_INV + 2 * 64 * 4;        // float [2][64]: per-token sums
    static constexpr int LDS = L_SUM + 2 * 64 * 4;
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert((L_U % 16) == 0 && (L_DM % 16) == 0 && (L_DAT % 16) == 0 && (L_RED % 16) == 0, "alignment");
};

struct Grad2Params {
    const void *q, *k;
    const float* g;
    const int8_t* s;
    const void* dout;
    const float* dv;            // dL/dV from the first phase, token layout [.., H, DV]
    const float* h_ckpt;        // chunk-start states (true frame)
    const float* G;             // dL/dS at each chunk's end, [slot][H][DK][DV]
    const unsigned char* gout;  // the first phase's dA, dM, U per (slot, head)
    size_t gout_bytes;
    const uint32_t* flags;      // per (slot, head): outside the anchors' envelope
    float *dq, *dk, *dg;
    const int32_t* cu;
    float scale;
    int T, H, ndocs;
    int gate_map;               // g holds the gate pre-activation (s unused); dg w.r.t. it
};

// Double-float sums (hi + lo, Knuth's two-sum) for the exact variant's
// cumulative log-gates: after a burst of strong decay b reaches hundreds,
// where one fp32 ulp would already spoil the O(1) factors e^{b_t - b_o}
// between the tokens that follow it.
struct DF { float hi, lo; };
__device__ __forceinline__ DF two_sum(float a, float b) {
    const float s = a + b, bb = s - a;
    return DF{s, (a - (s - bb)) + (b - bb)};
}
__device__ __forceinline__ DF df_add(DF a, DF b) {
    const DF s = two_sum(a.hi, b.hi);
    const float e = s.lo + (a.lo + b.lo), hi = s.hi + e;
    return DF{hi, e - (hi - s.hi)};
}

// e^x for x in natural units, clamped like exp2_clamped
__device__ __forceinline__ float ex2n(float x) { return __builtin_amdgcn_exp2f(fminf(x * kLog2e, 126.f)); }

// CW: key channels per workgroup (DK, or 64 of DK = 128 when no per-token sum
// over all channels is needed: two workgroups per chunk-head, part 0 and 1)
// GM: g holds the gate pre-activation (the optional gate map)
template <typename Tin, int DK, int DV, bool HG, bool NQK, bool EX, int CW, bool GM>
__device__ __forceinline__ void grad2_body(const Grad2Params& p, const int slot, const int h, const int part,
                                           unsigned char* smem)
{
    static_assert(CW == DK || (!HG && !NQK && !EX), "sums over all channels need the whole head in one workgroup");
    using SH = Grad2Shape<DK, DV, EX, CW>;
    constexpr bool F32 = sizeof(Tin) == 4;
    using PR = Prec<F32>;
    using GO = GradOut<DK, DV, F32>;
    constexpr int NW = SH::NW, NT = NW * 64;
    const int H = p.H;
    int tok0, L;
    size_t ck;   // checkpoint: equal-length [B][H][chunks][DK][DV], varlen [slot][H][DK][DV]
    const size_t ch = static_cast<size_t>(slot) * H + h;
    if (p.cu) {
        int lo = 0, hi = p.ndocs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (varlen_slot(p.cu[mid], mid, 0) <= slot) lo = mid; else hi = mid - 1;
        }
        const int j = slot - varlen_slot(p.cu[lo], lo, 0);
        const int len = p.cu[lo + 1] - p.cu[lo];
        if (64 * j >= len) return;   // unused slot (whole workgroup)
        tok0 = p.cu[lo] + 64 * j;
        L = min(64, len - 64 * j);
        ck = ch;
    } else {
        const int nch = (p.T + 63) / 64;
        const int b = slot / nch, j = slot - b * nch;
        tok0 = b * p.T + 64 * j;
        L = min(64, p.T - 64 * j);
        ck = (static_cast<size_t>(b) * H + h) * nch + j;
    }
    if (!EX && p.flags[ch] != 0u) return;   // the exact variant takes this chunk
    const int tid = EX ? opaque_tid() : static_cast<int>(threadIdx.x);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, n = l & 15, gq = l >> 4;
    const int c = CW * part + 16 * w + n;
    const unsigned char* const go = p.gout + ch * p.gout_bytes;
    float* const red = reinterpret_cast<float*>(smem + SH::L_RED);
    float* const inv = reinterpret_cast<float*>(smem + SH::L_INV);

    // ---- stage dV (split for the matrix cores) and U ------------------------
    const LdsMat dvm{smem + SH::L_DV, SH::PV, 64 * SH::PV};
    const LdsMat um{smem + SH::L_U, SH::PV, 64 * SH::PV};
    // The chunk's rows of the token tensors through buffer resources that end
    // after its last valid token: rows past it read as 0 and stores to them are
    // dropped, so no load or store below is guarded.  Offsets: a per-lane part
    // and a uniform part (row of the lane's token tile, value step).
    const size_t row0 = static_cast<size_t>(tok0) * H + h;
    const uint32_t rows = static_cast<uint32_t>((L - 1) * H + 1);   // token-head rows spanned
    constexpr int ES_IN = sizeof(Tin);
    {   // every load first, then the LDS writes (rows past the chunk read as 0)
        constexpr int NV = 64 * (DV / 8);                      // dV: 8-element units
        constexpr int UPR = DV * GO::ES / 16;                  // U: 16-byte units per row and plane
        constexpr int NU = GO::NP * 64 * UPR;
        constexpr int KV = (NV + NT - 1) / NT, KU = (NU + NT - 1) / NT;
        const __amdgpu_buffer_rsrc_t rdv = buffer_rsrc(p.dv + row0 * DV, rows * DV * 4);
        u32x4 xv[KV][2], xu[KU];
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int u = tid + k * NT, t = (u / (DV / 8)) & 63, v0 = 8 * (u % (DV / 8));
            const uint32_t off = static_cast<uint32_t>(t * H * DV + v0) * 4;
            xv[k][0] = buffer_load_u32x4(rdv, off, 0);
            xv[k][1] = buffer_load_u32x4(rdv, off, 16);
        }
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int u = min(tid + k * NT, NU - 1);
            const int pl = u / (64 * UPR), rr = (u / UPR) % 64, cu = u % UPR;
            xu[k] = *reinterpret_cast<const u32x4*>(go + GO::OFF_U + pl * GO::U_PLANE + static_cast<size_t>(rr) * GO::U_ROW +
                                                    cu * 16);
        }
#pragma unroll
        for (int k = 0; k < KV; ++k) {
            const int u = tid + k * NT, t = (u / (DV / 8)) & 63, v0 = 8 * (u % (DV / 8));
            const f32x4 a = __builtin_bit_cast(f32x4, xv[k][0]), b = __builtin_bit_cast(f32x4, xv[k][1]);
            const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            if (NV % NT == 0 || u < NV) PR::store8(dvm, t, v0, x);
        }
#pragma unroll
        for (int k = 0; k < KU; ++k) {
            const int u = tid + k * NT;
            const int pl = u / (64 * UPR), rr = (u / UPR) % 64, cu = u % UPR;
            if (NU % NT == 0 || u < NU)
                *reinterpret_cast<u32x4*>(smem + SH::L_U + (pl * 64 + rr) * SH::PV * GO::ES + cu * 16) = xu[k];
        }
    }

    lds_sync();   // dV, U staged
    // ---- phase a: dQh, dKe, dKB over the value channels ---------------------
    const __amdgpu_buffer_rsrc_t rS0 = buffer_rsrc(p.h_ckpt + ck * DK * DV, DK * DV * 4);
    const __amdgpu_buffer_rsrc_t rG = buffer_rsrc(p.G + ch * DK * DV, DK * DV * 4);
    const __amdgpu_buffer_rsrc_t rdO = buffer_rsrc(static_cast<const Tin*>(p.dout) + row0 * DV, rows * DV * ES_IN);
    // a lane's 8 K-slots of value step kv are the 8 adjacent value columns
    // 32 kv + 8 g .. +7 (the same in every operand), so a lane's dO row piece
    // is one 16-byte load
    const uint32_t vS = static_cast<uint32_t>(c * DV + 8 * gq) * 4;          // S0, G row c, columns 8g..
    const uint32_t vO = static_cast<uint32_t>(n * H * DV + 8 * gq) * ES_IN;  // dO row n of a tile, columns 8g..
    f32x4 aQ[4], aE[4], aB[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        aQ[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        aE[J] = aQ[J];
        aB[J] = aQ[J];
    }
    float sgs = 0.f;   // sum over the lane's value slots of G S0 (its channel)
    // S0, G and dO of value step kv (two 4-slot halves each), loaded one step
    // ahead of the products that use them
    constexpr int NKV = DV / 32;
    using DOF = std::conditional_t<F32, f32x4, u32x4>;
    f32x4 sv[2][2], gv[2][2];
    DOF ov[2][4][F32 ? 2 : 1];
    auto load_kv = [&](int kv, int slot) {
        sv[slot][0] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rS0, vS, 128 * kv));
        sv[slot][1] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rS0, vS, 128 * kv + 16));
        gv[slot][0] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rG, vS, 128 * kv));
        gv[slot][1] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rG, vS, 128 * kv + 16));
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const uint32_t so = static_cast<uint32_t>(16 * J * H * DV + 32 * kv) * ES_IN;
            if constexpr (F32) {
                ov[slot][J][0] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rdO, vO, so));
                ov[slot][J][1] = __builtin_bit_cast(f32x4, buffer_load_u32x4(rdO, vO, so + 16));
            } else {
                ov[slot][J][0] = buffer_load_u32x4(rdO, vO, so);
            }
        }
    };
    load_kv(0, 0);
#pragma unroll
    for (int kv = 0; kv < NKV; ++kv) {
        const int cur = kv & 1;
        if (kv + 1 < NKV) load_kv(kv + 1, cur ^ 1);
        const int va = 32 * kv + 8 * gq, vb = va + 4;
        const f32x4 s0a = sv[cur][0], s0b = sv[cur][1], ga = gv[cur][0], gb = gv[cur][1];
#pragma unroll
        for (int e = 0; e < 4; ++e) sgs += s0a[e] * ga[e] + s0b[e] * gb[e];
        const typename PR::F8 BS = PR::regs8(s0a, s0b), BG = PR::regs8(ga, gb);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            typename PR::F8 Ao;   // dO row 16J + n (bf16 inputs: exact in the hi plane)
            if constexpr (F32) {
                Ao.a = ov[cur][J][0];
                Ao.b = ov[cur][J][1];
            } else {
                Ao.hi = __builtin_bit_cast(bf16x8, ov[cur][J][0]);
                Ao.lo = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            }
            aQ[J] = PR::mma8(Ao, BS, aQ[J]);
            aE[J] = PR::mma8(PR::load4x2(dvm, 16 * J + n, va, vb), BS, aE[J]);
            aB[J] = PR::mma8(PR::load4x2(um, 16 * J + n, va, vb), BG, aB[J]);
        }
    }
    sgs += __shfl_xor(sgs, 16, 64);
    sgs += __shfl_xor(sgs, 32, 64);
    CKDA_FENCE();
    // ---- the lane's channel at its 16 tokens: gates, signs, q, k ------------
    float bl[4][4], kf[4][4], qf[4][4];
    uint32_t neg = 0;   // bit 4J + i: s < 0 at token 16J + 4g + i
    {
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(static_cast<const Tin*>(p.q) + row0 * DK, rows * DK * ES_IN);
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(static_cast<const Tin*>(p.k) + row0 * DK, rows * DK * ES_IN);
        constexpr int GX = HG ? 1 : DK;   // gate and sign elements per token-head row
        const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(p.g + row0 * GX, rows * GX * 4);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.s + row0 * GX, GM ? 0u : rows * GX);   // (unread with the map)
        const uint32_t lrow = static_cast<uint32_t>(4 * gq * H);   // the lane's first token row
        const uint32_t vq = (lrow * DK + c) * ES_IN, vg = (lrow * GX + (HG ? 0 : c));
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t tr = static_cast<uint32_t>((16 * J + i) * H);   // uniform row step
                bl[J][i] = buffer_load_f32(rg, 4 * vg, 4 * tr * GX);   // padding tokens read 0: no gate
                neg |= buffer_load_i8(rs, vg, tr * GX) < 0 ? (1u << (4 * J + i)) : 0u;   // (0 with the map)
                kf[J][i] = buffer_load_elem<Tin>(rk, vq, tr * DK * ES_IN);
                qf[J][i] = buffer_load_elem<Tin>(rq, vq, tr * DK * ES_IN);
            }
        if constexpr (GM) {   // the optional gate map, on the loaded pre-activations
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    neg |= bl[J][i] < 0.f ? (1u << (4 * J + i)) : 0u;
                    bl[J][i] = 16 * J + 4 * gq + i < L ? gate_map_g(bl[J][i]) : 0.f;
                }
        }
    }
    // per-token sums over all channels of two lane values val(J, i, 0 / 1):
    // the wave's 16 channels by a row scan, then 128 threads over the waves'
    // partials; out[64 * which + token]
    auto token_sums = [&](auto val, float* out) {
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sx = row_scan_add(val(J, i, 0)), sy = row_scan_add(val(J, i, 1));
                if (n == 15) {
                    red[w * 64 + 16 * J + 4 * gq + i] = sx;
                    red[(NW + w) * 64 + 16 * J + 4 * gq + i] = sy;
                }
            }
        lds_sync();
        if (tid < 128) {
            const int qq = tid >> 6, t = tid & 63;
            float a = 0.f;
#pragma unroll
            for (int x2 = 0; x2 < NW; ++x2) a += red[(qq * NW + x2) * 64 + t];
            out[tid] = a;
        }
        lds_sync();
    };
    if constexpr (NQK) {   // 1 / ||k||, 1 / ||q|| per token
        token_sums([&](int J, int i, int which) { return which ? qf[J][i] * qf[J][i] : kf[J][i] * kf[J][i]; }, inv);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            CKDA_FENCE();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * J + 4 * gq + i;
                kf[J][i] *= inv_norm(inv[tt]);
                qf[J][i] *= inv_norm(inv[64 + tt]);
            }
        }
    }
    // In-chunk sums of the log-gate, in natural units and kept tile-local:
    // for the lane's token (J, i), l = the in-tile inclusive prefix, r = the
    // in-tile exclusive suffix, T_J = the tile totals (lane order J, g, i:
    // within the lane, over the four lane groups, over the tiles).  Every
    // exponent below is a sum of such pieces, never the difference of two
    // long prefix sums (which at strong decay would cost the exponentials
    // their low bits).  bl holds g on entry and l on exit.
    uint32_t pbit = 0;   // bit 4J + i: P = -1 at the lane's token (J, i)
    float rs[4][4];      // r
    float T[4];          // tile totals (the same in all lanes of a channel)
    {
        float lt[4];
        uint32_t par[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            uint32_t pr = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i > 0) bl[J][i] += bl[J][i - 1];
                pr ^= (neg >> (4 * J + i)) & 1u;
                pbit |= pr << (4 * J + i);
            }
            lt[J] = bl[J][3];
            par[J] = pr;
#pragma unroll
            for (int i = 0; i < 4; ++i) rs[J][i] = lt[J] - bl[J][i];   // later tokens of the lane
        }
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            float ex = 0.f, ey = 0.f;   // groups g' < g, g' > g of tile J
            uint32_t px = 0;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const float tv = __shfl(lt[J], n + 16 * x, 64);
                const uint32_t pv = static_cast<uint32_t>(__shfl(static_cast<int>(par[J]), n + 16 * x, 64));
                if (x < gq) {
                    ex += tv;
                    px ^= pv;
                }
                if (x > gq) ey += tv;
            }
            float tt = lt[J];
            tt += __shfl_xor(tt, 16, 64);
            tt += __shfl_xor(tt, 32, 64);
            T[J] = tt;
            uint32_t pt = par[J];
            pt ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(pt), 16, 64));
            pt ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(pt), 32, 64));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bl[J][i] += ex;
                rs[J][i] += ey;
            }
            if (px) pbit ^= 0xFu << (4 * J);
#pragma unroll
            for (int J2 = J + 1; J2 < 4; ++J2)
                if (pt) pbit ^= 0xFu << (4 * J2);
        }
    }
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sgn = ((pbit >> (4 * J + i)) & 1u) << 31;
            kf[J][i] = __uint_as_float(__float_as_uint(kf[J][i]) ^ sgn);
            qf[J][i] = __uint_as_float(__float_as_uint(qf[J][i]) ^ sgn);
        }
    // anchors m0 = b at token 15, m1 = b at token 47; b_L = b at token 63 and
    // the sign of P_L (padding tokens carry no gate and no sign, so token 63
    // stands for L - 1).  With them, per token:
    //   b       = l + (T_0 + .. + T_{J-1})
    //   b_L - b = r + (T_{J+1} + .. + T_3)
    //   b - m0  = -r (J = 0), l (J = 1)
    //   b - m1  = -(r + T_1 + T_2), -(r + T_2), -r, l (J = 0..3)
    const float T12 = T[1] + T[2], T23 = T[2] + T[3];
    const float m1 = T[0] + T12, bL = m1 + T[3];
    const bool pL = (static_cast<uint32_t>(__shfl(static_cast<int>(pbit), n + 48, 64)) >> 15) & 1u;
    const float PLs = pL ? -1.f : 1.f;
    float xh[4][4];   // fast variant: b - m0 (J < 2), b - m1 (J >= 2); exact variant: b (high part)
    float xc[2][4];   // fast variant: b - m1 (J < 2)

    // per-token partials of dkf, dqf and db
    float pkf[4][4], pqf[4][4], pdb[4][4];
    float kbs = 0.f;   // sum over the lane's tokens of KB dKB
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float l = bl[J][i], r = rs[J][i];
            const float b = J == 0 ? l : J == 1 ? l + T[0] : J == 2 ? l + (T[0] + T[1]) : l + m1;
            const float xL = J == 0 ? r + (T[1] + T23) : J == 1 ? r + T23 : J == 2 ? r + T[3] : r;
            if constexpr (EX) {
                (void)xh;   // (the exact variant stages b itself below)
            } else {
                xh[J][i] = J == 0 ? -r : J == 1 ? l : J == 2 ? -r : l;
                if (J < 2) xc[J][i] = J == 0 ? -(r + T12) : -(r + T[2]);
            }
            const float eb = ex2n(b), ebl = ex2n(xL);
            const float dQh = p.scale * aQ[J][i], dKe = -aE[J][i], dKB = aB[J][i];
            const float kb = PLs * kf[J][i] * ebl;   // KB
            pkf[J][i] = dKe * eb + PLs * dKB * ebl;
            pqf[J][i] = dQh * eb;
            pdb[J][i] = kf[J][i] * eb * dKe + qf[J][i] * eb * dQh - kb * dKB;
            kbs += kb * dKB;
        }
    kbs += __shfl_xor(kbs, 16, 64);
    kbs += __shfl_xor(kbs, 32, 64);
    if (gq == 3) pdb[3][3] += kbs + PLs * ex2n(bL) * sgs;

    // ---- phase b: the Gamma-weighted sums through dA and dM -----------------
    lds_sync();   // dV and U consumed
    const LdsMat dam{smem + SH::L_DA, SH::PA, 64 * SH::PA};
    const LdsMat dmm{smem + SH::L_DM, SH::PA, 64 * SH::PA};
    const LdsMat datm{smem + SH::L_DAT, SH::PA, 64 * SH::PA};
    const LdsMat dmtm{smem + SH::L_DMT, SH::PA, 64 * SH::PA};
    {   // dA, dM as stored (row = output token) and, fast variant, transposed.
        // The block (0..31, 32..63) is never written nor read.  Lanes walk
        // rows, so the transposed writes (one row of the transpose per element
        // column) go to consecutive words: bf16 packs rows 2r, 2r+1 of one
        // column into one word; 32 row pairs of two 16-byte column units per
        // wave meet 64 distinct banks at the 72-element pitch.
        constexpr int EPU = 16 / GO::ES;                      // elements per 16-byte unit
        constexpr int UPR = 64 / EPU;                         // units per row
        constexpr int RPT = F32 ? 1 : 2;                      // rows per task
        constexpr int RG = 64 / RPT;                          // row groups per unit column
        constexpr int NTK = 2 * GO::NP * RG * UPR;            // tasks (both matrices, all planes)
        constexpr int KT = (NTK + NT - 1) / NT;
        u32x4 x[KT][RPT];
        auto task = [&](int q, int& mat, int& pl, int& r0, int& cu) {
            const int rg = q % RG;
            cu = (q / RG) % UPR;
            pl = (q / (RG * UPR)) % GO::NP;
            mat = q / (RG * UPR * GO::NP);
            r0 = RPT * rg;
        };
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            int mat, pl, r0, cu;
            task(min(tid + k * NT, NTK - 1), mat, pl, r0, cu);
            const unsigned char* src = go + (mat ? GO::OFF_DM : GO::OFF_DA) + pl * GO::A_PLANE + cu * 16;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                x[k][r] = (r0 < 32 && cu >= UPR / 2)
                              ? u32x4{0u, 0u, 0u, 0u}
                              : *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(r0 + r) * GO::A_ROW);
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const int q = tid + k * NT;
            int mat, pl, r0, cu;
            task(q, mat, pl, r0, cu);
            if ((NTK % NT != 0 && q >= NTK) || (r0 < 32 && cu >= UPR / 2)) continue;
            unsigned char* const nat = smem + (mat ? SH::L_DM : SH::L_DA) + pl * 64 * SH::PA * GO::ES;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                *reinterpret_cast<u32x4*>(nat + (r0 + r) * SH::PA * GO::ES + cu * 16) = x[k][r];
            if constexpr (!EX) {
                unsigned char* const tr = smem + (mat ? SH::L_DMT : SH::L_DAT) + pl * 64 * SH::PA * GO::ES;
                if constexpr (F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *reinterpret_cast<uint32_t*>(tr + (EPU * cu + e) * SH::PA * 4 + r0 * 4) = x[k][0][e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t lo = (x[k][0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        const uint32_t hi = (x[k][1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        *reinterpret_cast<uint32_t*>(tr + (EPU * cu + e) * SH::PA * 2 + r0 * 2) = lo | (hi << 16);
                    }
                }
            }
        }
    }
    if constexpr (EX) {   // kf, qf and b (as two parts) of the lane's channel at its tokens
        float* const xk = reinterpret_cast<float*>(smem + SH::L_X);
        uint16_t* const xlo = reinterpret_cast<uint16_t*>(smem + SH::L_XLO);
        constexpr int GX = HG ? 1 : DK;
        const __amdgpu_buffer_rsrc_t rg = buffer_rsrc(p.g + row0 * GX, rows * GX * 4);
        const uint32_t vg = static_cast<uint32_t>(4 * gq * H) * GX + (HG ? 0 : c);
        DF bd[4][4], lt[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gx = buffer_load_f32(rg, 4 * vg, 4 * static_cast<uint32_t>((16 * J + i) * H) * GX);
                const float gv = GM ? (16 * J + 4 * gq + i < L ? gate_map_g(gx) : 0.f) : gx;
                bd[J][i] = i == 0 ? DF{gv, 0.f} : df_add(bd[J][i - 1], DF{gv, 0.f});
            }
            lt[J] = bd[J][3];
        }
        DF pre{0.f, 0.f};   // the earlier tiles
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            DF ex{0.f, 0.f}, tt{0.f, 0.f};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const DF tv{__shfl(lt[J].hi, n + 16 * x, 64), __shfl(lt[J].lo, n + 16 * x, 64)};
                if (x < gq) ex = df_add(ex, tv);
                tt = df_add(tt, tv);   // the same order in every lane
            }
            const DF off = df_add(pre, ex);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * J + 4 * gq + i;
                const DF b = df_add(off, bd[J][i]);
                xk[t * DK + c] = kf[J][i];
                xk[(64 + t) * DK + c] = qf[J][i];
                xk[(128 + t) * DK + c] = b.hi;
                xlo[t * DK + c] = f32_to_bf16(b.lo);
            }
            pre = df_add(pre, tt);
        }
    }
    lds_sync();
    if constexpr (!EX) {
        // B operand over the tokens of half kt (the lane's tiles 2kt, 2kt+1):
        // x times e^{sg * y} per token, ya / yb the anchored exponents of the
        // two tiles
        auto bfrag = [&](const float (&x)[4][4], int kt, const float (&ya)[4], const float (&yb)[4], float sg) {
            f32x4 a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = x[2 * kt][i] * ex2n(sg * ya[i]);
                b[i] = x[2 * kt + 1][i] * ex2n(sg * yb[i]);
            }
            return PR::regs8(a, b);
        };
        const int k0 = 4 * gq, k1 = 32 + 4 * gq;   // K slots of half 0 and half 1
        // rows t: sums over i <= t (rK: dA with kf, rQ: dM with kf);
        // rows i: sums over t >= i (c0 over half 0, c1 over half 1: dA^T with
        // kf, dM^T with qf).  Anchors: m0 inside half 0, m1 inside half 1 and
        // across the halves.
        f32x4 rK[4], rQ[4], c0[2], c1[4];
        const f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f};
        {   // half 1 as the summed (row) token, e^{b - m1}: every tile
            const typename PR::F8 Xk = bfrag(kf, 1, xh[2], xh[3], 1.f), Xq = bfrag(qf, 1, xh[2], xh[3], 1.f);
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                c1[J] = PR::mma8(PR::load4x2(datm, 16 * J + n, k1, k1 + 16), Xk, z4);
                c1[J] = PR::mma8(PR::load4x2(dmtm, 16 * J + n, k1, k1 + 16), Xq, c1[J]);
            }
        }
        CKDA_FENCE();
        {   // inside half 0, e^{m0 - b} and e^{b - m0}: tiles 0 and 1
            const typename PR::F8 R = bfrag(kf, 0, xh[0], xh[1], -1.f);
            const typename PR::F8 Ck = bfrag(kf, 0, xh[0], xh[1], 1.f), Cq = bfrag(qf, 0, xh[0], xh[1], 1.f);
#pragma unroll
            for (int J = 0; J < 2; ++J) {
                rK[J] = PR::mma8(PR::load4x2(dam, 16 * J + n, k0, k0 + 16), R, z4);
                rQ[J] = PR::mma8(PR::load4x2(dmm, 16 * J + n, k0, k0 + 16), R, z4);
                c0[J] = PR::mma8(PR::load4x2(datm, 16 * J + n, k0, k0 + 16), Ck, z4);
                c0[J] = PR::mma8(PR::load4x2(dmtm, 16 * J + n, k0, k0 + 16), Cq, c0[J]);
            }
        }
        CKDA_FENCE();
        {   // rows of half 1 over both halves, e^{m1 - b}: tiles 2 and 3
            const typename PR::F8 R0 = bfrag(kf, 0, xc[0], xc[1], -1.f), R1 = bfrag(kf, 1, xh[2], xh[3], -1.f);
#pragma unroll
            for (int J = 2; J < 4; ++J) {
                rK[J] = PR::mma8(PR::load4x2(dam, 16 * J + n, k0, k0 + 16), R0, z4);
                rK[J] = PR::mma8(PR::load4x2(dam, 16 * J + n, k1, k1 + 16), R1, rK[J]);
                rQ[J] = PR::mma8(PR::load4x2(dmm, 16 * J + n, k0, k0 + 16), R0, z4);
                rQ[J] = PR::mma8(PR::load4x2(dmm, 16 * J + n, k1, k1 + 16), R1, rQ[J]);
            }
        }
        CKDA_FENCE();
#pragma unroll
        for (int J = 0; J < 4; ++J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float fr = ex2n(xh[J][i]);                        // e^{b_t - m}
                const float f1 = ex2n(-(J < 2 ? xc[J & 1][i] : xh[J][i]));   // e^{m1 - b_i}
                const float dkR = rK[J][i] * fr, dqR = rQ[J][i] * fr;
                const float dkC = J < 2 ? c0[J & 1][i] * ex2n(-xh[J][i]) + c1[J][i] * f1 : c1[J][i] * f1;
                pdb[J][i] += qf[J][i] * dqR + kf[J][i] * (dkR - dkC);
                pkf[J][i] += dkR + dkC;   // dkf
                pqf[J][i] += dqR;         // dqf
            }
        }
    } else {
        // entry by entry, e^{b_t - b_o} taken whole (b_t - b_o from the two
        // parts of each b); kf, qf, b of the other token o from LDS (16
        // distinct words per wave: broadcast reads); one token tile at a time
        const float* const xk = reinterpret_cast<const float*>(smem + SH::L_X);
        const uint16_t* const xlo = reinterpret_cast<const uint16_t*>(smem + SH::L_XLO);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            CKDA_FENCE();
            float dkR[4] = {0.f, 0.f, 0.f, 0.f}, dqR[4] = {0.f, 0.f, 0.f, 0.f}, dkC[4] = {0.f, 0.f, 0.f, 0.f};
            float bh[4], blo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * J + 4 * gq + i;
                bh[i] = xk[(128 + tt) * DK + c];
                blo[i] = bf16_to_f32(xlo[tt * DK + c]);
            }
#pragma unroll 1
            for (int o = 0; o < 64; ++o) {
                const float ko = xk[o * DK + c], qo = xk[(64 + o) * DK + c];
                const float bo = xk[(128 + o) * DK + c], bol = bf16_to_f32(xlo[o * DK + c]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 16 * J + 4 * gq + i;
                    const float dbt = (bh[i] - bo) + (blo[i] - bol);
                    const float gr = ex2n(dbt);    // Gamma_{t o}
                    const float gc = ex2n(-dbt);   // Gamma_{o t}
                    // dA, dM: zero on and above the diagonal (dA), above it (dM)
                    const float dA_to = o < tt ? PR::get1(dam, tt, o) : 0.f;
                    const float dM_to = o <= tt ? PR::get1(dmm, tt, o) : 0.f;
                    const float dA_ot = o > tt ? PR::get1(dam, o, tt) : 0.f;
                    const float dM_ot = o >= tt ? PR::get1(dmm, o, tt) : 0.f;
                    dkR[i] += dA_to * ko * gr;
                    dqR[i] += dM_to * ko * gr;
                    dkC[i] += (dA_ot * ko + dM_ot * qo) * gc;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pdb[J][i] += qf[J][i] * dqR[i] + kf[J][i] * (dkR[i] - dkC[i]);
                pkf[J][i] += dkR[i] + dkC[i];   // dkf
                pqf[J][i] += dqR[i];            // dqf
            }
        }
    }
    // dg: reverse cumulative sum of db over the chunk's tokens (in the lane,
    // over the later lane groups of the tile, then over the later tiles)
    {
        float tot[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
#pragma unroll
            for (int i = 2; i >= 0; --i) pdb[J][i] += pdb[J][i + 1];
            tot[J] = pdb[J][0];
        }
        float later = 0.f;
#pragma unroll
        for (int J = 3; J >= 0; --J) {
            float ex = 0.f;
#pragma unroll
            for (int x = 1; x < 4; ++x) {
                const float tv = __shfl(tot[J], n + 16 * x, 64);
                if (x > gq) ex += tv;
            }
            float tt = tot[J];
            tt += __shfl_xor(tt, 16, 64);
            tt += __shfl_xor(tt, 32, 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) pdb[J][i] += ex + later;
            later += tt;
        }
    }
    // back to the unfolded frame: dq^ = P dqf, dk^ = P dkf
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sgn = ((pbit >> (4 * J + i)) & 1u) << 31;
            pkf[J][i] = __uint_as_float(__float_as_uint(pkf[J][i]) ^ sgn);
            pqf[J][i] = __uint_as_float(__float_as_uint(pqf[J][i]) ^ sgn);
            kf[J][i] = __uint_as_float(__float_as_uint(kf[J][i]) ^ sgn);   // k^ (normalised when NQK)
            qf[J][i] = __uint_as_float(__float_as_uint(qf[J][i]) ^ sgn);
        }
    if constexpr (NQK) {   // dx = (dx^ - x^ (x^ . dx^)) / ||x|| per token
        float* const dots = reinterpret_cast<float*>(smem + SH::L_SUM);
        lds_sync();   // (the partial-sum area is reused)
        token_sums([&](int J, int i, int which) { return which ? qf[J][i] * pqf[J][i] : kf[J][i] * pkf[J][i]; },
                   dots);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            CKDA_FENCE();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * J + 4 * gq + i;
                pkf[J][i] = (pkf[J][i] - kf[J][i] * dots[tt]) * inv_norm(inv[tt]);
                pqf[J][i] = (pqf[J][i] - qf[J][i] * dots[64 + tt]) * inv_norm(inv[64 + tt]);
            }
        }
    }
    if constexpr (!HG) {
        if constexpr (GM) {   // dL/dx through the optional gate map (x reread, one token tile at a time)
            const __amdgpu_buffer_rsrc_t rgx = buffer_rsrc(p.g + row0 * DK, rows * DK * 4);
            const uint32_t vx = (static_cast<uint32_t>(4 * gq * H) * DK + c) * 4;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                CKDA_FENCE();
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pdb[J][i] *= gate_map_dgdx(buffer_load_f32(rgx, vx, static_cast<uint32_t>((16 * J + i) * H * DK) * 4));
            }
        }
    }
    // ---- outputs -------------------------------------------------------------
    {
        const __amdgpu_buffer_rsrc_t rdq = buffer_rsrc(p.dq + row0 * DK, rows * DK * 4);
        const __amdgpu_buffer_rsrc_t rdk = buffer_rsrc(p.dk + row0 * DK, rows * DK * 4);
        const __amdgpu_buffer_rsrc_t rdg = buffer_rsrc(p.dg + row0 * DK, HG ? 0u : rows * DK * 4);

        const uint32_t vq = (static_cast<uint32_t>(4 * gq * H) * DK + c) * 4;
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t so = static_cast<uint32_t>((16 * J + i) * H * DK) * 4;
                buffer_store_f32(rdk, vq, so, pkf[J][i]);
                buffer_store_f32(rdq, vq, so, pqf[J][i]);
                if constexpr (!HG) buffer_store_f32(rdg, vq, so, pdb[J][i]);
            }
    }
    if constexpr (HG) {   // one gate per (token, head): dg summed over the channels
        float* const sums = reinterpret_cast<float*>(smem + SH::L_SUM);
        lds_sync();
        token_sums([&](int J, int i, int) { return pdb[J][i]; }, sums);
        if (tid < L) {
            const size_t o = row0 + static_cast<size_t>(tid) * H;
            p.dg[o] = GM ? sums[tid] * gate_map_dgdx(p.g[o]) : sums[tid];   // dL/dx with the map
        }
    }
}

// channels per workgroup of the fast kernel
template <int DK, bool HG, bool NQK>
constexpr int grad2_cw() { return (HG || NQK || DK <= 64) ? DK : 64; }

// one workgroup per (chunk slot, head) and group of CW key channels, heads
// fastest.  With two channel groups, groups of eight chunk-heads take eight
// consecutive workgroups per channel group, so both halves of a chunk-head
// land on the same XCD (workgroups go to the XCDs in turn), where the
// operands both stage share its L2.
template <typename Tin, int DK, int DV, bool HG, bool NQK, bool GM>
__global__ void __launch_bounds__((grad2_cw<DK, HG, NQK>() * 4), 2) ckda_grad2_kernel(Grad2Params p, int nch)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CW = grad2_cw<DK, HG, NQK>();
    int chh = blockIdx.x, part = 0;
    if constexpr (CW < DK) {
        chh = (blockIdx.x / 16) * 8 + (blockIdx.x & 7);
        part = (blockIdx.x >> 3) & 1;
        if (chh >= nch) return;
    }
    grad2_body<Tin, DK, DV, HG, NQK, false, CW, GM>(p, chh / p.H, chh % p.H, part, smem);
}

// the exact variant over the flagged chunk-heads (whole heads): workgroup x
// looks at chunk-heads x*per .. x*per + per - 1 (per <= 64) and redoes the
// flagged ones in turn
template <typename Tin, int DK, int DV, bool HG, bool NQK, bool GM>
__global__ void __launch_bounds__(DK * 4, 2) ckda_grad2_exact_kernel(Grad2Params p, int nch, int per)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int c0 = blockIdx.x * per;
    const int l = threadIdx.x & 63;
    const bool f = l < per && c0 + l < nch && p.flags[c0 + l] != 0u;
    unsigned long long mask = __ballot(f);   // the same in every wave
    while (mask != 0ull) {
        const int j = __builtin_ctzll(mask);
        mask &= mask - 1ull;
        const int chh = c0 + j;
        grad2_body<Tin, DK, DV, HG, NQK, true, DK, GM>(p, chh / p.H, chh % p.H, 0, smem);
        lds_sync();   // before the next chunk-head reuses LDS
    }
}

template <typename Tin, int DK, int DV, bool HG, bool NQK, bool GM>
static hipError_t launch_grad2_g(const Grad2Params& p, int nslots, hipStream_t stream) {
    constexpr int CW = grad2_cw<DK, HG, NQK>();
    constexpr int LDS = Grad2Shape<DK, DV, false, CW>::LDS, LDS_EX = Grad2Shape<DK, DV, true>::LDS;
    const long long nch = static_cast<long long>(nslots) * p.H;
    if (nch == 0) return hipSuccess;
    const long long grid = CW == DK ? nch : (nch + 7) / 8 * 16;
    auto kern = ckda_grad2_kernel<Tin, DK, DV, HG, NQK, GM>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(CW * 4), LDS, stream, p, static_cast<int>(nch));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    auto kx = ckda_grad2_exact_kernel<Tin, DK, DV, HG, NQK, GM>;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kx), hipFuncAttributeMaxDynamicSharedMemorySize, LDS_EX);
    if (e != hipSuccess) return e;
    const int per = static_cast<int>(nch > 512 * 64LL ? 64 : (nch + 511) / 512);
    const long long gx = (nch + per - 1) / per;
    hipLaunchKernelGGL(kx, dim3(static_cast<unsigned>(gx)), dim3(DK * 4), LDS_EX, stream, p,
                       static_cast<int>(nch), per);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV, bool HG, bool NQK>
static hipError_t launch_grad2_t(const Grad2Params& p, int nslots, hipStream_t stream) {
    return p.gate_map ? launch_grad2_g<Tin, DK, DV, HG, NQK, true>(p, nslots, stream)
                      : launch_grad2_g<Tin, DK, DV, HG, NQK, false>(p, nslots, stream);
}

template <typename Tin>
static hipError_t launch_grad2_dt(const Grad2Params& p, const FwdArgs& A, int nslots, hipStream_t stream) {
#define CKDA_G2(DK_, DV_)                                                                           \
    if (A.DK == DK_ && A.DV == DV_) {                                                               \
        if (A.qk_norm)                                                                              \
            return A.head_gate ? launch_grad2_t<Tin, DK_, DV_, true, true>(p, nslots, stream)       \
                               : launch_grad2_t<Tin, DK_, DV_, false, true>(p, nslots, stream);     \
        return A.head_gate ? launch_grad2_t<Tin, DK_, DV_, true, false>(p, nslots, stream)          \
                           : launch_grad2_t<Tin, DK_, DV_, false, false>(p, nslots, stream);        \
    }
    CKDA_G2(32, 32) CKDA_G2(32, 64) CKDA_G2(32, 128)
    CKDA_G2(64, 32) CKDA_G2(64, 64) CKDA_G2(64, 128)
    CKDA_G2(128, 32) CKDA_G2(128, 64) CKDA_G2(128, 128)
#undef CKDA_G2
    return hipErrorInvalidValue;
}

hipError_t launch_grad2(const FwdArgs& A, const Grad2Args& G, int nslots, hipStream_t stream) {
    Grad2Params p{};
    p.q = A.q; p.k = A.k; p.g = A.g; p.s = A.s; p.dout = G.dout; p.dv = G.dv;
    p.h_ckpt = G.h_ckpt; p.G = G.G; p.gout = G.gout; p.gout_bytes = G.gout_bytes; p.flags = G.flags;
    p.dq = G.dq; p.dk = G.dk; p.dg = G.dg; p.cu = A.cu; p.scale = A.scale;
    p.T = A.T; p.H = A.H; p.ndocs = A.ndocs; p.gate_map = A.gate_map ? 1 : 0;
    return A.bf16 ? launch_grad2_dt<bf16_t>(p, A, nslots, stream) : launch_grad2_dt<float>(p, A, nslots, stream);
}

}  // namespace ckda
