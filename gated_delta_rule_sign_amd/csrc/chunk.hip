// chunk.hip -- chunk-local kernel of the chunked CKDA forward, and the
// standalone gate / sign-fold prep kernel.
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
    static constexpr int L_COLK = L_NRM + NCG * 64 * 8;       // operand [64][PC]
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
};

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
};

// HG: one gate per (token, head) (g, s [.., H]), broadcast over the channels;
// NQK: q and k normalised per (token, head) over the key channels
template <typename Tin, int DK, int DV, bool HG, bool NQK>
// second bound: waves per SIMD (two 8-wave workgroups per CU -> 4, at most 128 VGPRs)
__global__ void __launch_bounds__(ChunkShape<DK>::NW * 64, 4) ckda_chunk_kernel(ChunkParams p)
{
    using SH = ChunkShape<DK>;
    constexpr bool F32 = sizeof(Tin) == 4;
    using PR = Prec<F32>;
    using RC = Record<DK, DV, F32>;
    constexpr int NW = SH::NW, KSW = SH::KSW, NE = SH::NE, CG = SH::CG, PC = SH::PC;
    extern __shared__ __align__(16) unsigned char smem[];

    const int H = p.H;
    const int h = blockIdx.x % H;        // heads fastest: neighbouring workgroups share token rows
    const int slot = blockIdx.x / H;
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
        if (64 * j >= len) return;       // unused slot (whole workgroup)
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

    const int tid = threadIdx.x;
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
                const float gt = p.g[trow];
                const uint32_t sw = static_cast<uint32_t>(static_cast<uint8_t>(p.s[trow])) * 0x01010101u;
#pragma unroll
                for (int e = 0; e < 8; ++e) bs[8 * ks + e] = gt;
                par[2 * ks] = sw;
                par[2 * ks + 1] = sw;
            } else {
                const float4 a = reinterpret_cast<const float4*>(p.g + base)[0];
                const float4 b = reinterpret_cast<const float4*>(p.g + base)[1];
                const uint2 sv = *reinterpret_cast<const uint2*>(p.s + base);
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
        const float bt = p.beta[trow];
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
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CG * cgi + 32 * ks + 8 * gq;
        // anchors per channel (log2 units): b at token 15 (m0) and 47 (m1),
        // and the sum over the earlier tiles of this wave's token tile
        float b[8], mh[8], m1[8];
        if constexpr (HG) {   // equal across channels: one value per lane (the rest folds away)
            const float t0 = totb[c0], t1 = totb[DK + c0], t2 = totb[2 * DK + c0];
            const float pre = (R > 0 ? t0 : 0.f) + (R > 1 ? t1 : 0.f) + (R > 2 ? t2 : 0.f);
            const float m1v = t0 + t1 + t2, mhv = R < 2 ? t0 : m1v, bv = bs[8 * ks] + pre;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                b[e] = bv;
                m1[e] = m1v;
                mh[e] = mhv;
            }
        } else {
            float4 Tt[3][2];
#pragma unroll
            for (int x = 0; x < 3; ++x) {
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
        CKDA_FENCE();
        {   // Qh = qf e^b to the record; d = P_L e^{b_L} from token 63
            float qh[8], e0[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                e0[e] = __builtin_amdgcn_exp2f(fminf(b[e], 126.f));
                qh[e] = qf[e] * e0[e];
            }
            PR::gstore8(rec + RC::OFF_Q, RC::Q_PLANE, RC::Q_ROW, t, c0, qh);
            if (t == 63) {   // the sign of P_L: kf and k differ exactly in it (also for k = +-0)
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
        {   // row operands kf e^{b - m}, qf e^{b - m} (registers)
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
    for (int task = tid; task < DK * 8; task += NW * 64) {
        const int c = task % DK, tg = task / DK;
        const float B0 = totb[c], B1 = totb[DK + c], B2 = totb[2 * DK + c], B3 = totb[3 * DK + c];
        const float m = (tg >= 4) ? (B0 + B1 + B2) : B0;
        const uint32_t pw = totp[c / 4] ^ totp[DK / 4 + c / 4] ^ totp[DK / 2 + c / 4] ^ totp[3 * (DK / 4) + c / 4];
        const uint32_t sgn = (pw << (24 - 8 * (c & 3))) & 0x80000000u;
        const float f = __uint_as_float(
            __float_as_uint(__builtin_amdgcn_exp2f(fminf(B0 + B1 + B2 + B3 - m, 126.f))) ^ sgn);
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = f * PR::get1(colk, 8 * tg + j, c);
        PR::gstore8(rec + RC::OFF_K, RC::K_PLANE, RC::K_ROW, c, 8 * tg, x);
    }

    // ---- 3. A^T / M^T tiles (I, R), I <= R, over this wave's channels -------
    // lane (n, g) ends with row 16R + n, columns 16I + 4g .. +3 of A and M
    f32x4 accA[4], accM[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        accA[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        accM[I] = accA[I];
    }
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
        const int c0 = CG * cgi + 32 * ks + 8 * gq;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                const bool cross = (R >= 2) && (I < 2);
                const typename PR::F8 a = PR::load8(cross ? colkf : colk, 16 * I + n, c0);
                accA[I] = PR::mma8(a, rkB[ks], accA[I]);
                accM[I] = PR::mma8(a, rqB[ks], accM[I]);
            }
        }
    }
    f32x4* const part = reinterpret_cast<f32x4*>(smem + SH::L_PART);
    if (SH::NCG > 1 && cgi == 1) {
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                part[tri_index(R, I) * 64 + l] = accA[I];
                part[(10 + tri_index(R, I)) * 64 + l] = accM[I];
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
    for (int vi = 0; vi < VPW; ++vi) {
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
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) PR::store8f(rkm, t, CG * cgi + 32 * ks + 8 * gq, rkB[ks]);
    if (cgi == 0) {
        const int r = 16 * R + n;
        const float br = beta_s[r];
        if ((R & 1) == 0) {   // blocks (0,1), (2,3): read by the 32-token steps of the state pass
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            PR::gstore4(rec + RC::OFF_M, RC::M_PLANE, RC::M_ROW, r, 16 * (R + 1) + 4 * gq, zero);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I <= R) {
                f32x4 a = accA[I], m = accM[I];
                if (SH::NCG > 1) {
                    a += part[tri_index(R, I) * 64 + l];
                    m += part[(10 + tri_index(R, I)) * 64 + l];
                }
                f32x4 mv;
#pragma unroll
                for (int j = 0; j < 4; ++j) mv[j] = (I < R || 4 * gq + j <= n) ? m[j] : 0.f;
                PR::gstore4(rec + RC::OFF_M, RC::M_PLANE, RC::M_ROW, r, 16 * I + 4 * gq, mv);
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
        auto substitute = [&](const float (&rhs)[4][4], f32x4 (&X)[4]) {
            typename PR::F4 Xb[4];
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                f32x4 z;
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = beta_s[16 * J + 4 * gq + i] * rhs[J][i];
#pragma unroll
                for (int K = 0; K < J; ++K) z = PR::mma4(PR::load4(loffm, loff_index(J, K) * 64 + l, 0), Xb[K], z);
                X[J] = PR::mma4(PR::load4(ym, 16 * J + n, 4 * gq), PR::regs4(z), zero);
                Xb[J] = PR::regs4(X[J]);
            }
        };
#pragma unroll
        for (int vi = 0; vi < VPW; ++vi) {
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
#pragma unroll
                for (int J = 0; J < 4; ++J)
                    *reinterpret_cast<f32x4*>(rec + RC::OFF_U + ((J * (DV / 16) + vt) * 64 + l) * 16) = X[J];
            }
        }
        for (int ct = w; ct < DK / 16; ct += NW) {
            // kf e^b = (kf e^{b - m}) e^m, m the anchor of the token's half
            const int c = 16 * ct + n;
            const float m0 = totb[c], m1 = m0 + totb[DK + c] + totb[2 * DK + c];
            const float em0 = __builtin_amdgcn_exp2f(fminf(m0, 126.f));
            const float em1 = __builtin_amdgcn_exp2f(fminf(m1, 126.f));
            float rhs[4][4];
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) rhs[J][i] = PR::get1(rkm, 16 * J + 4 * gq + i, c) * (J < 2 ? em0 : em1);
            f32x4 X[4];
            substitute(rhs, X);
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; i += 2)
                    PR::gstore2c(rec + RC::OFF_W, RC::W_PLANE, RC::W_ROW, 16 * J + 4 * gq + i, 16 * ct + n,
                                 X[J][i], X[J][i + 1]);
        }
    }
}

template <typename Tin, int DK, int DV, bool HG, bool NQK>
static hipError_t launch_chunk_t(const FwdArgs& A, int nslots, hipStream_t stream) {
    using SH = ChunkShape<DK>;
    ChunkParams p;
    p.q = A.q; p.k = A.k; p.v = A.v; p.g = A.g; p.s = A.s; p.beta = A.beta;
    p.ws = static_cast<unsigned char*>(A.ws); p.cu = A.cu; p.T = A.T; p.H = A.H; p.ndocs = A.ndocs;
    const long long grid = static_cast<long long>(nslots) * A.H;
    if (grid == 0) return hipSuccess;
    auto kern = ckda_chunk_kernel<Tin, DK, DV, HG, NQK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(SH::NW * 64), SH::LDS, stream, p);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_chunk_dt(const FwdArgs& A, int nslots, hipStream_t stream) {
#define CKDA_CHUNK(DK_, DV_)                                                                      \
    if (A.DK == DK_ && A.DV == DV_) {                                                             \
        if (A.qk_norm)                                                                            \
            return A.head_gate ? launch_chunk_t<Tin, DK_, DV_, true, true>(A, nslots, stream)     \
                               : launch_chunk_t<Tin, DK_, DV_, false, true>(A, nslots, stream);   \
        return A.head_gate ? launch_chunk_t<Tin, DK_, DV_, true, false>(A, nslots, stream)        \
                           : launch_chunk_t<Tin, DK_, DV_, false, false>(A, nslots, stream);      \
    }
    CKDA_CHUNK(32, 32) CKDA_CHUNK(32, 64) CKDA_CHUNK(32, 128)
    CKDA_CHUNK(64, 32) CKDA_CHUNK(64, 64) CKDA_CHUNK(64, 128)
    CKDA_CHUNK(128, 32) CKDA_CHUNK(128, 64) CKDA_CHUNK(128, 128)
#undef CKDA_CHUNK
    return hipErrorInvalidValue;
}

hipError_t launch_chunk(const FwdArgs& A, int nslots, hipStream_t stream) {
    return A.bf16 ? launch_chunk_dt<bf16_t>(A, nslots, stream) : launch_chunk_dt<float>(A, nslots, stream);
}

// ---------------------------------------------------------------------------
// Standalone prep: one thread per (chunk, head, channel), serial over the
// chunk's tokens.  Same definitions as the prep inside the chunk kernel.
// ---------------------------------------------------------------------------
template <typename Tin>
__global__ void ckda_prep_kernel(int B, int T, int H, int DK, const Tin* __restrict__ q,
                                 const Tin* __restrict__ k, const float* __restrict__ g,
                                 const int8_t* __restrict__ s, float* __restrict__ b_out,
                                 int8_t* __restrict__ p_out, Tin* __restrict__ qf_out,
                                 Tin* __restrict__ kf_out)
{
    const int nt = (T + 63) / 64;
    const int c = blockIdx.y * blockDim.x + threadIdx.x;
    if (c >= DK) return;
    const int idx = blockIdx.x;            // (b * H + h) * nt + chunk
    const int chunk = idx % nt;
    const int bh = idx / nt;
    const int hh = bh % H, bb = bh / H;
    float run = 0.f;
    int sp = 1;
    const int t1 = min(T, chunk * 64 + 64);
    for (int t = chunk * 64; t < t1; ++t) {
        const size_t e = ((static_cast<size_t>(bb) * T + t) * H + hh) * DK + c;
        run += g[e];
        sp *= static_cast<int>(s[e]);
        b_out[e] = run;
        p_out[e] = static_cast<int8_t>(sp);
        const float pf = static_cast<float>(sp);
        Elem<Tin>::store(qf_out, e, pf * Elem<Tin>::load(q, e));
        Elem<Tin>::store(kf_out, e, pf * Elem<Tin>::load(k, e));
    }
}

hipError_t launch_prep(const PrepArgs& A, hipStream_t stream) {
    const int nt = (A.T + 63) / 64;
    const long long grid = static_cast<long long>(A.B) * A.H * nt;
    if (grid == 0) return hipSuccess;
    const int bs = A.DK < 128 ? A.DK : 128;
    dim3 gdim(static_cast<unsigned>(grid), (A.DK + bs - 1) / bs);
    if (A.bf16)
        hipLaunchKernelGGL(ckda_prep_kernel<bf16_t>, gdim, dim3(bs), 0, stream, A.B, A.T, A.H, A.DK,
                           static_cast<const bf16_t*>(A.q), static_cast<const bf16_t*>(A.k), A.g, A.s,
                           A.b_out, A.p_out, static_cast<bf16_t*>(A.qf_out), static_cast<bf16_t*>(A.kf_out));
    else
        hipLaunchKernelGGL(ckda_prep_kernel<float>, gdim, dim3(bs), 0, stream, A.B, A.T, A.H, A.DK,
                           static_cast<const float*>(A.q), static_cast<const float*>(A.k), A.g, A.s,
                           A.b_out, A.p_out, static_cast<float*>(A.qf_out), static_cast<float*>(A.kf_out));
    return hipGetLastError();
}

}  // namespace ckda
