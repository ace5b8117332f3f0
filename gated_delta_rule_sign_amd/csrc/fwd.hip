// fwd.hip -- chunked CKDA forward (equal-length and packed varlen) and the
// standalone gate / sign-fold prep kernel.
//
// Method: KDA-style WY/UT chunk-wise form of the recurrence (Complex KDA paper
// page, section 2 "Linear RNNs": DeltaNet/KDA admit WY-based chunk-wise
// implementations; section 1: the kernels are a small change to KDA's) with
// the signed gate carried as log-magnitude plus a sign product pushed onto q
// and k ("complex-kda-1.3B-100B" model card).  Per chunk of 64 tokens, in the
// chunk-local folded frame (sign product restarting at +1 each chunk):
//
//   b_r = sum_{i<=r} g_i,  P_r = prod_{i<=r} s_i,  qf = P q,  kf = P k
//   A_ri = sum_c kf_rc kf_ic e^{b_rc - b_ic}  (i < r),  M_ri likewise with qf_r (i <= r)
//   U = (I + Diag(beta) A)^{-1} Diag(beta) (V - (kf e^b) S)
//   O = scale ((qf e^b) S + M U)
//   S <- Diag(P_L e^{b_L}) S + Diag(P_L) (kf e^{b_L - b})^T U
//
// S is the true-frame state at the chunk start; nothing about the sign
// crosses a chunk boundary except through S itself.
//
// Work decomposition (gfx950): one 256-thread workgroup per (sequence or
// document, head, 64-wide value slice).  All four waves share the
// value-independent chunk work (prep, the A/M products, the 16x16 diagonal
// inverses of I + Diag(beta)A); wave w then owns value columns
// [16w, 16w+16) of the slice and keeps that 128x16 column block of S in
// MFMA accumulator registers for the whole sequence (value columns of S
// evolve independently).  Every product runs on bf16 MFMA with hi/lo split
// operands (see ckda_mfma.h).
//
// Exponent anchoring: e^{b_r - b_i} is factored as e^{b_r - m} e^{m - b_i}
// with m the cumulative gate at token 15 (tokens 0..31) or 47 (tokens 32..63);
// the cross-half block uses e^{b_r - m1} and e^{m1 - b_i}, both <= 1.
#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"

namespace ckda {

template <int DK, int DV>
struct FwdShape {
    static constexpr int NW = 8;                   // waves per workgroup (2 per SIMD)
    static constexpr int BV = DV < 64 ? DV : 64;   // value columns per workgroup
    static constexpr int NSLICE = DV / BV;
    static constexpr int NWC = BV / 16;            // value-column tiles of the slice
    static constexpr int NOCT = DK / 8;            // channel octets
    static constexpr int TG = (64 / NOCT) < 8 ? (64 / NOCT) : 8;   // token groups per wave (prep)
    static constexpr int TPL = 8 / TG;             // tokens per lane (8 tokens per wave)
    static constexpr int PREP_LANES = NOCT * TG;   // lanes active in the prep
    static constexpr int KS = DK / 32;             // 32-channel k-steps
    static constexpr int RT = DK / 16;             // 16-channel row tiles of the state
    static constexpr int PK = DK + 8;              // pitch of token-major operand rows
    static constexpr int PM = 64 + 4;              // pitch of M rows / channel-major rows
    static constexpr int PY = 16 + 4;              // pitch of 16x16 block rows
    // LDS carve-up (bytes; 4 bytes per staged operand element in both
    // precision policies).  Phase A (prep + A/M/S products) and phase B
    // (publish, solve, output, state update) alias the row operands.
    static constexpr int SZ_OP = 64 * PK * 4;      // one 64 x DK operand
    static constexpr int SZ_OPF = 32 * PK * 4;     // 32 x DK
    static constexpr int A_COLK = 0;               // column operands stay live into phase B
    static constexpr int A_COLKF = SZ_OP;
    static constexpr int A_ROWK = SZ_OP + SZ_OPF;
    static constexpr int A_ROWQ = A_ROWK + SZ_OP;
    static constexpr int A_END = A_ROWQ + SZ_OP;
    static constexpr int SZ_M = 64 * PM * 4;
    static constexpr int SZ_LOFF = 6 * 16 * PY * 4;
    static constexpr int SZ_Y = 4 * 16 * PY * 4;
    static constexpr int SZ_CKT = DK * PM * 4;
    static constexpr int SZ_RX = 4 * 64 * 16 * 4;  // V - K^S tiles exchanged inside wave pairs
    static constexpr int B_M = A_ROWK;
    static constexpr int B_LOFF = B_M + SZ_M;
    static constexpr int B_Y = B_LOFF + SZ_LOFF;
    static constexpr int B_CKT = B_Y + SZ_Y;
    static constexpr int B_RX = B_CKT + SZ_CKT;
    static constexpr int B_LDIAG = B_RX + SZ_RX;
    static constexpr int B_END = B_LDIAG + 4 * 16 * 17 * 4;
    static constexpr int UNION = A_END > B_END ? A_END : B_END;
    static constexpr int F_WTOT = UNION;                      // float [2][8][DK]
    static constexpr int F_CH = F_WTOT + 2 * NW * DK * 4;     // float [5][DK]
    static constexpr int F_BETA = F_CH + 5 * DK * 4;          // float [64]
    static constexpr int LDS_BYTES = F_BETA + 64 * 4;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((A_COLKF % 16) == 0 && (A_ROWK % 16) == 0 && (B_CKT % 16) == 0 && (B_RX % 16) == 0 &&
                  (B_LOFF % 16) == 0 && (B_Y % 16) == 0 && (B_LDIAG % 16) == 0 && (F_WTOT % 16) == 0,
                  "align");
};

// keep the scheduler from hoisting the next work unit's loads above this point
// (occupancy is one wave per SIMD, so unbounded hoisting only spills)
#define CKDA_FENCE() __builtin_amdgcn_sched_barrier(0)

// A zero the compiler cannot see through.  Adding it to the LDS base
// pointers at the start of every phase keeps their (loop-invariant) address
// arithmetic inside the chunk loop instead of hoisting hundreds of addresses
// into registers for the whole kernel.
__device__ __forceinline__ int opaque_zero() {
    int z = 0;
    asm volatile("" : "+s"(z));
    return z;
}
// The thread index, through the same kind of barrier to hoisting: lane-derived
// offsets are recomputed in every phase instead of living across the loop.
__device__ __forceinline__ int opaque_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for its global loads/stores still in flight (those are prefetches of
// the next chunk and output stores nobody in the workgroup reads).
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// off-diagonal 16x16 block index of (J, K), K < J
__device__ __forceinline__ int loff_index(int J, int K) { return (J * (J - 1)) / 2 + K; }

// 8 consecutive elements of a token row, kept in their storage form until use
template <typename Tin>
struct Raw8;
template <>
struct Raw8<bf16_t> {
    uint4 u;
    __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { u = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = (e < 2) ? u.x : (e < 4) ? u.y : (e < 6) ? u.z : u.w;
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <>
struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const float4*>(p)[0];
        b = reinterpret_cast<const float4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = make_float4(0.f, 0.f, 0.f, 0.f); b = a; }
    __device__ __forceinline__ float get(int e) const {
        switch (e) {
            case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
            case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
        }
    }
};

// The prep inputs of one lane for one chunk: channels 8co..8co+7 of the
// lane's TPL tokens (loaded one chunk ahead of use).
template <typename Tin, int TPL>
struct PrepIn {
    float4 g0[TPL], g1[TPL];
    uint2 s8[TPL];
    Raw8<Tin> q[TPL], k[TPL];
    float beta[TPL];
};

struct FwdParams {
    const void *q, *k, *v;
    const float* g;
    const int8_t* s;
    const float* beta;
    float scale;
    const float* h0;
    float* o;
    float* ht;
    float* h_ckpt;
    const int32_t* cu;
    int B, T, H, ndocs;
};

// A/M tiles of one chunk: x < 10 are tiles (R, I) of A, x >= 10 the same
// tiles of M, in the order (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) .. (3,3)
__device__ __forceinline__ int tile_R(int x) {
    const int y = x % 10;
    return y < 1 ? 0 : y < 3 ? 1 : y < 6 ? 2 : 3;
}
__device__ __forceinline__ int tile_I(int x) {
    const int y = x % 10;
    return y - (y < 1 ? 0 : y < 3 ? 1 : y < 6 ? 3 : 6);
}

template <typename Tin, int DK, int DV>
__global__ void __launch_bounds__(512, 1) ckda_fwd_kernel(FwdParams p)
{
    using SH = FwdShape<DK, DV>;
    // fp32 inputs run the fp32 matrix cores, bf16 inputs the split bf16 ones
    using PR = Prec<sizeof(Tin) == 4>;
    constexpr int NW = SH::NW, NOCT = SH::NOCT, TG = SH::TG, TPL = SH::TPL, KS = SH::KS, RT = SH::RT;
    constexpr int PK = SH::PK, PM = SH::PM, PY = SH::PY;
    extern __shared__ __align__(16) unsigned char smem[];

    // LDS views; CKDA_LDS_VIEWS() re-derives them from an opaque base (see opaque_zero)
#define CKDA_LDS_VIEWS()                                                                   \
    unsigned char* const sm_ = smem + opaque_zero();                                       \
    const LdsMat colk{sm_ + SH::A_COLK, PK, 64 * PK};                                      \
    const LdsMat colkf{sm_ + SH::A_COLKF, PK, 32 * PK};                                    \
    const LdsMat rowk{sm_ + SH::A_ROWK, PK, 64 * PK};                                      \
    const LdsMat rowq{sm_ + SH::A_ROWQ, PK, 64 * PK};                                      \
    const LdsMat mmat{sm_ + SH::B_M, PM, 64 * PM};                                         \
    const LdsMat loff{sm_ + SH::B_LOFF, PY, 6 * 16 * PY};                                  \
    const LdsMat ymat{sm_ + SH::B_Y, PY, 4 * 16 * PY};                                     \
    const LdsMat ckt{sm_ + SH::B_CKT, PM, DK * PM};                                        \
    float* const rx = reinterpret_cast<float*>(sm_ + SH::B_RX);      /* [4][64][16] */     \
    float* const ldiag = reinterpret_cast<float*>(sm_ + SH::B_LDIAG); /* [4][16][17] */    \
    float* const wtot_b = reinterpret_cast<float*>(sm_ + SH::F_WTOT); /* [NW][DK] */       \
    float* const wtot_p = wtot_b + NW * DK;                           /* [NW][DK] */       \
    float* const ch_em0 = reinterpret_cast<float*>(sm_ + SH::F_CH);   /* e^{m0} */         \
    float* const ch_em1 = ch_em0 + DK;                                /* e^{m1} */         \
    float* const ch_d = ch_em1 + DK;                                  /* P_L e^{b_L} */    \
    float* const ch_f0 = ch_d + DK;                         /* P_L e^{b_L - m0} */         \
    float* const ch_f1 = ch_f0 + DK;                        /* P_L e^{b_L - m1} */         \
    float* const beta_s = reinterpret_cast<float*>(sm_ + SH::F_BETA);                      \
    const int l = opaque_tid() & 63;                                                       \
    const int n = l & 15;                                                                  \
    const int gq = l >> 4;                                                                 \
    const int co = l % NOCT;                                                               \
    const int tg = l / NOCT;                                                               \
    const bool prep_lane = l < SH::PREP_LANES;                                             \
    const int col = slice * SH::BV + 16 * cw + n;                                          \
    (void)colk; (void)colkf; (void)rowk; (void)rowq; (void)mmat; (void)loff; (void)ymat;   \
    (void)ckt; (void)rx; (void)ldiag; (void)wtot_b; (void)wtot_p; (void)ch_em0;            \
    (void)ch_em1; (void)ch_d; (void)ch_f0; (void)ch_f1; (void)beta_s; (void)l; (void)n;    \
    (void)gq; (void)co; (void)tg; (void)prep_lane; (void)col

    const Tin* __restrict__ q = static_cast<const Tin*>(p.q);
    const Tin* __restrict__ k = static_cast<const Tin*>(p.k);
    const Tin* __restrict__ v = static_cast<const Tin*>(p.v);
    const int H = p.H;

    // ---- which (chain, value slice) this workgroup owns -------------------
    const int nchains = p.cu ? p.ndocs * H : p.B * H;
    int chain, slice;
    {
        const int bid = blockIdx.x;
        if (SH::NSLICE == 1) {
            chain = bid;
            slice = 0;
        } else {
            // the slices of one chain land on the same XCD (blocks are dealt
            // round-robin over 8 XCDs), so its shared inputs hit one L2
            const int grp = 8 * SH::NSLICE;
            const int full = (nchains / 8) * grp;
            if (bid < full) {
                const int r = bid % grp;
                chain = (bid / grp) * 8 + (r % 8);
                slice = r / 8;
            } else {
                const int r = bid - full;
                chain = (nchains / 8) * 8 + r / SH::NSLICE;
                slice = r % SH::NSLICE;
            }
        }
    }
    const int h = chain % H;
    int tok0, len, sidx;
    if (p.cu) {
        sidx = chain / H;
        tok0 = p.cu[sidx];
        len = p.cu[sidx + 1] - tok0;
    } else {
        tok0 = (chain / H) * p.T; len = p.T; sidx = chain / H;
    }
    const size_t st_off = (static_cast<size_t>(sidx) * H + h) * DK * DV;

    // wave roles (wave-uniform); lane roles are re-derived per phase
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int cw = w & 3;             // state phase: value-column tile ...
    const int hh = w >> 2;            // ... and token half (0: tokens 0..31)
    const bool has_col = cw < SH::NWC;

    // ---- state: 16-column block, C layout (rows 16rt + 4gq + i); the two
    // waves of a pair (w, w+4) hold identical copies ----------------------
    f32x4 S[RT];
    {
        const int gq = (threadIdx.x & 63) >> 4;
        const int col = slice * SH::BV + 16 * cw + (threadIdx.x & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[rt][i] = (has_col && p.h0) ? p.h0[st_off + static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] : 0.f;
    }

    const int nchunks = (len + 63) / 64;

    // ---- global loads, issued one chunk ahead of their use ----------------
    auto load_prep = [&](PrepIn<Tin, TPL>& in, int cc0, int LL) {
        const int l = opaque_tid() & 63;
        const int co = l % NOCT, tg = l / NOCT;
        const bool prep_lane = l < SH::PREP_LANES;
#pragma unroll
        for (int tt = 0; tt < TPL; ++tt) {
            const int t = 8 * w + tg * TPL + tt;
            if (prep_lane && t < LL) {
                const size_t row = static_cast<size_t>(tok0 + cc0 + t) * H + h;
                const size_t base = row * DK + 8 * co;
                in.g0[tt] = reinterpret_cast<const float4*>(p.g + base)[0];
                in.g1[tt] = reinterpret_cast<const float4*>(p.g + base)[1];
                in.s8[tt] = *reinterpret_cast<const uint2*>(p.s + base);
                in.q[tt].load(q + base);
                in.k[tt].load(k + base);
                in.beta[tt] = (co == 0) ? p.beta[row] : 0.f;
            } else {   // padding token: g = 0, s = +1, q = k = 0, beta = 0
                in.g0[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
                in.g1[tt] = in.g0[tt];
                in.s8[tt] = make_uint2(0x01010101u, 0x01010101u);
                in.q[tt].zero();
                in.k[tt].zero();
                in.beta[tt] = 0.f;
            }
        }
    };
    auto load_v = [&](float (&vv)[2][4], int cc0, int LL) {
        const int l = opaque_tid() & 63;
        const int gq = l >> 4;
        const int col = slice * SH::BV + 16 * cw + (l & 15);
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * (2 * hh + r2) + 4 * gq + i;
                vv[r2][i] = (has_col && t < LL)
                                ? Elem<Tin>::load(v, (static_cast<size_t>(tok0 + cc0 + t) * H + h) * DV + col)
                                : 0.f;
            }
    };
    PrepIn<Tin, TPL> pin;
    float vin[2][4];
    if (nchunks > 0) {
        load_prep(pin, 0, min(64, len));
        load_v(vin, 0, min(64, len));
    }

    for (int j = 0; j < nchunks; ++j) {
        const int c0 = j * 64;
        const int L = min(64, len - c0);
        const int Ln = min(64, len - c0 - 64);   // next chunk (<= 0: none)
        if (p.h_ckpt && has_col && hh == 0) {
            const int l = opaque_tid() & 63;
            const int gq = l >> 4;
            const int col = slice * SH::BV + 16 * cw + (l & 15);
            float* hc = p.h_ckpt + opaque_zero() +
                        (static_cast<size_t>(sidx) * H + h) * static_cast<size_t>(nchunks) * DK * DV +
                        static_cast<size_t>(j) * DK * DV;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) hc[static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] = S[rt][i];
        }

        // ================= P1: gate / sign-fold prep ========================
        // lane: channels 8co..8co+7 of tokens 8w + tg*TPL + tt (tt < TPL)
        {
        CKDA_LDS_VIEWS();
        float bl[TPL][8];
        uint32_t negmask = 0;         // bit 8*tt+e: running sign product is -1
        float run[8];
        uint32_t par = 0;             // bit e: parity of negative signs so far
#pragma unroll
        for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
        for (int tt = 0; tt < TPL; ++tt) {
            const int t = 8 * w + tg * TPL + tt;
            const float4 g0 = pin.g0[tt], g1 = pin.g1[tt];
            const uint2 s8 = pin.s8[tt];
            run[0] += g0.x; run[1] += g0.y; run[2] += g0.z; run[3] += g0.w;
            run[4] += g1.x; run[5] += g1.y; run[6] += g1.z; run[7] += g1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t byte = ((e < 4 ? s8.x : s8.y) >> (8 * (e & 3))) & 0xffu;
                par ^= (byte >> 7) << e;      // s = -1 has its sign bit set
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) bl[tt][e] = run[e];
            negmask |= par << (8 * tt);
            if (prep_lane && co == 0) beta_s[t] = pin.beta[tt];
        }
        // inclusive scan of the per-lane totals across the token groups of the wave
        float inc[8];
        uint32_t pinc = par;
#pragma unroll
        for (int e = 0; e < 8; ++e) inc[e] = run[e];
#pragma unroll
        for (int d = 1; d < TG; d *= 2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ob = __shfl_up(inc[e], d * NOCT, 64);
                if (tg >= d) inc[e] += ob;
            }
            const uint32_t op = static_cast<uint32_t>(__shfl_up(static_cast<int>(pinc), d * NOCT, 64));
            if (tg >= d) pinc ^= op;
        }
        if (prep_lane && tg == TG - 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                wtot_b[w * DK + 8 * co + e] = inc[e];
                wtot_p[w * DK + 8 * co + e] = ((pinc >> e) & 1u) ? -1.f : 1.f;
            }
        }
        lds_sync();
        float m0[8], m1[8], mh[8], bpre[8];
        uint32_t ppre = pinc ^ par;   // parity of the tokens before this lane's, inside the wave
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * co + e;
            float Bw[NW], Qw[NW];
#pragma unroll
            for (int x = 0; x < NW; ++x) { Bw[x] = wtot_b[x * DK + c]; Qw[x] = wtot_p[x * DK + c]; }
            m0[e] = Bw[0] + Bw[1];                    // b at token 15
            const float a = m0[e] + Bw[2] + Bw[3];    // b at token 31
            m1[e] = a + Bw[4] + Bw[5];                // b at token 47
            const float bL = m1[e] + Bw[6] + Bw[7];   // b at token 63
            float PL = 1.f, bp = 0.f, pp = 1.f;
#pragma unroll
            for (int x = 0; x < NW; ++x) {
                PL *= Qw[x];
                if (x < w) { bp += Bw[x]; pp *= Qw[x]; }
            }
            bpre[e] = bp + (inc[e] - run[e]);
            if (pp < 0.f) ppre ^= 1u << e;
            mh[e] = (w >= 4) ? m1[e] : m0[e];
            if (prep_lane && w == 0 && tg == 0) {
                ch_em0[c] = exp2_clamped(m0[e] * kLog2e);
                ch_em1[c] = exp2_clamped(m1[e] * kLog2e);
                ch_d[c] = PL * exp2_clamped(bL * kLog2e);
                ch_f0[c] = PL * exp2_clamped((bL - m0[e]) * kLog2e);
                ch_f1[c] = PL * exp2_clamped((bL - m1[e]) * kLog2e);
            }
            CKDA_FENCE();
        }
        if (prep_lane) {
#pragma unroll
            for (int tt = 0; tt < TPL; ++tt) {
                const int t = 8 * w + tg * TPL + tt;
                float rk[8], rq[8], ck[8];
                const uint32_t neg = ppre ^ ((negmask >> (8 * tt)) & 0xffu);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float b = bpre[e] + bl[tt][e];
                    const float P = ((neg >> e) & 1u) ? -1.f : 1.f;
                    const float e1 = exp2_clamped((b - mh[e]) * kLog2e);
                    const float e2 = exp2_clamped((mh[e] - b) * kLog2e);
                    const float kf = P * pin.k[tt].get(e);
                    rk[e] = kf * e1;
                    rq[e] = (P * pin.q[tt].get(e)) * e1;
                    ck[e] = kf * e2;
                }
                PR::store8(rowk, t, 8 * co, rk);
                PR::store8(rowq, t, 8 * co, rq);
                PR::store8(colk, t, 8 * co, ck);
                if (w < 4) {
                    float cf[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) cf[e] = ck[e] * exp2_clamped((m1[e] - m0[e]) * kLog2e);
                    PR::store8(colkf, t, 8 * co, cf);
                }
            }
        }
        if (Ln > 0) load_prep(pin, c0 + 64, Ln);
        lds_sync();
        }

        // ================= P2: A / M tiles and the S products ===============
        // wave w computes A^T / M^T tiles w, w+8, w+16 (of 20), and, for its
        // value-column tile cw, K^S and Q^S on the token tiles of half hh
        const int ntl = (w + 16 < 20) ? 3 : 2;
        f32x4 tacc[3];
        f32x4 Rt[2], OQ[2];            // V - K^S and Q^S for this wave's tokens and columns
        {
        CKDA_LDS_VIEWS();
#pragma unroll
        for (int x3 = 0; x3 < 3; ++x3) tacc[x3] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int ko = 32 * ks + 8 * gq;
#pragma unroll
            for (int x3 = 0; x3 < 3; ++x3) {
                if (x3 < ntl) {
                    const int x = w + 8 * x3;
                    const int R = tile_R(x), I = tile_I(x);
                    const bool cross = (R >= 2) && (I < 2);
                    const LdsMat& cm = cross ? colkf : colk;
                    const LdsMat& rm = (x < 10) ? rowk : rowq;
                    tacc[x3] = PR::mma8(PR::load8(cm, 16 * I + n, ko), PR::load8(rm, 16 * R + n, ko), tacc[x3]);
                }
            }
        }
        if (has_col) {
            // S' = Diag(e^{m_hh}) S as split B operands (only this half's anchor)
            const float* em = hh ? ch_em1 : ch_em0;
            f32x4 ak[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            f32x4 aq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                f32x4 a, b;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[i] = em[32 * ks + 4 * gq + i] * S[2 * ks][i];
                    b[i] = em[32 * ks + 16 + 4 * gq + i] * S[2 * ks + 1][i];
                }
                const typename PR::F8 Bs = PR::regs8(a, b);
                const int ka = 32 * ks + 4 * gq, kb = 32 * ks + 16 + 4 * gq;
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    const int r = 16 * (2 * hh + r2) + n;
                    ak[r2] = PR::mma8(PR::load4x2(rowk, r, ka, kb), Bs, ak[r2]);
                    aq[r2] = PR::mma8(PR::load4x2(rowq, r, ka, kb), Bs, aq[r2]);
                }
            }
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) Rt[r2][i] = vin[r2][i] - ak[r2][i];
                OQ[r2] = aq[r2];
            }
        }
        if (Ln > 0) load_v(vin, c0 + 64, Ln);
        lds_sync();
        }

        // ================= P2.5: publish -beta*A blocks, M, kf^T, R ========
        {
        CKDA_LDS_VIEWS();
#pragma unroll
        for (int x3 = 0; x3 < 3; ++x3) {
            if (x3 < ntl) {
                const int x = w + 8 * x3;
                const int R = tile_R(x), I = tile_I(x);
                const int r = 16 * R + n;
                const f32x4 val = tacc[x3];
                if (x < 10) {
                    const float br = beta_s[r];
                    if (R == I) {
                        float* dst = ldiag + (R * 16 + n) * 17 + 4 * gq;
#pragma unroll
                        for (int i = 0; i < 4; ++i) dst[i] = (4 * gq + i < n) ? br * val[i] : 0.f;
                    } else {
                        f32x4 nv;
#pragma unroll
                        for (int i = 0; i < 4; ++i) nv[i] = -br * val[i];
                        PR::store4(loff, loff_index(R, I) * 16 + n, 4 * gq, nv);
                    }
                } else {
                    f32x4 mv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) mv[i] = (R > I || 4 * gq + i <= n) ? val[i] : 0.f;
                    PR::store4(mmat, r, 16 * I + 4 * gq, mv);
                }
            }
        }
        // M . U reads the upper blocks (0,1) and (2,3) of M as part of its
        // 32-token k-steps: they must hold zeros (waves 6, 7 carry 2 tiles)
        if (w >= 6) {
            const int R = (w == 6) ? 0 : 2;
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            PR::store4(mmat, 16 * R + n, 16 * (R + 1) + 4 * gq, zero);
        }
        // transposed copy of the column operand (phase B leaves colk intact)
        if (prep_lane) {
#pragma unroll
            for (int tt = 0; tt < TPL; ++tt) {
                const int t = 8 * w + tg * TPL + tt;
#pragma unroll
                for (int e = 0; e < 8; ++e) PR::copy1(ckt, 8 * co + e, t, colk, t, 8 * co + e);
            }
        }
        // this wave's V - K^S tiles, for its partner wave
        if (has_col) {
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                for (int i = 0; i < 4; ++i) rx[(cw * 64 + 16 * (2 * hh + r2) + 4 * gq + i) * 16 + n] = Rt[r2][i];
        }
        lds_sync();
        }

        // ================= P3: inverses of the 16x16 diagonal blocks ========
        {
        CKDA_LDS_VIEWS();
        if (w < 4 && l < 16) {
            const int J = w;
            const int c = l;
            float y[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc -= ldiag[(J * 16 + r) * 17 + i] * y[i];
                y[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) PR::store1(ymat, J * 16 + r, c, y[r]);
        }
        lds_sync();
        }

        // ================= P4: U, O, state update ==========================
        {
        CKDA_LDS_VIEWS();
        if (has_col) {
            f32x4 Ra[4];
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int i = 0; i < 4; ++i) Ra[J][i] = rx[(cw * 64 + 16 * J + 4 * gq + i) * 16 + n];
            f32x4 U[4];
            typename PR::F4 Us[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                f32x4 z;
#pragma unroll
                for (int i = 0; i < 4; ++i) z[i] = beta_s[16 * J + 4 * gq + i] * Ra[J][i];
#pragma unroll
                for (int K = 0; K < J; ++K)
                    z = PR::mma4(PR::load4(loff, loff_index(J, K) * 16 + n, 4 * gq), Us[K], z);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                U[J] = PR::mma4(PR::load4(ymat, J * 16 + n, 4 * gq), PR::regs4(z), zero);
                Us[J] = PR::regs4(U[J]);
            }
            const typename PR::F8 U01 = PR::regs8(U[0], U[1]);
            const typename PR::F8 U23 = PR::regs8(U[2], U[3]);
            // O = Q^S + M U on this wave's token tiles
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int R = 2 * hh + r2;
                const int r = 16 * R + n;
                f32x4 acc = PR::mma8(PR::load4x2(mmat, r, 4 * gq, 16 + 4 * gq), U01, OQ[r2]);
                if (R >= 2) acc = PR::mma8(PR::load4x2(mmat, r, 32 + 4 * gq, 48 + 4 * gq), U23, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * R + 4 * gq + i;
                    if (t < L) p.o[(static_cast<size_t>(tok0 + c0 + t) * H + h) * DV + col] = p.scale * acc[i];
                }
            }
            // S <- Diag(d) S + Diag(f0) kf[0:32]^T U[0:32] + Diag(f1) kf[32:64]^T U[32:64]
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int c = 16 * rt + n;
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f32x4 acc0 = PR::mma8(PR::load4x2(ckt, c, 4 * gq, 16 + 4 * gq), U01, zero);
                const f32x4 acc1 = PR::mma8(PR::load4x2(ckt, c, 32 + 4 * gq, 48 + 4 * gq), U23, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cc = 16 * rt + 4 * gq + i;
                    S[rt][i] = ch_d[cc] * S[rt][i] + ch_f0[cc] * acc0[i] + ch_f1[cc] * acc1[i];
                }
            }
        }
        lds_sync();
        }
    }

    if (p.ht && has_col && hh == 0) {
        const int gq = (threadIdx.x & 63) >> 4;
        const int col = slice * SH::BV + 16 * cw + (threadIdx.x & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.ht[st_off + opaque_zero() + static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] = S[rt][i];
    }
#undef CKDA_LDS_VIEWS
}

template <typename Tin, int DK, int DV>
static hipError_t launch_fwd_t(const FwdArgs& A, hipStream_t stream) {
    using SH = FwdShape<DK, DV>;
    FwdParams p;
    p.q = A.q; p.k = A.k; p.v = A.v; p.g = A.g; p.s = A.s; p.beta = A.beta; p.scale = A.scale;
    p.h0 = A.h0; p.o = A.o; p.ht = A.ht; p.h_ckpt = A.h_ckpt; p.cu = A.cu;
    p.B = A.B; p.T = A.T; p.H = A.H; p.ndocs = A.ndocs;
    const int nchains = A.cu ? A.ndocs * A.H : A.B * A.H;
    const int grid = nchains * SH::NSLICE;
    if (grid == 0) return hipSuccess;
    auto kern = ckda_fwd_kernel<Tin, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::LDS_BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(SH::NW * 64), SH::LDS_BYTES, stream, p);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_fwd_dt(const FwdArgs& A, hipStream_t stream) {
#define CKDA_FWD(DK_, DV_) \
    if (A.DK == DK_ && A.DV == DV_) return launch_fwd_t<Tin, DK_, DV_>(A, stream);
    CKDA_FWD(32, 32) CKDA_FWD(32, 64) CKDA_FWD(32, 128)
    CKDA_FWD(64, 32) CKDA_FWD(64, 64) CKDA_FWD(64, 128)
    CKDA_FWD(128, 32) CKDA_FWD(128, 64) CKDA_FWD(128, 128)
#undef CKDA_FWD
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& A, hipStream_t stream) {
    return A.bf16 ? launch_fwd_dt<bf16_t>(A, stream) : launch_fwd_dt<float>(A, stream);
}

// ---------------------------------------------------------------------------
// Standalone prep: one thread per (chunk, head, channel), serial over the
// chunk's tokens.  Same definitions as the fused prep above.
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
