// state.hip -- state-passing kernel of the chunked CKDA forward.
//
// Consumes the per-(chunk, head) records of the chunk-local kernel
// (ckda_record.h) in chunk order and carries the state S (DK x DV, float32,
// true signed frame) across chunks:
//
//   U = u - W S,   O = scale (Qh S + M U),   S <- Diag(d) S + KbT U
//
// (the WY/UT chunk form of the recurrence; Complex KDA paper page, section 2
// "Linear RNNs").  Only these products depend on the state, so this is the
// sequential part of the forward; everything else ran in parallel before.
//
// Work decomposition (gfx950): one 256-thread workgroup per (sequence or
// document, head, 64-wide value slice); wave w owns value columns
// [16w, 16w+16) of the slice and keeps that DK x 16 block of S in MFMA
// accumulator registers for the whole sequence (value columns of S evolve
// independently, so the waves never exchange state).  Each chunk's record
// (W, Qh, KbT, M, d) is read from HBM once per workgroup into registers one
// chunk ahead, then staged in LDS and shared by the four waves; u is read by
// each wave straight into its C-layout registers.  All products are 16x16x16
// matrix-core tiles: the C/D layout of S and U doubles as the B operand.
#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"
#include "ckda_record.h"
#include "ckda_sync.h"

namespace ckda {

template <typename Tin, int DK, int DV>
struct StateShape {
    static constexpr bool F32 = sizeof(Tin) == 4;
    using RC = Record<DK, DV, F32>;
    static constexpr int NT = 256;                 // threads
    static constexpr int BV = DV < 64 ? DV : 64;   // value columns per workgroup
    static constexpr int NSLICE = DV / BV;
    static constexpr int NWC = BV / 16;            // waves that own columns
    static constexpr int RT = DK / 16;             // 16-row tiles of S
    static constexpr int ES = RC::ES, NP = RC::NP;
    // LDS rows carry 16 bytes of padding (row pitch = 4 banks mod 64)
    static constexpr int PW = (RC::W_ROW + 16) / ES;   // pitches in elements
    static constexpr int PQ = (RC::Q_ROW + 16) / ES;
    static constexpr int PKR = (RC::K_ROW + 16) / ES;
    static constexpr int PMR = (RC::M_ROW + 16) / ES;
    static constexpr int L_W = 0;
    static constexpr int L_Q = L_W + 64 * PW * ES;
    static constexpr int L_K = L_Q + NP * 64 * PQ * ES;
    static constexpr int L_M = L_K + NP * DK * PKR * ES;
    static constexpr int L_D = L_M + NP * 64 * PMR * ES;
    static constexpr int LDS = L_D + DK * 4;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// A block of ROWS rows of UPR 16-byte units, copied from the record into
// LDS rows of UPR units plus PAD bytes through registers: thread t moves
// units t, t + NT, ...
template <int ROWS, int UPR, int PAD, int NT>
struct Stage {
    static constexpr int UNITS = ROWS * UPR;
    static constexpr int N = (UNITS + NT - 1) / NT;
    static constexpr bool FULL = (UNITS % NT) == 0;
    static __device__ __forceinline__ bool has(int tid, int i) { return FULL || tid + NT * i < UNITS; }
    static __device__ __forceinline__ int lds_off(int tid, int i) {
        const int u = tid + NT * i;
        return (u / UPR) * (UPR * 16 + PAD) + (u % UPR) * 16;
    }
};

struct StateParams {
    const unsigned char* ws;
    const float* h0;
    float* o;
    float* ht;
    float* h_ckpt;
    const int32_t* cu;   // varlen document starts (device), or nullptr
    float scale;
    int B, T, H, ndocs;
};

template <typename Tin, int DK, int DV>
__global__ void __launch_bounds__(256, 1) ckda_state_kernel(StateParams p)
{
    using SH = StateShape<Tin, DK, DV>;
    using RC = typename SH::RC;
    using PR = Prec<SH::F32>;
    constexpr int RT = SH::RT, NP = SH::NP, NT = SH::NT;
    extern __shared__ __align__(16) unsigned char smem[];

    const int H = p.H;
    const int nchains = p.cu ? p.ndocs * H : p.B * H;
    int chain, slice;
    {
        const int bid = blockIdx.x;
        if (SH::NSLICE == 1) {
            chain = bid;
            slice = 0;
        } else {
            // the slices of one chain land on the same XCD (workgroups are
            // dealt round-robin over 8 XCDs), so the record is read from HBM
            // once and the other slices hit that XCD's L2
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
    const int sidx = chain / H;
    int tok0, len, slot0;
    if (p.cu) {
        tok0 = p.cu[sidx];
        len = p.cu[sidx + 1] - tok0;
        slot0 = varlen_slot(tok0, sidx, 0);
    } else {
        tok0 = sidx * p.T;
        len = p.T;
        slot0 = sidx * ((p.T + 63) / 64);
    }
    const int nchunks = (len + 63) / 64;
    const size_t st_off = (static_cast<size_t>(sidx) * H + h) * DK * DV;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool has_col = w < SH::NWC;
    const int vt = (slice * SH::BV) / 16 + w;   // the wave's 16-column tile of DV

    // ---- state: lane (n, g) holds rows 16rt + 4g + i of column 16vt + n ----
    f32x4 S[RT];
    {
        const int l = tid & 63, gq = l >> 4, col = 16 * vt + (l & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[rt][i] = (has_col && p.h0) ? p.h0[st_off + static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] : 0.f;
    }

    // one chunk's record, staged through registers: W, Qh, KbT, M, d are
    // consecutive in the record and in LDS (with padded rows)
    using StW = Stage<64, RC::W_ROW / 16, 16, NT>;
    using StQ = Stage<NP * 64, RC::Q_ROW / 16, 16, NT>;
    using StK = Stage<NP * DK, RC::K_ROW / 16, 16, NT>;
    using StM = Stage<NP * 64, RC::M_ROW / 16, 16, NT>;
    using StD = Stage<1, DK * 4 / 16, 0, NT>;
    constexpr int NW_ = StW::N, NQ_ = StQ::N, NK_ = StK::N, NM_ = StM::N, ND_ = StD::N;
    constexpr int NREG = NW_ + NQ_ + NK_ + NM_ + ND_;
    static_assert(StW::FULL && StQ::FULL && StK::FULL && StM::FULL, "unguarded staging loads");
    u32x4 stg[NREG];   // native vectors (a struct copy would keep them in scratch)
    f32x4 uin[4];
    // issue the global loads of chunk J's record (registers, one chunk ahead)
#define CKDA_LOAD_CHUNK(J)                                                                         \
    {                                                                                              \
        const unsigned char* rc_ =                                                                 \
            p.ws + (static_cast<size_t>(slot0 + (J)) * H + h) * RC::BYTES + opaque_zero();         \
        const int t_ = opaque_tid();                                                               \
        const u32x4* g_ = reinterpret_cast<const u32x4*>(rc_);                                     \
        _Pragma("unroll") for (int i_ = 0; i_ < NW_; ++i_) stg[i_] = g_[RC::OFF_W / 16 + t_ + NT * i_]; \
        _Pragma("unroll") for (int i_ = 0; i_ < NQ_; ++i_) stg[NW_ + i_] = g_[RC::OFF_Q / 16 + t_ + NT * i_]; \
        _Pragma("unroll") for (int i_ = 0; i_ < NK_; ++i_) stg[NW_ + NQ_ + i_] = g_[RC::OFF_K / 16 + t_ + NT * i_]; \
        _Pragma("unroll") for (int i_ = 0; i_ < NM_; ++i_) stg[NW_ + NQ_ + NK_ + i_] = g_[RC::OFF_M / 16 + t_ + NT * i_]; \
        _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                         \
            if (StD::has(t_, i_)) stg[NW_ + NQ_ + NK_ + NM_ + i_] = g_[RC::OFF_D / 16 + t_ + NT * i_]; \
        if (has_col) {                                                                             \
            const int l_ = t_ & 63;                                                                \
            _Pragma("unroll") for (int J_ = 0; J_ < 4; ++J_) uin[J_] =                             \
                *reinterpret_cast<const f32x4*>(rc_ + RC::OFF_U + ((J_ * (DV / 16) + vt) * 64 + l_) * 16); \
        }                                                                                          \
    }
    if (nchunks > 0) CKDA_LOAD_CHUNK(0)

    for (int j = 0; j < nchunks; ++j) {
        const int c0 = 64 * j;
        const int L = min(64, len - c0);
        {
            unsigned char* const sm = smem + opaque_zero();
            const int t = opaque_tid();
#pragma unroll
            for (int i = 0; i < NW_; ++i) *reinterpret_cast<u32x4*>(sm + SH::L_W + StW::lds_off(t, i)) = stg[i];
#pragma unroll
            for (int i = 0; i < NQ_; ++i) *reinterpret_cast<u32x4*>(sm + SH::L_Q + StQ::lds_off(t, i)) = stg[NW_ + i];
#pragma unroll
            for (int i = 0; i < NK_; ++i)
                *reinterpret_cast<u32x4*>(sm + SH::L_K + StK::lds_off(t, i)) = stg[NW_ + NQ_ + i];
#pragma unroll
            for (int i = 0; i < NM_; ++i)
                *reinterpret_cast<u32x4*>(sm + SH::L_M + StM::lds_off(t, i)) = stg[NW_ + NQ_ + NK_ + i];
#pragma unroll
            for (int i = 0; i < ND_; ++i)
                if (StD::has(t, i))
                    *reinterpret_cast<u32x4*>(sm + SH::L_D + StD::lds_off(t, i)) = stg[NW_ + NQ_ + NK_ + NM_ + i];
        }
        f32x4 u[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) u[J] = uin[J];
        lds_sync();
        if (j + 1 < nchunks) CKDA_LOAD_CHUNK(j + 1)

        if (has_col) {
            unsigned char* const sm = smem + opaque_zero();
            const LdsMat Wm{sm + SH::L_W, SH::PW, 0};
            const LdsMat Qm{sm + SH::L_Q, SH::PQ, 64 * SH::PQ};
            const LdsMat Km{sm + SH::L_K, SH::PKR, DK * SH::PKR};
            const LdsMat Mm{sm + SH::L_M, SH::PMR, 64 * SH::PMR};
            const float* dl = reinterpret_cast<const float*>(sm + SH::L_D);
            const int l = opaque_tid() & 63, n = l & 15, gq = l >> 4;
            const int col = 16 * vt + n;
            if (p.h_ckpt) {
                float* hc = p.h_ckpt + (static_cast<size_t>(sidx) * H + h) * static_cast<size_t>(nchunks) * DK * DV +
                            static_cast<size_t>(j) * DK * DV;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) hc[static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] = S[rt][i];
            }
            // W S and Qh S
            typename PR::F4 Sb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) Sb[rt] = PR::regs4(S[rt]);
            f32x4 X[4], Y[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                X[R] = f32x4{0.f, 0.f, 0.f, 0.f};
                Y[R] = X[R];
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    X[R] = PR::mma4s(PR::load4s(Wm, 16 * R + n, 16 * rt + 4 * gq), Sb[rt], X[R]);
                    Y[R] = PR::mma4(PR::load4(Qm, 16 * R + n, 16 * rt + 4 * gq), Sb[rt], Y[R]);
                }
            // U = u - W S
            typename PR::F4 Ub[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) Ub[R] = PR::regs4(u[R] - X[R]);
            // O = scale (Qh S + M U)
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 acc = Y[R];
#pragma unroll
                for (int K = 0; K <= R; ++K) acc = PR::mma4(PR::load4(Mm, 16 * R + n, 16 * K + 4 * gq), Ub[K], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = 16 * R + 4 * gq + i;
                    if (tt < L) p.o[(static_cast<size_t>(tok0 + c0 + tt) * H + h) * DV + col] = p.scale * acc[i];
                }
            }
            // S <- Diag(d) S + KbT U
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = 0; K < 4; ++K) acc = PR::mma4(PR::load4(Km, 16 * rt + n, 16 * K + 4 * gq), Ub[K], acc);
                const f32x4 dd = *reinterpret_cast<const f32x4*>(dl + 16 * rt + 4 * gq);
                S[rt] = dd * S[rt] + acc;
            }
        }
        lds_sync();
    }

    if (p.ht && has_col) {
        const int l = tid & 63, gq = l >> 4, col = 16 * vt + (l & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p.ht[st_off + opaque_zero() + static_cast<size_t>(16 * rt + 4 * gq + i) * DV + col] = S[rt][i];
    }
#undef CKDA_LOAD_CHUNK
}

template <typename Tin, int DK, int DV>
static hipError_t launch_state_t(const FwdArgs& A, hipStream_t stream) {
    using SH = StateShape<Tin, DK, DV>;
    StateParams p;
    p.ws = static_cast<const unsigned char*>(A.ws);
    p.h0 = A.h0; p.o = A.o; p.ht = A.ht; p.h_ckpt = A.h_ckpt; p.cu = A.cu; p.scale = A.scale;
    p.B = A.B; p.T = A.T; p.H = A.H; p.ndocs = A.ndocs;
    const int nchains = A.cu ? A.ndocs * A.H : A.B * A.H;
    const int grid = nchains * SH::NSLICE;
    if (grid == 0) return hipSuccess;
    auto kern = ckda_state_kernel<Tin, DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(SH::NT), SH::LDS, stream, p);
    return hipGetLastError();
}

template <typename Tin>
static hipError_t launch_state_dt(const FwdArgs& A, hipStream_t stream) {
#define CKDA_STATE(DK_, DV_) \
    if (A.DK == DK_ && A.DV == DV_) return launch_state_t<Tin, DK_, DV_>(A, stream);
    CKDA_STATE(32, 32) CKDA_STATE(32, 64) CKDA_STATE(32, 128)
    CKDA_STATE(64, 32) CKDA_STATE(64, 64) CKDA_STATE(64, 128)
    CKDA_STATE(128, 32) CKDA_STATE(128, 64) CKDA_STATE(128, 128)
#undef CKDA_STATE
    return hipErrorInvalidValue;
}

hipError_t launch_state(const FwdArgs& A, hipStream_t stream) {
    return A.bf16 ? launch_state_dt<bf16_t>(A, stream) : launch_state_dt<float>(A, stream);
}

// forward = chunk-local kernel over every (chunk, head), then the state pass
size_t fwd_workspace_bytes(int nslots, int H, int DK, int DV, bool bf16) {
    size_t rec = 0;
#define CKDA_REC(DK_, DV_) \
    if (DK == DK_ && DV == DV_) rec = bf16 ? Record<DK_, DV_, false>::BYTES : Record<DK_, DV_, true>::BYTES;
    CKDA_REC(32, 32) CKDA_REC(32, 64) CKDA_REC(32, 128)
    CKDA_REC(64, 32) CKDA_REC(64, 64) CKDA_REC(64, 128)
    CKDA_REC(128, 32) CKDA_REC(128, 64) CKDA_REC(128, 128)
#undef CKDA_REC
    return static_cast<size_t>(nslots) * H * rec;
}

hipError_t launch_fwd(const FwdArgs& A, int nslots, hipStream_t stream) {
    hipError_t e = launch_chunk(A, nslots, stream);
    if (e != hipSuccess) return e;
    return launch_state(A, stream);
}

}  // namespace ckda
