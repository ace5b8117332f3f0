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
// independently, so the waves never exchange state).  Four more waves only
// move data: they hold the next chunk's record (W, Qh, KbT, M and d) in
// registers, read one chunk ahead from HBM, and write it to LDS in two groups
// while the matrix-core waves work on the other group.  The u tiles, which
// only their own wave reads, go from the record straight into that wave's
// registers, one chunk ahead.  A wave that issues global loads stalls
// whenever the memory pipe is full; keeping those loads on separate waves
// lets the matrix-core waves run while the next record streams in.  Products are 16x16x32
// matrix-core tiles whose 8 K-slots per lane are two 4-row groups of the C/D
// layout (rows 4g..4g+3 of tiles 2k and 2k+1), so S and U feed the B side
// straight from their accumulator layout; the A side reads the matching
// elements (columns 32k + 4g .. +3 and 32k + 16 + 4g .. +3).
//
// Segment mode (chains much longer than the GPU has parallel work for):
// the chunk maps are affine in the state, S' = A_c S + B_c with
// A_c = Diag(d) - KbT W, and every column of S evolves on its own.  A chain
// of chunks is cut into segments of G chunks.  Phase 1 (no outputs, so no
// Qh S or M U products and no Qh / M staging) walks every segment but a
// chain's last: the first from the chain's start (its end state is
// start_1), each middle one with its value columns from zero (giving H_s,
// the segment's end state from zero) and DK "transition" columns from the
// identity with u = 0 (giving P_s, the product of the segment's A_c).
// Phase 2 (ckda_seg_scan_kernel) chains the starts:
// start_{s+1} = P_s start_s + H_s.  Phase 3 walks every segment from its
// true start and writes the outputs, checkpoints and final state.
#include <algorithm>
#include <atomic>
#include <vector>

#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"
#include "ckda_record.h"
#include "ckda_segments.h"
#include "ckda_sync.h"

namespace ckda {

template <typename Tin, int DK, int DV>
struct StateShape {
    static constexpr bool F32 = sizeof(Tin) == 4;
    using RC = Record<DK, DV, F32>;
    static constexpr int NT = 256;                 // threads per role (4 compute + 4 loader waves)
    static constexpr int BV = DV < 64 ? DV : 64;   // value columns per workgroup
    static constexpr int NSLICE = DV / BV;
    static constexpr int NTS = (DK + BV - 1) / BV;   // transition slices over the DK columns of P_s
    static constexpr int NWC = BV / 16;            // waves that own columns
    static constexpr int RT = DK / 16;             // 16-row tiles of S
    static constexpr int ES = RC::ES, NP = RC::NP;
    // Row padding of the staged matrices, chosen from bank-conflict counts on
    // gfx950: every fragment is read with 16-byte reads (bf16 regions are
    // staged with the A-operand column permutation, see Stage::put_a),
    // conflict-free at a row pitch of 8 mod 16 dwords.  (Rows of 64, 32 or 16
    // data dwords plus 8.)
    static constexpr int PADB = 32;
    static constexpr int PW = (RC::W_ROW + PADB) / ES;   // pitches in elements
    static constexpr int PQ = (RC::Q_ROW + PADB) / ES;
    static constexpr int PKR = (RC::K_ROW + PADB) / ES;
    static constexpr int PMR = (RC::M_ROW + PADB) / ES;
    static constexpr int L_W = 0;
    static constexpr int L_Q = L_W + NP * 64 * PW * ES;
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
    // write one unit (rows padded by a multiple of 8 bytes only: two 8-byte writes)
    static __device__ __forceinline__ void put(unsigned char* p, u32x4 v) {
        if constexpr (PAD % 16 == 0) {
            *reinterpret_cast<u32x4*>(p) = v;
        } else {
            *reinterpret_cast<u32x2*>(p) = v.xy;
            *reinterpret_cast<u32x2*>(p + 8) = v.zw;
        }
    }
    // write unit (tid, i) of a matrix read as matrix-core A operands into the
    // region at `base`.  PERM (bf16 elements): in each 32-column group,
    // columns 4g .. 4g+3 and 16+4g .. 16+4g+3 are stored side by side at 8g,
    // so that a lane group's fragment is one 16-byte read.  Unit uc holds
    // columns 32 (uc / 4) + 8q .. +7 (q = uc % 4); its half h belongs to lane
    // group (2q + h) % 4, in the group's first four slots for q < 2 and its
    // last four for q >= 2.
    template <bool PERM>
    static __device__ __forceinline__ void put_a(unsigned char* base, int tid, int i, u32x4 v) {
        if constexpr (!PERM) {
            put(base + lds_off(tid, i), v);
        } else {
            static_assert(UPR % 4 == 0 && PAD % 16 == 0, "32-column groups, 16-byte rows");
            const int u = tid + NT * i;
            const int uc = u % UPR, q = uc & 3;
            unsigned char* rb = base + (u / UPR) * (UPR * 16 + PAD) + 64 * (uc >> 2) + 8 * (q >> 1);
            *reinterpret_cast<u32x2*>(rb + 16 * ((2 * q) & 3)) = v.xy;
            *reinterpret_cast<u32x2*>(rb + 16 * ((2 * q + 1) & 3)) = v.zw;
        }
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
    // segment mode: G chunks per segment; segment s of chain d sits in
    // segment slot floor(cu[d] / 64G) + d + s (equal-length: d * nseg + s)
    int G, nsslots;
    float* seg_start;   // [nsslots][H][DK][DV] start state of segments s >= 1
    float* seg_h;       // [nsslots][H][DK][DV] end state from a zero start (middle segments)
    float* seg_p;       // [nsslots][H][DK][DK] segment map P_s (middle segments)
};


// SEG: segment mode, phase 3 with OUT, phase 1 without; otherwise (OUT set)
// one workgroup walks a whole chain's value slice
template <typename Tin, int DK, int DV, bool CKPT, bool SEG, bool OUT>
__global__ void __launch_bounds__(512, 2) ckda_state_kernel(StateParams p)
{
    using SH = StateShape<Tin, DK, DV>;
    using RC = typename SH::RC;
    using PR = Prec<SH::F32>;
    constexpr int RT = SH::RT, NP = SH::NP, NT = SH::NT, NWC = SH::NWC;
    extern __shared__ __align__(16) unsigned char smem[];

    const int H = p.H;
    // work items: chains (or, in segment mode, segment slots) x heads; NS
    // slices per item: the value slices, then (segment phase 1) the
    // transition slices over the DK columns of P_s
    constexpr int NS = (SEG && !OUT) ? SH::NSLICE + SH::NTS : SH::NSLICE;
    const int nitems = SEG ? p.nsslots * H : (p.cu ? p.ndocs * H : p.B * H);
    int item, slice;
    {
        const int bid = blockIdx.x;
        if (NS == 1) {
            item = bid;
            slice = 0;
        } else {
            // the slices of one item land on the same XCD (workgroups are
            // dealt round-robin over 8 XCDs), so the record is read from HBM
            // once and the other slices hit that XCD's L2
            const int grp = 8 * NS;
            const int full = (nitems / 8) * grp;
            if (bid < full) {
                const int r = bid % grp;
                item = (bid / grp) * 8 + (r % 8);
                slice = r / 8;
            } else {
                const int r = bid - full;
                item = (nitems / 8) * 8 + r / NS;
                slice = r % NS;
            }
        }
    }
    const int h = item % H;
    const int NTC = (p.T + 63) / 64;   // equal-length chunks per sequence
    int sidx, seg = 0, ss = 0;
    if (!SEG) {
        sidx = item / H;
    } else {
        ss = item / H;
        if (p.cu) {   // the document whose segment slots hold ss
            int lo = 0, hi = p.ndocs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seg_slot0(p.cu[mid], mid, p.G) <= ss) lo = mid; else hi = mid - 1;
            }
            sidx = lo;
            seg = ss - seg_slot0(p.cu[lo], lo, p.G);
        } else {
            const int nsegT = (NTC + p.G - 1) / p.G;
            sidx = ss / nsegT;
            seg = ss - sidx * nsegT;
        }
    }
    int tok0, len, slot0;
    if (p.cu) {
        tok0 = p.cu[sidx];
        len = p.cu[sidx + 1] - tok0;
        slot0 = varlen_slot(tok0, sidx, 0);
    } else {
        tok0 = sidx * p.T;
        len = p.T;
        slot0 = sidx * NTC;
    }
    const int nchunks = (len + 63) / 64;
    int jbeg = 0, nloop = nchunks, nseg = 1;
    bool trans = false;
    if (SEG) {
        nseg = (nchunks + p.G - 1) / p.G;
        trans = slice >= SH::NSLICE;
        // phase 1: every segment but the last (transition slices: the middle
        // ones); phase 3: every segment (a chain of no chunks has one)
        const bool run = OUT ? seg < max(nseg, 1) : (seg < nseg - 1 && (seg > 0 || !trans));
        if (!run) return;   // the whole workgroup, before any barrier
        jbeg = seg * p.G;
        nloop = min(p.G, nchunks - jbeg);
    }
    // first 16-column tile of the slice (transition slices: columns of P_s)
    const int vt0 = ((trans ? slice - SH::NSLICE : slice) * SH::BV) / 16;
    const int vtu0 = trans ? 0 : vt0;   // u tile of wave 0 (transition slices read tiles of slice 0 and zero them)
    const int slotb = slot0 + jbeg;     // record slot of the first chunk walked
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);

    if (w >= 4) {
        // ================= loader waves ====================================
        // Two register groups: A = W, Qh (read by the first products of a
        // chunk), B = KbT, M, d (read by the rest).  Two barriers per chunk j:
        //   X (W, Qh of j no longer read; B of j in LDS) -> write A of j+1,
        //     issue A loads of j+2
        //   Y (chunk j done; A of j+1 in LDS) -> write B of j+1, issue B
        //     loads of j+2
        // so group A is written while the second half of chunk j runs and
        // group B while the first half of chunk j+1 runs: no write lies
        // between two chunks.
        using StW = Stage<NP * 64, RC::W_ROW / 16, SH::PADB, NT>;
        using StQ = Stage<NP * 64, RC::Q_ROW / 16, SH::PADB, NT>;
        using StK = Stage<NP * DK, RC::K_ROW / 16, SH::PADB, NT>;
        using StM = Stage<NP * 64, RC::M_ROW / 16, SH::PADB, NT>;
        using StD = Stage<1, DK * 4 / 16, 0, NT>;
        constexpr int NW_ = StW::N, NQ_ = StQ::N, NK_ = StK::N, NM_ = StM::N, ND_ = StD::N;
        constexpr int O_Q = NW_, NA = NW_ + NQ_;
        constexpr int O_M = NK_, O_D = O_M + NM_, NB = O_D + ND_;
        static_assert(StW::FULL && StQ::FULL && StK::FULL && StM::FULL, "unguarded staging loads");
        u32x4 ga[NA], gb[NB];   // native vectors (a struct copy would keep them in scratch)
#define CKDA_REC(J) reinterpret_cast<const u32x4*>(p.ws + (static_cast<size_t>(slotb + (J)) * H + h) * RC::BYTES + opaque_zero())
#define CKDA_LOAD_A(J)                                                                                       \
        {                                                                                                    \
            const u32x4* g_ = CKDA_REC(J);                                                                   \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NW_; ++i_) ga[i_] = g_[RC::OFF_W / 16 + t_ + NT * i_];   \
            if (OUT)                                                                                         \
                _Pragma("unroll") for (int i_ = 0; i_ < NQ_; ++i_) ga[O_Q + i_] = g_[RC::OFF_Q / 16 + t_ + NT * i_]; \
        }
#define CKDA_LOAD_B(J)                                                                                       \
        {                                                                                                    \
            const u32x4* g_ = CKDA_REC(J);                                                                   \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NK_; ++i_) gb[i_] = g_[RC::OFF_K / 16 + t_ + NT * i_];   \
            if (OUT)                                                                                         \
                _Pragma("unroll") for (int i_ = 0; i_ < NM_; ++i_) gb[O_M + i_] = g_[RC::OFF_M / 16 + t_ + NT * i_]; \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) gb[O_D + i_] = g_[RC::OFF_D / 16 + t_ + NT * i_];                       \
        }
#define CKDA_STORE_A()                                                                                       \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NW_; ++i_)                                               \
                StW::template put_a<PR::kPermA>(sm_ + SH::L_W, t_, i_, ga[i_]);                                \
            if (OUT)                                                                                         \
                _Pragma("unroll") for (int i_ = 0; i_ < NQ_; ++i_)                                           \
                    StQ::template put_a<PR::kPermA>(sm_ + SH::L_Q, t_, i_, ga[O_Q + i_]);                      \
        }
#define CKDA_STORE_B()                                                                                       \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NK_; ++i_)                                               \
                StK::template put_a<PR::kPermA>(sm_ + SH::L_K, t_, i_, gb[i_]);                                \
            if (OUT)                                                                                         \
                _Pragma("unroll") for (int i_ = 0; i_ < NM_; ++i_)                                           \
                    StM::template put_a<PR::kPermA>(sm_ + SH::L_M, t_, i_, gb[O_M + i_]);                      \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) *reinterpret_cast<u32x4*>(sm_ + SH::L_D + StD::lds_off(t_, i_)) = gb[O_D + i_]; \
        }
        if (nloop > 0) {
            CKDA_LOAD_A(0)
            CKDA_LOAD_B(0)
            CKDA_STORE_A()
            CKDA_STORE_B()
            CKDA_LOAD_A(min(1, nloop - 1))
            CKDA_LOAD_B(min(1, nloop - 1))
        }
        lds_sync();   // record 0 in LDS
        // (the last chunks re-read the final record: no branches)
        for (int j = 0; j < nloop; ++j) {
            lds_sync();   // X: W, Qh of chunk j consumed
            CKDA_STORE_A()
            CKDA_LOAD_A(min(j + 2, nloop - 1))
            lds_sync();   // Y: chunk j consumed
            CKDA_STORE_B()
            CKDA_LOAD_B(min(j + 2, nloop - 1))
        }
#undef CKDA_REC
#undef CKDA_LOAD_A
#undef CKDA_LOAD_B
#undef CKDA_STORE_A
#undef CKDA_STORE_B
        return;
    }

    // ================= compute waves ==========================================
    const size_t st_off = (static_cast<size_t>(sidx) * H + h) * DK * DV;
    // (transition slices: only columns below DK exist)
    const bool has_col = w < NWC && (!trans || 16 * (vt0 + w) < DK);
    // the wave's 16-column tile of DV; waves without columns (DV < 64) run
    // the slice's last tile again with their stores switched off, so the
    // loop body has no branches around vector memory (the compiler's wait
    // insertion then knows how many stores are in flight)
    const int wt = min(w, NWC - 1);
    const int vt = vt0 + wt;

    // ---- state: lane (n, g) holds rows 16rt + 4g + i of column 16vt + n ----
    // start: h0 (or zero); segment mode: the identity for transition slices,
    // zero for the middle segments of phase 1, the scanned start in phase 3
    const float* src = p.h0 ? p.h0 + st_off : nullptr;
    if (SEG && seg > 0) src = OUT ? p.seg_start + (static_cast<size_t>(ss) * H + h) * DK * DV : nullptr;
    f32x4 S[RT];
    {
        const int l = threadIdx.x & 63, gq = l >> 4, col = 16 * vt + (l & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * gq + i;
                S[rt][i] = trans ? (row == col ? 1.f : 0.f)
                                 : ((has_col && src) ? src[static_cast<size_t>(row) * DV + col] : 0.f);
            }
    }

    // checkpoint of walked chunk j: equal-length [B,H,NT,DK,DV]; varlen
    // [slot][H][DK][DV] (the record's slot)
    const size_t ck0 = p.cu ? static_cast<size_t>(slotb) * H + h
                            : (static_cast<size_t>(sidx) * H + h) * static_cast<size_t>(nchunks) + jbeg;
    const int ckstep = p.cu ? H : 1;
    // the wave's u tiles (J, vtu0 + wt) of chunk j, in the C/D lane layout,
    // read straight from the record one chunk ahead (u is the one part of the
    // record no other wave needs, so it skips LDS); the last chunk re-reads
    // its own record
    auto u_src = [&](int jj) {
        return reinterpret_cast<const f32x4*>(p.ws + (static_cast<size_t>(slotb + jj) * H + h) * RC::BYTES +
                                              RC::OFF_U + opaque_zero()) +
               (vtu0 + wt) * 64 + (threadIdx.x & 63);
    };
    f32x4 un[4];
    if (nloop > 0) {
        const f32x4* us = u_src(0);
#pragma unroll
        for (int J = 0; J < 4; ++J) un[J] = us[J * (DV / 16) * 64];
    }
    lds_sync();   // record 0 in LDS
    for (int j = 0; j < nloop; ++j) {
        const int c0 = 64 * (jbeg + j);
        const int L = min(64, len - c0);
        f32x4 u[4];   // transition slices: u = 0 (P_s is the maps' linear part)
#pragma unroll
        for (int J = 0; J < 4; ++J) u[J] = (SEG && trans) ? f32x4{0.f, 0.f, 0.f, 0.f} : un[J];
        {
            const f32x4* us = u_src(min(j + 1, nloop - 1));
#pragma unroll
            for (int J = 0; J < 4; ++J) un[J] = us[J * (DV / 16) * 64];
        }
        {
            unsigned char* const sm = smem + opaque_zero();
            const LdsMat Wm{sm + SH::L_W, SH::PW, 64 * SH::PW};
            const LdsMat Qm{sm + SH::L_Q, SH::PQ, 64 * SH::PQ};
            const LdsMat Km{sm + SH::L_K, SH::PKR, DK * SH::PKR};
            const LdsMat Mm{sm + SH::L_M, SH::PMR, 64 * SH::PMR};
            const float* dl = reinterpret_cast<const float*>(sm + SH::L_D);
            const int l = opaque_tid() & 63, n = l & 15, gq = l >> 4;
            const int col = 16 * vt + n;
            if (CKPT && OUT) {   // the state at the chunk start (waves without columns store nothing)
                const float* hc = p.h_ckpt + (ck0 + static_cast<size_t>(j) * ckstep) * DK * DV;
                const __amdgpu_buffer_rsrc_t hrc = buffer_rsrc(hc, has_col ? DK * DV * 4 : 0);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        buffer_store_f32(hrc, static_cast<uint32_t>(((16 * rt + 4 * gq + i) * DV + col) * 4), S[rt][i]);
            }
            // The LDS fragments of step k+1 are read while the products of
            // step k run (fences keep the scheduler from sinking each read
            // next to its use, which would expose every LDS round trip: one
            // wave per SIMD has no other wave to hide it behind).
            constexpr int KS = RT / 2;
            // W S and Qh S: 32 channels per k-step, in steps of two 16-token
            // row blocks; the fragments of step s+1 are read while the 12
            // products of step s run (two steps in flight keep the operand
            // buffers at 64 registers)
            typename PR::F8 Sb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Sb[ks] = PR::regs8(S[2 * ks], S[2 * ks + 1]);
            f32x4 X[4], Y[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                X[R] = f32x4{0.f, 0.f, 0.f, 0.f};
                Y[R] = X[R];
            }
            {
                constexpr int NSTEP = 2 * KS;
                typename PR::F8 wa[2][2];
                typename PR::F8 qa[2][2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    wa[0][r] = PR::loadA(Wm, 16 * r + n, 0, gq);
                    if (OUT) qa[0][r] = PR::loadA(Qm, 16 * r + n, 0, gq);
                }
#pragma unroll
                for (int st = 0; st < NSTEP; ++st) {
                    const int ks = st / 2, R0 = 2 * (st % 2);
                    if (st + 1 < NSTEP) {
                        const int k1 = 32 * ((st + 1) / 2), R1 = 2 * ((st + 1) % 2);
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            wa[(st + 1) & 1][r] = PR::loadA(Wm, 16 * (R1 + r) + n, k1, gq);
                            if (OUT) qa[(st + 1) & 1][r] = PR::loadA(Qm, 16 * (R1 + r) + n, k1, gq);
                        }
                    }
                    CKDA_FENCE();
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        X[R0 + r] = PR::mma8(wa[st & 1][r], Sb[ks], X[R0 + r]);
                        if (OUT) Y[R0 + r] = PR::mma8(qa[st & 1][r], Sb[ks], Y[R0 + r]);
                    }
                    CKDA_FENCE();
                }
            }
            lds_sync();   // X: W, Qh consumed (the loaders refill them for chunk j+1); KbT, M, d in LDS
            // M fragments for the output and the first KbT fragments, read
            // while U is formed
            typename PR::F8 ma[6];
            if (OUT) {
#pragma unroll
                for (int R = 0, x = 0; R < 4; ++R)
#pragma unroll
                    for (int kt = 0; kt <= R / 2; ++kt, ++x)
                        ma[x] = PR::loadA(Mm, 16 * R + n, 32 * kt, gq);
            }
            typename PR::F8 ka[2][2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) ka[0][kt] = PR::loadA(Km, n, 32 * kt, gq);
            CKDA_FENCE();
            // U = u - W S, as B operands over 32 tokens per step
            typename PR::F8 Ub[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) Ub[kt] = PR::regs8(u[2 * kt] - X[2 * kt], u[2 * kt + 1] - X[2 * kt + 1]);
            // O = scale (Qh S + M U) (M is zero above its diagonal, also in
            // blocks (0,1) and (2,3) that the 32-token steps read); the
            // buffer covers the chunk's L valid rows
            if (OUT) {
                const __amdgpu_buffer_rsrc_t orc = buffer_rsrc(p.o + static_cast<size_t>(tok0 + c0) * H * DV,
                                                               has_col ? static_cast<uint32_t>(L * H * DV * 4) : 0u);
#pragma unroll
                for (int R = 0, x = 0; R < 4; ++R) {
                    f32x4 acc = Y[R];
#pragma unroll
                    for (int kt = 0; kt <= R / 2; ++kt, ++x) acc = PR::mma8(ma[x], Ub[kt], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tt = 16 * R + 4 * gq + i;
                        buffer_store_f32(orc, static_cast<uint32_t>(((tt * H + h) * DV + col) * 4), p.scale * acc[i]);
                    }
                }
            }
            // S <- Diag(d) S + KbT U
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (rt + 1 < RT) {
#pragma unroll
                    for (int kt = 0; kt < 2; ++kt)
                        ka[(rt + 1) & 1][kt] = PR::loadA(Km, 16 * (rt + 1) + n, 32 * kt, gq);
                }
                const f32x4 dd = *reinterpret_cast<const f32x4*>(dl + 16 * rt + 4 * gq);
                CKDA_FENCE();
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) acc = PR::mma8(ka[rt & 1][kt], Ub[kt], acc);
                S[rt] = dd * S[rt] + acc;
                CKDA_FENCE();
            }
        }
        lds_sync();   // Y: chunk j consumed (the loaders refill KbT, M, d for chunk j+1)
    }

    // the end state: ht (whole chains; phase 3, a chain's last segment), or
    // in phase 1 start_1 (first segments), H_s or P_s (middle segments)
    float* dst = p.ht ? p.ht + st_off : nullptr;
    int pitch = DV;
    if (SEG && !OUT) {
        if (seg == 0) {
            dst = p.seg_start + (static_cast<size_t>(ss + 1) * H + h) * DK * DV;
        } else {
            dst = trans ? p.seg_p + (static_cast<size_t>(ss) * H + h) * DK * DK
                        : p.seg_h + (static_cast<size_t>(ss) * H + h) * DK * DV;
            pitch = trans ? DK : DV;
        }
    } else if (SEG && seg < nseg - 1) {
        dst = nullptr;
    }
    if (dst && has_col) {
        const int l = threadIdx.x & 63, gq = l >> 4, col = 16 * vt + (l & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[opaque_zero() + static_cast<size_t>(16 * rt + 4 * gq + i) * pitch + col] = S[rt][i];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

// measured on MI355X (dk = dv = 128, bf16 records): a lone chain steps in
// about 3.1 us (the unit); 256 CUs complete about 53 workgroup chunk-steps
// per us, with one workgroup per CU or two; a step without the output
// products costs about 0.6 of one; a scan step about 3 units
constexpr SegCost kStateCost{0.64, 0.6, 3.0};

template <typename Tin, int DK, int DV, bool CKPT, bool SEG, bool OUT>
hipError_t launch_state_kernel(const StateParams& p, int grid, hipStream_t stream) {
    using SH = StateShape<Tin, DK, DV>;
    if (grid == 0) return hipSuccess;
    auto kern = ckda_state_kernel<Tin, DK, DV, CKPT && OUT, SEG, OUT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(2 * SH::NT), SH::LDS, stream, p);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV, bool CKPT>
hipError_t launch_state_c(const FwdArgs& A, size_t rec_bytes, hipStream_t stream) {
    using SH = StateShape<Tin, DK, DV>;
    StateParams p{};
    p.ws = static_cast<const unsigned char*>(A.ws);
    p.h0 = A.h0; p.o = A.o; p.ht = A.ht; p.h_ckpt = A.h_ckpt; p.cu = A.cu; p.scale = A.scale;
    p.B = A.B; p.T = A.T; p.H = A.H; p.ndocs = A.ndocs;
    const int nchains = A.cu ? A.ndocs * A.H : A.B * A.H;
    constexpr int NTS = SH::NTS;
    const bool varlen = A.cu != nullptr;
    const size_t avail = A.ws_bytes > align256(rec_bytes) ? A.ws_bytes - align256(rec_bytes) : 0;
    auto fits = [&](int G) {
        return seg_buffer_bytes(seg_slots(varlen, A.B, A.T, A.ndocs, G), A.H, DK, DV) <= avail;
    };
    const int G = plan_segments(chain_chunks(A.cu_host, varlen, A.ndocs, A.B, A.T), A.H, SH::NSLICE, NTS,
                                kStateCost, device_cus(stream), fits);
    if (G == 0) return launch_state_kernel<Tin, DK, DV, CKPT, false, true>(p, nchains * SH::NSLICE, stream);
    p.G = G;
    p.nsslots = seg_slots(varlen, A.B, A.T, A.ndocs, G);
    float* sb = reinterpret_cast<float*>(static_cast<unsigned char*>(A.ws) + align256(rec_bytes));
    const size_t per = static_cast<size_t>(p.nsslots) * A.H * DK * DV;
    p.seg_start = sb;
    p.seg_h = sb + per;
    p.seg_p = sb + 2 * per;
    hipError_t e = launch_state_kernel<Tin, DK, DV, CKPT, true, false>(p, p.nsslots * A.H * (SH::NSLICE + NTS), stream);
    if (e != hipSuccess) return e;
    const SegScanParams sp{A.cu, A.T, A.H, G, p.seg_start, p.seg_h, p.seg_p, 0};
    hipLaunchKernelGGL((ckda_seg_scan_kernel<DK, DV>), dim3(nchains * (DV / kScanCols)), dim3(256), 0, stream, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_state_kernel<Tin, DK, DV, CKPT, true, true>(p, p.nsslots * A.H * SH::NSLICE, stream);
}

template <typename Tin, int DK, int DV>
hipError_t launch_state_t(const FwdArgs& A, hipStream_t stream) {
    const size_t rec = static_cast<size_t>(A.cu ? (A.T + 63) / 64 + A.ndocs : A.B * ((A.T + 63) / 64)) * A.H *
                       Record<DK, DV, sizeof(Tin) == 4>::BYTES;
    return A.h_ckpt ? launch_state_c<Tin, DK, DV, true>(A, rec, stream)
                    : launch_state_c<Tin, DK, DV, false>(A, rec, stream);
}

template <typename Tin>
hipError_t launch_state_dt(const FwdArgs& A, hipStream_t stream) {
#define CKDA_STATE(DK_, DV_) \
    if (A.DK == DK_ && A.DV == DV_) return launch_state_t<Tin, DK_, DV_>(A, stream);
    CKDA_STATE(32, 32) CKDA_STATE(32, 64) CKDA_STATE(32, 128)
    CKDA_STATE(64, 32) CKDA_STATE(64, 64) CKDA_STATE(64, 128)
    CKDA_STATE(128, 32) CKDA_STATE(128, 64) CKDA_STATE(128, 128)
#undef CKDA_STATE
    return hipErrorInvalidValue;
}

size_t record_bytes(int DK, int DV, bool bf16) {
    size_t rec = 0;
#define CKDA_REC(DK_, DV_) \
    if (DK == DK_ && DV == DV_) rec = bf16 ? Record<DK_, DV_, false>::BYTES : Record<DK_, DV_, true>::BYTES;
    CKDA_REC(32, 32) CKDA_REC(32, 64) CKDA_REC(32, 128)
    CKDA_REC(64, 32) CKDA_REC(64, 64) CKDA_REC(64, 128)
    CKDA_REC(128, 32) CKDA_REC(128, 64) CKDA_REC(128, 128)
#undef CKDA_REC
    return rec;
}

}  // namespace

hipError_t launch_state(const FwdArgs& A, hipStream_t stream) {
    return A.bf16 ? launch_state_dt<bf16_t>(A, stream) : launch_state_dt<float>(A, stream);
}

namespace {
std::atomic<int> g_seg_chunks{0};   // 0: automatic, < 0: never, >= kSegMinChunks: that length
}  // namespace

void set_segment_chunks(int G) { g_seg_chunks.store(G); }
int segment_chunks() { return g_seg_chunks.load(); }
int segment_min_chunks() { return kSegMinChunks; }

int device_cus(hipStream_t stream) {
    static std::atomic<int> cached[64];
    hipDevice_t dev = 0;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        if (hipGetDevice(&dev) != hipSuccess) return 256;
    }
    if (dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load();
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n);
    }
    return n;
}

// forward = chunk-local kernel over every (chunk, head), then the state pass
size_t fwd_workspace_bytes(int nslots, int H, int DK, int DV, bool bf16) {
    return static_cast<size_t>(nslots) * H * record_bytes(DK, DV, bf16);
}

size_t fwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV, bool bf16) {
    const size_t rec = fwd_workspace_bytes(nslots, H, DK, DV, bf16);
    return align256(rec) + seg_buffer_bytes(nsslots_max, H, DK, DV);
}

hipError_t launch_fwd(const FwdArgs& A, int nslots, hipStream_t stream) {
    hipError_t e = launch_chunk(A, nslots, stream);
    if (e != hipSuccess) return e;
    return launch_state(A, stream);
}

}  // namespace ckda
