// rev.hip -- reverse (state-gradient) pass of the CKDA backward.
//
// The chunked forward's state step is affine in the state,
//   U = u - W S,   O = scale (Qh S + M U),   S' = Diag(d) S + KbT U,
// so the gradient G = dL/dS' at a chunk's end (true frame) goes back through
// the chunk by the adjoint step
//   dU = scale M^T dO + KbT^T G,   G_start = Diag(d) G + scale Qh^T dO - W^T dU
// (WY/UT chunk form of the recurrence, Complex KDA paper page, section 2
// "Linear RNNs"; the backward is the plain derivative of the forward since the
// pages' own backward convention is in an appendix they do not include).  The
// chunk quantities come from the reverse record (RevRecord, written by the
// chunk-local kernel in its REV mode: KB = KbT^T, QT = Qh^T, WT = W^T,
// MT = M^T, d), so the pass only runs these state-gradient products, one
// chain at a time, from the chain's last chunk to its first.
//
// Work decomposition (gfx950): as the forward's state pass, one 512-thread
// workgroup per (sequence or document, head, 64-wide value slice).  Waves
// 0..3 own 16 value columns each and keep that DK x 16 block of G in MFMA
// accumulator registers; waves 4..7 only move data, holding the next chunk's
// record in registers (read one chunk ahead) and writing it to LDS in two
// groups (A = KB, MT for the first products; B = QT, WT, d for the update)
// while the matrix-core waves work on the other group.  Each compute wave
// reads its dO tiles (16 tokens x 16 columns per tile, the C/D lane layout)
// straight from the input one chunk ahead.
//
// Outputs per chunk (in the chunk's record slot, for the chunk-parallel
// gradient pass): dU [64][DV] in C/D tiles and G at the chunk's end
// [DK][DV]; per chain dh0 = G at its start.
#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_prec.h"
#include "ckda_record.h"
#include "ckda_segments.h"
#include "ckda_sync.h"

namespace ckda {

template <typename Tin, int DK, int DV>
struct RevShape {
    static constexpr bool F32 = sizeof(Tin) == 4;
    using RC = RevRecord<DK, DV, F32>;
    static constexpr int NT = 256;                 // threads per role
    static constexpr int BV = DV < 64 ? DV : 64;   // value columns per workgroup
    static constexpr int NSLICE = DV / BV;
    static constexpr int NTS = (DK + BV - 1) / BV; // transition slices over the DK columns of P_s
    static constexpr int NWC = BV / 16;            // waves that own columns
    static constexpr int RT = DK / 16;             // 16-row tiles of G
    static constexpr int ES = RC::ES, NP = RC::NP;
    // rows padded by 32 bytes: 16-byte fragment reads conflict-free at a
    // pitch of 8 mod 16 dwords (as in the forward's state pass)
    static constexpr int PADB = 32;
    static constexpr int PKB = (RC::KB_ROW + PADB) / ES;
    static constexpr int PMT = (RC::MT_ROW + PADB) / ES;
    static constexpr int PQT = (RC::QT_ROW + PADB) / ES;
    static constexpr int PWT = (RC::WT_ROW + PADB) / ES;
    static constexpr int L_KB = 0;
    static constexpr int L_MT = L_KB + NP * 64 * PKB * ES;
    static constexpr int L_QT = L_MT + NP * 64 * PMT * ES;
    static constexpr int L_WT = L_QT + NP * DK * PQT * ES;
    static constexpr int L_D = L_WT + NP * DK * PWT * ES;
    static constexpr int LDS = L_D + DK * 4;
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// the forward state pass's staging helper, over the reverse record
template <int ROWS, int UPR, int PAD, int NT>
struct RStage {
    static constexpr int UNITS = ROWS * UPR;
    static constexpr int N = (UNITS + NT - 1) / NT;
    static constexpr bool FULL = (UNITS % NT) == 0;
    static __device__ __forceinline__ bool has(int tid, int i) { return FULL || tid + NT * i < UNITS; }
    static __device__ __forceinline__ int lds_off(int tid, int i) {
        const int u = tid + NT * i;
        return (u / UPR) * (UPR * 16 + PAD) + (u % UPR) * 16;
    }
    // unit (tid, i) of a matrix read as A operands; PERM (bf16): in each
    // 32-column group, columns 4g .. 4g+3 and 16+4g .. 16+4g+3 side by side at
    // 8g, so a lane group's fragment is one 16-byte read
    template <bool PERM>
    static __device__ __forceinline__ void put_a(unsigned char* base, int tid, int i, u32x4 v) {
        if constexpr (!PERM) {
            *reinterpret_cast<u32x4*>(base + lds_off(tid, i)) = v;
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

// Transposed staging of a forward-record matrix X [SR][SC] (planes as in the
// record) as X^T [SC][SR] in the A-operand layout RStage writes (target rows
// TPB bytes apart, the lo plane SC rows after the hi plane).  bf16: a task
// takes two source rows, so each target element pair (columns r, r+1) is one
// 4-byte LDS word; fp32: one row.
template <int SR, int SC, bool F32, int NT>
struct TStage {
    static constexpr int RPT = F32 ? 1 : 2;      // source rows per task
    static constexpr int EPU = F32 ? 4 : 8;      // elements per 16-byte unit
    static constexpr int NPL = F32 ? 1 : 2;      // planes
    static constexpr int ES = F32 ? 4 : 2;
    static constexpr int RG = SR / RPT, UC = SC / EPU;
    static constexpr int TASKS = NPL * RG * UC;
    static constexpr int N = TASKS / NT;         // tasks per thread
    static_assert(TASKS % NT == 0, "whole tasks per thread");
    // four lanes take consecutive units of one source row (64 contiguous
    // bytes), the next lanes the following row pairs: a load instruction
    // touches half as many cache lines as with one unit per row, for up to
    // four target rows per bank in a write (measured on layer_bwd: 1.84 ms
    // per backward against 1.92 ms with lanes walking row pairs only)
    static constexpr int LU = UC < 4 ? UC : 4;
    static_assert(UC % LU == 0, "whole lane groups per row");
    static __device__ __forceinline__ void task(int tid, int i, int& pl, int& u, int& r0) {
        const int q = tid + NT * i;
        r0 = RPT * ((q / LU) % RG);
        u = ((q / (LU * RG)) % (UC / LU)) * LU + q % LU;
        pl = q / (RG * UC);
    }
    static __device__ __forceinline__ void load(const unsigned char* src, int tid, int i, u32x4* v) {
        int pl, u, r0;
        task(tid, i, pl, u, r0);
        const unsigned char* a = src + static_cast<size_t>(pl) * SR * SC * ES + static_cast<size_t>(r0) * SC * ES + 16 * u;
#pragma unroll
        for (int r = 0; r < RPT; ++r) v[r] = *reinterpret_cast<const u32x4*>(a + r * SC * ES);
    }
    // storage column of target column c (bf16: the A-operand permutation)
    static __device__ __forceinline__ int scol(int c) {
        if constexpr (F32) return c;
        else return 32 * (c / 32) + 8 * ((c % 16) / 4) + 4 * ((c % 32) / 16) + (c % 4);
    }
    static __device__ __forceinline__ void store(unsigned char* dst, int tpb, int tid, int i, const u32x4* v) {
        int pl, u, r0;
        task(tid, i, pl, u, r0);
        unsigned char* b = dst + (pl * SC + EPU * u) * tpb + scol(r0) * ES;
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
            uint32_t w;
            if constexpr (F32) {
                w = v[0][e];
            } else {
                const uint32_t a = (v[0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const uint32_t c = (v[1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                w = a | (c << 16);
            }
            *reinterpret_cast<uint32_t*>(b + e * tpb) = w;
        }
    }
};

// SEG: segment mode (phase 3 with OUT, phase 1 without); otherwise (OUT set)
// whole chains.  Segment phase 1 walks every segment but a chain's first
// (its value columns from zero, or from dht for the chain's last segment;
// for the middle ones also DK transition columns from the identity with dO
// switched off) and writes the segment's start G (last segment: into the
// previous segment's end slot), H_s or P_s; phase 3 walks every segment from
// its end G and writes the per-chunk outputs (and dh0 at the chain's start).
// FR: p.ws holds the forward's chunk records (ckda_record.h Record), staged
// transposed; otherwise the reverse records of the backward's first pass
template <typename Tin, int DK, int DV, bool SEG, bool OUT, bool FR>
__global__ void __launch_bounds__(512, 2) ckda_rev_kernel(RevParams p)
{
    using SH = RevShape<Tin, DK, DV>;
    using RC = typename SH::RC;
    using PR = Prec<SH::F32>;
    constexpr int RT = SH::RT, NP = SH::NP, NT = SH::NT, NWC = SH::NWC;
    constexpr int NS = (SEG && !OUT) ? SH::NSLICE + SH::NTS : SH::NSLICE;
    extern __shared__ __align__(16) unsigned char smem[];

    const int H = p.H;
    const int nitems = SEG ? p.nsslots * H : (p.cu ? p.ndocs * H : p.B * H);
    int item, slice;
    {
        const int bid = blockIdx.x;
        if (NS == 1) {
            item = bid;
            slice = 0;
        } else {   // the slices of one item on one XCD (its L2 serves the second read of the record)
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
    const int NTC = (p.T + 63) / 64;
    int sidx, seg = 0, ss = 0;
    if (!SEG) {
        sidx = item / H;
    } else {
        ss = item / H;
        if (p.cu) {   // the document whose segment slots hold ss
            int lo = 0, hi = p.ndocs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seg_slot0(p.cu[mid], mid, p.seg_len) <= ss) lo = mid; else hi = mid - 1;
            }
            sidx = lo;
            seg = ss - seg_slot0(p.cu[lo], lo, p.seg_len);
        } else {
            const int nsegT = (NTC + p.seg_len - 1) / p.seg_len;
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
        nseg = (nchunks + p.seg_len - 1) / p.seg_len;
        trans = slice >= SH::NSLICE;
        // phase 1: every segment but the first (transition slices: the middle
        // ones); phase 3: every segment (a chain of no chunks has one)
        const bool run = OUT ? seg < max(nseg, 1) : (seg > 0 && seg < nseg && (seg < nseg - 1 || !trans));
        if (!run) return;   // the whole workgroup, before any barrier
        jbeg = seg * p.seg_len;
        nloop = max(0, min(p.seg_len, nchunks - jbeg));
    }
    const bool last = !SEG || seg >= nseg - 1;   // the walk starts at the chain's end (dht)
    // first 16-column tile of the slice (transition slices: columns of P_s)
    const int vt0 = ((trans ? slice - SH::NSLICE : slice) * SH::BV) / 16;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);

    // walk step j covers chunk nloop - 1 - j
    if (FR && w >= 4) {
        // ============ loader waves over the forward's records (transposed) ====
        using FRC = Record<DK, DV, SH::F32>;
        using TKB = TStage<DK, 64, SH::F32, NT>;   // KbT [DK][64] -> KB
        using TMT = TStage<64, 64, SH::F32, NT>;   // M -> M^T
        using TQT = TStage<64, DK, SH::F32, NT>;   // Qh [64][DK] -> Qh^T
        using TWT = TStage<64, DK, SH::F32, NT>;   // W -> W^T
        using StD = RStage<1, DK * 4 / 16, 0, NT>;
        constexpr int RPT = TKB::RPT;
        constexpr int NKB = TKB::N * RPT, NMT = TMT::N * RPT, NQT = TQT::N * RPT, NWT = TWT::N * RPT, ND_ = StD::N;
        constexpr int O_MT = NKB, NA = NKB + NMT;
        constexpr int O_WT = NQT, O_D = O_WT + NWT, NB = O_D + ND_;
        u32x4 ga[NA], gb[NB];
#define CKDA_FREC(J) (p.ws + (static_cast<size_t>(slot0 + jbeg + nloop - 1 - (J)) * H + h) * FRC::BYTES + opaque_zero())
#define CKDA_FLOAD_A(J)                                                                                      \
        {                                                                                                    \
            const unsigned char* r_ = CKDA_FREC(J);                                                          \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < TKB::N; ++i_) TKB::load(r_ + FRC::OFF_K, t_, i_, ga + RPT * i_); \
            _Pragma("unroll") for (int i_ = 0; i_ < TMT::N; ++i_) TMT::load(r_ + FRC::OFF_M, t_, i_, ga + O_MT + RPT * i_); \
        }
#define CKDA_FLOAD_B(J)                                                                                      \
        {                                                                                                    \
            const unsigned char* r_ = CKDA_FREC(J);                                                          \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < TQT::N; ++i_) TQT::load(r_ + FRC::OFF_Q, t_, i_, gb + RPT * i_); \
            _Pragma("unroll") for (int i_ = 0; i_ < TWT::N; ++i_) TWT::load(r_ + FRC::OFF_W, t_, i_, gb + O_WT + RPT * i_); \
            const u32x4* d_ = reinterpret_cast<const u32x4*>(r_ + FRC::OFF_D);                              \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) gb[O_D + i_] = d_[t_ + NT * i_];                                        \
        }
#define CKDA_FSTORE_A()                                                                                      \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < TKB::N; ++i_) TKB::store(sm_ + SH::L_KB, SH::PKB * SH::ES, t_, i_, ga + RPT * i_); \
            _Pragma("unroll") for (int i_ = 0; i_ < TMT::N; ++i_) TMT::store(sm_ + SH::L_MT, SH::PMT * SH::ES, t_, i_, ga + O_MT + RPT * i_); \
        }
#define CKDA_FSTORE_B()                                                                                      \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < TQT::N; ++i_) TQT::store(sm_ + SH::L_QT, SH::PQT * SH::ES, t_, i_, gb + RPT * i_); \
            _Pragma("unroll") for (int i_ = 0; i_ < TWT::N; ++i_) TWT::store(sm_ + SH::L_WT, SH::PWT * SH::ES, t_, i_, gb + O_WT + RPT * i_); \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) *reinterpret_cast<u32x4*>(sm_ + SH::L_D + StD::lds_off(t_, i_)) = gb[O_D + i_]; \
        }
        if (nloop > 0) {
            CKDA_FLOAD_A(0)
            CKDA_FLOAD_B(0)
            CKDA_FSTORE_A()
            CKDA_FSTORE_B()
            CKDA_FLOAD_A(min(1, nloop - 1))
            CKDA_FLOAD_B(min(1, nloop - 1))
        }
        lds_sync();   // record of walk step 0 in LDS
        for (int j = 0; j < nloop; ++j) {
            lds_sync();   // X: KB, MT of step j consumed
            CKDA_FSTORE_A()
            CKDA_FLOAD_A(min(j + 2, nloop - 1))
            lds_sync();   // Y: step j consumed
            CKDA_FSTORE_B()
            CKDA_FLOAD_B(min(j + 2, nloop - 1))
        }
#undef CKDA_FREC
#undef CKDA_FLOAD_A
#undef CKDA_FLOAD_B
#undef CKDA_FSTORE_A
#undef CKDA_FSTORE_B
        return;
    }
    if (!FR && w >= 4) {
        // ================= loader waves (as in the forward's state pass) ======
        using StKB = RStage<NP * 64, RC::KB_ROW / 16, SH::PADB, NT>;
        using StMT = RStage<NP * 64, RC::MT_ROW / 16, SH::PADB, NT>;
        using StQT = RStage<NP * DK, RC::QT_ROW / 16, SH::PADB, NT>;
        using StWT = RStage<NP * DK, RC::WT_ROW / 16, SH::PADB, NT>;
        using StD = RStage<1, DK * 4 / 16, 0, NT>;
        constexpr int NKB = StKB::N, NMT = StMT::N, NQT = StQT::N, NWT = StWT::N, ND_ = StD::N;
        constexpr int O_MT = NKB, NA = NKB + NMT;
        constexpr int O_WT = NQT, O_D = O_WT + NWT, NB = O_D + ND_;
        static_assert(StKB::FULL && StMT::FULL && StQT::FULL && StWT::FULL, "unguarded staging loads");
        u32x4 ga[NA], gb[NB];
#define CKDA_RREC(J) reinterpret_cast<const u32x4*>(p.ws + (static_cast<size_t>(slot0 + jbeg + nloop - 1 - (J)) * H + h) * RC::BYTES + opaque_zero())
#define CKDA_RLOAD_A(J)                                                                                      \
        {                                                                                                    \
            const u32x4* g_ = CKDA_RREC(J);                                                                  \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NKB; ++i_) ga[i_] = g_[RC::OFF_KB / 16 + t_ + NT * i_];  \
            _Pragma("unroll") for (int i_ = 0; i_ < NMT; ++i_) ga[O_MT + i_] = g_[RC::OFF_MT / 16 + t_ + NT * i_]; \
        }
#define CKDA_RLOAD_B(J)                                                                                      \
        {                                                                                                    \
            const u32x4* g_ = CKDA_RREC(J);                                                                  \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NQT; ++i_) gb[i_] = g_[RC::OFF_QT / 16 + t_ + NT * i_];  \
            _Pragma("unroll") for (int i_ = 0; i_ < NWT; ++i_) gb[O_WT + i_] = g_[RC::OFF_WT / 16 + t_ + NT * i_]; \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) gb[O_D + i_] = g_[RC::OFF_D / 16 + t_ + NT * i_];                       \
        }
#define CKDA_RSTORE_A()                                                                                      \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NKB; ++i_)                                               \
                StKB::template put_a<PR::kPermA>(sm_ + SH::L_KB, t_, i_, ga[i_]);                              \
            _Pragma("unroll") for (int i_ = 0; i_ < NMT; ++i_)                                               \
                StMT::template put_a<PR::kPermA>(sm_ + SH::L_MT, t_, i_, ga[O_MT + i_]);                       \
        }
#define CKDA_RSTORE_B()                                                                                      \
        {                                                                                                    \
            unsigned char* const sm_ = smem + opaque_zero();                                                 \
            const int t_ = opaque_tid() - NT;                                                                \
            _Pragma("unroll") for (int i_ = 0; i_ < NQT; ++i_)                                               \
                StQT::template put_a<PR::kPermA>(sm_ + SH::L_QT, t_, i_, gb[i_]);                              \
            _Pragma("unroll") for (int i_ = 0; i_ < NWT; ++i_)                                               \
                StWT::template put_a<PR::kPermA>(sm_ + SH::L_WT, t_, i_, gb[O_WT + i_]);                       \
            _Pragma("unroll") for (int i_ = 0; i_ < ND_; ++i_)                                               \
                if (StD::has(t_, i_)) *reinterpret_cast<u32x4*>(sm_ + SH::L_D + StD::lds_off(t_, i_)) = gb[O_D + i_]; \
        }
        if (nloop > 0) {
            CKDA_RLOAD_A(0)
            CKDA_RLOAD_B(0)
            CKDA_RSTORE_A()
            CKDA_RSTORE_B()
            CKDA_RLOAD_A(min(1, nloop - 1))
            CKDA_RLOAD_B(min(1, nloop - 1))
        }
        lds_sync();   // record of walk step 0 in LDS
        for (int j = 0; j < nloop; ++j) {
            lds_sync();   // X: KB, MT of step j consumed
            CKDA_RSTORE_A()
            CKDA_RLOAD_A(min(j + 2, nloop - 1))
            lds_sync();   // Y: step j consumed
            CKDA_RSTORE_B()
            CKDA_RLOAD_B(min(j + 2, nloop - 1))
        }
#undef CKDA_RREC
#undef CKDA_RLOAD_A
#undef CKDA_RLOAD_B
#undef CKDA_RSTORE_A
#undef CKDA_RSTORE_B
        return;
    }

    // ================= compute waves ==========================================
    const size_t st_off = (static_cast<size_t>(sidx) * H + h) * DK * DV;
    const bool has_col = w < NWC;
    const int wt = min(w, NWC - 1);
    const int vt = vt0 + wt;
    const int lane = threadIdx.x & 63;

    // G: lane (n, g) holds rows 16rt + 4g + i of column 16vt + n; starts at
    // dht (the chain's end), at the segment's end G (phase 3), at zero (phase
    // 1, middle segments) or at the identity (transition columns)
    f32x4 G[RT];
    {
        const int gq = lane >> 4, col = 16 * vt + (lane & 15);
        const float* src = last ? (p.dht ? p.dht + st_off : nullptr)
                                : (OUT ? p.seg_start + (static_cast<size_t>(ss) * H + h) * DK * DV : nullptr);
        // unconditional loads (a missing source or column reads 0): all in flight at once
        const __amdgpu_buffer_rsrc_t grc = buffer_rsrc(src, (has_col && src && !trans) ? DK * DV * 4 : 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * gq + i;
                const float v = buffer_load_f32(grc, static_cast<uint32_t>(row * DV + col) * 4, 0);
                G[rt][i] = trans ? (row == col ? 1.f : 0.f) : v;
            }
    }
    // dO tiles of walk step jj: lane (n, g) holds rows 16J + 4g + i of column
    // 16vt + n (the C/D layout), zero past the chunk's end; the address is
    // clamped into the chunk so every load is unconditional
    const Tin* dO = static_cast<const Tin*>(p.dout);
    // (buffer loads over the chunk's rows: rows past its end, and every row
    // of a transition slice, read as 0 with no branch, so all 16 are in
    // flight together)
    auto load_do = [&](int jj, f32x4 (&x)[4]) {
        const int c0 = 64 * (jbeg + nloop - 1 - jj);
        const int L = min(64, len - c0);
        const int gq = (opaque_tid() & 63) >> 4, col = 16 * vt + (lane & 15);
        const uint32_t bytes = trans ? 0u : static_cast<uint32_t>(((L - 1) * H + 1) * DV) * sizeof(Tin);
        const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(dO + (static_cast<size_t>(tok0 + c0) * H + h) * DV, bytes);
#pragma unroll
        for (int J = 0; J < 4; ++J)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tt = 16 * J + 4 * gq + i;
                x[J][i] = buffer_load_elem<Tin>(rc, static_cast<uint32_t>((tt * H * DV + col) * sizeof(Tin)), 0);
            }
    };
    f32x4 dn[4];
    if (nloop > 0) load_do(0, dn);
    lds_sync();   // record of step 0 in LDS
    for (int j = 0; j < nloop; ++j) {
        const int jc = jbeg + nloop - 1 - j;   // chunk index within the chain
        const size_t rslot = static_cast<size_t>(slot0 + jc) * H + h;
        f32x4 dOv[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) dOv[J] = dn[J] * p.scale;
        load_do(min(j + 1, nloop - 1), dn);
        {
            unsigned char* const sm = smem + opaque_zero();
            const LdsMat KBm{sm + SH::L_KB, SH::PKB, 64 * SH::PKB};
            const LdsMat MTm{sm + SH::L_MT, SH::PMT, 64 * SH::PMT};
            const LdsMat QTm{sm + SH::L_QT, SH::PQT, DK * SH::PQT};
            const LdsMat WTm{sm + SH::L_WT, SH::PWT, DK * SH::PWT};
            const float* dl = reinterpret_cast<const float*>(sm + SH::L_D);
            const int l = opaque_tid() & 63, n = l & 15, gq = l >> 4;
            const int col = 16 * vt + n;
            if (OUT) {   // G at this chunk's end, for the chunk-parallel pass
                const __amdgpu_buffer_rsrc_t grc = buffer_rsrc(p.G + rslot * DK * DV, has_col ? DK * DV * 4 : 0);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        buffer_store_f32(grc, static_cast<uint32_t>(((16 * rt + 4 * gq + i) * DV + col) * 4), G[rt][i]);
            }
            constexpr int KS = RT / 2;
            // X = KB G (32 channels per k-step, two 16-token row blocks at a
            // time; the next step's fragments are read while these products run)
            typename PR::F8 Gb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) Gb[ks] = PR::regs8(G[2 * ks], G[2 * ks + 1]);
            f32x4 X[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) X[R] = f32x4{0.f, 0.f, 0.f, 0.f};
            {
                constexpr int NSTEP = 2 * KS;
                typename PR::F8 ka[2][2];
#pragma unroll
                for (int r = 0; r < 2; ++r) ka[0][r] = PR::loadA(KBm, 16 * r + n, 0, gq);
#pragma unroll
                for (int st = 0; st < NSTEP; ++st) {
                    const int ks = st / 2, R0 = 2 * (st % 2);
                    if (st + 1 < NSTEP) {
                        const int k1 = 32 * ((st + 1) / 2), R1 = 2 * ((st + 1) % 2);
#pragma unroll
                        for (int r = 0; r < 2; ++r) ka[(st + 1) & 1][r] = PR::loadA(KBm, 16 * (R1 + r) + n, k1, gq);
                    }
                    CKDA_FENCE();
#pragma unroll
                    for (int r = 0; r < 2; ++r) X[R0 + r] = PR::mma8(ka[st & 1][r], Gb[ks], X[R0 + r]);
                    CKDA_FENCE();
                }
            }
            // dU = X + (scale dO)^T-side product M^T (scale dO): rows i of
            // 16-block R take tokens r >= i, i.e. the 32-token steps kt >= R / 2
            // (M^T is zero left of its diagonal, also in the blocks those
            // steps read)
            typename PR::F8 Db[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) Db[kt] = PR::regs8(dOv[2 * kt], dOv[2 * kt + 1]);
            f32x4 dU[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                f32x4 acc = X[R];
#pragma unroll
                for (int kt = R / 2; kt < 2; ++kt) acc = PR::mma8(PR::loadA(MTm, 16 * R + n, 32 * kt, gq), Db[kt], acc);
                dU[R] = acc;
            }
            lds_sync();   // X: KB, MT consumed (the loaders refill them); QT, WT, d in LDS
            if (OUT) {   // dU of this chunk (C/D tiles (R, vt), as u in the forward record)
                float* du = p.dU + rslot * 64 * DV;
                const __amdgpu_buffer_rsrc_t urc = buffer_rsrc(du, has_col ? 64 * DV * 4 : 0);
#pragma unroll
                for (int R = 0; R < 4; ++R)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        buffer_store_f32(urc, static_cast<uint32_t>((((R * (DV / 16) + vt) * 64 + l) * 4 + i) * 4), dU[R][i]);
            }
            // G <- Diag(d) G + Qh^T (scale dO) - W^T dU
            typename PR::F8 Nb[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) Nb[kt] = PR::regs8(-dU[2 * kt], -dU[2 * kt + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const f32x4 dd = *reinterpret_cast<const f32x4*>(dl + 16 * rt + 4 * gq);
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    acc = PR::mma8(PR::loadA(QTm, 16 * rt + n, 32 * kt, gq), Db[kt], acc);
                    acc = PR::mma8(PR::loadA(WTm, 16 * rt + n, 32 * kt, gq), Nb[kt], acc);
                }
                G[rt] = dd * G[rt] + acc;
            }
        }
        lds_sync();   // Y: step j consumed (the loaders refill QT, WT, d)
    }
    // where G at the walk's start goes: dh0 (the chain's start); phase 1: the
    // previous segment's end G (the chain's last segment), H_s or P_s
    float* dst = nullptr;
    size_t pitch = DV;
    if (!SEG || (OUT && seg == 0)) {
        dst = p.dh0 ? p.dh0 + st_off : nullptr;
    } else if (!OUT) {
        if (seg == nseg - 1) {
            dst = p.seg_start + (static_cast<size_t>(ss - 1) * H + h) * DK * DV;
        } else if (trans) {
            dst = p.seg_p + (static_cast<size_t>(ss) * H + h) * DK * DK;
            pitch = DK;
        } else {
            dst = p.seg_h + (static_cast<size_t>(ss) * H + h) * DK * DV;
        }
    }
    if (dst && has_col) {
        const int gq = lane >> 4, col = 16 * vt + (lane & 15);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[opaque_zero() + static_cast<size_t>(16 * rt + 4 * gq + i) * pitch + col] = G[rt][i];
    }
}

template <typename Tin, int DK, int DV, bool SEG, bool OUT>
static hipError_t launch_rev_k(const RevParams& p, long long grid, hipStream_t stream) {
    using SH = RevShape<Tin, DK, DV>;
    if (grid == 0) return hipSuccess;
    auto kern = p.fr ? ckda_rev_kernel<Tin, DK, DV, SEG, OUT, true> : ckda_rev_kernel<Tin, DK, DV, SEG, OUT, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(512), SH::LDS, stream, p);
    return hipGetLastError();
}

// whole chains (p.seg_len == 0) or segments in three launches: phase 1, the
// scan of the segment ends (from the chain's end backwards), phase 3
template <typename Tin, int DK, int DV>
static hipError_t launch_rev_t(const RevParams& p, int nchains, hipStream_t stream) {
    using SH = RevShape<Tin, DK, DV>;
    if (p.seg_len == 0) return launch_rev_k<Tin, DK, DV, false, true>(p, static_cast<long long>(nchains) * SH::NSLICE, stream);
    const long long items = static_cast<long long>(p.nsslots) * p.H;
    hipError_t e = launch_rev_k<Tin, DK, DV, true, false>(p, items * (SH::NSLICE + SH::NTS), stream);
    if (e != hipSuccess) return e;
    const SegScanParams sp{p.cu, p.T, p.H, p.seg_len, p.seg_start, p.seg_h, p.seg_p, 1};
    hipLaunchKernelGGL((ckda_seg_scan_kernel<DK, DV>), dim3(static_cast<unsigned>(nchains * (DV / kScanCols))), dim3(256),
                       0, stream, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_rev_k<Tin, DK, DV, true, true>(p, items * SH::NSLICE, stream);
}

template <typename Tin>
static hipError_t launch_rev_dt(const RevParams& p, int nchains, int DK, int DV, hipStream_t stream) {
#define CKDA_REV(DK_, DV_) \
    if (DK == DK_ && DV == DV_) return launch_rev_t<Tin, DK_, DV_>(p, nchains, stream);
    CKDA_REV(32, 32) CKDA_REV(32, 64) CKDA_REV(32, 128)
    CKDA_REV(64, 32) CKDA_REV(64, 64) CKDA_REV(64, 128)
    CKDA_REV(128, 32) CKDA_REV(128, 64) CKDA_REV(128, 128)
#undef CKDA_REV
    return hipErrorInvalidValue;
}

}  // namespace ckda

namespace ckda {
size_t rev_record_bytes(int DK, int DV, bool bf16) {
#define CKDA_RB(DK_, DV_) \
    if (DK == DK_ && DV == DV_) return bf16 ? RevRecord<DK_, DV_, false>::BYTES : RevRecord<DK_, DV_, true>::BYTES;
    CKDA_RB(32, 32) CKDA_RB(32, 64) CKDA_RB(32, 128)
    CKDA_RB(64, 32) CKDA_RB(64, 64) CKDA_RB(64, 128)
    CKDA_RB(128, 32) CKDA_RB(128, 64) CKDA_RB(128, 128)
#undef CKDA_RB
    return 0;
}

// measured on MI355X (dk = dv = 128, bf16 records), in units of a lone
// chain's chunk-step: about 0.45 workgroup chunk-steps per CU and unit when
// every CU runs one; a phase-1 step (no per-chunk stores) about 0.9 of one;
// a scan step about one unit
constexpr SegCost kRevCost{0.45, 0.9, 1.0};

int rev_segment_plan(const int32_t* cu_host, bool varlen, int ndocs, int B, int T, int H, int DK, int DV,
                     size_t seg_room, hipStream_t stream) {
    const int BV = DV < 64 ? DV : 64;
    auto fits = [&](int G) { return seg_buffer_bytes(seg_slots(varlen, B, T, ndocs, G), H, DK, DV) <= seg_room; };
    return plan_segments(chain_chunks(cu_host, varlen, ndocs, B, T), H, DV / BV, (DK + BV - 1) / BV, kRevCost,
                         device_cus(stream), fits);
}

// reverse pass over nchains chains: records from launch_chunk_rev in p.ws
hipError_t launch_rev(const RevParams& p, int nchains, int DK, int DV, bool bf16, hipStream_t stream) {
    return bf16 ? launch_rev_dt<bf16_t>(p, nchains, DK, DV, stream) : launch_rev_dt<float>(p, nchains, DK, DV, stream);
}
}  // namespace ckda
