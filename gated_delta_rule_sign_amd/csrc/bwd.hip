// bwd.hip -- CKDA backward: gradients of L = <do, o> + <dht, ht> through the
// chunked forward.
//
// Chunk-level reverse mode of the WY/UT form (Complex KDA paper page,
// section 2: WY-based chunk-wise implementations; the training backward
// itself is specified in an appendix missing from the pages, so the gradient
// here is the plain derivative of the forward: no gradient flows to the
// sign s, and dg = alpha * dL/dalpha for g = log|alpha|).
//
// Per chunk (64 tokens, chunk-local sign fold, anchor m = b at token 31):
//   K1 = kf e^{b-m}, K2 = kf e^{m-b}, Q1 = qf e^{b-m}, KB = kf e^{b_L-b}
//   A = strict_lower(K1 K2^T), M = lower(Q1 K2^T), X = I + Diag(beta) A,
//   Xi = X^{-1}, T = Xi Diag(beta), S' = Diag(e^m) S, U = T (V - K1 S')
// Reverse recurrence over chunks (the only sequential part), G = dL/dS at the
// chunk end in the true frame, dSt = Diag(P_L) G:
//   dU = M^T dO + KB dSt,  Z = T^T dU,
//   G_prev = Diag(e^m) (Q1^T dO - K1^T Z) + Diag(e^{b_L}) dSt
// Chunk-parallel gradients:
//   dM = lower(dO U^T), dKB = U dSt^T, dW' = -dU S'^T, dV = T^T dU,
//   dT = dU V^T + dW' K1^T, dK1 = T^T dW', dbeta1_i = sum_r dT_ri Xi_ri,
//   dX = -Xi^T (dT Diag(beta)) Xi^T, dXs = strict_lower(dX),
//   dbeta2_r = sum_i dXs_ri A_ri, dA = Diag(beta) dXs,
//   dK1 += dA K2, dK2 = dA^T K1 + dM^T Q1, dQ1 = dM K2 + dO S'^T,
//   dq~ = dQ1 e^{b-m}, dk~ = dK1 e^{b-m} + dK2 e^{m-b} + dKB e^{b_L-b},
//   db = Q1 dQ1 + K1 dK1 - K2 dK2 - KB dKB (+ sum(KB dKB) + e^{b_L} sum_v dSt S
//   at the chunk's last token), dg = reverse cumulative sum of db,
//   dq = P dq~, dk = P dk~.
//
// Implementation: every product is a batched fp32 matrix-core GEMM
// (v_mfma_f32_16x16x4_f32) over all chunk-heads at once, with intermediates
// in the caller's workspace; the reverse recurrence runs one workgroup per
// (sequence, head, 64-column slice) over the chunks, its operands staged in LDS.
#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_mfma.h"
#include "ckda_record.h"
#include "ckda_segments.h"

namespace ckda {

namespace {

// Workspace layout (floats), per chunk-head ch (NC = B*H*NT of them).
struct BwdWs {
    int NC, DK, DV;
    float* base;
    // [NC][64][DK]
    float *K1, *K2, *Q1, *KB, *dKB, *dW, *dK1, *dK2, *dQ1;
    // [NC][64][DV]
    float *V, *dO, *R, *U, *dU, *dV;
    // [NC][DK][DV]
    float* dSt;
    // [NC][64][64]
    float *A, *M, *Xi, *T, *dM, *dT, *Y1, *Tmp, *dX, *dA;
    // [NC][DK]
    float *em, *gC, *pC;
    // [NC][64]
    float *beta, *dbeta1, *dbeta2;

    __host__ __device__ static size_t floats(size_t NC, int DK, int DV) {
        return NC * (9ull * 64 * DK + 6ull * 64 * DV + 1ull * DK * DV + 10ull * 64 * 64 + 3ull * DK + 3ull * 64);
    }
    __host__ void carve(float* p, int nc, int dk, int dv) {
        NC = nc; DK = dk; DV = dv; base = p;
        const size_t n = nc;
        auto take = [&](size_t cnt) { float* r = p; p += cnt; return r; };
        K1 = take(n * 64 * dk); K2 = take(n * 64 * dk); Q1 = take(n * 64 * dk); KB = take(n * 64 * dk);
        dKB = take(n * 64 * dk); dW = take(n * 64 * dk);
        dK1 = take(n * 64 * dk); dK2 = take(n * 64 * dk); dQ1 = take(n * 64 * dk);
        V = take(n * 64 * dv); dO = take(n * 64 * dv); R = take(n * 64 * dv); U = take(n * 64 * dv);
        dU = take(n * 64 * dv); dV = take(n * 64 * dv);
        dSt = take(n * dk * dv);
        A = take(n * 4096); M = take(n * 4096); Xi = take(n * 4096); T = take(n * 4096); dM = take(n * 4096);
        dT = take(n * 4096); Y1 = take(n * 4096); Tmp = take(n * 4096); dX = take(n * 4096); dA = take(n * 4096);
        em = take(n * dk); gC = take(n * dk); pC = take(n * dk);
        beta = take(n * 64); dbeta1 = take(n * 64); dbeta2 = take(n * 64);
    }
};

// ---------------------------------------------------------------------------
// batched GEMM: for every batch element z (chunk-head),
//   C_z(i,j) = alpha * sum_k A_z(i,k) B_z(k,j) + beta * D_z(i,j)   (then mask)
// A_z(i,k) = A[z*sA + i*ar + k*ac], etc.; mask 1: keep j < i, 2: keep j <= i.
// ---------------------------------------------------------------------------
struct Gemm {
    int M, N, K;
    const float* A; long long sA; int ar, ac;
    const float* B; long long sB; int br, bc;
    float* C; long long sC; int cr;
    const float* D; long long sD; int dr;
    float alpha, beta;
    int mask;
    // optional scale of B's stored rows (row r of the stored matrix times
    // bs[z * sBs + r]: Diag(bs) B for B read as stored, B Diag(bs) for B
    // read transposed), applied while the slab is staged
    const float* bs; long long sBs;
    // C of batch element z: C + z sC, or with cn1 > 0 the three-level
    // decomposition z = (z2 cn2 + z1) cn1 + z0 -> C + z0 sC + z1 cs1 + z2 cs2
    // (a chunk-head's rows straight into a [B,T,H,D] output)
    int cn1, cn2; long long cs1, cs2;
};

// One workgroup per batch element: C (64 x N) = A (64 x K) B (K x N), N, K in
// {32, 64, 128}.  K is processed in slabs of 32: both operands of a slab are
// read with coalesced 16-byte loads into LDS in the layout their storage
// gives (row-major or transposed), then wave w forms rows 16w..16w+15 for all
// N/16 column tiles, so each A fragment serves every tile of the row block.
// About 28 KB of LDS, so several workgroups share a CU and hide each other's
// load latency.
constexpr int kKS = 32;          // slab width (K)
constexpr int kPK = kKS + 4;     // pitch of rows that run along K
constexpr int kPN = 64 + 4;      // pitch of rows that run along M or N (64-wide blocks)


// acc += sa * A_z B_z over the product's K (aT: A stored transposed, bT: B
// stored transposed, NT = N / 16).  Both operands go through LDS in 32-wide
// K slabs in the layout their storage gives; the next slab is read into
// registers (16-byte units, coalesced along rows) while the current one is
// multiplied.
template <bool aT, bool bT, int NT>
__device__ __forceinline__ void bgemm_accumulate(const Gemm& p, long long z, float sa, f32x4 (&acc)[NT], float* As,
                                                 float* Bs) {
    constexpr int NB = NT / 2 > 0 ? NT / 2 : 1;   // B units per thread (A: 2)
    const float* A = p.A + z * p.sA;
    const float* B = p.B + z * p.sB;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, n = l & 15, g = l >> 4;
    // unit e of a slab -> (row, 4-column group) of the staged block
    auto a_src = [&](int e, int k0) -> const float* {
        if constexpr (!aT) return A + static_cast<size_t>(e / 8) * p.ar + k0 + 4 * (e % 8);   // As[i][k], 64 x 32
        else return A + static_cast<size_t>(k0 + e / 16) * p.ac + 4 * (e % 16);              // As[k][i], 32 x 64
    };
    auto a_dst = [&](int e) -> float* {
        if constexpr (!aT) return As + (e / 8) * kPK + 4 * (e % 8);
        else return As + (e / 16) * kPN + 4 * (e % 16);
    };
    // B: bT -> Bs[j][k] (16 NT x 32); else Bs[k][j] in 64-wide blocks of j
    constexpr int BW = 16 * NT < 64 ? 16 * NT : 64;   // block width (not transposed)
    auto b_src = [&](int e, int k0) -> const float* {
        if constexpr (bT) return B + static_cast<size_t>(e / 8) * p.bc + k0 + 4 * (e % 8);
        else {
            const int blk = e / (32 * BW / 4), u = e % (32 * BW / 4);
            return B + static_cast<size_t>(k0 + u / (BW / 4)) * p.br + 64 * blk + 4 * (u % (BW / 4));
        }
    };
    auto b_dst = [&](int e) -> float* {
        if constexpr (bT) return Bs + (e / 8) * kPK + 4 * (e % 8);
        else {
            const int blk = e / (32 * BW / 4), u = e % (32 * BW / 4);
            return Bs + blk * kKS * kPN + (u / (BW / 4)) * kPN + 4 * (u % (BW / 4));
        }
    };
    f32x4 ra[2], rb[NB];
    float rs[NB];
    const float* bs = p.bs ? p.bs + z * p.sBs : nullptr;
    // stored row of B unit e: j (B read transposed) or k (as stored)
    auto b_row = [&](int e, int k0) -> int {
        if constexpr (bT) return e / 8;
        else return k0 + (e % (32 * BW / 4)) / (BW / 4);
    };
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) ra[i] = *reinterpret_cast<const f32x4*>(a_src(tid + 256 * i, k0));
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            rb[i] = *reinterpret_cast<const f32x4*>(b_src(tid + 256 * i, k0));
            rs[i] = bs ? bs[b_row(tid + 256 * i, k0)] : 1.f;
        }
    };
    load(0);
    for (int k0 = 0; k0 < p.K; k0 += kKS) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<f32x4*>(a_dst(tid + 256 * i)) = ra[i];
#pragma unroll
        for (int i = 0; i < NB; ++i) *reinterpret_cast<f32x4*>(b_dst(tid + 256 * i)) = rs[i] * rb[i];
        __syncthreads();
        if (k0 + kKS < p.K) load(k0 + kKS);
#pragma unroll 2
        for (int kk = 0; kk < kKS; kk += 4) {
            const int i = 16 * w + n, k = kk + g;
            const float a = sa * (aT ? As[k * kPN + i] : As[i * kPK + k]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int j = 16 * t + n;
                const float b = bT ? Bs[j * kPK + k] : Bs[(t / 4) * kKS * kPN + k * kPN + (j % 64)];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
    }
}

// C = p.alpha * (A1 B1 + (q.alpha / p.alpha) A2 B2) + p.beta * D, masked;
// the second product only when DUAL
template <bool aT, bool bT, int NT, bool DUAL = false, bool aT2 = false, bool bT2 = false>
__global__ void __launch_bounds__(256, 4) bgemm_kernel(Gemm p, Gemm q) {
    __shared__ __align__(16) float As[64 * kPK > kKS * kPN ? 64 * kPK : kKS * kPN];
    __shared__ __align__(16) float Bs[128 * kPK > 2 * kKS * kPN ? 128 * kPK : 2 * kKS * kPN];
    const long long z = blockIdx.x;
    float* C = p.cn1 > 0 ? p.C + (z % p.cn1) * p.sC + ((z / p.cn1) % p.cn2) * p.cs1 +
                               (z / (static_cast<long long>(p.cn1) * p.cn2)) * p.cs2
                         : p.C + z * p.sC;
    const float* D = p.D ? p.D + z * p.sD : nullptr;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    bgemm_accumulate<aT, bT, NT>(p, z, 1.f, acc, As, Bs);
    if constexpr (DUAL) bgemm_accumulate<aT2, bT2, NT>(q, z, q.alpha / p.alpha, acc, As, Bs);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * g + r, j = 16 * t + n;
            float val = p.alpha * acc[t][r];
            if (D) val += p.beta * D[i * p.dr + j];
            if (p.mask == 1 && j >= i) val = 0.f;
            if (p.mask == 2 && j > i) val = 0.f;
            C[i * p.cr + j] = val;
        }
    }
}

static bool gemm_shape_ok(const Gemm& g) {
    // shapes used by the backward: M = 64, N and K in {32, 64, 128}
    auto ok = [](int x) { return x == 32 || x == 64 || x == 128; };
    return g.M == 64 && ok(g.N) && ok(g.K);
}

hipError_t gemm(const Gemm& g, int nbatch, hipStream_t st) {
    if (!gemm_shape_ok(g)) return hipErrorInvalidValue;
    const bool aT = g.ar == 1, bT = g.bc != 1;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(nbatch), dim3(256), 0, st, g, g); };
#define CKDA_GEMM_N(AT, BT)                                                  \
    if (g.N == 32) go(bgemm_kernel<AT, BT, 2>);                              \
    else if (g.N == 64) go(bgemm_kernel<AT, BT, 4>);                         \
    else go(bgemm_kernel<AT, BT, 8>);
    if (aT && bT) { CKDA_GEMM_N(true, true) }
    else if (aT) { CKDA_GEMM_N(true, false) }
    else if (bT) { CKDA_GEMM_N(false, true) }
    else { CKDA_GEMM_N(false, false) }
#undef CKDA_GEMM_N
    return hipGetLastError();
}

// C = g.alpha A1 B1 + h.alpha A2 B2 (+ g.beta D) into g's output; the operand
// layouts of the pairs the backward fuses
hipError_t gemm2(const Gemm& g, const Gemm& h, int nbatch, hipStream_t st) {
    if (!gemm_shape_ok(g) || !gemm_shape_ok(h) || g.N != h.N || g.alpha == 0.f) return hipErrorInvalidValue;
    const bool a1 = g.ar == 1, b1 = g.bc != 1, a2 = h.ar == 1, b2 = h.bc != 1;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(nbatch), dim3(256), 0, st, g, h); };
#define CKDA_GEMM2(A1, B1, A2, B2)                                                   \
    if (a1 == A1 && b1 == B1 && a2 == A2 && b2 == B2) {                              \
        if (g.N == 32) go(bgemm_kernel<A1, B1, 2, true, A2, B2>);                    \
        else if (g.N == 64) go(bgemm_kernel<A1, B1, 4, true, A2, B2>);               \
        else go(bgemm_kernel<A1, B1, 8, true, A2, B2>);                              \
        return hipGetLastError();                                                    \
    }
    CKDA_GEMM2(false, true, false, true)     // dT = dU V^T + dW K1^T
    CKDA_GEMM2(true, false, false, false)    // dK1 = T^T dW + dA K2
    CKDA_GEMM2(true, false, true, false)     // dK2 = dA^T K1 + dM^T Q1
    CKDA_GEMM2(false, false, false, true)    // dQ1 = dM K2 + dO S'^T
#undef CKDA_GEMM2
    return hipErrorInvalidValue;
}

// C = alpha * op(A) op(B) (+ beta * D), all operands [NC][rows][cols] row-major.
// tA/tB: use the transpose of the stored matrix.
Gemm mk(int M, int N, int K, const float* A, int lda, long long sA, bool tA, const float* B, int ldb,
        long long sB, bool tB, float* C, int ldc, long long sC, float alpha = 1.f, const float* D = nullptr,
        float beta = 0.f, int mask = 0) {
    Gemm g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.sA = sA; g.ar = tA ? 1 : lda; g.ac = tA ? lda : 1;
    g.B = B; g.sB = sB; g.br = tB ? 1 : ldb; g.bc = tB ? ldb : 1;
    g.C = C; g.sC = sC; g.cr = ldc;
    g.D = D; g.sD = sC; g.dr = ldc;
    g.alpha = alpha; g.beta = beta; g.mask = mask;
    return g;
}

struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *g, *beta;
    const int8_t* s;
    const float *h_ckpt, *dht, *h0;
    float scale;
    float *dq, *dk, *dv, *dg, *dbeta, *dh0;
    int B, T, H, NT;
    const int32_t* cu;   // varlen document starts (device), or nullptr
    int ndocs;
    bool head_gate;      // g, s, dg per (token, head)
    bool qk_norm;        // q, k L2-normalised per (token, head) inside the path
    bool dv_direct;      // the dV products wrote dv itself (equal-length, whole chunks)
    // segmented reverse pass: G chunks per segment, buffers as in
    // ckda_segments.h (start = the dS entering a segment from its later end)
    int G, nsslots;
    float *seg_start, *seg_h, *seg_p;
};

// chunk-head ch -> (head, token row of the chunk start, valid tokens).
// Equal-length: ch = (b H + h) NT + j.  Varlen: ch = slot H + h, chunk j of
// document d in slot floor(cu[d]/64) + d + j (unused slots have L = 0).
// Checkpoints and workspace rows are indexed by ch in both modes.
struct ChunkIdx {
    int h, L;
    size_t trow0;
    __device__ ChunkIdx(int ch, const BwdParams& p) {
        if (p.cu) {
            const int slot = ch / p.H;
            h = ch % p.H;
            int lo = 0, hi = p.ndocs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (varlen_slot(p.cu[mid], mid, 0) <= slot) lo = mid; else hi = mid - 1;
            }
            const int j = slot - varlen_slot(p.cu[lo], lo, 0);
            const int len = p.cu[lo + 1] - p.cu[lo];
            trow0 = static_cast<size_t>(__builtin_amdgcn_readfirstlane(p.cu[lo] + 64 * j));
            L = __builtin_amdgcn_readfirstlane(max(0, min(64, len - 64 * j)));
        } else {
            const int j = ch % p.NT, bh = ch / p.NT;
            h = bh % p.H;
            trow0 = static_cast<size_t>(bh / p.H) * p.T + 64 * j;
            L = min(64, p.T - 64 * j);
        }
    }
};

// ---------------------------------------------------------------------------
// Chunk-local scans shared by the prep and final passes.  Thread layout: 4
// consecutive channels (a "quad") by a segment of NTOK consecutive tokens;
// a wave covers whole 512-byte token rows.  Every load is issued up front
// (rows past the chunk end read the last token and are masked at use), the
// per-segment inclusive scans meet through LDS, and
//   b = cumulative g (natural log),  P = cumulative sign product,
//   m = b at token 31 (the anchor),  bL = b at the last token,
// padding tokens carrying g = 0 and s = +1 (so m = b[min(31, L-1)]).
// ---------------------------------------------------------------------------
template <int DK, int NTHR>
struct QuadSeg {
    static constexpr int CQ = DK / 4;          // channel quads
    static constexpr int SEGS = NTHR / CQ;     // token segments
    static constexpr int NTOK = 64 / SEGS;     // tokens per thread
    static_assert(SEGS * NTOK == 64 && SEGS % 2 == 0, "segments");
};

template <typename T> __device__ __forceinline__ f32x4 load_quad(const T* p, size_t e);
template <> __device__ __forceinline__ f32x4 load_quad<float>(const float* p, size_t e) {
    return *reinterpret_cast<const f32x4*>(p + e);
}
template <> __device__ __forceinline__ f32x4 load_quad<bf16_t>(const bf16_t* p, size_t e) {
    const u32x2 u = *reinterpret_cast<const u32x2*>(p + e);
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                 __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 signs_quad(const int8_t* p, size_t e) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p + e);
    return f32x4{static_cast<float>(static_cast<int8_t>(u)), static_cast<float>(static_cast<int8_t>(u >> 8)),
                 static_cast<float>(static_cast<int8_t>(u >> 16)), static_cast<float>(static_cast<int8_t>(u >> 24))};
}
// g and s of token row `row` (chunk token t), channels 4 q4 .. +3: per channel,
// or (HG) the head's one gate broadcast
template <bool HG>
__device__ __forceinline__ void gate_quad(const BwdParams& p, size_t row, int h, int DK, int q4, f32x4& gq,
                                          f32x4& sq) {
    if constexpr (HG) {
        const size_t e = row * p.H + h;
        const float gt = p.g[e], st = static_cast<float>(p.s[e]);
        gq = f32x4{gt, gt, gt, gt};
        sq = f32x4{st, st, st, st};
    } else {
        const size_t e = (row * p.H + h) * DK + 4 * q4;
        gq = *reinterpret_cast<const f32x4*>(p.g + e);
        sq = signs_quad(p.s, e);
    }
}

// sum of x over the CQ quads of one token row (adjacent lanes, CQ <= 32)
template <int CQ>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int o = 1; o < CQ; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }
// x <- x / ||x|| per token row (every lane of the row calls it), inv <- 1 / ||x||
template <int CQ, int NTOK>
__device__ __forceinline__ void normalise_rows(f32x4 (&x)[NTOK], float (&inv)[NTOK]) {
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        inv[i] = inv_norm(row_sum<CQ>(dot4(x[i], x[i])));
        x[i] *= inv[i];
    }
}

__device__ __forceinline__ f32x4 exp2c4(f32x4 x) {
    return f32x4{exp2_clamped(x[0]), exp2_clamped(x[1]), exp2_clamped(x[2]), exp2_clamped(x[3])};
}

// prep: cumulative gate and sign product, anchored operands, V / dO copies
template <typename Tin, int DK, int DV, bool HG, bool NQK>
__global__ void __launch_bounds__(512) bwd_prep_kernel(BwdParams p, BwdWs W) {
    using QS = QuadSeg<DK, 512>;
    using QV = QuadSeg<DV, 512>;
    constexpr int CQ = QS::CQ, SEGS = QS::SEGS, NTOK = QS::NTOK;
    __shared__ f32x4 segb[SEGS][CQ], segp[SEGS][CQ];
    const int ch = blockIdx.x;
    const ChunkIdx ci(ch, p);
    const int tid = threadIdx.x, q4 = tid % CQ, seg = tid / CQ, tb = seg * NTOK;
    const size_t trow0 = ci.trow0;   // token row of the chunk start
    const size_t o64k = static_cast<size_t>(ch) * 64 * DK;
    const size_t o64v = static_cast<size_t>(ch) * 64 * DV;
    if (ci.L <= 0) {   // unused varlen slot: zero operands, so every later pass stays finite
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        for (int u = tid; u < 16 * DK; u += 512) {
            reinterpret_cast<f32x4*>(W.K1 + o64k)[u] = z;
            reinterpret_cast<f32x4*>(W.K2 + o64k)[u] = z;
            reinterpret_cast<f32x4*>(W.Q1 + o64k)[u] = z;
            reinterpret_cast<f32x4*>(W.KB + o64k)[u] = z;
        }
        for (int u = tid; u < 16 * DV; u += 512) {
            reinterpret_cast<f32x4*>(W.V + o64v)[u] = z;
            reinterpret_cast<f32x4*>(W.dO + o64v)[u] = z;
        }
        if (tid < 64) W.beta[static_cast<size_t>(ch) * 64 + tid] = 0.f;
        if (tid < DK) {
            W.em[static_cast<size_t>(ch) * DK + tid] = 1.f;
            W.gC[static_cast<size_t>(ch) * DK + tid] = 1.f;
            W.pC[static_cast<size_t>(ch) * DK + tid] = 1.f;
        }
        return;
    }
    const Tin* qp = static_cast<const Tin*>(p.q);
    const Tin* kp = static_cast<const Tin*>(p.k);
    f32x4 gv[NTOK], sg[NTOK], kv[NTOK], qv[NTOK];
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const size_t row = trow0 + min(tb + i, ci.L - 1);
        const size_t e = (row * p.H + ci.h) * DK + 4 * q4;
        gate_quad<HG>(p, row, ci.h, DK, q4, gv[i], sg[i]);
        kv[i] = load_quad(kp, e);
        qv[i] = load_quad(qp, e);
    }
    const int qv4 = tid % QV::CQ, segv = tid / QV::CQ;
    f32x4 vv[QV::NTOK], dd[QV::NTOK];
#pragma unroll
    for (int i = 0; i < QV::NTOK; ++i) {
        const size_t e = ((trow0 + min(segv * QV::NTOK + i, ci.L - 1)) * p.H + ci.h) * DV + 4 * qv4;
        vv[i] = load_quad(static_cast<const Tin*>(p.v), e);
        dd[i] = load_quad(static_cast<const Tin*>(p.dout), e);
    }
    f32x4 run = {0.f, 0.f, 0.f, 0.f}, par = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const bool valid = tb + i < ci.L;
        run += valid ? gv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        par *= valid ? sg[i] : f32x4{1.f, 1.f, 1.f, 1.f};
        gv[i] = run;
        sg[i] = par;
        if (!valid) kv[i] = qv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (NQK) {
        float ik[NTOK], iq[NTOK];
        normalise_rows<CQ>(kv, ik);
        normalise_rows<CQ>(qv, iq);
    }
    segb[seg][q4] = run;
    segp[seg][q4] = par;
    __syncthreads();
    f32x4 off = {0.f, 0.f, 0.f, 0.f}, poff = {1.f, 1.f, 1.f, 1.f}, m = off, bL = off, ptot = poff;
#pragma unroll 2
    for (int s2 = 0; s2 < SEGS; ++s2) {
        const f32x4 x = segb[s2][q4], y = segp[s2][q4];
        if (s2 < seg) { off += x; poff *= y; }
        if (s2 < SEGS / 2) m += x;
        bL += x;
        ptot *= y;
    }
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const int t = tb + i;
        const f32x4 b = gv[i] + off, P = sg[i] * poff;
        const f32x4 kf = P * kv[i], qf = P * qv[i];
        const f32x4 e1 = exp2c4((b - m) * kLog2e);
        const size_t o = o64k + static_cast<size_t>(t) * DK + 4 * q4;
        *reinterpret_cast<f32x4*>(W.K1 + o) = kf * e1;
        *reinterpret_cast<f32x4*>(W.K2 + o) = kf * exp2c4((m - b) * kLog2e);
        *reinterpret_cast<f32x4*>(W.Q1 + o) = qf * e1;
        *reinterpret_cast<f32x4*>(W.KB + o) = kf * exp2c4((bL - b) * kLog2e);
    }
    if (seg == 0) {
        const f32x4 em = exp2c4(m * kLog2e);
        *reinterpret_cast<f32x4*>(W.em + static_cast<size_t>(ch) * DK + 4 * q4) = em;
        *reinterpret_cast<f32x4*>(W.gC + static_cast<size_t>(ch) * DK + 4 * q4) = exp2c4(bL * kLog2e);
        *reinterpret_cast<f32x4*>(W.pC + static_cast<size_t>(ch) * DK + 4 * q4) = ptot;
    }
#pragma unroll
    for (int i = 0; i < QV::NTOK; ++i) {
        const int t = segv * QV::NTOK + i;
        const bool valid = t < ci.L;
        const size_t o = o64v + static_cast<size_t>(t) * DV + 4 * qv4;
        *reinterpret_cast<f32x4*>(W.V + o) = valid ? vv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(W.dO + o) = valid ? p.scale * dd[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (tid < 64) W.beta[static_cast<size_t>(ch) * 64 + tid] = (tid < ci.L) ? p.beta[(trow0 + tid) * p.H + ci.h] : 0.f;
}

// ---------------------------------------------------------------------------
// Xi = (I + Diag(beta) A)^{-1} (unit lower triangular) and T = Xi Diag(beta):
// 16x16 diagonal blocks by forward substitution, off-diagonal blocks by
// Xi_IJ = -Xi_II sum_{K=J}^{I-1} X_IK Xi_KJ.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_inverse_kernel(BwdWs W) {
    __shared__ float X[64][65];
    __shared__ float Y[64][65];
    __shared__ float Tm[16][17];
    const int ch = blockIdx.x;
    const float* A = W.A + static_cast<size_t>(ch) * 4096;
    const float* bt = W.beta + static_cast<size_t>(ch) * 64;
    for (int e = threadIdx.x; e < 4096; e += 256) {
        const int r = e / 64, i = e % 64;
        X[r][i] = (i < r) ? bt[r] * A[e] : 0.f;
        Y[r][i] = 0.f;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        const int J = threadIdx.x / 16, c = threadIdx.x % 16;
        float y[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= X[16 * J + r][16 * J + i] * y[i];
            y[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Y[16 * J + r][16 * J + c] = y[r];
    }
    __syncthreads();
    const int r = threadIdx.x / 16, c = threadIdx.x % 16;
    for (int d = 1; d < 4; ++d) {
        for (int J = 0; J + d < 4; ++J) {
            const int I = J + d;
            float acc = 0.f;
            for (int K = J; K < I; ++K)
                for (int k = 0; k < 16; ++k) acc += X[16 * I + r][16 * K + k] * Y[16 * K + k][16 * J + c];
            Tm[r][c] = acc;
            __syncthreads();
            float o = 0.f;
            for (int k = 0; k < 16; ++k) o -= Y[16 * I + r][16 * I + k] * Tm[k][c];
            Y[16 * I + r][16 * J + c] = o;
            __syncthreads();
        }
    }
    float* Xi = W.Xi + static_cast<size_t>(ch) * 4096;
    float* T = W.T + static_cast<size_t>(ch) * 4096;
    for (int e = threadIdx.x; e < 4096; e += 256) {
        const int rr = e / 64, i = e % 64;
        Xi[e] = Y[rr][i];
        T[e] = Y[rr][i] * bt[i];
    }
}

// ---------------------------------------------------------------------------
// Reverse recurrence over chunks, one 512-thread workgroup per (sequence,
// head, BV-column slice), BV = min(DV, 64).  Per chunk j (last to first), with
// G = dL/dS at the chunk end and dSt = Diag(pC) G:
//   dU = M^T dO + KB dSt,   Z = T^T dU,
//   G <- Diag(e^m) (Q1^T dO - K1^T Z) + Diag(e^{b_L}) dSt.
// Every operand is staged in LDS (fp32, rows padded so the fragment reads of
// v_mfma_f32_16x16x4_f32 are free of bank conflicts); G lives in LDS and is
// updated in place.  The chunk's Q1, K1 are read into registers while dU and
// Z are formed, and the next chunk's M, T, KB, dO while G is formed, so HBM
// latency hides behind the products.
// ---------------------------------------------------------------------------
// The work of one reverse-pass workgroup: its chain (bh = b H + h, or
// document H + h), value slice (or, segmented phase 1, slice of P_s's
// columns), and the chunks it walks, jbeg .. jend - 1 from the end.  NS
// slices per item: the value slices, then (phase 1) the transition slices.
struct RevWork {
    int bh, hh, seg, ss, nseg, v0, NT, slot0, jbeg, jend;
    bool trans, run;
    __device__ size_t chj(const BwdParams& p, int j) const {   // chunk j -> chunk-head
        return p.cu ? static_cast<size_t>(slot0 + j) * p.H + hh : static_cast<size_t>(bh) * NT + j;
    }
};
template <bool SEG, bool OUT>
__device__ __forceinline__ RevWork rev_work(const BwdParams& p, int NSL, int NS, int BV) {
    RevWork r{};
    const int item = blockIdx.x / NS, slice = blockIdx.x % NS;
    r.hh = item % p.H;
    if (!SEG) {
        r.bh = item;
    } else {
        r.ss = item / p.H;
        int d;
        if (p.cu) {
            int lo = 0, hi = p.ndocs - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seg_slot0(p.cu[mid], mid, p.G) <= r.ss) lo = mid; else hi = mid - 1;
            }
            d = lo;
            r.seg = r.ss - seg_slot0(p.cu[lo], lo, p.G);
        } else {
            const int nsegT = (p.NT + p.G - 1) / p.G;
            d = r.ss / nsegT;
            r.seg = r.ss - d * nsegT;
        }
        r.bh = d * p.H + r.hh;
    }
    r.trans = SEG && slice >= NSL;
    r.v0 = (r.trans ? slice - NSL : slice) * BV;
    if (p.cu) {
        const int d = r.bh / p.H;
        r.NT = __builtin_amdgcn_readfirstlane((p.cu[d + 1] - p.cu[d] + 63) / 64);
        r.slot0 = __builtin_amdgcn_readfirstlane(varlen_slot(p.cu[d], d, 0));
    } else {
        r.NT = p.NT;
    }
    r.jbeg = 0; r.jend = r.NT; r.nseg = 1; r.run = true;
    if (SEG) {
        r.nseg = (r.NT + p.G - 1) / p.G;
        // phase 3: every segment; phase 1: all but the chain's first (the
        // pass's last), transition slices only for the middle ones
        r.run = OUT ? r.seg < max(r.nseg, 1) : (r.seg > 0 && r.seg < r.nseg && (r.seg < r.nseg - 1 || !r.trans));
        r.jbeg = r.seg * p.G;
        r.jend = min(r.NT, r.jbeg + p.G);
    }
    return r;
}

template <int DK, int DV>
struct RevShape {
    static constexpr int BV = DV < 64 ? DV : 64;
    static constexpr int NSL = DV / BV;
    static constexpr int NTS = (DK + BV - 1) / BV;   // transition slices (segmented pass)
    static constexpr int CT = BV / 16;               // column tiles
    // pitches (floats): rows read as "k = lane group" need 16 mod 64, rows
    // read as "row = lane % 16" need 4 mod 64
    static constexpr int P64 = 64 + 16;              // M, T (64 x 64, read transposed)
    static constexpr int PKB = DK + 4;               // KB (64 x DK, row = token)
    static constexpr int PQK = DK + 16;              // Q1, K1 (64 x DK, read transposed)
    static constexpr int PV = BV + 16;               // dO, G, dU, Z (row = k)
    static constexpr int S1 = 2 * 64 * P64 + 64 * PKB;   // stage 1 of the shared region: M, T, KB
    static constexpr int S2 = 2 * 64 * PQK;              // stage 2: Q1, K1
    static constexpr int L_X = 0;
    static constexpr int L_DO = L_X + (S1 > S2 ? S1 : S2);
    static constexpr int L_G = L_DO + 64 * PV;
    static constexpr int L_UZ = L_G + DK * PV;
    static constexpr int L_SM = L_UZ + 64 * PV;      // pC, em, gC
    static constexpr int FLOATS = L_SM + 3 * DK;
    static constexpr int BYTES = FLOATS * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    // 16-byte units each thread moves per chunk
    static constexpr int NM = 64 * 64 / 4 / 512;     // M and T: 2 each
    static constexpr int NKB = 64 * DK / 4 / 512;    // KB, Q1, K1
    static constexpr int NDO = 64 * BV / 4 / 512;    // dO slice
    static_assert(NKB >= 1 && NDO >= 1, "units");
};

// SEG: segmented pass (ckda_segments.h), phase 3 with OUT (dSt, dU and dh0
// written), phase 1 without (segment maps only); otherwise one workgroup
// walks a whole chain's value slice.  In the reverse pass the first segment
// is the chain's last (it starts from dht).
template <int DK, int DV, bool SEG, bool OUT>
__global__ void __launch_bounds__(512) bwd_reverse_kernel(BwdParams p, BwdWs W) {
    using SH = RevShape<DK, DV>;
    constexpr int BV = SH::BV, CT = SH::CT, NM = SH::NM, NKB = SH::NKB, NDO = SH::NDO;
    constexpr int P64 = SH::P64, PKB = SH::PKB, PQK = SH::PQK, PV = SH::PV;
    extern __shared__ __align__(16) float lds[];
    float* const Xs = lds + SH::L_X;
    float* const Ms = Xs;                      // stage 1
    float* const Ts = Xs + 64 * P64;
    float* const KBs = Xs + 2 * 64 * P64;
    float* const Q1s = Xs;                     // stage 2
    float* const K1s = Xs + 64 * PQK;
    float* const dOs = lds + SH::L_DO;
    float* const Gs = lds + SH::L_G;
    float* const UZs = lds + SH::L_UZ;
    float* const pCs = lds + SH::L_SM;
    float* const ems = pCs + DK;
    float* const gCs = ems + DK;

    constexpr int NS = (SEG && !OUT) ? SH::NSL + SH::NTS : SH::NSL;
    const RevWork rw = rev_work<SEG, OUT>(p, SH::NSL, NS, BV);
    if (!rw.run) return;   // the whole workgroup, before any barrier
    const int bh = rw.bh, hh = rw.hh, seg = rw.seg, ss = rw.ss, nseg = rw.nseg, v0 = rw.v0, jbeg = rw.jbeg,
              jend = rw.jend;
    const bool trans = rw.trans;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, n = l & 15, g = l >> 4;
    auto chj = [&](int j) -> size_t { return rw.chj(p, j); };

    // ---- register staging ---------------------------------------------------
    f32x4 rM[NM], rT[NM], rKB[NKB], rDO[NDO], rSM;
    f32x4 rQ[NKB], rK[NKB];
    const int vl0 = trans ? 0 : v0;   // dO columns staged (transition slices zero them)
    auto load1 = [&](int j) {   // M, T, KB, dO slice, pC / em / gC of chunk j
        const size_t ch = chj(j);
        const f32x4* M4 = reinterpret_cast<const f32x4*>(W.M + ch * 4096);
        const f32x4* T4 = reinterpret_cast<const f32x4*>(W.T + ch * 4096);
        const f32x4* KB4 = reinterpret_cast<const f32x4*>(W.KB + ch * 64 * DK);
#pragma unroll
        for (int i = 0; i < NM; ++i) { rM[i] = M4[tid + 512 * i]; rT[i] = T4[tid + 512 * i]; }
#pragma unroll
        for (int i = 0; i < NKB; ++i) rKB[i] = KB4[tid + 512 * i];
#pragma unroll
        for (int i = 0; i < NDO; ++i) {
            const int u = tid + 512 * i, r = u / (BV / 4), c4 = u % (BV / 4);
            rDO[i] = *reinterpret_cast<const f32x4*>(W.dO + ch * 64 * DV + static_cast<size_t>(r) * DV + vl0 + 4 * c4);
        }
        // pC, em, gC: DK / 4 units each (clamped, so the load is unconditional)
        const int us = min(tid, 3 * (DK / 4) - 1), arr = us / (DK / 4), c4 = us % (DK / 4);
        const float* src = arr == 0 ? W.pC : arr == 1 ? W.em : W.gC;
        rSM = *reinterpret_cast<const f32x4*>(src + ch * DK + 4 * c4);
    };
    auto store1 = [&]() {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            const int u = tid + 512 * i, r = u / 16, c4 = u % 16;
            *reinterpret_cast<f32x4*>(Ms + r * P64 + 4 * c4) = rM[i];
            *reinterpret_cast<f32x4*>(Ts + r * P64 + 4 * c4) = rT[i];
        }
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int u = tid + 512 * i, r = u / (DK / 4), c4 = u % (DK / 4);
            *reinterpret_cast<f32x4*>(KBs + r * PKB + 4 * c4) = rKB[i];
        }
#pragma unroll
        for (int i = 0; i < NDO; ++i) {   // (transition slices: the map's linear part, dO = 0)
            const int u = tid + 512 * i, r = u / (BV / 4), c4 = u % (BV / 4);
            *reinterpret_cast<f32x4*>(dOs + r * PV + 4 * c4) = trans ? f32x4{0.f, 0.f, 0.f, 0.f} : rDO[i];
        }
        if (tid < 3 * (DK / 4)) *reinterpret_cast<f32x4*>(pCs + 4 * tid) = rSM;
    };
    auto load2 = [&](int j) {   // Q1, K1 of chunk j
        const size_t ch = chj(j);
        const f32x4* Q4 = reinterpret_cast<const f32x4*>(W.Q1 + ch * 64 * DK);
        const f32x4* K4 = reinterpret_cast<const f32x4*>(W.K1 + ch * 64 * DK);
#pragma unroll
        for (int i = 0; i < NKB; ++i) { rQ[i] = Q4[tid + 512 * i]; rK[i] = K4[tid + 512 * i]; }
    };
    auto store2 = [&]() {
#pragma unroll
        for (int i = 0; i < NKB; ++i) {
            const int u = tid + 512 * i, r = u / (DK / 4), c4 = u % (DK / 4);
            *reinterpret_cast<f32x4*>(Q1s + r * PQK + 4 * c4) = rQ[i];
            *reinterpret_cast<f32x4*>(K1s + r * PQK + 4 * c4) = rK[i];
        }
    };

    // ---- tiles: wave w owns TPW consecutive 16x16 tiles of a product ------
    constexpr int TU = 4 * CT, TPU = TU >= 8 ? TU / 8 : 1;             // 64 x BV products
    constexpr int TG = (DK / 16) * CT, TPG = TG >= 8 ? TG / 8 : 1;     // DK x BV product
    const bool actU = w * TPU < TU, actG = w * TPG < TG;

    // G = dht (or 0) at the chain's end; segmented: the identity for
    // transition slices, zero for the middle segments of phase 1, the
    // scanned start in phase 3
    const float* gsrc = p.dht ? p.dht + static_cast<size_t>(bh) * DK * DV : nullptr;
    if (SEG && seg < nseg - 1) gsrc = OUT ? p.seg_start + (static_cast<size_t>(ss) * p.H + hh) * DK * DV : nullptr;
    for (int e = tid; e < DK * BV; e += 512) {
        const int c = e / BV, v = e % BV;
        Gs[c * PV + v] = trans ? (c == v0 + v ? 1.f : 0.f) : (gsrc ? gsrc[static_cast<size_t>(c) * DV + v0 + v] : 0.f);
    }
    if (jend > jbeg) {   // (an empty document has no chunks: dh0 = dht)
        load1(jend - 1);
        store1();
    }
    __syncthreads();
    for (int j = jend - 1; j >= jbeg; --j) {
        const size_t ch = chj(j);
        load2(j);
        // dSt = Diag(pC) G to the workspace (slice columns)
        if (OUT) {
            for (int e = tid; e < DK * (BV / 4); e += 512) {
                const int c = e / (BV / 4), c4 = e % (BV / 4);
                const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + c * PV + 4 * c4);
                *reinterpret_cast<f32x4*>(W.dSt + ch * DK * DV + static_cast<size_t>(c) * DV + v0 + 4 * c4) = pCs[c] * gv;
            }
        }
        // dU = M^T dO + KB dSt
        if (actU) {
            f32x4 acc[TPU];
            int ti[TPU], tj[TPU];
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                const int tt = w * TPU + u;
                ti[u] = tt / CT; tj[u] = tt % CT;
                acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll 4
            for (int k0 = 0; k0 < 64; k0 += 4) {
#pragma unroll
                for (int u = 0; u < TPU; ++u) {
                    const float a = Ms[(k0 + g) * P64 + 16 * ti[u] + n];
                    const float b = dOs[(k0 + g) * PV + 16 * tj[u] + n];
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[u], 0, 0, 0);
                }
            }
#pragma unroll 4
            for (int k0 = 0; k0 < DK; k0 += 4) {
                const float pc = pCs[k0 + g];
#pragma unroll
                for (int u = 0; u < TPU; ++u) {
                    const float a = KBs[(16 * ti[u] + n) * PKB + k0 + g];
                    const float b = pc * Gs[(k0 + g) * PV + 16 * tj[u] + n];
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[u], 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < TPU; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) UZs[(16 * ti[u] + 4 * g + i) * PV + 16 * tj[u] + n] = acc[u][i];
        }
        __syncthreads();
        // dU to the workspace; Z = T^T dU (held in registers until dU is no longer read)
        if (OUT) {
            for (int e = tid; e < 64 * (BV / 4); e += 512) {
                const int r = e / (BV / 4), c4 = e % (BV / 4);
                *reinterpret_cast<f32x4*>(W.dU + ch * 64 * DV + static_cast<size_t>(r) * DV + v0 + 4 * c4) =
                    *reinterpret_cast<const f32x4*>(UZs + r * PV + 4 * c4);
            }
        }
        f32x4 zacc[TPU];
        int zti[TPU], ztj[TPU];
        if (actU) {
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                const int tt = w * TPU + u;
                zti[u] = tt / CT; ztj[u] = tt % CT;
                zacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll 4
            for (int k0 = 0; k0 < 64; k0 += 4) {
#pragma unroll
                for (int u = 0; u < TPU; ++u) {
                    const float a = Ts[(k0 + g) * P64 + 16 * zti[u] + n];
                    const float b = UZs[(k0 + g) * PV + 16 * ztj[u] + n];
                    zacc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, zacc[u], 0, 0, 0);
                }
            }
        }
        __syncthreads();
        // Z and this chunk's Q1, K1 to LDS; the next chunk's stage-1 loads go out
        if (actU) {
#pragma unroll
            for (int u = 0; u < TPU; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) UZs[(16 * zti[u] + 4 * g + i) * PV + 16 * ztj[u] + n] = zacc[u][i];
        }
        store2();
        load1(j > jbeg ? j - 1 : jbeg);
        __syncthreads();
        // G <- Diag(e^m) (Q1^T dO - K1^T Z) + Diag(e^{b_L} pC) G   (each wave its own tiles, in place)
        if (actG) {
            f32x4 acc[TPG];
            int ti[TPG], tj[TPG];
#pragma unroll
            for (int u = 0; u < TPG; ++u) {
                const int tt = w * TPG + u;
                ti[u] = tt / CT; tj[u] = tt % CT;
                acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll 4
            for (int k0 = 0; k0 < 64; k0 += 4) {
#pragma unroll
                for (int u = 0; u < TPG; ++u) {
                    const float aq = Q1s[(k0 + g) * PQK + 16 * ti[u] + n];
                    const float ak = -K1s[(k0 + g) * PQK + 16 * ti[u] + n];
                    const float bo = dOs[(k0 + g) * PV + 16 * tj[u] + n];
                    const float bz = UZs[(k0 + g) * PV + 16 * tj[u] + n];
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq, bo, acc[u], 0, 0, 0);
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak, bz, acc[u], 0, 0, 0);
                }
            }
#pragma unroll
            for (int u = 0; u < TPG; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * ti[u] + 4 * g + i, c = 16 * tj[u] + n;
                    Gs[r * PV + c] = ems[r] * acc[u][i] + gCs[r] * pCs[r] * Gs[r * PV + c];
                }
        }
        __syncthreads();
        store1();   // chunk j - 1 (on the last chunk walked: that chunk again, unused)
        __syncthreads();
    }
    // the end state: dh0 (whole chains; phase 3, the chain's first segment),
    // or in phase 1 the start of the next segment in pass order (the chain's
    // last segment), H_s or P_s (middle segments)
    float* dst = p.dh0 ? p.dh0 + static_cast<size_t>(bh) * DK * DV : nullptr;
    int pitch = DV, ncol = BV;
    if (SEG && !OUT) {
        if (seg == nseg - 1) {
            dst = p.seg_start + (static_cast<size_t>(ss - 1) * p.H + hh) * DK * DV;
        } else if (trans) {
            dst = p.seg_p + (static_cast<size_t>(ss) * p.H + hh) * DK * DK;
            pitch = DK;
            ncol = min(BV, DK - v0);   // (columns of P_s past DK do not exist)
        } else {
            dst = p.seg_h + (static_cast<size_t>(ss) * p.H + hh) * DK * DV;
        }
    } else if (SEG && seg > 0) {
        dst = nullptr;
    }
    if (dst) {
        for (int e = tid; e < DK * BV; e += 512) {
            const int c = e / BV, v = e % BV;
            if (v < ncol) dst[static_cast<size_t>(c) * pitch + v0 + v] = Gs[c * PV + v];
        }
    }
}

// ---------------------------------------------------------------------------
// The reverse pass with bf16 x3 matrix-core arithmetic (bf16 inputs): the
// recurrence of bwd_reverse_kernel, with every product operand staged once
// per chunk as bf16 hi and lo planes whose rows run along the product's K
// (x = hi + lo to about 2^-16 of x) and each 16x16 tile taking hi*hi +
// hi*lo + lo*hi per 32-wide K step (three 16x16x32 bf16 products instead of
// eight 16x16x4 fp32 ones).  Operands read transposed (M^T, T^T, Q1^T,
// -K1^T, and dO as the B side) are staged from column loads: a thread reads
// 8 consecutive rows of one column, coalesced across the wave.  dSt, dU and
// Z reach their planes straight from the accumulator layout, and G stays in
// registers in the accumulator layout of each wave's DK x BV tiles.  Lane
// (n, g) carries K indices 32 ks + 8g .. +7 in both operands.
template <int DK, int DV>
struct RevX3Shape {
    static constexpr int BV = DV < 64 ? DV : 64;
    static constexpr int NSL = DV / BV, NTS = (DK + BV - 1) / BV;
    static constexpr int CT = BV / 16;
    // bytes per staged row: K hi values, K lo values, 32 bytes of pad (a
    // pitch of 8 mod 16 dwords keeps the 16-byte fragment reads conflict-free)
    static constexpr int R64 = 64 * 4 + 32;              // K = 64 (tokens)
    static constexpr int RDK = DK * 4 + 32;              // K = DK
    static constexpr int LO64 = 64 * 2, LODK = DK * 2;   // lo plane offsets within a row
    static constexpr int L_MT = 0;                       // stage 1: M^T, T^T [64][64], KB [64][DK]
    static constexpr int L_TT = L_MT + 64 * R64;
    static constexpr int L_KB = L_TT + 64 * R64;
    static constexpr int S1 = L_KB + 64 * RDK;
    static constexpr int L_Q1T = 0;                      // stage 2: Q1^T, -K1^T [DK][64]
    static constexpr int L_K1T = L_Q1T + DK * R64;
    static constexpr int S2 = L_K1T + DK * R64;
    static constexpr int L_DOT = S1 > S2 ? S1 : S2;      // dO^T [BV][64]
    static constexpr int L_GT = L_DOT + BV * R64;        // dSt^T [BV][DK]
    static constexpr int L_UZ = L_GT + BV * RDK;         // dU^T, then Z^T [BV][64]
    static constexpr int L_SM = L_UZ + BV * R64;         // pC, em, gC: floats [3][DK]
    static constexpr int BYTES = L_SM + 3 * DK * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(R64 % 64 == 32 && RDK % 64 == 32, "row pitch 8 mod 16 dwords");
    // staging units per thread (512 threads)
    static constexpr int NUM = 64 * 8, NUDO = BV * 8, NUQ = DK * 8, NUKB = 64 * (DK / 8);
    static constexpr int UM = (NUM + 511) / 512, UDO = (NUDO + 511) / 512, UQ = (NUQ + 511) / 512,
                         UKB = (NUKB + 511) / 512;
    static constexpr int TU = 4 * CT, TPU = TU >= 8 ? TU / 8 : 1;           // 64 x BV tiles per wave
    static constexpr int TG = (DK / 16) * CT, TPG = TG >= 8 ? TG / 8 : 1;   // DK x BV tiles per wave
};

// 8 (4) values split into bf16 hi / lo planes of a staged row: hi at p, lo at p + lo_off
__device__ __forceinline__ void put8_x3(unsigned char* p, int lo_off, const float (&x)[8]) {
    const SplitPair a = split2(x[0], x[1]), b = split2(x[2], x[3]), c = split2(x[4], x[5]), d = split2(x[6], x[7]);
    *reinterpret_cast<u32x4*>(p) = u32x4{a.hi, b.hi, c.hi, d.hi};
    *reinterpret_cast<u32x4*>(p + lo_off) = u32x4{a.lo, b.lo, c.lo, d.lo};
}
__device__ __forceinline__ void put4_x3(unsigned char* p, int lo_off, f32x4 x) {
    const SplitPair a = split2(x[0], x[1]), b = split2(x[2], x[3]);
    *reinterpret_cast<u32x2*>(p) = u32x2{a.hi, b.hi};
    *reinterpret_cast<u32x2*>(p + lo_off) = u32x2{a.lo, b.lo};
}
// acc += A B over one 32-wide K step, fragments at pa / pb (hi; lo at + lo_off)
__device__ __forceinline__ f32x4 mma_x3(const unsigned char* pa, int alo, const unsigned char* pb, int blo, f32x4 acc) {
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(pa), al = *reinterpret_cast<const bf16x8*>(pa + alo);
    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(pb), bl = *reinterpret_cast<const bf16x8*>(pb + blo);
    return mfma32x3(ah, al, bh, bl, acc);
}

template <int DK, int DV, bool SEG, bool OUT>
__global__ void __launch_bounds__(512) bwd_reverse_x3_kernel(BwdParams p, BwdWs W) {
    using SH = RevX3Shape<DK, DV>;
    constexpr int BV = SH::BV, CT = SH::CT, R64 = SH::R64, RDK = SH::RDK, LO64 = SH::LO64, LODK = SH::LODK;
    constexpr int TU = SH::TU, TPU = SH::TPU, TG = SH::TG, TPG = SH::TPG;
    constexpr int UM = SH::UM, UDO = SH::UDO, UQ = SH::UQ, UKB = SH::UKB;
    extern __shared__ __align__(16) unsigned char smem[];
    float* const pCs = reinterpret_cast<float*>(smem + SH::L_SM);
    float* const ems = pCs + DK;
    float* const gCs = ems + DK;

    constexpr int NS = (SEG && !OUT) ? SH::NSL + SH::NTS : SH::NSL;
    const RevWork rw = rev_work<SEG, OUT>(p, SH::NSL, NS, BV);
    if (!rw.run) return;   // the whole workgroup, before any barrier
    const int bh = rw.bh, hh = rw.hh, seg = rw.seg, ss = rw.ss, nseg = rw.nseg, v0 = rw.v0, jbeg = rw.jbeg,
              jend = rw.jend;
    const bool trans = rw.trans;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, n = l & 15, g = l >> 4;
    const int vl0 = trans ? 0 : v0;   // dO columns staged (transition slices zero them)

    // ---- staging (loads into registers, then split into the planes) ----------
    float rM[UM][8], rT[UM][8], rDO[UDO][8], rQ[UQ][8], rK[UQ][8];
    f32x4 rKB[UKB][2], rSM;
    auto load1 = [&](int j) {   // M, T, KB, dO slice, pC / em / gC of chunk j (indices clamped)
        const size_t ch = rw.chj(p, j);
        const float* M = W.M + ch * 4096;
        const float* T = W.T + ch * 4096;
#pragma unroll
        for (int u = 0; u < UM; ++u) {
            const int e = min(tid + 512 * u, SH::NUM - 1), col = e % 64, kb = e / 64;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                rM[u][r] = M[(8 * kb + r) * 64 + col];
                rT[u][r] = T[(8 * kb + r) * 64 + col];
            }
        }
        const float* dO = W.dO + ch * 64 * DV + vl0;
#pragma unroll
        for (int u = 0; u < UDO; ++u) {
            const int e = min(tid + 512 * u, SH::NUDO - 1), col = e % BV, kb = e / BV;
#pragma unroll
            for (int r = 0; r < 8; ++r) rDO[u][r] = dO[static_cast<size_t>(8 * kb + r) * DV + col];
        }
        const float* KB = W.KB + ch * 64 * DK;
#pragma unroll
        for (int u = 0; u < UKB; ++u) {
            const int e = min(tid + 512 * u, SH::NUKB - 1), row = e / (DK / 8), cb = e % (DK / 8);
            rKB[u][0] = *reinterpret_cast<const f32x4*>(KB + row * DK + 8 * cb);
            rKB[u][1] = *reinterpret_cast<const f32x4*>(KB + row * DK + 8 * cb + 4);
        }
        const int us = min(tid, 3 * (DK / 4) - 1), arr = us / (DK / 4), c4 = us % (DK / 4);
        const float* src = arr == 0 ? W.pC : arr == 1 ? W.em : W.gC;
        rSM = *reinterpret_cast<const f32x4*>(src + ch * DK + 4 * c4);
    };
    auto store1 = [&]() {
#pragma unroll
        for (int u = 0; u < UM; ++u) {
            const int e = tid + 512 * u, col = e % 64, kb = e / 64;
            if (SH::NUM % 512 == 0 || e < SH::NUM) {
                put8_x3(smem + SH::L_MT + col * R64 + 16 * kb, LO64, rM[u]);
                put8_x3(smem + SH::L_TT + col * R64 + 16 * kb, LO64, rT[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < UDO; ++u) {
            const int e = tid + 512 * u, col = e % BV, kb = e / BV;
            if (SH::NUDO % 512 == 0 || e < SH::NUDO) {
                float x[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) x[r] = trans ? 0.f : rDO[u][r];   // (P_s: dO = 0)
                put8_x3(smem + SH::L_DOT + col * R64 + 16 * kb, LO64, x);
            }
        }
#pragma unroll
        for (int u = 0; u < UKB; ++u) {
            const int e = tid + 512 * u, row = e / (DK / 8), cb = e % (DK / 8);
            if (SH::NUKB % 512 == 0 || e < SH::NUKB) {
                const float x[8] = {rKB[u][0][0], rKB[u][0][1], rKB[u][0][2], rKB[u][0][3],
                                    rKB[u][1][0], rKB[u][1][1], rKB[u][1][2], rKB[u][1][3]};
                put8_x3(smem + SH::L_KB + row * RDK + 16 * cb, LODK, x);
            }
        }
        if (tid < 3 * (DK / 4)) *reinterpret_cast<f32x4*>(pCs + 4 * tid) = rSM;
    };
    auto load2 = [&](int j) {   // Q1, K1 of chunk j (columns)
        const size_t ch = rw.chj(p, j);
        const float* Q1 = W.Q1 + ch * 64 * DK;
        const float* K1 = W.K1 + ch * 64 * DK;
#pragma unroll
        for (int u = 0; u < UQ; ++u) {
            const int e = min(tid + 512 * u, SH::NUQ - 1), col = e % DK, kb = e / DK;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                rQ[u][r] = Q1[(8 * kb + r) * DK + col];
                rK[u][r] = K1[(8 * kb + r) * DK + col];
            }
        }
    };
    auto store2 = [&]() {
#pragma unroll
        for (int u = 0; u < UQ; ++u) {
            const int e = tid + 512 * u, col = e % DK, kb = e / DK;
            if (SH::NUQ % 512 == 0 || e < SH::NUQ) {
                float nk[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) nk[r] = -rK[u][r];
                put8_x3(smem + SH::L_Q1T + col * R64 + 16 * kb, LO64, rQ[u]);
                put8_x3(smem + SH::L_K1T + col * R64 + 16 * kb, LO64, nk);
            }
        }
    };

    // ---- tiles of this wave -------------------------------------------------
    const bool actU = w * TPU < TU, actG = w * TPG < TG;
    int uti[TPU], utj[TPU], gti[TPG], gtj[TPG];
#pragma unroll
    for (int u = 0; u < TPU; ++u) { uti[u] = (w * TPU + u) / CT; utj[u] = (w * TPU + u) % CT; }
#pragma unroll
    for (int u = 0; u < TPG; ++u) { gti[u] = (w * TPG + u) / CT; gtj[u] = (w * TPG + u) % CT; }

    // G at the pass's start: dht (or 0) at the chain's end; segmented: the
    // identity for transition slices, zero for the middle segments of phase
    // 1, the scanned start in phase 3.  Lane (n, g) of tile u holds rows
    // 16 gti + 4g + i, column 16 gtj + n.
    const float* gsrc = p.dht ? p.dht + static_cast<size_t>(bh) * DK * DV : nullptr;
    if (SEG && seg < nseg - 1) gsrc = OUT ? p.seg_start + (static_cast<size_t>(ss) * p.H + hh) * DK * DV : nullptr;
    f32x4 Gr[TPG];
#pragma unroll
    for (int u = 0; u < TPG; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * gti[u] + 4 * g + i, v = 16 * gtj[u] + n;
            Gr[u][i] = !actG ? 0.f
                     : trans ? (c == v0 + v ? 1.f : 0.f)
                             : (gsrc ? gsrc[static_cast<size_t>(c) * DV + v0 + v] : 0.f);
        }

    if (jend > jbeg) {   // (an empty document has no chunks: dh0 = dht)
        load1(jend - 1);
        store1();
    }
    __syncthreads();
    for (int j = jend - 1; j >= jbeg; --j) {
        const size_t ch = rw.chj(p, j);
        load2(j);
        // dSt = Diag(pC) G: planes for the dU product, fp32 to the workspace
        if (actG) {
#pragma unroll
            for (int u = 0; u < TPG; ++u) {
                const int c0 = 16 * gti[u] + 4 * g, v = 16 * gtj[u] + n;
                const f32x4 ds = *reinterpret_cast<const f32x4*>(pCs + c0) * Gr[u];
                put4_x3(smem + SH::L_GT + v * RDK + 2 * c0, LODK, ds);
                if (OUT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) W.dSt[ch * DK * DV + static_cast<size_t>(c0 + i) * DV + v0 + v] = ds[i];
                }
            }
        }
        __syncthreads();
        // dU = M^T dO + KB dSt (64 x BV)
        f32x4 ua[TPU];
        if (actU) {
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                ua[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                const unsigned char* am = smem + SH::L_MT + (16 * uti[u] + n) * R64 + 16 * g;
                const unsigned char* bo = smem + SH::L_DOT + (16 * utj[u] + n) * R64 + 16 * g;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ua[u] = mma_x3(am + 64 * ks, LO64, bo + 64 * ks, LO64, ua[u]);
                const unsigned char* ak = smem + SH::L_KB + (16 * uti[u] + n) * RDK + 16 * g;
                const unsigned char* bg = smem + SH::L_GT + (16 * utj[u] + n) * RDK + 16 * g;
#pragma unroll
                for (int ks = 0; ks < DK / 32; ++ks) ua[u] = mma_x3(ak + 64 * ks, LODK, bg + 64 * ks, LODK, ua[u]);
            }
            // dU^T planes (for Z), fp32 to the workspace
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                const int k0 = 16 * uti[u] + 4 * g, v = 16 * utj[u] + n;
                put4_x3(smem + SH::L_UZ + v * R64 + 2 * k0, LO64, ua[u]);
                if (OUT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) W.dU[ch * 64 * DV + static_cast<size_t>(k0 + i) * DV + v0 + v] = ua[u][i];
                }
            }
        }
        __syncthreads();
        // Z = T^T dU
        f32x4 za[TPU];
        if (actU) {
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                za[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                const unsigned char* at = smem + SH::L_TT + (16 * uti[u] + n) * R64 + 16 * g;
                const unsigned char* bu = smem + SH::L_UZ + (16 * utj[u] + n) * R64 + 16 * g;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) za[u] = mma_x3(at + 64 * ks, LO64, bu + 64 * ks, LO64, za[u]);
            }
        }
        __syncthreads();   // dU^T, M^T, T^T, KB consumed
        // Z^T planes; stage 2 (Q1^T, -K1^T) over stage 1; the next chunk's stage-1 loads go out
        if (actU) {
#pragma unroll
            for (int u = 0; u < TPU; ++u) {
                const int k0 = 16 * uti[u] + 4 * g, v = 16 * utj[u] + n;
                put4_x3(smem + SH::L_UZ + v * R64 + 2 * k0, LO64, za[u]);
            }
        }
        store2();
        load1(j > jbeg ? j - 1 : jbeg);
        __syncthreads();
        // G <- Diag(e^m) (Q1^T dO - K1^T Z) + Diag(e^{b_L} pC) G
        if (actG) {
#pragma unroll
            for (int u = 0; u < TPG; ++u) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const unsigned char* aq = smem + SH::L_Q1T + (16 * gti[u] + n) * R64 + 16 * g;
                const unsigned char* ak = smem + SH::L_K1T + (16 * gti[u] + n) * R64 + 16 * g;
                const unsigned char* bo = smem + SH::L_DOT + (16 * gtj[u] + n) * R64 + 16 * g;
                const unsigned char* bz = smem + SH::L_UZ + (16 * gtj[u] + n) * R64 + 16 * g;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    acc = mma_x3(aq + 64 * ks, LO64, bo + 64 * ks, LO64, acc);
                    acc = mma_x3(ak + 64 * ks, LO64, bz + 64 * ks, LO64, acc);
                }
                const int c0 = 16 * gti[u] + 4 * g;
                const f32x4 em4 = *reinterpret_cast<const f32x4*>(ems + c0);
                const f32x4 gc4 = *reinterpret_cast<const f32x4*>(gCs + c0);
                const f32x4 pc4 = *reinterpret_cast<const f32x4*>(pCs + c0);
                Gr[u] = em4 * acc + gc4 * pc4 * Gr[u];
            }
        }
        __syncthreads();   // Q1^T, K1^T, dO^T, Z^T, pC / em / gC consumed
        store1();   // chunk j - 1 (on the last chunk walked: that chunk again, unused)
        __syncthreads();
    }
    // the end state: dh0 (whole chains; phase 3, the chain's first segment),
    // or in phase 1 the start of the next segment in pass order (the chain's
    // last segment), H_s or P_s (middle segments)
    float* dst = p.dh0 ? p.dh0 + static_cast<size_t>(bh) * DK * DV : nullptr;
    int pitch = DV, ncol = BV;
    if (SEG && !OUT) {
        if (seg == nseg - 1) {
            dst = p.seg_start + (static_cast<size_t>(ss - 1) * p.H + hh) * DK * DV;
        } else if (trans) {
            dst = p.seg_p + (static_cast<size_t>(ss) * p.H + hh) * DK * DK;
            pitch = DK;
            ncol = min(BV, DK - v0);   // (columns of P_s past DK do not exist)
        } else {
            dst = p.seg_h + (static_cast<size_t>(ss) * p.H + hh) * DK * DV;
        }
    } else if (SEG && seg > 0) {
        dst = nullptr;
    }
    if (dst && actG) {
#pragma unroll
        for (int u = 0; u < TPG; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 16 * gti[u] + 4 * g + i, v = 16 * gtj[u] + n;
                if (v < ncol) dst[static_cast<size_t>(c) * pitch + v0 + v] = Gr[u][i];
            }
    }
}

// X3: the bf16 x3 variant (bf16 inputs), else fp32 matrix cores
template <int DK, int DV, bool SEG, bool OUT>
static hipError_t launch_reverse_k(const BwdParams& p, const BwdWs& W, int grid, bool x3, hipStream_t st) {
    if (grid == 0) return hipSuccess;
    auto go = [&](auto kern, int bytes) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(grid), dim3(512), bytes, st, p, W);
        return hipGetLastError();
    };
    if (x3) return go(bwd_reverse_x3_kernel<DK, DV, SEG, OUT>, RevX3Shape<DK, DV>::BYTES);
    return go(bwd_reverse_kernel<DK, DV, SEG, OUT>, RevShape<DK, DV>::BYTES);
}

// measured on MI355X (dk = dv = 128): a lone chain's reverse step is the
// unit (about 14.6 us); the GPU completes about 15.5 workgroup chunk-steps
// per us (0.88 per CU per unit); phase 1 skips only the dSt / dU stores; a
// scan step is about 6 us
constexpr SegCost kReverseCost{0.88, 0.9, 0.5};

// the reverse pass over every chain: whole chains, or segments (p.G > 0,
// buffers set) in three launches
template <int DK, int DV>
static hipError_t launch_reverse_t(const BwdParams& p, const BwdWs& W, bool x3, hipStream_t st) {
    using SH = RevShape<DK, DV>;
    const int nchains = (p.cu ? p.ndocs : p.B) * p.H;
    if (p.G == 0) return launch_reverse_k<DK, DV, false, true>(p, W, nchains * SH::NSL, x3, st);
    hipError_t e = launch_reverse_k<DK, DV, true, false>(p, W, p.nsslots * p.H * (SH::NSL + SH::NTS), x3, st);
    if (e != hipSuccess) return e;
    const SegScanParams sp{p.cu, p.T, p.H, p.G, p.seg_start, p.seg_h, p.seg_p, 1};
    hipLaunchKernelGGL((ckda_seg_scan_kernel<DK, DV>), dim3(nchains * (DV / kScanCols)), dim3(256), 0, st, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reverse_k<DK, DV, true, true>(p, W, p.nsslots * p.H * SH::NSL, x3, st);
}

static hipError_t launch_reverse(const BwdParams& p, const BwdWs& W, bool x3, hipStream_t st) {
#define CKDA_REV(DK_, DV_) \
    if (W.DK == DK_ && W.DV == DV_) return launch_reverse_t<DK_, DV_>(p, W, x3, st);
    CKDA_REV(32, 32) CKDA_REV(32, 64) CKDA_REV(32, 128)
    CKDA_REV(64, 32) CKDA_REV(64, 64) CKDA_REV(64, 128)
    CKDA_REV(128, 32) CKDA_REV(128, 64) CKDA_REV(128, 128)
#undef CKDA_REV
    return hipErrorInvalidValue;
}

// 64x64 per chunk-head, 256 threads: thread t owns row r = t / 4 and the
// 16 columns 16 (t % 4) .. +15 as four 16-byte units (coalesced rows).

// dbeta1_i = sum_r dT_ri Xi_ri (column sums) ; Y1 = dT Diag(beta)
__global__ void __launch_bounds__(256) bwd_dbeta1_kernel(BwdWs W) {
    __shared__ f32x4 part[64][16];
    const size_t ch = blockIdx.x;
    const int t = threadIdx.x, r = t >> 2, c0 = 16 * (t & 3);
    const f32x4* dT = reinterpret_cast<const f32x4*>(W.dT + ch * 4096 + r * 64 + c0);
    const f32x4* Xi = reinterpret_cast<const f32x4*>(W.Xi + ch * 4096 + r * 64 + c0);
    const f32x4* bt = reinterpret_cast<const f32x4*>(W.beta + ch * 64 + c0);
    f32x4* Y1 = reinterpret_cast<f32x4*>(W.Y1 + ch * 4096 + r * 64 + c0);
    f32x4 d[4], x[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { d[u] = dT[u]; x[u] = Xi[u]; b[u] = bt[u]; }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        Y1[u] = d[u] * b[u];
        part[r][4 * (t & 3) + u] = d[u] * x[u];
    }
    __syncthreads();
    if (t < 64) {   // column t: sum over the 64 rows
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int unit = t >> 2, lane = t & 3;
        for (int rr = 0; rr < 64; ++rr) acc += part[rr][unit];
        W.dbeta1[ch * 64 + t] = acc[lane];
    }
}

// dXs = strict_lower(dX); dbeta2_r = sum_i dXs_ri A_ri (row sums); dA = Diag(beta) dXs
__global__ void __launch_bounds__(256) bwd_dA_kernel(BwdWs W) {
    const size_t ch = blockIdx.x;
    const int t = threadIdx.x, r = t >> 2, c0 = 16 * (t & 3);
    const f32x4* dX = reinterpret_cast<const f32x4*>(W.dX + ch * 4096 + r * 64 + c0);
    const f32x4* A = reinterpret_cast<const f32x4*>(W.A + ch * 4096 + r * 64 + c0);
    f32x4* dA = reinterpret_cast<f32x4*>(W.dA + ch * 4096 + r * 64 + c0);
    const float br = W.beta[ch * 64 + r];
    f32x4 x[4], a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { x[u] = dX[u]; a[u] = A[u]; }
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = (c0 + 4 * u + e < r) ? x[u][e] : 0.f;
        dA[u] = br * m;
        const f32x4 pa = m * a[u];
        rs += pa[0] + pa[1] + pa[2] + pa[3];
    }
    // the row's four threads are adjacent lanes
    rs += __shfl_xor(rs, 1, 64);
    rs += __shfl_xor(rs, 2, 64);
    if ((t & 3) == 0) W.dbeta2[ch * 64 + r] = rs;
}

// gate gradient, unfold of the sign product, scatter to [B,T,H,.]
//   dq = P dQ1 e^{b-m},  dk = P (dK1 e^{b-m} + dK2 e^{m-b} + dKB e^{b_L-b}),
//   db = Q1 dQ1 + K1 dK1 - K2 dK2 - KB dKB  (+ sum_t KB dKB + e^{b_L} sum_v dSt S
//   at the last token),  dg = reverse cumulative sum of db over the chunk;
// b, P and the anchored operands are recomputed from g, s, q, k (the same
// scans as the prep).  With q and k normalised in the path (q^ = q/||q||),
// the gradients above are those of q^ and k^, and the chain rule through the
// normalisation gives dq = (dq^ - q^ (q^ . dq^)) / ||q||, the same for k.
template <int DK> constexpr int final_threads() { return 512; }   // the prep's segmentation: identical b

template <typename Tin, int DK, int DV, bool HG, bool NQK>
__global__ void __launch_bounds__(final_threads<DK>()) bwd_final_kernel(BwdParams p, BwdWs W) {
    constexpr int NTHR = final_threads<DK>();
    using QS = QuadSeg<DK, NTHR>;
    constexpr int CQ = QS::CQ, SEGS = QS::SEGS, NTOK = QS::NTOK;
    // segment totals: (b, P) of the scans, then (db, KB dKB) in the same space
    __shared__ f32x4 segb[SEGS][CQ], segp[SEGS][CQ];
    __shared__ __align__(16) float dgl[DK];
    f32x4 (&segdb)[SEGS][CQ] = segb;
    f32x4 (&segkb)[SEGS][CQ] = segp;
    const int ch = blockIdx.x;
    const ChunkIdx ci(ch, p);
    if (ci.L <= 0) return;   // unused varlen slot
    const int tid = threadIdx.x, q4 = tid % CQ, seg = tid / CQ, tb = seg * NTOK;
    const size_t trow0 = ci.trow0;
    const size_t o64k = static_cast<size_t>(ch) * 64 * DK;
    const size_t o64v = static_cast<size_t>(ch) * 64 * DV;
    f32x4 gv[NTOK], sg[NTOK], kv[NTOK], qv[NTOK], dq1[NTOK], dk1[NTOK], dk2[NTOK], dkb[NTOK];
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const size_t row = trow0 + min(tb + i, ci.L - 1);
        const size_t e = (row * p.H + ci.h) * DK + 4 * q4;
        gate_quad<HG>(p, row, ci.h, DK, q4, gv[i], sg[i]);
        kv[i] = load_quad(static_cast<const Tin*>(p.k), e);
        qv[i] = load_quad(static_cast<const Tin*>(p.q), e);
        const size_t o = o64k + static_cast<size_t>(tb + i) * DK + 4 * q4;
        dq1[i] = *reinterpret_cast<const f32x4*>(W.dQ1 + o);
        dk1[i] = *reinterpret_cast<const f32x4*>(W.dK1 + o);
        dk2[i] = *reinterpret_cast<const f32x4*>(W.dK2 + o);
        dkb[i] = *reinterpret_cast<const f32x4*>(W.dKB + o);
    }
    float ik[NTOK], iq[NTOK];
    if constexpr (NQK) {
        normalise_rows<CQ>(kv, ik);
        normalise_rows<CQ>(qv, iq);
    }
    f32x4 run = {0.f, 0.f, 0.f, 0.f}, par = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const bool valid = tb + i < ci.L;
        run += valid ? gv[i] : f32x4{0.f, 0.f, 0.f, 0.f};
        par *= valid ? sg[i] : f32x4{1.f, 1.f, 1.f, 1.f};
        gv[i] = run;
        sg[i] = par;
    }
    segb[seg][q4] = run;
    segp[seg][q4] = par;
    __syncthreads();
    f32x4 off = {0.f, 0.f, 0.f, 0.f}, poff = {1.f, 1.f, 1.f, 1.f}, m = off, bL = off;
#pragma unroll 2
    for (int s2 = 0; s2 < SEGS; ++s2) {
        const f32x4 x = segb[s2][q4];
        if (s2 < seg) { off += x; poff *= segp[s2][q4]; }
        if (s2 < SEGS / 2) m += x;
        bL += x;
    }
    f32x4 dbv[NTOK];
    f32x4 kbs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const bool valid = tb + i < ci.L;
        const f32x4 b = gv[i] + off, P = sg[i] * poff;
        const f32x4 kf = P * kv[i], qf = P * qv[i];
        const f32x4 e1 = exp2c4((b - m) * kLog2e), e2 = exp2c4((m - b) * kLog2e), e3 = exp2c4((bL - b) * kLog2e);
        const f32x4 kb = kf * e3;
        const f32x4 dbi = qf * e1 * dq1[i] + kf * e1 * dk1[i] - kf * e2 * dk2[i] - kb * dkb[i];
        // dq = P dq~ and dk = P dk~ (then through the normalisation)
        f32x4 dqo = P * (dq1[i] * e1), dko = P * (dk1[i] * e1 + dk2[i] * e2 + dkb[i] * e3);
        if constexpr (NQK) {   // every lane of the row takes part in the sums
            const float pq = row_sum<CQ>(dot4(qv[i], dqo)), pk = row_sum<CQ>(dot4(kv[i], dko));
            dqo = iq[i] * (dqo - pq * qv[i]);
            dko = ik[i] * (dko - pk * kv[i]);
        }
        if (valid) {
            const size_t e = ((trow0 + tb + i) * p.H + ci.h) * DK + 4 * q4;
            *reinterpret_cast<f32x4*>(p.dq + e) = dqo;
            *reinterpret_cast<f32x4*>(p.dk + e) = dko;
        }
        dbv[i] = valid ? dbi : f32x4{0.f, 0.f, 0.f, 0.f};
        kbs += valid ? kb * dkb[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // dGL_c = sum_v dSt[c][v] S[c][v]: TPR threads per row, NQ 16-byte units each,
    // read once the token operands are consumed (registers are free again)
    constexpr int TPR = (DV / 4) < (NTHR / DK) ? (DV / 4) : (NTHR / DK), NQ = (DV / 4) / TPR;
    const int gr = tid / TPR, gj = tid % TPR;
    f32x4 gs[NQ], gd[NQ];
    {
        const f32x4* S4 = reinterpret_cast<const f32x4*>(p.h_ckpt + static_cast<size_t>(ch) * DK * DV);
        const f32x4* D4 = reinterpret_cast<const f32x4*>(W.dSt + static_cast<size_t>(ch) * DK * DV);
        const int r = min(gr, DK - 1);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            gs[i] = S4[r * (DV / 4) + i * TPR + gj];
            gd[i] = D4[r * (DV / 4) + i * TPR + gj];
        }
    }
    // suffix sums of db inside the segment
    f32x4 suf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = NTOK - 1; i >= 0; --i) {
        suf += dbv[i];
        dbv[i] = suf;
    }
    __syncthreads();   // every thread has read the scan totals
    segdb[seg][q4] = suf;
    segkb[seg][q4] = kbs;
    {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NQ; ++i) acc += gs[i] * gd[i];
        float x = acc[0] + acc[1] + acc[2] + acc[3];
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) x += __shfl_xor(x, o, 64);
        if (gj == 0 && gr < DK) dgl[gr] = x;
    }
    __syncthreads();
    f32x4 later = {0.f, 0.f, 0.f, 0.f}, kbsum = later;
#pragma unroll 2
    for (int s2 = 0; s2 < SEGS; ++s2) {
        if (s2 > seg) later += segdb[s2][q4];
        kbsum += segkb[s2][q4];
    }
    const f32x4 dgl4 = *reinterpret_cast<const f32x4*>(dgl + 4 * q4);
    const f32x4 extra = kbsum + exp2c4(bL * kLog2e) * dgl4;   // at the last token, so in every dg
#pragma unroll
    for (int i = 0; i < NTOK; ++i) {
        const int t = tb + i;
        const f32x4 dgv = dbv[i] + later + extra;
        if constexpr (HG) {   // the head's gate: the sum over its channels
            float x = dgv[0] + dgv[1] + dgv[2] + dgv[3];
#pragma unroll
            for (int o = 1; o < CQ; o <<= 1) x += __shfl_xor(x, o, 64);   // the row's quads are adjacent lanes
            if (q4 == 0 && t < ci.L) p.dg[(trow0 + t) * p.H + ci.h] = x;
        } else if (t < ci.L) {
            const size_t e = ((trow0 + t) * p.H + ci.h) * DK + 4 * q4;
            *reinterpret_cast<f32x4*>(p.dg + e) = dgv;
        }
    }
    for (int u = tid; !p.dv_direct && u < 64 * (DV / 4); u += NTHR) {
        const int t = u / (DV / 4), c4 = u % (DV / 4);
        if (t < ci.L)
            *reinterpret_cast<f32x4*>(p.dv + ((trow0 + t) * p.H + ci.h) * DV + 4 * c4) =
                *reinterpret_cast<const f32x4*>(W.dV + o64v + static_cast<size_t>(t) * DV + 4 * c4);
    }
    if (tid < ci.L) {
        const size_t o = static_cast<size_t>(ch) * 64 + tid;
        p.dbeta[(trow0 + tid) * p.H + ci.h] = W.dbeta1[o] + W.dbeta2[o];
    }
}

// dst = src (or 0 when src is null), n floats
__global__ void fill_copy_kernel(float* dst, const float* src, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

template <typename Tin, int DK, int DV, bool HG, bool NQK>
static hipError_t launch_chunk_pass_hg(bool final_pass, const BwdParams& p, const BwdWs& W, int NC,
                                       hipStream_t st) {
    if (final_pass)
        hipLaunchKernelGGL((bwd_final_kernel<Tin, DK, DV, HG, NQK>), dim3(NC), dim3(final_threads<DK>()), 0, st, p,
                           W);
    else
        hipLaunchKernelGGL((bwd_prep_kernel<Tin, DK, DV, HG, NQK>), dim3(NC), dim3(512), 0, st, p, W);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV>
static hipError_t launch_chunk_pass_t(bool final_pass, const BwdParams& p, const BwdWs& W, int NC, hipStream_t st) {
    if (p.qk_norm)
        return p.head_gate ? launch_chunk_pass_hg<Tin, DK, DV, true, true>(final_pass, p, W, NC, st)
                           : launch_chunk_pass_hg<Tin, DK, DV, false, true>(final_pass, p, W, NC, st);
    return p.head_gate ? launch_chunk_pass_hg<Tin, DK, DV, true, false>(final_pass, p, W, NC, st)
                       : launch_chunk_pass_hg<Tin, DK, DV, false, false>(final_pass, p, W, NC, st);
}

// the prep (final_pass false) or final pass over every chunk-head
static hipError_t launch_chunk_pass(bool bf16, bool final_pass, const BwdParams& p, const BwdWs& W, int NC,
                                    hipStream_t st) {
#define CKDA_PASS(DK_, DV_)                                                                           \
    if (W.DK == DK_ && W.DV == DV_)                                                                   \
        return bf16 ? launch_chunk_pass_t<bf16_t, DK_, DV_>(final_pass, p, W, NC, st)                 \
                    : launch_chunk_pass_t<float, DK_, DV_>(final_pass, p, W, NC, st);
    CKDA_PASS(32, 32) CKDA_PASS(32, 64) CKDA_PASS(32, 128)
    CKDA_PASS(64, 32) CKDA_PASS(64, 64) CKDA_PASS(64, 128)
    CKDA_PASS(128, 32) CKDA_PASS(128, 64) CKDA_PASS(128, 128)
#undef CKDA_PASS
    return hipErrorInvalidValue;
}

}  // namespace

size_t bwd_workspace_bytes(int nslots, int H, int DK, int DV) {
    return BwdWs::floats(static_cast<size_t>(nslots) * H, DK, DV) * sizeof(float);
}

// checkpoints recomputed in the call (h_ckpt = nullptr): [nslots][H][DK][DV]
size_t bwd_ckpt_bytes(int nslots, int H, int DK, int DV) {
    return static_cast<size_t>(nslots) * H * DK * DV * sizeof(float);
}

// layout: per-chunk-head blocks | recomputed checkpoints | segment buffers
size_t bwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV) {
    return align256(bwd_workspace_bytes(nslots, H, DK, DV)) + align256(bwd_ckpt_bytes(nslots, H, DK, DV)) +
           seg_buffer_bytes(nsslots_max, H, DK, DV);
}

hipError_t launch_bwd(const BwdArgs& a, int nslots, hipStream_t st) {
    const int NT = (a.T + 63) / 64;
    const int NC = nslots * a.H;
    const int nchains = (a.cu ? a.ndocs : a.B) * a.H;
    const int DK = a.DK, DV = a.DV;
    BwdParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout; p.g = a.g; p.beta = a.beta; p.s = a.s;
    p.h_ckpt = a.h_ckpt; p.dht = a.dht; p.h0 = a.h0; p.scale = a.scale;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
    p.B = a.B; p.T = a.T; p.H = a.H; p.NT = NT; p.cu = a.cu; p.ndocs = a.ndocs; p.head_gate = a.head_gate;
    p.qk_norm = a.qk_norm;
    // dv straight from the dV products when every chunk is whole (the
    // products write all 64 rows of a chunk)
    p.dv_direct = !a.cu && a.T % 64 == 0;
    const size_t blocks = bwd_workspace_bytes(nslots, a.H, DK, DV);
    const size_t seg_off = align256(blocks) + align256(bwd_ckpt_bytes(nslots, a.H, DK, DV));
    {   // segmented reverse pass when the plan takes it and the workspace has room
        const bool varlen = a.cu != nullptr;
        const size_t avail = a.ws_bytes > seg_off ? a.ws_bytes - seg_off : 0;
        auto fits = [&](int G) {
            return seg_buffer_bytes(seg_slots(varlen, a.B, a.T, a.ndocs, G), a.H, DK, DV) <= avail;
        };
        const int BVr = DV < 64 ? DV : 64;
        p.G = plan_segments(chain_chunks(a.cu_host, varlen, a.ndocs, a.B, a.T), a.H, DV / BVr,
                            (DK + BVr - 1) / BVr, kReverseCost, device_cus(st), fits);
        if (p.G > 0) {
            p.nsslots = seg_slots(varlen, a.B, a.T, a.ndocs, p.G);
            float* sb = reinterpret_cast<float*>(static_cast<unsigned char*>(a.ws) + seg_off);
            const size_t per = static_cast<size_t>(p.nsslots) * a.H * DK * DV;
            p.seg_start = sb;
            p.seg_h = sb + per;
            p.seg_p = sb + 2 * per;
        }
    }
    if (NC == 0) {
        // no tokens: dh0 = dht (or 0)
        const size_t n = static_cast<size_t>(nchains) * DK * DV;
        if (a.dh0 && n > 0) {
            hipLaunchKernelGGL(fill_copy_kernel, dim3(static_cast<unsigned>((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                               dim3(256), 0, st, a.dh0, a.dht, n);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    BwdWs W;
    W.carve(static_cast<float*>(a.ws), NC, DK, DV);
    hipError_t e;
#define CKDA_CHECK(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
    if (!a.h_ckpt) {
        // checkpoints recomputed: a forward pass whose chunk records sit in the
        // blocks' first regions (K1 .. dV), whose outputs go to the regions
        // from dSt on (dSt and the [64 x 64] blocks: at least 64 DV floats per
        // chunk-head, all free until the backward's own passes run) and whose
        // checkpoints go to their own area after the blocks; records-only room
        // keeps its state pass on whole chains
        FwdArgs f{};
        f.B = a.B; f.T = a.T; f.H = a.H; f.DK = DK; f.DV = DV; f.bf16 = a.bf16;
        f.head_gate = a.head_gate; f.qk_norm = a.qk_norm;
        f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.s = a.s; f.beta = a.beta; f.scale = a.scale;
        f.h0 = a.h0; f.o = W.dSt; f.ht = nullptr;
        f.h_ckpt = reinterpret_cast<float*>(static_cast<unsigned char*>(a.ws) + align256(blocks));
        f.cu = a.cu; f.cu_host = a.cu_host; f.ndocs = a.ndocs;
        f.ws = a.ws; f.ws_bytes = fwd_workspace_bytes(nslots, a.H, DK, DV, a.bf16);
        CKDA_CHECK(launch_fwd(f, nslots, st));
        p.h_ckpt = f.h_ckpt;
    }
    CKDA_CHECK(launch_chunk_pass(a.bf16, false, p, W, NC, st));
    const long long s64k = 64LL * DK, s64v = 64LL * DV, skv = 1LL * DK * DV, s44 = 4096;
    // A = strict_lower(K1 K2^T), M = lower(Q1 K2^T)
    CKDA_CHECK(gemm(mk(64, 64, DK, W.K1, DK, s64k, false, W.K2, DK, s64k, true, W.A, 64, s44, 1.f, nullptr, 0.f, 1), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, DK, W.Q1, DK, s64k, false, W.K2, DK, s64k, true, W.M, 64, s44, 1.f, nullptr, 0.f, 2), NC, st));
    hipLaunchKernelGGL(bwd_inverse_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // U = T (V - K1 S')
    // S' = Diag(e^m) S of the chunk start, S read from the checkpoints and
    // scaled while staged (checkpoints of unused varlen slots are never
    // written; their products feed nothing)
    const float* ck = p.h_ckpt;
    auto with_em = [&](Gemm g) { g.bs = W.em; g.sBs = DK; return g; };
    CKDA_CHECK(gemm(with_em(mk(64, DV, DK, W.K1, DK, s64k, false, ck, DV, skv, false, W.R, DV, s64v, -1.f, W.V, 1.f)),
                    NC, st));
    CKDA_CHECK(gemm(mk(64, DV, 64, W.T, 64, s44, false, W.R, DV, s64v, false, W.U, DV, s64v), NC, st));
    // reverse recurrence: dSt, dU per chunk, dh0
    CKDA_CHECK(launch_reverse(p, W, a.bf16, st));
    // chunk-parallel gradients
    CKDA_CHECK(gemm(mk(64, 64, DV, W.dO, DV, s64v, false, W.U, DV, s64v, true, W.dM, 64, s44, 1.f, nullptr, 0.f, 2), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, DV, W.U, DV, s64v, false, W.dSt, DV, skv, true, W.dKB, DK, s64k), NC, st));
    CKDA_CHECK(gemm(with_em(mk(64, DK, DV, W.dU, DV, s64v, false, ck, DV, skv, true, W.dW, DK, s64k, -1.f)), NC, st));
    if (p.dv_direct) {   // chunk-head (b H + h) NT + j: 64 whole rows of dv from token b T + 64 j
        Gemm g = mk(64, DV, 64, W.T, 64, s44, true, W.dU, DV, s64v, false, a.dv, a.H * DV, 64LL * a.H * DV);
        g.cn1 = NT; g.cn2 = a.H; g.cs1 = DV; g.cs2 = static_cast<long long>(a.T) * a.H * DV;
        CKDA_CHECK(gemm(g, NC, st));
    } else {
        CKDA_CHECK(gemm(mk(64, DV, 64, W.T, 64, s44, true, W.dU, DV, s64v, false, W.dV, DV, s64v), NC, st));
    }
    // dT = dU V^T + dW K1^T
    CKDA_CHECK(gemm2(mk(64, 64, DV, W.dU, DV, s64v, false, W.V, DV, s64v, true, W.dT, 64, s44),
                     mk(64, 64, DK, W.dW, DK, s64k, false, W.K1, DK, s64k, true, W.dT, 64, s44), NC, st));
    hipLaunchKernelGGL(bwd_dbeta1_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // dX = -Xi^T (Y1 Xi^T)
    CKDA_CHECK(gemm(mk(64, 64, 64, W.Y1, 64, s44, false, W.Xi, 64, s44, true, W.Tmp, 64, s44), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, 64, W.Xi, 64, s44, true, W.Tmp, 64, s44, false, W.dX, 64, s44, -1.f), NC, st));
    hipLaunchKernelGGL(bwd_dA_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // dK1 = T^T dW + dA K2 ; dK2 = dA^T K1 + dM^T Q1 ; dQ1 = dM K2 + dO S'^T
    CKDA_CHECK(gemm2(mk(64, DK, 64, W.T, 64, s44, true, W.dW, DK, s64k, false, W.dK1, DK, s64k),
                     mk(64, DK, 64, W.dA, 64, s44, false, W.K2, DK, s64k, false, W.dK1, DK, s64k), NC, st));
    CKDA_CHECK(gemm2(mk(64, DK, 64, W.dA, 64, s44, true, W.K1, DK, s64k, false, W.dK2, DK, s64k),
                     mk(64, DK, 64, W.dM, 64, s44, true, W.Q1, DK, s64k, false, W.dK2, DK, s64k), NC, st));
    CKDA_CHECK(gemm2(mk(64, DK, 64, W.dM, 64, s44, false, W.K2, DK, s64k, false, W.dQ1, DK, s64k),
                     with_em(mk(64, DK, DV, W.dO, DV, s64v, false, ck, DV, skv, true, W.dQ1, DK, s64k)), NC, st));
    CKDA_CHECK(launch_chunk_pass(a.bf16, true, p, W, NC, st));
    CKDA_CHECK(hipGetLastError());
#undef CKDA_CHECK
    return hipSuccess;
}

}  // namespace ckda
