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

namespace ckda {

namespace {

// Workspace layout (floats), per chunk-head ch (NC = B*H*NT of them).
struct BwdWs {
    int NC, DK, DV;
    float* base;
    // [NC][64][DK]
    float *K1, *K2, *Q1, *KB, *Bb, *Pp, *dKB, *dW, *dK1, *dK2, *dQ1;
    // [NC][64][DV]
    float *V, *dO, *R, *U, *dU, *dV;
    // [NC][DK][DV]
    float *Sp, *dSt;
    // [NC][64][64]
    float *A, *M, *Xi, *T, *dM, *dT, *Y1, *Tmp, *dX, *dA;
    // [NC][DK]
    float *em, *gC, *pC;
    // [NC][64]
    float *beta, *dbeta1, *dbeta2;

    __host__ __device__ static size_t floats(size_t NC, int DK, int DV) {
        return NC * (11ull * 64 * DK + 6ull * 64 * DV + 2ull * DK * DV + 10ull * 64 * 64 + 3ull * DK + 3ull * 64);
    }
    __host__ void carve(float* p, int nc, int dk, int dv) {
        NC = nc; DK = dk; DV = dv; base = p;
        const size_t n = nc;
        auto take = [&](size_t cnt) { float* r = p; p += cnt; return r; };
        K1 = take(n * 64 * dk); K2 = take(n * 64 * dk); Q1 = take(n * 64 * dk); KB = take(n * 64 * dk);
        Bb = take(n * 64 * dk); Pp = take(n * 64 * dk); dKB = take(n * 64 * dk); dW = take(n * 64 * dk);
        dK1 = take(n * 64 * dk); dK2 = take(n * 64 * dk); dQ1 = take(n * 64 * dk);
        V = take(n * 64 * dv); dO = take(n * 64 * dv); R = take(n * 64 * dv); U = take(n * 64 * dv);
        dU = take(n * 64 * dv); dV = take(n * 64 * dv);
        Sp = take(n * dk * dv); dSt = take(n * dk * dv);
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

__device__ __forceinline__ void stage_slab(float* dst, int pitch, const float* src, int rows, int cols, int ld, int r0,
                                           int c0) {
    // copy src[(r0 + r) * ld + c0 + c] for r < rows, c < cols (a multiple of 4) into dst[r * pitch + c]
    const int q = cols / 4;
    for (int e = threadIdx.x; e < rows * q; e += 256) {
        const int r = e / q, c4 = (e % q) * 4;
        const float4 v = *reinterpret_cast<const float4*>(src + static_cast<size_t>(r0 + r) * ld + c0 + c4);
        *reinterpret_cast<float4*>(dst + r * pitch + c4) = v;
    }
}

template <bool aT, bool bT, int NT>   // aT: A stored transposed, bT: B stored transposed, NT = N / 16
__global__ void __launch_bounds__(256) bgemm_kernel(Gemm p) {
    __shared__ __align__(16) float As[64 * kPK > kKS * kPN ? 64 * kPK : kKS * kPN];
    __shared__ __align__(16) float Bs[128 * kPK > 2 * kKS * kPN ? 128 * kPK : 2 * kKS * kPN];
    const long long z = blockIdx.x;
    const float* A = p.A + z * p.sA;
    const float* B = p.B + z * p.sB;
    float* C = p.C + z * p.sC;
    const float* D = p.D ? p.D + z * p.sD : nullptr;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 15, g = l >> 4;
    // A transposed: element (i, k) at k * ac + i; B transposed: element (k, j) at j * bc + k
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < p.K; k0 += kKS) {
        if constexpr (!aT) stage_slab(As, kPK, A, 64, kKS, p.ar, 0, k0);      // As[i][k]
        else stage_slab(As, kPN, A, kKS, 64, p.ac, k0, 0);                    // As[k][i]
        if constexpr (!bT) {                                                   // Bs[k][j], 64-wide blocks of j
#pragma unroll
            for (int h = 0; h < 16 * NT; h += 64)
                stage_slab(Bs + (h / 64) * kKS * kPN, kPN, B, kKS, 16 * NT - h < 64 ? 16 * NT - h : 64, p.br, k0, h);
        } else {                                                               // Bs[j][k]
            stage_slab(Bs, kPK, B, 16 * NT, kKS, p.bc, 0, k0);
        }
        __syncthreads();
#pragma unroll 2
        for (int kk = 0; kk < kKS; kk += 4) {
            const int i = 16 * w + n, k = kk + g;
            const float a = aT ? As[k * kPN + i] : As[i * kPK + k];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int j = 16 * t + n;
                const float b = bT ? Bs[j * kPK + k] : Bs[(t / 4) * kKS * kPN + k * kPN + (j % 64)];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();
    }
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

hipError_t gemm(const Gemm& g, int nbatch, hipStream_t st) {
    // shapes used by the backward: M = 64, N and K in {32, 64, 128}
    auto ok = [](int x) { return x == 32 || x == 64 || x == 128; };
    if (g.M != 64 || !ok(g.N) || !ok(g.K)) return hipErrorInvalidValue;
    const bool aT = g.ar == 1, bT = g.bc != 1;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(nbatch), dim3(256), 0, st, g); };
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
};

// chunk-head ch -> (b, h, chunk j, first token, valid tokens)
struct ChunkIdx {
    int b, h, j, t0, L;
    __device__ ChunkIdx(int ch, int H, int NT, int T) {
        j = ch % NT;
        const int bh = ch / NT;
        h = bh % H;
        b = bh / H;
        t0 = j * 64;
        L = min(64, T - t0);
    }
};

// ---------------------------------------------------------------------------
// prep: chunk-local cumulative gate, sign product and anchored operands
// ---------------------------------------------------------------------------
template <typename Tin>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p, BwdWs W) {
    const int ch = blockIdx.x;
    const int DK = W.DK, DV = W.DV;
    const ChunkIdx ci(ch, p.H, p.NT, p.T);
    const int c = threadIdx.x;
    const size_t trow0 = static_cast<size_t>(ci.b) * p.T + ci.t0;   // token row of the chunk start
    const size_t o64k = static_cast<size_t>(ch) * 64 * DK;
    const size_t o64v = static_cast<size_t>(ch) * 64 * DV;
    if (c < DK) {
        float run = 0.f, par = 1.f;
        for (int t = 0; t < 64; ++t) {
            if (t < ci.L) {
                const size_t e = ((trow0 + t) * p.H + ci.h) * DK + c;
                run += p.g[e];
                par *= static_cast<float>(p.s[e]);
            }
            W.Bb[o64k + t * DK + c] = run;
            W.Pp[o64k + t * DK + c] = par;
        }
        const float m = W.Bb[o64k + min(31, ci.L - 1) * DK + c];
        const float bL = run;
        for (int t = 0; t < 64; ++t) {
            float K1 = 0.f, K2 = 0.f, Q1 = 0.f, KB = 0.f;
            if (t < ci.L) {
                const size_t e = ((trow0 + t) * p.H + ci.h) * DK + c;
                const float b = W.Bb[o64k + t * DK + c];
                const float P = W.Pp[o64k + t * DK + c];
                const float kf = P * Elem<Tin>::load(static_cast<const Tin*>(p.k), e);
                const float qf = P * Elem<Tin>::load(static_cast<const Tin*>(p.q), e);
                const float e1 = exp2_clamped((b - m) * kLog2e);
                K1 = kf * e1;
                K2 = kf * exp2_clamped((m - b) * kLog2e);
                Q1 = qf * e1;
                KB = kf * exp2_clamped((bL - b) * kLog2e);
            }
            W.K1[o64k + t * DK + c] = K1;
            W.K2[o64k + t * DK + c] = K2;
            W.Q1[o64k + t * DK + c] = Q1;
            W.KB[o64k + t * DK + c] = KB;
        }
        W.em[static_cast<size_t>(ch) * DK + c] = exp2_clamped(m * kLog2e);
        W.gC[static_cast<size_t>(ch) * DK + c] = exp2_clamped(bL * kLog2e);
        W.pC[static_cast<size_t>(ch) * DK + c] = par;
    }
    if (c < DV) {
        for (int t = 0; t < 64; ++t) {
            float vv = 0.f, dd = 0.f;
            if (t < ci.L) {
                const size_t e = ((trow0 + t) * p.H + ci.h) * DV + c;
                vv = Elem<Tin>::load(static_cast<const Tin*>(p.v), e);
                dd = p.scale * Elem<Tin>::load(static_cast<const Tin*>(p.dout), e);
            }
            W.V[o64v + t * DV + c] = vv;
            W.dO[o64v + t * DV + c] = dd;
        }
    }
    if (c < 64) W.beta[static_cast<size_t>(ch) * 64 + c] = (c < ci.L) ? p.beta[(trow0 + c) * p.H + ci.h] : 0.f;
    // S' = Diag(e^m) S for the chunk-start state (h_ckpt is [B,H,NT,DK,DV] = [NC][DK][DV])
    __syncthreads();
    const float* S = p.h_ckpt + static_cast<size_t>(ch) * DK * DV;
    float* Sp = W.Sp + static_cast<size_t>(ch) * DK * DV;
    const float* em = W.em + static_cast<size_t>(ch) * DK;
    for (int e = threadIdx.x; e < DK * DV; e += blockDim.x) Sp[e] = em[e / DV] * S[e];
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
template <int DK, int DV>
struct RevShape {
    static constexpr int BV = DV < 64 ? DV : 64;
    static constexpr int NSL = DV / BV;
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

template <int DK, int DV>
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

    const int bh = blockIdx.x / SH::NSL;
    const int v0 = (blockIdx.x % SH::NSL) * BV;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, n = l & 15, g = l >> 4;
    const int NT = p.NT;

    // ---- register staging ---------------------------------------------------
    f32x4 rM[NM], rT[NM], rKB[NKB], rDO[NDO], rSM;
    f32x4 rQ[NKB], rK[NKB];
    auto load1 = [&](int j) {   // M, T, KB, dO slice, pC / em / gC of chunk j
        const size_t ch = static_cast<size_t>(bh) * NT + j;
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
            rDO[i] = *reinterpret_cast<const f32x4*>(W.dO + ch * 64 * DV + static_cast<size_t>(r) * DV + v0 + 4 * c4);
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
        for (int i = 0; i < NDO; ++i) {
            const int u = tid + 512 * i, r = u / (BV / 4), c4 = u % (BV / 4);
            *reinterpret_cast<f32x4*>(dOs + r * PV + 4 * c4) = rDO[i];
        }
        if (tid < 3 * (DK / 4)) *reinterpret_cast<f32x4*>(pCs + 4 * tid) = rSM;
    };
    auto load2 = [&](int j) {   // Q1, K1 of chunk j
        const size_t ch = static_cast<size_t>(bh) * NT + j;
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

    // G = dht (or 0)
    for (int e = tid; e < DK * BV; e += 512) {
        const int c = e / BV, v = e % BV;
        Gs[c * PV + v] = p.dht ? p.dht[(static_cast<size_t>(bh) * DK + c) * DV + v0 + v] : 0.f;
    }
    load1(NT - 1);
    store1();
    __syncthreads();
    for (int j = NT - 1; j >= 0; --j) {
        const size_t ch = static_cast<size_t>(bh) * NT + j;
        load2(j);
        // dSt = Diag(pC) G to the workspace (slice columns)
        for (int e = tid; e < DK * (BV / 4); e += 512) {
            const int c = e / (BV / 4), c4 = e % (BV / 4);
            const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + c * PV + 4 * c4);
            *reinterpret_cast<f32x4*>(W.dSt + ch * DK * DV + static_cast<size_t>(c) * DV + v0 + 4 * c4) = pCs[c] * gv;
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
        for (int e = tid; e < 64 * (BV / 4); e += 512) {
            const int r = e / (BV / 4), c4 = e % (BV / 4);
            *reinterpret_cast<f32x4*>(W.dU + ch * 64 * DV + static_cast<size_t>(r) * DV + v0 + 4 * c4) =
                *reinterpret_cast<const f32x4*>(UZs + r * PV + 4 * c4);
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
        load1(j > 0 ? j - 1 : 0);
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
        store1();   // chunk j - 1 (on the last chunk: chunk 0 again, unused)
        __syncthreads();
    }
    if (p.dh0) {
        for (int e = tid; e < DK * BV; e += 512) {
            const int c = e / BV, v = e % BV;
            p.dh0[(static_cast<size_t>(bh) * DK + c) * DV + v0 + v] = Gs[c * PV + v];
        }
    }
}

template <int DK, int DV>
static hipError_t launch_reverse_t(const BwdParams& p, const BwdWs& W, hipStream_t st) {
    using SH = RevShape<DK, DV>;
    auto kern = bwd_reverse_kernel<DK, DV>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SH::BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(p.B * p.H * SH::NSL), dim3(512), SH::BYTES, st, p, W);
    return hipGetLastError();
}

static hipError_t launch_reverse(const BwdParams& p, const BwdWs& W, hipStream_t st) {
#define CKDA_REV(DK_, DV_) \
    if (W.DK == DK_ && W.DV == DV_) return launch_reverse_t<DK_, DV_>(p, W, st);
    CKDA_REV(32, 32) CKDA_REV(32, 64) CKDA_REV(32, 128)
    CKDA_REV(64, 32) CKDA_REV(64, 64) CKDA_REV(64, 128)
    CKDA_REV(128, 32) CKDA_REV(128, 64) CKDA_REV(128, 128)
#undef CKDA_REV
    return hipErrorInvalidValue;
}

// dbeta1_i = sum_r dT_ri Xi_ri ; Y1 = dT Diag(beta)
__global__ void __launch_bounds__(256) bwd_dbeta1_kernel(BwdWs W) {
    const size_t ch = blockIdx.x;
    const float* dT = W.dT + ch * 4096;
    const float* Xi = W.Xi + ch * 4096;
    const float* bt = W.beta + ch * 64;
    float* Y1 = W.Y1 + ch * 4096;
    for (int e = threadIdx.x; e < 4096; e += 256) Y1[e] = dT[e] * bt[e % 64];
    if (threadIdx.x < 64) {
        const int i = threadIdx.x;
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) acc += dT[r * 64 + i] * Xi[r * 64 + i];
        W.dbeta1[ch * 64 + i] = acc;
    }
}

// dXs = strict_lower(dX); dbeta2_r = sum_i dXs_ri A_ri; dA = Diag(beta) dXs
__global__ void __launch_bounds__(256) bwd_dA_kernel(BwdWs W) {
    const size_t ch = blockIdx.x;
    const float* dX = W.dX + ch * 4096;
    const float* A = W.A + ch * 4096;
    const float* bt = W.beta + ch * 64;
    float* dA = W.dA + ch * 4096;
    for (int e = threadIdx.x; e < 4096; e += 256) {
        const int r = e / 64, i = e % 64;
        dA[e] = (i < r) ? bt[r] * dX[e] : 0.f;
    }
    if (threadIdx.x < 64) {
        const int r = threadIdx.x;
        float acc = 0.f;
        for (int i = 0; i < r; ++i) acc += dX[r * 64 + i] * A[r * 64 + i];
        W.dbeta2[ch * 64 + r] = acc;
    }
}

// gate gradient, unfold of the sign product, scatter to [B,T,H,.]
__global__ void __launch_bounds__(256) bwd_final_kernel(BwdParams p, BwdWs W) {
    const int ch = blockIdx.x;
    const int DK = W.DK, DV = W.DV;
    const ChunkIdx ci(ch, p.H, p.NT, p.T);
    const size_t trow0 = static_cast<size_t>(ci.b) * p.T + ci.t0;
    const size_t o64k = static_cast<size_t>(ch) * 64 * DK;
    const size_t o64v = static_cast<size_t>(ch) * 64 * DV;
    const int c = threadIdx.x;
    // dGL_c = sum_v dSt[c][v] S[c][v]: row sums read along the rows (coalesced),
    // one wave per row, reduced across the wave
    __shared__ float dgl[128];
    {
        const float* S = p.h_ckpt + static_cast<size_t>(ch) * DK * DV;
        const float* dSt = W.dSt + static_cast<size_t>(ch) * DK * DV;
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        for (int r = w; r < DK; r += 4) {
            float x = 0.f;
            for (int v = l; v < DV; v += 64) x += dSt[r * DV + v] * S[r * DV + v];
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
            if (l == 0) dgl[r] = x;
        }
    }
    __syncthreads();
    if (c < DK) {
        const float dGL = dgl[c];
        const float m = W.Bb[o64k + min(31, ci.L - 1) * DK + c];
        const float bL = W.Bb[o64k + (ci.L - 1) * DK + c];
        float kbsum = 0.f;
        for (int t = 0; t < ci.L; ++t) kbsum += W.KB[o64k + t * DK + c] * W.dKB[o64k + t * DK + c];
        float acc = 0.f;
        for (int t = ci.L - 1; t >= 0; --t) {
            const size_t o = o64k + t * DK + c;
            const float b = W.Bb[o], P = W.Pp[o];
            const float e1 = exp2_clamped((b - m) * kLog2e);
            const float e2 = exp2_clamped((m - b) * kLog2e);
            const float e3 = exp2_clamped((bL - b) * kLog2e);
            const float dq = W.dQ1[o] * e1;
            const float dk = W.dK1[o] * e1 + W.dK2[o] * e2 + W.dKB[o] * e3;
            float db = W.Q1[o] * W.dQ1[o] + W.K1[o] * W.dK1[o] - W.K2[o] * W.dK2[o] - W.KB[o] * W.dKB[o];
            if (t == ci.L - 1) db += kbsum + exp2_clamped(bL * kLog2e) * dGL;
            acc += db;
            const size_t e = ((trow0 + t) * p.H + ci.h) * DK + c;
            p.dq[e] = P * dq;
            p.dk[e] = P * dk;
            p.dg[e] = acc;
        }
    }
    if (c < DV) {
        for (int t = 0; t < ci.L; ++t) p.dv[((trow0 + t) * p.H + ci.h) * DV + c] = W.dV[o64v + t * DV + c];
    }
    if (c < ci.L) {
        const size_t o = static_cast<size_t>(ch) * 64 + c;
        p.dbeta[(trow0 + c) * p.H + ci.h] = W.dbeta1[o] + W.dbeta2[o];
    }
}

// dst = src (or 0 when src is null), n floats
__global__ void fill_copy_kernel(float* dst, const float* src, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int H, int DK, int DV) {
    const size_t NC = static_cast<size_t>(B) * H * ((T + 63) / 64);
    return BwdWs::floats(NC, DK, DV) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    const int NT = (a.T + 63) / 64;
    const int NC = a.B * a.H * NT;
    const int DK = a.DK, DV = a.DV;
    BwdParams p{};
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout; p.g = a.g; p.beta = a.beta; p.s = a.s;
    p.h_ckpt = a.h_ckpt; p.dht = a.dht; p.h0 = a.h0; p.scale = a.scale;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dg = a.dg; p.dbeta = a.dbeta; p.dh0 = a.dh0;
    p.B = a.B; p.T = a.T; p.H = a.H; p.NT = NT;
    if (NC == 0) {
        // no tokens: dh0 = dht (or 0)
        const size_t n = static_cast<size_t>(a.B) * a.H * DK * DV;
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
    if (a.bf16)
        hipLaunchKernelGGL(bwd_prep_kernel<bf16_t>, dim3(NC), dim3(256), 0, st, p, W);
    else
        hipLaunchKernelGGL(bwd_prep_kernel<float>, dim3(NC), dim3(256), 0, st, p, W);
    CKDA_CHECK(hipGetLastError());
    const long long s64k = 64LL * DK, s64v = 64LL * DV, skv = 1LL * DK * DV, s44 = 4096;
    // A = strict_lower(K1 K2^T), M = lower(Q1 K2^T)
    CKDA_CHECK(gemm(mk(64, 64, DK, W.K1, DK, s64k, false, W.K2, DK, s64k, true, W.A, 64, s44, 1.f, nullptr, 0.f, 1), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, DK, W.Q1, DK, s64k, false, W.K2, DK, s64k, true, W.M, 64, s44, 1.f, nullptr, 0.f, 2), NC, st));
    hipLaunchKernelGGL(bwd_inverse_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // U = T (V - K1 S')
    CKDA_CHECK(gemm(mk(64, DV, DK, W.K1, DK, s64k, false, W.Sp, DV, skv, false, W.R, DV, s64v, -1.f, W.V, 1.f), NC, st));
    CKDA_CHECK(gemm(mk(64, DV, 64, W.T, 64, s44, false, W.R, DV, s64v, false, W.U, DV, s64v), NC, st));
    // reverse recurrence: dSt, dU per chunk, dh0
    CKDA_CHECK(launch_reverse(p, W, st));
    // chunk-parallel gradients
    CKDA_CHECK(gemm(mk(64, 64, DV, W.dO, DV, s64v, false, W.U, DV, s64v, true, W.dM, 64, s44, 1.f, nullptr, 0.f, 2), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, DV, W.U, DV, s64v, false, W.dSt, DV, skv, true, W.dKB, DK, s64k), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, DV, W.dU, DV, s64v, false, W.Sp, DV, skv, true, W.dW, DK, s64k, -1.f), NC, st));
    CKDA_CHECK(gemm(mk(64, DV, 64, W.T, 64, s44, true, W.dU, DV, s64v, false, W.dV, DV, s64v), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, DV, W.dU, DV, s64v, false, W.V, DV, s64v, true, W.dT, 64, s44), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, DK, W.dW, DK, s64k, false, W.K1, DK, s64k, true, W.dT, 64, s44, 1.f, W.dT, 1.f), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, 64, W.T, 64, s44, true, W.dW, DK, s64k, false, W.dK1, DK, s64k), NC, st));
    hipLaunchKernelGGL(bwd_dbeta1_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // dX = -Xi^T (Y1 Xi^T)
    CKDA_CHECK(gemm(mk(64, 64, 64, W.Y1, 64, s44, false, W.Xi, 64, s44, true, W.Tmp, 64, s44), NC, st));
    CKDA_CHECK(gemm(mk(64, 64, 64, W.Xi, 64, s44, true, W.Tmp, 64, s44, false, W.dX, 64, s44, -1.f), NC, st));
    hipLaunchKernelGGL(bwd_dA_kernel, dim3(NC), dim3(256), 0, st, W);
    CKDA_CHECK(hipGetLastError());
    // dK1 += dA K2 ; dK2 = dA^T K1 + dM^T Q1 ; dQ1 = dM K2 + dO S'^T
    CKDA_CHECK(gemm(mk(64, DK, 64, W.dA, 64, s44, false, W.K2, DK, s64k, false, W.dK1, DK, s64k, 1.f, W.dK1, 1.f), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, 64, W.dA, 64, s44, true, W.K1, DK, s64k, false, W.dK2, DK, s64k), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, 64, W.dM, 64, s44, true, W.Q1, DK, s64k, false, W.dK2, DK, s64k, 1.f, W.dK2, 1.f), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, 64, W.dM, 64, s44, false, W.K2, DK, s64k, false, W.dQ1, DK, s64k), NC, st));
    CKDA_CHECK(gemm(mk(64, DK, DV, W.dO, DV, s64v, false, W.Sp, DV, skv, true, W.dQ1, DK, s64k, 1.f, W.dQ1, 1.f), NC, st));
    hipLaunchKernelGGL(bwd_final_kernel, dim3(NC), dim3(256), 0, st, p, W);
    CKDA_CHECK(hipGetLastError());
#undef CKDA_CHECK
    return hipSuccess;
}

}  // namespace ckda
