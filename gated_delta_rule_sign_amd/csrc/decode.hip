// decode.hip -- one recurrent CKDA step for N independent sequences.
//
// Recurrent form of the recurrence (paper page, section 1: the models are
// purely recurrent; model card "complex-kda-1.3B-100B": log-magnitude gate,
// sign product pushed onto q and k).  The state is kept in the folded frame
// St = Diag(P) S, so only |alpha| = exp(g) ever multiplies it:
//
//   P  <- P * s                       (running sign product, int8 +-1)
//   kf  = P * k,  qf = P * q,  a = exp(g)
//   x   = St^T (a * kf),  y = St^T (a * qf)        (one read of St)
//   u   = beta * (v - x)
//   o   = scale * (y + (kf . qf) u)
//   St <- Diag(a) St + kf u^T                     (one write of St)
//
// Work split: one 256-thread workgroup per (sequence, head).  Thread t owns
// value columns 4*(t % (DV/4)) .. +3 and a band of DK/RG rows, RG = 256/(DV/4)
// row bands; partial column sums are combined through LDS.  Each state row
// band is streamed with 16-byte loads/stores, a wave covering whole rows.
// The per-row parameters (a, kf, a*kf, a*qf) are formed once, by the first
// DK threads while the state loads are in flight, and shared through LDS.
//
// With q and k normalised in the step (x/||x|| over the key channels, a zero
// vector left at zero) the row parameters keep the raw q and k and the two
// inverse norms ik, iq scale the column sums instead: x and y by ik and iq,
// kf . qf by ik iq, and the state update's kf u^T through u ik.
#include "ckda_device.h"
#include "ckda_launch.h"

namespace ckda {

// HG: one gate per head (g, s [N,H]), broadcast over the channels;
// NQK: q and k L2-normalised per (sequence, head)
// GM: g and beta hold pre-activations (the optional gate map; s unread)
template <typename Tin, int DK, int DV, bool HG, bool NQK, bool GM>
__global__ void __launch_bounds__(256, 4)
decode_step_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                   const float* __restrict__ g, const int8_t* __restrict__ s,
                   const float* __restrict__ beta, float scale, float* __restrict__ state,
                   int8_t* __restrict__ sign_prod, float* __restrict__ o)
{
    constexpr int CG = DV / 4;          // column groups (4 columns each)
    constexpr int RG = 256 / CG;        // row bands
    constexpr int R = DK / RG;          // rows per thread
    constexpr int NWK = (DK + 63) / 64; // waves that hold a row
    static_assert(CG * RG == 256 && R * RG == DK && R >= 1, "tile");

    __shared__ float4 red_x[RG][CG];
    __shared__ float4 red_y[RG][CG];
    __shared__ __align__(16) float row_a[DK], row_kf[DK], row_ak[DK], row_aq[DK];
    __shared__ float red_kq[NWK], red_kk[NWK], red_qq[NWK];

    const int nh = blockIdx.x;                   // n * H + h
    const int t = threadIdx.x;
    const int cg = t % CG;
    const int rg = t / CG;
    const int r0 = rg * R;

    const size_t kbase = static_cast<size_t>(nh) * DK;
    const size_t vbase = static_cast<size_t>(nh) * DV;
    float4* st = reinterpret_cast<float4*>(state + static_cast<size_t>(nh) * DK * DV);

    // row parameters: every thread loads row min(t, DK - 1) (unconditional, so
    // these loads are issued ahead of the state stream and retire first)
    const int tr = t < DK ? t : DK - 1;
    const float gx = HG ? g[nh] : g[kbase + tr];
    // the optional gate map: sign and log-magnitude from the pre-activation
    int s0;
    float g0;
    if constexpr (GM) {
        s0 = gx < 0.f ? -1 : 1;
        g0 = gate_map_g(gx);
    } else {
        s0 = HG ? s[nh] : s[kbase + tr];
        g0 = gx;
    }
    const int sp0 = sign_prod[kbase + tr];
    const float k0 = Elem<Tin>::load(k, kbase + tr), q0 = Elem<Tin>::load(q, kbase + tr);
    float4 S[R];
#pragma unroll
    for (int i = 0; i < R; ++i) S[i] = st[(r0 + i) * CG + cg];
    if (t < NWK * 64) {
        float kq = 0.f, kk = 0.f, qq = 0.f;
        if (t < DK) {
            const int p = sp0 * s0;
            sign_prod[kbase + t] = static_cast<int8_t>(p);
            const float pf = static_cast<float>(p);
            const float a = __builtin_amdgcn_exp2f(g0 * kLog2e);
            const float kf = pf * k0;
            const float qf = pf * q0;
            row_a[t] = a;
            row_kf[t] = kf;
            row_ak[t] = a * kf;
            row_aq[t] = a * qf;
            kq = kf * qf;
            kk = k0 * k0;
            qq = q0 * q0;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            kq += __shfl_xor(kq, off, 64);
            if constexpr (NQK) {
                kk += __shfl_xor(kk, off, 64);
                qq += __shfl_xor(qq, off, 64);
            }
        }
        if ((t & 63) == 0) {
            red_kq[t >> 6] = kq;
            if constexpr (NQK) {
                red_kk[t >> 6] = kk;
                red_qq[t >> 6] = qq;
            }
        }
    }
    __syncthreads();
    float4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const float ak = row_ak[r0 + i], aq = row_aq[r0 + i];
        x.x += ak * S[i].x; x.y += ak * S[i].y; x.z += ak * S[i].z; x.w += ak * S[i].w;
        y.x += aq * S[i].x; y.y += aq * S[i].y; y.z += aq * S[i].z; y.w += aq * S[i].w;
    }
    red_x[rg][cg] = x;
    red_y[rg][cg] = y;
    __syncthreads();
    float4 X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j) {
        const float4 a4 = red_x[j][cg], b4 = red_y[j][cg];
        X.x += a4.x; X.y += a4.y; X.z += a4.z; X.w += a4.w;
        Y.x += b4.x; Y.y += b4.y; Y.z += b4.z; Y.w += b4.w;
    }
    float KQ = 0.f;
#pragma unroll
    for (int j = 0; j < NWK; ++j) KQ += red_kq[j];
    float ik = 1.f;
    if constexpr (NQK) {
        float KK = 0.f, QQ = 0.f;
#pragma unroll
        for (int j = 0; j < NWK; ++j) {
            KK += red_kk[j];
            QQ += red_qq[j];
        }
        ik = inv_norm(KK);
        const float iq = inv_norm(QQ);
        X.x *= ik; X.y *= ik; X.z *= ik; X.w *= ik;
        Y.x *= iq; Y.y *= iq; Y.z *= iq; Y.w *= iq;
        KQ *= ik * iq;
    }
    const float bt = GM ? gate_map_beta(beta[nh]) : beta[nh];
    const int c0 = 4 * cg;
    float4 u;
    u.x = bt * (Elem<Tin>::load(v, vbase + c0 + 0) - X.x);
    u.y = bt * (Elem<Tin>::load(v, vbase + c0 + 1) - X.y);
    u.z = bt * (Elem<Tin>::load(v, vbase + c0 + 2) - X.z);
    u.w = bt * (Elem<Tin>::load(v, vbase + c0 + 3) - X.w);
    if (rg == 0) {
        float4 ov;
        ov.x = scale * (Y.x + KQ * u.x);
        ov.y = scale * (Y.y + KQ * u.y);
        ov.z = scale * (Y.z + KQ * u.z);
        ov.w = scale * (Y.w + KQ * u.w);
        reinterpret_cast<float4*>(o + vbase)[cg] = ov;
    }
    if constexpr (NQK) {   // kf ik u^T
        u.x *= ik; u.y *= ik; u.z *= ik; u.w *= ik;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const float a = row_a[r0 + i], kf = row_kf[r0 + i];
        float4 n;
        n.x = a * S[i].x + kf * u.x;
        n.y = a * S[i].y + kf * u.y;
        n.z = a * S[i].z + kf * u.z;
        n.w = a * S[i].w + kf * u.w;
        st[(r0 + i) * CG + cg] = n;
    }
}

template <typename Tin, int DK, int DV, bool GM>
static hipError_t launch_decode_g(const DecodeArgs& A, hipStream_t stream) {
    auto kern = A.qk_norm ? (A.head_gate ? decode_step_kernel<Tin, DK, DV, true, true, GM>
                                         : decode_step_kernel<Tin, DK, DV, false, true, GM>)
                          : (A.head_gate ? decode_step_kernel<Tin, DK, DV, true, false, GM>
                                         : decode_step_kernel<Tin, DK, DV, false, false, GM>);
    hipLaunchKernelGGL(kern, dim3(A.N * A.H), dim3(256), 0, stream,
                       static_cast<const Tin*>(A.q), static_cast<const Tin*>(A.k),
                       static_cast<const Tin*>(A.v), A.g, A.s, A.beta, A.scale, A.state,
                       A.sign_prod, A.o);
    return hipGetLastError();
}

template <typename Tin, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& A, hipStream_t stream) {
    return A.gate_map ? launch_decode_g<Tin, DK, DV, true>(A, stream) : launch_decode_g<Tin, DK, DV, false>(A, stream);
}

template <typename Tin>
static hipError_t launch_decode_dt(const DecodeArgs& A, hipStream_t stream) {
#define CKDA_DEC(DK_, DV_) \
    if (A.DK == DK_ && A.DV == DV_) return launch_decode_t<Tin, DK_, DV_>(A, stream);
    CKDA_DEC(32, 32) CKDA_DEC(32, 64) CKDA_DEC(32, 128)
    CKDA_DEC(64, 32) CKDA_DEC(64, 64) CKDA_DEC(64, 128)
    CKDA_DEC(128, 32) CKDA_DEC(128, 64) CKDA_DEC(128, 128)
#undef CKDA_DEC
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& A, hipStream_t stream) {
    if (A.N == 0 || A.H == 0) return hipSuccess;
    return A.bf16 ? launch_decode_dt<bf16_t>(A, stream) : launch_decode_dt<float>(A, stream);
}

}  // namespace ckda
