// conv.hip -- the optional short convolution of the pre-mixer prep: a
// depthwise causal convolution of width 4 over tokens, one filter per channel
// ("complex-kda-1.3B-100B" model card, Architecture: a short convolution of
// width 4), optionally followed by SiLU:
//   z_t[c] = sum_{j=0..3} w[c][j] x_{t-3+j}[c],   y_t = z_t or z_t sigmoid(z_t)
// with the history before a sequence (or document) zero, or the three inputs
// that preceded it (a carried window, [3][C] per sequence).
//
// The work is a stream over [T][C] with no reuse beyond three tokens, so the
// kernels are laid out for HBM, not for the matrix cores: a thread takes four
// adjacent channels (one 8- or 16-byte access per token row, a wave covering
// 256 contiguous channels) and a run of 64 tokens, keeping the last three
// inputs in registers.  blockIdx.x is the token run (or the sequence), y the
// group of 1024 channels, so every thread of a workgroup shares its token run
// and document switches are uniform branches.
//
// Backward: dz = dy act'(z), dx_t = sum_j w_j dz_{t+3-j} (inside the
// document), dw_j = sum_t dz_t x_{t-3+j}, and the window's gradient from the
// first three tokens of each document.  dw is summed per 64-token run into a
// workspace, then over the runs in a fixed order (deterministic).
#include "ckda_conv.h"
#include "ckda_device.h"

namespace ckda {

namespace {

constexpr int kConvThreads = 256;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Vec4<bf16_t> {
    static __device__ __forceinline__ f32x4 load(const bf16_t* p) {
        const u32x2 u = *reinterpret_cast<const u32x2*>(p);
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ void store(bf16_t* p, f32x4 v) {
        *reinterpret_cast<u32x2*>(p) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
    }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float sigmoid_f(float z) {
    return 1.f / (1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// The document holding token t (t < T): d, its first token and its end.
struct Doc {
    int d, beg, end;
};
__device__ __forceinline__ Doc doc_of(const ConvArgs& a, int t) {
    if (!a.cu) {
        const int L = a.T / a.N;
        const int d = t / L;
        return Doc{d, d * L, d * L + L};
    }
    // the last document whose start is <= t: it is the non-empty one holding t
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return Doc{lo, a.cu[lo], a.cu[lo + 1]};
}
// the document that starts at token t = (previous document's end), skipping empty ones
__device__ __forceinline__ Doc doc_next(const ConvArgs& a, Doc D) {
    if (!a.cu) return Doc{D.d + 1, D.end, D.end + (D.end - D.beg)};
    int d = D.d + 1;
    while (a.cu[d + 1] <= D.end) ++d;
    return Doc{d, a.cu[d], a.cu[d + 1]};
}

// input at token t of document D (t >= D.beg - 3): x, or the window row, or 0
template <typename Tin>
__device__ __forceinline__ f32x4 input_at(const ConvArgs& a, const Doc& D, int t, int c) {
    if (t >= D.beg) return Vec4<Tin>::load(static_cast<const Tin*>(a.x) + static_cast<size_t>(t) * a.C + c);
    if (!a.state0) return zero4();
    return Vec4<Tin>::load(static_cast<const Tin*>(a.state0) +
                           (static_cast<size_t>(D.d) * (kConvWidth - 1) + (kConvWidth - 1) + (t - D.beg)) * a.C + c);
}

// taps of channels c .. c+3: wt[j][e] = w[c + e][j]
__device__ __forceinline__ void load_taps(const float* w, int c, f32x4 (&wt)[kConvWidth]) {
    f32x4 r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = *reinterpret_cast<const f32x4*>(w + static_cast<size_t>(c + e) * kConvWidth);
#pragma unroll
    for (int j = 0; j < kConvWidth; ++j) wt[j] = f32x4{r[0][j], r[1][j], r[2][j], r[3][j]};
}

__device__ __forceinline__ f32x4 conv4(const f32x4 (&wt)[kConvWidth], f32x4 h3, f32x4 h2, f32x4 h1, f32x4 x) {
    f32x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = fmaf(wt[3][e], x[e], fmaf(wt[2][e], h1[e], fmaf(wt[1][e], h2[e], wt[0][e] * h3[e])));
    return z;
}

__device__ __forceinline__ f32x4 act4(f32x4 z, bool silu) {
    if (!silu) return z;
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = z[e] * sigmoid_f(z[e]);
    return y;
}

// d act / dz
__device__ __forceinline__ f32x4 dact4(f32x4 z, bool silu) {
    if (!silu) return f32x4{1.f, 1.f, 1.f, 1.f};
    f32x4 g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float s = sigmoid_f(z[e]);
        g[e] = s * (1.f + z[e] * (1.f - s));
    }
    return g;
}

// ---- forward: y over one 64-token run of 4 channels per thread -------------
template <typename Tin>
__global__ void __launch_bounds__(kConvThreads) conv_fwd_kernel(ConvArgs a) {
    const int c = 4 * (blockIdx.y * kConvThreads + static_cast<int>(threadIdx.x));
    if (c >= a.C) return;   // (no barriers below)
    const int t0 = blockIdx.x * kConvSeg, t1 = min(t0 + kConvSeg, a.T);
    f32x4 wt[kConvWidth];
    load_taps(a.w, c, wt);
    Doc D = doc_of(a, t0);
    f32x4 h1 = input_at<Tin>(a, D, t0 - 1, c), h2 = input_at<Tin>(a, D, t0 - 2, c), h3 = input_at<Tin>(a, D, t0 - 3, c);
    const Tin* x = static_cast<const Tin*>(a.x);
    Tin* y = static_cast<Tin*>(a.y);
    constexpr int G = 8;   // tokens whose loads are issued together
    for (int t = t0; t < t1;) {
        if (t + G <= t1 && t + G <= D.end) {   // no document starts inside the group (uniform)
            f32x4 xs[G];
#pragma unroll
            for (int i = 0; i < G; ++i) xs[i] = Vec4<Tin>::load(x + static_cast<size_t>(t + i) * a.C + c);
#pragma unroll
            for (int i = 0; i < G; ++i) {
                Vec4<Tin>::store(y + static_cast<size_t>(t + i) * a.C + c, act4(conv4(wt, h3, h2, h1, xs[i]), a.silu));
                h3 = h2;
                h2 = h1;
                h1 = xs[i];
            }
            t += G;
            continue;
        }
        if (t == D.end) {   // uniform over the launch column
            D = doc_next(a, D);
            h1 = input_at<Tin>(a, D, t - 1, c);
            h2 = input_at<Tin>(a, D, t - 2, c);
            h3 = input_at<Tin>(a, D, t - 3, c);
        }
        const size_t o = static_cast<size_t>(t) * a.C + c;
        const f32x4 xt = Vec4<Tin>::load(x + o);
        Vec4<Tin>::store(y + o, act4(conv4(wt, h3, h2, h1, xt), a.silu));
        h3 = h2;
        h2 = h1;
        h1 = xt;
        ++t;
    }
}

// ---- per document: the outgoing window (forward) or the incoming window's
// gradient (backward), one thread per (document, 4 channels) ----------------
template <typename Tin>
__global__ void __launch_bounds__(kConvThreads) conv_window_kernel(ConvArgs a, int backward) {
    const int c = 4 * (blockIdx.y * kConvThreads + static_cast<int>(threadIdx.x));
    const int d = blockIdx.x;
    if (c >= a.C) return;
    Doc D;
    if (a.cu) D = Doc{d, a.cu[d], a.cu[d + 1]};
    else D = Doc{d, d * (a.T / a.N), (d + 1) * (a.T / a.N)};
    const int L = D.end - D.beg;
    if (!backward) {
        // row j = input at token end - 3 + j (rows are read before any is
        // written over, so the output may be the incoming window itself)
        f32x4 r[kConvWidth - 1];
#pragma unroll
        for (int j = 0; j < kConvWidth - 1; ++j) r[j] = input_at<Tin>(a, D, D.end - (kConvWidth - 1) + j, c);
        Tin* so = static_cast<Tin*>(a.state_out);
#pragma unroll
        for (int j = 0; j < kConvWidth - 1; ++j)
            Vec4<Tin>::store(so + (static_cast<size_t>(d) * (kConvWidth - 1) + j) * a.C + c, r[j]);
        return;
    }
    // dstate0 row i = sum_{j <= i} w_j dz_{beg + i - j} (tokens inside the document)
    f32x4 wt[kConvWidth];
    load_taps(a.w, c, wt);
    f32x4 hx[2 * kConvWidth - 1];   // inputs at beg - 3 .. beg + 2 (index + 3)
#pragma unroll
    for (int i = 0; i < 2 * kConvWidth - 2; ++i)
        hx[i] = (i < kConvWidth - 1 || i - (kConvWidth - 1) < L) ? input_at<Tin>(a, D, D.beg - (kConvWidth - 1) + i, c)
                                                                 : zero4();
    f32x4 dz[kConvWidth - 1];
#pragma unroll
    for (int i = 0; i < kConvWidth - 1; ++i) {
        if (i < L) {
            const f32x4 z = conv4(wt, hx[i], hx[i + 1], hx[i + 2], hx[i + 3]);
            const f32x4 g = Vec4<float>::load(a.dy + static_cast<size_t>(D.beg + i) * a.C + c);
            const f32x4 da = dact4(z, a.silu);
#pragma unroll
            for (int e = 0; e < 4; ++e) dz[i][e] = g[e] * da[e];
        } else {
            dz[i] = zero4();
        }
    }
#pragma unroll
    for (int i = 0; i < kConvWidth - 1; ++i) {
        f32x4 s = zero4();
#pragma unroll
        for (int j = 0; j <= i; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[e] = fmaf(wt[j][e], dz[i - j][e], s[e]);
        Vec4<float>::store(a.dstate0 + (static_cast<size_t>(d) * (kConvWidth - 1) + i) * a.C + c, s);
    }
}

// ---- backward over one run: dx, and this run's part of dw ------------------
template <typename Tin>
__global__ void __launch_bounds__(kConvThreads) conv_bwd_kernel(ConvArgs a) {
    const int c = 4 * (blockIdx.y * kConvThreads + static_cast<int>(threadIdx.x));
    if (c >= a.C) return;
    const int t0 = blockIdx.x * kConvSeg, t1 = min(t0 + kConvSeg, a.T);
    f32x4 wt[kConvWidth];
    load_taps(a.w, c, wt);
    Doc D = doc_of(a, t0);
    f32x4 h1 = input_at<Tin>(a, D, t0 - 1, c), h2 = input_at<Tin>(a, D, t0 - 2, c), h3 = input_at<Tin>(a, D, t0 - 3, c);
    const Tin* x = static_cast<const Tin*>(a.x);
    f32x4 dw[kConvWidth];
#pragma unroll
    for (int j = 0; j < kConvWidth; ++j) dw[j] = zero4();
    // dz of tokens t-3 .. t (z0 oldest) with their documents (-1: past the end)
    f32x4 z0 = zero4(), z1 = zero4(), z2 = zero4(), z3 = zero4();
    int d0 = -1, d1 = -1, d2 = -1, d3 = -1;
    const int tend = t1 + kConvWidth - 1;   // dz up to t1 + 2 feeds dx of the run's last tokens
    // one token: dz from its input, dy and history; dw; the ring; dx of t - 3
    auto token = [&](int t, bool real, f32x4 xt, f32x4 g) {
        f32x4 dz = zero4();
        int dd = -1;
        if (real) {
            const f32x4 da = dact4(conv4(wt, h3, h2, h1, xt), a.silu);
#pragma unroll
            for (int e = 0; e < 4; ++e) dz[e] = g[e] * da[e];
            dd = D.d;
            if (t < t1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dw[0][e] = fmaf(dz[e], h3[e], dw[0][e]);
                    dw[1][e] = fmaf(dz[e], h2[e], dw[1][e]);
                    dw[2][e] = fmaf(dz[e], h1[e], dw[2][e]);
                    dw[3][e] = fmaf(dz[e], xt[e], dw[3][e]);
                }
            }
            h3 = h2;
            h2 = h1;
            h1 = xt;
        }
        z0 = z1; z1 = z2; z2 = z3; z3 = dz;
        d0 = d1; d1 = d2; d2 = d3; d3 = dd;
        if (t >= t0 + kConvWidth - 1) {   // token t - 3 has all its dz: dx_{t-3}
            const int tt = t - (kConvWidth - 1);
            const float m1 = d1 == d0 ? 1.f : 0.f, m2 = d2 == d0 ? 1.f : 0.f, m3 = d3 == d0 ? 1.f : 0.f;
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r[e] = fmaf(wt[0][e], m3 * z3[e], fmaf(wt[1][e], m2 * z2[e], fmaf(wt[2][e], m1 * z1[e], wt[3][e] * z0[e])));
            Vec4<float>::store(a.dx + static_cast<size_t>(tt) * a.C + c, r);
        }
    };
    constexpr int G = 4;   // tokens whose loads are issued together
    for (int t = t0; t < tend;) {
        if (t + G <= t1 && t + G <= D.end) {   // real tokens of one document, all in the run (uniform)
            f32x4 xs[G], gs[G];
#pragma unroll
            for (int i = 0; i < G; ++i) {
                const size_t o = static_cast<size_t>(t + i) * a.C + c;
                xs[i] = Vec4<Tin>::load(x + o);
                gs[i] = Vec4<float>::load(a.dy + o);
            }
#pragma unroll
            for (int i = 0; i < G; ++i) token(t + i, true, xs[i], gs[i]);
            t += G;
            continue;
        }
        if (t < a.T) {   // uniform over the launch column
            if (t == D.end) {
                D = doc_next(a, D);
                h1 = input_at<Tin>(a, D, t - 1, c);
                h2 = input_at<Tin>(a, D, t - 2, c);
                h3 = input_at<Tin>(a, D, t - 3, c);
            }
            const size_t o = static_cast<size_t>(t) * a.C + c;
            token(t, true, Vec4<Tin>::load(x + o), Vec4<float>::load(a.dy + o));
        } else {
            token(t, false, zero4(), zero4());
        }
        ++t;
    }
    float* pp = a.partial + static_cast<size_t>(blockIdx.x) * a.C * kConvWidth + static_cast<size_t>(c) * kConvWidth;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4*>(pp + e * kConvWidth) = f32x4{dw[0][e], dw[1][e], dw[2][e], dw[3][e]};
}

// dw[i] = sum over the runs of partial[run][i], in a fixed order: a
// workgroup takes 32 columns (8 float4 quads) and 32 row groups; row group g
// sums runs g, g + 32, ..., then the 32 group sums are added in order.
constexpr int kDwQuads = 8, kDwGroups = 32;
__global__ void __launch_bounds__(kDwQuads * kDwGroups) conv_dw_kernel(const float* partial, int nrun, int n, float* dw) {
    __shared__ f32x4 red[kDwGroups][kDwQuads];
    const int q = static_cast<int>(threadIdx.x) % kDwQuads, g = static_cast<int>(threadIdx.x) / kDwQuads;
    const int col = 4 * (blockIdx.x * kDwQuads + q);   // n is a multiple of 16
    f32x4 acc = zero4();
    if (col < n) {
        int r = g;
        for (; r + 3 * kDwGroups < nrun; r += 4 * kDwGroups) {   // four loads in flight
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(partial + static_cast<size_t>(r) * n + col);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(partial + static_cast<size_t>(r + kDwGroups) * n + col);
            const f32x4 a2 = *reinterpret_cast<const f32x4*>(partial + static_cast<size_t>(r + 2 * kDwGroups) * n + col);
            const f32x4 a3 = *reinterpret_cast<const f32x4*>(partial + static_cast<size_t>(r + 3 * kDwGroups) * n + col);
            acc += a0;
            acc += a1;
            acc += a2;
            acc += a3;
        }
        for (; r < nrun; r += kDwGroups) acc += *reinterpret_cast<const f32x4*>(partial + static_cast<size_t>(r) * n + col);
    }
    red[g][q] = acc;
    __syncthreads();
    if (g == 0 && col < n) {
        f32x4 s = red[0][q];
        for (int k = 1; k < kDwGroups; ++k) s += red[k][q];
        *reinterpret_cast<f32x4*>(dw + col) = s;
    }
}

// ---- one decode step per (sequence, 4 channels) ----------------------------
template <typename Tin>
__global__ void __launch_bounds__(kConvThreads) conv_step_kernel(int N, int C, int silu, const Tin* x, const float* w,
                                                                 Tin* window, Tin* y) {
    const int c = 4 * (blockIdx.y * kConvThreads + static_cast<int>(threadIdx.x));
    const int n = blockIdx.x;
    if (c >= C || n >= N) return;
    f32x4 wt[kConvWidth];
    load_taps(w, c, wt);
    Tin* wn = window + static_cast<size_t>(n) * (kConvWidth - 1) * C + c;
    const f32x4 r0 = Vec4<Tin>::load(wn), r1 = Vec4<Tin>::load(wn + C), r2 = Vec4<Tin>::load(wn + 2 * C);
    const f32x4 xt = Vec4<Tin>::load(x + static_cast<size_t>(n) * C + c);
    Vec4<Tin>::store(y + static_cast<size_t>(n) * C + c, act4(conv4(wt, r0, r1, r2, xt), silu != 0));
    Vec4<Tin>::store(wn, r1);
    Vec4<Tin>::store(wn + C, r2);
    Vec4<Tin>::store(wn + 2 * C, xt);
}

template <typename Tin>
hipError_t conv_fwd_t(const ConvArgs& a, hipStream_t st) {
    const unsigned gy = static_cast<unsigned>((a.C / 4 + kConvThreads - 1) / kConvThreads);
    if (a.T > 0) {
        hipLaunchKernelGGL(conv_fwd_kernel<Tin>, dim3(static_cast<unsigned>((a.T + kConvSeg - 1) / kConvSeg), gy),
                           dim3(kConvThreads), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.state_out && a.N > 0) {
        hipLaunchKernelGGL(conv_window_kernel<Tin>, dim3(static_cast<unsigned>(a.N), gy), dim3(kConvThreads), 0, st, a, 0);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename Tin>
hipError_t conv_bwd_t(const ConvArgs& a, hipStream_t st) {
    const unsigned gy = static_cast<unsigned>((a.C / 4 + kConvThreads - 1) / kConvThreads);
    const int nrun = (a.T + kConvSeg - 1) / kConvSeg;
    hipError_t e;
    if (a.T > 0) {
        hipLaunchKernelGGL(conv_bwd_kernel<Tin>, dim3(static_cast<unsigned>(nrun), gy), dim3(kConvThreads), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int n = a.C * kConvWidth;
    hipLaunchKernelGGL(conv_dw_kernel, dim3(static_cast<unsigned>((n / 4 + kDwQuads - 1) / kDwQuads)),
                       dim3(kDwQuads * kDwGroups), 0, st, a.partial, nrun, n, a.dw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.dstate0 && a.N > 0) {
        hipLaunchKernelGGL(conv_window_kernel<Tin>, dim3(static_cast<unsigned>(a.N), gy), dim3(kConvThreads), 0, st, a, 1);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
    return a.bf16 ? conv_fwd_t<bf16_t>(a, st) : conv_fwd_t<float>(a, st);
}

hipError_t launch_conv_bwd(const ConvArgs& a, hipStream_t st) {
    return a.bf16 ? conv_bwd_t<bf16_t>(a, st) : conv_bwd_t<float>(a, st);
}

hipError_t launch_conv_step(int N, int C, bool bf16, bool silu, const void* x, const float* w, void* window,
                            void* y, hipStream_t st) {
    if (N == 0 || C == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(N), static_cast<unsigned>((C / 4 + kConvThreads - 1) / kConvThreads));
    if (bf16)
        hipLaunchKernelGGL(conv_step_kernel<bf16_t>, grid, dim3(kConvThreads), 0, st, N, C, silu ? 1 : 0,
                           static_cast<const bf16_t*>(x), w, static_cast<bf16_t*>(window), static_cast<bf16_t*>(y));
    else
        hipLaunchKernelGGL(conv_step_kernel<float>, grid, dim3(kConvThreads), 0, st, N, C, silu ? 1 : 0,
                           static_cast<const float*>(x), w, static_cast<float*>(window), static_cast<float*>(y));
    return hipGetLastError();
}

}  // namespace ckda
