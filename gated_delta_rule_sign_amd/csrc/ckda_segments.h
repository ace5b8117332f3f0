// ckda_segments.h -- segmented (chunk-parallel) passes over long chains,
// shared by the forward's state pass and the backward's reverse pass.
//
// Both passes carry a DK x DV matrix along a chain of chunks with a map that
// is affine in it and acts on its rows (so every value column evolves on its
// own): forward S' = A_c S + B_c, backward G' = A'_c G + B'_c.  A chain is
// cut into segments of G chunks; segment s (in the pass's own order) has map
// X_out = P_s X_in + H_s, where H_s is the segment run from X_in = 0 and P_s
// the same recurrence run on DK "transition" columns started from the
// identity with the inhomogeneous terms switched off.  Segment slot of
// segment s of chain d: floor(cu[d] / 64G) + d + s (equal-length chains:
// d * ceil(NT / G) + s), as chunk slots do with 64.
#pragma once
#include <algorithm>
#include <vector>

#include "ckda_device.h"

namespace ckda {

// first segment slot of chain d (varlen document start cu_d)
__host__ __device__ inline int seg_slot0(int cu_d, int d, int G) { return cu_d / (64 * G) + d; }

struct SegScanParams {
    const int32_t* cu;   // varlen document starts, or nullptr (equal-length)
    int T, H, G;
    float* start;        // [nsslots][H][DK][DV]: X_in of each segment
    const float* hs;     // [nsslots][H][DK][DV]: H_s
    const float* ps;     // [nsslots][H][DK][DK]: P_s
    int reverse;         // 0: the pass runs segments 0, 1, ..; 1: n-1, n-2, ..
};

// Phase 2 of a segmented pass: per (chain, head, 16-column slice) of a chain
// with more than two segments, the middle segments chain the starts.  In
// pass order the first segment's end state is already the second's start
// (written by phase 1); then start_next(s) = P_s start_s + H_s for every
// middle segment s (forward: s = 1 .. n-2 into s + 1; reverse: s = n-2 .. 1
// into s - 1).  fp32 FMA: thread t owns row t/2, columns 8(t%2) .. +7 of the
// slice; it holds its row of P_s in flight at once (L2 latency once per step)
// and reads the slice of start_s from LDS (two addresses per wave:
// broadcasts).
constexpr int kScanCols = 16;
template <int DK, int DV>
__global__ void __launch_bounds__(256) ckda_seg_scan_kernel(SegScanParams p)
{
    constexpr int NSL = DV / kScanCols, NTH = 2 * DK;
    static_assert(NTH <= 256, "threads");
    __shared__ __align__(16) float Ssl[DK * kScanCols];   // the slice of start_s
    const int H = p.H;
    const int slice = blockIdx.x % NSL;
    const int h = (blockIdx.x / NSL) % H;
    const int d = blockIdx.x / (NSL * H);
    const int NTC = (p.T + 63) / 64;
    int len, ss0;
    if (p.cu) {
        len = p.cu[d + 1] - p.cu[d];
        ss0 = seg_slot0(p.cu[d], d, p.G);
    } else {
        len = p.T;
        ss0 = d * ((NTC + p.G - 1) / p.G);
    }
    const int nseg = ((len + 63) / 64 + p.G - 1) / p.G;
    if (nseg <= 2) return;
    const int tid = threadIdx.x;
    const int c0 = slice * kScanCols;
    const size_t sdv = static_cast<size_t>(DK) * DV;
    const int step = p.reverse ? -1 : 1;
    const int sfirst = p.reverse ? nseg - 2 : 1;
    {   // the start of the first middle segment
        const float* src = p.start + (static_cast<size_t>(ss0 + sfirst) * H + h) * sdv;
        for (int e = tid; e < DK * kScanCols; e += 256)
            Ssl[e] = src[static_cast<size_t>(e / kScanCols) * DV + c0 + e % kScanCols];
    }
    __syncthreads();
    const int r = tid >> 1, cb = 8 * (tid & 1);
    for (int m = 0, sgi = sfirst; m < nseg - 2; ++m, sgi += step) {
        const size_t it = static_cast<size_t>(ss0 + sgi) * H + h;
        float acc[8];
        if (tid < NTH) {
            const float* Hs = p.hs + it * sdv + static_cast<size_t>(r) * DV + c0 + cb;
            const f32x4 h0 = *reinterpret_cast<const f32x4*>(Hs), h1 = *reinterpret_cast<const f32x4*>(Hs + 4);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc[c] = h0[c];
                acc[4 + c] = h1[c];
            }
            const f32x4* P = reinterpret_cast<const f32x4*>(p.ps + it * DK * DK + static_cast<size_t>(r) * DK);
            f32x4 prow[DK / 4];
#pragma unroll
            for (int k4 = 0; k4 < DK / 4; ++k4) prow[k4] = P[k4];
#pragma unroll
            for (int k4 = 0; k4 < DK / 4; ++k4) {
                const f32x4 pr = prow[k4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float* sr = Ssl + (4 * k4 + kk) * kScanCols + cb;
                    const f32x4 s0 = *reinterpret_cast<const f32x4*>(sr), s1 = *reinterpret_cast<const f32x4*>(sr + 4);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        acc[c] = fmaf(pr[kk], s0[c], acc[c]);
                        acc[4 + c] = fmaf(pr[kk], s1[c], acc[4 + c]);
                    }
                }
            }
        }
        __syncthreads();   // every read of start_s done
        if (tid < NTH) {
            float* dst = p.start + (static_cast<size_t>(ss0 + sgi + step) * H + h) * sdv +
                         static_cast<size_t>(r) * DV + c0 + cb;
            *reinterpret_cast<f32x4*>(Ssl + r * kScanCols + cb) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4*>(Ssl + r * kScanCols + cb + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
            *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr int kSegMinChunks = 16;
int segment_chunks();   // the process-wide setting (ckda_set_segment_chunks)

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// segment slots for segments of G chunks
inline int seg_slots(bool varlen, int B, int T, int ndocs, int G) {
    if (varlen) return (T + 64 * G - 1) / (64 * G) + ndocs;
    return B * (((T + 63) / 64 + G - 1) / G);
}

// start states, H_s (DK x DV each) and P_s (DK x DK) per slot and head, fp32
inline size_t seg_buffer_bytes(size_t nsslots, int H, int DK, int DV) {
    return nsslots * H * (2 * static_cast<size_t>(DK) * DV + static_cast<size_t>(DK) * DK) * sizeof(float);
}

// chunks of every chain (varlen: from the host copy of cu; empty when absent)
inline std::vector<int> chain_chunks(const int32_t* cu_host, bool varlen, int ndocs, int B, int T) {
    std::vector<int> nch;
    if (varlen) {
        if (cu_host)
            for (int d = 0; d < ndocs; ++d) nch.push_back((cu_host[d + 1] - cu_host[d] + 63) / 64);
    } else {
        nch.assign(B, (T + 63) / 64);
    }
    return nch;
}

// compute units of the device that `stream` belongs to (the current device
// for the null stream)
int device_cus(hipStream_t stream);

// Per-pass constants of the cost model below, in units of one chunk-step of
// a workgroup that has its CU to itself.
struct SegCost {
    double cu_rate;     // workgroup chunk-steps the GPU completes per unit, per CU
    double no_out;      // cost of a phase-1 step (no outputs) relative to a full one
    double scan_step;   // units per scan step
};

// Segment length, 0 for whole chains.  A phase takes at least its longest
// item and at least its total work (workgroup chunk-steps) over the GPU's
// throughput R = cu_rate * CUs.  Whole chains: max(longest chain, W / R).
// Segments of G chunks: phase 1 (the first segment in pass order, value
// slices only, and value + transition slices of the middle segments, at
// no_out of a full step) + phase 3 (every segment: W again, in items of at
// most G chunks) + the scan + launch gaps.  The segment plan is taken when
// it is below 0.8 of the whole-chain estimate.  fits(G): the workspace holds
// the segment buffers; cus: compute units of the GPU that runs the passes.
template <typename Fits>
int plan_segments(const std::vector<int>& nch, int H, int nslice, int ntrans, const SegCost& c, int cus, Fits fits) {
    const int forced = segment_chunks();
    if (forced < 0 || H == 0 || nch.empty()) return 0;
    int maxn = 0;
    double tot = 0;
    for (int n : nch) { maxn = n > maxn ? n : maxn; tot += n; }
    if (forced > 0) return (maxn > forced && fits(forced)) ? forced : 0;
    const double R = c.cu_rate * cus;
    const double W = tot * H * nslice;
    const double t0 = std::max(static_cast<double>(maxn), W / R);
    int best = 0;
    double tbest = 0.8 * t0;
    for (int G = kSegMinChunks; G < maxn; G *= 2) {
        if (!fits(G)) continue;
        double w1 = 0;
        int maxseg = 0;
        for (int n : nch) {
            const int ns = (n + G - 1) / G;
            maxseg = std::max(maxseg, ns);
            if (ns >= 2) w1 += static_cast<double>(nslice) * G + static_cast<double>(ns - 2) * (nslice + ntrans) * G;
        }
        const double t = std::max(static_cast<double>(G), c.no_out * w1 * H / R) +
                         std::max(static_cast<double>(G), W / R) + c.scan_step * std::max(0, maxseg - 2) + 2.0;
        if (t < tbest) { tbest = t; best = G; }
    }
    return best;
}

}  // namespace ckda
