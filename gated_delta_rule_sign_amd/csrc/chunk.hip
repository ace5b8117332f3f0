// chunk.hip -- the chunked forward's chunk-local kernel (kernel body in
// ckda_chunk.h), and the standalone gate / sign-fold prep kernel.
#include "ckda_chunk.h"

namespace ckda {

hipError_t launch_chunk(const FwdArgs& A, int nslots, hipStream_t stream) {
    const ChunkParams p = chunk_params(A);
    return A.bf16 ? launch_chunk_dt<bf16_t, kModeFwd>(p, A, nslots, stream)
                  : launch_chunk_dt<float, kModeFwd>(p, A, nslots, stream);
}

size_t grad_out_bytes(int DK, int DV, bool bf16) {
#define CKDA_GOB(DK_, DV_) \
    if (DK == DK_ && DV == DV_) return bf16 ? GradOut<DK_, DV_, false>::BYTES : GradOut<DK_, DV_, true>::BYTES;
    CKDA_GOB(32, 32) CKDA_GOB(32, 64) CKDA_GOB(32, 128)
    CKDA_GOB(64, 32) CKDA_GOB(64, 64) CKDA_GOB(64, 128)
    CKDA_GOB(128, 32) CKDA_GOB(128, 64) CKDA_GOB(128, 128)
#undef CKDA_GOB
    return 0;
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
