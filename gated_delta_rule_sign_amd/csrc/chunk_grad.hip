// chunk_grad.hip -- the backward's first chunk-parallel gradient phase: the
// chunk-local kernel (ckda_chunk.h) in its gradient mode.
#include "ckda_chunk.h"

namespace ckda {

hipError_t launch_grad1(const FwdArgs& A, const Grad1Args& G, int nslots, hipStream_t stream) {
    ChunkParams p = chunk_params(A);
    p.flags = const_cast<uint32_t*>(G.flags);   // read only (the exact pass's list)
    p.h_ckpt = G.h_ckpt; p.dU = G.dU; p.dout = G.dout; p.dv = G.dv; p.dbeta = G.dbeta;
    p.gout = G.gout; p.gout_bytes = G.gout_bytes; p.scale = A.scale;
    return A.bf16 ? launch_chunk_dt<bf16_t, kModeGrad>(p, A, nslots, stream)
                  : launch_chunk_dt<float, kModeGrad>(p, A, nslots, stream);
}

}  // namespace ckda
