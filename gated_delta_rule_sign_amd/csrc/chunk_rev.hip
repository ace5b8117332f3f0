// chunk_rev.hip -- the backward's reverse-record pass: the chunk-local kernel
// (ckda_chunk.h) in its reverse-record mode.
#include "ckda_chunk.h"

namespace ckda {

hipError_t launch_chunk_rev(const FwdArgs& A, uint32_t* flags, int nslots, hipStream_t stream) {
    ChunkParams p = chunk_params(A);
    p.flags = flags;
    return A.bf16 ? launch_chunk_dt<bf16_t, kModeRev>(p, A, nslots, stream)
                  : launch_chunk_dt<float, kModeRev>(p, A, nslots, stream);
}

}  // namespace ckda
