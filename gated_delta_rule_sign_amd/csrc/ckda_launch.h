// ckda_launch.h -- host-side launcher interfaces between the C ABI layer and
// the kernel translation units.  Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ckda {

struct DecodeArgs {
    int N, H, DK, DV;
    bool bf16;
    bool head_gate;   // g, s per head ([N,H]) instead of per channel
    bool qk_norm;     // q, k normalised per head before use
    const void *q, *k, *v;
    const float* g;
    const int8_t* s;
    const float* beta;
    float scale;
    float* state;
    int8_t* sign_prod;
    float* o;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

struct PrepArgs {
    int B, T, H, DK;
    bool bf16;
    const void *q, *k;
    const float* g;
    const int8_t* s;
    float* b_out;
    int8_t* p_out;
    void *qf_out, *kf_out;
};
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);

struct FwdArgs {
    // equal-length mode: B sequences of T tokens; varlen mode: nchains docs
    int B, T, H, DK, DV;
    bool bf16;
    bool head_gate;   // g, s per (token, head) instead of per channel
    bool qk_norm;     // q, k normalised per (token, head) before use
    const void *q, *k, *v;
    const float* g;
    const int8_t* s;
    const float* beta;
    float scale;
    const float* h0;
    float* o;
    float* ht;
    float* h_ckpt;
    // varlen: document n covers tokens cu[n] .. cu[n+1]-1 (device pointer);
    // nullptr selects the equal-length mode
    const int32_t* cu;
    const int32_t* cu_host;   // the same offsets on the host (varlen), for the state-pass plan
    int ndocs;
    void* ws;          // at least fwd_workspace_bytes(nslots, ...) bytes
    size_t ws_bytes;   // its size: room beyond the records enables the segmented state pass
};
// nslots: chunk slots (equal-length: B * ceil(T/64); varlen: ceil(T/64) + N)
// records only (the minimum workspace)
size_t fwd_workspace_bytes(int nslots, int H, int DK, int DV, bool bf16);
// records plus the segment buffers for up to nsslots_max segment slots
size_t fwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV, bool bf16);
// segment length of the state pass: 0 automatic, < 0 never, >= segment_min_chunks() forced
void set_segment_chunks(int G);
int segment_chunks();
int segment_min_chunks();
hipError_t launch_chunk(const FwdArgs& a, int nslots, hipStream_t stream);
hipError_t launch_state(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int nslots, hipStream_t stream);

struct BwdArgs {
    int B, T, H, DK, DV;
    bool bf16;
    bool head_gate;   // g, s, dg per (token, head) instead of per channel
    bool qk_norm;     // q, k normalised per (token, head); dq, dk w.r.t. the raw q, k
    const void *q, *k, *v;
    const float* g;
    const int8_t* s;
    const float* beta;
    float scale;
    const float* h0;
    const float* h_ckpt;   // nullptr: recomputed in the call
    const void* dout;
    const float* dht;
    float *dq, *dk, *dv, *dg, *dbeta, *dh0;
    // varlen: as in FwdArgs (documents from cu, h0 / dht / dh0 per document,
    // checkpoints per chunk slot); nullptr selects the equal-length mode
    const int32_t* cu;
    const int32_t* cu_host;   // the same offsets on the host (varlen), for the reverse-pass plan
    int ndocs;
    void* ws;          // at least bwd_workspace_bytes(nslots, ...) bytes
    size_t ws_bytes;   // its size: room beyond that enables the segmented reverse pass
};
// nslots: chunk slots, as for the forward; the minimum workspace
size_t bwd_workspace_bytes(int nslots, int H, int DK, int DV);
// checkpoints recomputed in the call when h_ckpt is nullptr
size_t bwd_ckpt_bytes(int nslots, int H, int DK, int DV);
// blocks, then room for recomputed checkpoints, then the segment buffers for
// up to nsslots_max segment slots
size_t bwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV);
hipError_t launch_bwd(const BwdArgs& a, int nslots, hipStream_t stream);

}  // namespace ckda
