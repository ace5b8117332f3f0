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
    bool gate_map;    // g, beta hold pre-activations (the optional gate map); s unused
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
    bool gate_map;    // g, beta hold pre-activations (the optional gate map); s unused
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
// the chunk-local pass writing the backward's reverse-pass records (RevRecord)
// and a compact envelope flag per (slot, head) into flags
hipError_t launch_chunk_rev(const FwdArgs& a, uint32_t* flags, int nslots, hipStream_t stream);

// the backward's first chunk-parallel gradient phase (chunk.hip, kModeGrad)
struct Grad1Args {
    const uint32_t* flags;   // from launch_chunk_rev on the same inputs
    const float* h_ckpt;     // chunk-start states: [B,H,NT,DK,DV] (varlen [slot][H][DK][DV])
    const float* dU;         // [slot][H] blocks of 64 x DV from the reverse pass
    const void* dout;
    float* dv;
    float* dbeta;
    unsigned char* gout;     // [slot][H] blocks of gout_bytes (dA, dM, U)
    size_t gout_bytes;
};
hipError_t launch_grad1(const FwdArgs& a, const Grad1Args& g, int nslots, hipStream_t stream);
size_t grad_out_bytes(int DK, int DV, bool bf16);
// the backward's second chunk-parallel gradient phase (grad.hip): dq, dk, dg
struct Grad2Args {
    const uint32_t* flags;          // as for Grad1Args
    const float* h_ckpt;            // as for Grad1Args
    const float* G;                 // [slot][H] blocks of DK x DV: dL/dS at each chunk's end
    const unsigned char* gout;      // the first phase's blocks
    size_t gout_bytes;
    const void* dout;
    const float* dv;                // the first phase's dv
    float *dq, *dk, *dg;
};
hipError_t launch_grad2(const FwdArgs& a, const Grad2Args& g, int nslots, hipStream_t stream);
// the backward's reverse (state-gradient) pass (rev.hip), over the records of
// launch_chunk_rev: one chain per (sequence or document, head)
struct RevParams {
    const unsigned char* ws;   // reverse records, [slot][H] blocks of rev_record_bytes
                               // (fr: the forward's chunk records, [slot][H] Records)
    int fr;
    const void* dout;          // dO [.., T, H, DV] (input dtype)
    const float* dht;          // [chains][H][DK][DV] or nullptr (zero)
    float* dh0;                // [chains][H][DK][DV] or nullptr
    float* dU;                 // [slot][H] blocks of 64 x DV, C/D tiles
    float* G;                  // [slot][H][DK][DV]: G at each chunk's end
    const int32_t* cu;         // varlen document starts (device), or nullptr
    float scale;
    int B, T, H, ndocs;
    // segment mode (seg_len > 0 chunks per segment): per segment slot and
    // head the end G of each segment, H_s (DK x DV) and P_s (DK x DK)
    int seg_len, nsslots;
    float *seg_start, *seg_h, *seg_p;
};
// the reverse pass's cost constants for plan_segments
int rev_segment_plan(const int32_t* cu_host, bool varlen, int ndocs, int B, int T, int H, int DK, int DV,
                     size_t seg_room, hipStream_t stream);
hipError_t launch_rev(const RevParams& p, int nchains, int DK, int DV, bool bf16, hipStream_t stream);
size_t rev_record_bytes(int DK, int DV, bool bf16);
hipError_t launch_state(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd(const FwdArgs& a, int nslots, hipStream_t stream);

struct BwdArgs {
    int B, T, H, DK, DV;
    bool bf16;
    bool head_gate;   // g, s, dg per (token, head) instead of per channel
    bool qk_norm;     // q, k normalised per (token, head); dq, dk w.r.t. the raw q, k
    bool gate_map;    // g, beta hold pre-activations; dg, dbeta w.r.t. them; s unused
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
    // the chunk records of the forward call on the same inputs (its
    // workspace), or nullptr: the backward then writes reverse records itself
    const void* fwd_records;
    size_t fwd_records_bytes;
};
// nslots: chunk slots, as for the forward; the minimum workspace
size_t bwd_workspace_bytes(int nslots, int H, int DK, int DV);
// checkpoints recomputed in the call when h_ckpt is nullptr
size_t bwd_ckpt_bytes(int nslots, int H, int DK, int DV);
// blocks, then room for recomputed checkpoints, then the segment buffers for
// up to nsslots_max segment slots
size_t bwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV);
// blocks, then the segment buffers (the caller gives the checkpoints)
size_t bwd_workspace_bytes_given_ckpt(int nslots, int nsslots_max, int H, int DK, int DV);
hipError_t launch_bwd(const BwdArgs& a, int nslots, hipStream_t stream);

}  // namespace ckda
