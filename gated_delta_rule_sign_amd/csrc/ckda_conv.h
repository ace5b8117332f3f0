// ckda_conv.h -- host-side interface of the short convolution kernels
// (conv.hip): the optional width-4 part of the pre-mixer prep.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ckda {

constexpr int kConvWidth = 4;   // taps; tap 3 takes the current token
constexpr int kConvSeg = 64;    // tokens per thread run in the sequence kernels

// One call's sequences: N documents over T tokens as cu [N+1] (device), or,
// with cu == nullptr, N equal sequences of T / N tokens each.  x, y, state
// rows hold C channels; `bf16` selects the element type of x, y and the
// windows (else float32).  Weights w [C][4] float32.
struct ConvArgs {
    int N, T, C;
    bool bf16, silu;
    const int32_t* cu;
    const void* x;
    const float* w;
    const void* state0;   // [N][3][C] or nullptr (zero history)
    void* y;
    void* state_out;      // [N][3][C] or nullptr
    // backward
    const float* dy;
    float* dx;
    float* dw;
    float* dstate0;       // [N][3][C] float32 or nullptr
    float* partial;       // workspace: [ceil(T / kConvSeg)][C][4] float32
};

inline size_t conv_bwd_workspace_bytes(int T, int C) {
    return static_cast<size_t>((T + kConvSeg - 1) / kConvSeg) * C * kConvWidth * sizeof(float);
}

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_bwd(const ConvArgs& a, hipStream_t stream);
// one decode step: x, y [N][C]; window [N][3][C] updated in place
hipError_t launch_conv_step(int N, int C, bool bf16, bool silu, const void* x, const float* w, void* window,
                            void* y, hipStream_t stream);

}  // namespace ckda
