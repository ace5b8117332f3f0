// bwd.hip -- CKDA backward: gradients of L = <do, o> + <dht, ht> through the
// chunked forward; the host-side plan of its four passes.
//
// The backward is the plain reverse-mode derivative of the WY/UT chunk form
// the forward computes (Complex KDA paper page, section 2 "Linear RNNs":
// DeltaNet/KDA admit WY-based chunk-wise implementations).  The pages' own
// training backward is in an appendix they do not include, so no gradient
// flows to the sign s, and dg = alpha dL/dalpha for g = log|alpha|.
//
// Passes, in stream order:
//  1. reverse records (chunk-local kernel, reverse-record mode, chunk_rev.hip):
//     per (chunk slot, head) the chunk's KB = KbT^T, Qh^T, W^T, M^T and d,
//     and a flag for chunks outside the anchors' envelope;
//  2. reverse pass (rev.hip): per chain, from its last chunk to its first,
//     dU = scale M^T dO + KbT^T G and G <- Diag(d) G + scale Qh^T dO - W^T dU,
//     writing dU and the chunk-end G per chunk and dh0 per chain;
//  3. first gradient phase (chunk-local kernel, gradient mode, chunk_grad.hip):
//     per chunk X^-1, U, dV = dv, dbeta, and dA, dM handed to
//  4. the second gradient phase (grad.hip): dq, dk, dg.
// Passes 1, 3 and 4 are chunk-parallel over every chunk-head at once; only
// pass 2 walks chunks in order.
//
// Workspace (each region 256-byte aligned), NC = chunk slots x heads:
//   blocks  NC x max(reverse record, first-phase output): the reverse records
//           of pass 1, then (after pass 2 has read them) the first phase's
//           dA, dM and U;
//   dU      NC x 64 x DV floats;
//   G       NC x max(DK, 64) x DV floats (DK x DV used; the extra room holds
//           the recomputed forward's output when the caller gives no
//           checkpoints);
//   flags   NC words;
//   ckpt    NC x DK x DV floats, only when h_ckpt is NULL: the checkpoints of
//           a forward pass run in the call (its records over blocks and dU,
//           which a forward record never exceeds);
//   seg     the segment buffers of the reverse pass (segment mode, when the
//           plan takes it and they fit): per segment slot and head its end G,
//           H_s and P_s.  With the caller's checkpoints the ckpt room is
//           unused and the segment buffers start there; without them they
//           follow it.
#include "ckda_device.h"
#include "ckda_launch.h"
#include "ckda_record.h"
#include "ckda_segments.h"

namespace ckda {

namespace {

struct BwdLayout {
    size_t blk;   // bytes per chunk-head block
    size_t off_du, off_g, off_flags, off_ckpt, end_ckpt;
    BwdLayout(int nslots, int H, int DK, int DV) {
        const size_t NC = static_cast<size_t>(nslots) * H;
        const size_t rr = rev_record_bytes(DK, DV, false), go = grad_out_bytes(DK, DV, false);
        blk = rr > go ? rr : go;
        off_du = align256(NC * blk);
        off_g = off_du + align256(NC * 64 * DV * 4);
        off_flags = off_g + align256(NC * static_cast<size_t>(DK > 64 ? DK : 64) * DV * 4);
        off_ckpt = off_flags + align256(NC * 4);
        end_ckpt = off_ckpt + align256(NC * static_cast<size_t>(DK) * DV * 4);
    }
};

// the forward records' flag words (chunks outside the anchors' envelope) as
// the flag array the gradient phases read
__global__ void gather_flags_kernel(const unsigned char* rec, size_t bytes, size_t flag_off, uint32_t* flags, int n) {
    const int i = blockIdx.x * 256 + static_cast<int>(threadIdx.x);
    if (i < n) flags[i] = *reinterpret_cast<const uint32_t*>(rec + static_cast<size_t>(i) * bytes + flag_off);
}

void fwd_record_geometry(int DK, int DV, bool bf16, size_t& bytes, size_t& flag_off) {
    bytes = flag_off = 0;
#define CKDA_FRG(DK_, DV_)                                                                                  \
    if (DK == DK_ && DV == DV_) {                                                                          \
        bytes = bf16 ? Record<DK_, DV_, false>::BYTES : Record<DK_, DV_, true>::BYTES;                     \
        flag_off = bf16 ? Record<DK_, DV_, false>::OFF_FLAG : Record<DK_, DV_, true>::OFF_FLAG;            \
    }
    CKDA_FRG(32, 32) CKDA_FRG(32, 64) CKDA_FRG(32, 128)
    CKDA_FRG(64, 32) CKDA_FRG(64, 64) CKDA_FRG(64, 128)
    CKDA_FRG(128, 32) CKDA_FRG(128, 64) CKDA_FRG(128, 128)
#undef CKDA_FRG
}

__global__ void copy_or_zero_kernel(float* dst, const float* src, size_t n) {
    for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

size_t bwd_workspace_bytes(int nslots, int H, int DK, int DV) { return BwdLayout(nslots, H, DK, DV).off_ckpt; }

// checkpoints recomputed in the call (h_ckpt = nullptr): [nslots][H][DK][DV]
size_t bwd_ckpt_bytes(int nslots, int H, int DK, int DV) {
    const BwdLayout l(nslots, H, DK, DV);
    return l.end_ckpt - l.off_ckpt;
}

// the whole layout: checkpoint room, then the segment buffers for up to
// nsslots_max segment slots
size_t bwd_workspace_bytes_full(int nslots, int nsslots_max, int H, int DK, int DV) {
    return BwdLayout(nslots, H, DK, DV).end_ckpt + seg_buffer_bytes(nsslots_max, H, DK, DV);
}

// the layout when the caller gives the checkpoints: the segment buffers take
// the checkpoint room's place
size_t bwd_workspace_bytes_given_ckpt(int nslots, int nsslots_max, int H, int DK, int DV) {
    return BwdLayout(nslots, H, DK, DV).off_ckpt + seg_buffer_bytes(nsslots_max, H, DK, DV);
}

hipError_t launch_bwd(const BwdArgs& a, int nslots, hipStream_t st) {
    const int NC = nslots * a.H;
    const int nchains = (a.cu ? a.ndocs : a.B) * a.H;
    const int DK = a.DK, DV = a.DV;
    if (NC == 0) {   // no tokens: dh0 = dht (or 0)
        const size_t n = static_cast<size_t>(nchains) * DK * DV;
        if (a.dh0 && n > 0) {
            const size_t nb = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
            hipLaunchKernelGGL(copy_or_zero_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st, a.dh0, a.dht, n);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    const BwdLayout lay(nslots, a.H, DK, DV);
    unsigned char* const ws = static_cast<unsigned char*>(a.ws);
    float* const du = reinterpret_cast<float*>(ws + lay.off_du);
    float* const gg = reinterpret_cast<float*>(ws + lay.off_g);
    uint32_t* const flags = reinterpret_cast<uint32_t*>(ws + lay.off_flags);
    hipError_t e;
#define CKDA_CHECK(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
    FwdArgs f{};
    f.B = a.B; f.T = a.T; f.H = a.H; f.DK = DK; f.DV = DV; f.bf16 = a.bf16;
    f.head_gate = a.head_gate; f.qk_norm = a.qk_norm; f.gate_map = a.gate_map;
    f.q = a.q; f.k = a.k; f.v = a.v; f.g = a.g; f.s = a.s; f.beta = a.beta; f.scale = a.scale;
    f.cu = a.cu; f.cu_host = a.cu_host; f.ndocs = a.ndocs;
    const float* ck = a.h_ckpt;
    if (!ck) {
        // checkpoints from a forward pass in the call: records over blocks and
        // dU, output o over G, checkpoints in their own region; records-only
        // room keeps its state pass on whole chains
        FwdArgs r = f;
        r.h0 = a.h0;
        r.o = gg;
        r.ht = nullptr;
        r.h_ckpt = reinterpret_cast<float*>(ws + lay.off_ckpt);
        r.ws = ws;
        r.ws_bytes = fwd_workspace_bytes(nslots, a.H, DK, DV, a.bf16);
        if (r.ws_bytes > lay.off_g) return hipErrorInvalidValue;   // (record sizes rule this out)
        CKDA_CHECK(launch_fwd(r, nslots, st));
        ck = r.h_ckpt;
    }
    f.ws = ws;
    RevParams rp{};
    if (a.fwd_records) {
        // the forward's own records: the reverse pass stages them transposed,
        // and their flags become the gradient phases' flag array
        size_t rb, fo;
        fwd_record_geometry(DK, DV, a.bf16, rb, fo);
        hipLaunchKernelGGL(gather_flags_kernel, dim3(static_cast<unsigned>((NC + 255) / 256)), dim3(256), 0, st,
                           static_cast<const unsigned char*>(a.fwd_records), rb, fo, flags, NC);
        CKDA_CHECK(hipGetLastError());
        rp.ws = static_cast<const unsigned char*>(a.fwd_records);
        rp.fr = 1;
    } else {
        CKDA_CHECK(launch_chunk_rev(f, flags, nslots, st));
        rp.ws = ws;
        rp.fr = 0;
    }
    rp.dout = a.dout; rp.dht = a.dht; rp.dh0 = a.dh0; rp.dU = du; rp.G = gg;
    rp.cu = a.cu; rp.scale = a.scale; rp.B = a.B; rp.T = a.T; rp.H = a.H; rp.ndocs = a.ndocs;
    {   // segmented reverse pass when the plan takes it and the workspace has room
        const bool varlen = a.cu != nullptr;
        const size_t seg0 = a.h_ckpt ? lay.off_ckpt : lay.end_ckpt;
        const size_t room = a.ws_bytes > seg0 ? a.ws_bytes - seg0 : 0;
        rp.seg_len = rev_segment_plan(a.cu_host, varlen, a.ndocs, a.B, a.T, a.H, DK, DV, room, st);
        if (rp.seg_len > 0) {
            rp.nsslots = seg_slots(varlen, a.B, a.T, a.ndocs, rp.seg_len);
            float* sb = reinterpret_cast<float*>(ws + seg0);
            const size_t per = static_cast<size_t>(rp.nsslots) * a.H * DK * DV;
            rp.seg_start = sb;
            rp.seg_h = sb + per;
            rp.seg_p = sb + 2 * per;
        }
    }
    CKDA_CHECK(launch_rev(rp, nchains, DK, DV, a.bf16, st));
    Grad1Args g1{};
    g1.flags = flags; g1.h_ckpt = ck; g1.dU = du; g1.dout = a.dout; g1.dv = a.dv; g1.dbeta = a.dbeta;
    g1.gout = ws; g1.gout_bytes = lay.blk;
    CKDA_CHECK(launch_grad1(f, g1, nslots, st));
    Grad2Args g2{};
    g2.flags = flags; g2.h_ckpt = ck; g2.G = gg; g2.gout = ws; g2.gout_bytes = lay.blk;
    g2.dout = a.dout; g2.dv = a.dv; g2.dq = a.dq; g2.dk = a.dk; g2.dg = a.dg;
    CKDA_CHECK(launch_grad2(f, g2, nslots, st));
#undef CKDA_CHECK
    return hipSuccess;
}

}  // namespace ckda
