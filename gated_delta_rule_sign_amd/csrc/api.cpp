// api.cpp -- the C ABI of libckda.so (declared in include/ckda.h).
//
// Every check runs on the host before anything is enqueued; on failure the
// call returns a status, records a message for ckda_last_error() and leaves
// every output untouched.  Kernels are launched on the caller's stream and
// the call returns without synchronising.
#include "../../include/ckda.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ckda_launch.h"

namespace {

thread_local char g_err[512] = "";

ckda_status_t fail(ckda_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

ckda_status_t ok() {
    g_err[0] = '\0';
    return CKDA_OK;
}

ckda_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(CKDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool head_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ckda_status_t check_dtype(ckda_dtype_t dt) {
    if (dt != CKDA_F32 && dt != CKDA_BF16) return fail(CKDA_ERR_DTYPE, "unknown dtype code %d", int(dt));
    return CKDA_OK;
}

ckda_status_t check_flags(ckda_flags_t flags) {
    if (flags & ~(CKDA_GATE_HEAD | CKDA_QK_L2NORM))
        return fail(CKDA_ERR_UNSUPPORTED, "unknown option flags 0x%x", unsigned(flags));
    return CKDA_OK;
}

ckda_status_t check_heads(int DK, int DV) {
    if (DK <= 0 || DV <= 0) return fail(CKDA_ERR_SHAPE, "head sizes must be positive (DK=%d, DV=%d)", DK, DV);
    if (!head_ok(DK) || !head_ok(DV))
        return fail(CKDA_ERR_UNSUPPORTED, "head sizes DK=%d, DV=%d not supported (32, 64 or 128)", DK, DV);
    return CKDA_OK;
}

#define CKDA_REQUIRE(ptr)                                                            \
    do {                                                                             \
        if ((ptr) == nullptr) return fail(CKDA_ERR_NULL, "argument '%s' is NULL", #ptr); \
    } while (0)

#define CKDA_ALIGNED(ptr)                                                                   \
    do {                                                                                    \
        if ((ptr) != nullptr && !aligned16(ptr))                                            \
            return fail(CKDA_ERR_UNSUPPORTED, "argument '%s' is not 16-byte aligned", #ptr); \
    } while (0)

#define CKDA_TRY(expr)                          \
    do {                                        \
        const ckda_status_t st_ = (expr);       \
        if (st_ != CKDA_OK) return st_;         \
    } while (0)

// token-tensor element counts must fit the kernels' 32-bit chain/token indices
bool too_big(long long tokens, int H) { return tokens * static_cast<long long>(H) >= (1LL << 31); }

// chunk slots of the forward workspace (one record per slot and head)
int fwd_slots(int B, int T) { return B * ((T + 63) / 64); }
int varlen_slots(int N, int T_total) { return (T_total + 63) / 64 + N; }

// cu_seqlens (host copy): N+1 values, starts at 0, non-decreasing, ends at T_total
ckda_status_t check_cu(int N, int T_total, const int32_t* cu) {
    CKDA_REQUIRE(cu);
    if (cu[0] != 0) return fail(CKDA_ERR_SEQLENS, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int i = 0; i < N; ++i)
        if (cu[i + 1] < cu[i]) return fail(CKDA_ERR_SEQLENS, "cu_seqlens decreases at %d", i);
    if (cu[N] != T_total) return fail(CKDA_ERR_SEQLENS, "cu_seqlens[N] = %d, expected T_total = %d", cu[N], T_total);
    return CKDA_OK;
}

ckda_status_t check_varlen_sizes(int N, int T_total, int H) {
    if (too_big(T_total, H)) return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if (static_cast<long long>(N) * H >= (1LL << 31) / 2) return fail(CKDA_ERR_UNSUPPORTED, "too many documents");
    if (static_cast<long long>(varlen_slots(N, T_total)) * H >= (1LL << 31))
        return fail(CKDA_ERR_UNSUPPORTED, "too many chunks");
    return CKDA_OK;
}

}  // namespace

extern "C" {

int ckda_abi_version(void) { return CKDA_ABI_VERSION; }

int ckda_varlen_chunk_slots(int N, int T_total) {
    if (N < 0 || T_total < 0) return 0;
    return varlen_slots(N, T_total);
}

const char* ckda_status_string(ckda_status_t s) {
    switch (s) {
        case CKDA_OK: return "ok";
        case CKDA_ERR_NULL: return "null pointer";
        case CKDA_ERR_SHAPE: return "bad shape";
        case CKDA_ERR_DTYPE: return "bad dtype";
        case CKDA_ERR_UNSUPPORTED: return "unsupported";
        case CKDA_ERR_SEQLENS: return "bad cu_seqlens";
        case CKDA_ERR_WORKSPACE: return "workspace too small";
        case CKDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* ckda_last_error(void) { return g_err; }

ckda_status_t ckda_chunk_prep(int B, int T, int H, int DK, ckda_dtype_t in_dtype, const void* q,
                              const void* k, const float* g, const int8_t* s, float* b_out,
                              int8_t* p_out, void* qf_out, void* kf_out, ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    if (B < 0 || T < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    CKDA_TRY(check_heads(DK, DK));
    if (too_big(static_cast<long long>(B) * T, H)) return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if (static_cast<long long>(B) * H * ((T + 63) / 64) >= (1LL << 31))
        return fail(CKDA_ERR_UNSUPPORTED, "too many chunks");
    if (B * T * H == 0) return ok();
    CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(g); CKDA_REQUIRE(s);
    CKDA_REQUIRE(b_out); CKDA_REQUIRE(p_out); CKDA_REQUIRE(qf_out); CKDA_REQUIRE(kf_out);
    ckda::PrepArgs a{B, T, H, DK, in_dtype == CKDA_BF16, q, k, g, s, b_out, p_out, qf_out, kf_out};
    return hip_status(ckda::launch_prep(a, static_cast<hipStream_t>(stream)), "ckda_chunk_prep launch");
}

size_t ckda_fwd_workspace_bytes(int B, int T, int H, int DK, int DV, ckda_dtype_t dt) {
    if (B < 0 || T < 0 || H < 0 || !head_ok(DK) || !head_ok(DV) || (dt != CKDA_F32 && dt != CKDA_BF16)) return 0;
    const int G = ckda::segment_min_chunks();
    const long long nss = static_cast<long long>(B) * (((T + 63) / 64 + G - 1) / G);
    return ckda::fwd_workspace_bytes_full(fwd_slots(B, T), static_cast<int>(nss), H, DK, DV, dt == CKDA_BF16);
}

size_t ckda_fwd_varlen_workspace_bytes(int N, int T_total, int H, int DK, int DV, ckda_dtype_t dt) {
    if (N < 0 || T_total < 0 || H < 0 || !head_ok(DK) || !head_ok(DV) || (dt != CKDA_F32 && dt != CKDA_BF16))
        return 0;
    const int G = ckda::segment_min_chunks();
    const int nss = (T_total + 64 * G - 1) / (64 * G) + N;
    return ckda::fwd_workspace_bytes_full(varlen_slots(N, T_total), nss, H, DK, DV, dt == CKDA_BF16);
}

ckda_status_t ckda_set_segment_chunks(int G) {
    if (G > 0 && G < ckda::segment_min_chunks())
        return fail(CKDA_ERR_UNSUPPORTED, "segments of %d chunks: at least %d", G, ckda::segment_min_chunks());
    ckda::set_segment_chunks(G);
    return ok();
}

ckda_status_t ckda_fwd_chunked(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                               ckda_flags_t flags, const void* q, const void* k, const void* v,
                               const float* g, const int8_t* s, const float* beta, float scale,
                               const float* h0, float* o, float* ht, float* h_ckpt, void* workspace,
                               size_t workspace_bytes, ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    CKDA_TRY(check_flags(flags));
    if (B < 0 || T < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    CKDA_TRY(check_heads(DK, DV));
    if (too_big(static_cast<long long>(B) * T, H)) return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if (static_cast<long long>(B) * ((T + 63) / 64) * H >= (1LL << 31))
        return fail(CKDA_ERR_UNSUPPORTED, "too many chunks");
    if (static_cast<long long>(B) * H >= (1LL << 31)) return fail(CKDA_ERR_UNSUPPORTED, "too many heads");
    if (B * H == 0) return ok();
    if (T > 0) { CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g); CKDA_REQUIRE(s); CKDA_REQUIRE(beta); CKDA_REQUIRE(o); }
    CKDA_ALIGNED(q); CKDA_ALIGNED(k); CKDA_ALIGNED(g); CKDA_ALIGNED(s); CKDA_ALIGNED(workspace);
    const int nslots = fwd_slots(B, T);
    const size_t need = ckda::fwd_workspace_bytes(nslots, H, DK, DV, in_dtype == CKDA_BF16);
    if (need > 0) {
        CKDA_REQUIRE(workspace);
        if (workspace_bytes < need)
            return fail(CKDA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    }
    ckda::FwdArgs a{};
    a.B = B; a.T = T; a.H = H; a.DK = DK; a.DV = DV; a.bf16 = in_dtype == CKDA_BF16;
    a.head_gate = (flags & CKDA_GATE_HEAD) != 0; a.qk_norm = (flags & CKDA_QK_L2NORM) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s; a.beta = beta; a.scale = scale;
    a.h0 = h0; a.o = o; a.ht = ht; a.h_ckpt = h_ckpt; a.cu = nullptr; a.cu_host = nullptr; a.ndocs = 0;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    return hip_status(ckda::launch_fwd(a, nslots, static_cast<hipStream_t>(stream)), "ckda_fwd_chunked launch");
}

ckda_status_t ckda_fwd_varlen(int N, int T_total, const int32_t* cu, const int32_t* cu_dev, int H,
                              int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q,
                              const void* k, const void* v, const float* g, const int8_t* s,
                              const float* beta, float scale, const float* h0, float* o, float* ht,
                              float* h_ckpt, void* workspace, size_t workspace_bytes,
                              ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    CKDA_TRY(check_flags(flags));
    if (N < 0 || T_total < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (N=%d, T=%d, H=%d)", N, T_total, H);
    CKDA_TRY(check_heads(DK, DV));
    CKDA_TRY(check_varlen_sizes(N, T_total, H));
    CKDA_TRY(check_cu(N, T_total, cu));
    if (N * H == 0) return ok();
    CKDA_REQUIRE(cu_dev);
    if (T_total > 0) { CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g); CKDA_REQUIRE(s); CKDA_REQUIRE(beta); CKDA_REQUIRE(o); }
    CKDA_ALIGNED(q); CKDA_ALIGNED(k); CKDA_ALIGNED(g); CKDA_ALIGNED(s); CKDA_ALIGNED(workspace);
    const int nslots = varlen_slots(N, T_total);
    const size_t need = ckda::fwd_workspace_bytes(nslots, H, DK, DV, in_dtype == CKDA_BF16);
    if (need > 0) {
        CKDA_REQUIRE(workspace);
        if (workspace_bytes < need)
            return fail(CKDA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    }
    ckda::FwdArgs a{};
    a.B = 1; a.T = T_total; a.H = H; a.DK = DK; a.DV = DV; a.bf16 = in_dtype == CKDA_BF16;
    a.head_gate = (flags & CKDA_GATE_HEAD) != 0; a.qk_norm = (flags & CKDA_QK_L2NORM) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s; a.beta = beta; a.scale = scale;
    a.h0 = h0; a.o = o; a.ht = ht; a.h_ckpt = h_ckpt;
    a.cu = cu_dev; a.cu_host = cu; a.ndocs = N; a.ws = workspace; a.ws_bytes = workspace_bytes;
    return hip_status(ckda::launch_fwd(a, nslots, static_cast<hipStream_t>(stream)), "ckda_fwd_varlen launch");
}

ckda_status_t ckda_decode_step(int N, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                               const void* q,
                               const void* k, const void* v, const float* g, const int8_t* s,
                               const float* beta, float scale, float* state, int8_t* sign_prod,
                               float* o, ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    CKDA_TRY(check_flags(flags));
    if (N < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (N=%d, H=%d)", N, H);
    CKDA_TRY(check_heads(DK, DV));
    if (static_cast<long long>(N) * H >= (1LL << 31)) return fail(CKDA_ERR_UNSUPPORTED, "too many heads");
    if (N * H == 0) return ok();
    CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g); CKDA_REQUIRE(s);
    CKDA_REQUIRE(beta); CKDA_REQUIRE(state); CKDA_REQUIRE(sign_prod); CKDA_REQUIRE(o);
    CKDA_ALIGNED(state); CKDA_ALIGNED(o);
    ckda::DecodeArgs a{N, H, DK, DV, in_dtype == CKDA_BF16, (flags & CKDA_GATE_HEAD) != 0,
                       (flags & CKDA_QK_L2NORM) != 0, q, k, v, g, s, beta,
                       scale, state, sign_prod, o};
    return hip_status(ckda::launch_decode(a, static_cast<hipStream_t>(stream)), "ckda_decode_step launch");
}

size_t ckda_bwd_workspace_bytes(int B, int T, int H, int DK, int DV) {
    if (B < 0 || T < 0 || H < 0 || !head_ok(DK) || !head_ok(DV)) return 0;
    const int G = ckda::segment_min_chunks();
    const long long nss = static_cast<long long>(B) * (((T + 63) / 64 + G - 1) / G);
    return ckda::bwd_workspace_bytes_full(fwd_slots(B, T), static_cast<int>(nss), H, DK, DV);
}

size_t ckda_bwd_varlen_workspace_bytes(int N, int T_total, int H, int DK, int DV) {
    if (N < 0 || T_total < 0 || H < 0 || !head_ok(DK) || !head_ok(DV)) return 0;
    const int G = ckda::segment_min_chunks();
    const int nss = (T_total + 64 * G - 1) / (64 * G) + N;
    return ckda::bwd_workspace_bytes_full(varlen_slots(N, T_total), nss, H, DK, DV);
}

namespace {

// shared tail of ckda_bwd / ckda_bwd_varlen: pointer checks, workspace, launch
ckda_status_t bwd_common(ckda::BwdArgs& a, int nslots, bool any_tokens, const void* workspace,
                         size_t workspace_bytes, ckda_stream_t stream, const char* what) {
    if (any_tokens) {
        CKDA_REQUIRE(a.q); CKDA_REQUIRE(a.k); CKDA_REQUIRE(a.v); CKDA_REQUIRE(a.g); CKDA_REQUIRE(a.s);
        CKDA_REQUIRE(a.beta); CKDA_REQUIRE(a.dout);
        CKDA_REQUIRE(a.dq); CKDA_REQUIRE(a.dk); CKDA_REQUIRE(a.dv); CKDA_REQUIRE(a.dg); CKDA_REQUIRE(a.dbeta);
    }
    CKDA_ALIGNED(a.q); CKDA_ALIGNED(a.k); CKDA_ALIGNED(a.v); CKDA_ALIGNED(a.g); CKDA_ALIGNED(a.s);
    CKDA_ALIGNED(a.dout); CKDA_ALIGNED(a.h_ckpt);
    CKDA_ALIGNED(a.dq); CKDA_ALIGNED(a.dk); CKDA_ALIGNED(a.dv); CKDA_ALIGNED(a.dg);
    // h_ckpt nullptr: checkpoints recomputed into the workspace, after the blocks
    size_t need = ckda::bwd_workspace_bytes(nslots, a.H, a.DK, a.DV);
    const bool recompute = any_tokens && !a.h_ckpt;
    if (recompute) need = ((need + 255) & ~static_cast<size_t>(255)) + ckda::bwd_ckpt_bytes(nslots, a.H, a.DK, a.DV);
    if (need > 0) {
        CKDA_REQUIRE(workspace);
        CKDA_ALIGNED(workspace);
        if (workspace_bytes < need)
            return fail(CKDA_ERR_WORKSPACE, "workspace %zu bytes, need %zu%s", workspace_bytes, need,
                        recompute ? " (checkpoints recomputed)" : "");
    }
    a.ws = const_cast<void*>(workspace);
    a.ws_bytes = workspace_bytes;
    return hip_status(ckda::launch_bwd(a, nslots, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

ckda_status_t ckda_bwd(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                       const void* q, const void* k, const void* v, const float* g, const int8_t* s,
                       const float* beta, float scale, const float* h0, const float* h_ckpt,
                       const void* dout, const float* dht, float* dq, float* dk, float* dv,
                       float* dg, float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                       ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    CKDA_TRY(check_flags(flags));
    if (B < 0 || T < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (B=%d, T=%d, H=%d)", B, T, H);
    CKDA_TRY(check_heads(DK, DV));
    if (too_big(static_cast<long long>(B) * T, H)) return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if (static_cast<long long>(B) * ((T + 63) / 64) * H >= (1LL << 31))
        return fail(CKDA_ERR_UNSUPPORTED, "too many chunks");
    if (static_cast<long long>(B) * H >= (1LL << 31)) return fail(CKDA_ERR_UNSUPPORTED, "too many heads");
    if (B * H == 0) return ok();
    ckda::BwdArgs a{};
    a.B = B; a.T = T; a.H = H; a.DK = DK; a.DV = DV; a.bf16 = in_dtype == CKDA_BF16;
    a.head_gate = (flags & CKDA_GATE_HEAD) != 0; a.qk_norm = (flags & CKDA_QK_L2NORM) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s; a.beta = beta; a.scale = scale; a.h0 = h0;
    a.h_ckpt = h_ckpt; a.dout = dout; a.dht = dht; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
    a.dbeta = dbeta; a.dh0 = dh0; a.cu = nullptr; a.ndocs = 0;
    return bwd_common(a, fwd_slots(B, T), T > 0, workspace, workspace_bytes, stream, "ckda_bwd launch");
}

ckda_status_t ckda_bwd_varlen(int N, int T_total, const int32_t* cu, const int32_t* cu_dev, int H,
                              int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q,
                              const void* k,
                              const void* v, const float* g, const int8_t* s, const float* beta,
                              float scale, const float* h0, const float* h_ckpt, const void* dout,
                              const float* dht, float* dq, float* dk, float* dv, float* dg,
                              float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                              ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    CKDA_TRY(check_flags(flags));
    if (N < 0 || T_total < 0 || H < 0) return fail(CKDA_ERR_SHAPE, "negative size (N=%d, T=%d, H=%d)", N, T_total, H);
    CKDA_TRY(check_heads(DK, DV));
    CKDA_TRY(check_varlen_sizes(N, T_total, H));
    CKDA_TRY(check_cu(N, T_total, cu));
    if (N * H == 0) return ok();
    CKDA_REQUIRE(cu_dev);
    ckda::BwdArgs a{};
    a.B = 1; a.T = T_total; a.H = H; a.DK = DK; a.DV = DV; a.bf16 = in_dtype == CKDA_BF16;
    a.head_gate = (flags & CKDA_GATE_HEAD) != 0; a.qk_norm = (flags & CKDA_QK_L2NORM) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s; a.beta = beta; a.scale = scale; a.h0 = h0;
    a.h_ckpt = h_ckpt; a.dout = dout; a.dht = dht; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
    a.dbeta = dbeta; a.dh0 = dh0; a.cu = cu_dev; a.cu_host = cu; a.ndocs = N;
    return bwd_common(a, varlen_slots(N, T_total), T_total > 0, workspace, workspace_bytes, stream,
                      "ckda_bwd_varlen launch");
}

}  // extern "C"
