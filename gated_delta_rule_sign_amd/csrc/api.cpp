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
#include <initializer_list>
#include <mutex>

#include "ckda_conv.h"
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
    if (flags & ~(CKDA_GATE_HEAD | CKDA_QK_L2NORM | CKDA_GATE_MAP))
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

// A device buffer as the host sees it: [p, p + n) bytes.
struct Span {
    const void* p;
    size_t n;
    const char* name;
};

bool overlaps(const Span& a, const Span& b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Outputs (the workspace among them) must not overlap an input or each other:
// the kernels read inputs after other workgroups have started writing.
ckda_status_t check_no_alias(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (const Span* o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlaps(*o, i)) return fail(CKDA_ERR_UNSUPPORTED, "output '%s' overlaps input '%s'", o->name, i.name);
        for (const Span* o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(*o, *o2)) return fail(CKDA_ERR_UNSUPPORTED, "outputs '%s' and '%s' overlap", o->name, o2->name);
    }
    return CKDA_OK;
}

// byte sizes of the token tensors of one call: n token-heads
struct TokBytes {
    size_t qk, v, g, s, beta, o;
    TokBytes(long long n, int DK, int DV, bool bf16, bool head_gate) {
        const size_t es = bf16 ? 2 : 4, nn = static_cast<size_t>(n);
        qk = nn * DK * es; v = nn * DV * es;
        g = nn * (head_gate ? 1 : DK) * 4; s = nn * (head_gate ? 1 : DK);
        beta = nn * 4; o = nn * DV * 4;
    }
};

// The chunk records of ckda_fwd_chunked_noalloc.  Host code never uses the
// array's name as an address: its device address, per device, comes from
// hipGetSymbolAddress with that device current, on the first call there.
__device__ __align__(256) unsigned char scratch[CKDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(hipStream_t stream, void** out) {
    hipDevice_t dev = 0;
    if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
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

}  // extern "C"

namespace {

// ckda_fwd_chunked and its no-allocation variant.  ws == nullptr selects the
// fixed scratch array (whole chains; records only).
ckda_status_t fwd_chunked_common(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                                 const void* q, const void* k, const void* v, const float* g, const int8_t* s,
                                 const float* beta, float scale, const float* h0, float* o, float* ht,
                                 float* h_ckpt, void* workspace, size_t workspace_bytes, bool noalloc,
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
    if (T > 0) { CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g); CKDA_REQUIRE(beta); CKDA_REQUIRE(o); }
    if (T > 0 && !(flags & CKDA_GATE_MAP)) CKDA_REQUIRE(s);
    CKDA_ALIGNED(q); CKDA_ALIGNED(k); CKDA_ALIGNED(g); CKDA_ALIGNED(s); CKDA_ALIGNED(workspace);
    const int nslots = fwd_slots(B, T);
    const size_t need = ckda::fwd_workspace_bytes(nslots, H, DK, DV, in_dtype == CKDA_BF16);
    if (noalloc) {
        if (need > CKDA_NOALLOC_SCRATCH_BYTES)
            return fail(CKDA_ERR_UNSUPPORTED,
                        "ckda_fwd_chunked_noalloc: the records of %d chunk-heads need %zu bytes, more than its "
                        "fixed %zu-byte scratch; use ckda_fwd_chunked with a workspace",
                        nslots * H, need, static_cast<size_t>(CKDA_NOALLOC_SCRATCH_BYTES));
        if (need > 0) {
            CKDA_TRY(hip_status(scratch_address(static_cast<hipStream_t>(stream), &workspace),
                                "ckda_fwd_chunked_noalloc scratch address"));
            workspace_bytes = need;   // records only: the state pass keeps whole chains
        }
    } else if (need > 0) {
        CKDA_REQUIRE(workspace);
        if (workspace_bytes < need)
            return fail(CKDA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    }
    ckda::FwdArgs a{};
    a.B = B; a.T = T; a.H = H; a.DK = DK; a.DV = DV; a.bf16 = in_dtype == CKDA_BF16;
    a.head_gate = (flags & CKDA_GATE_HEAD) != 0; a.qk_norm = (flags & CKDA_QK_L2NORM) != 0;
    a.gate_map = (flags & CKDA_GATE_MAP) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s ? s : reinterpret_cast<const int8_t*>(g); a.beta = beta; a.scale = scale;
    a.h0 = h0; a.o = o; a.ht = ht; a.h_ckpt = h_ckpt; a.cu = nullptr; a.cu_host = nullptr; a.ndocs = 0;
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    {
        const TokBytes tb(static_cast<long long>(B) * T * H, DK, DV, a.bf16, a.head_gate);
        const size_t st = static_cast<size_t>(B) * H * DK * DV * 4;
        CKDA_TRY(check_no_alias({{o, tb.o, "o"}, {ht, st, "ht"}, {h_ckpt, static_cast<size_t>(nslots) * H * DK * DV * 4, "h_ckpt"},
                                 {workspace, workspace_bytes, "workspace"}},
                                {{q, tb.qk, "q"}, {k, tb.qk, "k"}, {v, tb.v, "v"}, {g, tb.g, "g"}, {s, tb.s, "s"},
                                 {beta, tb.beta, "beta"}, {h0, st, "h0"}}));
    }
    return hip_status(ckda::launch_fwd(a, nslots, static_cast<hipStream_t>(stream)),
                      noalloc ? "ckda_fwd_chunked_noalloc launch" : "ckda_fwd_chunked launch");
}

}  // namespace

extern "C" {

ckda_status_t ckda_fwd_chunked(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                               ckda_flags_t flags, const void* q, const void* k, const void* v,
                               const float* g, const int8_t* s, const float* beta, float scale,
                               const float* h0, float* o, float* ht, float* h_ckpt, void* workspace,
                               size_t workspace_bytes, ckda_stream_t stream) {
    return fwd_chunked_common(B, T, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, o, ht, h_ckpt,
                              workspace, workspace_bytes, false, stream);
}

ckda_status_t ckda_fwd_chunked_noalloc(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype,
                                       ckda_flags_t flags, const void* q, const void* k, const void* v,
                                       const float* g, const int8_t* s, const float* beta, float scale,
                                       const float* h0, float* o, float* ht, float* h_ckpt,
                                       ckda_stream_t stream) {
    return fwd_chunked_common(B, T, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, o, ht, h_ckpt,
                              nullptr, 0, true, stream);
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
    if (T_total > 0) { CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g); CKDA_REQUIRE(beta); CKDA_REQUIRE(o); }
    if (T_total > 0 && !(flags & CKDA_GATE_MAP)) CKDA_REQUIRE(s);
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
    a.gate_map = (flags & CKDA_GATE_MAP) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s ? s : reinterpret_cast<const int8_t*>(g); a.beta = beta; a.scale = scale;
    a.h0 = h0; a.o = o; a.ht = ht; a.h_ckpt = h_ckpt;
    a.cu = cu_dev; a.cu_host = cu; a.ndocs = N; a.ws = workspace; a.ws_bytes = workspace_bytes;
    {
        const TokBytes tb(static_cast<long long>(T_total) * H, DK, DV, a.bf16, a.head_gate);
        const size_t st = static_cast<size_t>(N) * H * DK * DV * 4;
        CKDA_TRY(check_no_alias({{o, tb.o, "o"}, {ht, st, "ht"}, {h_ckpt, static_cast<size_t>(nslots) * H * DK * DV * 4, "h_ckpt"},
                                 {workspace, workspace_bytes, "workspace"}},
                                {{q, tb.qk, "q"}, {k, tb.qk, "k"}, {v, tb.v, "v"}, {g, tb.g, "g"}, {s, tb.s, "s"},
                                 {beta, tb.beta, "beta"}, {h0, st, "h0"}, {cu_dev, (static_cast<size_t>(N) + 1) * 4, "cu_seqlens"}}));
    }
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
    CKDA_REQUIRE(q); CKDA_REQUIRE(k); CKDA_REQUIRE(v); CKDA_REQUIRE(g);
    if (!(flags & CKDA_GATE_MAP)) CKDA_REQUIRE(s);
    CKDA_REQUIRE(beta); CKDA_REQUIRE(state); CKDA_REQUIRE(sign_prod); CKDA_REQUIRE(o);
    CKDA_ALIGNED(state); CKDA_ALIGNED(o);
    // with the gate map s is never read (a NULL s stands in as g's address)
    ckda::DecodeArgs a{N, H, DK, DV, in_dtype == CKDA_BF16, (flags & CKDA_GATE_HEAD) != 0,
                       (flags & CKDA_QK_L2NORM) != 0, (flags & CKDA_GATE_MAP) != 0, q, k, v, g,
                       s ? s : reinterpret_cast<const int8_t*>(g), beta, scale, state, sign_prod, o};
    {   // state and sign_prod are updated in place: outputs here
        const TokBytes tb(static_cast<long long>(N) * H, DK, DV, a.bf16, a.head_gate);
        const size_t st = static_cast<size_t>(N) * H * DK * DV * 4;
        CKDA_TRY(check_no_alias({{o, tb.o, "o"}, {state, st, "state"},
                                 {sign_prod, static_cast<size_t>(N) * H * DK, "sign_prod"}},
                                {{q, tb.qk, "q"}, {k, tb.qk, "k"}, {v, tb.v, "v"}, {g, tb.g, "g"}, {s, tb.s, "s"},
                                 {beta, tb.beta, "beta"}}));
    }
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

size_t ckda_bwd_workspace_bytes_given_ckpt(int B, int T, int H, int DK, int DV) {
    if (B < 0 || T < 0 || H < 0 || !head_ok(DK) || !head_ok(DV)) return 0;
    const int G = ckda::segment_min_chunks();
    const long long nss = static_cast<long long>(B) * (((T + 63) / 64 + G - 1) / G);
    return ckda::bwd_workspace_bytes_given_ckpt(fwd_slots(B, T), static_cast<int>(nss), H, DK, DV);
}

size_t ckda_bwd_varlen_workspace_bytes_given_ckpt(int N, int T_total, int H, int DK, int DV) {
    if (N < 0 || T_total < 0 || H < 0 || !head_ok(DK) || !head_ok(DV)) return 0;
    const int G = ckda::segment_min_chunks();
    const int nss = (T_total + 64 * G - 1) / (64 * G) + N;
    return ckda::bwd_workspace_bytes_given_ckpt(varlen_slots(N, T_total), nss, H, DK, DV);
}

namespace {

// the forward's workspace as the backward's reverse records: checkpoints
// given, the records' whole area present and aligned
ckda_status_t check_fwd_records(ckda::BwdArgs& a, int nslots, bool any_tokens, const void* fwd_ws, size_t fwd_ws_bytes) {
    if (!any_tokens) return CKDA_OK;
    if (!a.h_ckpt)
        return fail(CKDA_ERR_NULL, "the forward records go with that call's checkpoints: h_ckpt is NULL");
    CKDA_REQUIRE(fwd_ws);
    CKDA_ALIGNED(fwd_ws);
    const size_t need = ckda::fwd_workspace_bytes(nslots, a.H, a.DK, a.DV, a.bf16);
    if (fwd_ws_bytes < need)
        return fail(CKDA_ERR_WORKSPACE, "forward workspace %zu bytes, its records take %zu", fwd_ws_bytes, need);
    a.fwd_records = fwd_ws;
    a.fwd_records_bytes = need;
    return CKDA_OK;
}

// shared tail of ckda_bwd / ckda_bwd_varlen: pointer checks, workspace, launch
ckda_status_t bwd_common(ckda::BwdArgs& a, int nslots, bool any_tokens, const void* workspace,
                         size_t workspace_bytes, ckda_stream_t stream, const char* what) {
    if (any_tokens) {
        CKDA_REQUIRE(a.q); CKDA_REQUIRE(a.k); CKDA_REQUIRE(a.v); CKDA_REQUIRE(a.g);
        if (!a.gate_map) CKDA_REQUIRE(a.s);
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
    {
        const long long n = static_cast<long long>(a.B) * a.T * a.H;
        const TokBytes tb(n, a.DK, a.DV, a.bf16, a.head_gate);
        const size_t st = static_cast<size_t>(a.cu ? a.ndocs : a.B) * a.H * a.DK * a.DV * 4;
        const size_t ck = static_cast<size_t>(nslots) * a.H * a.DK * a.DV * 4;
        const size_t dob = tb.v;   // dout: the input dtype, [.., DV]
        CKDA_TRY(check_no_alias({{a.dq, static_cast<size_t>(n) * a.DK * 4, "dq"}, {a.dk, static_cast<size_t>(n) * a.DK * 4, "dk"},
                                 {a.dv, tb.o, "dv"}, {a.dg, tb.g, "dg"}, {a.dbeta, tb.beta, "dbeta"},
                                 {a.dh0, st, "dh0"}, {workspace, workspace_bytes, "workspace"}},
                                {{a.q, tb.qk, "q"}, {a.k, tb.qk, "k"}, {a.v, tb.v, "v"}, {a.g, tb.g, "g"}, {a.s, tb.s, "s"},
                                 {a.beta, tb.beta, "beta"}, {a.h0, st, "h0"}, {a.h_ckpt, ck, "h_ckpt"},
                                 {a.dout, dob, "dout"}, {a.dht, st, "dht"}, {a.fwd_records, a.fwd_records_bytes, "fwd_workspace"},
                                 {a.cu, a.cu ? (static_cast<size_t>(a.ndocs) + 1) * 4 : 0, "cu_seqlens"}}));
    }
    return hip_status(ckda::launch_bwd(a, nslots, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

static ckda_status_t bwd_equal(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                               const void* q, const void* k, const void* v, const float* g, const int8_t* s,
                               const float* beta, float scale, const float* h0, const float* h_ckpt,
                               const void* fwd_ws, size_t fwd_ws_bytes, bool with_records,
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
    a.gate_map = (flags & CKDA_GATE_MAP) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s ? s : reinterpret_cast<const int8_t*>(g); a.beta = beta; a.scale = scale; a.h0 = h0;
    a.h_ckpt = h_ckpt; a.dout = dout; a.dht = dht; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
    a.dbeta = dbeta; a.dh0 = dh0; a.cu = nullptr; a.ndocs = 0;
    if (with_records) CKDA_TRY(check_fwd_records(a, fwd_slots(B, T), T > 0, fwd_ws, fwd_ws_bytes));
    return bwd_common(a, fwd_slots(B, T), T > 0, workspace, workspace_bytes, stream,
                      with_records ? "ckda_bwd_with_records launch" : "ckda_bwd launch");
}

ckda_status_t ckda_bwd(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                       const void* q, const void* k, const void* v, const float* g, const int8_t* s,
                       const float* beta, float scale, const float* h0, const float* h_ckpt,
                       const void* dout, const float* dht, float* dq, float* dk, float* dv,
                       float* dg, float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                       ckda_stream_t stream) {
    return bwd_equal(B, T, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, h_ckpt, nullptr, 0, false,
                     dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes, stream);
}

ckda_status_t ckda_bwd_with_records(int B, int T, int H, int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                                    const void* q, const void* k, const void* v, const float* g, const int8_t* s,
                                    const float* beta, float scale, const float* h0, const float* h_ckpt,
                                    const void* fwd_workspace, size_t fwd_workspace_bytes, const void* dout,
                                    const float* dht, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                                    float* dh0, void* workspace, size_t workspace_bytes, ckda_stream_t stream) {
    return bwd_equal(B, T, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, h_ckpt, fwd_workspace,
                     fwd_workspace_bytes, true, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes,
                     stream);
}

static ckda_status_t bwd_docs(int N, int T_total, const int32_t* cu, const int32_t* cu_dev, int H,
                              int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q,
                              const void* k,
                              const void* v, const float* g, const int8_t* s, const float* beta,
                              float scale, const float* h0, const float* h_ckpt,
                              const void* fwd_ws, size_t fwd_ws_bytes, bool with_records, const void* dout,
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
    a.gate_map = (flags & CKDA_GATE_MAP) != 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.s = s ? s : reinterpret_cast<const int8_t*>(g); a.beta = beta; a.scale = scale; a.h0 = h0;
    a.h_ckpt = h_ckpt; a.dout = dout; a.dht = dht; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg;
    a.dbeta = dbeta; a.dh0 = dh0; a.cu = cu_dev; a.cu_host = cu; a.ndocs = N;
    if (with_records) CKDA_TRY(check_fwd_records(a, varlen_slots(N, T_total), T_total > 0, fwd_ws, fwd_ws_bytes));
    return bwd_common(a, varlen_slots(N, T_total), T_total > 0, workspace, workspace_bytes, stream,
                      with_records ? "ckda_bwd_varlen_with_records launch" : "ckda_bwd_varlen launch");
}

ckda_status_t ckda_bwd_varlen(int N, int T_total, const int32_t* cu, const int32_t* cu_dev, int H,
                              int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* q,
                              const void* k, const void* v, const float* g, const int8_t* s, const float* beta,
                              float scale, const float* h0, const float* h_ckpt, const void* dout,
                              const float* dht, float* dq, float* dk, float* dv, float* dg,
                              float* dbeta, float* dh0, void* workspace, size_t workspace_bytes,
                              ckda_stream_t stream) {
    return bwd_docs(N, T_total, cu, cu_dev, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, h_ckpt,
                    nullptr, 0, false, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace, workspace_bytes, stream);
}

ckda_status_t ckda_bwd_varlen_with_records(int N, int T_total, const int32_t* cu, const int32_t* cu_dev, int H,
                                           int DK, int DV, ckda_dtype_t in_dtype, ckda_flags_t flags,
                                           const void* q, const void* k, const void* v, const float* g,
                                           const int8_t* s, const float* beta, float scale, const float* h0,
                                           const float* h_ckpt, const void* fwd_workspace,
                                           size_t fwd_workspace_bytes, const void* dout, const float* dht,
                                           float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dh0,
                                           void* workspace, size_t workspace_bytes, ckda_stream_t stream) {
    return bwd_docs(N, T_total, cu, cu_dev, H, DK, DV, in_dtype, flags, q, k, v, g, s, beta, scale, h0, h_ckpt,
                    fwd_workspace, fwd_workspace_bytes, true, dout, dht, dq, dk, dv, dg, dbeta, dh0, workspace,
                    workspace_bytes, stream);
}


// ---------------------------------------------------------------------------
// Short convolution (the optional width-4 part of the pre-mixer prep)
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// shape, dtype, flag and sequence checks shared by the two sequence calls;
// fills a's sequence fields
ckda_status_t conv_common(int N, int T, const int32_t* cu_host, const int32_t* cu_dev, int C,
                          ckda_dtype_t dt, ckda_flags_t flags, ckda::ConvArgs& a) {
    CKDA_TRY(check_dtype(dt));
    if (flags & ~CKDA_CONV_SILU) return fail(CKDA_ERR_UNSUPPORTED, "unknown option flags 0x%x", unsigned(flags));
    if (N < 0 || T < 0 || C < 0) return fail(CKDA_ERR_SHAPE, "negative size (N=%d, T=%d, C=%d)", N, T, C);
    if (C % 4 != 0) return fail(CKDA_ERR_UNSUPPORTED, "C=%d channels: a multiple of 4 is required", C);
    if (static_cast<long long>(T) * C >= (1LL << 40) || C > (1 << 28))
        return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if ((cu_host == nullptr) != (cu_dev == nullptr))
        return fail(CKDA_ERR_SEQLENS, "give both cu_seqlens copies (host and device) or neither");
    if (cu_host) {
        CKDA_TRY(check_cu(N, T, cu_host));
    } else if (T > 0 && (N == 0 || T % N != 0)) {
        return fail(CKDA_ERR_SHAPE, "without cu_seqlens, T_total=%d must split into N=%d equal sequences", T, N);
    }
    a.N = N; a.T = T; a.C = C; a.bf16 = dt == CKDA_BF16; a.silu = (flags & CKDA_CONV_SILU) != 0;
    a.cu = cu_dev;
    return CKDA_OK;
}

}  // namespace

extern "C" {

size_t ckda_short_conv_bwd_workspace_bytes(int T_total, int C) {
    if (T_total < 0 || C < 0 || C % 4 != 0) return 0;
    return ckda::conv_bwd_workspace_bytes(T_total, C);
}

ckda_status_t ckda_short_conv_fwd(int N, int T_total, const int32_t* cu_seqlens_host,
                                  const int32_t* cu_seqlens_dev, int C, ckda_dtype_t in_dtype,
                                  ckda_flags_t flags, const void* x, const float* w, const void* state0,
                                  void* y, void* state_out, ckda_stream_t stream) {
    ckda::ConvArgs a{};
    CKDA_TRY(conv_common(N, T_total, cu_seqlens_host, cu_seqlens_dev, C, in_dtype, flags, a));
    if (C == 0 || (T_total == 0 && !state_out)) return ok();
    if (T_total > 0) { CKDA_REQUIRE(x); CKDA_REQUIRE(w); CKDA_REQUIRE(y); }
    CKDA_ALIGNED(x); CKDA_ALIGNED(w); CKDA_ALIGNED(state0); CKDA_ALIGNED(y); CKDA_ALIGNED(state_out);
    const size_t es = a.bf16 ? 2 : 4;
    const size_t xb = static_cast<size_t>(T_total) * C * es, wb = static_cast<size_t>(C) * 16;
    const size_t sb = static_cast<size_t>(N) * 3 * C * es;
    // the outgoing window may be the incoming one (updated in place), or apart from it
    const void* s0_other = state_out == state0 ? nullptr : state0;
    CKDA_TRY(check_no_alias({{y, xb, "y"}, {state_out, sb, "state_out"}},
                            {{x, xb, "x"}, {w, wb, "w"}, {s0_other, sb, "state0"}}));
    a.x = x; a.w = w; a.state0 = state0; a.y = y; a.state_out = state_out;
    return hip_status(ckda::launch_conv_fwd(a, static_cast<hipStream_t>(stream)), "ckda_short_conv_fwd launch");
}

ckda_status_t ckda_short_conv_bwd(int N, int T_total, const int32_t* cu_seqlens_host,
                                  const int32_t* cu_seqlens_dev, int C, ckda_dtype_t in_dtype,
                                  ckda_flags_t flags, const void* x, const float* w, const void* state0,
                                  const float* dy, float* dx, float* dw, float* dstate0, void* workspace,
                                  size_t workspace_bytes, ckda_stream_t stream) {
    ckda::ConvArgs a{};
    CKDA_TRY(conv_common(N, T_total, cu_seqlens_host, cu_seqlens_dev, C, in_dtype, flags, a));
    if (C == 0) return ok();
    CKDA_REQUIRE(w); CKDA_REQUIRE(dw);
    if (T_total > 0) { CKDA_REQUIRE(x); CKDA_REQUIRE(dy); CKDA_REQUIRE(dx); }
    CKDA_ALIGNED(x); CKDA_ALIGNED(w); CKDA_ALIGNED(state0); CKDA_ALIGNED(dy); CKDA_ALIGNED(dx); CKDA_ALIGNED(dw);
    CKDA_ALIGNED(dstate0); CKDA_ALIGNED(workspace);
    const size_t need = ckda::conv_bwd_workspace_bytes(T_total, C);
    if (need > 0) {
        CKDA_REQUIRE(workspace);
        if (workspace_bytes < need)
            return fail(CKDA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
    }
    const size_t es = a.bf16 ? 2 : 4;
    const size_t xb = static_cast<size_t>(T_total) * C * es, fb = static_cast<size_t>(T_total) * C * 4;
    const size_t wb = static_cast<size_t>(C) * 16, sb = static_cast<size_t>(N) * 3 * C;
    CKDA_TRY(check_no_alias({{dx, fb, "dx"}, {dw, wb, "dw"}, {dstate0, sb * 4, "dstate0"}, {workspace, workspace_bytes, "workspace"}},
                            {{x, xb, "x"}, {w, wb, "w"}, {state0, sb * es, "state0"}, {dy, fb, "dy"}}));
    a.x = x; a.w = w; a.state0 = state0; a.dy = dy; a.dx = dx; a.dw = dw; a.dstate0 = dstate0;
    a.partial = static_cast<float*>(workspace);
    return hip_status(ckda::launch_conv_bwd(a, static_cast<hipStream_t>(stream)), "ckda_short_conv_bwd launch");
}

ckda_status_t ckda_short_conv_step(int N, int C, ckda_dtype_t in_dtype, ckda_flags_t flags, const void* x,
                                   const float* w, void* window, void* y, ckda_stream_t stream) {
    CKDA_TRY(check_dtype(in_dtype));
    if (flags & ~CKDA_CONV_SILU) return fail(CKDA_ERR_UNSUPPORTED, "unknown option flags 0x%x", unsigned(flags));
    if (N < 0 || C < 0) return fail(CKDA_ERR_SHAPE, "negative size (N=%d, C=%d)", N, C);
    if (C % 4 != 0) return fail(CKDA_ERR_UNSUPPORTED, "C=%d channels: a multiple of 4 is required", C);
    if (static_cast<long long>(N) * C >= (1LL << 40) || C > (1 << 28))
        return fail(CKDA_ERR_UNSUPPORTED, "tensor too large");
    if (N == 0 || C == 0) return ok();
    CKDA_REQUIRE(x); CKDA_REQUIRE(w); CKDA_REQUIRE(window); CKDA_REQUIRE(y);
    CKDA_ALIGNED(x); CKDA_ALIGNED(w); CKDA_ALIGNED(window); CKDA_ALIGNED(y);
    const size_t es = in_dtype == CKDA_BF16 ? 2 : 4;
    const size_t xb = static_cast<size_t>(N) * C * es;
    CKDA_TRY(check_no_alias({{y, xb, "y"}, {window, 3 * xb, "window"}}, {{x, xb, "x"}, {w, static_cast<size_t>(C) * 16, "w"}}));
    return hip_status(ckda::launch_conv_step(N, C, in_dtype == CKDA_BF16, (flags & CKDA_CONV_SILU) != 0, x, w,
                                             window, y, static_cast<hipStream_t>(stream)),
                      "ckda_short_conv_step launch");
}

}  // extern "C"
