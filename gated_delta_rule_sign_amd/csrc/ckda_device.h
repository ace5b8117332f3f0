// ckda_device.h -- small device helpers shared by the CKDA kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// element types of the token tensors
// ---------------------------------------------------------------------------
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round-to-nearest-even float -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}
// two floats -> packed bf16 pair, a in bits 0..15 (one v_cvt_pk_bf16_f32)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i].bits); }
    static __device__ __forceinline__ void store(bf16_t* p, size_t i, float x) { p[i].bits = f32_to_bf16(x); }
};

// 8 consecutive elements of a token row, kept in their storage form until use
template <typename Tin>
struct Raw8;
template <>
struct Raw8<bf16_t> {
    u32x4 u;   // a native vector: a HIP_vector_type copy is a memcpy that can pin it in scratch
    __device__ __forceinline__ void load(const bf16_t* p) { u = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void zero() { u = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ float get(int e) const {
        const uint32_t w = u[e >> 1];
        return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    }
};
template <>
struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = reinterpret_cast<const f32x4*>(p)[0];
        b = reinterpret_cast<const f32x4*>(p)[1];
    }
    __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ float get(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// A raw buffer resource over `bytes` bytes at `base`: buffer stores beyond
// the range are dropped by the hardware range check and loads return 0, so
// a partially valid tile is written with unconditional stores (a guarded
// store is a branch, which also hides the count of outstanding vector memory
// operations from the compiler's wait insertion).  Dword 3 = 0x00020000 is
// the gfx9-family raw 32-bit format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void buffer_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, static_cast<int>(byte_off), 0, 0);
}
__device__ __forceinline__ void buffer_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, static_cast<int>(voff), static_cast<int>(soff), 0);
}
// loads through a raw buffer resource: a per-lane byte offset plus a uniform
// one (kept in a scalar register); out-of-range bytes read as 0
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
__device__ __forceinline__ uint32_t buffer_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}
__device__ __forceinline__ int buffer_load_i8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return static_cast<int8_t>(__builtin_amdgcn_raw_buffer_load_b8(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
__device__ __forceinline__ u32x2 buffer_load_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
__device__ __forceinline__ u32x4 buffer_load_u32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}
// an element of a token tensor (bf16 or fp32) as fp32
template <typename T>
__device__ __forceinline__ float buffer_load_elem(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(T) == 4) return buffer_load_f32(r, voff, soff);
    else return bf16_to_f32(static_cast<uint16_t>(buffer_load_u16(r, voff, soff)));
}

// exp(x) through the hardware base-2 exponential; the argument is clamped so
// that no infinity can be produced (exp2(126) is finite in fp32)
__device__ __forceinline__ float exp2_clamped(float x2) {
    return __builtin_amdgcn_exp2f(fminf(x2, 126.0f));
}

// The optional gate map (CKDA_GATE_MAP): the gate pre-activation x gives the
// signed gate alpha = tanh(x), carried as g = log max(|alpha|, e^kGateLogFloor)
// and its sign (x < 0), and the beta pre-activation y gives beta =
// 2 sigmoid(y) in (0, 2) (a reading of the Complex KDA paper page, section 3
// "CKDA.": gates in [-1, 1], beta in [0, 2], a magnitude floor).  The floor
// keeps every 16-token run of log-gates at -64 or above, inside the chunk
// kernels' anchored fast path.  Backward: dg/dx = (1 - tanh^2 x) / tanh x
// = 2 / sinh 2x above the floor, 0 on it; dbeta/dy = beta (1 - beta / 2).
// Both come from u = e^{-2|x|} (one hardware exp2): tanh|x| = (1 - u) / (1 + u)
// and 2 / sinh 2|x| = 4u / ((1 - u)(1 + u)), where 1 - u is exact for u >= 1/2,
// so the error is u's rounding carried through 1 - u: about 3e-6 in log tanh|x|
// at the floor's edge (|x| near 0.018), under 1e-6 from |x| = 0.1 on, and a
// relative 2e-6 in the derivative.  (A float32 model of these steps against
// float64 gives 1.3e-6 and 1.9e-6, and the same floor decisions, over 3e6
// points.)  Where tanh|x| rounds to 1 the log is 0, the gate's magnitude 1
// within 2^-24.
constexpr float kGateLogFloor = -4.0f;
__device__ __forceinline__ float gate_u(float x) { return __builtin_amdgcn_exp2f(-2.8853900817779268f * fabsf(x)); }
__device__ __forceinline__ float gate_log_tanh_u(float u) {   // log tanh|x|; -inf at x = 0
    return 0.69314718055994531f * __builtin_amdgcn_logf((1.f - u) * __builtin_amdgcn_rcpf(1.f + u));
}
__device__ __forceinline__ float gate_map_g(float x) { return fmaxf(gate_log_tanh_u(gate_u(x)), kGateLogFloor); }
__device__ __forceinline__ float gate_map_dgdx(float x) {
    const float u = gate_u(x);
    if (!(gate_log_tanh_u(u) >= kGateLogFloor)) return 0.f;
    return copysignf(4.f * u * __builtin_amdgcn_rcpf((1.f - u) * (1.f + u)), x);
}
__device__ __forceinline__ float gate_map_beta(float y) { return 2.f / (1.f + expf(-y)); }

// 1 / sqrt(ss) for a vector's sum of squares ss, through the hardware
// reciprocal square root (about 1 ulp on normal inputs).  A squared norm below
// fp32's normal range (the zero vector among them) gives 0, so such a vector
// normalises to zero instead of to infinities.
__device__ __forceinline__ float inv_norm(float ss) {
    return ss >= 1.17549435e-38f ? __builtin_amdgcn_rsqf(ss) : 0.f;
}

}  // namespace ckda
