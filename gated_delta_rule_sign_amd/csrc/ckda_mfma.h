// ckda_mfma.h -- split-precision bf16 MFMA helpers for gfx950.
//
// A float x is carried as hi + lo with hi = bf16(x), lo = bf16(x - hi)
// (about 16 significant bits).  A product is taken as
//     hi(a) hi(b) + hi(a) lo(b) + lo(a) hi(b)
// on the bf16 matrix cores with fp32 accumulation; lo(a) lo(b) is dropped.
//
// Lane layouts used (wave64, L = lane):
//  * v_mfma_f32_16x16x32_bf16: A lane L supplies row (L % 16), B lane L
//    column (L % 16), each with 8 K-slots; slot j of lane group (L / 16) of A
//    meets slot j of the same group of B.  The kernels only rely on that
//    pairing, so each product chooses its own K order.
//  * C/D of every 16x16 MFMA: lane L holds rows 4*(L/16) + i (i = 0..3) of
//    column (L % 16).
//  * v_mfma_f32_16x16x16_bf16: as above with 4 K-slots; its B operand layout
//    coincides with the C/D layout, so a result tile feeds the next product
//    directly.
#pragma once
#include "ckda_device.h"

namespace ckda {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct Split8 { bf16x8 hi, lo; };
struct Split4 { s16x4 hi, lo; };

__device__ __forceinline__ void split1(float x, uint16_t& h, uint16_t& l) {
    h = f32_to_bf16(x);
    l = f32_to_bf16(x - bf16_to_f32(h));
}

// two floats at once (one packed conversion per plane): hi and lo pairs,
// element a in bits 0..15
struct SplitPair { uint32_t hi, lo; };
__device__ __forceinline__ SplitPair split2(float a, float b) {
    const uint32_t h = cvt_pk_bf16(a, b);
    const float ha = __uint_as_float(h << 16), hb = __uint_as_float(h & 0xffff0000u);
    return SplitPair{h, cvt_pk_bf16(a - ha, b - hb)};
}

__device__ __forceinline__ Split4 split4(f32x4 x) {
    const SplitPair p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
    Split4 r;
    r.hi = __builtin_bit_cast(s16x4, u32x2{p0.hi, p1.hi});
    r.lo = __builtin_bit_cast(s16x4, u32x2{p0.lo, p1.lo});
    return r;
}

// slots 0..3 from a, 4..7 from b
__device__ __forceinline__ Split8 split8(f32x4 a, f32x4 b) {
    const SplitPair p0 = split2(a[0], a[1]), p1 = split2(a[2], a[3]);
    const SplitPair p2 = split2(b[0], b[1]), p3 = split2(b[2], b[3]);
    Split8 r;
    r.hi = __builtin_bit_cast(bf16x8, u32x4{p0.hi, p1.hi, p2.hi, p3.hi});
    r.lo = __builtin_bit_cast(bf16x8, u32x4{p0.lo, p1.lo, p2.lo, p3.lo});
    return r;
}

__device__ __forceinline__ f32x4 mfma32x3(const bf16x8& ah, const bf16x8& al, const bf16x8& bh,
                                         const bf16x8& bl, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ f32x4 mfma16x3(const s16x4& ah, const s16x4& al, const s16x4& bh,
                                         const s16x4& bl, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    return acc;
}

// LDS fragment loads of bf16 data stored as uint16_t
__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {           // 16-byte aligned
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 lds4x2(const uint16_t* p0, const uint16_t* p1) {  // 8-byte aligned
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ s16x4 lds4s(const uint16_t* p) {            // 8-byte aligned
    return *reinterpret_cast<const s16x4*>(p);
}

}  // namespace ckda
