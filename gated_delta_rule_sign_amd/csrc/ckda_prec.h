// ckda_prec.h -- matrix-core precision policies for the chunked kernels.
//
// Operands staged in LDS take 4 bytes per element in both policies:
//  * Prec<false> (bf16 inputs): two bf16 planes, hi = bf16(x) and
//    lo = bf16(x - hi); a product is hi*hi + hi*lo + lo*hi on the bf16
//    matrix cores (v_mfma_f32_16x16x32_bf16 / 16x16x16), fp32 accumulate.
//  * Prec<true> (fp32 inputs): one fp32 plane; products on the fp32 matrix
//    cores (v_mfma_f32_16x16x4_f32), one instruction per K-slot.
//
// Fragment conventions (wave64, lane L, n = L % 16, g = L / 16):
//  * Frag8: 8 K-slots per lane.  A lane (n, g) supplies row n, B lane (n, g)
//    column n; slot j of A lane (., g) meets slot j of B lane (., g).  Each
//    call site picks which K index each (g, j) carries, identically for A
//    and B.
//  * Frag4: 4 K-slots, for 16x16x16 products.  Its B layout equals the C/D
//    layout of a 16x16 result (lane (n, g) holds rows 4g..4g+3, column n).
//  * C/D: lane (n, g) holds rows 4g + i (i = 0..3) of column n.
#pragma once
#include "ckda_mfma.h"

namespace ckda {

// An LDS operand region: `rows x pitch` elements; in the bf16 policy the lo
// plane follows the hi plane at `plane` elements.
struct LdsMat {
    unsigned char* base;
    int pitch;   // elements per row
    int plane;   // elements between the hi and lo planes (bf16 policy)
};

template <bool F32>
struct Prec;

template <>
struct Prec<false> {
    struct F8 { bf16x8 hi, lo; };
    struct F4 { s16x4 hi, lo; };
    static constexpr int kBytes = 4;   // per element, both planes together

    static __device__ __forceinline__ uint16_t* hp(const LdsMat& m, int r, int c) {
        return reinterpret_cast<uint16_t*>(m.base) + r * m.pitch + c;
    }
    static __device__ __forceinline__ uint16_t* lp(const LdsMat& m, int r, int c) {
        return reinterpret_cast<uint16_t*>(m.base) + m.plane + r * m.pitch + c;
    }
    // 8 consecutive elements (16-byte aligned in each plane)
    static __device__ __forceinline__ void store8(const LdsMat& m, int r, int c, const float (&x)[8]) {
        SplitPair sp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[i] = split2(x[2 * i], x[2 * i + 1]);
        *reinterpret_cast<u32x4*>(hp(m, r, c)) = u32x4{sp[0].hi, sp[1].hi, sp[2].hi, sp[3].hi};
        *reinterpret_cast<u32x4*>(lp(m, r, c)) = u32x4{sp[0].lo, sp[1].lo, sp[2].lo, sp[3].lo};
    }
    // 4 consecutive elements (8-byte aligned)
    static __device__ __forceinline__ void store4(const LdsMat& m, int r, int c, f32x4 x) {
        const SplitPair p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
        *reinterpret_cast<u32x2*>(hp(m, r, c)) = u32x2{p0.hi, p1.hi};
        *reinterpret_cast<u32x2*>(lp(m, r, c)) = u32x2{p0.lo, p1.lo};
    }
    static __device__ __forceinline__ void store1(const LdsMat& m, int r, int c, float x) {
        uint16_t h, l;
        split1(x, h, l);
        *hp(m, r, c) = h;
        *lp(m, r, c) = l;
    }
    // copy one element between regions without re-rounding
    static __device__ __forceinline__ void copy1(const LdsMat& d, int dr, int dc, const LdsMat& s, int sr, int sc) {
        *hp(d, dr, dc) = *hp(s, sr, sc);
        *lp(d, dr, dc) = *lp(s, sr, sc);
    }
    // an 8-slot fragment (elements c .. c+7 of row r) back to LDS
    static __device__ __forceinline__ void store8f(const LdsMat& m, int r, int c, const F8& x) {
        *reinterpret_cast<bf16x8*>(hp(m, r, c)) = x.hi;
        *reinterpret_cast<bf16x8*>(lp(m, r, c)) = x.lo;
    }
    // one element back as hi + lo
    static __device__ __forceinline__ float get1(const LdsMat& m, int r, int c) {
        return bf16_to_f32(*hp(m, r, c)) + bf16_to_f32(*lp(m, r, c));
    }
    static __device__ __forceinline__ F8 load8(const LdsMat& m, int r, int c) {
        return F8{lds8(hp(m, r, c)), lds8(lp(m, r, c))};
    }
    static __device__ __forceinline__ F8 load4x2(const LdsMat& m, int r, int ca, int cb) {
        return F8{lds4x2(hp(m, r, ca), hp(m, r, cb)), lds4x2(lp(m, r, ca), lp(m, r, cb))};
    }
    // A fragment of the 32-wide k-step at k0 for lane group g (columns
    // k0 + 4g .. +3 and k0 + 16 + 4g .. +3) from a region staged with those
    // two column quads side by side at k0 + 8g: one 16-byte read per plane
    // (a ds_read_b128 moves data at twice the rate of the split
    // ds_read2_b64 on gfx950)
    static constexpr bool kPermA = true;
    static __device__ __forceinline__ F8 loadA(const LdsMat& m, int r, int k0, int g) {
        return load8(m, r, k0 + 8 * g);
    }
    static __device__ __forceinline__ F4 load4(const LdsMat& m, int r, int c) {
        return F4{lds4s(hp(m, r, c)), lds4s(lp(m, r, c))};
    }
    static __device__ __forceinline__ F8 regs8(f32x4 a, f32x4 b) {
        const Split8 s = split8(a, b);
        return F8{s.hi, s.lo};
    }
    // slot e of a fragment back as one float (hi + lo)
    static __device__ __forceinline__ float get8(const F8& f, int e) {
        return static_cast<float>(f.hi[e]) + static_cast<float>(f.lo[e]);
    }
    static __device__ __forceinline__ F4 regs4(f32x4 a) {
        const Split4 s = split4(a);
        return F4{s.hi, s.lo};
    }
    static __device__ __forceinline__ f32x4 mma8(const F8& a, const F8& b, f32x4 acc) {
        return mfma32x3(a.hi, a.lo, b.hi, b.lo, acc);
    }
    static __device__ __forceinline__ f32x4 mma4(const F4& a, const F4& b, f32x4 acc) {
        return mfma16x3(a.hi, a.lo, b.hi, b.lo, acc);
    }

    // global (workspace) stores: row-major planes of `row` bytes per row,
    // lo plane `plane` bytes after the hi plane
    static __device__ __forceinline__ void gstore8(unsigned char* base, size_t plane, int row, int r, int c,
                                                   const float (&x)[8]) {
        SplitPair sp[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[i] = split2(x[2 * i], x[2 * i + 1]);
        unsigned char* p = base + static_cast<size_t>(r) * row + 2 * c;
        *reinterpret_cast<u32x4*>(p) = u32x4{sp[0].hi, sp[1].hi, sp[2].hi, sp[3].hi};
        *reinterpret_cast<u32x4*>(p + plane) = u32x4{sp[0].lo, sp[1].lo, sp[2].lo, sp[3].lo};
    }
    static __device__ __forceinline__ void gstore4(unsigned char* base, size_t plane, int row, int r, int c, f32x4 x) {
        const SplitPair p0 = split2(x[0], x[1]), p1 = split2(x[2], x[3]);
        unsigned char* p = base + static_cast<size_t>(r) * row + 2 * c;
        *reinterpret_cast<u32x2*>(p) = u32x2{p0.hi, p1.hi};
        *reinterpret_cast<u32x2*>(p + plane) = u32x2{p0.lo, p1.lo};
    }
    // two elements of one column (rows r and r + 1) of a two-plane matrix
    static __device__ __forceinline__ void gstore2c(unsigned char* base, size_t plane, int row, int r, int c,
                                                    float x0, float x1) {
        const SplitPair sp = split2(x0, x1);
        unsigned char* p = base + static_cast<size_t>(r) * row + 2 * c;
        *reinterpret_cast<uint16_t*>(p) = static_cast<uint16_t>(sp.hi);
        *reinterpret_cast<uint16_t*>(p + row) = static_cast<uint16_t>(sp.hi >> 16);
        *reinterpret_cast<uint16_t*>(p + plane) = static_cast<uint16_t>(sp.lo);
        *reinterpret_cast<uint16_t*>(p + plane + row) = static_cast<uint16_t>(sp.lo >> 16);
    }
    // N elements of one column c (rows r0 .. r0 + N - 1) of a two-plane matrix
    template <int N>
    static __device__ __forceinline__ void gstore_col(unsigned char* base, size_t plane, int row, int r0, int c,
                                                      const float* x) {
        unsigned char* p = base + static_cast<size_t>(r0) * row + 2 * c;
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const SplitPair sp = split2(x[i], x[i + 1]);
            *reinterpret_cast<uint16_t*>(p + static_cast<size_t>(i) * row) = static_cast<uint16_t>(sp.hi);
            *reinterpret_cast<uint16_t*>(p + static_cast<size_t>(i + 1) * row) = static_cast<uint16_t>(sp.hi >> 16);
            *reinterpret_cast<uint16_t*>(p + plane + static_cast<size_t>(i) * row) = static_cast<uint16_t>(sp.lo);
            *reinterpret_cast<uint16_t*>(p + plane + static_cast<size_t>(i + 1) * row) =
                static_cast<uint16_t>(sp.lo >> 16);
        }
    }
};

template <>
struct Prec<true> {
    struct F8 { f32x4 a, b; };
    struct F4 { f32x4 a; };
    static constexpr int kBytes = 4;

    static __device__ __forceinline__ float* fp(const LdsMat& m, int r, int c) {
        return reinterpret_cast<float*>(m.base) + r * m.pitch + c;
    }
    static __device__ __forceinline__ void store8(const LdsMat& m, int r, int c, const float (&x)[8]) {
        float4* p = reinterpret_cast<float4*>(fp(m, r, c));
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void store4(const LdsMat& m, int r, int c, f32x4 x) {
        *reinterpret_cast<float4*>(fp(m, r, c)) = make_float4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ void store1(const LdsMat& m, int r, int c, float x) { *fp(m, r, c) = x; }
    static __device__ __forceinline__ void copy1(const LdsMat& d, int dr, int dc, const LdsMat& s, int sr, int sc) {
        *fp(d, dr, dc) = *fp(s, sr, sc);
    }
    static __device__ __forceinline__ float get1(const LdsMat& m, int r, int c) { return *fp(m, r, c); }
    static __device__ __forceinline__ void store8f(const LdsMat& m, int r, int c, const F8& x) {
        float4* p = reinterpret_cast<float4*>(fp(m, r, c));
        p[0] = make_float4(x.a[0], x.a[1], x.a[2], x.a[3]);
        p[1] = make_float4(x.b[0], x.b[1], x.b[2], x.b[3]);
    }
    static __device__ __forceinline__ f32x4 ld4(const float* p) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        f32x4 r = {v.x, v.y, v.z, v.w};
        return r;
    }
    static __device__ __forceinline__ F8 load8(const LdsMat& m, int r, int c) {
        return F8{ld4(fp(m, r, c)), ld4(fp(m, r, c + 4))};
    }
    static __device__ __forceinline__ F8 load4x2(const LdsMat& m, int r, int ca, int cb) {
        return F8{ld4(fp(m, r, ca)), ld4(fp(m, r, cb))};
    }
    // fp32 regions are staged unpermuted: two 16-byte reads already
    static constexpr bool kPermA = false;
    static __device__ __forceinline__ F8 loadA(const LdsMat& m, int r, int k0, int g) {
        return load4x2(m, r, k0 + 4 * g, k0 + 16 + 4 * g);
    }
    static __device__ __forceinline__ F4 load4(const LdsMat& m, int r, int c) { return F4{ld4(fp(m, r, c))}; }
    static __device__ __forceinline__ F8 regs8(f32x4 a, f32x4 b) { return F8{a, b}; }
    static __device__ __forceinline__ float get8(const F8& f, int e) { return e < 4 ? f.a[e] : f.b[e - 4]; }
    static __device__ __forceinline__ F4 regs4(f32x4 a) { return F4{a}; }
    static __device__ __forceinline__ f32x4 mma8(const F8& x, const F8& y, f32x4 acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a[j], y.a[j], acc, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.b[j], y.b[j], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 mma4(const F4& x, const F4& y, f32x4 acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x.a[j], y.a[j], acc, 0, 0, 0);
        return acc;
    }


    static __device__ __forceinline__ void gstore8(unsigned char* base, size_t, int row, int r, int c,
                                                   const float (&x)[8]) {
        float4* p = reinterpret_cast<float4*>(base + static_cast<size_t>(r) * row + 4 * c);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    static __device__ __forceinline__ void gstore4(unsigned char* base, size_t, int row, int r, int c, f32x4 x) {
        *reinterpret_cast<float4*>(base + static_cast<size_t>(r) * row + 4 * c) = make_float4(x[0], x[1], x[2], x[3]);
    }
    static __device__ __forceinline__ void gstore2c(unsigned char* base, size_t, int row, int r, int c,
                                                    float x0, float x1) {
        float* p = reinterpret_cast<float*>(base + static_cast<size_t>(r) * row + 4 * c);
        p[0] = x0;
        *reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(p) + row) = x1;
    }
    template <int N>
    static __device__ __forceinline__ void gstore_col(unsigned char* base, size_t, int row, int r0, int c,
                                                      const float* x) {
        unsigned char* p = base + static_cast<size_t>(r0) * row + 4 * c;
#pragma unroll
        for (int i = 0; i < N; ++i) *reinterpret_cast<float*>(p + static_cast<size_t>(i) * row) = x[i];
    }
};

}  // namespace ckda
