// MFMA operand handling shared by the scoring kernels (gfx950).
//
// Query rows are the A operand (32 heads per block of rows), key rows the B
// operand (32 keys per block of columns), the d axis the contraction; the
// element types feed v_mfma_f32_32x32x16_bf16 (bf16, and OCP e4m3 widened
// exactly to bf16), v_mfma_f32_32x32x2_f32 (fp32) with fp32 accumulation, or,
// when asked for, v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 as it is).  Every kernel that uses these operands with the same
// instruction order gets bit-identical dot products.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsai {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// MFMA operand handling.  For every dtype, lane (hh = lane / 32, r = lane % 32)
// supplies row r of A and column r of B; the contraction slots a lane owns
// are the contiguous half d in [hh*D/2, hh*D/2 + D/2), split into KS steps.
// A and B use the same slot -> d map, so the products pair up correctly.
// load_a therefore also loads a key row as B straight from global memory;
// raw_row + from_raw split it into the loads (RAW 16-byte vectors per lane)
// and the conversion, so loads can be issued ahead of use.
// ---------------------------------------------------------------------------
template <int DT, int D> struct Op;

// The RAW 16-byte vectors of row `row` (D codes of ES bytes) that lane half
// hh contributes: bytes [hh * D * ES / 2, (hh + 1) * D * ES / 2).
template <class O, int D>
__device__ inline void raw_row(const char *row, int hh, uint4 (&raw)[O::RAW])
{
    const uint4 *p = reinterpret_cast<const uint4 *>(row + hh * (D / 2) * O::ES);
#pragma unroll
    for (int i = 0; i < O::RAW; ++i) raw[i] = p[i];
}

template <int D> struct Op<1, D> {  // bf16
    using A = bf16x8;
    static constexpr int ES = 2, KS = D / 16, NCH = D * 2 / 16, GCH = NCH, RAW = KS;
    static constexpr int CPK = 1;  // 16-byte LDS chunks per operand
    __device__ static A from_chunks(const uint4 *c) { return __builtin_bit_cast(A, c[0]); }
    __device__ static void store_chunk(uint4 *tile, int r, int gch, uint4 v, int swz)
    {
        tile[r * NCH + (gch ^ swz)] = v;
    }
    __device__ static void load_a(const char *row, int hh, A (&a)[KS])
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(row + hh * (D / 2) * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = __builtin_bit_cast(A, p[ks]);
    }
    __device__ static void load_b(const uint4 *tile, int r, int hh, int swz, A (&b)[KS])
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            b[ks] = __builtin_bit_cast(A, tile[r * NCH + ((hh * KS + ks) ^ swz)]);
    }
    __device__ static void from_raw(const uint4 (&raw)[RAW], A (&a)[KS])
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = __builtin_bit_cast(A, raw[ks]);
    }
    __device__ static void load_b_one(const uint4 *tile, int r, int hh, int swz, int ks, A &b)
    {
        b = __builtin_bit_cast(A, tile[r * NCH + ((hh * KS + ks) ^ swz)]);
    }
    __device__ static f32x16 mma(A a, A b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static A zero() { return __builtin_bit_cast(A, make_uint4(0, 0, 0, 0)); }
};

// OCP e4m3 codes, widened exactly to bf16 (every e4m3 value is a bf16 value)
// and contracted on the bf16 MFMA with fp32 accumulation.  The native
// f8f6f4 MFMA is not used: its 64-product dot is accumulated at reduced
// precision (measured on gfx950: error up to 2^-12 of the sum of |products|
// on random codes, 2^-15 on normal-like data), against 2^-24 for bf16.
template <int D> struct Op<2, D> : Op<1, D> {
    using A = bf16x8;
    static constexpr int ES = 1, KS = D / 16, NCH = D * 2 / 16, GCH = D / 16, RAW = KS / 2;
    static constexpr int CPK = 1;
    template <bool HI> __device__ static uint32_t widen2(uint32_t w)
    {
        auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
        return __builtin_bit_cast(uint32_t, v);
    }
    // 16 fp8 codes -> two 16-B chunks of 8 bf16
    __device__ static void widen16(uint4 x, uint4 &lo, uint4 &hi)
    {
        lo = make_uint4(widen2<false>(x.x), widen2<true>(x.x), widen2<false>(x.y), widen2<true>(x.y));
        hi = make_uint4(widen2<false>(x.z), widen2<true>(x.z), widen2<false>(x.w), widen2<true>(x.w));
    }
    __device__ static void load_a(const char *row, int hh, A (&a)[KS])
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(row + hh * (D / 2));
#pragma unroll
        for (int c = 0; c < KS / 2; ++c) {
            uint4 lo, hi;
            widen16(p[c], lo, hi);
            a[2 * c] = __builtin_bit_cast(A, lo);
            a[2 * c + 1] = __builtin_bit_cast(A, hi);
        }
    }
    __device__ static void from_raw(const uint4 (&raw)[RAW], A (&a)[KS])
    {
#pragma unroll
        for (int c = 0; c < KS / 2; ++c) {
            uint4 lo, hi;
            widen16(raw[c], lo, hi);
            a[2 * c] = __builtin_bit_cast(A, lo);
            a[2 * c + 1] = __builtin_bit_cast(A, hi);
        }
    }
    // global chunk gch of a key row (16 codes) -> LDS chunks 2*gch, 2*gch+1
    __device__ static void store_chunk(uint4 *tile, int r, int gch, uint4 v, int swz)
    {
        uint4 lo, hi;
        widen16(v, lo, hi);
        tile[r * NCH + ((2 * gch) ^ swz)] = lo;
        tile[r * NCH + ((2 * gch + 1) ^ swz)] = hi;
    }
};

// OCP e4m3 codes contracted as they are on the gfx950 scaled f8f6f4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, both formats e4m3, both block scales
// 2^0), 64 products per instruction.  A lane supplies 32 codes of its row
// (A) or key (B): the contiguous half d in [hh*D/2, hh*D/2 + D/2) split into
// KS = D/64 operands, the same slot -> d map for A and B.  Each operand is
// two 16-byte chunks; keys stay e4m3 in LDS (half the bytes of a widened
// tile).  The instruction's internal accumulation is narrower than fp32
// (its products are summed at reduced precision before the fp32 add), so
// this instance is used only when the caller asks for it.
template <int D> struct Op<3, D> {
    static_assert(D % 64 == 0, "one operand covers 32 codes of each lane half");
    using A = i32x8;
    static constexpr int ES = 1, KS = D / 64, NCH = D / 16, GCH = NCH, RAW = 2 * KS;
    static constexpr int CPK = 2;
    __device__ static A from_chunks(const uint4 *c)
    {
        return A{(int)c[0].x, (int)c[0].y, (int)c[0].z, (int)c[0].w,
                 (int)c[1].x, (int)c[1].y, (int)c[1].z, (int)c[1].w};
    }
    __device__ static void store_chunk(uint4 *tile, int r, int gch, uint4 v, int swz)
    {
        tile[r * NCH + (gch ^ swz)] = v;
    }
    __device__ static void load_a(const char *row, int hh, A (&a)[KS])
    {
        const uint4 *p = reinterpret_cast<const uint4 *>(row + hh * (D / 2));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = from_chunks(p + 2 * ks);
    }
    __device__ static void load_b(const uint4 *tile, int r, int hh, int swz, A (&b)[KS])
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load_b_one(tile, r, hh, swz, ks, b[ks]);
    }
    __device__ static void load_b_one(const uint4 *tile, int r, int hh, int swz, int ks, A &b)
    {
        const uint4 c[2] = {tile[r * NCH + ((hh * 2 * KS + 2 * ks) ^ swz)],
                            tile[r * NCH + ((hh * 2 * KS + 2 * ks + 1) ^ swz)]};
        b = from_chunks(c);
    }
    __device__ static void from_raw(const uint4 (&raw)[RAW], A (&a)[KS])
    {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = from_chunks(raw + 2 * ks);
    }
    __device__ static f32x16 mma(A a, A b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    }
    __device__ static A zero() { return A{0, 0, 0, 0, 0, 0, 0, 0}; }
};

template <int D> struct Op<0, D> {  // fp32
    using A = float;
    static constexpr int ES = 4, KS = D / 2, NCH = D * 4 / 16, GCH = NCH, RAW = KS / 4;
    static constexpr int CPK = 0;  // operands are single floats (no chunk loads)
    __device__ static A from_chunks(const uint4 *) { return 0.f; }  // not used
    __device__ static void store_chunk(uint4 *tile, int r, int gch, uint4 v, int swz)
    {
        tile[r * NCH + (gch ^ swz)] = v;
    }
    __device__ static void load_a(const char *row, int hh, A (&a)[KS])
    {
        const float4 *p = reinterpret_cast<const float4 *>(row + hh * (D / 2) * 4);
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            float4 v = p[c];
            a[4 * c] = v.x; a[4 * c + 1] = v.y; a[4 * c + 2] = v.z; a[4 * c + 3] = v.w;
        }
    }
    __device__ static void load_b(const uint4 *tile, int r, int hh, int swz, A (&b)[KS])
    {
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            uint4 v = tile[r * NCH + ((hh * (KS / 4) + c) ^ swz)];
            b[4 * c] = __uint_as_float(v.x); b[4 * c + 1] = __uint_as_float(v.y);
            b[4 * c + 2] = __uint_as_float(v.z); b[4 * c + 3] = __uint_as_float(v.w);
        }
    }
    __device__ static void from_raw(const uint4 (&raw)[RAW], A (&a)[KS])
    {
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            a[4 * c] = __uint_as_float(raw[c].x); a[4 * c + 1] = __uint_as_float(raw[c].y);
            a[4 * c + 2] = __uint_as_float(raw[c].z); a[4 * c + 3] = __uint_as_float(raw[c].w);
        }
    }
    __device__ static void load_b_one(const uint4 *tile, int r, int hh, int swz, int ks, A &b)
    {
        const uint4 v = tile[r * NCH + ((hh * (KS / 4) + ks / 4) ^ swz)];
        const uint32_t w = ks % 4 == 0 ? v.x : ks % 4 == 1 ? v.y : ks % 4 == 2 ? v.z : v.w;
        b = __uint_as_float(w);
    }
    __device__ static f32x16 mma(A a, A b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static A zero() { return 0.f; }
};

}  // namespace
}  // namespace dsai
