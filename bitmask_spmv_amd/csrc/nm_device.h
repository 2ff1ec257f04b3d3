// nm_device.h -- small device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nmk {

constexpr int kWave = 64;  // CDNA wavefront width

// Native 4 x 32-bit vector (16-byte global / LDS accesses, non-temporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resources: loads past num_records return zero without touching memory,
// so a wave can always issue the same number of loads (the in-order vmcnt counter
// then lets one batch be awaited while the next is still in flight).
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw (untyped) buffer descriptor word 3
constexpr int kLoadNT = 2;              // cache policy: non-temporal (streamed once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// bf16 pattern -> fp32 (exact: bf16 is the upper half of binary32).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 pattern, round to nearest, ties to even (finite inputs; overflow -> inf).
// Integer form, so no denormal mode or hardware conversion setting can change it.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Exact widening of a binary32 bit pattern (normal or subnormal, sign dropped) to
// binary64, done with integer operations so no fp32 denormal flushing can apply.
__device__ __forceinline__ double abs_f32bits_to_f64(uint32_t u) {
    uint32_t e = (u >> 23) & 0xFFu;
    uint32_t m = u & 0x7FFFFFu;
    uint64_t d;
    if (e == 0) {
        if (m == 0) return 0.0;
        int sh = __clz(m) - 8;  // brings the leading one to bit 23
        m <<= sh;
        d = ((uint64_t)(1023 - 126 - sh) << 52) | ((uint64_t)(m & 0x7FFFFFu) << 29);
    } else {
        d = ((uint64_t)(e - 127 + 1023) << 52) | ((uint64_t)m << 29);
    }
    return __longlong_as_double((long long)d);
}

// binary64 (non-negative, finite) -> binary32 bits, round to nearest even, integer form
// (subnormal results handled; no flush-to-zero).
__device__ __forceinline__ uint32_t f64_to_f32_rne_bits(double v) {
    uint64_t u = (uint64_t)__double_as_longlong(v);
    int e = (int)((u >> 52) & 0x7FFu);
    if (e == 0) return 0u;  // below 2^-1022: rounds to +0 in binary32
    uint64_t mant = (u & ((1ull << 52) - 1)) | (1ull << 52);
    int ef = e - 1023 + 127;
    if (ef >= 255) return 0x7F800000u;
    int shift = ef >= 1 ? 29 : 29 + (1 - ef);
    if (shift > 54) return 0u;  // below half of the smallest subnormal
    uint64_t q = mant >> shift;
    uint64_t rem = mant & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (ef >= 1) return ((uint32_t)ef << 23) + (uint32_t)q - (1u << 23);
    return (uint32_t)q;
}

// Correctly rounded fp64 square root of s >= 0: the hardware-assisted sqrt is followed
// by an exact neighbour test (sign of s - r*r_next computed with one fused rounding),
// so the result does not depend on the accuracy of the first approximation as long as
// it is within one ulp.
__device__ __forceinline__ double sqrt_rn_f64(double s) {
    if (!(s > 0.0)) return 0.0;
    double r = __builtin_sqrt(s);
    long long rb = __double_as_longlong(r);
    double rp = __longlong_as_double(rb + 1);
    double rm = __longlong_as_double(rb - 1);
    if (__builtin_fma(-r, rp, s) > 0.0)
        r = rp;
    else if (__builtin_fma(-r, rm, s) <= 0.0)
        r = rm;
    return r;
}

// Sum over the 64 lanes of a wavefront, returned in every lane.  Four DPP steps
// (quad swaps, half-row and row mirrors) leave each 16-lane row holding its row sum;
// the rows then meet through the gfx950 lane swaps (rows 0+1 and 2+3, then the two
// halves), added in a fixed order in every lane, so the result does not depend on
// timing: (r0 + r1) + (r2 + r3).
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Lanes at the same position of the four 16-lane rows added, (r0 + r1) + (r2 + r3), the
// result in all four of them.
__device__ __forceinline__ float cross_rows_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // [r0 r0 r2 r2], [r1 r1 r3 r3]
    const float w = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const uint32_t uw = __float_as_uint(w);
    const auto q = __builtin_amdgcn_permlane32_swap(uw, uw, false, false);  // [lo lo], [hi hi]
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm(1,0,3,2)
    v = dpp_add<0x4E>(v);   // quad_perm(2,3,0,1)
    v = dpp_add<0x141>(v);  // row_half_mirror
    v = dpp_add<0x140>(v);  // row_mirror
    return cross_rows_sum(v);
}

// Gated-MLP epilogue (kEpiSwiGLU, nm_kernels.h): h = silu(g) * u in fp32.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + __expf(-g)) * u; }

// Position of the lowest set bit of m, and 31 when m has no bit set.  (__builtin_ctz is
// undefined for 0, so a "& 31" applied to it may be folded away and the hardware's
// bit scan then yields -1; or-ing in bit 31 keeps every result a valid column.)
__device__ __forceinline__ int low_bit(uint32_t m) { return __builtin_ctz(m | 0x80000000u); }

}  // namespace nmk
