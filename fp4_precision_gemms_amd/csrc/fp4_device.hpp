// fp4_device.hpp -- device-side scalar building blocks for gfx950: bf16
// unpacking, Philox4x32-10, E2M1 / E8M0 / E4M3 encoders, the sign vector of
// the randomized Hadamard transform.  Everything here is exact integer or
// single-rounding binary32 arithmetic, so each function is bit-reproducible.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

// ---------------------------------------------------------------------------
// bf16 halves of a packed 32-bit word (little-endian: element 0 low)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): 10 rounds, multipliers 0xD2511F53 /
// 0xCD9E8D57, Weyl key increments 0x9E3779B9 / 0xBB67AE85.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        // one 32 x 32 -> 64-bit product each (a single v_mad_u64_u32 instead
        // of separate low and high multiplies)
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1,
                       (uint32_t)p0);
    }
    return c;
}

// The four words that cover stream indices 4g .. 4g+3 of `purpose`.
__device__ __forceinline__ uint4 stream4(uint64_t seed, uint32_t purpose, uint64_t g) {
    return philox4x32_10(make_uint4((uint32_t)g, (uint32_t)(g >> 32), purpose, 0u),
                         (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t word_of(uint4 w, int i) {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// ---------------------------------------------------------------------------
// E2M1: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} coded 0..7, bit 3 = sign.
// ---------------------------------------------------------------------------

// Round-to-nearest-even, saturating.  For |v| < 2 the grid step is 0.5 and
// the code is rint(2|v|) (v_rndne: ties to even, and codes 0..4 are exactly
// the half-units).  For 2 <= |v| the code is 4 + 2*(exponent-1) + mantissa
// bit after rounding the binary32 mantissa to one bit, ties to even.
__device__ __forceinline__ uint32_t e2m1_rtn(float v) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 28) & 8u;
    const uint32_t a = bits & 0x7FFFFFFFu;
    uint32_t m;
    if (a < 0x40000000u) {                         // |v| < 2
        m = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
    } else {
        // round mantissa to 1 bit, ties to even: add 0x1FFFFF + lsb, drop 22 bits
        const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
        const uint32_t q = (r >> 22) - (128u << 1); // (exp-1)*2 + mbit, exp = biased-127
        m = q + 4u;                                 // 2 -> 4, 3 -> 5, 4 -> 6, 6 -> 7
        m = (a >= 0x40A00001u) ? 7u : m;            // |v| > 5 rounds to 6 (saturates)
    }
    return sign | m;
}

// Stochastic rounding with the comparator (u >> 8) * 2^-24 < p, p the
// fractional position of |v| between its grid neighbours; |v| >= 6 gives 6.
// Branch-free: the grid step is 0.5 below 2, 1 below 4 and 2 below 8, so
// t = |v| / step (an exact power-of-two scaling) has integer part
// code - 2k for the region k = 0, 1, 2 and fractional part p.  A NaN gives
// code 6 (never reached from a block with a finite scale).
__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t u) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t sign = (bits >> 28) & 8u;
    const float a = __uint_as_float(bits & 0x7FFFFFFFu);
    const float r = (float)(u >> 8) * 0x1p-24f;
    const bool lo = a < 2.0f, mid = a < 4.0f;
    const float t = a * (lo ? 2.0f : (mid ? 1.0f : 0.5f));
    const float fl = __builtin_floorf(t);
    uint32_t m = (uint32_t)fl + (lo ? 0u : (mid ? 2u : 4u)) + (r < t - fl ? 1u : 0u);
    m = a < 6.0f ? m : (a >= 6.0f ? 7u : 6u);
    return sign | m;
}

// E8M0 scale byte of a block from the bit pattern of its largest magnitude
// (sign cleared): floor(log2 m) - 2 + 127 = biased exponent - 2, clamped at
// 0; a NaN or infinite maximum gives 0xFF.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t mbits) {
    const uint32_t E = mbits >> 23;
    return E == 255u ? 255u : (E < 2u ? 0u : E - 2u);
}

// 2^-(byte-127) as binary32, valid for byte in [0, 252].
__device__ __forceinline__ float inv_scale_from_e8m0(uint32_t byte) {
    return __uint_as_float((254u - byte) << 23);
}

// ---------------------------------------------------------------------------
// E4M3 ("fn": no infinities, max 448).  Non-negative finite inputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t code) {
    const uint32_t e = (code >> 3) & 15u, m = code & 7u;
    return e == 0u ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Largest code whose value is <= a, with that value and the gap to the next
// code (a < 448).
__device__ __forceinline__ uint32_t e4m3_floor(float a, float* lo, float* gap) {
    if (a < 0x1p-6f) {                               // subnormal: k * 2^-9
        const float k = __builtin_floorf(a * 512.0f);
        *lo = k * 0x1p-9f;
        *gap = 0x1p-9f;
        return (uint32_t)k;
    }
    const uint32_t b = __float_as_uint(a);
    const uint32_t e = (b >> 23) - 127u + 7u;        // biased E4M3 exponent, 1..15
    *lo = __uint_as_float(b & 0xFFF00000u);
    *gap = __uint_as_float((b & 0x7F800000u) - (3u << 23));
    return (e << 3) | ((b >> 20) & 7u);
}

__device__ __forceinline__ uint32_t e4m3_rne(float a) {
    if (a >= 448.0f) return 0x7Eu;
    float lo, gap;
    const uint32_t c = e4m3_floor(a, &lo, &gap);
    const float d = a - lo;                          // exact
    const float half = gap * 0.5f;
    if (d > half || (d == half && (c & 1u))) return c + 1u;
    return c;
}

__device__ __forceinline__ uint32_t e4m3_sr(float a, uint32_t u) {
    if (a >= 448.0f) return 0x7Eu;
    float lo, gap;
    const uint32_t c = e4m3_floor(a, &lo, &gap);
    // (a - lo) / gap as a product with the exact reciprocal of the power of
    // two gap (2^-9 .. 2^5): the same binary32 result, without a division
    const float p = (a - lo) * __uint_as_float((254u << 23) - __float_as_uint(gap));
    const float r = (float)(u >> 8) * 0x1p-24f;
    return r < p ? c + 1u : c;
}

// ---------------------------------------------------------------------------
// Hadamard sign word: bit j set means element j of every n-block is negated.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t hadamard_sign_word(int had, uint64_t seed) {
    return had == 2 ? stream4(seed, 1u, 0u).x : 0u;
}

// x * (+-1) as a sign-bit flip (exact, also for zeros).
__device__ __forceinline__ float flip_if(float x, uint32_t bit) {
    return __uint_as_float(__float_as_uint(x) ^ (bit << 31));
}

}  // namespace fp4dev
