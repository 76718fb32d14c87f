// kvq_device.h -- device helpers shared by the gfx950 kernels of libkvq.
//
// Number-format primitives (BF16 directed rounding, OCP E4M3 encode through
// the hardware converter, exact code -> bf16 conversions) and the MFMA
// wrapper.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bits_to_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
// Pair of bf16 from its 32 bits.  Takes the word by value: this compiler's
// __builtin_bit_cast of a vector-element lvalue (v[i]) reads element 0 for
// every i, so element accesses are always passed through a function argument.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }
__device__ __forceinline__ uint32_t f32_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 bits (low 16 of u) -> fp32, exact.
__device__ __forceinline__ float bf16lo(uint32_t u) { return bits_to_f32(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return bits_to_f32(u & 0xFFFF0000u); }

// Smallest bf16 >= f (finite f); result as bf16 bits.  The upper half of an
// fp32 is the bf16 truncation toward zero; a non-zero lower half on a positive
// value means the ceiling is one unit further from zero.
__device__ __forceinline__ uint32_t bf16_up_bits(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t t = u >> 16;
    if ((u & 0xFFFFu) != 0u && !(u >> 31)) t += 1u;
    return t;
}
// Largest bf16 <= f.
__device__ __forceinline__ uint32_t bf16_down_bits(float f) {
    uint32_t u = f32_to_bits(f);
    uint32_t t = u >> 16;
    if ((u & 0xFFFFu) != 0u && (u >> 31)) t += 1u;
    return t;
}

// Two fp32 -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 -> bf16 pairs hi = rne(a), lo = rne(a - hi) (low half = a0);
// returns {hi, lo}.  The remainders a - hi are exact and come from one dot
// product each, a + hi.x * m0.x + hi.y * m0.y with m0 = (-1, 0) and
// m1 = (0, -1) as bf16 pairs.  The caller passes m0 = 0x0000BF80 and
// m1 = 0xBF800000 from registers the compiler cannot see through (see
// opaque_sgpr): as inline constants they are encoded as the fp32 -1.0, and
// the remainders came out wrong.
__device__ __forceinline__ u32x2_t split_bf16(float a0, float a1, uint32_t m0, uint32_t m1) {
    const uint32_t hi = pack_bf16_rne(a0, a1);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(hi), as_bf16x2(m0), a0, false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(hi), as_bf16x2(m1), a1, false);
    return u32x2_t{hi, pack_bf16_rne(r0, r1)};
}

// A wave-uniform constant in an SGPR that the compiler treats as unknown.
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t c) {
    __asm__("" : "+s"(c));
    return c;
}

// Four fp32 -> four OCP E4M3 codes (byte i = code of the i-th argument):
// nearest-even through the gfx950 converter after an explicit clamp to
// +-448 (saturation); -0 keeps its sign; NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    float ca = fminf(fmaxf(a, -448.0f), 448.0f);
    float cb = fminf(fmaxf(b, -448.0f), 448.0f);
    float cc = fminf(fmaxf(c, -448.0f), 448.0f);
    float cd = fminf(fmaxf(d, -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, w, true);
    uint32_t r = (uint32_t)w;
    if (a != a) r = (r & 0xFFFFFF00u) | 0x7Fu;
    if (b != b) r = (r & 0xFFFF00FFu) | 0x7F00u;
    if (c != c) r = (r & 0xFF00FFFFu) | 0x7F0000u;
    if (d != d) r = (r & 0x00FFFFFFu) | 0x7F000000u;
    return r;
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> packed exact bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// Four fp32 -> four OCP E5M2 codes, as e4m3_encode4: nearest-even through the
// gfx950 converter (its BF8 format is OCP E5M2) after an explicit clamp to
// +-57344 (saturation, no infinities); -0 keeps its sign; NaN gives 0x7F.
__device__ __forceinline__ uint32_t e5m2_encode4(float a, float b, float c, float d) {
    float ca = fminf(fmaxf(a, -57344.0f), 57344.0f);
    float cb = fminf(fmaxf(b, -57344.0f), 57344.0f);
    float cc = fminf(fmaxf(c, -57344.0f), 57344.0f);
    float cd = fminf(fmaxf(d, -57344.0f), 57344.0f);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(ca, cb, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(cc, cd, w, true);
    uint32_t r = (uint32_t)w;
    if (a != a) r = (r & 0xFFFFFF00u) | 0x7Fu;
    if (b != b) r = (r & 0xFFFF00FFu) | 0x7F00u;
    if (c != c) r = (r & 0xFF00FFFFu) | 0x7F0000u;
    if (d != d) r = (r & 0x00FFFFFFu) | 0x7F000000u;
    return r;
}

// Two E5M2 codes (bytes 0,1 or 2,3 of w) -> packed exact bf16 pair (two
// mantissa bits and exponents down to 2^-16 fit bf16 exactly).
template <bool HI>
__device__ __forceinline__ uint32_t e5m2x2_to_bf16x2(uint32_t w) {
    bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, v);
}

// The dtype codes of the kernels' templates (as kvq_dtype in kvq.h).
constexpr int kFP8 = 1;    // OCP E4M3
constexpr int kINT8 = 2;   // u8 asymmetric
constexpr int kE5M2 = 4;   // OCP E5M2
constexpr bool is_fp8_format(int dt) { return dt == kFP8 || dt == kE5M2; }

// Two FP8 codes of format DT -> packed exact bf16 pair.
template <int DT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    if constexpr (DT == kE5M2) return e5m2x2_to_bf16x2<HI>(w);
    else return e4m3x2_to_bf16x2<HI>(w);
}

// Byte select: result byte i = selector byte i of `sel` choosing from
// {lo bytes 0..3 (values 0..3), hi bytes 0..3 (values 4..7)}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two u8 codes (byte positions BA, BB of wa, wb) -> packed exact bf16 pair.
// The fp32 value of a byte is exact and has at most 8 significant bits, so its
// upper half is the exact bf16.
template <int BA>
__device__ __forceinline__ float u8_to_f32(uint32_t w) {
    return (float)((w >> (8 * BA)) & 0xFFu);
}
__device__ __forceinline__ uint32_t hi_halves(float a, float b) {
    return perm(f32_to_bits(b), f32_to_bits(a), 0x07060302u);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));


__device__ __forceinline__ float f16_value(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    f16x2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4_t mfma_16x16x32_f16(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Maximum (minimum) over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane
// groups of a 16-column MFMA tile) with the gfx950 lane-swap instructions, in
// registers.
template <bool MAX>
__device__ __forceinline__ float extreme_over_groups(float v) {
    const uint32_t u = f32_to_bits(v);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const float a0 = bits_to_f32(s32[0]), a1 = bits_to_f32(s32[1]);
    const float m = MAX ? fmaxf(a0, a1) : fminf(a0, a1);
    const uint32_t w = f32_to_bits(m);
    const auto s16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    const float b0 = bits_to_f32(s16[0]), b1 = bits_to_f32(s16[1]);
    return MAX ? fmaxf(b0, b1) : fminf(b0, b1);
}
__device__ __forceinline__ float max_over_groups(float v) { return extreme_over_groups<true>(v); }

// DPP move within rows of 16 lanes (row_ror:n = 0x120 + n, quad_perm = 0x00-0xFF).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}

// Maximum (minimum) over each group of 8 lanes in registers: lane ^ 1 and
// lane ^ 2 by quad permutations, then the mirror within the half row (lane
// 7 - i), which pairs each quad with the other.
template <bool MAX>
__device__ __forceinline__ float group8_extreme(float v) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    v = op(v, bits_to_f32(dpp_mov<0xB1>(f32_to_bits(v))));    // quad_perm [1,0,3,2]
    v = op(v, bits_to_f32(dpp_mov<0x4E>(f32_to_bits(v))));    // quad_perm [2,3,0,1]
    return op(v, bits_to_f32(dpp_mov<0x141>(f32_to_bits(v))));  // row_half_mirror
}

// Maximum (minimum) over the whole wave in registers: rotations by 1, 2, 4, 8
// within each row of 16 lanes, then across the four rows.
template <bool MAX>
__device__ __forceinline__ float wave_extreme(float v) {
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
    v = op(v, bits_to_f32(dpp_mov<0x121>(f32_to_bits(v))));
    v = op(v, bits_to_f32(dpp_mov<0x122>(f32_to_bits(v))));
    v = op(v, bits_to_f32(dpp_mov<0x124>(f32_to_bits(v))));
    v = op(v, bits_to_f32(dpp_mov<0x128>(f32_to_bits(v))));
    return extreme_over_groups<MAX>(v);
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
    return (T)__builtin_amdgcn_readfirstlane((int)v);
}

}  // namespace kvq
