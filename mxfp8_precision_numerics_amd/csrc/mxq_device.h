// Device-side helpers shared by the gfx950 kernels of libmxq (internal; not part of the C ABI).
//
// Conversion instructions used (behaviour checked on gfx950 before use, and by the parity tests):
//   v_cvt_scalef32_pk_fp8_bf16  two bf16 -> two E4M3, computing x / 2^E where E is the exponent field of the
//                               fp32 scale operand (mantissa ignored); round to nearest even, subnormals kept.
//                               It does not saturate: a result beyond 448 becomes a NaN pattern, so callers
//                               either prove |x/s| <= 448 (the rceil rule) or patch those lanes.
//   v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32  two fp32 -> two E4M3 / E5M2, RNE, no saturation (same caveat).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

enum : int { RULE_RCEIL = 0, RULE_FLOOR = 1 };

// Operand range classes for the FP8 matrix instruction (the GEMM's range check and the quantizers' range words use
// the same definition): a 64-value window of K (one instruction's K span) is wide if it holds a nonzero code and at
// least kWideCount of its codes lie more than kWideBinades binades below the window's largest, a code's binade being
// its exponent field plus, for MX, its 32-block's scale byte.
constexpr int kWideBinades = 6, kWideCount = 24;

// Per-16-bit-lane unsigned max of two packed pairs.
__device__ __forceinline__ uint32_t max_u16x2_pk(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Largest magnitude (bits 6..0) among the 8 FP8 codes of two words.
__device__ __forceinline__ uint32_t max_code_mag8(uint32_t m0, uint32_t m1) {
    const uint32_t lo = max_u16x2_pk(m0 & 0x00FF00FFu, m1 & 0x00FF00FFu);
    const uint32_t hi = max_u16x2_pk(m0 & 0xFF00FF00u, m1 & 0xFF00FF00u);
    return max(max(lo & 0xFFFFu, lo >> 16), max(hi & 0xFFFFu, hi >> 16) >> 8);
}

// How many of the 4 code magnitudes (bits 6..0 of each byte of m) lie below th (0 <= th <= 128).
__device__ __forceinline__ int count_below4(uint32_t m, uint32_t th4) {
    return 4 - __builtin_popcount(((m | 0x80808080u) - th4) & 0x80808080u);
}

// ------------------------------------------------------------------ streaming (non-temporal) memory access
__device__ __forceinline__ uint4 ldnt16(const void* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldnt8(const void* p) {
    u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void stnt16(void* p, uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void stnt8(void* p, uint2 v) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
enum : int { FMT_E4M3 = 0, FMT_E5M2 = 1 };

// ------------------------------------------------------------------ integer helpers on bf16 bit patterns
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Largest |x| bit pattern among the 8 bf16 values of a 16-byte chunk (NaN patterns sort above infinity).
__device__ __forceinline__ uint32_t amax_bits8(uint4 v) {
    uint32_t m = max_u16x2(max_u16x2(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu), max_u16x2(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
    return max(m & 0xFFFFu, m >> 16);
}

// Max across each group of 4 consecutive lanes (DPP quad permutations).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    return v;
}

// E8M0 scale byte for a 32-value block from the bit pattern of its largest magnitude.
//   rceil: smallest e with amax <= 448 * 2^e. For amax = (1 + m/128) 2^(E-127): e = E-127-8 if m <= 0x60
//          (1 + m/128 <= 1.75 = 448/256), else one more. Zero and bf16 subnormals clamp to e = -127 (byte 0).
//   floor: e = floor(log2 amax) - 8 = E - 127 - 8, clamped likewise.
//   Infinity clamps to e = 127 (byte 254); a NaN gives byte 255.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits, int rule) {
    // selects rather than branches: the non-finite case is rare but a branch costs every block its exec-mask juggling
    const int E = (int)(amax_bits >> 7), mant = (int)(amax_bits & 0x7F);
    const int b = max(E - 8 + ((rule == RULE_RCEIL && mant > 0x60) ? 1 : 0), 0);
    const uint32_t nonfinite = amax_bits == 0x7F80u ? 254u : 255u;
    return amax_bits >= 0x7F80u ? nonfinite : (uint32_t)b;
}

// The same rule for an fp32 block maximum (magnitude bits): NaN -> 0xFF, +inf -> 254 (e = 127), otherwise
// E - 8 (+1 under rceil when the mantissa exceeds 0.75, i.e. amax > 448 * 2^(E-135)), clamped at 0.
__device__ __forceinline__ uint32_t mx_scale_byte_f32(uint32_t abs_bits, int rule) {
    if (abs_bits >= 0x7F800000u) return abs_bits == 0x7F800000u ? 254u : 255u;
    int E = (int)(abs_bits >> 23), mant = (int)(abs_bits & 0x7FFFFF);
    int b = E - 8 + ((rule == RULE_RCEIL && mant > 0x600000) ? 1 : 0);
    return b < 0 ? 0u : (uint32_t)b;
}

// 2^-(e) for the block exponent e = byte - 127 as an fp32 multiplier; byte 254 (and NaN's 255, encoded as if
// e = 127) give the subnormal 2^-127. Multiplying by it scales exactly wherever the result can reach E4M3's range.
__device__ __forceinline__ float mx_inv_scale_f32(uint32_t byte) {
    return byte < 254u ? __uint_as_float((254u - byte) << 23) : __uint_as_float(0x00400000u);
}

// fp32 scale operand for v_cvt_scalef32_*: only its exponent field is read, so byte -> exponent bits
// (a mantissa bit is set so the byte-0 pattern is a subnormal rather than zero).
__device__ __forceinline__ float scale_operand(uint32_t byte) {
    return __uint_as_float((__builtin_elementwise_min(byte, 254u) << 23) | 0x00400000u);
}

// ------------------------------------------------------------------ conversions
template <bool HI>
__device__ __forceinline__ uint32_t cvt_mx_pair(uint32_t old, uint32_t bf16_pair, float scale) {
    v2s o = __builtin_bit_cast(v2s, old);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(v2bf, bf16_pair), scale, HI);
    return __builtin_bit_cast(uint32_t, o);
}

// 4 bf16 (two pairs) -> 4 E4M3 codes in one dword, divided by the block scale.
__device__ __forceinline__ uint32_t cvt_mx_quad(uint32_t p0, uint32_t p1, float scale) {
    // the two conversions write bytes 0-1 and 2-3, so the first one's untouched half can start as any value (an
    // unspecified one spares a register copy)
    return cvt_mx_pair<true>(cvt_mx_pair<false>(__builtin_nondeterministic_value(p0), p0, scale), p1, scale);
}

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_f32_pair(uint32_t old, float a, float b) {
    if constexpr (FMT == FMT_E4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
    else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Saturating clamp to +-fmax that keeps NaN (the hardware converts NaN to a NaN code).
__device__ __forceinline__ float clamp_keep_nan(float v, float fmax) {
    float c = __builtin_fminf(__builtin_fmaxf(v, -fmax), fmax);
    return (v != v) ? v : c;
}

// Patch the codes of one dword (4 E4M3 codes of 4 bf16 inputs) where the fast conversion is not exact:
// NaN inputs get 0x7F|sign, inputs at or above thr (bit pattern of 464 * 2^e, or +inf) saturate to 0x7E|sign.
__device__ __forceinline__ uint32_t mx_patch4(uint32_t codes, uint32_t p0, uint32_t p1, uint32_t thr) {
    uint32_t in[4] = {p0 & 0xFFFFu, p0 >> 16, p1 & 0xFFFFu, p1 >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t ax = in[i] & 0x7FFFu, sg = (in[i] >> 8) & 0x80u;
        uint32_t fix = ax > 0x7F80u ? (0x7Fu | sg) : (0x7Eu | sg);
        bool need = ax > 0x7F80u || ax >= thr;
        codes = need ? ((codes & ~(0xFFu << (8 * i))) | (fix << (8 * i))) : codes;
    }
    return codes;
}

// Threshold bit pattern (bf16 magnitude) at and above which x / 2^(byte-127) rounds beyond 448.
__device__ __forceinline__ uint32_t mx_sat_threshold(uint32_t byte) {
    uint32_t b = byte > 254u ? 254u : byte;
    uint32_t expf = b + 8u;                     // exponent field of 464 * 2^(b-127) = 1.8125 * 2^(b-119)
    return expf >= 255u ? 0x7F80u : ((expf << 7) | 0x68u);
}

// ------------------------------------------------------------------ exponential for SwiGLU and its backward
// A fixed fp32 sequence: Cody-Waite reduction by k ln2 (k = rint(x log2 e), ln2 split into a 16-bit high part and a
// low part), the degree-6 Taylor polynomial of e^r in Horner form, exact scaling by 2^k. Every operation is rounded
// on its own (callers build without contraction), so any implementation following it computes the same value; its
// error against the true exponential is a few ulp.
__device__ __forceinline__ float exp_fixed(float x) {
    if (x != x) return x;
    if (x > 88.75f) return __uint_as_float(0x7F800000u);
    if (x < -104.0f) return 0.0f;
    const float t = x * 1.44269504f;
    const float k = __builtin_rintf(t);
    const float a = k * 0.693145751953125f;
    float r = x - a;
    const float b = k * 1.42860677e-06f;
    r = r - b;
    float p = 1.0f / 720.0f;
    p = p * r; p = p + 1.0f / 120.0f;
    p = p * r; p = p + 1.0f / 24.0f;
    p = p * r; p = p + 1.0f / 6.0f;
    p = p * r; p = p + 0.5f;
    p = p * r; p = p + 1.0f;
    p = p * r; p = p + 1.0f;
    return __builtin_ldexpf(p, (int)k);
}

// h = silu(g) u with silu(g) = g / (1 + e^-g): one rounding per operation, in this order.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    const float e = exp_fixed(-g);
    const float d = 1.0f + e;
    const float silu = g / d;
    return silu * u;
}

}  // namespace mxq
