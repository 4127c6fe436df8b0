// Device helpers shared by the MXFP8 kernels (gfx950 / CDNA4).
//
// Number format: OCP Microscaling Formats (MX) v1.0, MXFP8 with E4M3 elements
// and E8M0 block scales (the format of "End-to-End MXFP8 Reinforcement
// Learning on Blackwell", Figure 1 and Table 10 row F6).  All conversions are
// integer bit manipulation on the BF16 input, so no rounding mode, denormal
// mode or hardware converter can change a byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// Largest |value| of a block as a BF16 magnitude pattern.  For non-negative
// IEEE patterns integer order equals value order, so the block maximum is an
// integer max of (bits & 0x7FFF); NaN and Inf give patterns >= 0x7F80.
__host__ __device__ __forceinline__ uint32_t bf16_mag(uint32_t bits) { return bits & 0x7FFFu; }

// E8M0 scale code from the block's largest magnitude pattern:
// floor(log2(amax)) - 8 + 127 = biased_exponent(amax) - 8, clamped at 0 (an
// all-zero or tiny block gets 0); a block holding NaN/Inf gets 0xFF.
__host__ __device__ __forceinline__ uint32_t scale_code(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F80u)
        return 0xFFu;
    int c = (int)(amax_bits >> 7) - 8;
    return c < 0 ? 0u : (uint32_t)c;
}

// E4M3 code of bf16(bits) / 2^(c-127) for a finite BF16 and c in 0..254.
// Round to nearest even, clamp to 448, keep subnormals and the sign of zero.
//   value = sig * 2^(E - 134), sig = 8-bit significand, E = max(exp, 1)
//   t     = value / 2^(c-127) = sig * 2^(E - c - 7)
//   en    = floor(log2 t) = E - c - 7 + msb(sig)
//   quantum of t in E4M3: 2^(max(en, -6) - 3); n = RNE(t / quantum)
//   code  = (max(en, -6) + 6) * 8 + n  (n runs 8..16 in a normal binade and
//           0..8 in the subnormal one; 16 and 8 carry into the next binade)
__host__ __device__ __forceinline__ uint32_t e4m3_code(uint32_t bits, int c)
{
    uint32_t sign = (bits >> 8) & 0x80u;
    uint32_t a = bits & 0x7FFFu;
    int e = (int)(a >> 7);
    int sig = (int)(a & 0x7Fu) | (e ? 0x80 : 0);
    if (sig == 0)
        return sign;
    int E = e ? e : 1;
    int msb = 31 - __builtin_clz((uint32_t)sig);
    int en = E - c - 7 + msb;
    int ee = en < -6 ? -6 : en;
    int sh = ee - E + c + 4;  // right shift taking sig to units of the quantum
    int n;
    if (sh <= 0) {
        n = sig << (-sh);  // exact (only bf16 subnormals with few bits)
    } else {
        if (sh > 31)
            sh = 31;
        uint32_t us = (uint32_t)sig;
        uint32_t q = us >> sh;
        uint32_t rem = us & ((1u << sh) - 1u);
        uint32_t half = 1u << (sh - 1);
        q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
        n = (int)q;
    }
    int code = (ee + 6) * 8 + n;
    if (code > 0x7E)
        code = 0x7E;
    return sign | (uint32_t)code;
}

// The same code, branch-free, for the hot loops (about 12 VALU operations
// instead of the shifts and data-dependent branches above):
//   t = bf16 * 2^(127 - c) is exact in FP32 (|t| < 512; results below the FP32
//   normal range round to zero in E4M3 anyway, and keep their sign);
//   for |t| >= 2^-6 the E4M3 code is the FP32 exponent/top-3-mantissa field
//   after rounding the mantissa to 3 bits (RNE on the bit pattern; a carry
//   moves into the exponent, as it must), minus the bias difference 120 << 3;
//   for |t| < 2^-6 the code is the number of 2^-9 quanta, obtained by the FP32
//   addition |t| + 2^14 (whose ulp is 2^-9, so the hardware's round-to-
//   nearest-even does the rounding);
//   min(code, 0x7E) saturates; the sign bit comes from the input.
// c must not be 0xFF (NaN blocks are handled by the caller).
__host__ __device__ __forceinline__ uint32_t e4m3_code_fast(uint32_t bits, int c)
{
    const float v = __builtin_bit_cast(float, (bits & 0x7FFFu) << 16);  // |value|
    const float a = ldexpf(v, 127 - c);
    const uint32_t u = __builtin_bit_cast(uint32_t, a);
    const uint32_t rn = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
    const uint32_t cn = rn - (120u << 3);
    const uint32_t cs = __builtin_bit_cast(uint32_t, a + 16384.0f) - 0x46800000u;  // 16384.0f = 0x46800000
    uint32_t code = (a < 0.015625f) ? cs : cn;
    code = code < 0x7Eu ? code : 0x7Eu;
    return code | ((bits >> 8) & 0x80u);
}

// Encode two BF16 packed in a 32-bit word (low half first) into two bytes.
__host__ __device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, int c)
{
    return e4m3_code_fast(w & 0xFFFFu, c) | (e4m3_code_fast(w >> 16, c) << 8);
}

// Encode a uint4 holding 8 BF16 into 8 E4M3 bytes (a NaN/Inf block gives 0x7F).
__host__ __device__ __forceinline__ uint2 e4m3_x8(uint4 v, int c, bool nan_block)
{
    uint2 r;
    if (nan_block) {
        r.x = r.y = 0x7F7F7F7Fu;
        return r;
    }
    r.x = e4m3_pair(v.x, c) | (e4m3_pair(v.y, c) << 16);
    r.y = e4m3_pair(v.z, c) | (e4m3_pair(v.w, c) << 16);
    return r;
}

__host__ __device__ __forceinline__ uint32_t max_mag_x8(uint4 v)
{
    uint32_t m = max(bf16_mag(v.x), bf16_mag(v.x >> 16));
    m = max(m, max(bf16_mag(v.y), bf16_mag(v.y >> 16)));
    m = max(m, max(bf16_mag(v.z), bf16_mag(v.z >> 16)));
    m = max(m, max(bf16_mag(v.w), bf16_mag(v.w >> 16)));
    return m;
}

}  // namespace mx
