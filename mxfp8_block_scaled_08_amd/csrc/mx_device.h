// Device helpers shared by the MXFP8 kernels (gfx950 / CDNA4).
//
// Number format: OCP Microscaling Formats (MX) v1.0, MXFP8 with E4M3 elements
// and E8M0 block scales (the format of "End-to-End MXFP8 Reinforcement
// Learning on Blackwell", Figure 1 and Table 10 row F6).
//
// The block scale is integer bit manipulation on the BF16 maximum.  The
// elements go through CDNA4's scaled down-conversion (v_cvt_scalef32_pk_fp8_bf16),
// which divides two BF16 values by 2^(e-127), e being the exponent field of
// its FP32 scale operand, and rounds to nearest even into OCP E4M3, keeping
// subnormals and the sign of zero.  It does not saturate: a magnitude that
// rounds above 448 comes out as the NaN code 0x7F/0xFF, which saturate_codes
// turns into 0x7E/0xFE.  Together the two are byte-identical to the
// specification's encoding for every finite BF16 and every scale code 0..254.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// E8M0 scale code from the block's largest magnitude pattern (bits & 0x7FFF,
// whose integer order is value order for non-negative IEEE patterns):
// floor(log2(amax)) - 8 + 127 = biased_exponent(amax) - 8, clamped at 0 (an
// all-zero or tiny block gets 0); a block holding NaN/Inf (pattern >= 0x7F80)
// gets 0xFF.
__host__ __device__ __forceinline__ uint32_t scale_code(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F80u)
        return 0xFFu;
    int c = (int)(amax_bits >> 7) - 8;
    return c < 0 ? 0u : (uint32_t)c;
}

// Packed unsigned 16-bit maximum of two words (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

// Magnitude patterns of the two BF16 in a word.
__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }

// The scale operand: an FP32 whose exponent field is the scale code (code 0
// gives +0.0f, which the instruction reads as 2^-127 like any other code).
__device__ __forceinline__ float cvt_scale(uint32_t c) { return __builtin_bit_cast(float, c << 23); }

// Overflowed codes to the largest finite magnitude: every byte whose low seven
// bits are all ones (0x7F, 0xFF) loses bit 0.  In a block with no NaN/Inf input
// those bytes can only come from overflow.  Adding 1 to the low seven bits of
// each byte sets bit 7 exactly for those bytes, without carries between bytes.
__device__ __forceinline__ uint32_t saturate_codes(uint32_t u)
{
    const uint32_t t = (u & 0x7F7F7F7Fu) + 0x01010101u;
    return u ^ ((t >> 7) & 0x01010101u);
}

// Four BF16 (w0 low, w0 high, w1 low, w1 high) -> four E4M3 bytes in that order.
// Both halves of the result are written, so the tied "old" operand can be any
// register; w0, which is dead afterwards, saves a move.
__device__ __forceinline__ uint32_t cvt_x4(uint32_t w0, uint32_t w1, float scale)
{
    i16x2_t r = __builtin_bit_cast(i16x2_t, w0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w1), scale, true);
    return saturate_codes(__builtin_bit_cast(uint32_t, r));
}

// A NaN/Inf block (scale code 0xFF) encodes every element as 0x7F.
__device__ __forceinline__ uint32_t nan_block_select(uint32_t codes, uint32_t c)
{
    return c == 0xFFu ? 0x7F7F7F7Fu : codes;
}

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));

// Streaming accesses: a pass over far more data than L2 and the Infinity
// Cache hold, each input byte read once and each output byte written once,
// with the non-temporal cache policy (the nt bit; STREAM is the same policy
// as the cache-policy operand of buffer accesses), whose lines are evicted
// first.  Measured on the layer pass: the elementwise passes run faster with
// it, and so do the products that follow them, since the passes' outputs are
// written back to HBM while they run instead of being evicted, dirty, from
// the Infinity Cache by the product's own reads.
constexpr int STREAM = 2;

__device__ __forceinline__ uint4 ld_stream(const void *p)
{
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u_t *>(p)));
}

__device__ __forceinline__ void st_stream(void *p, uint4 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(v4u_t, v), reinterpret_cast<v4u_t *>(p));
}

__device__ __forceinline__ void st_stream(void *p, uint2 v)
{
    __builtin_nontemporal_store(__builtin_bit_cast(v2u_t, v), reinterpret_cast<v2u_t *>(p));
}

// Buffer resource for a byte range: uniform base and size in SGPRs, so each
// lane supplies only a 32-bit offset.  Word 3 selects 32-bit data format
// (what untyped buffer accesses on gfx9-family targets expect).  Loads whose
// per-lane offset falls outside [0, bytes) read zero and such stores are
// dropped.  Callers pass values that every lane holds alike; reading them
// from the first lane says so to the compiler, which would otherwise wrap
// each access in a loop over the distinct values it cannot rule out.
// SwiGLU of two packed BF16 pairs (gate g, up u; element 0 in the low half):
// h = g * sigmoid(g) * u in FP32, the sigmoid taken from exp(-|g|) (no
// overflow for any g; the library exp, subnormal results kept) and the
// hardware reciprocal of 1 + exp(-|g|) (in [1, 2]: within 1 ulp), rounded to
// BF16 by the hardware's nearest-even conversion.  One definition for every
// kernel that forms h, so they agree bit for bit.
__device__ __forceinline__ uint32_t swiglu_bf16x2(uint32_t gs, uint32_t us)
{
    typedef float f2_t __attribute__((ext_vector_type(2)));
    float hv[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const float g = __builtin_bit_cast(float, e ? (gs & 0xFFFF0000u) : (gs << 16));
        const float v = __builtin_bit_cast(float, e ? (us & 0xFFFF0000u) : (us << 16));
        const float t = expf(-fabsf(g));
        const float sig = (g >= 0.0f ? 1.0f : t) * __builtin_amdgcn_rcpf(1.0f + t);
        hv[e] = g * sig * v;
    }
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{hv[0], hv[1]}), bf16x2_t));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void *base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    void *ub = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, 0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

}  // namespace mx
