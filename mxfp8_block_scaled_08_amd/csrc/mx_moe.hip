// MoE token dispatch and combine around the grouped GEMM (gfx950).
//
// The MoE layers of "End-to-End MXFP8 Reinforcement Learning on Blackwell"
// (Table 2: Qwen3-30B-A3B, 128 experts, 8 routed per token) run the expert
// GEMMs on rows sorted by expert.  Dispatch builds that order and the GEMM's
// A operand in one pass over the activations; combine undoes it.
//
// Order.  Assignment a = t * topk + j (token t, its j-th expert) is placed at
// row offsets[e] + (number of earlier assignments to the same expert e): a
// stable sort by expert, so the result depends only on the routing.  Three
// small kernels compute it without atomics on the result: per chunk of 256
// assignments an LDS histogram of experts (LDS atomics only count, so the
// counts are exact); per expert a scan over the chunks plus the experts'
// exclusive scan (the offsets); per assignment its rank among the earlier
// assignments of its chunk with the same expert, from the chunk's experts in
// LDS.  The scan runs as one workgroup per expert over its chunks, then one
// over the experts' totals.  Expert ids outside [0, experts) are not routed (slot -1).
//
// Quantize + scatter.  Row i of the permuted operand is the quantized row of
// token src_token[i].  All routed copies of a token are the same bytes, so the
// kernel goes token by token: it reads each token row once (non-temporal) and
// quantizes it once, with the row-wise kernel's lane layout (8 BF16 per lane,
// four lanes per 32-element block, DPP quad maximum, CDNA4's scaled
// conversion).  It then stores the codes and each block's scale byte, at its
// place in the GEMM's rearranged layout, to every row the token's
// assignments were placed at.  The operand's reads fall from one token row
// per routed copy (8 per token) to one per token.
#include "mx_device.h"
#include "mx_launch.h"

#include <mutex>

#include <algorithm>

namespace mx {

// MOE_CHUNK (mx_launch.h): routing assignments per counting workgroup

__global__ __launch_bounds__(MOE_CHUNK) void moe_count_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                               int experts, int32_t *__restrict__ counts)
{
    __shared__ int hist[MOE_MAX_EXPERTS];
    for (int g = threadIdx.x; g < experts; g += MOE_CHUNK)
        hist[g] = 0;
    __syncthreads();
    const int64_t a = (int64_t)blockIdx.x * MOE_CHUNK + threadIdx.x;
    if (a < n) {
        const int e = ids[a];
        if (e >= 0 && e < experts)
            atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int g = threadIdx.x; g < experts; g += MOE_CHUNK)
        counts[(int64_t)blockIdx.x * experts + g] = hist[g];
}

// Per expert g (one workgroup each): exclusive scan of its column of chunk
// counts, in place, so counts[c][g] becomes the number of g's assignments in
// chunks before c; the column's total goes to offsets[g].  Thread t takes a
// contiguous run of chunks; the runs' sums are scanned across the workgroup.
constexpr int MOE_SCAN_THREADS = 256;

__global__ __launch_bounds__(MOE_SCAN_THREADS) void moe_scan_chunks_kernel(int32_t *__restrict__ counts,
                                                                         int64_t chunks, int experts,
                                                                         int64_t *__restrict__ totals)
{
    __shared__ int64_t wsum[MOE_SCAN_THREADS / 64];
    const int g = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t per = (chunks + MOE_SCAN_THREADS - 1) / MOE_SCAN_THREADS;
    const int64_t c0 = min((int64_t)t * per, chunks), c1 = min(c0 + per, chunks);
    int64_t sum = 0;
    for (int64_t c = c0; c < c1; c++)
        sum += counts[c * experts + g];
    int64_t incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    int64_t run = incl - sum;
    for (int w = 0; w < wave; w++)
        run += wsum[w];
    for (int64_t c = c0; c < c1; c++) {
        const int32_t v = counts[c * experts + g];
        counts[c * experts + g] = (int32_t)run;
        run += v;
    }
    if (t == MOE_SCAN_THREADS - 1)
        totals[g] = run;
}

// One workgroup: the experts' totals (in offsets[0..experts-1]) scanned into
// the offsets, offsets[experts] = the routed count.
__global__ __launch_bounds__(MOE_MAX_EXPERTS) void moe_scan_experts_kernel(int experts,
                                                                          int64_t *__restrict__ offsets)
{
    __shared__ int64_t wsum[MOE_MAX_EXPERTS / 64];
    const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
    const int64_t v = g < experts ? offsets[g] : 0;
    int64_t incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    if (lane == 63)
        wsum[wave] = incl;
    __syncthreads();
    int64_t base = 0;
    for (int w = 0; w < wave; w++)
        base += wsum[w];
    if (g < experts)
        offsets[g] = base + incl - v;
    if (g == experts - 1)
        offsets[experts] = base + incl;
}

__global__ __launch_bounds__(MOE_CHUNK) void moe_place_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                               int topk, int experts,
                                                               const int32_t *__restrict__ base,
                                                               const int64_t *__restrict__ offsets,
                                                               int32_t *__restrict__ src_token,
                                                               int32_t *__restrict__ slot)
{
    __shared__ int ex[MOE_CHUNK];
    const int i = threadIdx.x;
    const int64_t a = (int64_t)blockIdx.x * MOE_CHUNK + i;
    int e = -1;
    if (a < n) {
        e = ids[a];
        if (e < 0 || e >= experts)
            e = -1;
    }
    ex[i] = e;
    __syncthreads();
    if (a >= n)
        return;
    if (e < 0) {
        slot[a] = -1;
        return;
    }
    int rank = 0;
    for (int j = 0; j < i; j++)
        rank += ex[j] == e;
    const int32_t p = (int32_t)offsets[e] + base[(int64_t)blockIdx.x * experts + e] + rank;
    slot[a] = p;
    src_token[p] = (int32_t)(a / topk);
}

constexpr int MOE_Q_THREADS = 256;

// Unit u = 8 consecutive elements of token row u / upr.  The row is read
// and quantized once; its codes and scale bytes go to every row of the
// permuted operand the token is routed to (slot[t * topk + j], j < topk;
// -1 for an assignment that is not routed).  Those rows are exactly
// [0, offsets[experts]); the rest are not written.
__global__ __launch_bounds__(MOE_Q_THREADS) void moe_scatter_quantize_kernel(
    const uint16_t *__restrict__ x, int64_t ld_x, const int32_t *__restrict__ slot, int topk,
    uint8_t *__restrict__ q, int64_t ld_q, uint8_t *__restrict__ s_swz, int64_t units, uint32_t upr,
    int64_t kt)
{
    for (int64_t u = (int64_t)blockIdx.x * MOE_Q_THREADS + threadIdx.x; u - (threadIdx.x & 3) < units;
         u += (int64_t)gridDim.x * MOE_Q_THREADS) {
        // upr is a multiple of 32, so a quad shares its row
        const int64_t t = u / upr;
        const int64_t cu = u - t * upr;
        const bool live = u < units;
        const uint4 w = live ? ld_stream(x + t * ld_x + cu * 8) : make_uint4(0, 0, 0, 0);
        uint32_t m = pk_max_u16(pk_max_u16(mag2(w.x), mag2(w.y)), pk_max_u16(mag2(w.z), mag2(w.w)));
        m = max(m & 0xFFFFu, m >> 16);
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
        if (!live)
            continue;
        const uint32_t c = scale_code(m);
        const float sc = cvt_scale(c);
        uint2 out;
        out.x = nan_block_select(cvt_x4(w.x, w.y, sc), c);
        out.y = nan_block_select(cvt_x4(w.z, w.w, sc), c);
        const int64_t b = cu >> 2;  // 32-element block of the row
        const int64_t s_in = ((b >> 3) * 256) + 32 * (b & 1) * 4 + ((b & 7) >> 1);
        for (int j = 0; j < topk; j++) {
            const int64_t row = slot[t * topk + j];
            if (row < 0)
                continue;
            st_stream(q + row * ld_q + cu * 8, out);
            if ((threadIdx.x & 3) == 0)
                s_swz[(row >> 5) * kt * 256 + s_in + (row & 31) * 4] = (uint8_t)c;
        }
    }
}

// Scratch of mx_moe_dispatch_noalloc: the chunk counts of the stable sort in
// a device array instead of a caller's workspace, for callers that cannot
// allocate.  Each device holds its own copy for the life of the process; in
// host code `scratch` names a host-side stand-in, so the device address is
// looked up (hipGetSymbolAddress) once per device, with that device
// current, and only that address is handed to kernels.
static __device__ __align__(256) int32_t scratch[MOE_NOALLOC_SCRATCH_BYTES / 4];

hipError_t moe_noalloc_scratch(void **ptr)
{
    constexpr int MAX_DEVICES = 64;
    static std::mutex mu;
    static void *per_device[MAX_DEVICES];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (per_device[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

// The dispatch's ordering: offsets, src_token and slot (four small kernels,
// the chunk counts in ws).
static void launch_dispatch_order(const int32_t *topk_ids, int64_t tokens, int64_t topk, int64_t experts,
                                  int64_t *offsets, int32_t *src_token, int32_t *slot, void *ws,
                                  hipStream_t stream)
{
    const int64_t n = tokens * topk;
    const int64_t chunks = (n + MOE_CHUNK - 1) / MOE_CHUNK;
    int32_t *counts = (int32_t *)ws;  // [chunks][experts], every entry written by moe_count_kernel
    hipLaunchKernelGGL(moe_count_kernel, dim3((unsigned)chunks), dim3(MOE_CHUNK), 0, stream, topk_ids, n,
                       (int)experts, counts);
    hipLaunchKernelGGL(moe_scan_chunks_kernel, dim3((unsigned)experts), dim3(MOE_SCAN_THREADS), 0, stream,
                       counts, chunks, (int)experts, offsets);
    hipLaunchKernelGGL(moe_scan_experts_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, stream, (int)experts,
                       offsets);
    hipLaunchKernelGGL(moe_place_kernel, dim3((unsigned)chunks), dim3(MOE_CHUNK), 0, stream, topk_ids, n,
                       (int)topk, (int)experts, counts, (const int64_t *)offsets, src_token, slot);
}

hipError_t launch_moe_dispatch(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                               const int32_t *topk_ids, int64_t topk, int64_t experts,
                               int64_t *offsets, int32_t *src_token, int32_t *slot, void *q,
                               int64_t ld_q, void *s_swz, void *ws, hipStream_t stream)
{
    launch_dispatch_order(topk_ids, tokens, topk, experts, offsets, src_token, slot, ws, stream);
    const uint32_t upr = (uint32_t)(hidden / 8);
    const int64_t units = tokens * upr;
    const int64_t per_pass = (int64_t)MOE_Q_THREADS;
    const int64_t blocks = std::min<int64_t>((units + per_pass - 1) / per_pass, 65536);
    hipLaunchKernelGGL(moe_scatter_quantize_kernel, dim3((unsigned)blocks), dim3(MOE_Q_THREADS), 0, stream,
                       (const uint16_t *)x, ld_x, (const int32_t *)slot, (int)topk, (uint8_t *)q, ld_q,
                       (uint8_t *)s_swz, units, upr, (hidden / 32 + 7) / 8);
    return hipGetLastError();
}

hipError_t launch_moe_dispatch_dual_grouped(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                            const int32_t *topk_ids, int64_t topk, int64_t experts,
                                            int64_t *offsets, int32_t *src_token, int32_t *slot, void *q,
                                            int64_t ld_q, void *s_swz, int64_t *pad, void *qt, int64_t ld_qt,
                                            int64_t k_cap, void *st_swz, void *ws, hipStream_t stream)
{
    launch_dispatch_order(topk_ids, tokens, topk, experts, offsets, src_token, slot, ws, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    return launch_quantize_colwise_grouped(x, tokens * topk, hidden, ld_x, offsets, experts, pad, qt, ld_qt,
                                           k_cap, st_swz, stream, q, ld_q, s_swz, false, src_token,
                                           tokens * ld_x * 2);
}

// Combine: thread -> 8 consecutive columns of one token; the token's slots in
// order j = 0..topk-1, FP32 sums of weight * value, BF16 (nearest even) out.
// Slots outside [0, tokens * topk) contribute nothing.  TOPK > 0 (the top-8
// routing): the token's slots, weights and rows are all loaded before the
// sums, so its TOPK row loads are in flight together; the sums are the same
// fused multiply-adds in the same order as the general path's.
__device__ __forceinline__ void combine_acc(float (&acc)[8], float w, uint4 v)
{
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        acc[2 * k] = fmaf(w, __builtin_bit_cast(float, wd[k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(w, __builtin_bit_cast(float, wd[k] & 0xFFFF0000u), acc[2 * k + 1]);
    }
}

template <int TOPK>
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t *__restrict__ y, int64_t ld_y,
                                                          const int32_t *__restrict__ slot,
                                                          const float *__restrict__ weights, int topk,
                                                          uint16_t *__restrict__ out, int64_t ld_out,
                                                          int64_t units, uint32_t upr, int64_t rows_y)
{
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
        const int64_t t = u / upr;
        const int64_t cu = u - t * upr;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (TOPK > 0) {
            constexpr int K = TOPK > 0 ? TOPK : 1;
            int32_t p[K];
            float w[K];
            uint4 v[K];
#pragma unroll
            for (int j = 0; j < K; j++) {
                p[j] = slot[t * K + j];
                w[j] = weights[t * K + j];
            }
#pragma unroll
            for (int j = 0; j < K; j++)
                v[j] = (p[j] >= 0 && p[j] < rows_y)
                           ? ld_stream(y + (int64_t)p[j] * ld_y + cu * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int j = 0; j < K; j++)
                if (p[j] >= 0 && p[j] < rows_y)
                    combine_acc(acc, w[j], v[j]);
        } else {
            for (int j = 0; j < topk; j++) {
                const int32_t p = slot[t * topk + j];
                if (p < 0 || p >= rows_y)  // unrouted, or not a row of y
                    continue;
                combine_acc(acc, weights[t * topk + j],
                            ld_stream(y + (int64_t)p * ld_y + cu * 8));
            }
        }
        typedef float f2_t __attribute__((ext_vector_type(2)));
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; k++)
            o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{acc[2 * k], acc[2 * k + 1]}), bf16x2_t));
        st_stream(out + t * ld_out + cu * 8, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

hipError_t launch_moe_combine(const void *y, int64_t tokens, int64_t hidden, int64_t ld_y,
                              const int32_t *slot, const float *weights, int64_t topk, void *out,
                              int64_t ld_out, hipStream_t stream)
{
    const uint32_t upr = (uint32_t)(hidden / 8);
    const int64_t units = tokens * upr;
    const int64_t blocks = std::min<int64_t>((units + 255) / 256, 65536);
    if (topk == 8)
        hipLaunchKernelGGL(moe_combine_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t *)y, ld_y, slot, weights, (int)topk, (uint16_t *)out, ld_out, units,
                           upr, tokens * topk);
    else
        hipLaunchKernelGGL(moe_combine_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t *)y, ld_y, slot, weights, (int)topk, (uint16_t *)out, ld_out, units,
                           upr, tokens * topk);
    return hipGetLastError();
}

// SwiGLU between the expert projections, fused with the row-wise
// quantization of its output (the down projection's A operand).  Unit u = 8
// consecutive outputs of row u / upr: one 16-byte load of the gate half and
// one of the up half, h = g * sigmoid(g) * u in FP32 with the sigmoid taken
// from exp(-|g|) (no overflow for any g), rounded to BF16 by the hardware's
// nearest-even conversion; then the row-wise quantizer's quad layout (four
// lanes per 32-element block, DPP quad maximum, scaled conversion) and the
// scale byte stored at its rearranged position.  h itself is stored too when
// asked for.
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(
    const uint16_t *__restrict__ gu, int64_t ld_gu, int64_t F, uint16_t *__restrict__ h, int64_t ld_h,
    uint8_t *__restrict__ q, int64_t ld_q, uint8_t *__restrict__ s_swz, int64_t units, uint32_t upr,
    int64_t kt)
{
    for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u - (threadIdx.x & 3) < units;
         u += (int64_t)gridDim.x * 256) {
        // upr is a multiple of 4, so a quad shares its row
        const int64_t row = u / upr;
        const int64_t cu = u - row * upr;
        const bool live = u < units;
        uint4 gw = make_uint4(0, 0, 0, 0), uw = make_uint4(0, 0, 0, 0);
        if (live) {
            gw = ld_stream(gu + row * ld_gu + cu * 8);
            uw = ld_stream(gu + row * ld_gu + F + cu * 8);
        }
        const uint32_t hw[4] = {swiglu_bf16x2(gw.x, uw.x), swiglu_bf16x2(gw.y, uw.y), swiglu_bf16x2(gw.z, uw.z),
                                swiglu_bf16x2(gw.w, uw.w)};
        if (live && h != nullptr)
            st_stream(h + row * ld_h + cu * 8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        uint32_t m = pk_max_u16(pk_max_u16(mag2(hw[0]), mag2(hw[1])), pk_max_u16(mag2(hw[2]), mag2(hw[3])));
        m = max(m & 0xFFFFu, m >> 16);
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
        m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
        if (!live)
            continue;
        const uint32_t c = scale_code(m);
        const float sc = cvt_scale(c);
        uint2 out;
        out.x = nan_block_select(cvt_x4(hw[0], hw[1], sc), c);
        out.y = nan_block_select(cvt_x4(hw[2], hw[3], sc), c);
        st_stream(q + row * ld_q + cu * 8, out);
        if ((threadIdx.x & 3) == 0) {
            const int64_t b = cu >> 2;  // 32-element block of the row
            s_swz[((row >> 5) * kt + (b >> 3)) * 256 + (32 * (b & 1) + (row & 31)) * 4 + ((b & 7) >> 1)] =
                (uint8_t)c;
        }
    }
}

hipError_t launch_swiglu_quantize(const void *gu, int64_t rows, int64_t F, int64_t ld_gu, void *h,
                                  int64_t ld_h, void *q, int64_t ld_q, void *s_swz, hipStream_t stream)
{
    const uint32_t upr = (uint32_t)(F / 8);
    const int64_t units = rows * upr;
    const int64_t blocks = std::min<int64_t>((units + 255) / 256, 65536);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(swiglu_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       (const uint16_t *)gu, ld_gu, F, (uint16_t *)h, ld_h, (uint8_t *)q, ld_q,
                       (uint8_t *)s_swz, units, upr, (F / 32 + 7) / 8);
    return hipGetLastError();
}

}  // namespace mx
