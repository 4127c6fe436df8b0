// Internal launcher declarations: called by the C ABI layer (mx_api.cpp)
// after every argument has been validated.  Each returns the HIP status of
// its launch and never synchronizes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

hipError_t launch_quantize_rowwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *q, int64_t ld_q, void *s, int64_t ld_s,
                                   hipStream_t stream);

// Row-wise with the scales stored in the rearranged layout (tile (rt, kt)
// at s_swz + (rt * s_tiles + kt) * 256); cols % 256 == 0.
hipError_t launch_quantize_rowwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                       void *q, int64_t ld_q, void *s_swz, int64_t s_tiles,
                                       hipStream_t stream);

hipError_t launch_quantize_colwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *qt, int64_t ld_qt, void *st, int64_t ld_st,
                                   hipStream_t stream);

// Column-wise with the scales ([cols][rows/32]) stored in the rearranged
// layout (tile (ct, rt) at st_swz + (ct * st_tiles + rt) * 256);
// rows % 256 == 0, cols % 32 == 0.
hipError_t launch_quantize_colwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                       void *qt, int64_t ld_qt, void *st_swz, int64_t st_tiles,
                                       hipStream_t stream);

// One tensor of a batched row-wise quantization with rearranged scales
// (tile (rt, kt) at s_swz + (rt * s_tiles + kt) * 256); cols % 256 == 0.
struct RowJob {
    const void *x;
    int64_t rows, cols, ld_x;
    void *q;
    int64_t ld_q;
    void *s_swz;
    int64_t s_tiles;
};
constexpr int QR_MAX_JOBS = 8;

// n in 1..QR_MAX_JOBS jobs, one launch; empty jobs are allowed.
hipError_t launch_quantize_rowwise_batch(const RowJob *jobs, int n, hipStream_t stream);

// One tensor of a dual (row-wise + column-wise) quantization.  s_swz /
// st_swz: tile (0, 0) of its rearranged scales; tile (rt, kt) at
// + (rt * s_tiles + kt) * 256 (st_tiles likewise).
struct DualJob {
    const void *x;
    int64_t rows, cols, ld_x;
    void *q;
    int64_t ld_q;
    void *s_swz;
    int64_t s_tiles;
    void *qt;
    int64_t ld_qt;
    void *st_swz;
    int64_t st_tiles;
    // count tensors of this shape, tensor i at x + i * x_stride elements and
    // its outputs at the given byte strides (stacked expert weights)
    int64_t count;
    int64_t x_stride, q_stride, s_stride, qt_stride, st_stride;
};
constexpr int QD_MAX_JOBS = 16;

// n in 1..QD_MAX_JOBS jobs, one launch; empty jobs are allowed.
hipError_t launch_quantize_dual(const DualJob *jobs, int n, hipStream_t stream);

hipError_t launch_scale_swizzle(const void *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                                void *s_swz, hipStream_t stream);

// Bytes of workspace a dense product needs for its split tail on the
// current device (0: no split).  The split applies when the 256 x 256 tiles
// leave a partial last round of compute units, C is BF16 and every tile is
// full width with 16-byte stores (vec16: c 16-byte aligned, ld_c % 8 == 0,
// N % 256 == 0).  Host-only: reads the device's compute-unit count.
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int c_dtype, bool vec16);
// Whether C at c with leading dimension ld_c takes the full-line BF16 stores.
bool gemm_vec16(const void *c, int64_t ld_c, int c_dtype);

// c_dtype: 0 = BF16, 1 = FP32 (the mx_dtype values).  ws: at least
// gemm_workspace_bytes(...) bytes, 16-byte aligned (may be null when that is 0).
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void *a_q, int64_t ld_a,
                       const void *a_s, const void *b_q, int64_t ld_b, const void *b_s,
                       void *c, int64_t ld_c, int c_dtype, void *ws, hipStream_t stream);

hipError_t launch_grouped_gemm(int64_t G, int64_t M_total, int64_t N, int64_t K,
                               const int64_t *offsets, const void *a_q, int64_t ld_a,
                               const void *a_s, const void *b_q, const void *b_s, void *c,
                               int64_t ld_c, int c_dtype, hipStream_t stream);

// MoE dispatch: stable order of the routed (token, expert) assignments by
// expert, then the permuted rows gathered and quantized row-wise, scales in
// the rearranged layout.  G <= MOE_MAX_EXPERTS, hidden % 256 == 0.
// ws: moe_dispatch_workspace_bytes(...) bytes, 4-byte aligned (the
// per-chunk expert counts; every byte is rewritten before it is read).
constexpr int MOE_MAX_EXPERTS = 1024;
constexpr int MOE_CHUNK = 256;  // routing assignments per counting workgroup
inline int64_t moe_dispatch_workspace_bytes(int64_t tokens, int64_t topk, int64_t experts)
{
    return (tokens * topk + MOE_CHUNK - 1) / MOE_CHUNK * experts * 4;
}
hipError_t launch_moe_dispatch(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                               const int32_t *topk_ids, int64_t topk, int64_t experts,
                               int64_t *offsets, int32_t *src_token, int32_t *slot, void *q,
                               int64_t ld_q, void *s_swz, void *ws, hipStream_t stream);
// The dispatch's ordering as launch_moe_dispatch, then the permuted rows
// (row p = token src_token[p] of x) quantized row-wise into q / s_swz and per
// expert column-wise into qt / st_swz / pad (launch_quantize_colwise_grouped
// over rows_total = tokens * topk with the dispatch's offsets); tokens * ld_x
// * 2 < 2^31.
hipError_t launch_moe_dispatch_dual_grouped(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                            const int32_t *topk_ids, int64_t topk, int64_t experts,
                                            int64_t *offsets, int32_t *src_token, int32_t *slot, void *q,
                                            int64_t ld_q, void *s_swz, int64_t *pad, void *qt, int64_t ld_qt,
                                            int64_t k_cap, void *st_swz, void *ws, hipStream_t stream);

// The current device's copy of the dispatch's static scratch array
// (MOE_NOALLOC_SCRATCH_BYTES), looked up once per device.
constexpr int64_t MOE_NOALLOC_SCRATCH_BYTES = (int64_t)4 << 20;
hipError_t moe_noalloc_scratch(void **ptr);

// MoE combine: out[t] = sum_j weights[t][j] * y[slot[t][j]] (slots < 0 skipped).
hipError_t launch_moe_combine(const void *y, int64_t tokens, int64_t hidden, int64_t ld_y,
                              const int32_t *slot, const float *weights, int64_t topk, void *out,
                              int64_t ld_out, hipStream_t stream);

// Per-expert column-wise quantization into 256-aligned column ranges (the
// MoE weight gradient's operands): the ranges' start offsets into pad, then
// the codes and rearranged scales.  G <= MOE_MAX_EXPERTS, cols % 32 == 0,
// k_cap % 256 == 0 and at least the capacity for rows and G.
// With q non-null, also the row-wise quantization of the same rows (q at
// [rows][ld_q], scales rearranged with cols/256 tiles per 32-row tile row);
// cols % 256 == 0 then.  With swiglu (q non-null), x is a gate/up output
// [rows][ld_x] with ld_x >= 2 cols and the rows quantized are its SwiGLU.
// With src (q non-null), row p is row src[p] of x, whose x_bytes (< 2^31)
// bytes hold the token rows.
hipError_t launch_quantize_colwise_grouped(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                          const int64_t *offsets, int64_t G, int64_t *pad,
                                          void *qt, int64_t ld_qt, int64_t k_cap, void *st_swz,
                                          hipStream_t stream, void *q = nullptr, int64_t ld_q = 0,
                                          void *s_swz = nullptr, bool swiglu = false,
                                          const int32_t *src = nullptr, int64_t x_bytes = 0);

// Per-expert product along K: C_g = A[:, r_g] . B[:, r_g]^T for the column
// ranges r_g = [k_offsets[g], k_offsets[g+1]), C_g at c + g * M * ld_c.
// K % 256 == 0, G <= MOE_MAX_EXPERTS.  ws: WGRAD_WORKSPACE_BYTES, 4-byte
// aligned (the tile counter, cleared by a kernel before the product).
constexpr int64_t WGRAD_WORKSPACE_BYTES = 256;
hipError_t launch_grouped_gemm_wgrad(int64_t G, int64_t M, int64_t N, int64_t K,
                                     const int64_t *k_offsets, const void *a_q, int64_t ld_a,
                                     const void *a_s, const void *b_q, int64_t ld_b,
                                     const void *b_s, void *c, int64_t ld_c, int c_dtype,
                                     void *ws, hipStream_t stream);

// SwiGLU of gu's halves ([0, F) gate, [F, 2F) up) fused with the row-wise
// quantization of the BF16 result; h (BF16 [rows][ld_h]) stored when not
// null.  F % 256 == 0.
hipError_t launch_swiglu_quantize(const void *gu, int64_t rows, int64_t F, int64_t ld_gu, void *h,
                                  int64_t ld_h, void *q, int64_t ld_q, void *s_swz, hipStream_t stream);

// Debug check of device offsets off[0..G] (see mx_debug.hip): waits for the
// stream (the one wait in the library, under MX_DEBUG only), then *first_bad = the first entry breaking the stated properties
// (in [0, total], multiple of align, ranges at least min_len long,
// off[0] == 0 if first_zero, off[G] == total if exact_end), or -1.
hipError_t check_offsets(const int64_t *off, int64_t G, int64_t total, int64_t align, int64_t min_len,
                         bool first_zero, bool exact_end, hipStream_t stream, int64_t *first_bad);

}  // namespace mx
