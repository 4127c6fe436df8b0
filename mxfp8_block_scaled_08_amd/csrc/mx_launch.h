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

hipError_t launch_quantize_colwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *qt, int64_t ld_qt, void *st, int64_t ld_st,
                                   hipStream_t stream);

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
};
constexpr int QD_MAX_JOBS = 16;

// n in 1..QD_MAX_JOBS jobs, one launch; empty jobs are allowed.
hipError_t launch_quantize_dual(const DualJob *jobs, int n, hipStream_t stream);

hipError_t launch_scale_swizzle(const void *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                                void *s_swz, hipStream_t stream);

// c_dtype: 0 = BF16, 1 = FP32 (the mx_dtype values).
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void *a_q, int64_t ld_a,
                       const void *a_s, const void *b_q, int64_t ld_b, const void *b_s,
                       void *c, int64_t ld_c, int c_dtype, hipStream_t stream);

hipError_t launch_grouped_gemm(int64_t G, int64_t M_total, int64_t N, int64_t K,
                               const int64_t *offsets, const void *a_q, int64_t ld_a,
                               const void *a_s, const void *b_q, const void *b_s, void *c,
                               int64_t ld_c, int c_dtype, hipStream_t stream);

}  // namespace mx
