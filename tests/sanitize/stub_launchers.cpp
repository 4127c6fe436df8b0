// Stand-ins for the HIP launchers, for building the C-ABI layer (mx_api.cpp)
// on the host alone with AddressSanitizer and UndefinedBehaviorSanitizer:
// every launcher records that it was reached and returns hipSuccess without
// touching any pointer, so calls with fake device addresses run the whole
// validation path.  The split-tail plan is the library's own (mx_plan.h) on
// 256 compute units.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../mxfp8_block_scaled_08_amd/csrc/mx_launch.h"
#include "../../mxfp8_block_scaled_08_amd/csrc/mx_plan.h"

extern "C" {
int64_t stub_launches = 0;
int64_t stub_last_ws = 0;  // workspace pointer handed to the last launch that takes one
}

namespace mx {

static hipError_t hit(const void *ws = nullptr)
{
    stub_launches++;
    stub_last_ws = (int64_t)(uintptr_t)ws;
    return hipSuccess;
}

hipError_t launch_quantize_rowwise(const void *, int64_t, int64_t, int64_t, void *, int64_t, void *, int64_t,
                                   hipStream_t) { return hit(); }
hipError_t launch_quantize_rowwise_swz(const void *, int64_t, int64_t, int64_t, void *, int64_t, void *, int64_t,
                                       hipStream_t) { return hit(); }
hipError_t launch_quantize_colwise(const void *, int64_t, int64_t, int64_t, void *, int64_t, void *, int64_t,
                                   hipStream_t) { return hit(); }
hipError_t launch_quantize_colwise_swz(const void *, int64_t, int64_t, int64_t, void *, int64_t, void *, int64_t,
                                       hipStream_t) { return hit(); }
hipError_t launch_quantize_rowwise_batch(const RowJob *, int, hipStream_t) { return hit(); }
hipError_t launch_quantize_dual(const DualJob *, int, hipStream_t) { return hit(); }
hipError_t launch_scale_swizzle(const void *, int64_t, int64_t, int64_t, void *, hipStream_t) { return hit(); }
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int c_dtype, bool vec16)
{
    return split_plan(M, N, K, c_dtype, vec16, 256).bytes();
}
bool gemm_vec16(const void *c, int64_t ld_c, int c_dtype)
{
    return c_dtype == 0 && (uintptr_t)c % 16 == 0 && ld_c % 8 == 0;
}
hipError_t launch_gemm(int64_t, int64_t, int64_t, const void *, int64_t, const void *, const void *, int64_t,
                       const void *, void *, int64_t, int, void *ws, hipStream_t) { return hit(ws); }
hipError_t launch_grouped_gemm(int64_t, int64_t, int64_t, int64_t, const int64_t *, const void *, int64_t,
                               const void *, const void *, const void *, void *, int64_t, int,
                               hipStream_t) { return hit(); }
hipError_t launch_moe_dispatch(const void *, int64_t, int64_t, int64_t, const int32_t *, int64_t, int64_t,
                               int64_t *, int32_t *, int32_t *, void *, int64_t, void *, void *ws,
                               hipStream_t) { return hit(ws); }
hipError_t launch_moe_dispatch_dual_grouped(const void *, int64_t, int64_t, int64_t, const int32_t *, int64_t,
                                            int64_t, int64_t *, int32_t *, int32_t *, void *, int64_t, void *,
                                            int64_t *, void *, int64_t, int64_t, void *, void *ws,
                                            hipStream_t) { return hit(ws); }
hipError_t moe_noalloc_scratch(void **ptr)
{
    *ptr = (void *)(uintptr_t)0x5000000000ull;  // a fake device address, never dereferenced
    return hipSuccess;
}
hipError_t launch_moe_combine(const void *, int64_t, int64_t, int64_t, const int32_t *, const float *, int64_t,
                              void *, int64_t, hipStream_t) { return hit(); }
hipError_t launch_quantize_colwise_grouped(const void *, int64_t, int64_t, int64_t, const int64_t *, int64_t,
                                          int64_t *, void *, int64_t, int64_t, void *, hipStream_t, void *,
                                          int64_t, void *, bool, const int32_t *, int64_t) { return hit(); }
hipError_t launch_grouped_gemm_wgrad(int64_t, int64_t, int64_t, int64_t, const int64_t *, const void *, int64_t,
                                     const void *, const void *, int64_t, const void *, void *, int64_t, int,
                                     void *ws, hipStream_t) { return hit(ws); }
hipError_t launch_swiglu_quantize(const void *, int64_t, int64_t, int64_t, void *, int64_t, void *, int64_t,
                                  void *, hipStream_t) { return hit(); }
hipError_t check_offsets(const int64_t *, int64_t, int64_t, int64_t, int64_t, bool, bool, hipStream_t,
                         int64_t *first_bad)
{
    *first_bad = -1;
    return hipSuccess;
}

}  // namespace mx
