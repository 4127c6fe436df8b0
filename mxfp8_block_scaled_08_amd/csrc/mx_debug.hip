// Optional checks of the device-resident offsets the grouped entry points
// read (MX_DEBUG set in the environment).  The offsets never reach the host
// on the normal path: the kernels clamp them into range, so offsets that
// break their stated properties give unspecified but in-bounds results.
// Under MX_DEBUG an entry point first runs this check, waits for it and
// returns MX_ERR_INVALID_ARG naming the first bad entry instead of
// launching (a loud error for a silent one; the MXFP8 RL paper, "End-to-End
// MXFP8 Reinforcement Learning on Blackwell", found most of its weight-sync
// failures silent, Table 10).  The wait makes it unusable inside HIP graph
// capture, so it is off by default.
#include "mx_device.h"
#include "mx_launch.h"

#include <atomic>
#include <climits>

namespace mx {

// Result words of the checks: a device array (no allocation), one word per
// check in flight, taken round robin; each device holds its own copy, found
// with hipGetSymbolAddress while that device is current.
constexpr int DEBUG_SLOTS = 64;
static __device__ __align__(256) int debug_flags[DEBUG_SLOTS];

// One workgroup: entry g of off[0..G] fails when it is outside [0, total],
// not a multiple of align, (first_zero) g == 0 and nonzero, (exact_end)
// g == G and not total, or (g < G) the range [off[g], off[g+1]) is shorter
// than min_len (negative included).  *flag = the first failing g + 1, or 0.
__global__ __launch_bounds__(256) void check_offsets_kernel(const int64_t *__restrict__ off, int64_t G,
                                                            int64_t total, int64_t align, int64_t min_len,
                                                            int first_zero, int exact_end, int *flag)
{
    __shared__ int s_bad;
    if (threadIdx.x == 0)
        s_bad = INT_MAX;
    __syncthreads();
    int bad = INT_MAX;
    for (int64_t g = threadIdx.x; g <= G && g < INT_MAX; g += 256) {
        const int64_t v = off[g];
        bool ok = v >= 0 && v <= total && v % align == 0;
        if (g == 0 && first_zero)
            ok = ok && v == 0;
        if (g == G && exact_end)
            ok = ok && v == total;
        if (g < G)
            ok = ok && off[g + 1] - v >= min_len;
        if (!ok)
            bad = min(bad, (int)g);
    }
    atomicMin(&s_bad, bad);
    __syncthreads();
    if (threadIdx.x == 0)
        *flag = s_bad == INT_MAX ? 0 : s_bad + 1;
}

hipError_t check_offsets(const int64_t *off, int64_t G, int64_t total, int64_t align, int64_t min_len,
                         bool first_zero, bool exact_end, hipStream_t stream, int64_t *first_bad)
{
    *first_bad = -1;
    void *base = nullptr;
    hipError_t e0 = hipGetSymbolAddress(&base, HIP_SYMBOL(debug_flags));
    if (e0 != hipSuccess)
        return e0;
    static std::atomic<unsigned> next{0};
    int *flag = (int *)base + next.fetch_add(1) % DEBUG_SLOTS;
    hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(256), 0, stream, off, G, total, align, min_len,
                       (int)first_zero, (int)exact_end, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    int h = 0;
    e = hipMemcpyAsync(&h, flag, sizeof h, hipMemcpyDeviceToHost, stream);
    if (e != hipSuccess)
        return e;
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return e;
    *first_bad = h - 1;
    return hipSuccess;
}

}  // namespace mx
