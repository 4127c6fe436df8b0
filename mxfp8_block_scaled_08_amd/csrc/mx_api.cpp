// C ABI of libmxfp8.so (declared in include/mxfp8.h): argument validation,
// status reporting, and dispatch to the HIP launchers.
//
// Every entry point validates all of its arguments before it touches HIP, so
// an invalid call writes nothing and returns a status naming the problem
// (the paper "End-to-End MXFP8 Reinforcement Learning on Blackwell" found
// five of its seven weight-sync failures silent, Table 10; errors here are
// loud).  Nothing here or in the launchers allocates device or host memory,
// synchronizes or reads device memory; scratch memory (the split tail's
// partial tiles, the dispatch's chunk counts, the weight gradient's tile
// counter) is a workspace the caller passes, its size given by host-only
// queries.  The one exception is the opt-in check of device-resident offsets
// under MX_DEBUG, which waits for its result.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mxfp8.h"
#include "mx_launch.h"

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

mx_status ok()
{
    g_err[0] = '\0';
    return MX_OK;
}

mx_status hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(MX_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + n) and [q, q + m) overlap (n, m in bytes, both > 0)
bool overlap(const void *p, int64_t n, const void *q, int64_t m)
{
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return n > 0 && m > 0 && a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// byte extent of a row-major [rows][ld] buffer whose rows use `used` elements
int64_t extent(int64_t rows, int64_t used, int64_t ld, int64_t elem)
{
    if (rows <= 0 || used <= 0)
        return 0;
    return ((rows - 1) * ld + used) * elem;
}

// The caller's workspace: at least `need` bytes, `align`-aligned, not
// overlapping any of the n buffers given (MX_OK when need is 0).
mx_status check_workspace(const char *fn, const void *ws, int64_t ws_bytes, int64_t need, uintptr_t align,
                          const void *const *bufs, const int64_t *lens, int n)
{
    if (ws_bytes < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative workspace_bytes", fn);
    if (need <= 0)
        return MX_OK;
    if (!ws || ws_bytes < need)
        return fail(MX_ERR_INVALID_ARG, "%s: needs a workspace of %lld bytes, got %lld at %p", fn,
                    (long long)need, (long long)ws_bytes, ws);
    if ((uintptr_t)ws % align != 0)
        return fail(MX_ERR_ALIGN, "%s: workspace must be %d-byte aligned", fn, (int)align);
    for (int i = 0; i < n; i++)
        if (bufs[i] && lens[i] > 0) {
            const uintptr_t a = (uintptr_t)ws, b = (uintptr_t)bufs[i];
            if (a < b + (uintptr_t)lens[i] && b < a + (uintptr_t)need)
                return fail(MX_ERR_OVERLAP, "%s: workspace overlaps buffer %d", fn, i);
        }
    return MX_OK;
}

int64_t swz_bytes(int64_t rows, int64_t kb)
{
    if (rows <= 0 || kb <= 0)
        return 0;
    return ((rows + 31) / 32) * ((kb + 7) / 8) * 256;
}

// MX_DEBUG set to anything but "" or "0": the grouped entry points check
// their device offsets before launching (read at every call, so a process
// can switch it on and off).
bool debug_checks()
{
    const char *e = std::getenv("MX_DEBUG");
    return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

// The MX_DEBUG offsets check of an entry point: MX_OK, or MX_ERR_INVALID_ARG
// naming the first bad entry (MX_ERR_HIP if the check itself fails).
mx_status debug_offsets(const char *fn, const char *what, const int64_t *off, int64_t G, int64_t total,
                        int64_t align, int64_t min_len, bool first_zero, bool exact_end, void *stream)
{
    int64_t bad = -1;
    const hipError_t e = mx::check_offsets(off, G, total, align, min_len, first_zero, exact_end,
                                           (hipStream_t)stream, &bad);
    if (e != hipSuccess)
        return fail(MX_ERR_HIP, "%s: MX_DEBUG check of %s failed: %s", fn, what, hipGetErrorString(e));
    if (bad >= 0)
        return fail(MX_ERR_INVALID_ARG, "%s: %s[%lld] breaks the stated properties (MX_DEBUG check)", fn, what,
                    (long long)bad);
    return MX_OK;
}

}  // namespace

extern "C" {

int mx_abi_version(void) { return MXFP8_ABI_VERSION; }

const char *mx_status_string(int status)
{
    switch (status) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARG: return "MX_ERR_INVALID_ARG";
    case MX_ERR_SHAPE: return "MX_ERR_SHAPE";
    case MX_ERR_ALIGN: return "MX_ERR_ALIGN";
    case MX_ERR_OVERLAP: return "MX_ERR_OVERLAP";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    default: return "MX_ERR_UNKNOWN";
    }
}

const char *mx_last_error(void) { return g_err; }

int64_t mx_scale_swizzled_bytes(int64_t rows, int64_t kblocks) { return swz_bytes(rows, kblocks); }

mx_status mx_quantize_rowwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *q,
                              int64_t ld_q, void *s, int64_t ld_s, void *stream)
{
    const char *fn = "mx_quantize_rowwise";
    if (rows < 0 || cols < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld cols=%lld", fn,
                    (long long)rows, (long long)cols);
    if (cols % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of the 32-element block", fn,
                    (long long)cols);
    if (ld_x < cols || ld_q < cols || ld_s < cols / 32)
        return fail(MX_ERR_INVALID_ARG,
                    "%s: leading dimension too small (ld_x=%lld ld_q=%lld ld_s=%lld, cols=%lld)",
                    fn, (long long)ld_x, (long long)ld_q, (long long)ld_s, (long long)cols);
    if (rows == 0 || cols == 0)
        return ok();
    if (!x || !q || !s)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || !aligned(q, 16) || ld_x % 8 != 0 || ld_q % 16 != 0)
        return fail(MX_ERR_ALIGN, "%s: x and q need 16-byte aligned rows (ld_x %% 8, ld_q %% 16)",
                    fn);
    const int64_t ex = extent(rows, cols, ld_x, 2), eq = extent(rows, cols, ld_q, 1),
                  es = extent(rows, cols / 32, ld_s, 1);
    if (overlap(x, ex, q, eq) || overlap(x, ex, s, es) || overlap(q, eq, s, es))
        return fail(MX_ERR_OVERLAP, "%s: input and outputs overlap", fn);
    return hip_status(mx::launch_quantize_rowwise(x, rows, cols, ld_x, q, ld_q, s, ld_s,
                                                  (hipStream_t)stream),
                      fn);
}

// Checks of one row-wise job with rearranged scales; `who` names it in messages.
static mx_status check_rowwise_swz(const char *who, const mx_rowwise_job &j)
{
    const int64_t rows = j.rows, cols = j.cols;
    if (rows < 0 || cols < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld cols=%lld", who, (long long)rows,
                    (long long)cols);
    if (cols % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of the 32-element block", who,
                    (long long)cols);
    if (cols % 256 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: cols=%lld: this build needs cols %% 256 == 0", who,
                    (long long)cols);
    if (j.ld_x < cols || j.ld_q < cols || j.s_tiles < cols / 256)
        return fail(MX_ERR_INVALID_ARG, "%s: ld_x=%lld, ld_q=%lld or s_tiles=%lld too small", who,
                    (long long)j.ld_x, (long long)j.ld_q, (long long)j.s_tiles);
    if (rows == 0 || cols == 0)
        return MX_OK;
    if (!j.x || !j.q || !j.s_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", who);
    if (!aligned(j.x, 16) || !aligned(j.q, 8) || j.ld_x % 8 != 0 || j.ld_q % 8 != 0)
        return fail(MX_ERR_ALIGN, "%s: x needs 16-byte aligned rows (ld_x %% 8), q 8-byte (ld_q %% 8)", who);
    const int64_t ex = extent(rows, cols, j.ld_x, 2), eq = extent(rows, cols, j.ld_q, 1);
    const int64_t es = (((rows + 31) / 32 - 1) * j.s_tiles + cols / 256) * 256;
    if (overlap(j.x, ex, j.q, eq) || overlap(j.x, ex, j.s_swz, es) || overlap(j.q, eq, j.s_swz, es))
        return fail(MX_ERR_OVERLAP, "%s: input and outputs must not overlap", who);
    return MX_OK;
}

mx_status mx_quantize_rowwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *q,
                                  int64_t ld_q, void *s_swz, int64_t s_tiles, void *stream)
{
    const char *fn = "mx_quantize_rowwise_swz";
    const mx_status st = check_rowwise_swz(fn, mx_rowwise_job{x, rows, cols, ld_x, q, ld_q, s_swz, s_tiles});
    if (st != MX_OK)
        return st;
    if (rows == 0 || cols == 0)
        return ok();
    return hip_status(mx::launch_quantize_rowwise_swz(x, rows, cols, ld_x, q, ld_q, s_swz, s_tiles,
                                                      (hipStream_t)stream),
                      fn);
}

mx_status mx_quantize_rowwise_swz_batch(const mx_rowwise_job *jobs, int n_jobs, void *stream)
{
    const char *fn = "mx_quantize_rowwise_swz_batch";
    if (n_jobs < 0 || n_jobs > MX_ROWWISE_MAX_JOBS)
        return fail(MX_ERR_INVALID_ARG, "%s: n_jobs=%d outside 0..%d", fn, n_jobs, MX_ROWWISE_MAX_JOBS);
    if (n_jobs == 0)
        return ok();
    if (!jobs)
        return fail(MX_ERR_INVALID_ARG, "%s: null job array", fn);
    static_assert(MX_ROWWISE_MAX_JOBS == mx::QR_MAX_JOBS, "job limits differ");
    mx::RowJob rj[MX_ROWWISE_MAX_JOBS];
    int n = 0;
    for (int i = 0; i < n_jobs; i++) {
        char who[96];
        snprintf(who, sizeof who, "%s: job %d", fn, i);
        const mx_status st = check_rowwise_swz(who, jobs[i]);
        if (st != MX_OK)
            return st;
        const mx_rowwise_job &a = jobs[i];
        if (a.rows == 0 || a.cols == 0)
            continue;
        // a job's input must not be written by another job
        const int64_t ex = extent(a.rows, a.cols, a.ld_x, 2);
        for (int k = 0; k < n_jobs; k++) {
            const mx_rowwise_job &b = jobs[k];
            if (k == i || b.rows == 0 || b.cols == 0)
                continue;
            const int64_t es = (((b.rows + 31) / 32 - 1) * b.s_tiles + b.cols / 256) * 256;
            if (overlap(a.x, ex, b.q, extent(b.rows, b.cols, b.ld_q, 1)) || overlap(a.x, ex, b.s_swz, es))
                return fail(MX_ERR_OVERLAP, "%s: job %d's input overlaps job %d's outputs", fn, i, k);
        }
        rj[n++] = mx::RowJob{a.x, a.rows, a.cols, a.ld_x, a.q, a.ld_q, a.s_swz, a.s_tiles};
    }
    if (n == 0)
        return ok();
    return hip_status(mx::launch_quantize_rowwise_batch(rj, n, (hipStream_t)stream), fn);
}

mx_status mx_quantize_colwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *qt,
                              int64_t ld_qt, void *st, int64_t ld_st, void *stream)
{
    const char *fn = "mx_quantize_colwise";
    if (rows < 0 || cols < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld cols=%lld", fn,
                    (long long)rows, (long long)cols);
    if (rows % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: rows=%lld is not a multiple of the 32-element block", fn,
                    (long long)rows);
    if (cols % 8 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 8", fn, (long long)cols);
    if (ld_x < cols || ld_qt < rows || ld_st < rows / 32)
        return fail(MX_ERR_INVALID_ARG,
                    "%s: leading dimension too small (ld_x=%lld ld_qt=%lld ld_st=%lld)", fn,
                    (long long)ld_x, (long long)ld_qt, (long long)ld_st);
    if (rows == 0 || cols == 0)
        return ok();
    if (!x || !qt || !st)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || !aligned(qt, 16) || ld_x % 8 != 0 || ld_qt % 16 != 0)
        return fail(MX_ERR_ALIGN,
                    "%s: x and qt need 16-byte aligned rows (ld_x %% 8, ld_qt %% 16)", fn);
    const int64_t ex = extent(rows, cols, ld_x, 2), eq = extent(cols, rows, ld_qt, 1),
                  es = extent(cols, rows / 32, ld_st, 1);
    if (overlap(x, ex, qt, eq) || overlap(x, ex, st, es) || overlap(qt, eq, st, es))
        return fail(MX_ERR_OVERLAP, "%s: input and outputs overlap", fn);
    return hip_status(mx::launch_quantize_colwise(x, rows, cols, ld_x, qt, ld_qt, st, ld_st,
                                                  (hipStream_t)stream),
                      fn);
}

mx_status mx_quantize_colwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *qt,
                                  int64_t ld_qt, void *st_swz, int64_t st_tiles, void *stream)
{
    const char *fn = "mx_quantize_colwise_swz";
    if (rows < 0 || cols < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld cols=%lld", fn,
                    (long long)rows, (long long)cols);
    if (rows % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: rows=%lld is not a multiple of the 32-element block", fn,
                    (long long)rows);
    if (cols % 8 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 8", fn, (long long)cols);
    if (rows % 256 != 0 || cols % 32 != 0)
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: rows=%lld, cols=%lld: this build needs rows %% 256 == 0 and cols %% 32 == 0", fn,
                    (long long)rows, (long long)cols);
    if (ld_x < cols || ld_qt < rows || st_tiles < rows / 256)
        return fail(MX_ERR_INVALID_ARG, "%s: ld_x=%lld, ld_qt=%lld or st_tiles=%lld too small", fn,
                    (long long)ld_x, (long long)ld_qt, (long long)st_tiles);
    if (rows == 0 || cols == 0)
        return ok();
    if (!x || !qt || !st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || !aligned(qt, 16) || ld_x % 8 != 0 || ld_qt % 16 != 0)
        return fail(MX_ERR_ALIGN,
                    "%s: x and qt need 16-byte aligned rows (ld_x %% 8, ld_qt %% 16)", fn);
    const int64_t ex = extent(rows, cols, ld_x, 2), eq = extent(cols, rows, ld_qt, 1);
    const int64_t es = ((cols / 32 - 1) * st_tiles + rows / 256) * 256;
    if (overlap(x, ex, qt, eq) || overlap(x, ex, st_swz, es) || overlap(qt, eq, st_swz, es))
        return fail(MX_ERR_OVERLAP, "%s: input and outputs overlap", fn);
    return hip_status(mx::launch_quantize_colwise_swz(x, rows, cols, ld_x, qt, ld_qt, st_swz, st_tiles,
                                                      (hipStream_t)stream),
                      fn);
}

// Checks of one dual-quantization job; `who` names it in messages.
static mx_status check_dual_job(const char *who, const mx_dual_job &j)
{
    const int64_t rows = j.rows, cols = j.cols;
    if (rows < 0 || cols < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld cols=%lld", who,
                    (long long)rows, (long long)cols);
    if (rows % 32 != 0 || cols % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: rows=%lld and cols=%lld must be multiples of the 32-element block",
                    who, (long long)rows, (long long)cols);
    if (j.ld_x < cols || j.ld_q < cols || j.ld_qt < rows)
        return fail(MX_ERR_INVALID_ARG,
                    "%s: leading dimension too small (ld_x=%lld ld_q=%lld ld_qt=%lld)", who,
                    (long long)j.ld_x, (long long)j.ld_q, (long long)j.ld_qt);
    const int64_t kt_row = (cols / 32 + 7) / 8, kt_col = (rows / 32 + 7) / 8;
    if (j.s_tiles < kt_row || j.st_tiles < kt_col)
        return fail(MX_ERR_INVALID_ARG,
                    "%s: tiles per rearranged row too small (s_tiles=%lld < %lld or st_tiles=%lld < %lld)",
                    who, (long long)j.s_tiles, (long long)kt_row, (long long)j.st_tiles, (long long)kt_col);
    if (rows == 0 || cols == 0)
        return MX_OK;
    if (!j.x || !j.q || !j.s_swz || !j.qt || !j.st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", who);
    if (!aligned(j.x, 16) || !aligned(j.q, 16) || !aligned(j.qt, 16) || j.ld_x % 8 != 0 ||
        j.ld_q % 16 != 0 || j.ld_qt % 16 != 0)
        return fail(MX_ERR_ALIGN,
                    "%s: x, q and qt need 16-byte aligned rows (ld_x %% 8, ld_q %% 16, ld_qt %% 16)", who);
    if (!aligned(j.s_swz, 4) || !aligned(j.st_swz, 4))
        return fail(MX_ERR_ALIGN, "%s: s_swz and st_swz must be 4-byte aligned", who);
    if (j.ld_q >= ((int64_t)1 << 24) || j.ld_qt >= ((int64_t)1 << 24))
        return fail(MX_ERR_UNSUPPORTED, "%s: ld_q and ld_qt must be below 2^24 (32-bit offsets within a tile)", who);
    // byte extents: the rearranged outputs span their last tile row's tiles
    const int64_t ex = extent(rows, cols, j.ld_x, 2), eq = extent(rows, cols, j.ld_q, 1),
                  eqt = extent(cols, rows, j.ld_qt, 1);
    const int64_t es = ((rows / 32 - 1) * j.s_tiles + kt_row) * 256,
                  est = ((cols / 32 - 1) * j.st_tiles + kt_col) * 256;
    const void *outs[4] = {j.q, j.s_swz, j.qt, j.st_swz};
    const int64_t lens[4] = {eq, es, eqt, est};
    for (int i = 0; i < 4; i++) {
        if (overlap(j.x, ex, outs[i], lens[i]))
            return fail(MX_ERR_OVERLAP, "%s: input and an output overlap", who);
        for (int k = i + 1; k < 4; k++)
            if (overlap(outs[i], lens[i], outs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: two outputs overlap", who);
    }
    return MX_OK;
}

static mx::DualJob to_job(const mx_dual_job &j)
{
    return mx::DualJob{j.x, j.rows, j.cols, j.ld_x, j.q, j.ld_q, j.s_swz, j.s_tiles,
                       j.qt, j.ld_qt, j.st_swz, j.st_tiles, 1, 0, 0, 0, 0, 0};
}

mx_status mx_quantize_dual(const void *x, int64_t rows, int64_t cols, int64_t ld_x, void *q,
                           int64_t ld_q, void *s_swz, int64_t s_tiles, void *qt, int64_t ld_qt,
                           void *st_swz, int64_t st_tiles, void *stream)
{
    const char *fn = "mx_quantize_dual";
    const mx_dual_job j{x, rows, cols, ld_x, q, ld_q, s_swz, s_tiles, qt, ld_qt, st_swz, st_tiles};
    const mx_status st = check_dual_job(fn, j);
    if (st != MX_OK)
        return st;
    if (rows == 0 || cols == 0)
        return ok();
    const mx::DualJob dj = to_job(j);
    return hip_status(mx::launch_quantize_dual(&dj, 1, (hipStream_t)stream), fn);
}

mx_status mx_quantize_dual_batch(const mx_dual_job *jobs, int n_jobs, void *stream)
{
    const char *fn = "mx_quantize_dual_batch";
    if (n_jobs < 0 || n_jobs > MX_DUAL_MAX_JOBS)
        return fail(MX_ERR_INVALID_ARG, "%s: n_jobs=%d outside 0..%d", fn, n_jobs, MX_DUAL_MAX_JOBS);
    if (n_jobs == 0)
        return ok();
    if (!jobs)
        return fail(MX_ERR_INVALID_ARG, "%s: null job array", fn);
    mx::DualJob dj[MX_DUAL_MAX_JOBS];
    int n = 0;
    for (int i = 0; i < n_jobs; i++) {
        char who[96];
        snprintf(who, sizeof who, "%s: job %d", fn, i);
        const mx_status st = check_dual_job(who, jobs[i]);
        if (st != MX_OK)
            return st;
        // a job's input must not be written by another job
        for (int k = 0; k < n_jobs; k++) {
            if (k == i || jobs[k].rows <= 0 || jobs[k].cols <= 0 || jobs[i].rows <= 0 || jobs[i].cols <= 0)
                continue;
            const mx_dual_job &a = jobs[i], &b = jobs[k];
            const int64_t ex = extent(a.rows, a.cols, a.ld_x, 2);
            if (overlap(a.x, ex, b.q, extent(b.rows, b.cols, b.ld_q, 1)) ||
                overlap(a.x, ex, b.qt, extent(b.cols, b.rows, b.ld_qt, 1)))
                return fail(MX_ERR_OVERLAP, "%s: job %d's input overlaps job %d's codes", fn, i, k);
        }
        if (jobs[i].rows > 0 && jobs[i].cols > 0)
            dj[n++] = to_job(jobs[i]);
    }
    if (n == 0)
        return ok();
    return hip_status(mx::launch_quantize_dual(dj, n, (hipStream_t)stream), fn);
}

mx_status mx_quantize_dual_experts(const void *x, int64_t num_experts, int64_t rows, int64_t cols,
                                   void *q, void *s_swz, void *qt, void *st_swz, void *stream)
{
    const char *fn = "mx_quantize_dual_experts";
    if (num_experts < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: num_experts=%lld < 0", fn, (long long)num_experts);
    if (num_experts > (1 << 20))
        return fail(MX_ERR_UNSUPPORTED, "%s: num_experts=%lld too large", fn, (long long)num_experts);
    // one expert's job: contiguous [rows][cols] in, [rows][cols] and [cols][rows] out
    const int64_t s_tiles = (cols / 32 + 7) / 8, st_tiles = (rows / 32 + 7) / 8;
    const mx_dual_job j{x, rows, cols, cols, q, cols, s_swz, s_tiles, qt, rows, st_swz, st_tiles};
    const mx_status st = check_dual_job(fn, j);
    if (st != MX_OK)
        return st;
    if (num_experts == 0 || rows == 0 || cols == 0)
        return ok();
    const int64_t n = rows * cols, sb = swz_bytes(rows, cols / 32), stb = swz_bytes(cols, rows / 32);
    if (n * num_experts >= ((int64_t)1 << 40))
        return fail(MX_ERR_UNSUPPORTED, "%s: stack too large", fn);
    // the whole stacks: the input against every output, the outputs pairwise
    const void *bufs[5] = {x, q, s_swz, qt, st_swz};
    const int64_t lens[5] = {2 * n * num_experts, n * num_experts, sb * num_experts, n * num_experts,
                             stb * num_experts};
    for (int i = 0; i < 5; i++)
        for (int k = i + 1; k < 5; k++)
            if (overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    mx::DualJob dj = to_job(j);
    dj.count = num_experts;
    dj.x_stride = n;
    dj.q_stride = n;
    dj.s_stride = sb;
    dj.qt_stride = n;
    dj.st_stride = stb;
    if (num_experts * ((rows + 255) / 256) * ((cols + 255) / 256 + 7) >= ((int64_t)1 << 31))
        return fail(MX_ERR_UNSUPPORTED, "%s: too many blocks for one launch", fn);
    return hip_status(mx::launch_quantize_dual(&dj, 1, (hipStream_t)stream), fn);
}

}  // extern "C"

namespace {

// Arguments of the MoE dispatch (both entry points): MX_OK or the first problem.
mx_status check_dispatch(const char *fn, const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                         const int32_t *topk_ids, int64_t topk, int64_t num_experts, int64_t *offsets,
                         int32_t *src_token, int32_t *slot, void *q, int64_t ld_q, void *s_swz,
                         const void **bufs, int64_t *lens)
{
    if (tokens < 0 || hidden < 0 || topk < 1 || num_experts < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: need tokens, hidden >= 0, topk, num_experts >= 1", fn);
    if (hidden % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: hidden=%lld is not a multiple of the 32-element block", fn,
                    (long long)hidden);
    if (hidden % 256 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: hidden=%lld: this build needs hidden %% 256 == 0", fn,
                    (long long)hidden);
    if (num_experts > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_experts=%lld > %d", fn, (long long)num_experts,
                    mx::MOE_MAX_EXPERTS);
    if (tokens * topk >= ((int64_t)1 << 31) / 2)
        return fail(MX_ERR_UNSUPPORTED, "%s: tokens * topk must stay below 2^30", fn);
    if (ld_x < hidden || ld_q < hidden)
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small (ld_x=%lld ld_q=%lld)", fn,
                    (long long)ld_x, (long long)ld_q);
    if (!offsets)
        return fail(MX_ERR_INVALID_ARG, "%s: null offsets", fn);
    if (tokens == 0 || hidden == 0) {
        // nothing routed: offsets all zero would need a device write; refuse
        // instead of leaving them unwritten
        return fail(MX_ERR_INVALID_ARG, "%s: tokens and hidden must be positive", fn);
    }
    if (!x || !topk_ids || !src_token || !slot || !q || !s_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || !aligned(q, 16) || ld_x % 8 != 0 || ld_q % 16 != 0)
        return fail(MX_ERR_ALIGN, "%s: x and q need 16-byte aligned rows (ld_x %% 8, ld_q %% 16)", fn);
    if (!aligned(topk_ids, 4) || !aligned(src_token, 4) || !aligned(slot, 4) || !aligned(offsets, 8))
        return fail(MX_ERR_ALIGN, "%s: index arrays need their natural alignment", fn);
    const int64_t n = tokens * topk;
    const void *b7[7] = {x, topk_ids, offsets, src_token, slot, q, s_swz};
    const int64_t l7[7] = {extent(tokens, hidden, ld_x, 2), n * 4, (num_experts + 1) * 8, n * 4, n * 4,
                           extent(n, hidden, ld_q, 1), swz_bytes(n, hidden / 32)};
    for (int i = 0; i < 7; i++) {
        bufs[i] = b7[i];
        lens[i] = l7[i];
    }
    for (int i = 0; i < 7; i++)
        for (int k = i + 1; k < 7; k++)
            if ((i >= 2 || k >= 2) && overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    return MX_OK;
}

}  // namespace

extern "C" {

mx_status mx_moe_dispatch(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                          const int32_t *topk_ids, int64_t topk, int64_t num_experts,
                          int64_t *offsets, int32_t *src_token, int32_t *slot, void *q, int64_t ld_q,
                          void *s_swz, void *workspace, int64_t workspace_bytes, void *stream)
{
    const char *fn = "mx_moe_dispatch";
    const void *bufs[7];
    int64_t lens[7];
    mx_status st = check_dispatch(fn, x, tokens, hidden, ld_x, topk_ids, topk, num_experts, offsets, src_token,
                                  slot, q, ld_q, s_swz, bufs, lens);
    if (st != MX_OK)
        return st;
    st = check_workspace(fn, workspace, workspace_bytes, mx::moe_dispatch_workspace_bytes(tokens, topk, num_experts),
                         4, bufs, lens, 7);
    if (st != MX_OK)
        return st;
    return hip_status(mx::launch_moe_dispatch(x, tokens, hidden, ld_x, topk_ids, topk, num_experts,
                                              offsets, src_token, slot, q, ld_q, s_swz, workspace,
                                              (hipStream_t)stream),
                      fn);
}

mx_status mx_moe_dispatch_dual_grouped(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                      const int32_t *topk_ids, int64_t topk, int64_t num_experts,
                                      int64_t *offsets, int32_t *src_token, int32_t *slot, void *q,
                                      int64_t ld_q, void *s_swz, int64_t *pad_offsets, void *qt, int64_t ld_qt,
                                      int64_t k_cap, void *st_swz, void *workspace, int64_t workspace_bytes,
                                      void *stream)
{
    const char *fn = "mx_moe_dispatch_dual_grouped";
    const void *bufs[10];
    int64_t lens[10];
    mx_status st = check_dispatch(fn, x, tokens, hidden, ld_x, topk_ids, topk, num_experts, offsets, src_token,
                                  slot, q, ld_q, s_swz, bufs, lens);
    if (st != MX_OK)
        return st;
    const int64_t n = tokens * topk;
    if (k_cap % 256 != 0 || k_cap < mx_grouped_k_capacity(n, num_experts))
        return fail(MX_ERR_INVALID_ARG,
                    "%s: k_cap=%lld must be a multiple of 256 and at least "
                    "mx_grouped_k_capacity(tokens * topk, num_experts) = %lld",
                    fn, (long long)k_cap, (long long)mx_grouped_k_capacity(n, num_experts));
    if (ld_qt < k_cap)
        return fail(MX_ERR_INVALID_ARG, "%s: ld_qt=%lld < k_cap=%lld", fn, (long long)ld_qt, (long long)k_cap);
    if (!pad_offsets || !qt || !st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(qt, 16) || ld_qt % 16 != 0 || !aligned(st_swz, 4) || !aligned(pad_offsets, 8) ||
        !aligned(s_swz, 4))
        return fail(MX_ERR_ALIGN, "%s: qt needs 16-byte aligned rows (ld_qt %% 16), the scales 4 bytes, "
                                  "pad_offsets 8 bytes", fn);
    // the gathered rows' offsets into x, the row-wise codes' into q, the
    // column-wise codes' into qt and the grouped tiles are formed in 32 bits
    if (extent(tokens, hidden, ld_x, 2) >= ((int64_t)1 << 31) || ld_x >= ((int64_t)1 << 22) ||
        ld_q >= ((int64_t)1 << 24) || ld_qt >= ((int64_t)1 << 24) ||
        k_cap / 256 * (hidden / 256) >= ((int64_t)1 << 31))
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: operand too large for this build (x below 2^31 bytes, ld_x < 2^22, ld_q and ld_qt < 2^24)",
                    fn);
    bufs[7] = pad_offsets;
    lens[7] = (num_experts + 1) * 8;
    bufs[8] = qt;
    lens[8] = extent(hidden, k_cap, ld_qt, 1);
    bufs[9] = st_swz;
    lens[9] = swz_bytes(hidden, k_cap / 32);
    for (int i = 7; i < 10; i++)
        for (int k = 0; k < i; k++)
            if (overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    st = check_workspace(fn, workspace, workspace_bytes, mx::moe_dispatch_workspace_bytes(tokens, topk, num_experts),
                         4, bufs, lens, 10);
    if (st != MX_OK)
        return st;
    return hip_status(mx::launch_moe_dispatch_dual_grouped(x, tokens, hidden, ld_x, topk_ids, topk, num_experts,
                                                           offsets, src_token, slot, q, ld_q, s_swz, pad_offsets,
                                                           qt, ld_qt, k_cap, st_swz, workspace,
                                                           (hipStream_t)stream),
                      fn);
}

mx_status mx_moe_dispatch_noalloc(const void *x, int64_t tokens, int64_t hidden, int64_t ld_x,
                                  const int32_t *topk_ids, int64_t topk, int64_t num_experts,
                                  int64_t *offsets, int32_t *src_token, int32_t *slot, void *q, int64_t ld_q,
                                  void *s_swz, void *stream)
{
    const char *fn = "mx_moe_dispatch_noalloc";
    const void *bufs[7];
    int64_t lens[7];
    mx_status st = check_dispatch(fn, x, tokens, hidden, ld_x, topk_ids, topk, num_experts, offsets, src_token,
                                  slot, q, ld_q, s_swz, bufs, lens);
    if (st != MX_OK)
        return st;
    const int64_t need = mx::moe_dispatch_workspace_bytes(tokens, topk, num_experts);
    static_assert(mx::MOE_NOALLOC_SCRATCH_BYTES == MX_MOE_DISPATCH_NOALLOC_SCRATCH_BYTES,
                  "the header states the scratch size");
    if (need > mx::MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: %lld tokens x top-%lld over %lld experts need %lld bytes of scratch, more than the "
                    "%lld this entry point holds (use mx_moe_dispatch with a workspace)",
                    fn, (long long)tokens, (long long)topk, (long long)num_experts, (long long)need,
                    (long long)mx::MOE_NOALLOC_SCRATCH_BYTES);
    void *scratch = nullptr;
    const hipError_t e = mx::moe_noalloc_scratch(&scratch);
    if (e != hipSuccess)
        return fail(MX_ERR_HIP, "%s: device scratch lookup failed: %s", fn, hipGetErrorString(e));
    return hip_status(mx::launch_moe_dispatch(x, tokens, hidden, ld_x, topk_ids, topk, num_experts,
                                              offsets, src_token, slot, q, ld_q, s_swz, scratch,
                                              (hipStream_t)stream),
                      fn);
}

int64_t mx_moe_dispatch_workspace_bytes(int64_t tokens, int64_t topk, int64_t num_experts)
{
    if (tokens <= 0 || topk <= 0 || num_experts <= 0 || num_experts > mx::MOE_MAX_EXPERTS ||
        tokens * topk >= ((int64_t)1 << 30))
        return 0;
    return mx::moe_dispatch_workspace_bytes(tokens, topk, num_experts);
}

int64_t mx_grouped_k_capacity(int64_t rows_total, int64_t num_groups)
{
    if (rows_total < 0 || num_groups < 1)
        return 0;
    return (rows_total + 255) / 256 * 256 + 256 * num_groups;
}

mx_status mx_quantize_colwise_grouped(const void *x, int64_t rows_total, int64_t cols, int64_t ld_x,
                                      const int64_t *group_offsets, int64_t num_groups,
                                      int64_t *pad_offsets, void *qt, int64_t ld_qt, int64_t k_cap,
                                      void *st_swz, void *stream)
{
    const char *fn = "mx_quantize_colwise_grouped";
    if (rows_total < 0 || cols < 1 || num_groups < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: need rows_total >= 0, cols >= 1, num_groups >= 1", fn);
    if (num_groups > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_groups=%lld > %d", fn, (long long)num_groups,
                    mx::MOE_MAX_EXPERTS);
    if (cols % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 32", fn, (long long)cols);
    if (k_cap % 256 != 0 || k_cap < mx_grouped_k_capacity(rows_total, num_groups))
        return fail(MX_ERR_INVALID_ARG,
                    "%s: k_cap=%lld must be a multiple of 256 and at least "
                    "mx_grouped_k_capacity(rows_total, num_groups) = %lld",
                    fn, (long long)k_cap, (long long)mx_grouped_k_capacity(rows_total, num_groups));
    if (ld_x < cols || ld_qt < k_cap)
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small (ld_x=%lld ld_qt=%lld)", fn,
                    (long long)ld_x, (long long)ld_qt);
    if ((!x && rows_total > 0) || !group_offsets || !pad_offsets || !qt || !st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(qt, 16) || ld_qt % 16 != 0 || !aligned(st_swz, 4) ||
        !aligned(group_offsets, 8) || !aligned(pad_offsets, 8))
        return fail(MX_ERR_ALIGN,
                    "%s: x and qt need 16-byte aligned rows (ld_x %% 8, ld_qt %% 16), st_swz 4 bytes, "
                    "the offsets 8 bytes",
                    fn);
    if (k_cap / 256 * ((cols + 255) / 256) >= ((int64_t)1 << 31) || ld_x >= ((int64_t)1 << 22) ||
        ld_qt >= ((int64_t)1 << 24))
        return fail(MX_ERR_UNSUPPORTED, "%s: operand too large for this build (ld_x < 2^22, ld_qt < 2^24)", fn);
    const void *bufs[5] = {x, group_offsets, pad_offsets, qt, st_swz};
    const int64_t lens[5] = {rows_total > 0 ? extent(rows_total, cols, ld_x, 2) : 0, (num_groups + 1) * 8,
                             (num_groups + 1) * 8, extent(cols, k_cap, ld_qt, 1), swz_bytes(cols, k_cap / 32)};
    for (int i = 0; i < 5; i++)
        for (int k = i + 1; k < 5; k++)
            if ((i >= 2 || k >= 2) && overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    if (debug_checks()) {
        const mx_status dst =
            debug_offsets(fn, "group_offsets", group_offsets, num_groups, rows_total, 1, 0, false, false, stream);
        if (dst != MX_OK)
            return dst;
    }
    return hip_status(mx::launch_quantize_colwise_grouped(x, rows_total, cols, ld_x, group_offsets,
                                                          num_groups, pad_offsets, qt, ld_qt, k_cap,
                                                          st_swz, (hipStream_t)stream),
                      fn);
}

mx_status mx_quantize_dual_grouped(const void *x, int64_t rows_total, int64_t cols, int64_t ld_x,
                                   const int64_t *group_offsets, int64_t num_groups, int64_t *pad_offsets,
                                   void *q, int64_t ld_q, void *s_swz, void *qt, int64_t ld_qt, int64_t k_cap,
                                   void *st_swz, void *stream)
{
    const char *fn = "mx_quantize_dual_grouped";
    if (rows_total < 0 || cols < 1 || num_groups < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: need rows_total >= 0, cols >= 1, num_groups >= 1", fn);
    if (num_groups > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_groups=%lld > %d", fn, (long long)num_groups,
                    mx::MOE_MAX_EXPERTS);
    if (cols % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: cols=%lld is not a multiple of 32", fn, (long long)cols);
    if (cols % 256 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: cols=%lld: this build needs cols %% 256 == 0", fn, (long long)cols);
    if (k_cap % 256 != 0 || k_cap < mx_grouped_k_capacity(rows_total, num_groups))
        return fail(MX_ERR_INVALID_ARG,
                    "%s: k_cap=%lld must be a multiple of 256 and at least "
                    "mx_grouped_k_capacity(rows_total, num_groups) = %lld",
                    fn, (long long)k_cap, (long long)mx_grouped_k_capacity(rows_total, num_groups));
    if (ld_x < cols || ld_qt < k_cap || ld_q < cols)
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small (ld_x=%lld ld_q=%lld ld_qt=%lld)", fn,
                    (long long)ld_x, (long long)ld_q, (long long)ld_qt);
    if ((!x && rows_total > 0) || (!q && rows_total > 0) || (!s_swz && rows_total > 0) || !group_offsets ||
        !pad_offsets || !qt || !st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(x, 16) || ld_x % 8 != 0 || !aligned(qt, 16) || ld_qt % 16 != 0 || !aligned(st_swz, 4) ||
        !aligned(q, 16) || ld_q % 16 != 0 || !aligned(s_swz, 4) || !aligned(group_offsets, 8) ||
        !aligned(pad_offsets, 8))
        return fail(MX_ERR_ALIGN,
                    "%s: x, q and qt need 16-byte aligned rows (ld_x %% 8, ld_q %% 16, ld_qt %% 16), "
                    "s_swz and st_swz 4 bytes, the offsets 8 bytes",
                    fn);
    if (k_cap / 256 * ((cols + 255) / 256) >= ((int64_t)1 << 31) || ld_x >= ((int64_t)1 << 22) ||
        ld_qt >= ((int64_t)1 << 24) || ld_q >= ((int64_t)1 << 24))
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: operand too large for this build (ld_x < 2^22, ld_q and ld_qt < 2^24)", fn);
    const void *bufs[7] = {x, group_offsets, pad_offsets, qt, st_swz, q, s_swz};
    const int64_t lens[7] = {rows_total > 0 ? extent(rows_total, cols, ld_x, 2) : 0, (num_groups + 1) * 8,
                             (num_groups + 1) * 8, extent(cols, k_cap, ld_qt, 1), swz_bytes(cols, k_cap / 32),
                             extent(rows_total, cols, ld_q, 1), swz_bytes(rows_total, cols / 32)};
    for (int i = 0; i < 7; i++)
        for (int k = i + 1; k < 7; k++)
            if ((i >= 2 || k >= 2) && overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    if (debug_checks()) {
        // the row-wise output covers the rows of the experts only: under
        // MX_DEBUG the offsets must also start at 0 and end at rows_total
        const mx_status dst =
            debug_offsets(fn, "group_offsets", group_offsets, num_groups, rows_total, 1, 0, true, true, stream);
        if (dst != MX_OK)
            return dst;
    }
    return hip_status(mx::launch_quantize_colwise_grouped(x, rows_total, cols, ld_x, group_offsets, num_groups,
                                                          pad_offsets, qt, ld_qt, k_cap, st_swz,
                                                          (hipStream_t)stream, rows_total > 0 ? q : nullptr,
                                                          ld_q, s_swz),
                      fn);
}

mx_status mx_swiglu_quantize_dual_grouped(const void *gu, int64_t rows_total, int64_t F, int64_t ld_gu,
                                          const int64_t *group_offsets, int64_t num_groups, int64_t *pad_offsets,
                                          void *q, int64_t ld_q, void *s_swz, void *qt, int64_t ld_qt,
                                          int64_t k_cap, void *st_swz, void *stream)
{
    const char *fn = "mx_swiglu_quantize_dual_grouped";
    if (rows_total < 0 || F < 1 || num_groups < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: need rows_total >= 0, F >= 1, num_groups >= 1", fn);
    if (num_groups > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_groups=%lld > %d", fn, (long long)num_groups,
                    mx::MOE_MAX_EXPERTS);
    if (F % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: F=%lld is not a multiple of 32", fn, (long long)F);
    if (F % 256 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: F=%lld: this build needs F %% 256 == 0", fn, (long long)F);
    if (k_cap % 256 != 0 || k_cap < mx_grouped_k_capacity(rows_total, num_groups))
        return fail(MX_ERR_INVALID_ARG,
                    "%s: k_cap=%lld must be a multiple of 256 and at least "
                    "mx_grouped_k_capacity(rows_total, num_groups) = %lld",
                    fn, (long long)k_cap, (long long)mx_grouped_k_capacity(rows_total, num_groups));
    if (ld_gu < 2 * F || ld_qt < k_cap || ld_q < F)
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small (ld_gu=%lld ld_q=%lld ld_qt=%lld)", fn,
                    (long long)ld_gu, (long long)ld_q, (long long)ld_qt);
    if ((!gu && rows_total > 0) || (!q && rows_total > 0) || (!s_swz && rows_total > 0) || !group_offsets ||
        !pad_offsets || !qt || !st_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(gu, 16) || ld_gu % 8 != 0 || !aligned(qt, 16) || ld_qt % 16 != 0 || !aligned(st_swz, 4) ||
        !aligned(q, 16) || ld_q % 16 != 0 || !aligned(s_swz, 4) || !aligned(group_offsets, 8) ||
        !aligned(pad_offsets, 8))
        return fail(MX_ERR_ALIGN,
                    "%s: gu, q and qt need 16-byte aligned rows (ld_gu %% 8, ld_q %% 16, ld_qt %% 16), "
                    "s_swz and st_swz 4 bytes, the offsets 8 bytes",
                    fn);
    if (k_cap / 256 * (F / 256) >= ((int64_t)1 << 31) || ld_gu >= ((int64_t)1 << 22) ||
        ld_qt >= ((int64_t)1 << 24) || ld_q >= ((int64_t)1 << 24))
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: operand too large for this build (ld_gu < 2^22, ld_q and ld_qt < 2^24)", fn);
    const void *bufs[7] = {gu, group_offsets, pad_offsets, qt, st_swz, q, s_swz};
    const int64_t lens[7] = {rows_total > 0 ? extent(rows_total, 2 * F, ld_gu, 2) : 0, (num_groups + 1) * 8,
                             (num_groups + 1) * 8, extent(F, k_cap, ld_qt, 1), swz_bytes(F, k_cap / 32),
                             extent(rows_total, F, ld_q, 1), swz_bytes(rows_total, F / 32)};
    for (int i = 0; i < 7; i++)
        for (int k = i + 1; k < 7; k++)
            if ((i >= 2 || k >= 2) && overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    if (debug_checks()) {
        // the row-wise output covers the rows of the experts only: under
        // MX_DEBUG the offsets must also start at 0 and end at rows_total
        const mx_status dst =
            debug_offsets(fn, "group_offsets", group_offsets, num_groups, rows_total, 1, 0, true, true, stream);
        if (dst != MX_OK)
            return dst;
    }
    return hip_status(mx::launch_quantize_colwise_grouped(gu, rows_total, F, ld_gu, group_offsets, num_groups,
                                                          pad_offsets, qt, ld_qt, k_cap, st_swz,
                                                          (hipStream_t)stream, rows_total > 0 ? q : nullptr,
                                                          ld_q, s_swz, rows_total > 0),
                      fn);
}

mx_status mx_swiglu_quantize(const void *gu, int64_t rows, int64_t F, int64_t ld_gu, void *h, int64_t ld_h,
                             void *q, int64_t ld_q, void *s_swz, void *stream)
{
    const char *fn = "mx_swiglu_quantize";
    if (rows < 0 || F < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size rows=%lld F=%lld", fn, (long long)rows, (long long)F);
    if (F % 32 != 0)
        return fail(MX_ERR_SHAPE, "%s: F=%lld is not a multiple of the 32-element block", fn, (long long)F);
    if (F % 256 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: F=%lld: this build needs F %% 256 == 0", fn, (long long)F);
    if (ld_gu < 2 * F || ld_q < F || (h && ld_h < F))
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small (ld_gu=%lld ld_h=%lld ld_q=%lld)", fn,
                    (long long)ld_gu, (long long)ld_h, (long long)ld_q);
    if (rows == 0 || F == 0)
        return ok();
    if (!gu || !q || !s_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(gu, 16) || ld_gu % 8 != 0 || !aligned(q, 16) || ld_q % 16 != 0 ||
        (h && (!aligned(h, 16) || ld_h % 8 != 0)))
        return fail(MX_ERR_ALIGN, "%s: gu, h and q need 16-byte aligned rows (ld_gu %% 8, ld_h %% 8, ld_q %% 16)",
                    fn);
    if (rows * (F / 8) >= ((int64_t)1 << 40))
        return fail(MX_ERR_UNSUPPORTED, "%s: too large", fn);
    const void *bufs[4] = {gu, h, q, s_swz};
    const int64_t lens[4] = {extent(rows, 2 * F, ld_gu, 2), h ? extent(rows, F, ld_h, 2) : 0,
                             extent(rows, F, ld_q, 1), swz_bytes(rows, F / 32)};
    for (int i = 0; i < 4; i++)
        for (int k = i + 1; k < 4; k++)
            if (overlap(bufs[i], lens[i], bufs[k], lens[k]))
                return fail(MX_ERR_OVERLAP, "%s: buffers %d and %d overlap", fn, i, k);
    return hip_status(mx::launch_swiglu_quantize(gu, rows, F, ld_gu, h, ld_h, q, ld_q, s_swz, (hipStream_t)stream),
                      fn);
}

mx_status mx_moe_combine(const void *y, int64_t tokens, int64_t hidden, int64_t ld_y,
                         const int32_t *slot, const float *weights, int64_t topk, void *out,
                         int64_t ld_out, void *stream)
{
    const char *fn = "mx_moe_combine";
    if (tokens < 0 || hidden < 0 || topk < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: need tokens, hidden >= 0, topk >= 1", fn);
    if (hidden % 8 != 0)
        return fail(MX_ERR_SHAPE, "%s: hidden=%lld is not a multiple of 8", fn, (long long)hidden);
    if (ld_y < hidden || ld_out < hidden)
        return fail(MX_ERR_INVALID_ARG, "%s: leading dimension too small", fn);
    if (tokens == 0 || hidden == 0)
        return ok();
    if (!y || !slot || !weights || !out)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(y, 16) || !aligned(out, 16) || ld_y % 8 != 0 || ld_out % 8 != 0 || !aligned(slot, 4) ||
        !aligned(weights, 4))
        return fail(MX_ERR_ALIGN, "%s: y and out need 16-byte aligned rows (ld %% 8)", fn);
    const int64_t eo = extent(tokens, hidden, ld_out, 2);
    if (overlap(out, eo, slot, tokens * topk * 4) || overlap(out, eo, weights, tokens * topk * 4) ||
        overlap(out, eo, y, extent(tokens * topk, hidden, ld_y, 2)))
        return fail(MX_ERR_OVERLAP, "%s: out overlaps y or the routing", fn);
    return hip_status(mx::launch_moe_combine(y, tokens, hidden, ld_y, slot, weights, topk, out, ld_out,
                                             (hipStream_t)stream),
                      fn);
}

mx_status mx_scale_swizzle(const void *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                           void *s_swz, void *stream)
{
    const char *fn = "mx_scale_swizzle";
    if (rows < 0 || kblocks < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size", fn);
    if (ld_s < kblocks)
        return fail(MX_ERR_INVALID_ARG, "%s: ld_s=%lld < kblocks=%lld", fn, (long long)ld_s,
                    (long long)kblocks);
    if (rows == 0 || kblocks == 0)
        return ok();
    if (!s || !s_swz)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!aligned(s_swz, 4))
        return fail(MX_ERR_ALIGN, "%s: s_swz must be 4-byte aligned", fn);
    if (overlap(s, extent(rows, kblocks, ld_s, 1), s_swz, swz_bytes(rows, kblocks)))
        return fail(MX_ERR_OVERLAP, "%s: input and output overlap", fn);
    return hip_status(mx::launch_scale_swizzle(s, rows, kblocks, ld_s, s_swz, (hipStream_t)stream),
                      fn);
}

static mx_status check_gemm_common(const char *fn, int64_t M, int64_t N, int64_t K,
                                   const void *a_q, int64_t ld_a, const void *a_s,
                                   const void *b_q, int64_t ld_b, const void *b_s, void *c,
                                   int64_t ld_c, int c_dtype)
{
    if (M < 0 || N < 0 || K < 0)
        return fail(MX_ERR_INVALID_ARG, "%s: negative size M=%lld N=%lld K=%lld", fn,
                    (long long)M, (long long)N, (long long)K);
    if (c_dtype != MX_BF16 && c_dtype != MX_F32)
        return fail(MX_ERR_INVALID_ARG, "%s: c_dtype=%d is neither MX_BF16 nor MX_F32", fn,
                    c_dtype);
    if (K % 32 != 0 || K == 0)
        return fail(MX_ERR_SHAPE, "%s: K=%lld must be a positive multiple of 32", fn,
                    (long long)K);
    if (K % 128 != 0)
        return fail(MX_ERR_UNSUPPORTED, "%s: K=%lld: this build needs K %% 128 == 0", fn,
                    (long long)K);
    if (ld_a < K || ld_b < K || ld_c < N)
        return fail(MX_ERR_INVALID_ARG,
                    "%s: leading dimension too small (ld_a=%lld ld_b=%lld ld_c=%lld)", fn,
                    (long long)ld_a, (long long)ld_b, (long long)ld_c);
    if (M == 0 || N == 0)
        return MX_OK;
    if (!a_q || !a_s || !b_q || !b_s || !c)
        return fail(MX_ERR_INVALID_ARG, "%s: null pointer", fn);
    const uintptr_t ce = c_dtype == MX_BF16 ? 2 : 4;
    if (!aligned(a_q, 16) || !aligned(b_q, 16) || ld_a % 16 != 0 || ld_b % 16 != 0 ||
        !aligned(a_s, 4) || !aligned(b_s, 4) || !aligned(c, ce))
        return fail(MX_ERR_ALIGN,
                    "%s: operands need 16-byte aligned rows, scales 4-byte alignment, C its "
                    "element size",
                    fn);
    // Row offsets inside a 256-row tile (of A, B and C) and offsets into a
    // rearranged scale buffer are formed in 32 bits.
    if ((int64_t)256 * ld_a >= ((int64_t)1 << 31) || (int64_t)256 * ld_b >= ((int64_t)1 << 31) ||
        (int64_t)256 * ld_c * (int64_t)ce >= ((int64_t)1 << 31))
        return fail(MX_ERR_UNSUPPORTED, "%s: leading dimension too large for this build", fn);
    if (swz_bytes(M, K / 32) >= ((int64_t)1 << 32) || swz_bytes(N, K / 32) >= ((int64_t)1 << 32))
        return fail(MX_ERR_UNSUPPORTED, "%s: operand too large for this build", fn);
    return MX_OK;
}

int64_t mx_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int c_dtype)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0 || (c_dtype != MX_BF16 && c_dtype != MX_F32))
        return 0;
    return mx::gemm_workspace_bytes(M, N, K, c_dtype, true);
}

mx_status mx_gemm(int64_t M, int64_t N, int64_t K, const void *a_q, int64_t ld_a,
                  const void *a_s_swz, const void *b_q, int64_t ld_b, const void *b_s_swz,
                  void *c, int64_t ld_c, int c_dtype, void *workspace, int64_t workspace_bytes,
                  void *stream)
{
    const char *fn = "mx_gemm";
    mx_status st =
        check_gemm_common(fn, M, N, K, a_q, ld_a, a_s_swz, b_q, ld_b, b_s_swz, c, ld_c, c_dtype);
    if (st != MX_OK)
        return st;
    if (M == 0 || N == 0)
        return ok();
    const int64_t ce = c_dtype == MX_BF16 ? 2 : 4;
    const int64_t ec = extent(M, N, ld_c, ce);
    if (overlap(c, ec, a_q, extent(M, K, ld_a, 1)) || overlap(c, ec, b_q, extent(N, K, ld_b, 1)) ||
        overlap(c, ec, a_s_swz, swz_bytes(M, K / 32)) ||
        overlap(c, ec, b_s_swz, swz_bytes(N, K / 32)))
        return fail(MX_ERR_OVERLAP, "%s: C overlaps an input", fn);
    const void *bufs[5] = {a_q, b_q, a_s_swz, b_s_swz, c};
    const int64_t lens[5] = {extent(M, K, ld_a, 1), extent(N, K, ld_b, 1), swz_bytes(M, K / 32),
                             swz_bytes(N, K / 32), ec};
    const int64_t need = mx::gemm_workspace_bytes(M, N, K, c_dtype, mx::gemm_vec16(c, ld_c, c_dtype));
    st = check_workspace(fn, workspace, workspace_bytes, need, 16, bufs, lens, 5);
    if (st != MX_OK)
        return st;
    return hip_status(mx::launch_gemm(M, N, K, a_q, ld_a, a_s_swz, b_q, ld_b, b_s_swz, c, ld_c,
                                      c_dtype, workspace, (hipStream_t)stream),
                      fn);
}

mx_status mx_grouped_gemm(int64_t num_groups, int64_t M_total, int64_t N, int64_t K,
                          const int64_t *group_offsets, const void *a_q, int64_t ld_a,
                          const void *a_s_swz, const void *b_q, const void *b_s_swz, void *c,
                          int64_t ld_c, int c_dtype, void *stream)
{
    const char *fn = "mx_grouped_gemm";
    if (num_groups < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: num_groups=%lld < 1", fn, (long long)num_groups);
    if (num_groups > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_groups=%lld > %d", fn, (long long)num_groups,
                    mx::MOE_MAX_EXPERTS);
    mx_status st = check_gemm_common(fn, M_total, N, K, a_q, ld_a, a_s_swz, b_q, K, b_s_swz, c,
                                     ld_c, c_dtype);
    if (st != MX_OK)
        return st;
    if (M_total == 0 || N == 0)
        return ok();
    if (!group_offsets)
        return fail(MX_ERR_INVALID_ARG, "%s: null group_offsets", fn);
    if (!aligned(group_offsets, 8))
        return fail(MX_ERR_ALIGN, "%s: group_offsets must be 8-byte aligned", fn);
    // tile numbers are formed in 32 bits: the experts' row tiles (at most one
    // partial tile each) times the column tiles
    if (((M_total + 255) / 256 + num_groups) * ((N + 255) / 256) >= ((int64_t)1 << 31))
        return fail(MX_ERR_UNSUPPORTED, "%s: more than 2^31 - 1 output tiles", fn);
    const int64_t ce = c_dtype == MX_BF16 ? 2 : 4;
    const int64_t ec = extent(M_total, N, ld_c, ce);
    const int64_t eb = num_groups * N * K;
    const int64_t ebs = num_groups * swz_bytes(N, K / 32);
    if (overlap(c, ec, a_q, extent(M_total, K, ld_a, 1)) || overlap(c, ec, b_q, eb) ||
        overlap(c, ec, a_s_swz, swz_bytes(M_total, K / 32)) || overlap(c, ec, b_s_swz, ebs) ||
        overlap(c, ec, group_offsets, (num_groups + 1) * 8))
        return fail(MX_ERR_OVERLAP, "%s: C overlaps an input", fn);
    if (debug_checks() &&
        (st = debug_offsets(fn, "group_offsets", group_offsets, num_groups, M_total, 1, 0, true, true, stream)) !=
            MX_OK)
        return st;
    return hip_status(mx::launch_grouped_gemm(num_groups, M_total, N, K, group_offsets, a_q, ld_a,
                                              a_s_swz, b_q, b_s_swz, c, ld_c, c_dtype,
                                              (hipStream_t)stream),
                      fn);
}

mx_status mx_grouped_gemm_wgrad(int64_t num_groups, int64_t M, int64_t N, int64_t k_cap,
                                const int64_t *k_offsets, const void *a_q, int64_t ld_a,
                                const void *a_s_swz, const void *b_q, int64_t ld_b,
                                const void *b_s_swz, void *c, int64_t ld_c, int c_dtype, void *workspace,
                                int64_t workspace_bytes, void *stream)
{
    const char *fn = "mx_grouped_gemm_wgrad";
    if (num_groups < 1)
        return fail(MX_ERR_INVALID_ARG, "%s: num_groups=%lld < 1", fn, (long long)num_groups);
    if (num_groups > mx::MOE_MAX_EXPERTS)
        return fail(MX_ERR_UNSUPPORTED, "%s: num_groups=%lld > %d", fn, (long long)num_groups,
                    mx::MOE_MAX_EXPERTS);
    mx_status st = check_gemm_common(fn, M, N, k_cap, a_q, ld_a, a_s_swz, b_q, ld_b, b_s_swz, c, ld_c,
                                     c_dtype);
    if (st != MX_OK)
        return st;
    if (k_cap % 256 != 0)
        return fail(MX_ERR_SHAPE, "%s: k_cap=%lld must be a multiple of 256", fn, (long long)k_cap);
    if (M == 0 || N == 0)
        return ok();
    if (!k_offsets)
        return fail(MX_ERR_INVALID_ARG, "%s: null k_offsets", fn);
    if (!aligned(k_offsets, 8))
        return fail(MX_ERR_ALIGN, "%s: k_offsets must be 8-byte aligned", fn);
    const int64_t ce = c_dtype == MX_BF16 ? 2 : 4;
    if ((num_groups * M) * ld_c >= ((int64_t)1 << 62) / ce)
        return fail(MX_ERR_UNSUPPORTED, "%s: C too large", fn);
    if (num_groups * ((M + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 31))
        return fail(MX_ERR_UNSUPPORTED, "%s: more than 2^31 - 1 output tiles", fn);
    const int64_t ec = extent(num_groups * M, N, ld_c, ce);
    if (overlap(c, ec, a_q, extent(M, k_cap, ld_a, 1)) || overlap(c, ec, b_q, extent(N, k_cap, ld_b, 1)) ||
        overlap(c, ec, a_s_swz, swz_bytes(M, k_cap / 32)) || overlap(c, ec, b_s_swz, swz_bytes(N, k_cap / 32)) ||
        overlap(c, ec, k_offsets, (num_groups + 1) * 8))
        return fail(MX_ERR_OVERLAP, "%s: C overlaps an input", fn);
    const void *bufs[6] = {a_q, b_q, a_s_swz, b_s_swz, k_offsets, c};
    const int64_t lens[6] = {extent(M, k_cap, ld_a, 1), extent(N, k_cap, ld_b, 1), swz_bytes(M, k_cap / 32),
                             swz_bytes(N, k_cap / 32), (num_groups + 1) * 8, ec};
    st = check_workspace(fn, workspace, workspace_bytes, mx::WGRAD_WORKSPACE_BYTES, 4, bufs, lens, 6);
    if (st != MX_OK)
        return st;
    if (debug_checks() &&
        (st = debug_offsets(fn, "k_offsets", k_offsets, num_groups, k_cap, 256, 256, false, false, stream)) != MX_OK)
        return st;
    return hip_status(mx::launch_grouped_gemm_wgrad(num_groups, M, N, k_cap, k_offsets, a_q, ld_a, a_s_swz,
                                                    b_q, ld_b, b_s_swz, c, ld_c, c_dtype, workspace,
                                                    (hipStream_t)stream),
                      fn);
}

int64_t mx_grouped_gemm_wgrad_workspace_bytes(void) { return mx::WGRAD_WORKSPACE_BYTES; }

}  // extern "C"
