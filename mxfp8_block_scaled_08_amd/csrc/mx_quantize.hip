// MXFP8 quantization kernels for gfx950: BF16 -> E4M3 elements + E8M0 scales.
//
// "MXFP8 quantization" is one of the three kernel categories the MXFP8 RL
// paper ("End-to-End MXFP8 Reinforcement Learning on Blackwell", Table 6)
// adds to a micro-batch; Figure 1 has the same quantizer produce the weights
// synchronized to the sampler.  Both kernels are HBM-bound: 2 bytes are read
// and 1 + 1/32 bytes written per element, so they are built around 128-bit
// coalesced loads, in-register encoding and wide stores.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

// ---------------------------------------------------------------------------
// Row-wise: each lane owns 8 consecutive BF16 (one 16-byte load); the four
// lanes of a DPP quad own one 32-element block.  The block maximum is two
// quad-permute steps; lane 0 of the quad stores the scale byte.  Every wave
// reads 1 KiB contiguous per load and writes 512 B of codes per store.
// UNROLL independent units per lane keep enough loads in flight to cover
// HBM latency.

constexpr int QR_THREADS = 256;
constexpr int QR_UNROLL = 4;

template <bool CONTIG>
__global__ __launch_bounds__(QR_THREADS) void quantize_rowwise_kernel(
    const uint16_t *__restrict__ x, int64_t ld_x, uint8_t *__restrict__ q, int64_t ld_q,
    uint8_t *__restrict__ s, int64_t ld_s, int64_t units, uint32_t units_per_row)
{
    const int64_t per_block = (int64_t)QR_THREADS * QR_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * per_block + threadIdx.x; base < units;
         base += (int64_t)gridDim.x * per_block) {
        uint4 v[QR_UNROLL];
        int64_t xo[QR_UNROLL];
#pragma unroll
        for (int i = 0; i < QR_UNROLL; i++) {
            int64_t u = base + (int64_t)i * QR_THREADS;
            if (CONTIG) {
                xo[i] = u * 8;
            } else {
                int64_t row = u / units_per_row;
                int64_t cu = u - row * units_per_row;
                xo[i] = row * ld_x + cu * 8;
            }
            if (u < units)
                v[i] = *reinterpret_cast<const uint4 *>(x + xo[i]);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < QR_UNROLL; i++) {
            int64_t u = base + (int64_t)i * QR_THREADS;
            // units is a multiple of 4 and u % 4 == lane % 4, so a quad is
            // either entirely in range or entirely out of it.
            uint32_t m = max_mag_x8(v[i]);
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false)); // [1,0,3,2]
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false)); // [2,3,0,1]
            if (u >= units)
                continue;
            uint32_t c = scale_code(m);
            uint2 out = e4m3_x8(v[i], (int)c, c == 0xFFu);
            int64_t qo, so;
            if (CONTIG) {
                qo = u * 8;
                so = u >> 2;
            } else {
                int64_t row = u / units_per_row;
                int64_t cu = u - row * units_per_row;
                qo = row * ld_q + cu * 8;
                so = row * ld_s + (cu >> 2);
            }
            *reinterpret_cast<uint2 *>(q + qo) = out;
            if ((threadIdx.x & 3) == 0)
                s[so] = (uint8_t)c;
        }
    }
}

// ---------------------------------------------------------------------------
// Column-wise: a workgroup quantizes a tile of 128 rows x 256 columns.  The
// tile is read with 16-byte row-contiguous loads into LDS; then thread j owns
// column j of the tile, reads its 128 values down the column (consecutive
// lanes read consecutive LDS halfwords: no bank conflicts), and writes the
// four 32-element blocks as 128 contiguous bytes of the transposed output
// row qt[col][...] plus four scale bytes.

constexpr int QC_THREADS = 256;
constexpr int QC_ROWS = 128;
constexpr int QC_COLS = 256;

__global__ __launch_bounds__(QC_THREADS) void quantize_colwise_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t *__restrict__ qt, int64_t ld_qt, uint8_t *__restrict__ st, int64_t ld_st,
    int64_t tiles_c)
{
    __shared__ uint16_t tile[QC_ROWS][QC_COLS];
    const int64_t tr = blockIdx.x / tiles_c;
    const int64_t tc = blockIdx.x - tr * tiles_c;
    const int64_t r0 = tr * QC_ROWS, c0 = tc * QC_COLS;
    const int nrows = (int)min((int64_t)QC_ROWS, rows - r0);  // multiple of 32
    const int ncols = (int)min((int64_t)QC_COLS, cols - c0);  // multiple of 8
    const int tid = threadIdx.x;

    // load: 8 rows x 256 columns per pass, 16 passes
    {
        const int col8 = tid & 31;
        const int rsub = tid >> 5;
        uint4 v[QC_ROWS / 8];
#pragma unroll
        for (int p = 0; p < QC_ROWS / 8; p++) {
            int r = p * 8 + rsub;
            if (r < nrows && col8 * 8 < ncols)
                v[p] = *reinterpret_cast<const uint4 *>(x + (r0 + r) * ld_x + c0 + col8 * 8);
            else
                v[p] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < QC_ROWS / 8; p++)
            *reinterpret_cast<uint4 *>(&tile[p * 8 + rsub][col8 * 8]) = v[p];
    }
    __syncthreads();

    const int j = tid;
    if (j >= ncols)
        return;
    uint8_t *qrow = qt + (c0 + j) * ld_qt + r0;
    uint8_t *srow = st + (c0 + j) * ld_st + r0 / 32;
    for (int b = 0; b < nrows / 32; b++) {
        uint32_t w[16];
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            uint32_t lo = tile[32 * b + 2 * i][j];
            uint32_t hi = tile[32 * b + 2 * i + 1][j];
            w[i] = lo | (hi << 16);
            m = max(m, max(lo & 0x7FFFu, hi & 0x7FFFu));
        }
        uint32_t c = scale_code(m);
        uint32_t o[8];
        if (c == 0xFFu) {
#pragma unroll
            for (int i = 0; i < 8; i++)
                o[i] = 0x7F7F7F7Fu;
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++)
                o[i] = e4m3_pair(w[2 * i], (int)c) | (e4m3_pair(w[2 * i + 1], (int)c) << 16);
        }
        uint4 *dst = reinterpret_cast<uint4 *>(qrow + 32 * b);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        srow[b] = (uint8_t)c;
    }
}

// ---------------------------------------------------------------------------
// Scale rearrangement: one thread writes one 4-byte word of the GEMM layout
// (word w of tile (rt, kt) holds, for row 32rt + w%32, the scales of blocks
// 8kt + h, +2, +4, +6 with h = w/32), padding with 0x7F.

constexpr int SW_THREADS = 256;

__global__ __launch_bounds__(SW_THREADS) void scale_swizzle_kernel(
    const uint8_t *__restrict__ s, int64_t rows, int64_t kblocks, int64_t ld_s,
    uint32_t *__restrict__ out, int64_t words, int64_t KT)
{
    for (int64_t d = (int64_t)blockIdx.x * SW_THREADS + threadIdx.x; d < words;
         d += (int64_t)gridDim.x * SW_THREADS) {
        int64_t tile = d >> 6;
        int lane = (int)(d & 63);
        int h = lane >> 5, r = lane & 31;
        int64_t rt = tile / KT, kt = tile - rt * KT;
        int64_t row = rt * 32 + r;
        uint32_t word = 0;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            int64_t blk = kt * 8 + 2 * t + h;
            uint32_t byte = (row < rows && blk < kblocks) ? s[row * ld_s + blk] : 0x7Fu;
            word |= byte << (8 * t);
        }
        out[d] = word;
    }
}

// ---------------------------------------------------------------------------
// launchers (arguments already validated by the C ABI layer)

hipError_t launch_quantize_rowwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *q, int64_t ld_q, void *s, int64_t ld_s,
                                   hipStream_t stream)
{
    int64_t units = rows * (cols / 8);
    uint32_t upr = (uint32_t)(cols / 8);
    int64_t per_block = (int64_t)QR_THREADS * QR_UNROLL;
    int64_t blocks = (units + per_block - 1) / per_block;
    int64_t max_blocks = 256 * 8 * 4;  // grid-stride beyond ~4 waves of work per CU
    if (blocks > max_blocks)
        blocks = max_blocks;
    bool contig = (ld_x == cols) && (ld_q == cols) && (ld_s == cols / 32);
    if (contig)
        hipLaunchKernelGGL(quantize_rowwise_kernel<true>, dim3((unsigned)blocks), dim3(QR_THREADS),
                           0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q, ld_q, (uint8_t *)s,
                           ld_s, units, upr);
    else
        hipLaunchKernelGGL(quantize_rowwise_kernel<false>, dim3((unsigned)blocks),
                           dim3(QR_THREADS), 0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q,
                           ld_q, (uint8_t *)s, ld_s, units, upr);
    return hipGetLastError();
}

hipError_t launch_quantize_colwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *qt, int64_t ld_qt, void *st, int64_t ld_st,
                                   hipStream_t stream)
{
    int64_t tiles_r = (rows + QC_ROWS - 1) / QC_ROWS;
    int64_t tiles_c = (cols + QC_COLS - 1) / QC_COLS;
    hipLaunchKernelGGL(quantize_colwise_kernel, dim3((unsigned)(tiles_r * tiles_c)),
                       dim3(QC_THREADS), 0, stream, (const uint16_t *)x, rows, cols, ld_x,
                       (uint8_t *)qt, ld_qt, (uint8_t *)st, ld_st, tiles_c);
    return hipGetLastError();
}

hipError_t launch_scale_swizzle(const void *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                                void *s_swz, hipStream_t stream)
{
    int64_t KT = (kblocks + 7) / 8;
    int64_t words = ((rows + 31) / 32) * KT * 64;
    int64_t blocks = (words + SW_THREADS - 1) / SW_THREADS;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(scale_swizzle_kernel, dim3((unsigned)blocks), dim3(SW_THREADS), 0, stream,
                       (const uint8_t *)s, rows, kblocks, ld_s, (uint32_t *)s_swz, words, KT);
    return hipGetLastError();
}

}  // namespace mx
