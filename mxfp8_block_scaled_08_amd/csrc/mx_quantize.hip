// MXFP8 quantization kernels for gfx950: BF16 -> E4M3 elements + E8M0 scales.
//
// "MXFP8 quantization" is one of the three kernel categories the MXFP8 RL
// paper ("End-to-End MXFP8 Reinforcement Learning on Blackwell", Table 6)
// adds to a micro-batch; Figure 1 has the same quantizer produce the weights
// synchronized to the sampler.  The kernels are HBM-bound: 2 bytes are read
// and 1 + 1/32 bytes written per element and orientation, so they are built
// around 128-bit coalesced loads, in-register encoding and wide stores, with
// the non-temporal cache policy on every streaming access (mx_device.h).
// Measured on MI355X over 1 GiB: row-wise passes reach about 5.9 TB/s on any
// shape; passes that write a transposed output (column-wise, dual) 4.8-5.3
// TB/s, the less the wider the matrix (each workgroup reads 256-512 bytes
// of each of its rows).
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

// ---------------------------------------------------------------------------
// Row-wise: each lane owns 8 consecutive BF16 (one 16-byte load); the four
// lanes of a DPP quad own one 32-element block.  The block maximum is two
// quad-permute steps; lane 0 of the quad stores the scale byte.  Every wave
// reads 1 KiB contiguous per load and writes 512 B of codes per store.
// UNROLL independent units per lane keep enough loads in flight to cover
// HBM latency.  SWZ: the scale byte goes straight to its place in the GEMM's
// rearranged layout (ld_s then holds the tiles per 32-row tile row), which
// saves the separate rearrangement pass.

constexpr int QR_THREADS = 256;
constexpr int QR_UNROLL = 4;

// The units base, base + QR_THREADS, .. (QR_UNROLL of them) of one tensor.
template <bool CONTIG, bool SWZ>
__device__ __forceinline__ void quantize_rowwise_units(const uint16_t *__restrict__ x, int64_t ld_x,
                                                       uint8_t *__restrict__ q, int64_t ld_q,
                                                       uint8_t *__restrict__ s, int64_t ld_s,
                                                       int64_t units, uint32_t units_per_row,
                                                       int64_t base)
{
    {
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
                v[i] = ld_stream(x + xo[i]);
            else
                v[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < QR_UNROLL; i++) {
            int64_t u = base + (int64_t)i * QR_THREADS;
            // units is a multiple of 4 and u % 4 == lane % 4, so a quad is
            // either entirely in range or entirely out of it.
            const uint4 &w = v[i];
            uint32_t m = pk_max_u16(pk_max_u16(mag2(w.x), mag2(w.y)), pk_max_u16(mag2(w.z), mag2(w.w)));
            m = max(m & 0xFFFFu, m >> 16);
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false)); // [1,0,3,2]
            m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false)); // [2,3,0,1]
            if (u >= units)
                continue;
            const uint32_t c = scale_code(m);
            const float sc = cvt_scale(c);
            uint2 out;
            out.x = nan_block_select(cvt_x4(w.x, w.y, sc), c);
            out.y = nan_block_select(cvt_x4(w.z, w.w, sc), c);
            int64_t qo, so;
            if (CONTIG && !SWZ) {
                qo = u * 8;
                so = u >> 2;
            } else {
                int64_t row = u / units_per_row;
                int64_t cu = u - row * units_per_row;
                qo = CONTIG ? u * 8 : row * ld_q + cu * 8;
                if (SWZ) {
                    const int64_t b = cu >> 2;  // 32-element block of the row
                    so = ((row >> 5) * ld_s + (b >> 3)) * 256 + (32 * (b & 1) + (row & 31)) * 4 + ((b & 7) >> 1);
                } else {
                    so = row * ld_s + (cu >> 2);
                }
            }
            st_stream(q + qo, out);
            if ((threadIdx.x & 3) == 0)
                s[so] = (uint8_t)c;
        }
    }
}

template <bool CONTIG, bool SWZ>
__global__ __launch_bounds__(QR_THREADS) void quantize_rowwise_kernel(
    const uint16_t *__restrict__ x, int64_t ld_x, uint8_t *__restrict__ q, int64_t ld_q,
    uint8_t *__restrict__ s, int64_t ld_s, int64_t units, uint32_t units_per_row)
{
    const int64_t per_block = (int64_t)QR_THREADS * QR_UNROLL;
    for (int64_t base = (int64_t)blockIdx.x * per_block + threadIdx.x; base < units;
         base += (int64_t)gridDim.x * per_block)
        quantize_rowwise_units<CONTIG, SWZ>(x, ld_x, q, ld_q, s, ld_s, units, units_per_row, base);
}

// Several tensors in one launch, scales rearranged: job j takes workgroups
// first[j] .. first[j+1] - 1, each QR_THREADS * QR_UNROLL units of its
// tensor (the forward activations of a layer in one launch instead of one
// small launch each).
struct RowBatch {
    RowJob job[QR_MAX_JOBS];
    int64_t first[QR_MAX_JOBS + 1];
    int n;
};

__global__ __launch_bounds__(QR_THREADS) void quantize_rowwise_batch_kernel(RowBatch B)
{
    int j = 0;
    while (j + 1 < B.n && (int64_t)blockIdx.x >= B.first[j + 1])
        j++;
    const RowJob &J = B.job[j];
    const int64_t units = J.rows * (J.cols / 8);
    const int64_t base = ((int64_t)blockIdx.x - B.first[j]) * (QR_THREADS * QR_UNROLL) + threadIdx.x;
    quantize_rowwise_units<false, true>((const uint16_t *)J.x, J.ld_x, (uint8_t *)J.q, J.ld_q,
                                        (uint8_t *)J.s_swz, J.s_tiles, units, (uint32_t)(J.cols / 8), base);
}

// ---------------------------------------------------------------------------
// Column-wise: a block is 32 consecutive rows of one column, and the output is
// transposed (qt[col][row], st[col][row / 32]).  No LDS: each wave covers a
// 128-row x 64-column tile; lane = 16 * rb + 8 * half + cg owns columns
// c0 .. c0+7 (cg selects the 8-column group) and rows 16 * half .. +15 of row
// block rb.  Every load is a 16-byte vector of 8 columns (eight lanes read one
// 128-byte line of a row).  The lane's packed per-column maxima over its 16
// rows are combined with the other half of the block by a DPP rotation of 8
// within each 16-lane row (lane ^ 8).  v_perm pairs two rows of one column in
// a word for the scaled conversion, so the lane's 16 codes of a column form
// one 16-byte store, and the eight lanes of a column write one full 128-byte
// line of qt.  Four waves side by side make a 128 x 256 workgroup tile.
//
// Tile order.  Workgroup b runs on XCD b mod 8.  For a wide matrix (at least
// QC_WIDE column tiles) XCD x takes a contiguous range of tiles numbered in
// groups of QC_GROUP_R tile-rows (tile-row fastest), so the tiles it runs
// together form a compact block: long contiguous runs of both the rows of x
// it reads and the rows of qt it writes (12288 x 24576: 4.3 -> 4.9 TB/s).
// Otherwise tiles go in row-major order, which gives XCD x the column tiles
// c = x (mod 8): for a tall matrix of few column tiles each XCD then writes
// whole rows of qt in sequence (196608 x 2048: 4.95 TB/s against 4.6 with
// the grouped order).

constexpr int QC_THREADS = 256;
constexpr int QC_TILE_R = 128;
constexpr int QC_TILE_C = 256;
constexpr int QC_WIDE = 32;
constexpr int QC_GROUP_R = 32;

// SWZ: each scale byte goes straight to its place in the rearranged layout
// of the [cols][rows/32] scales (ld_st then holds the tiles per 32-column
// tile row), which saves the separate rearrangement pass.
template <bool SWZ>
__global__ __launch_bounds__(QC_THREADS) void quantize_colwise_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    uint8_t *__restrict__ qt, int64_t ld_qt, uint8_t *__restrict__ st, int64_t ld_st,
    int64_t tiles_r, int64_t tiles_c)
{
    const int lane = threadIdx.x & 63;
    const int cg = lane & 7, half = (lane >> 3) & 1, rb = lane >> 4;
    int64_t tr, tc;
    if (tiles_c >= QC_WIDE) {
        // the grid is a multiple of 8; numbers past the last tile do nothing
        const int64_t t = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
        if (t >= tiles_r * tiles_c)
            return;
        const int64_t per_group = QC_GROUP_R * tiles_c;
        const int64_t grp = t / per_group, first = grp * QC_GROUP_R;
        const int64_t gr = min(tiles_r - first, (int64_t)QC_GROUP_R);
        const int64_t in = t - grp * per_group;
        tr = first + in % gr;
        tc = in / gr;
    } else {
        tr = blockIdx.x / tiles_c;
        tc = blockIdx.x - tr * tiles_c;
    }
    const int64_t c0 = tc * QC_TILE_C + (threadIdx.x >> 6) * 64 + cg * 8;
    const int64_t r0 = tr * QC_TILE_R + rb * 32 + half * 16;
    // rows % 32 == 0 and cols % 8 == 0: a lane's rows and columns are either
    // all in range or all out of it, and both halves of a block agree.
    const bool active = c0 < cols && r0 < rows;
    // Lanes out of range read rows 0..15 of column group 0 (present whenever
    // the grid is not empty) and store nothing; their DPP partner lane ^ 8 is
    // out of range too, so those values never reach a stored block.
    const uint16_t *src = x + (active ? r0 * ld_x + c0 : 0);
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; i++)
        v[i] = ld_stream(src + i * ld_x);
    // packed maxima of columns (0,1), (2,3), (4,5), (6,7)
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; i++) {
        m[0] = pk_max_u16(m[0], mag2(v[i].x));
        m[1] = pk_max_u16(m[1], mag2(v[i].y));
        m[2] = pk_max_u16(m[2], mag2(v[i].z));
        m[3] = pk_max_u16(m[3], mag2(v[i].w));
    }
#pragma unroll
    for (int k = 0; k < 4; k++)  // row_ror:8 - the other half of the block
        m[k] = pk_max_u16(m[k], (uint32_t)__builtin_amdgcn_mov_dpp((int)m[k], 0x128, 0xF, 0xF, false));
    if (!active)
        return;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t c = scale_code((m[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        const float sc = cvt_scale(c);
        // bytes 0,1 (column j even) or 2,3 (odd) of the row pair's words
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint4 &a = v[4 * k], &b = v[4 * k + 1], &cc = v[4 * k + 2], &d = v[4 * k + 3];
            const int wi = j >> 1;
            const uint32_t wa = wi == 0 ? a.x : wi == 1 ? a.y : wi == 2 ? a.z : a.w;
            const uint32_t wb = wi == 0 ? b.x : wi == 1 ? b.y : wi == 2 ? b.z : b.w;
            const uint32_t wc = wi == 0 ? cc.x : wi == 1 ? cc.y : wi == 2 ? cc.z : cc.w;
            const uint32_t wd = wi == 0 ? d.x : wi == 1 ? d.y : wi == 2 ? d.z : d.w;
            const uint32_t p01 = __builtin_amdgcn_perm(wb, wa, sel);  // rows 4k, 4k+1
            const uint32_t p23 = __builtin_amdgcn_perm(wd, wc, sel);  // rows 4k+2, 4k+3
            o[k] = nan_block_select(cvt_x4(p01, p23, sc), c);
        }
        st_stream(qt + (c0 + j) * ld_qt + r0, make_uint4(o[0], o[1], o[2], o[3]));
        if (half == 0) {
            const int64_t col = c0 + j, b = r0 >> 5;  // scale row and 32-element block
            if (SWZ)
                st[((col >> 5) * ld_st + (b >> 3)) * 256 + (32 * (b & 1) + (col & 31)) * 4 + ((b & 7) >> 1)] =
                    (uint8_t)c;
            else
                st[col * ld_st + b] = (uint8_t)c;
        }
    }
}

// ---------------------------------------------------------------------------
// Both orientations in one pass, scales straight into the rearranged layout
// (the weight-sync pair: the row-wise operand of the forward product and the
// column-wise one of the backward product from one read of the BF16 weight).
// A 512-thread workgroup takes a 256 x 256 tile as 2 x 4 waves of the
// column-wise kernel's 128 x 64 wave tile, so the column-wise half is that
// kernel's.  Row-wise, lane (rb, half, cg) holds 8 columns of 16 rows; the
// four lanes cg & ~3 .. | 3 of a row hold one 32-column block, whose maximum
// they combine by two DPP quad exchanges; each lane converts its 8 elements
// of each row into LDS (8 bytes), and after the workgroup's barrier sixteen
// threads write each row's 256 codes as two whole 128-byte lines (the
// lanes' own 8-byte stores left half lines, 5.31 TB/s).  The tile's scales are exactly 8 rearranged 256-byte tiles per
// orientation (256 rows x 8 blocks row-wise, 256 columns x 8 blocks
// column-wise): the codes are placed in LDS at their rearranged positions
// (byte (32h + r) * 4 + t of tile r / 32 for block 2t + h, the layout of
// mx_scale_swizzle), the rest left 0x7F, and each thread then stores one
// word of each, 256 contiguous bytes per tile.

constexpr int QD_THREADS = 512;
constexpr int QD_TILE = 256;

// Several tensors in one launch (a layer's weights): job j takes blocks
// first[j] .. first[j+1] - 1, each tensor's count a multiple of 8 when it uses
// the per-XCD order, so a block's XCD is still its number mod 8.  A job may
// stand for several tensors of one shape at fixed strides (stacked expert
// weights): tensor i takes the i-th equal run of the job's blocks.
struct DualBatch {
    DualJob job[QD_MAX_JOBS];
    int64_t first[QD_MAX_JOBS + 1];
    int n;
};

__global__ __launch_bounds__(QD_THREADS) void quantize_dual_kernel(DualBatch B)
{
    __shared__ uint32_t lds_s[8 * 64];   // row-wise scales: 8 rearranged tiles
    __shared__ uint32_t lds_st[8 * 64];  // column-wise scales: 8 rearranged tiles
    __shared__ __attribute__((aligned(16))) uint8_t lds_q[QD_TILE * QD_TILE];  // row-wise codes
    int jb = 0;
    while (jb + 1 < B.n && (int64_t)blockIdx.x >= B.first[jb + 1])
        jb++;
    const DualJob &J = B.job[jb];
    // a job of count tensors takes count equal runs of nb blocks
    const int64_t nb = (B.first[jb + 1] - B.first[jb]) / J.count;
    int64_t b = (int64_t)blockIdx.x - B.first[jb];
    const int64_t item = b / nb;
    b -= item * nb;
    const uint16_t *__restrict__ x = (const uint16_t *)J.x + item * J.x_stride;
    const int64_t rows = J.rows, cols = J.cols, ld_x = J.ld_x;
    uint8_t *__restrict__ q = (uint8_t *)J.q + item * J.q_stride;
    uint8_t *__restrict__ s_swz = (uint8_t *)J.s_swz + item * J.s_stride;
    uint8_t *__restrict__ qt = (uint8_t *)J.qt + item * J.qt_stride;
    uint8_t *__restrict__ st_swz = (uint8_t *)J.st_swz + item * J.st_stride;
    const int64_t ld_q = J.ld_q, s_tiles = J.s_tiles, ld_qt = J.ld_qt, st_tiles = J.st_tiles;
    const int64_t tiles_r = (rows + QD_TILE - 1) / QD_TILE, tiles_c = (cols + QD_TILE - 1) / QD_TILE;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 2, wc = wave & 3;
    const int cg = lane & 7, half = (lane >> 3) & 1, rb = lane >> 4;
    int64_t tr, tc;
    if (tiles_c >= QC_WIDE) {
        // XCD x (block b on XCD b mod 8) takes the x-th contiguous eighth of
        // the tiles in row-major order (against the column-wise kernel's
        // tile-row-fastest groups: 250 -> 244 us on a 12288 x 24576 tensor)
        const int64_t t = (b & 7) * (nb >> 3) + (b >> 3);
        if (t >= tiles_r * tiles_c)
            return;
        tr = t / tiles_c;
        tc = t - tr * tiles_c;
    } else {
        tr = b / tiles_c;
        tc = b - tr * tiles_c;
    }
    const int64_t R0 = tr * QD_TILE, C0 = tc * QD_TILE;
    const int64_t c0 = C0 + wc * 64 + cg * 8;
    const int64_t r0 = R0 + wr * 128 + rb * 32 + half * 16;
    // rows % 32 == 0 and cols % 32 == 0: a lane's rows and columns are all in
    // range or all out, and so are its DPP partners (the other half of its
    // column block, the other lanes of its row block)
    const bool active = c0 < cols && r0 < rows;
    lds_s[tid] = 0x7F7F7F7Fu;
    lds_st[tid] = 0x7F7F7F7Fu;
    const uint16_t *src = x + (active ? r0 * ld_x + c0 : 0);
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; i++)
        v[i] = ld_stream(src + i * ld_x);
    // column-wise maxima (per column, the lane's 16 rows) and row-wise ones
    // (per row, the lane's 8 columns) in one pass, each magnitude used by
    // both as soon as it is formed (two passes keep all 64 magnitudes live)
    uint32_t m[4] = {0, 0, 0, 0};
    uint32_t rmax[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t ax = mag2(v[i].x), ay = mag2(v[i].y), az = mag2(v[i].z), aw = mag2(v[i].w);
        m[0] = pk_max_u16(m[0], ax);
        m[1] = pk_max_u16(m[1], ay);
        m[2] = pk_max_u16(m[2], az);
        m[3] = pk_max_u16(m[3], aw);
        const uint32_t w = pk_max_u16(pk_max_u16(ax, ay), pk_max_u16(az, aw));
        rmax[i] = max(w & 0xFFFFu, w >> 16);
    }
#pragma unroll
    for (int k = 0; k < 4; k++)  // row_ror:8 - the other half of the column block
        m[k] = pk_max_u16(m[k], (uint32_t)__builtin_amdgcn_mov_dpp((int)m[k], 0x128, 0xF, 0xF, false));
    // a row's 32-column block is the lane's quad: quad_perm [1,0,3,2] and
    // [2,3,0,1]
#pragma unroll
    for (int i = 0; i < 16; i++) {
        uint32_t a = rmax[i];
        a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, false));
        a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xF, 0xF, false));
        rmax[i] = a;
    }
    __syncthreads();  // the 0x7F fill precedes every scale byte
    uint8_t *bs = reinterpret_cast<uint8_t *>(lds_s);
    uint8_t *bst = reinterpret_cast<uint8_t *>(lds_st);
    // the tile's 256 rows of qt from column R0 as one buffer range (256 ld_qt
    // < 2^32): column j of the lane is row j ld_qt past its first
    const __amdgpu_buffer_rsrc_t rq = byte_range(qt + C0 * ld_qt + R0, (uint32_t)(QD_TILE * ld_qt));
    const uint32_t qoff = (uint32_t)((wc * 64 + cg * 8) * ld_qt + wr * 128 + rb * 32 + half * 16);
    if (active) {
        // column-wise, as quantize_colwise_kernel
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const uint32_t c = scale_code((m[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            const float sc = cvt_scale(c);
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint4 &a = v[4 * k], &b = v[4 * k + 1], &cc = v[4 * k + 2], &d = v[4 * k + 3];
                const int wi = j >> 1;
                const uint32_t wa = wi == 0 ? a.x : wi == 1 ? a.y : wi == 2 ? a.z : a.w;
                const uint32_t wb = wi == 0 ? b.x : wi == 1 ? b.y : wi == 2 ? b.z : b.w;
                const uint32_t wcw = wi == 0 ? cc.x : wi == 1 ? cc.y : wi == 2 ? cc.z : cc.w;
                const uint32_t wd = wi == 0 ? d.x : wi == 1 ? d.y : wi == 2 ? d.z : d.w;
                const uint32_t p01 = __builtin_amdgcn_perm(wb, wa, sel);
                const uint32_t p23 = __builtin_amdgcn_perm(wd, wcw, sel);
                o[k] = nan_block_select(cvt_x4(p01, p23, sc), c);
            }
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u_t, make_uint4(o[0], o[1], o[2], o[3])), rq,
                                                   qoff, (int)(j * ld_qt), STREAM);
            if (half == 0) {
                // rearranged row = column wc*64 + cg*8 + j of the tile, block wr*4 + rb
                const int col = wc * 64 + cg * 8 + j, blk = wr * 4 + rb;
                bst[(col >> 5) * 256 + (32 * (blk & 1) + (col & 31)) * 4 + (blk >> 1)] = (uint8_t)c;
            }
        }
        // row-wise
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t c = scale_code(rmax[i]);
            const float sc = cvt_scale(c);
            const uint32_t o0 = nan_block_select(cvt_x4(v[i].x, v[i].y, sc), c);
            const uint32_t o1 = nan_block_select(cvt_x4(v[i].z, v[i].w, sc), c);
            *reinterpret_cast<uint2 *>(&lds_q[(wr * 128 + rb * 32 + half * 16 + i) * QD_TILE + wc * 64 + cg * 8]) =
                make_uint2(o0, o1);
            if ((cg & 3) == 0) {
                // rearranged row = tile row wr*128 + rb*32 + half*16 + i, block wc*2 + cg/4
                const int row = wr * 128 + rb * 32 + half * 16 + i, blk = wc * 2 + (cg >> 2);
                bs[(row >> 5) * 256 + (32 * (blk & 1) + (row & 31)) * 4 + (blk >> 1)] = (uint8_t)c;
            }
        }
    }
    __syncthreads();
    // row-wise codes out of LDS: 16 threads per row of the tile, 16 bytes
    // each, so every store instruction writes whole 128-byte lines (rows and
    // columns past the tensor: rows % 32 == 0 and cols % 32 == 0, so a
    // 16-byte chunk is all inside or all outside)
    {
        // (one buffer range over the tile's rows that exist, 256 ld_q < 2^32)
        const __amdgpu_buffer_rsrc_t rr =
            byte_range(q + R0 * ld_q + C0, (uint32_t)(min(rows - R0, (int64_t)QD_TILE) * ld_q));
#pragma unroll
        for (int k = 0; k < QD_TILE * QD_TILE / 16 / QD_THREADS; k++) {
            const int idx = tid + k * QD_THREADS;
            const int r = idx >> 4, ch = idx & 15;
            if (C0 + ch * 16 < cols)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(v4u_t, *reinterpret_cast<const uint4 *>(&lds_q[r * QD_TILE + ch * 16])), rr,
                    (uint32_t)(r * ld_q + ch * 16), 0, STREAM);
        }
    }
    // thread -> word tid & 63 of rearranged tile tid >> 6 (its 32-row tile
    // row of each orientation; the tile's 8 blocks are this tile's 256-K group)
    const int t = tid >> 6, w = tid & 63;
    if (R0 + 32 * t < rows)
        reinterpret_cast<uint32_t *>(s_swz + ((R0 / 32 + t) * s_tiles + C0 / 256) * 256)[w] = lds_s[tid];
    if (C0 + 32 * t < cols)
        reinterpret_cast<uint32_t *>(st_swz + ((C0 / 32 + t) * st_tiles + R0 / 256) * 256)[w] = lds_st[tid];
}

// Scale rearrangement.  A half-wave takes one 32-row tile row rt and a run of
// up to SW_KT consecutive 256-K groups kt; lane r owns row 32rt + r.  Per
// group the lane reads the row's 8 scale bytes (blocks 8kt .. 8kt+7) as one
// 8-byte load and splits them with v_perm into the word of lane slot r
// (blocks 8kt, +2, +4, +6) and of slot 32 + r (blocks 8kt+1, +3, +5, +7); the
// 32 lanes then write each 128-byte half of the tile with one store each.
// Rows past the tensor and blocks past kblocks are the 0x7F padding.  The
// 8-byte path needs 8-byte aligned scale rows; otherwise bytes are read one
// at a time.

constexpr int SW_THREADS = 256;
constexpr int SW_KT = 4;  // 256-K groups per half-wave

template <bool ALIGNED8>
__global__ __launch_bounds__(SW_THREADS) void scale_swizzle_kernel(
    const uint8_t *__restrict__ s, int64_t rows, int64_t kblocks, int64_t ld_s,
    uint32_t *__restrict__ out, int64_t KT, int64_t runs, int64_t halves)
{
    const int64_t hw = ((int64_t)blockIdx.x * SW_THREADS + threadIdx.x) >> 5;
    if (hw >= halves)
        return;
    const int r = threadIdx.x & 31;
    const int64_t rt = hw / runs;
    const int64_t kt0 = (hw - rt * runs) * SW_KT;
    const int64_t row = rt * 32 + r;
    const bool row_ok = row < rows;
    const uint8_t *srow = s + (row_ok ? row : 0) * ld_s;
#pragma unroll
    for (int u = 0; u < SW_KT; u++) {
        const int64_t kt = kt0 + u;
        if (kt >= KT)
            break;
        uint32_t lo = 0x7F7F7F7Fu, hi = 0x7F7F7F7Fu;
        if (row_ok) {
            if (ALIGNED8 && 8 * kt + 8 <= kblocks) {
                const uint2 v = *reinterpret_cast<const uint2 *>(srow + 8 * kt);
                lo = v.x;
                hi = v.y;
            } else {
                uint32_t b[8];
#pragma unroll
                for (int e = 0; e < 8; e++)
                    b[e] = 8 * kt + e < kblocks ? srow[8 * kt + e] : 0x7Fu;
                lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
            }
        }
        uint32_t *tile = out + (rt * KT + kt) * 64;
        tile[r] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);       // blocks 0, 2, 4, 6
        tile[32 + r] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);  // blocks 1, 3, 5, 7
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
        hipLaunchKernelGGL((quantize_rowwise_kernel<true, false>), dim3((unsigned)blocks), dim3(QR_THREADS),
                           0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q, ld_q, (uint8_t *)s,
                           ld_s, units, upr);
    else
        hipLaunchKernelGGL((quantize_rowwise_kernel<false, false>), dim3((unsigned)blocks),
                           dim3(QR_THREADS), 0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q,
                           ld_q, (uint8_t *)s, ld_s, units, upr);
    return hipGetLastError();
}

hipError_t launch_quantize_rowwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                       void *q, int64_t ld_q, void *s_swz, int64_t s_tiles,
                                       hipStream_t stream)
{
    int64_t units = rows * (cols / 8);
    uint32_t upr = (uint32_t)(cols / 8);
    int64_t per_block = (int64_t)QR_THREADS * QR_UNROLL;
    int64_t blocks = (units + per_block - 1) / per_block;
    int64_t max_blocks = 256 * 8 * 4;
    if (blocks > max_blocks)
        blocks = max_blocks;
    bool contig = (ld_x == cols) && (ld_q == cols);
    if (contig)
        hipLaunchKernelGGL((quantize_rowwise_kernel<true, true>), dim3((unsigned)blocks), dim3(QR_THREADS),
                           0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q, ld_q, (uint8_t *)s_swz,
                           s_tiles, units, upr);
    else
        hipLaunchKernelGGL((quantize_rowwise_kernel<false, true>), dim3((unsigned)blocks),
                           dim3(QR_THREADS), 0, stream, (const uint16_t *)x, ld_x, (uint8_t *)q,
                           ld_q, (uint8_t *)s_swz, s_tiles, units, upr);
    return hipGetLastError();
}

hipError_t launch_quantize_colwise(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                   void *qt, int64_t ld_qt, void *st, int64_t ld_st,
                                   hipStream_t stream)
{
    const int64_t tiles_c = (cols + QC_TILE_C - 1) / QC_TILE_C;
    const int64_t tiles_r = (rows + QC_TILE_R - 1) / QC_TILE_R;
    int64_t blocks = tiles_r * tiles_c;
    if (tiles_c >= QC_WIDE)
        blocks = (blocks + 7) / 8 * 8;
    hipLaunchKernelGGL(quantize_colwise_kernel<false>, dim3((unsigned)blocks), dim3(QC_THREADS), 0,
                       stream, (const uint16_t *)x, rows, cols, ld_x, (uint8_t *)qt, ld_qt,
                       (uint8_t *)st, ld_st, tiles_r, tiles_c);
    return hipGetLastError();
}

hipError_t launch_quantize_colwise_swz(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                       void *qt, int64_t ld_qt, void *st_swz, int64_t st_tiles,
                                       hipStream_t stream)
{
    const int64_t tiles_c = (cols + QC_TILE_C - 1) / QC_TILE_C;
    const int64_t tiles_r = (rows + QC_TILE_R - 1) / QC_TILE_R;
    int64_t blocks = tiles_r * tiles_c;
    if (tiles_c >= QC_WIDE)
        blocks = (blocks + 7) / 8 * 8;
    hipLaunchKernelGGL(quantize_colwise_kernel<true>, dim3((unsigned)blocks), dim3(QC_THREADS), 0,
                       stream, (const uint16_t *)x, rows, cols, ld_x, (uint8_t *)qt, ld_qt,
                       (uint8_t *)st_swz, st_tiles, tiles_r, tiles_c);
    return hipGetLastError();
}

hipError_t launch_quantize_rowwise_batch(const RowJob *jobs, int n, hipStream_t stream)
{
    RowBatch B{};
    B.n = n;
    int64_t blocks = 0;
    const int64_t per_block = (int64_t)QR_THREADS * QR_UNROLL;
    for (int j = 0; j < n; j++) {
        B.job[j] = jobs[j];
        B.first[j] = blocks;
        blocks += (jobs[j].rows * (jobs[j].cols / 8) + per_block - 1) / per_block;
    }
    B.first[n] = blocks;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(quantize_rowwise_batch_kernel, dim3((unsigned)blocks), dim3(QR_THREADS), 0,
                       stream, B);
    return hipGetLastError();
}

hipError_t launch_quantize_dual(const DualJob *jobs, int n, hipStream_t stream)
{
    DualBatch B{};
    B.n = n;
    int64_t blocks = 0;
    for (int j = 0; j < n; j++) {
        B.job[j] = jobs[j];
        B.first[j] = blocks;
        const int64_t tiles_r = (jobs[j].rows + QD_TILE - 1) / QD_TILE;
        const int64_t tiles_c = (jobs[j].cols + QD_TILE - 1) / QD_TILE;
        int64_t nb = tiles_r * tiles_c;
        if (tiles_c >= QC_WIDE)
            nb = (nb + 7) / 8 * 8;
        blocks += nb * jobs[j].count;
    }
    B.first[n] = blocks;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(quantize_dual_kernel, dim3((unsigned)blocks), dim3(QD_THREADS), 0, stream, B);
    return hipGetLastError();
}

hipError_t launch_scale_swizzle(const void *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                                void *s_swz, hipStream_t stream)
{
    const int64_t KT = (kblocks + 7) / 8;
    const int64_t runs = (KT + SW_KT - 1) / SW_KT;
    const int64_t halves = ((rows + 31) / 32) * runs;
    const int64_t blocks = (halves * 32 + SW_THREADS - 1) / SW_THREADS;
    const bool aligned8 = ((uintptr_t)s % 8 == 0) && (ld_s % 8 == 0);
    if (aligned8)
        hipLaunchKernelGGL(scale_swizzle_kernel<true>, dim3((unsigned)blocks), dim3(SW_THREADS), 0,
                           stream, (const uint8_t *)s, rows, kblocks, ld_s, (uint32_t *)s_swz, KT,
                           runs, halves);
    else
        hipLaunchKernelGGL(scale_swizzle_kernel<false>, dim3((unsigned)blocks), dim3(SW_THREADS), 0,
                           stream, (const uint8_t *)s, rows, kblocks, ld_s, (uint32_t *)s_swz, KT,
                           runs, halves);
    return hipGetLastError();
}

}  // namespace mx
