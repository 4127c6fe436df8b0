// Per-expert column-wise quantization for the MoE weight gradient (gfx950).
//
// The update_actor stage of the MoE learner in "End-to-End MXFP8
// Reinforcement Learning on Blackwell" (Table 8; Table 2 for Qwen3-30B-A3B,
// 128 experts, top-8) needs each expert's weight gradient dW_g = dY_g^T X_g:
// a contraction over that expert's token rows only.  Its operands are the
// column-wise quantized dY and X, and a 32-row block must not hold rows of two
// experts.  Layout: expert g's rows [offsets[g], offsets[g+1]) become columns
// [pad[g], pad[g+1]) of the transposed operand, each range max(256, m_g
// rounded up to 256) columns long so that every range is a whole number of
// the GEMM's 256-K scale groups; the columns past an expert's rows hold zero
// codes (zero rows appended: they leave every block maximum unchanged) and
// the blocks made only of them get scale code 0.
//
// pad_offsets_kernel: one workgroup, thread g takes expert g; a block-wide
// scan of the range lengths.  The offsets are clamped into [0, rows] and made
// nondecreasing first, and the results at k_cap, so any offsets give
// in-bounds ranges.
//
// quantize_colwise_grouped_kernel: a 512-thread workgroup takes 256 columns
// of the padded operand (one expert's, since every range is 256-aligned) by
// 256 of x's columns, as 2 x 4 waves of 128 padded rows x 64 columns: the
// column-wise lane layout of the dual quantizer (lane = 32-row block, half,
// 8-column group; 16 rows x 8 columns per lane; the halves of a block meet
// through one DPP rotation; v_perm pairs two rows of a column for the scaled
// conversion).  The tile's rows of x are one buffer range, [first row, first
// row + valid rows), so the loads of rows past the expert's last read zero
// without a per-row test; a lane stores 16 codes of each of its 8 columns.
// The scale bytes go to LDS at their rearranged positions, and each thread
// stores one word: 8 whole 256-byte tiles of the rearranged layout per
// workgroup.  Registers: the 16 rows a lane holds take 64 VGPRs, and each
// magnitude feeds the column-wise and the row-wise maxima in the same pass
// (computed in two passes, all 64 magnitudes stayed live and the row-wise
// variant needed 147 VGPRs: one workgroup per CU instead of two).
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

constexpr int QG_THREADS = 512;
constexpr int QG_TILE = 256;

__global__ __launch_bounds__(MOE_MAX_EXPERTS) void pad_offsets_kernel(const int64_t *__restrict__ offsets,
                                                                      int G, int64_t rows, int64_t k_cap,
                                                                      int64_t *__restrict__ pad)
{
    __shared__ int64_t wsum[MOE_MAX_EXPERTS / 64];
    const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
    int64_t len = 0;
    if (g < G) {
        const int64_t lo = min(max(offsets[g], (int64_t)0), rows);
        const int64_t hi = min(max(offsets[g + 1], lo), rows);
        len = max((int64_t)QG_TILE, (hi - lo + QG_TILE - 1) / QG_TILE * QG_TILE);
    }
    int64_t incl = len;
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
    if (g < G)
        pad[g] = min(base + incl - len, k_cap);
    if (g == G - 1)
        pad[G] = min(base + incl, k_cap);
}

// ROW: also the row-wise quantization of the same rows from the same loads
// (the data gradient's operand): the row-wise blocks of a lane's 16 rows
// combine over its 4-lane quad as in the dual quantizer.  The codes and
// scale bytes are staged in LDS, then written row by row: sixteen threads
// store a row's 256 codes as two whole 128-byte lines, and one thread a
// row's eight scale bytes as the two 4-byte words they form in the
// rearranged layout (rows of an expert start anywhere, so a row's scales do
// not fill whole tiles).
// LOAD selects where the tile's BF16 rows come from:
//  - QG_PLAIN: rows [src0, src0 + valid) of x.
//  - QG_SWIGLU: x is the gate/up projection output [rows][ld_x] (gate in
//    columns [0, cols), up in [cols, 2 cols)) and the tile quantizes h =
//    SwiGLU(gate, up) (swiglu_bf16x2, the same h as mx_swiglu_quantize's),
//    formed in registers from one load of each half: the MoE down
//    projection's row-wise A operand and its weight gradient's per-expert
//    column-wise operand, with h itself never written.
//  - QG_GATHER: row p of the operand is row src[p] of x (the token
//    activations, x_bytes bytes in all): the MoE dispatch's permuted rows,
//    quantized row-wise (the gate_up projection's A operand) and per expert
//    column-wise (its weight gradient's operand) without the permuted BF16
//    rows ever being written.
constexpr int QG_PLAIN = 0, QG_SWIGLU = 1, QG_GATHER = 2;
template <bool ROW, int LOAD>
__global__ __launch_bounds__(QG_THREADS) void quantize_colwise_grouped_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t cols, int64_t ld_x,
    const int64_t *__restrict__ offsets, const int64_t *__restrict__ pad, int G,
    uint8_t *__restrict__ qt, int64_t ld_qt, uint8_t *__restrict__ st_swz, int64_t st_tiles,
    int64_t tiles_c, uint8_t *__restrict__ q, int64_t ld_q, uint8_t *__restrict__ s_swz, int64_t s_tiles,
    const int32_t *__restrict__ src, uint32_t x_bytes)
{
    __shared__ uint32_t lds_st[8 * 64];
    __shared__ __attribute__((aligned(16))) uint8_t lds_q[ROW ? QG_TILE * QG_TILE : 1];  // row-wise codes
    __shared__ uint8_t lds_rs[ROW ? QG_TILE * 8 : 1];  // row-wise scale bytes, 8 per row
    __shared__ __attribute__((aligned(16))) int32_t lds_src[LOAD == QG_GATHER ? QG_TILE : 1];  // the tile's tokens
    const int64_t tr = blockIdx.x / tiles_c, tc = blockIdx.x - tr * tiles_c;
    const int64_t P0 = tr * QG_TILE;  // first padded column (row of the padded operand)
    // The expert whose range holds P0 is the last g with pad[g] <= P0; the
    // ranges are nondecreasing and pad[0] = 0, so g = #{j in 1..G : pad[j] <=
    // P0}.  Every thread tests up to two entries (G <= 1024) and the
    // workgroup counts them: one round of loads instead of a dependent
    // binary search.  g == G means P0 is past the last range.
    int hits = 0;
    for (int j = (int)threadIdx.x + 1; j <= G; j += QG_THREADS)
        hits += pad[j] <= P0 ? 1 : 0;
    const int g = __syncthreads_count(hits >= 1) + __syncthreads_count(hits >= 2);
    if (g >= G)
        return;  // past the last expert's range: nothing to write
    const int64_t glo = min(max(offsets[g], (int64_t)0), rows);
    const int64_t ghi = min(max(offsets[g + 1], glo), rows);
    const int64_t src0 = glo + (P0 - pad[g]);
    const int valid = (int)min(max(ghi - src0, (int64_t)0), (int64_t)QG_TILE);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 2, wc = wave & 3;
    const int cg = lane & 7, half = (lane >> 3) & 1, rb = lane >> 4;
    const int64_t C0 = tc * QG_TILE;
    const int64_t c0 = C0 + wc * 64 + cg * 8;
    const int rl0 = wr * 128 + rb * 32 + half * 16;  // the lane's first row within the tile
    // cols % 32 == 0: a lane's 8 columns are all in range or all out, and so
    // are those of its DPP partner (the other half of its block)
    const bool active = c0 < cols;
    lds_st[tid] = 0x7F7F7F7Fu;
    // the tile's rows of x, [src0, src0 + valid), as one buffer range: loads
    // of rows past it (the next expert's, or past x) and of inactive lanes
    // (offset 2^31, past any range: 256 ld_x * 2 < 2^31) read zero
    const __amdgpu_buffer_rsrc_t rx = byte_range(x + (valid > 0 ? src0 * ld_x : 0), (uint32_t)(valid * ld_x * 2));
    const uint32_t voff = active ? (uint32_t)(rl0 * ld_x + c0) * 2u : 0x80000000u;
    const uint32_t vstep = active ? (uint32_t)ld_x * 2u : 0u;
    uint4 v[16];
    if (LOAD == QG_GATHER) {
        // each row from its token: the tile's 256 token numbers are loaded
        // once (one coalesced load) into LDS; one range over all of x (below
        // 2^31 bytes), rows past the tile's valid ones and inactive lanes at
        // an offset past it (they read zero).  Plain loads: every token row
        // is read by each of its routed copies' tiles, and those repeat reads
        // hit in cache often enough that streaming loads were slower (232 ->
        // 275 us for 163840 routed rows).
        if (tid < QG_TILE)
            lds_src[tid] = tid < valid ? src[src0 + tid] : -1;
        __syncthreads();
        const __amdgpu_buffer_rsrc_t rg = byte_range(x, x_bytes);
        // the lane's 16 token numbers in four 16-byte LDS reads (rl0 is a
        // multiple of 16), so the 16 row loads issue back to back
        int32_t tk[16];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int4 w = reinterpret_cast<const int4 *>(lds_src + rl0)[k];
            tk[4 * k] = w.x;
            tk[4 * k + 1] = w.y;
            tk[4 * k + 2] = w.z;
            tk[4 * k + 3] = w.w;
        }
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int32_t t = tk[i];
            const uint32_t off = (active && t >= 0) ? (uint32_t)((int64_t)t * ld_x + c0) * 2u : 0xFFFFFFF0u;
            v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
        }
    } else if (LOAD == QG_SWIGLU) {
        // the up half: cols * 2 bytes further along the row (an inactive
        // lane's offset stays past the range).  A lane's 32 loads do not fit
        // the register budget of two workgroups per CU at once, and left to
        // the compiler they issued 2-5 at a time between the SwiGLU
        // arithmetic.  Instead groups of 4 rows (8 loads) run two ahead:
        // group k+2 is loaded while group k is formed, about 16 loads stay
        // in flight, and the barriers keep the scheduler from merging the
        // phases (172 -> 156 us on the 163840-row gate_up output)
        const uint32_t uoff = (uint32_t)(cols * 2);
        uint4 g[4][4], u[4][4];
#pragma unroll
        for (int k = 0; k < 2; k++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                g[k][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + (4 * k + i) * vstep, 0, STREAM));
                u[k][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + (4 * k + i) * vstep + uoff, 0, STREAM));
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < 4; k++) {
#pragma unroll
            for (int i = 0; i < 4; i++)
                v[4 * k + i] = make_uint4(swiglu_bf16x2(g[k][i].x, u[k][i].x), swiglu_bf16x2(g[k][i].y, u[k][i].y),
                                          swiglu_bf16x2(g[k][i].z, u[k][i].z), swiglu_bf16x2(g[k][i].w, u[k][i].w));
            if (k + 2 < 4) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    g[k + 2][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + (4 * (k + 2) + i) * vstep, 0, STREAM));
                    u[k + 2][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + (4 * (k + 2) + i) * vstep + uoff, 0, STREAM));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++)
            v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + i * vstep, 0, STREAM));
    }
    // column-wise maxima (per column, the lane's 16 rows) and, with ROW, the
    // row-wise ones (per row, the lane's 8 columns) in one pass, each
    // magnitude used by both as soon as it is formed
    uint32_t m[4] = {0, 0, 0, 0};
    uint32_t rmax[ROW ? 16 : 1];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const uint32_t ax = mag2(v[i].x), ay = mag2(v[i].y), az = mag2(v[i].z), aw = mag2(v[i].w);
        m[0] = pk_max_u16(m[0], ax);
        m[1] = pk_max_u16(m[1], ay);
        m[2] = pk_max_u16(m[2], az);
        m[3] = pk_max_u16(m[3], aw);
        if (ROW) {
            const uint32_t w = pk_max_u16(pk_max_u16(ax, ay), pk_max_u16(az, aw));
            rmax[i] = max(w & 0xFFFFu, w >> 16);
        }
    }
#pragma unroll
    for (int k = 0; k < 4; k++)  // row_ror:8 - the other half of the column block
        m[k] = pk_max_u16(m[k], (uint32_t)__builtin_amdgcn_mov_dpp((int)m[k], 0x128, 0xF, 0xF, false));
    if (ROW) {
        // the row's 32-column block is the lane's quad: quad_perm [1,0,3,2]
        // and [2,3,0,1]
#pragma unroll
        for (int i = 0; i < 16; i++) {
            uint32_t a = rmax[i];
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, false));
            a = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xF, 0xF, false));
            rmax[i] = a;
        }
    }
    __syncthreads();  // the 0x7F fill precedes every scale byte
    uint8_t *bst = reinterpret_cast<uint8_t *>(lds_st);
    // the tile's 256 rows of qt from column P0 (256 ld_qt < 2^32): lane
    // offset of its first row, column j's row j ld_qt further
    const __amdgpu_buffer_rsrc_t rq = byte_range(qt + C0 * ld_qt + P0, (uint32_t)(QG_TILE * ld_qt));
    const uint32_t qoff = (uint32_t)((wc * 64 + cg * 8) * ld_qt + rl0);
    if (active) {
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
                const uint32_t wcw = wi == 0 ? cc.x : wi == 1 ? cc.y : wi == 2 ? cc.z : cc.w;
                const uint32_t wd = wi == 0 ? d.x : wi == 1 ? d.y : wi == 2 ? d.z : d.w;
                const uint32_t p01 = __builtin_amdgcn_perm(wb, wa, sel);   // rows 4k, 4k+1
                const uint32_t p23 = __builtin_amdgcn_perm(wd, wcw, sel);  // rows 4k+2, 4k+3
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
    }
    if (ROW) {
        // row-wise codes and scale bytes, staged (every lane is active: cols
        // % 256 == 0; rows past the valid ones hold zeros and are staged but
        // not written out)
        const int cl = wc * 64 + cg * 8;  // the lane's first column within the tile
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const uint32_t c = scale_code(rmax[i]);
            const float sc = cvt_scale(c);
            const uint32_t o0 = nan_block_select(cvt_x4(v[i].x, v[i].y, sc), c);
            const uint32_t o1 = nan_block_select(cvt_x4(v[i].z, v[i].w, sc), c);
            *reinterpret_cast<uint2 *>(&lds_q[(rl0 + i) * QG_TILE + cl]) = make_uint2(o0, o1);
            if ((cg & 3) == 0)
                lds_rs[(rl0 + i) * 8 + (cl >> 5)] = (uint8_t)c;
        }
    }
    __syncthreads();
    if (ROW) {
        // codes: 16 threads per row, 16 bytes each (cols % 256 == 0 here, so
        // every row of the tile has its 256 columns)
        // (one buffer range over rows [src0, src0 + valid): the stores of the
        // rows past it are dropped; 256 ld_q < 2^32)
        const __amdgpu_buffer_rsrc_t rr = byte_range(q + (valid > 0 ? src0 * ld_q : 0) + C0,
                                                     (uint32_t)(valid * ld_q));
#pragma unroll
        for (int k = 0; k < QG_TILE * QG_TILE / 16 / QG_THREADS; k++) {
            const int idx = tid + k * QG_THREADS;
            const int r = idx >> 4, ch = idx & 15;
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(v4u_t, *reinterpret_cast<const uint4 *>(&lds_q[r * QG_TILE + ch * 16])), rr,
                (uint32_t)(r * ld_q + ch * 16), 0, STREAM);
        }
        // scales: blocks 2t + h of the row go to byte t of word h
        if (tid < QG_TILE && tid < valid) {
            const int r = tid;
            const int64_t row = src0 + r;
            const uint8_t *b = &lds_rs[r * 8];
            const uint32_t w0 = b[0] | (b[2] << 8) | (b[4] << 16) | ((uint32_t)b[6] << 24);
            const uint32_t w1 = b[1] | (b[3] << 8) | (b[5] << 16) | ((uint32_t)b[7] << 24);
            uint32_t *tile = reinterpret_cast<uint32_t *>(s_swz + ((row >> 5) * s_tiles + C0 / 256) * 256);
            tile[row & 31] = w0;
            tile[32 + (row & 31)] = w1;
        }
    }
    // thread -> word tid & 63 of the rearranged tile of 32-column row tid >> 6
    const int t = tid >> 6, w = tid & 63;
    if (C0 + 32 * t < cols)
        reinterpret_cast<uint32_t *>(st_swz + ((C0 / 32 + t) * st_tiles + tr) * 256)[w] = lds_st[tid];
}

hipError_t launch_quantize_colwise_grouped(const void *x, int64_t rows, int64_t cols, int64_t ld_x,
                                          const int64_t *offsets, int64_t G, int64_t *pad,
                                          void *qt, int64_t ld_qt, int64_t k_cap, void *st_swz,
                                          hipStream_t stream, void *q, int64_t ld_q, void *s_swz, bool swiglu,
                                          const int32_t *src, int64_t x_bytes)
{
    hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(MOE_MAX_EXPERTS), 0, stream, offsets, (int)G,
                       rows, k_cap, pad);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int64_t tiles_c = (cols + QG_TILE - 1) / QG_TILE;
    const int64_t tiles_r = k_cap / QG_TILE;
    const int64_t blocks = tiles_r * tiles_c;
    if (blocks == 0)
        return hipSuccess;
    if (src != nullptr)
        hipLaunchKernelGGL((quantize_colwise_grouped_kernel<true, QG_GATHER>), dim3((unsigned)blocks),
                           dim3(QG_THREADS), 0, stream, (const uint16_t *)x, rows, cols, ld_x, offsets,
                           (const int64_t *)pad, (int)G, (uint8_t *)qt, ld_qt, (uint8_t *)st_swz, k_cap / QG_TILE,
                           tiles_c, (uint8_t *)q, ld_q, (uint8_t *)s_swz, cols / 256, src, (uint32_t)x_bytes);
    else if (swiglu)
        hipLaunchKernelGGL((quantize_colwise_grouped_kernel<true, QG_SWIGLU>), dim3((unsigned)blocks),
                           dim3(QG_THREADS), 0, stream, (const uint16_t *)x, rows, cols, ld_x, offsets,
                           (const int64_t *)pad, (int)G, (uint8_t *)qt, ld_qt, (uint8_t *)st_swz, k_cap / QG_TILE,
                           tiles_c, (uint8_t *)q, ld_q, (uint8_t *)s_swz, cols / 256, nullptr, 0u);
    else if (q != nullptr)
        hipLaunchKernelGGL((quantize_colwise_grouped_kernel<true, QG_PLAIN>), dim3((unsigned)blocks),
                           dim3(QG_THREADS), 0, stream, (const uint16_t *)x, rows, cols, ld_x, offsets,
                           (const int64_t *)pad, (int)G, (uint8_t *)qt, ld_qt, (uint8_t *)st_swz, k_cap / QG_TILE,
                           tiles_c, (uint8_t *)q, ld_q, (uint8_t *)s_swz, cols / 256, nullptr, 0u);
    else
        hipLaunchKernelGGL((quantize_colwise_grouped_kernel<false, QG_PLAIN>), dim3((unsigned)blocks),
                           dim3(QG_THREADS), 0, stream, (const uint16_t *)x, rows, cols, ld_x, offsets,
                           (const int64_t *)pad, (int)G, (uint8_t *)qt, ld_qt, (uint8_t *)st_swz, k_cap / QG_TILE,
                           tiles_c, nullptr, (int64_t)0, nullptr, (int64_t)0, nullptr, 0u);
    return hipGetLastError();
}

}  // namespace mx
