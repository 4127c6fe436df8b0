// Block-scaled MXFP8 GEMM for gfx950 (CDNA4): dense and grouped per expert.
//
// The learner's "MXFP8 GEMMs" and the MoE expert GEMMs of "End-to-End MXFP8
// Reinforcement Learning on Blackwell" (Figure 1; Table 2 for the models;
// Table 6 for the GEMM's share of a micro-batch) are dense contractions, so
// they run on the matrix cores: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies
// 32x64 E4M3 by 64x32 E4M3 with one E8M0 scale per lane and FP32 accumulate.
//
// Matrix-core operand layout (32x32x64, E4M3), measured on gfx950: lane
// l = 32h + r holds 32 bytes of row r; its bytes 0-15 belong to the
// instruction's first 32-element K block and bytes 16-31 to the second, and
// the scale of block x for row r is taken from lane 32x + r.  So lane (h, r)
// loads the 16-byte chunks h and 2 + h of each 64-K step: MX block 2s + x
// of step s is split over the two lane groups (16 bytes each) in byte half
// x, and its E8M0 scale sits in lane 32x + r.  The rearranged scale layout
// (mx_scale_swizzle) gives lane 32x + r one 4-byte word per 256 K whose byte
// t is the scale of block 8kt + 2t + x: exactly the scale that lane must
// supply at k-step t.  The instruction always reads byte 0 of its scale
// operand on this target, so the kernel shifts byte t down instead of relying
// on the byte-select field.
//
// Roles are swapped so the accumulator layout suits row-major C: the B tile
// (N rows) feeds the instruction's first operand and the A tile (M rows) its
// second, so each lane ends up holding 4 consecutive columns of one row of C
// per register group and writes them with one vector store.
//
// Tiling: a 256-thread workgroup (4 waves, 2x2) owns a 256x256 tile of C;
// each wave owns 128x128 = 4x4 matrix-core tiles (256 FP32 accumulators per
// lane, held in AGPRs).  K advances 128 per stage through two LDS buffers
// (A and B: 256 rows x 128 bytes each, 64 KiB per stage) filled by direct
// global->LDS loads (global_load_lds_dwordx4): no VGPR staging.  A stage is
// two 64-K matrix-core steps; the loads of stage k+2 are issued in the middle
// of stage k, as soon as every wave has read stage k's buffer, so a load has
// about one stage of matrix-core time to land.
// Each load instruction writes 1 KiB of LDS linearly by lane, so the lane's
// global address picks which 16-byte chunk lands where: eight lanes fetch one
// full 128-byte row (one cache line), and the eight chunks of a row are
// XOR-permuted by (row >> 1) & 7.  A 16-byte LDS read is serviced 16 lanes at
// a time, in the lane groups {0-3, 12-15, 20-27} and {4-11, 16-19, 28-31} of
// each half-wave (measured with in-bounds probes and the LDS bank-conflict
// counter), each cycle covering 64 banks = 256 bytes = two rows.  The eight
// rows of each parity in a group differ in (row >> 1) & 7, so every lane of a
// group gets its own 16-byte bank slot.  The fragments of the next step are
// read from LDS while the matrix cores run the current one.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int GM_THREADS = 256;
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int STAGES = 2;
constexpr int TM = 4, TN = 4;      // 32x32 sub-tiles per wave along M and N
constexpr int GROUP_M = 4;         // tile-rows walked together for L2 reuse
constexpr int STAGE_BYTES = BM * BK;  // one operand, one stage (32 KiB)
constexpr int DMA_PER_WAVE = STAGE_BYTES / 1024 / 4;  // 1 KiB per instruction, 4 waves

struct GemmParams {
    int64_t M, N, K;
    const uint8_t *a;
    int64_t ld_a;
    const uint8_t *as;
    const uint8_t *b;
    int64_t ld_b;
    const uint8_t *bs;
    void *c;
    int64_t ld_c;
    int64_t tiles_m, tiles_n;
    const int64_t *offsets;  // grouped only
    int64_t G;
    int64_t b_group_stride, bs_group_stride;
    uint32_t as_bytes, bs_bytes;  // rearranged scale bytes of A (all rows) and of one B
    int vec_store;
};

__device__ __forceinline__ int chunk_perm(int row) { return (row >> 1) & 7; }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// Buffer resource for a byte range: uniform base and size in SGPRs, so each
// lane supplies only a 32-bit offset.  Word 3 selects 32-bit data format
// (what untyped buffer loads on gfx9-family targets expect).  Loads whose
// per-lane offset falls outside the range return zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
#define MX_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// Workgroup barrier for the LDS ring.  __syncthreads() would also wait for
// every outstanding vector-memory load (its release fence must cover the LDS
// writes of the direct-to-LDS loads), draining the whole pipeline each step.
// Here each wave waits only for its own LDS reads (so a buffer can be
// refilled) and the loads of the stage about to be read were already waited
// for with MX_WAIT_VMCNT; the "memory" clobber keeps the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void lds_ring_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

template <bool GROUPED, int CT>
__global__ __launch_bounds__(GM_THREADS, 1) void mx_gemm_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t sA[STAGES][STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[STAGES][STAGE_BYTES];
    // per wave: the TM + TN scale words of each lane for one 256-K group
    __shared__ __attribute__((aligned(1024))) uint32_t sS[4][TM + TN][64];
    __shared__ int64_t s_grp[3];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    int64_t m0, n0, m_end;
    const uint8_t *B = p.b;
    const uint8_t *BS = p.bs;

    if (!GROUPED) {
        int64_t pid = blockIdx.x;
        const int64_t num = gridDim.x;
        // consecutive workgroups are dealt to the 8 XCDs in turn: renumber so
        // each XCD walks a contiguous range of tiles (shared L2 panels)
        if ((num & 7) == 0)
            pid = (pid & 7) * (num >> 3) + (pid >> 3);
        const int64_t per_group = GROUP_M * p.tiles_n;
        const int64_t grp = pid / per_group;
        const int64_t first_m = grp * GROUP_M;
        const int64_t gm = min(p.tiles_m - first_m, (int64_t)GROUP_M);
        const int64_t in = pid - grp * per_group;
        m0 = (first_m + in % gm) * BM;
        n0 = (in / gm) * BN;
        m_end = p.M;
    } else {
        // tile (m-tile id, n-tile): find the expert whose rows hold m-tile id
        const int64_t mt_id = blockIdx.x / p.tiles_n;
        const int64_t tn = blockIdx.x - mt_id * p.tiles_n;
        n0 = tn * BN;
        if (wave == 0) {
            int64_t running = 0;
            for (int64_t g0 = 0; g0 < p.G; g0 += 64) {
                const int64_t g = g0 + lane;
                int64_t lo = 0, hi = 0;
                if (g < p.G) {
                    lo = min(max(p.offsets[g], (int64_t)0), p.M);
                    hi = min(max(p.offsets[g + 1], lo), p.M);
                }
                const int64_t cnt = (hi - lo + BM - 1) / BM;
                int64_t incl = cnt;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    int64_t o = __shfl_up(incl, d, 64);
                    if (lane >= d)
                        incl += o;
                }
                const int64_t excl = running + incl - cnt;
                if (cnt > 0 && mt_id >= excl && mt_id < excl + cnt) {
                    s_grp[0] = g;
                    s_grp[1] = lo + (mt_id - excl) * BM;
                    s_grp[2] = hi;
                }
                running += __shfl(incl, 63, 64);
            }
            if (lane == 0 && mt_id >= running)
                s_grp[0] = -1;
        }
        __syncthreads();
        const int64_t g = s_grp[0];
        if (g < 0)
            return;
        m0 = s_grp[1];
        m_end = s_grp[2];
        B = p.b + g * p.b_group_stride;
        BS = p.bs + g * p.bs_group_stride;
    }

    const int64_t N = p.N;
    const int64_t KT256 = (p.K + 255) / 256;  // scale words per 32-row tile
    const int KIT = (int)(p.K / BK);

    // ---- direct-to-LDS plan.  Instruction i of this wave fills LDS rows
    // 8*(8*wave + i) .. +8 of a stage; lane -> row + lane/8, slot lane%8,
    // fetching global chunk slot ^ perm(row) of that row.
    const uint8_t *a_tile = p.a + m0 * p.ld_a;
    const uint8_t *b_tile = B + n0 * p.ld_b;
    const uint32_t a_tile_bytes = (uint32_t)(min(m_end - m0, (int64_t)BM) * p.ld_a);
    const uint32_t b_tile_bytes = (uint32_t)(min(N - n0, (int64_t)BN) * p.ld_b);
    uint32_t a_src[DMA_PER_WAVE], b_src[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; i++) {
        const int row = 8 * (DMA_PER_WAVE * wave + i) + (lane >> 3);
        const int chunk = (lane & 7) ^ chunk_perm(row);
        const int64_t ra = min(m0 + row, m_end - 1) - m0;
        const int64_t rb = min(n0 + row, N - 1) - n0;
        a_src[i] = (uint32_t)(ra * p.ld_a + chunk * 16);
        b_src[i] = (uint32_t)(rb * p.ld_b + chunk * 16);
    }
    const uint32_t lds_a0 = (uint32_t)(uintptr_t)&sA[0][0];
    const uint32_t lds_b0 = (uint32_t)(uintptr_t)&sB[0][0];
    // Loads of stage st into buffer buf.  A stage past the end (live false)
    // gets an empty range: its loads move no data and write zeros into a
    // buffer nobody reads again, which keeps the main loop branch-free.
    auto dma_stage = [&](int st, int buf, bool live) {
        const __amdgpu_buffer_rsrc_t ra = byte_range(a_tile, live ? a_tile_bytes : 0u);
        const __amdgpu_buffer_rsrc_t rb = byte_range(b_tile, live ? b_tile_bytes : 0u);
        const uint32_t koff = (uint32_t)st * BK;  // scalar offset, added after the range check
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; i++) {
            const uint32_t off = (uint32_t)(buf * STAGE_BYTES + 1024 * (DMA_PER_WAVE * wave + i));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lptr_t)(uintptr_t)(lds_a0 + off), 16,
                                                     a_src[i], koff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lptr_t)(uintptr_t)(lds_b0 + off), 16,
                                                     b_src[i], koff, 0, 0);
        }
    };

    // ---- per-lane scale words.  The lane's row is r32 within every 32-row
    // sub-tile; sub-tiles are 32 rows apart, i.e. one scale tile (KT256 * 256
    // bytes) apart.  Each 256-K group's words travel through LDS: one 4-byte
    // direct-to-LDS load per sub-tile puts lane l's word at word l of the
    // wave's region, and the lane reads it back when the group starts.  Rows
    // past the operand fall outside the resource's range and read zero.
    const int h = lane >> 5;
    const int r32 = lane & 31;
    uint32_t sa_off[TM], sb_off[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int64_t row = m0 + wm * 128 + i * 32 + r32;
        sa_off[i] = (uint32_t)((row >> 5) * KT256 * 256 + (h * 32 + (row & 31)) * 4);
    }
#pragma unroll
    for (int i = 0; i < TN; i++) {
        const int64_t row = n0 + wn * 128 + i * 32 + r32;
        sb_off[i] = (uint32_t)((row >> 5) * KT256 * 256 + (h * 32 + (row & 31)) * 4);
    }
    const uint32_t lds_s0 = (uint32_t)(uintptr_t)&sS[wave][0][0];
    auto dma_scales = [&](int group, bool live) {
        const __amdgpu_buffer_rsrc_t rsa = byte_range(p.as, live ? p.as_bytes : 0u);
        const __amdgpu_buffer_rsrc_t rsb = byte_range(BS, live ? p.bs_bytes : 0u);
        const uint32_t kw = (uint32_t)group * 256;
#pragma unroll
        for (int i = 0; i < TM; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lptr_t)(uintptr_t)(lds_s0 + 256 * i), 4,
                                                     sa_off[i], kw, 0, 0);
#pragma unroll
        for (int i = 0; i < TN; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lptr_t)(uintptr_t)(lds_s0 + 256 * (TM + i)),
                                                     4, sb_off[i], kw, 0, 0);
    };
    auto read_scales = [&](uint32_t *xa, uint32_t *xb) {
#pragma unroll
        for (int i = 0; i < TM; i++)
            xa[i] = sS[wave][i][lane];
#pragma unroll
        for (int i = 0; i < TN; i++)
            xb[i] = sS[wave][TM + i][lane];
    };

    // ---- per-lane LDS read offsets of the matrix-core fragments.  At step
    // s (0, 1) of a stage the lane needs chunk 4s + h (bytes 0-15 of the
    // operand) and chunk 4s + 2 + h (bytes 16-31) of its row.  Rows of the
    // sub-tiles are 32 apart, which leaves chunk_perm unchanged, and the chunk
    // bits are disjoint, so the four chunks sit at the step-0 offset XOR
    // 64s + 32t.  One register per (s, t) and operand; sub-tile and buffer
    // are immediate offsets of the LDS read.
    uint32_t a_rd[4], b_rd[4];
    {
        const uint32_t la0 = (uint32_t)((wm * 128 + r32) * BK + ((h ^ chunk_perm(r32)) * 16));
        const uint32_t lb0 = (uint32_t)((wn * 128 + r32) * BK + ((h ^ chunk_perm(r32)) * 16));
#pragma unroll
        for (int x = 0; x < 4; x++) {
            a_rd[x] = la0 ^ (32u * x);
            b_rd[x] = lb0 ^ (32u * x);
        }
    }

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++)
                acc[i][j][v] = 0.0f;

    auto read_frags = [&](int buf, int step, v8i *xa, v8i *xb) {
        const uint8_t *A_ = &sA[buf][0];
        const uint8_t *B_ = &sB[buf][0];
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const v4i lo = *reinterpret_cast<const v4i *>(A_ + a_rd[2 * step] + i * 32 * BK);
            const v4i hi = *reinterpret_cast<const v4i *>(A_ + a_rd[2 * step + 1] + i * 32 * BK);
            xa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < TN; i++) {
            const v4i lo = *reinterpret_cast<const v4i *>(B_ + b_rd[2 * step] + i * 32 * BK);
            const v4i hi = *reinterpret_cast<const v4i *>(B_ + b_rd[2 * step + 1] + i * 32 * BK);
            xb[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    // ---- prologue: scale words of the first 256 K, stages 0 and 1 in flight
    dma_scales(0, true);
    dma_stage(0, 0, true);
    dma_stage(1, 1, KIT > 1);
    MX_WAIT_VMCNT(2 * DMA_PER_WAVE);  // stage 1's loads may still be in flight
    lds_ring_barrier();
    uint32_t wa[TM], wb[TN];
    read_scales(wa, wb);
    v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    read_frags(0, 0, fa0, fb0);

#define MX_MFMA_STEP(FA, FB, SHIFT)                                                          \
    _Pragma("unroll") for (int i = 0; i < TN; i++) {                                         \
        const int sbv = (int)(wb[i] >> (SHIFT));                                             \
        _Pragma("unroll") for (int j = 0; j < TM; j++)                                       \
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                     \
                FB[i], FA[j], acc[i][j], 0, 0, 0, sbv, 0, (int)(wa[j] >> (SHIFT)));          \
    }

    // Stage st uses buffer st & 1 and scale bytes 2*(st & 1) and 2*(st & 1) + 1
    // of the current 256-K words.  On entry the step-0 fragments are in
    // fa0/fb0.  First half: read step 1's fragments while step 0 runs (one
    // LDS read between consecutive matrix-core instructions).  Then wait until
    // this wave's loads of stage st+1 have landed and every wave is done with
    // buffer st & 1.  Second half, while step 1 runs: read the scale words
    // staged in LDS, issue the loads of stage st+2 into buffer st & 1 (after
    // the scale words of group (st+2)/2), and read stage st+1's step-0
    // fragments from the other buffer.  The scale words read on a group's
    // last stage (odd st) belong to the next group and replace the current
    // ones; on an even stage the read races the new loads and is discarded.
    // Past the end the loads are empty and the fragment reads unused, so the
    // body has no branches and the interleaving below applies to all of it.
    for (int st = 0; st < KIT; st++) {
        const int buf = st & 1;
        const int shift = 16 * buf;
        read_frags(buf, 1, fa1, fb1);
        MX_MFMA_STEP(fa0, fb0, shift)
#pragma unroll
        for (int q = 0; q < TM * TN; q++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix core
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        MX_WAIT_VMCNT(0);
        lds_ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
        uint32_t na[TM], nb[TN];
        read_scales(na, nb);
        const bool live = st + 2 < KIT;
        dma_scales((st + 2) >> 1, live);
        dma_stage(st + 2, buf, live);
        read_frags(buf ^ 1, 0, fa0, fb0);
        MX_MFMA_STEP(fa1, fb1, shift + 8)
        __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 1);  // scale words
#pragma unroll
        for (int q = 0; q < TM * TN / 2; q++) {  // 16 matrix-core, 24 loads, 16 LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x010, 2, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x010, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
#pragma unroll
        for (int i = 0; i < TM; i++)
            wa[i] = buf ? na[i] : wa[i];
#pragma unroll
        for (int i = 0; i < TN; i++)
            wb[i] = buf ? nb[i] : wb[i];
    }
    MX_WAIT_VMCNT(0);  // no load may still write LDS when the workgroup ends
#undef MX_MFMA_STEP

    // ---- epilogue: lane holds C[m][n..n+3] for each register group
#pragma unroll
    for (int i = 0; i < TN; i++) {
#pragma unroll
        for (int j = 0; j < TM; j++) {
            const int64_t m = m0 + wm * 128 + j * 32 + r32;
            if (m >= m_end)
                continue;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int64_t n = n0 + wn * 128 + i * 32 + 8 * q + 4 * h;
                const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if (CT == 0) {
                    uint16_t *crow = reinterpret_cast<uint16_t *>(p.c) + m * p.ld_c;
                    if (p.vec_store && n + 3 < N) {
                        uint2 w;
                        w.x = f32_to_bf16_rne(v0) | (f32_to_bf16_rne(v1) << 16);
                        w.y = f32_to_bf16_rne(v2) | (f32_to_bf16_rne(v3) << 16);
                        *reinterpret_cast<uint2 *>(crow + n) = w;
                    } else {
                        if (n + 0 < N) crow[n + 0] = (uint16_t)f32_to_bf16_rne(v0);
                        if (n + 1 < N) crow[n + 1] = (uint16_t)f32_to_bf16_rne(v1);
                        if (n + 2 < N) crow[n + 2] = (uint16_t)f32_to_bf16_rne(v2);
                        if (n + 3 < N) crow[n + 3] = (uint16_t)f32_to_bf16_rne(v3);
                    }
                } else {
                    float *crow = reinterpret_cast<float *>(p.c) + m * p.ld_c;
                    if (p.vec_store && n + 3 < N) {
                        *reinterpret_cast<float4 *>(crow + n) = make_float4(v0, v1, v2, v3);
                    } else {
                        if (n + 0 < N) crow[n + 0] = v0;
                        if (n + 1 < N) crow[n + 1] = v1;
                        if (n + 2 < N) crow[n + 2] = v2;
                        if (n + 3 < N) crow[n + 3] = v3;
                    }
                }
            }
        }
    }
}

// Bytes of a rearranged scale buffer: 32-row x 8-block tiles of 256 bytes.
static int64_t scale_bytes(int64_t rows, int64_t K)
{
    return ((rows + 31) / 32) * ((K / 32 + 7) / 8) * 256;
}

static int vec_ok(const void *c, int64_t ld_c, int c_dtype)
{
    const uintptr_t align = c_dtype == 0 ? 8 : 16;
    return ((uintptr_t)c % align == 0) && (ld_c % 4 == 0);
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void *a_q, int64_t ld_a,
                       const void *a_s, const void *b_q, int64_t ld_b, const void *b_s,
                       void *c, int64_t ld_c, int c_dtype, hipStream_t stream)
{
    GemmParams p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.a = (const uint8_t *)a_q;
    p.ld_a = ld_a;
    p.as = (const uint8_t *)a_s;
    p.b = (const uint8_t *)b_q;
    p.ld_b = ld_b;
    p.bs = (const uint8_t *)b_s;
    p.c = c;
    p.ld_c = ld_c;
    p.tiles_m = (M + BM - 1) / BM;
    p.tiles_n = (N + BN - 1) / BN;
    p.as_bytes = (uint32_t)scale_bytes(M, K);
    p.bs_bytes = (uint32_t)scale_bytes(N, K);
    p.vec_store = vec_ok(c, ld_c, c_dtype);
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    if (c_dtype == 0)
        hipLaunchKernelGGL((mx_gemm_kernel<false, 0>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<false, 1>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int64_t G, int64_t M_total, int64_t N, int64_t K,
                               const int64_t *offsets, const void *a_q, int64_t ld_a,
                               const void *a_s, const void *b_q, const void *b_s, void *c,
                               int64_t ld_c, int c_dtype, hipStream_t stream)
{
    GemmParams p{};
    p.M = M_total;
    p.N = N;
    p.K = K;
    p.a = (const uint8_t *)a_q;
    p.ld_a = ld_a;
    p.as = (const uint8_t *)a_s;
    p.b = (const uint8_t *)b_q;
    p.ld_b = K;
    p.bs = (const uint8_t *)b_s;
    p.c = c;
    p.ld_c = ld_c;
    p.offsets = offsets;
    p.G = G;
    p.b_group_stride = N * K;
    p.bs_group_stride = scale_bytes(N, K);
    p.as_bytes = (uint32_t)scale_bytes(M_total, K);
    p.bs_bytes = (uint32_t)p.bs_group_stride;
    // upper bound on sum_g ceil(m_g / BM): every group adds at most one partial tile
    p.tiles_m = (M_total + BM - 1) / BM + G;
    p.tiles_n = (N + BN - 1) / BN;
    p.vec_store = vec_ok(c, ld_c, c_dtype);
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    if (c_dtype == 0)
        hipLaunchKernelGGL((mx_gemm_kernel<true, 0>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<true, 1>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mx
