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
// lane, held in AGPRs).  K advances 64 per stage through a ring of 4 LDS
// stages (A and B: 256 rows x 64 bytes each, 32 KiB per stage) filled by
// direct global->LDS loads (global_load_lds_dwordx4): no VGPR staging, and
// three stages stay in flight while the matrix cores work on the fourth.
// Each load instruction writes 1 KiB of LDS linearly by lane, so the lane's
// global address picks which 16-byte chunk lands where: the four chunks of a
// 64-byte row are XOR-permuted by (row >> 3) & 3.  A 16-byte LDS read is
// serviced 16 lanes at a time, in the lane groups {0-3, 12-15, 20-27} and
// {4-11, 16-19, 28-31} of each half-wave (measured with in-bounds probes and
// the LDS bank-conflict counter), each cycle covering 64 banks = 256 bytes.
// Within a group the four rows with equal row % 4 differ in bits 3-4, so the
// permutation gives every lane of a group its own 16-byte bank slot.  The
// fragments of stage k+1 are read from LDS while the matrix cores run stage k.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int GM_THREADS = 256;
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int STAGES = 4;
constexpr int TM = 4, TN = 4;      // 32x32 sub-tiles per wave along M and N
constexpr int GROUP_M = 4;         // tile-rows walked together for L2 reuse
constexpr int STAGE_BYTES = BM * BK;  // one operand, one stage (16 KiB)
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
    int vec_store;
};

__device__ __forceinline__ int chunk_perm(int row) { return (row >> 3) & 3; }

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

// Vector-memory operations a wave issues per stage of DMA, and the scale
// words it loads per 256-K group (both 8 here, so every count below is a
// multiple of OPS_PER_STAGE).
constexpr int OPS_PER_STAGE = 2 * DMA_PER_WAVE;
static_assert(TM + TN == OPS_PER_STAGE, "wait counts assume 8 scale words per group");

// Operations issued at main-loop iteration j: the scale words of group
// j/4 + 1 (first iteration of a group) followed by the DMA of stage j + 4.
__device__ __forceinline__ int ops_at_iteration(int j, int KIT)
{
    int n = (j + STAGES < KIT) ? OPS_PER_STAGE : 0;
    if ((j & 3) == 0 && j + 4 < KIT)
        n += TM + TN;
    return n;
}

// How many vector-memory operations were issued after the DMA of stage s
// by the time iteration s-1 starts waiting for it.  Stages 0..3 are issued
// by the prologue, stage s >= 4 by iteration s-4 (after its scale words).
__device__ __forceinline__ int pending_after_stage(int s, int KIT)
{
    const int it = s - 1;
    int n = 0;
    if (s < STAGES) {
        const int last_prologue = min(KIT, STAGES) - 1;
        n += (last_prologue - s) * OPS_PER_STAGE;
        for (int j = 0; j < it; j++)
            n += ops_at_iteration(j, KIT);
    } else {
        n += ops_at_iteration(it - 2, KIT) + ops_at_iteration(it - 1, KIT);
    }
    return n;
}

template <bool GROUPED, int CT>
__global__ __launch_bounds__(GM_THREADS, 1) void mx_gemm_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(1024))) uint8_t sA[STAGES][STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[STAGES][STAGE_BYTES];
    __shared__ int64_t s_grp[3];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    // 16*(4*wave + i) .. +16 of a stage; lane -> row + lane/4, slot lane%4,
    // fetching global chunk slot ^ perm(row) of that row.
    const uint8_t *a_tile = p.a + m0 * p.ld_a;
    const uint8_t *b_tile = B + n0 * p.ld_b;
    uint32_t a_src[DMA_PER_WAVE], b_src[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; i++) {
        const int row = 16 * (DMA_PER_WAVE * wave + i) + (lane >> 2);
        const int chunk = (lane & 3) ^ chunk_perm(row);
        const int64_t ra = min(m0 + row, m_end - 1) - m0;
        const int64_t rb = min(n0 + row, N - 1) - n0;
        a_src[i] = (uint32_t)(ra * p.ld_a + chunk * 16);
        b_src[i] = (uint32_t)(rb * p.ld_b + chunk * 16);
    }
    const uint32_t lds_a0 = (uint32_t)(uintptr_t)&sA[0][0];
    const uint32_t lds_b0 = (uint32_t)(uintptr_t)&sB[0][0];
    auto dma_stage = [&](int st) {
        const int buf = st & (STAGES - 1);
        const uint8_t *a_k = a_tile + (int64_t)st * BK;
        const uint8_t *b_k = b_tile + (int64_t)st * BK;
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; i++) {
            const uint32_t off = (uint32_t)(buf * STAGE_BYTES + 1024 * (DMA_PER_WAVE * wave + i));
            __builtin_amdgcn_global_load_lds((gptr_t)(a_k + a_src[i]),
                                             (lptr_t)(uintptr_t)(lds_a0 + off), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gptr_t)(b_k + b_src[i]),
                                             (lptr_t)(uintptr_t)(lds_b0 + off), 16, 0, 0);
        }
    };

    // ---- per-lane scale words: row of this lane in each 32-row sub-tile
    const int h = lane >> 5;
    const int r32 = lane & 31;
    // the lane's row is r32 within every 32-row sub-tile; sub-tiles are 32
    // rows apart, i.e. one scale tile (KT256 * 256 bytes) apart
    const uint8_t *sa_base = p.as;
    const uint8_t *sb_base = BS;
    uint32_t sa_off[TM], sb_off[TN];
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int64_t row = min(m0 + wm * 128 + i * 32 + r32, m_end - 1);
        sa_off[i] = (uint32_t)((row >> 5) * KT256 * 256 + (h * 32 + (row & 31)) * 4);
    }
#pragma unroll
    for (int i = 0; i < TN; i++) {
        const int64_t row = min(n0 + wn * 128 + i * 32 + r32, N - 1);
        sb_off[i] = (uint32_t)((row >> 5) * KT256 * 256 + (h * 32 + (row & 31)) * 4);
    }

    // ---- per-lane LDS read offsets of the matrix-core fragments: chunk h
    // (bytes 0-15 of the operand) and chunk 2 + h (bytes 16-31) of the lane's
    // row.  Rows of the sub-tiles are 32 apart, which leaves chunk_perm
    // unchanged, so one offset serves all four (plus i * 32 rows); chunk 2 + h
    // sits in slot (h ^ perm) ^ 2, i.e. at the first offset XOR 32.
    const uint32_t la0 = (uint32_t)((wm * 128 + r32) * BK + ((h ^ chunk_perm(r32)) * 16));
    const uint32_t lb0 = (uint32_t)((wn * 128 + r32) * BK + ((h ^ chunk_perm(r32)) * 16));

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++)
                acc[i][j][v] = 0.0f;

    auto read_frags = [&](int st, v8i *xa, v8i *xb) {
        const int buf = st & (STAGES - 1);
        const uint8_t *A_ = &sA[buf][0];
        const uint8_t *B_ = &sB[buf][0];
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const uint4 lo = *reinterpret_cast<const uint4 *>(A_ + la0 + i * 32 * BK);
            const uint4 hi = *reinterpret_cast<const uint4 *>(A_ + ((la0 + i * 32 * BK) ^ 32));
            xa[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < TN; i++) {
            const uint4 lo = *reinterpret_cast<const uint4 *>(B_ + lb0 + i * 32 * BK);
            const uint4 hi = *reinterpret_cast<const uint4 *>(B_ + ((lb0 + i * 32 * BK) ^ 32));
            xb[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };

    // ---- prologue: scale words of the first 256 K, stages 0..3 in flight
    uint32_t wa[TM], wb[TN], wa_next[TM], wb_next[TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
        wa[i] = *reinterpret_cast<const uint32_t *>(sa_base + sa_off[i]);
#pragma unroll
    for (int i = 0; i < TN; i++)
        wb[i] = *reinterpret_cast<const uint32_t *>(sb_base + sb_off[i]);
#pragma unroll
    for (int st = 0; st < STAGES; st++)
        if (st < KIT)
            dma_stage(st);
    // stage 0 has landed once only the later prologue stages are outstanding
    {
        const int later = min(KIT, STAGES) - 1;
        if (later >= 3)
            MX_WAIT_VMCNT(3 * OPS_PER_STAGE);
        else if (later == 2)
            MX_WAIT_VMCNT(2 * OPS_PER_STAGE);
        else if (later == 1)
            MX_WAIT_VMCNT(1 * OPS_PER_STAGE);
        else
            MX_WAIT_VMCNT(0);
    }
    lds_ring_barrier();
    v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    read_frags(0, fa0, fb0);

    // One iteration `it`: the fragments of stage it are in registers (CUR);
    // wait for stage it+1, barrier, issue [scale words of the next 256-K
    // group, on the group's first iteration] then [DMA of stage it+4], read
    // stage it+1's fragments (NXT) and run stage it on the matrix cores.
#define MX_STEP(POS, CUR_A, CUR_B, NXT_A, NXT_B)                                              \
    {                                                                                        \
        const int it = kg + (POS);                                                           \
        if (it < KIT) {                                                                      \
            if (it + 1 < KIT) {                                                              \
                const int pend = pending_after_stage(it + 1, KIT);                           \
                if (pend >= 3 * OPS_PER_STAGE)                                               \
                    MX_WAIT_VMCNT(3 * OPS_PER_STAGE);                                        \
                else if (pend >= 2 * OPS_PER_STAGE)                                          \
                    MX_WAIT_VMCNT(2 * OPS_PER_STAGE);                                        \
                else if (pend >= OPS_PER_STAGE)                                              \
                    MX_WAIT_VMCNT(OPS_PER_STAGE);                                            \
                else                                                                         \
                    MX_WAIT_VMCNT(0);                                                        \
            }                                                                                \
            lds_ring_barrier();                                                              \
            if ((POS) == 0 && it + 4 < KIT) {                                                \
                const int64_t kw = (int64_t)((it + 4) >> 2) * 256;                           \
                _Pragma("unroll") for (int i = 0; i < TM; i++)                               \
                    wa_next[i] = *reinterpret_cast<const uint32_t *>(sa_base + kw + sa_off[i]); \
                _Pragma("unroll") for (int i = 0; i < TN; i++)                               \
                    wb_next[i] = *reinterpret_cast<const uint32_t *>(sb_base + kw + sb_off[i]); \
            }                                                                                \
            if (it + STAGES < KIT)                                                           \
                dma_stage(it + STAGES);                                                      \
            if (it + 1 < KIT)                                                                \
                read_frags(it + 1, NXT_A, NXT_B);                                            \
            _Pragma("unroll") for (int i = 0; i < TN; i++) {                                 \
                const int sbv = (int)(wb[i] >> (8 * (POS)));                                 \
                _Pragma("unroll") for (int j = 0; j < TM; j++)                               \
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(             \
                        CUR_B[i], CUR_A[j], acc[i][j], 0, 0, 0, sbv, 0,                      \
                        (int)(wa[j] >> (8 * (POS))));                                        \
            }                                                                                \
        }                                                                                    \
    }

    for (int kg = 0; kg < KIT; kg += 4) {
        MX_STEP(0, fa0, fb0, fa1, fb1)
        MX_STEP(1, fa1, fb1, fa0, fb0)
        MX_STEP(2, fa0, fb0, fa1, fb1)
        MX_STEP(3, fa1, fb1, fa0, fb0)
        if (kg + 4 < KIT) {
#pragma unroll
            for (int i = 0; i < TM; i++)
                wa[i] = wa_next[i];
#pragma unroll
            for (int i = 0; i < TN; i++)
                wb[i] = wb_next[i];
        }
    }
#undef MX_STEP

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
    p.bs_group_stride = ((N + 31) / 32) * ((K / 32 + 7) / 8) * 256;
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
