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
// lane, held in AGPRs).  K advances 64 per stage (one matrix-core step)
// through a ring of four LDS stages (A and B: 256 rows x 64 bytes each, 32
// KiB per stage; 128 KiB in all), one barrier per stage.  Operands travel
// in pairs of stages: the 128 bytes of a row that two stages need are one
// cache line, loaded by one 16-byte-per-lane load instruction per 8 rows
// into registers, and written to the ring two stages later, when both of
// their ring stages are free.  Whole-line requests keep the load path's
// request count at one per line (loading each 64-byte half on its own
// doubled it and saturated the texture address unit), and staging through
// registers lets a pair's loads go out while the ring is still full, spread
// over the stage, with two stages of time to land.
// In LDS the four 16-byte chunks of a 64-byte row are XOR-permuted by
// (row >> 2) & 3.  A 16-byte LDS read is serviced 16 lanes at a time, in the
// lane groups {0-3, 12-15, 20-27} and {4-11, 16-19, 28-31} of each half-wave
// (measured with in-bounds probes and the LDS bank-conflict counter), each
// cycle covering 64 banks = 256 bytes = four rows; the four rows of each
// residue mod 4 in a group differ in (row >> 2) & 3, so every lane of a
// group gets its own 16-byte bank slot.  The A fragments of the next stage
// are read while the matrix cores run the current one; the B fragments one
// sub-tile ahead.
#include "mx_device.h"
#include "mx_launch.h"
#include "mx_plan.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

namespace mx {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256;
constexpr int BK = 64;             // K bytes per stage: one matrix-core step
constexpr int NBUF = 4;            // stages in the LDS ring (one 256-K group)
constexpr int GM_THREADS = 256;    // 4 waves, one per SIMD, 2x2 over the tile
constexpr int TM = 4, TN = 4;      // 32x32 sub-tiles per wave along M and N (128x128)
constexpr int GROUP_M = 4;         // tile-rows walked together for L2 reuse
constexpr int STAGE_BYTES = BM * BK;  // one operand, one stage (16 KiB)

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
    int vec_store;  // C rows allow 4-element vector stores
    int vec16;      // BF16 C: rows allow 16-byte stores (8 elements)
    // Split tail (dense only): tiles dp_tiles .. dp_tiles + split_tiles - 1
    // are each cut into split_s K ranges of whole 256-K groups, one workgroup
    // per range.  Each range writes its FP32 partial tile to ws (slot
    // tile * split_s + range, BM * BN floats); split_reduce_kernel then sums
    // the slots of each tile in range order and writes C.
    int64_t dp_tiles;
    int split_tiles, split_s;
    float *ws;
    // K-grouped: the tile counter the workgroups take tiles from after their
    // first (zero at launch)
    int *counter;
};

// The 16-byte slot of a 64-byte LDS row that holds chunk c is c ^ chunk_perm(row).
__device__ __forceinline__ int chunk_perm(int row) { return (row >> 2) & 3; }

// Two FP32 -> packed BF16 (low half first), round to nearest even: one
// v_cvt_pk_bf16_f32 on this target (NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{lo, hi}), bf16x2_t));
}


// Values every lane holds alike, moved to scalar registers.
__device__ __forceinline__ int64_t uniform(int64_t x)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <typename T> __device__ __forceinline__ const T *uniform(const T *x)
{
    return reinterpret_cast<const T *>(uniform((int64_t)(uintptr_t)x));
}

// A wave-uniform value the compiler must take as unknown at this point, so
// that what it derives from it (a divisor's reciprocal) is formed where it is
// used and not kept in vector registers across the main loop.
__device__ __forceinline__ int64_t opaque(int64_t x)
{
    asm volatile("" : "+s"(x));
    return x;
}

// Tile t of a GROUP_M-row band walk over tiles_m x tiles_n tiles -> (m, n):
// the bands of GROUP_M tile-rows are taken in turn, and within a band the
// tiles column by column.  t < GROUP_M * tiles_n * ceil(tiles_m / GROUP_M)
// and tiles_n < 2^21, so the in-band index fits 32 bits; the band height
// (GROUP_M, less for the last band) is 1 to 4, divided by shifts or by the
// exact multiply-high for 3.
__device__ __forceinline__ void band_walk(int64_t t, int64_t tiles_m, int64_t tiles_n, int64_t &m,
                                          int64_t &n)
{
    static_assert(GROUP_M == 4, "the band division below assumes bands of at most 4 tile-rows");
    const int64_t per_band = opaque(GROUP_M * tiles_n);
    const int64_t band = t / per_band;
    const int64_t first_m = band * GROUP_M;
    const uint32_t gm = (uint32_t)min(tiles_m - first_m, (int64_t)GROUP_M);
    const uint32_t in = (uint32_t)(t - band * per_band);
    const uint32_t q = gm == 4   ? in >> 2
                       : gm == 2 ? in >> 1
                       : gm == 1 ? in
                                 : (uint32_t)(((uint64_t)in * 0xAAAAAAABull) >> 33);
    m = first_m + (int64_t)(in - q * gm);
    n = (int64_t)q;
}

// Workgroup barrier for the LDS ring.  __syncthreads() would also wait for
// every outstanding vector-memory load (its release fence is conservative),
// draining the register prefetch each stage.  The ring is only written and
// read with LDS instructions, so each wave waits for its own LDS writes and
// reads and then meets the others; the "memory" clobber keeps the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_ring_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Coordinates of one 256x256 output tile, and the 64-K stages of it a unit
// of work covers: ns stages from stage kb (both multiples of 4: whole 256-K
// groups).
// (32-bit fields: row and column counts are below 2^29, experts at most
// 1024; a workgroup holds three tiles at a time in scalar registers.)
struct Tile {
    int m0, n0, m_end;
    int g;  // expert (grouped modes), else 0
    int kb, ns;
    int sp;  // split-tail slot (tile * split_s + range), or -1 for a whole tile
};

constexpr int GROUP_TABLE = 1024;  // experts whose tile table fits in LDS

// MODE: 0 dense; 1 grouped along M (rows of A sorted by expert, expert g's
// rows multiply B_g); 2 grouped along K (the per-expert weight gradient:
// expert g contracts the K range [offsets[g], offsets[g+1]) of A and B, both
// 256-aligned, into its own C_g = C + g * M * ld_c).
// SPLIT: the launch has a split tail (dense, BF16 C only).  A separate
// instantiation, since carrying that path costs the other launches 1-4 %.
template <int MODE, int CT, bool SPLIT>
__global__ __launch_bounds__(GM_THREADS, 1) void mx_gemm_kernel(GemmParams p)
{
    constexpr bool GROUPED = MODE == 1;
    constexpr bool KGROUPED = MODE == 2;
    constexpr int NW = 4, WN = 128;  // waves; columns of C per wave
    __shared__ __attribute__((aligned(1024))) uint8_t sA[NBUF][STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t sB[NBUF][STAGE_BYTES];
    // grouped: per expert g, its first m-tile number and its clamped row range
    // K-grouped: per expert g its stage range [s_lo[g], s_hi[g]), and s_pref[r]
    // the expert of rank r by decreasing stage count
    constexpr bool TABLE = GROUPED || KGROUPED;
    __shared__ int s_pref[TABLE ? GROUP_TABLE + 1 : 1];
    __shared__ int s_lo[TABLE ? GROUP_TABLE : 1], s_hi[TABLE ? GROUP_TABLE : 1];
    __shared__ int s_wsum[NW];
    __shared__ int64_t s_next[2];  // K-grouped: tiles taken ahead

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int h = lane >> 5;
    const int r32 = lane & 31;
    const int64_t N = p.N;
    const int64_t KT256 = (p.K + 255) / 256;  // scale words per 32-row tile
    const int KIT = (int)(p.K / BK);
    const int KITP = (KIT + 3) & ~3;  // stages per tile, padded to whole 256-K groups

    // ---- tile enumeration
    int64_t ntiles;
    if (KGROUPED) {
        // Stage ranges, clamped so that every expert has at least one 256-K
        // group inside [0, K) whatever the offsets hold (for offsets that are
        // 256-aligned and at least 256 apart, as mx_quantize_colwise_grouped
        // writes them, the clamps change nothing).  An expert with no rows
        // then contracts its zero padding and writes a zero C_g.
        const int G = (int)p.G;
        const int KG = (int)(p.K / 256);
        for (int g = tid; g < G; g += GM_THREADS) {
            const int64_t lo = min(max(p.offsets[g], (int64_t)0), p.K);
            const int64_t hi = min(max(p.offsets[g + 1], lo), p.K);
            const int glo = min((int)(lo / 256), KG - 1);
            const int ghi = min(max((int)((hi + 255) / 256), glo + 1), KG);
            s_lo[g] = 4 * glo;
            s_hi[g] = 4 * ghi;
        }
        __syncthreads();
        // rank by decreasing stage count (ties by expert number): tiles are
        // dealt longest first
        for (int g = tid; g < G; g += GM_THREADS) {
            const int ns = s_hi[g] - s_lo[g];
            int rank = 0;
            for (int h = 0; h < G; h++) {
                const int nh = s_hi[h] - s_lo[h];
                rank += (nh > ns || (nh == ns && h < g)) ? 1 : 0;
            }
            s_pref[rank] = g;
        }
        __syncthreads();
        ntiles = p.G * p.tiles_m * p.tiles_n;
    } else if (!GROUPED) {
        ntiles = p.tiles_m * p.tiles_n;
    } else {
        // (p.G <= GROUP_TABLE: the library takes at most that many experts)
        // each thread takes a contiguous run of experts; block-wide exclusive
        // scan of their m-tile counts (ceil(rows / BM))
        const int G = (int)p.G;
        const int per = (G + GM_THREADS - 1) / GM_THREADS;
        const int g0 = tid * per, g1 = min(g0 + per, G);
        int sum = 0;
        for (int g = g0; g < g1; g++) {
            const int64_t lo = min(max(p.offsets[g], (int64_t)0), p.M);
            const int64_t hi = min(max(p.offsets[g + 1], lo), p.M);
            s_lo[g] = (int)lo;
            s_hi[g] = (int)hi;
            sum += (int)((hi - lo + BM - 1) / BM);
        }
        int incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d)
                incl += o;
        }
        if (lane == 63)
            s_wsum[wave] = incl;
        __syncthreads();
        int run = incl - sum;
        for (int w = 0; w < wave; w++)
            run += s_wsum[w];
        for (int g = g0; g < g1; g++) {
            s_pref[g] = run;
            run += (s_hi[g] - s_lo[g] + BM - 1) / BM;
        }
        if (tid == GM_THREADS - 1) {
            int tot = 0;
            for (int w = 0; w < NW; w++)
                tot += s_wsum[w];
            s_pref[G] = tot;
        }
        __syncthreads();
        ntiles = (int64_t)s_pref[G] * p.tiles_n;
    }
    // Workgroups are dealt to the 8 XCDs in turn (workgroup b runs on XCD
    // b % 8), and each XCD has its own L2: give XCD x a contiguous eighth of
    // the tiles, walked by its workgroups in step, so that tiles running
    // together on one XCD share A and B panels.
    // A split tail's units are dealt the same way: XCD x takes a contiguous
    // eighth of them, so the K ranges of one tile run on one XCD.
    const int64_t whole = TABLE ? ntiles : p.dp_tiles;
    int64_t t_first, t_step, t_end;
    if (gridDim.x % 8 == 0) {
        const int64_t x = blockIdx.x & 7, per_xcd = (whole + 7) / 8;
        t_first = x * per_xcd + (blockIdx.x >> 3);
        t_step = gridDim.x >> 3;
        t_end = min((x + 1) * per_xcd, whole);
    } else {
        t_first = blockIdx.x;
        t_step = gridDim.x;
        t_end = whole;
    }
    int64_t my_tiles = t_first < t_end ? (t_end - t_first + t_step - 1) / t_step : 0;
    // K-grouped: tiles in rank order (an expert's tiles together, longest
    // experts first).  Tile v of the first P = gridDim.x goes to virtual slot
    // v, which runs on workgroup (v mod P/8) * 8 + v / (P/8), so neighbouring
    // tiles of one expert share an XCD and its L2.  After that a workgroup
    // takes the next tile in rank order from a counter when it is two tiles
    // from needing it (its next two tiles must be known: the loads of a
    // tile's first stages run during the previous tile), so the longest
    // remaining tiles go to the workgroups that free up first.
    const int64_t P = gridDim.x;
    int64_t vslot = blockIdx.x;
    int64_t t_nxt = 0;  // K-grouped: the tile after the current one
    if (KGROUPED) {
        if (P % 8 == 0)
            vslot = (int64_t)(blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);
        my_tiles = INT64_MAX;  // ended by the loop once no tile is left
        if (tid == 0) {
            s_next[1] = P + __hip_atomic_fetch_add(p.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_next[0] = P + __hip_atomic_fetch_add(p.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        t_nxt = uniform(s_next[1]);
    }
    int split_u = -1;  // this workgroup's split-tail unit
    if (SPLIT) {
        const int64_t u = gridDim.x % 8 == 0 ? (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                                             : (int64_t)blockIdx.x;
        if (u < (int64_t)p.split_tiles * p.split_s)
            split_u = (int)u;
    }
    const int has_split = split_u >= 0 ? 1 : 0;
    const int64_t my_units = my_tiles + has_split;
    if (my_units == 0)
        return;

    // tile number -> coordinates
    int g_cur = 0;  // grouped: experts are met in increasing order
    auto coords = [&](int64_t pid) -> Tile {
        Tile c;
        if (KGROUPED) {
            const uint32_t per_expert = (uint32_t)opaque(p.tiles_m * p.tiles_n);
            const int64_t r = (uint32_t)pid / per_expert;  // (32-bit: tile numbers are below 2^31)
            const int g = __builtin_amdgcn_readfirstlane(s_pref[r]);
            int64_t mt, nt;
            band_walk(pid - r * per_expert, p.tiles_m, p.tiles_n, mt, nt);
            c.m0 = (int)(mt * BM);
            c.n0 = (int)(nt * BN);
            c.m_end = (int)p.M;
            c.g = g;
            c.kb = __builtin_amdgcn_readfirstlane(s_lo[g]);
            c.ns = __builtin_amdgcn_readfirstlane(s_hi[g]) - c.kb;
            return c;
        }
        if (!GROUPED) {
            int64_t mt, nt;
            band_walk(pid, p.tiles_m, p.tiles_n, mt, nt);
            c.m0 = (int)(mt * BM);
            c.n0 = (int)(nt * BN);
            c.m_end = (int)p.M;
            c.g = 0;
            return c;
        }
        // (32-bit: tile numbers and counts are below 2^31)
        const uint32_t tn = (uint32_t)opaque(p.tiles_n), pid32 = (uint32_t)pid;
        const uint32_t mt32 = pid32 / tn;
        c.n0 = (int)((pid32 - mt32 * tn) * BN);
        const int mt = (int)mt32;
        // first expert whose tiles end beyond mt, searching forward from the
        // last one found (a workgroup's tiles come in increasing order); pid <
        // ntiles guarantees a hit, and the loop is bounded either way
        const int G = (int)p.G;
        if (s_pref[g_cur] > mt)
            g_cur = 0;
        int found = -1;
        for (int gb = g_cur; gb < G && found < 0; gb += 64) {
            const int gg = gb + lane;
            const uint64_t m = __ballot(gg < G && s_pref[gg + 1] > mt);
            if (m)
                found = gb + __builtin_ctzll(m);
        }
        g_cur = found < 0 ? G - 1 : found;
        const int g = g_cur;
        c.m0 = __builtin_amdgcn_readfirstlane(s_lo[g] + (mt - s_pref[g]) * BM);
        c.m_end = __builtin_amdgcn_readfirstlane(s_hi[g]);
        c.g = __builtin_amdgcn_readfirstlane(g);
        return c;
    };
    // a tile's B operand and its rearranged scales (per expert when grouped
    // by rows)
    auto b_of = [&](const Tile &T) -> const uint8_t * {
        return GROUPED ? p.b + (int64_t)T.g * p.b_group_stride : p.b;
    };
    auto bs_of = [&](const Tile &T) -> const uint8_t * {
        return GROUPED ? p.bs + (int64_t)T.g * p.bs_group_stride : p.bs;
    };
    // unit k of this workgroup: its split-tail unit first, then whole tiles
    auto unit = [&](int64_t k) -> Tile {
        if (SPLIT && has_split && k == 0) {
            const int r = split_u / p.split_s, sidx = split_u - r * p.split_s;
            Tile c = coords(p.dp_tiles + r);
            const int KG = KITP / 4;  // 256-K groups
            const int g0 = (int)((int64_t)sidx * KG / p.split_s);
            const int g1 = (int)((int64_t)(sidx + 1) * KG / p.split_s);
            c.kb = 4 * g0;
            c.ns = 4 * (g1 - g0);
            c.sp = split_u;
            return c;
        }
        if (KGROUPED) {  // the first unit only; later ones come from the counter
            Tile c = coords(vslot);
            c.sp = -1;
            return c;
        }
        Tile c = coords(t_first + (k - has_split) * t_step);
        c.kb = 0;
        c.ns = KITP;
        c.sp = -1;
        return c;
    };

    // ---- operand loads.  Two consecutive stages of a tile (128 K: one
    // 128-byte cache line of each row) of A and of B are loaded together
    // into registers, 16 bytes per lane and instruction, and written to the
    // LDS ring two stages later.  Instruction i of this wave covers rows
    // 8*wave + 32*i .. +8 of an operand: lane l takes row (l & 31) / 4 of
    // them and chunk (l & 3) + 4 * (l / 32) of the row's 128 bytes, so each
    // half-wave holds one stage of the pair (one 64-byte half of every row)
    // and writes it to its ring stage as 8 consecutive 64-byte LDS rows.  In
    // LDS chunk c of a row sits in slot c ^ perm(row) (rows 32 apart share
    // the permutation, so one offset register serves all eight
    // instructions); a half-wave's 32 lanes then cover 8 rows x 4 slots,
    // every 16-lane service group distinct 16-byte bank slots.  Rows past
    // the operand (or past the expert, which are never stored) need no clamp:
    // the tile's buffer range ends at the operand's last row and reads beyond
    // it return zero.
    constexpr int PAIR_LOADS = 2 * (BM / 32);  // per wave: 8 of A, 8 of B
    const int prow = 8 * wave + ((lane & 31) >> 2);
    const int pchunk = (lane & 3) + 4 * (lane >> 5);
    const uint32_t a_src = (uint32_t)(prow * p.ld_a + pchunk * 16);
    const uint32_t b_src = (uint32_t)(prow * p.ld_b + pchunk * 16);
    const uint32_t a_step = (uint32_t)(32 * p.ld_a), b_step = (uint32_t)(32 * p.ld_b);
    const uint32_t w_off = (uint32_t)((lane >> 5) * STAGE_BYTES + prow * BK +
                                      (((lane & 3) ^ chunk_perm(prow)) * 16));
    // Loads of stages st, st + 1 (st even) of tile T, load q into R[q] (A
    // rows for q < 8, then B rows).  A pair past the end or of padding (live
    // false) gets an empty range and loads zeros, which keeps the main loop
    // branch-free.  (32-bit sizes: row counts are below 2^29; a 64-bit
    // compare would need a vector register for a uniform value.)
    auto pair_load_one = [&](const Tile &T, int st, bool live, v4i *R, int q) {
        const uint32_t ab = (uint32_t)min((int)(p.M - T.m0), BM) * (uint32_t)p.ld_a;
        const uint32_t bb = (uint32_t)min((int)(N - T.n0), BN) * (uint32_t)p.ld_b;
        const uint32_t koff = (uint32_t)(T.kb + st) * BK;
        if (q < PAIR_LOADS / 2)
            R[q] = __builtin_amdgcn_raw_buffer_load_b128(byte_range(p.a + (int64_t)T.m0 * p.ld_a, live ? ab : 0u),
                                                         a_src + (uint32_t)q * a_step, koff, 0);
        else
            R[q] = __builtin_amdgcn_raw_buffer_load_b128(byte_range(b_of(T) + (int64_t)T.n0 * p.ld_b, live ? bb : 0u),
                                                         b_src + (uint32_t)(q - PAIR_LOADS / 2) * b_step, koff, 0);
    };
    auto pair_loads = [&](const Tile &T, int st, bool live, v4i *R) {
#pragma unroll
        for (int q = 0; q < PAIR_LOADS; q++)
            pair_load_one(T, st, live, R, q);
    };
    // write R[q] of a pair into ring stages t0, t0 + 1
    auto pair_write_one = [&](int t0, const v4i *R, int q) {
        uint8_t *base = q < PAIR_LOADS / 2 ? &sA[0][0] : &sB[0][0];
        *reinterpret_cast<v4i *>(base + t0 * STAGE_BYTES + w_off + (q % (PAIR_LOADS / 2)) * 32 * BK) = R[q];
    };

    // ---- scale words.  Per 256-K group the lane (h, r) supplies, for A
    // sub-tile i, the word of row m0 + wm*128 + 32i + r: entry 32h + (row &
    // 31) of the row's 32-row scale tile, whose group g sits at g * 256
    // within the tile's KT256 * 256 bytes (likewise for B).  Each is one
    // 4-byte load into a register, a group ahead.  Rows past the operand fall
    // outside the resource's range and read zero.
    const uint32_t stile = (uint32_t)(KT256 * 256);  // bytes per 32-row scale tile (below 2^32)
    struct ScaleLanes {
        uint32_t a, b;  // the lane's offsets for sub-tile 0 (sub-tile i adds i * stile)
    };
    auto scale_lanes = [&](const Tile &T) -> ScaleLanes {
        const int x = (int)(T.m0 & 31) + r32;
        const int ta = (int)(T.m0 >> 5) + wm * 4 + (x >> 5), tb = (int)(T.n0 >> 5) + wn * (WN / 32);
        return ScaleLanes{(uint32_t)ta * stile + (uint32_t)((h * 32 + (x & 31)) * 4),
                          (uint32_t)tb * stile + (uint32_t)((h * 32 + r32) * 4)};
    };
    auto load_scales = [&](const Tile &T, const ScaleLanes &S, int group, bool live, uint32_t *xa,
                           uint32_t *xb) {
        const __amdgpu_buffer_rsrc_t rsa = byte_range(p.as, live ? p.as_bytes : 0u);
        const __amdgpu_buffer_rsrc_t rsb = byte_range(bs_of(T), live ? p.bs_bytes : 0u);
        // scalar offset, within the row's scale tile (readfirstlane: the
        // compiler may select the tile's fields in vector registers, and a
        // vector soffset would become a loop over distinct values)
        const uint32_t kw = __builtin_amdgcn_readfirstlane((uint32_t)group * 256);
#pragma unroll
        for (int i = 0; i < TM; i++)
            xa[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsa, S.a + (uint32_t)i * stile, kw, 0);
#pragma unroll
        for (int i = 0; i < TN; i++)
            xb[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsb, S.b + (uint32_t)i * stile, kw, 0);
    };
    static_assert(TN % 2 == 0, "BF16 stores pair adjacent sub-tiles");

    // ---- per-lane LDS read offsets of the matrix-core fragments.  The lane
    // needs chunk h (bytes 0-15 of the operand) and chunk 2 + h (bytes
    // 16-31) of its row's 64 bytes.  Rows of the sub-tiles are 32 apart,
    // which leaves chunk_perm unchanged, and chunk 2 + h sits in the slot of
    // chunk h XOR 2, so the second read is at the first offset XOR 32.  The
    // sub-tile and the ring buffer are immediate offsets of the LDS read.
    const uint32_t a_lo = (uint32_t)((wm * 128 + r32) * BK + ((h ^ chunk_perm(r32)) * 16));
    const uint32_t b_lo = (uint32_t)((wn * WN + r32) * BK + ((h ^ chunk_perm(r32)) * 16));
    const uint32_t a_hi = a_lo ^ 32u, b_hi = b_lo ^ 32u;
    // A sub-tile i (rows wm*128 + 32i ..) and B sub-tile i of ring buffer buf
    auto read_a = [&](int buf, int i) -> v8i {
        const uint8_t *A_ = &sA[buf][0] + i * 32 * BK;
        const v4i lo = *reinterpret_cast<const v4i *>(A_ + a_lo);
        const v4i hi = *reinterpret_cast<const v4i *>(A_ + a_hi);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_b = [&](int buf, int i) -> v8i {
        const uint8_t *B_ = &sB[buf][0] + i * 32 * BK;
        const v4i lo = *reinterpret_cast<const v4i *>(B_ + b_lo);
        const v4i hi = *reinterpret_cast<const v4i *>(B_ + b_hi);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    v16f acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int v = 0; v < 16; v++)
                acc[i][j][v] = 0.0f;

    // Per-lane offset of C within a tile for band j = 0: row wm*128 + r32,
    // columns from wn*WN + 4h.  Band j adds j * c_band, wave-uniform (the
    // sub-tile and register group add immediates), so one register serves
    // every band.  The row offsets stay in the vector offset, which the
    // buffer range check covers (the scalar offset is added after it).
    constexpr int CE = CT == 0 ? 2 : 4;  // bytes per C element
    const uint32_t c_band = (uint32_t)(32 * p.ld_c * CE);
    // BF16 C is stored after three lane exchanges (see the epilogue): lane l
    // writes 8 columns, chunk k = ((l >> 5) & 1) | (((l >> 4) & 1) << 1) of
    // sub-tile pair half (l >> 3) & 1, of row l & 7 of an 8-row quarter of the
    // pair's 32-row band (rows 0-7; rows 8-15, 16-23 and 24-31 add scalar
    // offsets too).
    uint32_t c_off;
    if (CT == 0) {
        const int row = wm * 128 + (lane & 7);
        const int col = wn * WN + ((lane >> 3) & 1) * 32 + (((lane >> 5) & 1) | (((lane >> 4) & 1) << 1)) * 8;
        c_off = (uint32_t)((row * p.ld_c + col) * CE);
    } else {
        c_off = (uint32_t)(((wm * 128 + r32) * p.ld_c + wn * WN + 4 * h) * CE);
    }

    // ---- the workgroup's stages: its units' stages numbered continuously,
    // so the pipeline runs across units.  Every unit has a multiple of 4
    // stages, so stage u of the sequence uses ring buffer u % 4, which is
    // also its position t in its 256-K group.
    Tile cur = unit(0);
    ScaleLanes cur_sl = scale_lanes(cur);

    // prologue: stages 0 and 1 into the ring, stages 2 and 3 into registers,
    // the first group's scale words; then stage 0's fragments
    v4i R[PAIR_LOADS];
    pair_loads(cur, 0, cur.kb < KIT, R);
#pragma unroll
    for (int q = 0; q < PAIR_LOADS; q++)
        pair_write_one(0, R, q);
    pair_loads(cur, 2, cur.kb + 2 < KIT, R);
    // the unit after the current one (K-grouped: taken from the counter)
    bool nxt_ok;
    Tile nxt;
    if (KGROUPED) {
        nxt_ok = t_nxt < ntiles;
        nxt = nxt_ok ? coords(t_nxt) : cur;
    } else {
        nxt_ok = 1 < my_units;
        nxt = nxt_ok ? unit(1) : cur;
    }
    uint32_t wa[TM], wb[TN], na[TM], nb[TN];
    load_scales(cur, cur_sl, cur.kb >> 2, true, wa, wb);
    lds_ring_barrier();
    // The A fragments of a stage are read during the previous stage (two
    // register sets, alternating); the B fragments one sub-tile ahead: the
    // first during the previous stage, sub-tile i + 1 while the instructions
    // of sub-tile i run.
    v8i fa0[TM], fa1[TM], fb_first;
#pragma unroll
    for (int i = 0; i < TM; i++)
        fa0[i] = read_a(0, i);
    fb_first = read_b(0, 0);


    // BF16 stores of one 32-row band j of the wave's C, sub-tile i in x[i].
    // Register group q of lane (h, r) holds columns 8q + 4h .. +3 of
    // row r (r = lane & 31) as two packed words.  Swapping group 1 of
    // the lower half-wave with group 0 of the upper one
    // (v_permlane32_swap), and group 3 with group 2, leaves lane
    // (h, r) with 16-byte chunks h (columns 8h..8h+7) in s1 and 2 + h
    // in s2.  Swapping the odd 16-lane rows of s1 with the even ones of
    // s2 (v_permlane16_swap) then gathers all four chunks of rows 0-15
    // in s1 and of rows 16-31 in s2, lane l holding row l & 15.  Last,
    // within each 16-lane row, lanes 8-15 of sub-tile i trade with
    // lanes 0-7 of sub-tile i + 1 (DPP row shifts by 8, bank-masked):
    // then one store writes whole 128-byte lines, 64 bytes of each of
    // the two sub-tiles, of 8 rows.
    // The stores are non-temporal.  C is never read back here, and
    // with the default policy each round of tiles' output fills the
    // L2 and evicts the operand panels that the next round reuses;
    // streaming whole lines keeps them resident.
    auto store_band = [&](const __amdgpu_buffer_rsrc_t &rc, uint32_t cb, int j, const v16f *x) {
        const uint32_t row8 = (uint32_t)(8 * p.ld_c * CE);
        {
            uint32_t s1[TN][4], s2[TN][4];
#pragma unroll
            for (int i = 0; i < TN; i++) {
                uint32_t w[4][2];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    w[q][0] = pack_bf16x2(x[i][4 * q + 0], x[i][4 * q + 1]);
                    w[q][1] = pack_bf16x2(x[i][4 * q + 2], x[i][4 * q + 3]);
                }
#pragma unroll
                for (int q = 0; q < 4; q += 2) {
#pragma unroll
                    for (int d = 0; d < 2; d++) {
                        const auto sw = __builtin_amdgcn_permlane32_swap(w[q][d], w[q + 1][d],
                                                                         false, false);
                        w[q][d] = sw[0];
                        w[q + 1][d] = sw[1];
                    }
                }
                const uint32_t t1[4] = {w[0][0], w[0][1], w[1][0], w[1][1]};
                const uint32_t t2[4] = {w[2][0], w[2][1], w[3][0], w[3][1]};
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const auto sw = __builtin_amdgcn_permlane16_swap(t1[d], t2[d], false, false);
                    s1[i][d] = sw[0];
                    s2[i][d] = sw[1];
                }
            }
#pragma unroll
            for (int i = 0; i < TN; i += 2) {
                // row_shr:8 into lanes 8-15 (banks 2, 3), row_shl:8 into lanes 0-7
                uint32_t x1[4], y1[4], x2[4], y2[4];
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    x1[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)s1[i][d], (int)s1[i + 1][d],
                                                                  0x118, 0xF, 0xC, false);
                    y1[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)s1[i + 1][d], (int)s1[i][d],
                                                                  0x108, 0xF, 0x3, false);
                    x2[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)s2[i][d], (int)s2[i + 1][d],
                                                                  0x118, 0xF, 0xC, false);
                    y2[d] = (uint32_t)__builtin_amdgcn_update_dpp((int)s2[i + 1][d], (int)s2[i][d],
                                                                  0x108, 0xF, 0x3, false);
                }
                const uint32_t col = (uint32_t)(i * 32 * CE);
                constexpr int NT = 2;  // cache policy: non-temporal
                const uint32_t o = cb + (uint32_t)j * c_band + col;
                __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]},
                                                       rc, o, 0, NT);
                __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)y1[0], (int)y1[1], (int)y1[2], (int)y1[3]},
                                                       rc, o + row8, 0, NT);
                __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)x2[0], (int)x2[1], (int)x2[2], (int)x2[3]},
                                                       rc, o + 2 * row8, 0, NT);
                __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)y2[0], (int)y2[1], (int)y2[2], (int)y2[3]},
                                                       rc, o + 3 * row8, 0, NT);
            }
        }
    };

    // Stage u of the sequence (64 K) uses ring buffer u % 4 = t, its
    // position in its 256-K group, and byte t of the group's scale words.
    // On entry its fragments are in registers (set t & 1) and stage u+1 is
    // in the ring for every wave.  While the stage's 16 matrix-core
    // instructions run, the wave
    //   - at even t, writes the pair of stages u+2, u+3 that it loaded at
    //     stage u-2 into ring buffers (t+2) % 4 and (t+3) % 4 (their
    //     fragments were read at stages u-3 and u-2, before the last
    //     barrier), and loads the pair u+4, u+5 into the same registers, one
    //     128-byte line of each row: the load path sees a steady stream of
    //     whole-line requests, each with two stages' time to land;
    //   - at t = 3, loads the next group's scale words (consumed at the next stage);
    //   - reads stage u+1's fragments into the other register set.
    // A barrier then makes this wave's LDS writes and reads complete for
    // every wave.  The compiler places the waits for the loads, which only
    // feed registers.  Past the end the loads are empty (their range is) and
    // the fragment reads unused, so the body has no branches.  After a
    // unit's last stage its accumulators are stored and cleared.
    for (int64_t k = 0; k < my_units; k++) {
        // nxt: the unit after this one (loaded during this unit's last group)
        const ScaleLanes nxt_sl = scale_lanes(nxt);
        const int ng = cur.ns >> 2;  // 256-K groups of this unit
        auto group = [&](int gi) {
            // the next group: of this unit, or the next unit's first (every
            // unit has at least one); it exists when it is in this unit or a
            // next unit exists
            const bool same = gi + 1 < ng;
            const Tile &ld = same ? cur : nxt;
            const ScaleLanes &ld_sl = same ? cur_sl : nxt_sl;
            const int st4 = same ? 4 * (gi + 1) : 0;  // its first stage within ld
            const bool live = same || nxt_ok;
            auto stage = [&](auto T_) {
                constexpr int t = decltype(T_)::value;
                v8i *FA = (t & 1) ? fa1 : fa0, *NA = (t & 1) ? fa0 : fa1;
                constexpr int nbuf = (t + 1) & 3;  // the next stage's buffer
                const bool pl = live && ld.kb + st4 + t < KIT;
                constexpr bool pairs = t == 0 || t == 2;
                if (t == 3)
                    load_scales(ld, ld_sl, (ld.kb + st4) >> 2, live, na, nb);
                // Per B sub-tile i: read B sub-tile i + 1 (or the next
                // stage's first) and the next stage's A sub-tile i, then at
                // even t a quarter of the pair writes and loads, while the
                // four matrix-core instructions of row i run.  LDS writes and
                // reads stay in program order (the compiler cannot tell the
                // ring buffers apart), so reads come first in each row.
                v8i xb = fb_first;
#pragma unroll
                for (int i = 0; i < TN; i++) {
                    const v8i xn = i + 1 < TN ? read_b(t, i + 1) : read_b(nbuf, 0);
                    NA[i] = read_a(nbuf, i);
                    if (pairs) {
#pragma unroll
                        for (int q = 4 * i; q < 4 * i + 4; q++) {
                            pair_write_one((t + 2) & 3, R, q);
                            pair_load_one(ld, st4 + t, pl, R, q);
                        }
                    }
                    const int sbv = (int)(wb[i] >> (8 * t));
#pragma unroll
                    for (int j = 0; j < TM; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            xb, FA[j], acc[i][j], 0, 0, 0, sbv, 0, (int)(wa[j] >> (8 * t)));
                    xb = xn;
                }
                fb_first = xb;
#pragma unroll
                for (int i = 0; i < TN; i++) {  // per row: 4 matrix-core, 4 LDS reads (+ 4 writes, 4 loads)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    if (t == 3)
                        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // scale words
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        if (q > 0)
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (pairs) {
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (t == 3) {
#pragma unroll
                    for (int i = 0; i < TM; i++)
                        wa[i] = na[i];
#pragma unroll
                    for (int i = 0; i < TN; i++)
                        wb[i] = nb[i];
                }
                lds_ring_barrier();
                __builtin_amdgcn_sched_barrier(0);
            };
            stage(std::integral_constant<int, 0>{});
            stage(std::integral_constant<int, 1>{});
            stage(std::integral_constant<int, 2>{});
            stage(std::integral_constant<int, 3>{});
        };
        for (int gi = 0; gi < ng; gi++)
            group(gi);
        // the unit after the next one
        bool nxt2_ok = false;
        Tile nxt2 = nxt;
        if (nxt_ok) {
            if (KGROUPED) {
                const int64_t t2 = uniform(s_next[k & 1]);  // the tile of unit k + 2
                nxt2_ok = t2 < ntiles;
                nxt2 = nxt2_ok ? coords(t2) : nxt;
            } else {
                nxt2_ok = k + 2 < my_units;
                nxt2 = nxt2_ok ? unit(k + 2) : nxt;
            }
            // K-grouped: take the tile of unit k + 3 (its slot was last read
            // at the end of unit k - 1, before this unit's barriers)
            if (KGROUPED && tid == 0)
                s_next[(k + 1) & 1] =
                    P + __hip_atomic_fetch_add(p.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // ---- split-tail unit (BF16 C, whole-width tiles only): its FP32
        // partial tile goes to its workspace slot, lane-major per sub-tile
        // and register group (64 lanes x 16 bytes per store, whole lines,
        // non-temporal: nothing here reads it back)
        const bool split_unit = SPLIT && cur.sp >= 0;
        if (split_unit) {
            const __amdgpu_buffer_rsrc_t rw = byte_range(p.ws, (uint32_t)(p.split_tiles * p.split_s) *
                                                                   (uint32_t)(BM * BN * 4));
            const uint32_t base = (uint32_t)cur.sp * (BM * BN * 4) + (uint32_t)(wave * (BM * BN / NW) + lane * 4) * 4;
#pragma unroll
            for (int i = 0; i < TN; i++)
#pragma unroll
                for (int j = 0; j < TM; j++) {
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        typedef float f4_t __attribute__((ext_vector_type(4)));
                        const f4_t v{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), rw,
                                                               base + (uint32_t)(((i * TM + j) * 4 + q) * 1024), 0, 2);
                    }
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        acc[i][j][v] = 0.0f;
                }
        } else if ((CT == 0 ? p.vec16 : p.vec_store) && cur.n0 + BN <= N) {
            // whole-width tile: buffer stores relative to the tile's first
            // element; the range ends after the tile's last valid row, so the
            // stores of rows past it (past M, or past the expert) are dropped
            const uint32_t rows_valid = (uint32_t)min(cur.m_end - cur.m0, BM);
            // K-grouped: expert g's C starts at row g * M
            const int64_t c_row = (KGROUPED ? (int64_t)cur.g * p.M : 0) + cur.m0;
            const __amdgpu_buffer_rsrc_t rc =
                byte_range((const uint8_t *)p.c + (c_row * p.ld_c + (int64_t)cur.n0) * CE,
                           rows_valid * (uint32_t)(p.ld_c * CE));
            // the band offsets are formed here, per tile, not kept in
            // registers across the main loop
            uint32_t cb = c_off;
            asm volatile("" : "+v"(cb));
            if (CT == 0) {
#pragma unroll
                for (int j = 0; j < TM; j++) {
                    v16f x[TN];
#pragma unroll
                    for (int i = 0; i < TN; i++)
                        x[i] = acc[i][j];
                    store_band(rc, cb, j, x);
#pragma unroll
                    for (int i = 0; i < TN; i++)
#pragma unroll
                        for (int v = 0; v < 16; v++)
                            acc[i][j][v] = 0.0f;
                }
            } else {
#pragma unroll
                for (int i = 0; i < TN; i++) {
#pragma unroll
                    for (int j = 0; j < TM; j++) {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            typedef float f4_t __attribute__((ext_vector_type(4)));
                            const f4_t v{acc[i][j][4 * q + 0], acc[i][j][4 * q + 1],
                                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(v4i, v), rc,
                                cb + (uint32_t)j * c_band + (uint32_t)((i * 32 + 8 * q) * CE), 0, 0);
                        }
#pragma unroll
                        for (int v = 0; v < 16; v++)
                            acc[i][j][v] = 0.0f;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < TN; i++) {
#pragma unroll
                for (int j = 0; j < TM; j++) {
                    const int64_t m = cur.m0 + wm * 128 + j * 32 + r32;
                    const int64_t mc = m + (KGROUPED ? (int64_t)cur.g * p.M : 0);  // row of C
                    if (m < cur.m_end) {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int64_t n = cur.n0 + wn * WN + i * 32 + 8 * q + 4 * h;
                            const float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
                            const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                            if (CT == 0) {
                                uint16_t *crow = reinterpret_cast<uint16_t *>(p.c) + mc * p.ld_c;
                                const uint32_t w0 = pack_bf16x2(v0, v1), w1 = pack_bf16x2(v2, v3);
                                if (p.vec_store && n + 3 < N) {
                                    *reinterpret_cast<uint2 *>(crow + n) = make_uint2(w0, w1);
                                } else {
                                    if (n + 0 < N) crow[n + 0] = (uint16_t)w0;
                                    if (n + 1 < N) crow[n + 1] = (uint16_t)(w0 >> 16);
                                    if (n + 2 < N) crow[n + 2] = (uint16_t)w1;
                                    if (n + 3 < N) crow[n + 3] = (uint16_t)(w1 >> 16);
                                }
                            } else {
                                float *crow = reinterpret_cast<float *>(p.c) + mc * p.ld_c;
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
#pragma unroll
                    for (int v = 0; v < 16; v++)
                        acc[i][j][v] = 0.0f;
                }
            }
        }
        if (!nxt_ok)
            break;
        cur = nxt;
        cur_sl = nxt_sl;
        nxt = nxt2;
        nxt_ok = nxt2_ok;
    }
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // the prefetch past the end: let it land
}

static int vec_ok(const void *c, int64_t ld_c, int c_dtype)
{
    const uintptr_t align = c_dtype == 0 ? 8 : 16;
    return ((uintptr_t)c % align == 0) && (ld_c % 4 == 0);
}

static int vec16_ok(const void *c, int64_t ld_c, int c_dtype)
{
    return c_dtype == 0 && ((uintptr_t)c % 16 == 0) && (ld_c % 8 == 0);
}

bool gemm_vec16(const void *c, int64_t ld_c, int c_dtype) { return vec16_ok(c, ld_c, c_dtype) != 0; }

// Bytes of a rearranged scale buffer: 32-row x 8-block tiles of 256 bytes.
static int64_t scale_bytes(int64_t rows, int64_t K)
{
    return ((rows + 31) / 32) * ((K / 32 + 7) / 8) * 256;
}

// Compute units of the current device (one persistent workgroup each: the
// kernel's LDS admits one workgroup per CU).
static int cu_count()
{
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// the split-tail plan (mx_plan.h) takes the kernel's tile and stage sizes
static_assert(PLAN_BM == BM && PLAN_BN == BN && PLAN_BK == 2 * BK, "plan and kernel tiles agree");

int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int c_dtype, bool vec16)
{
    return split_plan(M, N, K, c_dtype, vec16, cu_count()).bytes();
}

// Sums of the split tail: thread t of tile r's 16384 takes float4 t of the
// tile's slots (the partial-tile layout above: wave, sub-tile (i, j),
// register group q, lane), adds the split_s slots in range order and writes
// the four BF16 of C they hold, row wm*128 + 32j + (lane & 31), columns
// wn*128 + 32i + 8q + 4(lane >> 5) .. +3.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmParams p)
{
    constexpr int NW = 4;
    constexpr int PER_WAVE = BM * BN / 4 / NW;  // float4 per wave region
    const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int r = (int)(gt >> 14);
    const int t = (int)(gt & 16383);
    if (r >= p.split_tiles)
        return;
    const int wave = t / PER_WAVE, idx = (t % PER_WAVE) >> 6, lane = t & 63;
    const int q = idx & 3, j = (idx >> 2) & 3, i = idx >> 4;
    static_assert(PER_WAVE / 64 == TN * TM * 4, "one float4 per lane per (sub-tile, group)");
    const int row = (wave & 1) * 128 + j * 32 + (lane & 31);
    const int col = (wave >> 1) * (32 * TN) + i * 32 + 8 * q + 4 * (lane >> 5);
    // tile dp_tiles + r: the kernel's tile order (GROUP_M tile-rows at a time)
    const int64_t pid = p.dp_tiles + r;
    const int64_t per_group = GROUP_M * p.tiles_n;
    const int64_t grp = pid / per_group;
    const int64_t first_m = grp * GROUP_M;
    const int64_t gm = min(p.tiles_m - first_m, (int64_t)GROUP_M);
    const int64_t in = pid - grp * per_group;
    const int64_t m = (first_m + in % gm) * BM + row;
    const int64_t n = (in / gm) * BN + col;
    if (m >= p.M)
        return;
    const float4 *src = reinterpret_cast<const float4 *>(p.ws) + (int64_t)r * p.split_s * (BM * BN / 4) + t;
    float4 a = src[0];
    for (int sidx = 1; sidx < p.split_s; sidx++) {
        const float4 b = src[(int64_t)sidx * (BM * BN / 4)];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(p.c) + m * p.ld_c + n) =
        make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const void *a_q, int64_t ld_a,
                       const void *a_s, const void *b_q, int64_t ld_b, const void *b_s,
                       void *c, int64_t ld_c, int c_dtype, void *ws, hipStream_t stream)
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
    p.vec16 = vec16_ok(c, ld_c, c_dtype);
    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t cus = cu_count();
    p.dp_tiles = tiles;
    unsigned grid = (unsigned)std::min<int64_t>(tiles, cus);
    // split tail (the caller's workspace holds the FP32 partial tiles; its
    // size was checked against the plan before the launch)
    const SplitPlan sp = split_plan(M, N, K, c_dtype, p.vec16 != 0, cus);
    const bool split = sp.bytes() > 0;
    if (split) {
        p.dp_tiles = tiles - sp.rem;
        p.split_tiles = (int)sp.rem;
        p.split_s = (int)sp.S;
        p.ws = (float *)ws;
        grid = (unsigned)std::max<int64_t>(std::min<int64_t>(p.dp_tiles, cus), sp.rem * sp.S);
    }
    if (split)
        hipLaunchKernelGGL((mx_gemm_kernel<0, 0, true>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else if (c_dtype == 0)
        hipLaunchKernelGGL((mx_gemm_kernel<0, 0, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<0, 1, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    hipError_t err = hipGetLastError();
    if (split) {
        if (err == hipSuccess) {
            hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)(p.split_tiles * (BM * BN / 4 / 256))),
                               dim3(256), 0, stream, p);
            err = hipGetLastError();
        }
    }
    return err;
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
    p.tiles_n = (N + BN - 1) / BN;
    p.vec_store = vec_ok(c, ld_c, c_dtype);
    p.vec16 = vec16_ok(c, ld_c, c_dtype);
    // the tile count depends on the device-side offsets: one workgroup per CU,
    // each walking the tiles the kernel enumerates
    const unsigned grid = (unsigned)cu_count();
    if (c_dtype == 0)
        hipLaunchKernelGGL((mx_gemm_kernel<1, 0, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<1, 1, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    return hipGetLastError();
}

__global__ void zero_counter_kernel(int *counter)
{
    if (threadIdx.x == 0)
        *counter = 0;
}

hipError_t launch_grouped_gemm_wgrad(int64_t G, int64_t M, int64_t N, int64_t K,
                                     const int64_t *k_offsets, const void *a_q, int64_t ld_a,
                                     const void *a_s, const void *b_q, int64_t ld_b,
                                     const void *b_s, void *c, int64_t ld_c, int c_dtype,
                                     void *ws, hipStream_t stream)
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
    p.offsets = k_offsets;
    p.G = G;
    p.tiles_m = (M + BM - 1) / BM;
    p.tiles_n = (N + BN - 1) / BN;
    p.as_bytes = (uint32_t)scale_bytes(M, K);
    p.bs_bytes = (uint32_t)scale_bytes(N, K);
    p.vec_store = vec_ok(c, ld_c, c_dtype);
    p.vec16 = vec16_ok(c, ld_c, c_dtype);
    const int64_t tiles = G * p.tiles_m * p.tiles_n;
    const unsigned grid = (unsigned)std::min<int64_t>(tiles, cu_count());
    p.counter = (int *)ws;  // zeroed by a kernel (not a memset node), so replays of a captured call work
    hipLaunchKernelGGL(zero_counter_kernel, dim3(1), dim3(64), 0, stream, p.counter);
    if (c_dtype == 0)
        hipLaunchKernelGGL((mx_gemm_kernel<2, 0, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((mx_gemm_kernel<2, 1, false>), dim3(grid), dim3(GM_THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace mx
