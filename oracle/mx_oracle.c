/*
 * CPU oracle for MXFP8 quantization, scale rearrangement and block-scaled
 * GEMM.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Sources followed:
 *  - "End-to-End MXFP8 Reinforcement Learning on Blackwell" (abstract;
 *    Figure 1; Table 6; Table 10 rows F3, F4, F6): MXFP8 operands with
 *    power-of-two E8M0 block scales, a scale-rearrangement pass feeding the
 *    GEMM, dense and per-expert MXFP8 GEMMs.
 *  - OCP Microscaling Formats (MX) Specification v1.0: block of 32, shared
 *    scale X = 2^(floor(log2(amax)) - emax_elem) with emax_elem = 8 for E4M3,
 *    elements rounded to nearest (ties to even) and saturated to +-448.
 *
 * Everything is plain scalar code in double precision.  Every function
 * follows the definition it cites; nothing is blocked, fused or reordered.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - all-zero block: scale code 0x00;  amax below 2^-119: scale code 0x00.
 *  - a block holding NaN or Inf: scale code 0xFF and every element 0x7F.
 *  - a negative value that rounds to zero keeps its sign (0x80).
 *  - column-wise output is stored transposed: qT[col][row], sT[col][row/32].
 *  - rearranged scale layout: 32-row x 8-block tiles of 256 bytes, tile
 *    (rt, kt) at byte (rt*KT + kt)*256, entry (row r, block 8kt + 2t + h) at
 *    byte (32h + r)*4 + t inside the tile, padding 0x7F.
 *
 * Parity pins (tests/test_oracle_pins.py): brute-force nearest-code search
 * over all 256 E4M3 codes, exhaustive scale-rule check over every BF16 amax,
 * hand-derived golden blocks, exact rational GEMM on tiny inputs, closed
 * forms, and the invariants the pages rely on (power-of-two scales,
 * byte-for-byte determinism, idempotent re-quantization).  The MoE pieces
 * (tests/test_oracle_moe_pins.py, test_oracle_moe_bwd_pins.py,
 * test_oracle_swiglu_pins.py): dispatch order against a loop definition,
 * combine by exact special cases, the per-expert column-wise layout against
 * an element loop and a planted straddling block, the per-expert weight
 * gradient by exact rational sums and the unquantized product, the double ->
 * BF16 rounding by brute-force nearest search, silu by closed forms.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ---- BF16 ------------------------------------------------------------- */

/* BF16 is the upper half of an IEEE binary32; widening to double is exact. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---- E4M3 (OCP "E4M3FN"): sign, 4 exponent bits (bias 7), 3 mantissa bits.
 * Normal codes e = 1..15 give (1 + m/8) * 2^(e-7) except e = 15, m = 7 which
 * is NaN; e = 0 gives the subnormals (m/8) * 2^-6.  Largest finite 448. */

double oracle_e4m3_decode(uint8_t q)
{
    int s = q >> 7;
    int e = (q >> 3) & 15;
    int m = q & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);          /* (m/8) * 2^-6 */
    else
        mag = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -mag : mag;
}

/* Encode a finite double as E4M3: round to the nearest representable value,
 * ties to the even mantissa, clamp magnitudes above 448 to 448, keep the
 * sign of zero.  Precondition: t is finite. */
uint8_t oracle_e4m3_encode(double t)
{
    uint8_t sign = signbit(t) ? 0x80 : 0x00;
    double a = fabs(t);
    int e2, E, biased;
    double quantum, n, r;
    if (a == 0.0)
        return sign;
    /* the binade of a: a in [2^E, 2^(E+1)) */
    frexp(a, &e2);
    E = e2 - 1;
    /* below the smallest normal binade the spacing stays that of 2^-6 */
    if (E < -6)
        E = -6;
    quantum = ldexp(1.0, E - 3); /* 3 mantissa bits */
    n = nearbyint(a / quantum);  /* exact division; default mode is ties-to-even */
    r = n * quantum;
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    /* write the representable magnitude r back as exponent and mantissa */
    if (r < ldexp(1.0, -6))
        return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -9)));
    frexp(r, &e2);
    E = e2 - 1;
    biased = E + 7;
    return (uint8_t)(sign | (biased << 3) | (int)(r / ldexp(1.0, E - 3) - 8.0));
}

/* ---- E8M0 scale: code c in 0..254 means 2^(c-127); 255 is NaN. ---------- */

double oracle_e8m0_decode(uint8_t c)
{
    if (c == 0xFF)
        return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* Shared scale of a block from its largest magnitude: the exponent of
 * floor(log2(amax)) minus the largest E4M3 exponent (448 = 1.75 * 2^8). */
uint8_t oracle_scale_code(double amax)
{
    int e2, c;
    if (isnan(amax) || isinf(amax))
        return 0xFF;
    if (amax == 0.0)
        return 0x00;
    frexp(amax, &e2);
    c = (e2 - 1) - 8 + 127;
    if (c < 0)
        c = 0;
    if (c > 254)
        c = 254;
    return (uint8_t)c;
}

/* One block of 32 BF16 values v[i*vs] -> 32 codes q[i*qs] and a scale byte. */
void oracle_quantize_block(const uint16_t *v, ptrdiff_t vs, uint8_t *q, ptrdiff_t qs,
                           uint8_t *s)
{
    double x[32], amax = 0.0, X;
    int i, nonfinite = 0;
    uint8_t c;
    for (i = 0; i < 32; i++) {
        x[i] = oracle_bf16_to_double(v[i * vs]);
        if (!isfinite(x[i]))
            nonfinite = 1;
        else if (fabs(x[i]) > amax)
            amax = fabs(x[i]);
    }
    if (nonfinite) {
        *s = 0xFF;
        for (i = 0; i < 32; i++)
            q[i * qs] = 0x7F;
        return;
    }
    c = oracle_scale_code(amax);
    *s = c;
    X = ldexp(1.0, (int)c - 127);
    for (i = 0; i < 32; i++)
        q[i * qs] = oracle_e4m3_encode(x[i] / X); /* a power-of-two rescale: exact */
}

/* Row-wise: blocks of 32 consecutive elements along each row.
 * x[rows][ld_x] BF16 -> q[rows][ld_q], s[rows][ld_s] (cols/32 bytes used). */
void oracle_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t *q, int64_t ld_q, uint8_t *s, int64_t ld_s)
{
    int64_t r, b;
    for (r = 0; r < rows; r++)
        for (b = 0; b < cols / 32; b++)
            oracle_quantize_block(x + r * ld_x + 32 * b, 1, q + r * ld_q + 32 * b, 1,
                                  s + r * ld_s + b);
}

/* Column-wise: blocks of 32 consecutive elements down each column, written
 * transposed: qt[cols][ld_qt] (rows bytes used), st[cols][ld_st] (rows/32). */
void oracle_quantize_colwise(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x,
                             uint8_t *qt, int64_t ld_qt, uint8_t *st, int64_t ld_st)
{
    int64_t c, b;
    for (c = 0; c < cols; c++)
        for (b = 0; b < rows / 32; b++)
            oracle_quantize_block(x + 32 * b * ld_x + c, ld_x, qt + c * ld_qt + 32 * b, 1,
                                  st + c * ld_st + b);
}

/* ---- scale rearrangement --------------------------------------------- */

int64_t oracle_swizzled_bytes(int64_t rows, int64_t kblocks)
{
    return ((rows + 31) / 32) * ((kblocks + 7) / 8) * 256;
}

/* Byte position of scale (row, block) inside the rearranged buffer. */
int64_t oracle_swizzle_offset(int64_t row, int64_t blk, int64_t kblocks)
{
    int64_t KT = (kblocks + 7) / 8;
    int64_t rt = row / 32, r = row % 32;
    int64_t kt = blk / 8, j = blk % 8;
    int64_t t = j / 2, h = j % 2;
    return (rt * KT + kt) * 256 + (32 * h + r) * 4 + t;
}

void oracle_scale_swizzle(const uint8_t *s, int64_t rows, int64_t kblocks, int64_t ld_s,
                          uint8_t *out)
{
    int64_t n = oracle_swizzled_bytes(rows, kblocks), i, r, b;
    for (i = 0; i < n; i++)
        out[i] = 0x7F;
    for (r = 0; r < rows; r++)
        for (b = 0; b < kblocks; b++)
            out[oracle_swizzle_offset(r, b, kblocks)] = s[r * ld_s + b];
}

void oracle_scale_unswizzle(const uint8_t *in, int64_t rows, int64_t kblocks, uint8_t *s,
                            int64_t ld_s)
{
    int64_t r, b;
    for (r = 0; r < rows; r++)
        for (b = 0; b < kblocks; b++)
            s[r * ld_s + b] = in[oracle_swizzle_offset(r, b, kblocks)];
}

/* ---- dequantization and GEMM -------------------------------------------- */

/* deq(q, c) = dec_E4M3(q) * 2^(c-127), exact in double. */
double oracle_dequant(uint8_t q, uint8_t c)
{
    return oracle_e4m3_decode(q) * oracle_e8m0_decode(c);
}

/* One output entry C[i][j] = sum_k deqA[i][k] * deqB[j][k] in double, and
 * the bound sum_k |deqA[i][k]| * |deqB[j][k]|.  Operands are K-contiguous:
 * qa row i at qa + i*ld_a, its scales (plain, not rearranged) at
 * sa + i*ld_sa; likewise for B row j. */
void oracle_gemm_entry(int64_t K, const uint8_t *qa_row, const uint8_t *sa_row,
                       const uint8_t *qb_row, const uint8_t *sb_row, double *c, double *bnd)
{
    double acc = 0.0, b = 0.0, p;
    int64_t k;
    for (k = 0; k < K; k++) {
        p = oracle_dequant(qa_row[k], sa_row[k / 32]) * oracle_dequant(qb_row[k], sb_row[k / 32]);
        acc += p;
        b += fabs(p);
    }
    *c = acc;
    *bnd = b;
}

/* Full dense product C[M][N] = deq(A)[M][K] * deq(B)[N][K]^T (double). */
void oracle_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *qa, int64_t ld_a,
                 const uint8_t *sa, int64_t ld_sa, const uint8_t *qb, int64_t ld_b,
                 const uint8_t *sb, int64_t ld_sb, double *c, double *bnd)
{
    int64_t i, j;
    for (i = 0; i < M; i++)
        for (j = 0; j < N; j++)
            oracle_gemm_entry(K, qa + i * ld_a, sa + i * ld_sa, qb + j * ld_b, sb + j * ld_sb,
                              c + i * N + j, bnd + i * N + j);
}

/* Selected entries (rows[e], cols[e]) of the same product. */
void oracle_gemm_sampled(int64_t n, const int64_t *rows, const int64_t *cols, int64_t K,
                         const uint8_t *qa, int64_t ld_a, const uint8_t *sa, int64_t ld_sa,
                         const uint8_t *qb, int64_t ld_b, const uint8_t *sb, int64_t ld_sb,
                         double *c, double *bnd)
{
    int64_t e;
    for (e = 0; e < n; e++)
        oracle_gemm_entry(K, qa + rows[e] * ld_a, sa + rows[e] * ld_sa, qb + cols[e] * ld_b,
                          sb + cols[e] * ld_sb, c + e, bnd + e);
}

/* Per-expert product: rows offsets[g] .. offsets[g+1]-1 of A multiply expert
 * g's weight B_g[N][K] (at qb + g*N*ld_b, scales at sb + g*N*ld_sb).
 * Selected entries only; the expert of a row is found from the offsets. */
void oracle_grouped_gemm_sampled(int64_t n, const int64_t *rows, const int64_t *cols,
                                 int64_t G, const int64_t *offsets, int64_t N, int64_t K,
                                 const uint8_t *qa, int64_t ld_a, const uint8_t *sa,
                                 int64_t ld_sa, const uint8_t *qb, int64_t ld_b,
                                 const uint8_t *sb, int64_t ld_sb, double *c, double *bnd)
{
    int64_t e, g;
    for (e = 0; e < n; e++) {
        int64_t i = rows[e];
        for (g = 0; g < G; g++)
            if (offsets[g] <= i && i < offsets[g + 1])
                break;
        oracle_gemm_entry(K, qa + i * ld_a, sa + i * ld_sa, qb + (g * N + cols[e]) * ld_b,
                          sb + (g * N + cols[e]) * ld_sb, c + e, bnd + e);
    }
}

/* ---- array helpers for the Python wrapper (loops over the scalars above) */

void oracle_e4m3_encode_array(const double *t, int64_t n, uint8_t *q)
{
    int64_t i;
    for (i = 0; i < n; i++)
        q[i] = oracle_e4m3_encode(t[i]);
}

void oracle_e4m3_decode_array(const uint8_t *q, int64_t n, double *t)
{
    int64_t i;
    for (i = 0; i < n; i++)
        t[i] = oracle_e4m3_decode(q[i]);
}

void oracle_scale_code_array(const double *amax, int64_t n, uint8_t *c)
{
    int64_t i;
    for (i = 0; i < n; i++)
        c[i] = oracle_scale_code(amax[i]);
}

/* Row-wise dequantization of q[rows][ld_q] with plain scales s[rows][ld_s]. */
void oracle_dequantize_rowwise(const uint8_t *q, int64_t rows, int64_t cols, int64_t ld_q,
                               const uint8_t *s, int64_t ld_s, double *out)
{
    int64_t r, k;
    for (r = 0; r < rows; r++)
        for (k = 0; k < cols; k++)
            out[r * cols + k] = oracle_dequant(q[r * ld_q + k], s[r * ld_s + k / 32]);
}

/* ---- MoE backward: per-expert column-wise operands and weight gradients --
 * The update_actor stage of the MoE learner (paper Table 8; Table 2 for the
 * 128-expert, top-8 model) needs each expert's weight gradient
 * dW_g = dY_g^T X_g, a contraction over that expert's token rows only.  Both
 * operands are quantized column-wise in 32-row blocks, and a block may not
 * hold rows of two experts.  Layout (ours): expert g's rows
 * [offsets[g], offsets[g+1]) become columns [pad[g], pad[g+1]) of the
 * transposed operand, with pad[0] = 0 and
 * pad[g+1] = pad[g] + max(256, m_g rounded up to a multiple of 256); the
 * columns past the expert's m_g rows hold zero codes (zero rows appended,
 * which leave every block maximum unchanged). */

void oracle_grouped_pad_offsets(int64_t G, const int64_t *offsets, int64_t *pad)
{
    int64_t g, m, len;
    pad[0] = 0;
    for (g = 0; g < G; g++) {
        m = offsets[g + 1] - offsets[g];
        len = ((m + 255) / 256) * 256;
        if (len < 256)
            len = 256;
        pad[g + 1] = pad[g] + len;
    }
}

/* x[rows_total][ld_x] BF16, rows sorted by expert -> qt[cols][ld_qt] and
 * st[cols][ld_st] (plain scales, one per 32 columns of qt), columns laid out
 * by pad (from oracle_grouped_pad_offsets).  Columns past pad[G] are left
 * untouched. */
void oracle_quantize_colwise_grouped(const uint16_t *x, int64_t cols, int64_t ld_x, int64_t G,
                                     const int64_t *offsets, const int64_t *pad, uint8_t *qt,
                                     int64_t ld_qt, uint8_t *st, int64_t ld_st)
{
    int64_t g, c, b, i, row;
    uint16_t v[32];
    for (g = 0; g < G; g++)
        for (c = 0; c < cols; c++)
            for (b = 0; b < (pad[g + 1] - pad[g]) / 32; b++) {
                for (i = 0; i < 32; i++) {
                    row = offsets[g] + 32 * b + i;
                    v[i] = row < offsets[g + 1] ? x[row * ld_x + c] : 0x0000; /* +0.0 */
                }
                oracle_quantize_block(v, 1, qt + c * ld_qt + pad[g] + 32 * b, 1,
                                      st + c * ld_st + pad[g] / 32 + b);
            }
}

/* Selected entries of the per-expert weight gradient: entry e is
 * C_g[rows[e]][cols[e]] with g = groups[e], i.e.
 * sum over k in [pad[g], pad[g+1]) of deqA[row][k] * deqB[col][k]
 * (A = qa[M][ld_a], B = qb[N][ld_b], plain scales one per 32 of k). */
void oracle_grouped_wgrad_sampled(int64_t n, const int64_t *groups, const int64_t *rows,
                                  const int64_t *cols, const int64_t *pad, const uint8_t *qa,
                                  int64_t ld_a, const uint8_t *sa, int64_t ld_sa,
                                  const uint8_t *qb, int64_t ld_b, const uint8_t *sb,
                                  int64_t ld_sb, double *c, double *bnd)
{
    int64_t e, g, lo, len;
    for (e = 0; e < n; e++) {
        g = groups[e];
        lo = pad[g];
        len = pad[g + 1] - lo;
        oracle_gemm_entry(len, qa + rows[e] * ld_a + lo, sa + rows[e] * ld_sa + lo / 32,
                          qb + cols[e] * ld_b + lo, sb + cols[e] * ld_sb + lo / 32, c + e,
                          bnd + e);
    }
}

/* ---- SwiGLU between the MoE expert projections ---------------------------
 * Qwen3's expert MLP (paper Table 2: Qwen3-30B-A3B) feeds the down
 * projection with h = silu(g) * u, silu(g) = g / (1 + exp(-g)), where g and u
 * are the gate and up halves of the gate_up product.  The learner keeps
 * activations in BF16 (paper Figure 1: BF16 activations quantized to MXFP8
 * before each MXFP8 GEMM), so h is rounded once to BF16 (nearest, ties to
 * even) and then quantized row-wise like any GEMM input. */

double oracle_swiglu_f64(double g, double u)
{
    return g * u / (1.0 + exp(-g));
}

/* double -> BF16 bit pattern, round to nearest, ties to even, one rounding:
 * 8 significant bits for normal results, multiples of 2^-133 below 2^-126,
 * +-Inf from 2^128 * (1 - 2^-9) up; NaN stays NaN. */
uint16_t oracle_double_to_bf16(double v)
{
    double a, q;
    int e;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v))
        return 0x7FC0;
    a = fabs(v);
    if (a == 0.0)
        return sign;
    frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    if (e - 1 >= -126)
        q = ldexp(rint(ldexp(a, 8 - e)), e - 8);   /* 8 significant bits */
    else
        q = ldexp(rint(ldexp(a, 133)), -133);      /* subnormal spacing 2^-133 */
    if (q >= ldexp(1.0, 128))
        return sign | 0x7F80;
    if (q == 0.0)
        return sign;
    /* q is exactly a BF16 value: read its fields */
    frexp(q, &e);
    if (e - 1 >= -126) {
        uint16_t E = (uint16_t)(e - 1 + 127);
        uint16_t M = (uint16_t)(ldexp(q, 8 - e) - 128.0);
        return sign | (uint16_t)(E << 7) | M;
    }
    return sign | (uint16_t)ldexp(q, 133);
}

/* gu[rows][ld_gu]: columns [0, F) the gate g, [F, 2F) the up u (BF16) ->
 * h[rows][F] BF16 bit patterns. */
void oracle_swiglu_bf16(const uint16_t *gu, int64_t rows, int64_t F, int64_t ld_gu, uint16_t *h)
{
    int64_t r, j;
    for (r = 0; r < rows; r++)
        for (j = 0; j < F; j++)
            h[r * F + j] = oracle_double_to_bf16(oracle_swiglu_f64(
                oracle_bf16_to_double(gu[r * ld_gu + j]), oracle_bf16_to_double(gu[r * ld_gu + F + j])));
}
