/*
 * sage_oracle.c -- CPU oracle for the SageAttention2-style quantized attention
 * forward ("sage2" in the pages' benchmark artefacts).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's cpu_baseline leg
 * do.  It shares no code, header, table or constant with the HIP library: every
 * block size, scale constant and layout arrives as a function argument.
 *
 * Plain, slow, obviously correct.  Floating point is fp64 except where the method
 * itself fixes an fp32 decision (quantisation), where the same fp32 operation is
 * written out.  Build with gcc -O2 -ffp-contract=off -fopenmp (no fast-math): the
 * fp32 divisions, subtractions and nearbyintf calls below must be IEEE-exact.
 *
 * Sources.  The pages are three JSON benchmark artefacts of one repository:
 *   [latency]  "gb10-sage2-p0-interleave-softmax-latency.json"
 *   [profile]  "gb10-sampling-component-profile-1344x768-124f-seed440420.json"
 *   [strided]  "gb10-sage-strided-nhd-summary-1344x768-124f-seed440420.json"
 * They name the stages (profile, attention_internal_p50_milliseconds.sage2:
 * qk_quantize, v_quantize, attention_forward, framework_and_k_smoothing_estimate),
 * the shapes (latency, q_shape = [1, 37810, 56, 128]; h_msa_shape = [37810, 5376])
 * and the strided NHD input / token-major output dataflow (strided, dataflow).
 * They print no arithmetic.  The recipe written out here is SageAttention2's:
 * INT8 Q/K with per-tile fp32 scales amax/127 and round-to-nearest-even, K
 * smoothed by its per-head token mean, FP8 (OCP E4M3FN) V with per-channel
 * scales amax/448, an online softmax over 64-key tiles and FP8 P.  Each reading
 * taken where the method leaves a choice open is stated at the function.
 *
 * Parity of every function here is pinned by the CPU tests (library routines,
 * closed forms, invariants, brute force); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef long long i64;

/* ---------------------------------------------------------------- bf16 ---- */
/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element (b, n, h, d) of a [B, N, H, D] view with d-stride 1 and the other
 * strides in elements (strided NHD views of the packed QKV buffer, or HND). */
static float load_bf16(const uint16_t *base, i64 sb, i64 sn, i64 sh, int b, int n, int h, int d)
{
    return bf16_to_f32(base[(i64)b * sb + (i64)n * sn + (i64)h * sh + d]);
}

/* ---------------------------------------------------------- OCP E4M3FN ---- */
/* OCP 8-bit floating point, E4M3 "FN" flavour: sign, 4 exponent bits (bias 7),
 * 3 mantissa bits.  e = 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there
 * is no infinity; the largest finite magnitude is S.1111.110 = 448. */
double sage_oracle_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Round the fp32 value x to E4M3FN: nearest, ties to even, magnitudes beyond
 * 448 saturate to 448, the sign of zero is kept.  (Reading: the method's FP8 is
 * the OCP E4M3FN encoding with saturating round-to-nearest-even.) */
uint8_t sage_oracle_e4m3_encode(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (isnan(x))
        return sign | 0x7F;
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid: multiples of 2^-9; a*512 is exact in fp64 */
        double q = nearbyint(a * 512.0); /* 0..8; 8 is the code of 2^-6 */
        return sign | (uint8_t)q;
    }
    int e2;
    frexp(a, &e2);        /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;       /* a = (1 + mant) * 2^E, E in -6..8 */
    double mant = a / ldexp(1.0, E) - 1.0;  /* exact */
    double q = nearbyint(mant * 8.0);        /* ties to even; 0..8 */
    if (q == 8.0) {
        q = 0.0;
        E += 1;
    }
    int code = ((E + 7) << 3) | (int)q;
    if (code > 0x7E)
        code = 0x7E;
    return sign | (uint8_t)code;
}

void sage_oracle_e4m3_encode_array(const float *x, i64 n, uint8_t *out)
{
    for (i64 i = 0; i < n; i++)
        out[i] = sage_oracle_e4m3_encode(x[i]);
}

void sage_oracle_e4m3_decode_array(const uint8_t *c, i64 n, double *out)
{
    for (i64 i = 0; i < n; i++)
        out[i] = sage_oracle_e4m3_decode(c[i]);
}

/* ---------------------------------- OCP microscaling (MX) formats ---- */
/* E2M1 (the FP4 element type of MXFP4, OCP Microscaling Formats v1.0): a sign
 * bit, a 2-bit exponent (bias 1) and a 1-bit mantissa.  Codes 0..7 are the
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (0 and 0.5 subnormal); bit 3 is the
 * sign.  There is no infinity or NaN. */
double sage_oracle_e2m1_decode(uint8_t c)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double m = mag[c & 7];
    return (c & 8) ? -m : m;
}

/* Nearest E2M1 magnitude, ties to the even code, saturating at 6; the sign of
 * zero is kept.  (Written as a search over the eight magnitudes.) */
uint8_t sage_oracle_e2m1_encode(double x)
{
    uint8_t sign = signbit(x) ? 8 : 0;
    double a = fabs(x);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(a - sage_oracle_e2m1_decode((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return sign | (uint8_t)best;
}

/* MX quantisation (OCP Microscaling Formats v1.0, conversion to an MX block):
 * rows of `cols` values (cols a multiple of 32) in blocks of 32 consecutive
 * values.  Per block: amax = max |x_i|; shared exponent X = floor(log2 amax) -
 * emax_elem, with emax_elem the exponent of the element type's largest normal
 * (8 for E4M3, 2 for E2M1), clamped to [-127, 127]; X = -127 when amax = 0
 * (reading: the spec leaves the all-zero block's scale open; the smallest is
 * taken).  The scale is the E8M0 byte X + 127; each element is the element
 * type's round-to-nearest-even, saturating encoding of x_i / 2^X.
 * fmt 0: MXFP8 with E4M3 elements, one byte each.  fmt 1: MXFP4 with E2M1
 * elements, two per byte, the even element in the low nibble.
 * codes: rows * cols (fmt 0) or rows * cols / 2 (fmt 1) bytes; scales:
 * rows * cols / 32 bytes. */
void sage_oracle_mx_quantize(const double *x, i64 rows, int cols, int fmt, uint8_t *codes, uint8_t *scales)
{
    int emax = fmt == 0 ? 8 : 2;
    int nb = cols / 32;
    for (i64 r = 0; r < rows; r++)
        for (int blk = 0; blk < nb; blk++) {
            const double *v = x + r * cols + blk * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; i++)
                if (fabs(v[i]) > amax)
                    amax = fabs(v[i]);
            int X = -127;
            if (amax > 0.0) {
                int e2;
                frexp(amax, &e2); /* amax = f * 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
                X = (e2 - 1) - emax;
                if (X < -127)
                    X = -127;
                if (X > 127)
                    X = 127;
            }
            scales[r * nb + blk] = (uint8_t)(X + 127);
            for (int i = 0; i < 32; i++) {
                double y = ldexp(v[i], -X); /* exact: a power-of-two scaling */
                if (fmt == 0) {
                    codes[r * cols + blk * 32 + i] = sage_oracle_e4m3_encode((float)y);
                } else {
                    uint8_t c = sage_oracle_e2m1_encode(y);
                    i64 byte = (r * cols + blk * 32 + i) / 2;
                    if (i % 2 == 0)
                        codes[byte] = c;
                    else
                        codes[byte] |= (uint8_t)(c << 4);
                }
            }
        }
}

/* ------------------------------------------------------------- K mean ---- */
/* K smoothing statistic: the token mean of K per (batch, head, channel).
 * Reading: summed in fp64, first over `chunk` consecutive tokens in ascending
 * order, then the chunk partials in ascending order, then one division by N in
 * fp64 and one rounding to fp32.  km has layout [B, H, D]. */
void sage_oracle_kmean(const uint16_t *k, i64 sb, i64 sn, i64 sh,
                       int B, int N, int H, int D, int chunk, float *km)
{
    int nchunks = (N + chunk - 1) / chunk;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int d = 0; d < D; d++) {
                double total = 0.0;
                for (int c = 0; c < nchunks; c++) {
                    double part = 0.0;
                    int n1 = (c + 1) * chunk < N ? (c + 1) * chunk : N;
                    for (int n = c * chunk; n < n1; n++)
                        part += (double)load_bf16(k, sb, sn, sh, b, n, h, d);
                    total += part;
                }
                km[((i64)b * H + h) * D + d] = (float)(total / (double)N);
            }
}

/* ------------------------------------------------------ INT8 blocks ---- */
/* One quantisation block of `rows` tokens x D channels, values already fp32.
 * scale = amax / 127 (one IEEE fp32 division); code = clamp(rne(x / scale),
 * -127, 127) with x / scale one IEEE fp32 division and ties to even.  A block
 * whose amax is 0 gets scale 0 and all-zero codes. */
static void quant_block_int8(const float *x, int rows, int D, int8_t *codes, i64 code_row_stride,
                             float *scale)
{
    float amax = 0.0f;
    for (int r = 0; r < rows; r++)
        for (int d = 0; d < D; d++)
            amax = fmaxf(amax, fabsf(x[(i64)r * D + d]));
    if (amax == 0.0f) {
        *scale = 0.0f;
        for (int r = 0; r < rows; r++)
            for (int d = 0; d < D; d++)
                codes[(i64)r * code_row_stride + d] = 0;
        return;
    }
    float s = amax / 127.0f;
    *scale = s;
    for (int r = 0; r < rows; r++)
        for (int d = 0; d < D; d++) {
            float t = nearbyintf(x[(i64)r * D + d] / s);
            if (t > 127.0f)
                t = 127.0f;
            if (t < -127.0f)
                t = -127.0f;
            codes[(i64)r * code_row_stride + d] = (int8_t)t;
        }
}

/* Q quantisation: one scale per (batch, head, `blk` consecutive tokens); the
 * last block of a head holds the N % blk remaining tokens.  codes [B, H, N, D]
 * (logical, unpadded), scales [B, H, ceil(N / blk)]. */
void sage_oracle_quant_q(const uint16_t *q, i64 sb, i64 sn, i64 sh,
                         int B, int N, int H, int D, int blk, int8_t *codes, float *scales)
{
    int nblk = (N + blk - 1) / blk;
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int t = 0; t < nblk; t++) {
                int n0 = t * blk, rows = (N - n0) < blk ? (N - n0) : blk;
                float *x = (float *)malloc(sizeof(float) * (size_t)rows * D);
                for (int r = 0; r < rows; r++)
                    for (int d = 0; d < D; d++)
                        x[(i64)r * D + d] = load_bf16(q, sb, sn, sh, b, n0 + r, h, d);
                quant_block_int8(x, rows, D, codes + (((i64)b * H + h) * N + n0) * D, D,
                                 scales + ((i64)b * H + h) * nblk + t);
                free(x);
            }
}

/* K quantisation after smoothing: x = (fp32) k - km[b, h, d] (one fp32
 * subtraction, not re-rounded to bf16), then blocks of `blk` tokens exactly as
 * for Q.  codes [B, H, N, D], scales [B, H, ceil(N / blk)]. */
void sage_oracle_quant_k(const uint16_t *k, i64 sb, i64 sn, i64 sh,
                         int B, int N, int H, int D, const float *km, int blk,
                         int8_t *codes, float *scales)
{
    int nblk = (N + blk - 1) / blk;
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int t = 0; t < nblk; t++) {
                int n0 = t * blk, rows = (N - n0) < blk ? (N - n0) : blk;
                const float *m = km + ((i64)b * H + h) * D;
                float *x = (float *)malloc(sizeof(float) * (size_t)rows * D);
                for (int r = 0; r < rows; r++)
                    for (int d = 0; d < D; d++)
                        x[(i64)r * D + d] = load_bf16(k, sb, sn, sh, b, n0 + r, h, d) - m[d];
                quant_block_int8(x, rows, D, codes + (((i64)b * H + h) * N + n0) * D, D,
                                 scales + ((i64)b * H + h) * nblk + t);
                free(x);
            }
}

/* ------------------------------------------------------- V to E4M3 ---- */
/* V quantisation: one scale per (batch, head, channel) over all N tokens,
 * sv = amax / 448 (one IEEE fp32 division), code = E4M3FN(v / sv) with v / sv
 * one IEEE fp32 division.  amax 0 gives sv 0 and codes 0x00.
 * codes [B, H, N, D] (logical), scales [B, H, D]. */
void sage_oracle_quant_v(const uint16_t *v, i64 sb, i64 sn, i64 sh,
                         int B, int N, int H, int D, uint8_t *codes, float *scales)
{
#pragma omp parallel for collapse(3) schedule(static)
    for (int b = 0; b < B; b++)
        for (int h = 0; h < H; h++)
            for (int d = 0; d < D; d++) {
                float amax = 0.0f;
                for (int n = 0; n < N; n++)
                    amax = fmaxf(amax, fabsf(load_bf16(v, sb, sn, sh, b, n, h, d)));
                float sv = amax / 448.0f;
                uint8_t *c = codes + ((i64)b * H + h) * (i64)N * D + d;
                scales[((i64)b * H + h) * D + d] = amax == 0.0f ? 0.0f : sv;
                for (int n = 0; n < N; n++) {
                    if (amax == 0.0f)
                        c[(i64)n * D] = 0x00;
                    else
                        c[(i64)n * D] = sage_oracle_e4m3_encode(load_bf16(v, sb, sn, sh, b, n, h, d) / sv);
                }
            }
}

/* ------------------------------------------------ exact attention ---- */
/* The plain definition: row i of softmax(Q K^T * sm_scale), computed in fp64
 * from the bf16 inputs.  p receives the N normalised probabilities. */
void sage_oracle_softmax_row(const uint16_t *q, i64 qsb, i64 qsn, i64 qsh,
                             const uint16_t *k, i64 ksb, i64 ksn, i64 ksh,
                             int N, int D, int b, int h, int i, double sm_scale, double *p)
{
    double m = -INFINITY, l = 0.0;
    const uint16_t *qi = q + (i64)b * qsb + (i64)i * qsn + (i64)h * qsh;
    for (int j = 0; j < N; j++) {
        const uint16_t *kj = k + (i64)b * ksb + (i64)j * ksn + (i64)h * ksh;
        double s = 0.0;
        for (int d = 0; d < D; d++)
            s += (double)bf16_to_f32(qi[d]) * (double)bf16_to_f32(kj[d]);
        p[j] = s * sm_scale;
        if (p[j] > m)
            m = p[j];
    }
    for (int j = 0; j < N; j++) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (int j = 0; j < N; j++)
        p[j] /= l;
}

/* O = softmax(Q K^T * sm_scale) V for selected query rows; non-causal, no mask,
 * all N keys.  rows[(b*H + h)*nrows + r] names the query row of output row r;
 * out has layout [B, H, nrows, D]. */
void sage_oracle_attn_exact(const uint16_t *q, i64 qsb, i64 qsn, i64 qsh,
                            const uint16_t *k, i64 ksb, i64 ksn, i64 ksh,
                            const uint16_t *v, i64 vsb, i64 vsn, i64 vsh,
                            int B, int N, int H, int D, double sm_scale,
                            const int *rows, int nrows, double *out)
{
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < H; h++)
                for (int r = 0; r < nrows; r++) {
                    int i = rows[((i64)b * H + h) * nrows + r];
                    double *o = out + (((i64)b * H + h) * nrows + r) * D;
                    sage_oracle_softmax_row(q, qsb, qsn, qsh, k, ksb, ksn, ksh, N, D, b, h, i, sm_scale, p);
                    /* o_d = sum_j p_j v_jd, each channel summed in ascending j */
                    for (int d = 0; d < D; d++)
                        o[d] = 0.0;
                    for (int j = 0; j < N; j++)
                        for (int d = 0; d < D; d++)
                            o[d] += p[j] * (double)load_bf16(v, vsb, vsn, vsh, b, j, h, d);
                }
        free(p);
    }
}

/* ------------------------------------- quantised method, step by step ---- */
/* The quantised forward as the method computes it, from the codes and scales
 * (logical layouts as produced above: codes [B, H, N, D], Q/K scales
 * [B, H, ceil(N / qblk or kblk)], V scales [B, H, D]):
 *   a_ij = sum_d qc_id * kc_jd                      exact integer
 *   s_ij = a_ij * sq[i / qblk] * sk[j / kblk] * sm_scale
 *   for key tiles of `ptile` keys in ascending order (the last one partial):
 *     m_t   = max(m_{t-1}, max_j s_ij)              m_{-1} = -inf
 *     alpha = exp(m_{t-1} - m_t)
 *     p_ij  = exp(s_ij - m_t)
 *     l     = alpha * l + sum_j p_ij                unrounded p
 *     pq_ij = E4M3FN(fp32(pscale * p_ij))           (if round_p; else pscale * p)
 *     acc_d = alpha * acc_d + sum_j pq_ij * E4M3FN^-1(vc_jd)
 *   o_id = acc_d * sv_d / (pscale * l)
 * Readings: P is rounded relative to the running maximum after each tile (no
 * thresholded rescaling, no split over keys); the normaliser sums P before it
 * is rounded; pscale (448) maps p in (0, 1] onto the E4M3 range and is divided
 * out at the end.  round_p = 0 keeps P unrounded; the pins use it to check the
 * tile walk on inputs that quantise exactly. */
void sage_oracle_attn_method(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks,
                             const uint8_t *vc, const float *vs,
                             int B, int N, int H, int D, int qblk, int kblk, int ptile,
                             double sm_scale, double pscale, int round_p,
                             const int *rows, int nrows, double *out)
{
    int nqb = (N + qblk - 1) / qblk, nkb = (N + kblk - 1) / kblk;
    double vdec[256];
    for (int c = 0; c < 256; c++)
        vdec[c] = sage_oracle_e4m3_decode((uint8_t)c);
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)ptile);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < H; h++)
                for (int r = 0; r < nrows; r++) {
                    i64 bh = (i64)b * H + h;
                    int i = rows[bh * nrows + r];
                    const int8_t *qi = qc + (bh * N + i) * D;
                    double sq = qs[bh * nqb + i / qblk];
                    double m = -INFINITY, l = 0.0;
                    for (int d = 0; d < D; d++)
                        acc[d] = 0.0;
                    for (int j0 = 0; j0 < N; j0 += ptile) {
                        int j1 = j0 + ptile < N ? j0 + ptile : N;
                        double mt = m;
                        for (int j = j0; j < j1; j++) {
                            const int8_t *kj = kc + (bh * N + j) * D;
                            i64 a = 0;
                            for (int d = 0; d < D; d++)
                                a += (i64)qi[d] * (i64)kj[d];
                            s[j - j0] = (double)a * sq * (double)ks[bh * nkb + j / kblk] * sm_scale;
                            if (s[j - j0] > mt)
                                mt = s[j - j0];
                        }
                        double alpha = exp(m - mt); /* m = -inf on the first tile: 0 */
                        l *= alpha;
                        for (int d = 0; d < D; d++)
                            acc[d] *= alpha;
                        for (int j = j0; j < j1; j++) {
                            double p = exp(s[j - j0] - mt);
                            double pq = round_p ? sage_oracle_e4m3_decode(
                                                      sage_oracle_e4m3_encode((float)(pscale * p)))
                                                : pscale * p;
                            const uint8_t *vj = vc + (bh * N + j) * D;
                            l += p;
                            for (int d = 0; d < D; d++)
                                acc[d] += pq * vdec[vj[d]];
                        }
                        m = mt;
                    }
                    double *o = out + (bh * nrows + r) * D;
                    for (int d = 0; d < D; d++)
                        o[d] = acc[d] * (double)vs[bh * D + d] / (pscale * l);
                }
        free(s);
        free(acc);
    }
}

/* ------------------------------ INT8 Q K^T with an unquantised P.V ---- */
/* bf16 of an fp32 value: round to nearest, ties to even (finite values), as the
 * bfloat16 format is defined (the upper 16 bits of an IEEE binary32). */
static uint16_t bf16_rne_bits(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    uint32_t lower = u & 0xFFFFu, upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

static double bf16_rne(float x)
{
    return (double)bf16_to_f32(bf16_rne_bits(x));
}

/* The "sol_int8_qk" precision split of the profile page
 * (sampling_stage_step_2_seconds.sol_int8_qk_tau_1_3_exact_conditioning_kv:
 * Q and K quantised, V not), dense.  Scores and the tile walk are those of
 * sage_oracle_attn_method; V is the bf16 view itself:
 *   for key tiles of `ptile` keys in ascending order:
 *     m_t = max(m_{t-1}, max_j s_ij);  alpha = exp(m_{t-1} - m_t)
 *     p_ij = exp(s_ij - m_t);  l = alpha * l + sum_j p_ij        unrounded p
 *     acc_d = alpha * acc_d + sum_j bf16(fp32(p_ij)) * v_jd      (if round_p)
 *   o_id = acc_d / l
 * Reading: P is rounded to bf16 from its fp32 value (the precision the kernel
 * holds p in) relative to the running maximum after each tile, as for E4M3 P in
 * the fully quantised method. */
void sage_oracle_attn_int8qk(const int8_t *qc, const float *qs, const int8_t *kc, const float *ks,
                             const uint16_t *v, i64 vsb, i64 vsn, i64 vsh,
                             int B, int N, int H, int D, int qblk, int kblk, int ptile,
                             double sm_scale, int round_p, const int *rows, int nrows, double *out)
{
    int nqb = (N + qblk - 1) / qblk, nkb = (N + kblk - 1) / kblk;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)ptile);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for collapse(3) schedule(dynamic, 4)
        for (int b = 0; b < B; b++)
            for (int h = 0; h < H; h++)
                for (int r = 0; r < nrows; r++) {
                    i64 bh = (i64)b * H + h;
                    int i = rows[bh * nrows + r];
                    const int8_t *qi = qc + (bh * N + i) * D;
                    double sq = qs[bh * nqb + i / qblk];
                    double m = -INFINITY, l = 0.0;
                    for (int d = 0; d < D; d++)
                        acc[d] = 0.0;
                    for (int j0 = 0; j0 < N; j0 += ptile) {
                        int j1 = j0 + ptile < N ? j0 + ptile : N;
                        double mt = m;
                        for (int j = j0; j < j1; j++) {
                            const int8_t *kj = kc + (bh * N + j) * D;
                            i64 a = 0;
                            for (int d = 0; d < D; d++)
                                a += (i64)qi[d] * (i64)kj[d];
                            s[j - j0] = (double)a * sq * (double)ks[bh * nkb + j / kblk] * sm_scale;
                            if (s[j - j0] > mt)
                                mt = s[j - j0];
                        }
                        double alpha = exp(m - mt); /* m = -inf on the first tile: 0 */
                        l *= alpha;
                        for (int d = 0; d < D; d++)
                            acc[d] *= alpha;
                        for (int j = j0; j < j1; j++) {
                            double p = exp(s[j - j0] - mt);
                            double pq = round_p ? bf16_rne((float)p) : p;
                            l += p;
                            for (int d = 0; d < D; d++)
                                acc[d] += pq * (double)load_bf16(v, vsb, vsn, vsh, b, j, h, d);
                        }
                        m = mt;
                    }
                    double *o = out + (bh * nrows + r) * D;
                    for (int d = 0; d < D; d++)
                        o[d] = acc[d] / l;
                }
        free(s);
        free(acc);
    }
}

/* ------------------------------------------- RMSNorm + RoPE of Q and K ---- */
/* [strided] dataflow.qk_transform: before quantisation, Q and K go through
 * RMSNorm and rotary position embedding, in place on their strided views;
 * [profile] representative_block_24_p50_milliseconds.sage2.rms_rope prices the
 * step.  The pages print no formula.  Reading (the plainest one for a per-head
 * [B, N, H, D] view):
 *   - RMSNorm over the D channels of one (b, n, h) row with a learned weight
 *     gamma[D] shared by all heads: r = 1 / sqrt(mean_d x_d^2 + eps),
 *     y_d = x_d * r * gamma_d;
 *   - RoPE on adjacent channel pairs (2i, 2i+1) with a per-token angle table
 *     rope[n][i] = (cos, sin) shared by batches and heads:
 *     (a, b) -> (a cos - b sin, a sin + b cos);
 *   - the result stored as bf16, rounded once (nearest even).
 *
 * The bf16 result decides INT8 codes downstream, so the fp32 evaluation is
 * written out:
 *   ss  = the exact sum of the squares x_d^2, rounded once to fp32 (nearest,
 *         ties to even; +inf beyond the largest finite value): no summation
 *         order enters;
 *   r   = 1 / sqrtf(ss / D + eps)          (IEEE sqrt and division)
 *   n_d = (x_d * r) * gamma_d
 *   y   = (n_2i * c - n_2i+1 * s,  n_2i * s + n_2i+1 * c)
 * every operation after ss rounded to fp32, none fused. */

/* A bf16 value (exactly representable in x) is +-M * 2^(E - 134) with E its
 * biased exponent field and M <= 255 an integer (the hidden bit included; a
 * subnormal has E = 0 and is read as E = 1 without the hidden bit), so its
 * square M^2 * 2^(2E - 268) is a whole number of units of 2^-266.  The squares
 * of a row are added as integers in a fixed-point accumulator of 9 64-bit words
 * (the largest possible row sum, 512 squares of the largest finite bf16 value
 * 255^2 * 2^506 each, stays below 2^531 < 2^576), and the total is rounded to
 * fp32 once. */
#define SQ_WORDS 9

static void sq_add(uint64_t *acc, uint32_t m2, int shift)
{
    int w = shift / 64, off = shift % 64;
    uint64_t lo = (uint64_t)m2 << off;
    uint64_t hi = off > 48 ? (uint64_t)m2 >> (64 - off) : 0;   /* m2 < 2^16 */
    uint64_t old = acc[w];
    acc[w] = old + lo;
    uint64_t carry = acc[w] < old;
    for (int i = w + 1; i < SQ_WORDS && (hi | carry); i++) {
        old = acc[i];
        acc[i] = old + hi + carry;        /* hi + carry <= 2^16: wraps iff the word decreases */
        carry = acc[i] < old;
        hi = 0;
    }
}

static int sq_bit(const uint64_t *acc, int i)
{
    return (int)((acc[i / 64] >> (i % 64)) & 1u);
}

static float exact_sum_squares_f32(const float *x, int n)
{
    uint64_t acc[SQ_WORDS];
    memset(acc, 0, sizeof acc);
    for (int d = 0; d < n; d++) {
        uint32_t u;
        memcpy(&u, &x[d], 4);
        uint32_t e = (u >> 23) & 0xFF, m = (u >> 16) & 0x7F;
        if (e == 0 && m == 0)
            continue;
        if (e == 0)
            e = 1;                       /* subnormal: no hidden bit */
        else
            m |= 0x80;
        sq_add(acc, m * m, 2 * (int)e - 2);
    }
    int t = -1;                          /* the highest set bit */
    for (int i = 64 * SQ_WORDS - 1; i >= 0 && t < 0; i--)
        if (sq_bit(acc, i))
            t = i;
    if (t < 0)
        return 0.0f;
    /* keep 24 significant bits, or the bits at or above the fp32 subnormal
     * quantum 2^-149 = bit 117 of the accumulator */
    int p = t - 23 > 117 ? t - 23 : 117;
    uint32_t q = 0;
    for (int i = t; i >= p; i--)
        q = (q << 1) | (uint32_t)sq_bit(acc, i);
    int half = p > 0 ? sq_bit(acc, p - 1) : 0, sticky = 0;
    for (int i = p - 2; i >= 0 && !sticky; i--)
        sticky = sq_bit(acc, i);
    if (half && (sticky || (q & 1u)))
        q++;
    return ldexpf((float)q, p - 266);    /* exact, or +inf past the fp32 range */
}

/* The exact-sum rounding alone, for its pins: rows x n bf16 bit patterns. */
void sage_oracle_sum_squares(const uint16_t *bits, i64 rows, int n, float *out)
{
    float *x = malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (i64 r = 0; r < rows; r++) {
        for (int d = 0; d < n; d++)
            x[d] = bf16_to_f32(bits[r * n + d]);
        out[r] = exact_sum_squares_f32(x, n);
    }
    free(x);
}

void sage_oracle_norm_rope(const uint16_t *x, i64 sb, i64 sn, i64 sh, int B, int N, int H, int D,
                           const float *gamma, const float *rope, float eps, uint16_t *out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int n = 0; n < N; n++)
            for (int h = 0; h < H; h++) {
                float xr[512], nr[512];
                for (int d = 0; d < D; d++) xr[d] = load_bf16(x, sb, sn, sh, b, n, h, d);
                float ss = exact_sum_squares_f32(xr, D);
                float r = 1.0f / sqrtf(ss / (float)D + eps);
                for (int d = 0; d < D; d++) nr[d] = (xr[d] * r) * gamma[d];
                uint16_t *o = out + (((i64)b * N + n) * H + h) * D;
                for (int i = 0; i < D / 2; i++) {
                    float c = rope[((i64)n * (D / 2) + i) * 2], s = rope[((i64)n * (D / 2) + i) * 2 + 1];
                    float a = nr[2 * i], e = nr[2 * i + 1];
                    float y0 = a * c - e * s;
                    float y1 = a * s + e * c;
                    o[2 * i] = bf16_rne_bits(y0);
                    o[2 * i + 1] = bf16_rne_bits(y1);
                }
            }
}

/* The same transform in fp64 without any intermediate rounding and without the
 * bf16 rounding (any summation order: exact enough to bound the fp32 one). */
void sage_oracle_norm_rope_f64(const uint16_t *x, i64 sb, i64 sn, i64 sh, int B, int N, int H, int D,
                               const float *gamma, const float *rope, double eps, double *out)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; b++)
        for (int n = 0; n < N; n++)
            for (int h = 0; h < H; h++) {
                double ss = 0.0;
                for (int d = 0; d < D; d++) {
                    double v = load_bf16(x, sb, sn, sh, b, n, h, d);
                    ss += v * v;
                }
                double r = 1.0 / sqrt(ss / D + eps);
                double *o = out + (((i64)b * N + n) * H + h) * D;
                for (int i = 0; i < D / 2; i++) {
                    double c = rope[((i64)n * (D / 2) + i) * 2], s = rope[((i64)n * (D / 2) + i) * 2 + 1];
                    double a = load_bf16(x, sb, sn, sh, b, n, h, 2 * i) * r * gamma[2 * i];
                    double e = load_bf16(x, sb, sn, sh, b, n, h, 2 * i + 1) * r * gamma[2 * i + 1];
                    o[2 * i] = a * c - e * s;
                    o[2 * i + 1] = a * s + e * c;
                }
            }
}

/* Threads the OpenMP loops above use (reported beside oracle timings). */
#ifdef _OPENMP
#include <omp.h>
#endif
int sage_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following parallel loops (timing of the single-thread case). */
void sage_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n);
#else
    (void)n;
#endif
}
