/*
 * qgemv_oracle.c -- plain, slow, fp64 CPU oracle for the decode-time
 * weight-only quantized GEMV  y[M,N] = x[M,K] . dequant(W[N,K])^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The GPU product path never calls
 * it, and it shares no code, header, table or helper with the HIP sources.
 *
 * Every function is the plain definition written out: decode each stored
 * value exactly, dequantize one weight at a time, multiply and add in double
 * precision.  No blocking, fusion or reordering.  Build with
 *     gcc -O2 -ffp-contract=off -fPIC -shared
 * so that no multiply-add is contracted (the bit-identity rules in section
 * 2.3 of "62 . r59 -- q4_K W_dsc plane + riders" forbid FMA contraction when
 * the pre-decoded plane is formed).
 *
 * Sources (the pages; the oracle follows them, nothing else):
 *  - int4 MatMulNBits blockwise layout: named by the onnx-genai pull request
 *    #1000 ("Summary", "What it does": int4 MatMulNBits decode GEMV with
 *    per-column fp32 accumulation).  The tensor layout is not spelled out on
 *    the page; the reading used here is the ONNX-Runtime one: W row n holds
 *    K/2 bytes with element 2i in the low nibble of byte i, one fp16 scale per
 *    (n, block), 4-bit zero points packed two per byte with the even block in
 *    the low nibble, each row of zero points padded to a whole byte, and a
 *    missing zero-point tensor meaning 8.  PARITY OF THE LAYOUT IS UNPINNED BY
 *    THE PAGES (convention only); the arithmetic w = s * (q - zp) is pinned.
 *  - q4_K super-block and get_scale_min_k4: "62 . r59 -- q4_K W_dsc plane +
 *    riders", section 2.1 (the per-(chunk,row) rank-1 coefficients d*sc and
 *    -dmin*m) and section 3.2 (the 144-byte block: d at byte 0, dmin at byte
 *    2, twelve packed 6-bit scale/min bytes at 4..16, and the two decode
 *    paths for chunk < 4 and chunk >= 4).  The order of the 4-bit quants inside
 *    the 128 quant bytes is not given on the page; the reading used here is
 *    the public llama.cpp/GGUF one: within each 64-element half-pair, element
 *    64g+l (l < 32) is the low nibble of quant byte 32g+l and element 64g+32+l
 *    is its high nibble.  PARITY OF THE NIBBLE ORDER IS UNPINNED BY THE PAGES.
 *  - W_dsc plane: same page, section 2.2 (chunk-major, float2 per (chunk,row),
 *    size N*K/4 bytes) and section 2.3 (exact f16->f32, exact u8->f32, one f32
 *    multiply, exact negation).
 *  - bf16 dense GEMV: the AstrAI backend commit list (bf16 GEMV primitive for
 *    M = 1..8, any positive K and any storage offset).
 *  - q4_K prefill with 8-bit activations (MMQ): "62 . r59 -- q4_K W_dsc plane
 *    + riders", section 2.1 (the rank-1 rescale of each (chunk, row) integer
 *    dot product by d*sc and -dmin*m) and section 3.2 (the dispatch arm
 *    quantizes the activations to 8 bits in a prepass before the integer
 *    matrix product).  The page does not spell out the activation rule; the
 *    reading used here is the plain symmetric one, per block of 32
 *    consecutive k of one activation row (one weight chunk, so one activation
 *    scale multiplies each chunk's integer sum): d = amax/127 in binary32,
 *    q = x/d in binary32 rounded half away from zero, d = 0 and q = 0 for an
 *    all-zero block.  The result is the exact value of
 *        sum_c d_a[c] * (dv[c] * sum_{k in c} q_w[k]*q_a[k]
 *                        + mv[c] * sum_{k in c} q_a[k])
 *    evaluated in double.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Exact decoders of the stored floating-point formats.                      */
/* ------------------------------------------------------------------------ */

/* IEEE 754 binary16 -> double, exactly (1 sign, 5 exponent, 10 fraction bits,
 * bias 15; exponent 0 = subnormal with scale 2^-24; exponent 31 = inf/nan). */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 -> double, exactly: a bfloat16 is the upper 16 bits of an IEEE
 * binary32 (1 sign, 8 exponent, 7 fraction bits, bias 127). */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);
    } else if (e == 255) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(128 + f), e - 134);
    }
    return sign ? -v : v;
}

/* binary32 bit pattern -> double, exactly. */
double oracle_f32bits_to_f64(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round a double to the nearest representable value of a binary format with
 * `p` significand bits (incl. the hidden bit), minimum normal exponent
 * `emin` (value 2^emin) and largest finite value `maxv`; ties to even.  The
 * result is returned as a double (exactly representable in the format). */
static double round_to_format(double v, int p, int emin, double maxv)
{
    if (isnan(v) || isinf(v) || v == 0.0)
        return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
    int exp_unit = e - 1;       /* a in [2^exp_unit, 2^(exp_unit+1)) */
    if (exp_unit < emin)
        exp_unit = emin;        /* subnormal range: fixed spacing */
    double ulp = ldexp(1.0, exp_unit - (p - 1));
    double q = a / ulp;         /* exact: division by a power of two */
    double fl = floor(q);
    double r = q - fl;
    double n;
    if (r > 0.5)
        n = fl + 1.0;
    else if (r < 0.5)
        n = fl;
    else
        n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double out = n * ulp;
    /* overflow: values that round past the largest finite become infinity */
    double max_exp_unit_ulp = ldexp(1.0, ilogb(maxv) - (p - 1));
    if (out > maxv) {
        if (a >= maxv + max_exp_unit_ulp / 2.0)
            out = INFINITY;
        else
            out = maxv;
    }
    return v < 0 ? -out : out;
}

double oracle_round_f16(double v) { return round_to_format(v, 11, -14, 65504.0); }
double oracle_round_bf16(double v) { return round_to_format(v, 8, -126, 0x1.FEp127); }
double oracle_round_f32(double v) { return round_to_format(v, 24, -126, 0x1.FFFFFEp127); }

/* Spacing of a binary format at |v| (the "one output ulp" of the tolerance):
 * 2^(floor(log2|v|) - (p-1)) in the normal range, the subnormal spacing below. */
static double ulp_of_format(double v, int p, int emin)
{
    double a = fabs(v);
    int exp_unit = emin;
    if (a != 0.0 && !isinf(a) && !isnan(a)) {
        int e;
        frexp(a, &e);
        exp_unit = e - 1;
        if (exp_unit < emin)
            exp_unit = emin;
    }
    return ldexp(1.0, exp_unit - (p - 1));
}

double oracle_ulp_f16(double v) { return ulp_of_format(v, 11, -14); }
double oracle_ulp_bf16(double v) { return ulp_of_format(v, 8, -126); }
double oracle_ulp_f32(double v) { return ulp_of_format(v, 24, -126); }

/* ------------------------------------------------------------------------ */
/* int4 MatMulNBits blockwise weights.                                      */
/* ------------------------------------------------------------------------ */

/* Bytes per row of the zero-point tensor: one nibble per block, rounded up
 * to a whole byte. */
int64_t oracle_int4_zp_row_bytes(int64_t K, int64_t block_size)
{
    int64_t nblocks = K / block_size;
    return (nblocks + 1) / 2;
}

/* The 4-bit code of weight (n, k): byte k/2 of row n, low nibble for even k. */
int oracle_int4_code(const uint8_t *w, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = w[n * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* The zero point of block b in row n (8 when there is no zero-point tensor). */
int oracle_int4_zero_point(const uint8_t *zp, int64_t K, int64_t block_size,
                           int64_t n, int64_t b)
{
    if (zp == NULL)
        return 8;
    uint8_t byte = zp[n * oracle_int4_zp_row_bytes(K, block_size) + b / 2];
    return (b % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Dequantized weight w[n,k] = scale[n, k/bs] * (q - zp).  The value is exact
 * in binary32 and in double (an 11-bit significand times an integer of
 * magnitude <= 15). */
double oracle_int4_weight(const uint8_t *w, const uint16_t *scales,
                          const uint8_t *zp, int64_t K, int64_t block_size,
                          int64_t n, int64_t k)
{
    int64_t b = k / block_size;
    int64_t nblocks = K / block_size;
    double s = oracle_f16_to_f64(scales[n * nblocks + b]);
    int q = oracle_int4_code(w, K, n, k);
    int z = oracle_int4_zero_point(zp, K, block_size, n, b);
    return s * (double)(q - z);
}

/* Dequantize rows [n0, n0+rows) into out[rows][K]. */
void oracle_int4_dequant_rows(const uint8_t *w, const uint16_t *scales,
                              const uint8_t *zp, int64_t K, int64_t block_size,
                              int64_t n0, int64_t rows, double *out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < K; k++)
            out[r * K + k] = oracle_int4_weight(w, scales, zp, K, block_size,
                                                n0 + r, k);
}

/* ------------------------------------------------------------------------ */
/* q4_K super-blocks (144 bytes per 256 weights).                           */
/* ------------------------------------------------------------------------ */

#define Q4K_BLOCK_BYTES 144
#define Q4K_BLOCK_ELEMS 256

/* Decode the 6-bit scale and 6-bit min of chunk cc (0..7) from the twelve
 * packed bytes, following the two bit paths of get_scale_min_k4. */
void oracle_q4k_scale_min(const uint8_t *sc, int cc, int *s, int *m)
{
    if (cc < 4) {
        *s = sc[cc] & 63;
        *m = sc[cc + 4] & 63;
    } else {
        *s = (sc[cc + 4] & 0x0F) | ((sc[cc - 4] >> 6) << 4);
        *m = (sc[cc + 4] >> 4) | ((sc[cc] >> 6) << 4);
    }
}

static const uint8_t *q4k_block(const uint8_t *w, int64_t K, int64_t n,
                                int64_t sb)
{
    int64_t blocks_per_row = K / Q4K_BLOCK_ELEMS;
    return w + (n * blocks_per_row + sb) * Q4K_BLOCK_BYTES;
}

static uint16_t read_le16(const uint8_t *p)
{
    return (uint16_t)(p[0] | (p[1] << 8));
}

/* The rank-1 coefficients of chunk c (global chunk index, c = k/32) in row n:
 * dv = f32(d) * sc and mv = -(f32(dmin) * m).  Both products are exact in
 * binary32 (at most 17 significant bits), so computing them in double and
 * converting gives the same bits as the single f32 multiply of the page; the
 * negation is applied last, so m == 0 or dmin == 0 yields -0.0. */
void oracle_q4k_coeffs(const uint8_t *w, int64_t K, int64_t n, int64_t c,
                       float *dv, float *mv)
{
    const uint8_t *blk = q4k_block(w, K, n, c / 8);
    double d = oracle_f16_to_f64(read_le16(blk + 0));
    double dmin = oracle_f16_to_f64(read_le16(blk + 2));
    int s, m;
    oracle_q4k_scale_min(blk + 4, (int)(c % 8), &s, &m);
    *dv = (float)(d * (double)s);
    *mv = -(float)(dmin * (double)m);
}

/* The 4-bit quant of weight (n, k) (GGUF nibble order, see the file header). */
int oracle_q4k_code(const uint8_t *w, int64_t K, int64_t n, int64_t k)
{
    const uint8_t *blk = q4k_block(w, K, n, k / Q4K_BLOCK_ELEMS);
    const uint8_t *qs = blk + 16;
    int e = (int)(k % Q4K_BLOCK_ELEMS);
    int cc = e / 32;
    int l = e % 32;
    int g = cc / 2;
    uint8_t byte = qs[32 * g + l];
    return (cc % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Dequantized weight from given coefficients: the binary32 value nearest to
 * dv*q + mv (dv*q is exact; one rounding of the sum). */
static double q4k_weight_from(double dv, double mv, int q)
{
    return (double)(float)(dv * (double)q + mv);
}

/* Dequantized q4_K weight w[n,k], decoded from the super-block. */
double oracle_q4k_weight(const uint8_t *w, int64_t K, int64_t n, int64_t k)
{
    float dv, mv;
    oracle_q4k_coeffs(w, K, n, k / 32, &dv, &mv);
    return q4k_weight_from(dv, mv, oracle_q4k_code(w, K, n, k));
}

/* Same weight, with the coefficients read from a W_dsc plane. */
double oracle_q4k_weight_plane(const uint8_t *w, const float *plane, int64_t N,
                               int64_t K, int64_t n, int64_t k)
{
    int64_t c = k / 32;
    double dv = (double)plane[(c * N + n) * 2 + 0];
    double mv = (double)plane[(c * N + n) * 2 + 1];
    return q4k_weight_from(dv, mv, oracle_q4k_code(w, K, n, k));
}

void oracle_q4k_dequant_rows(const uint8_t *w, int64_t K, int64_t n0,
                             int64_t rows, double *out)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t k = 0; k < K; k++)
            out[r * K + k] = oracle_q4k_weight(w, K, n0 + r, k);
}

/* Build the chunk-major W_dsc plane: entry (c, n) at float index (c*N+n)*2
 * holds (dv, mv) of chunk c of row n.  N*K/32 entries, N*K/4 bytes. */
void oracle_q4k_build_plane(const uint8_t *w, int64_t N, int64_t K,
                            float *plane)
{
    int64_t nchunk = K / 32;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t c = 0; c < nchunk; c++) {
            float dv, mv;
            oracle_q4k_coeffs(w, K, n, c, &dv, &mv);
            plane[(c * N + n) * 2 + 0] = dv;
            plane[(c * N + n) * 2 + 1] = mv;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The GEMV itself.                                                         */
/* ------------------------------------------------------------------------ */

/* Activation element x[m,k] as a double, from its stored type. */
enum { ORACLE_X_F16 = 0, ORACLE_X_BF16 = 1, ORACLE_X_F32 = 2 };

static double x_at(const void *x, int xtype, int64_t ldx, int64_t m, int64_t k)
{
    switch (xtype) {
    case ORACLE_X_F16:
        return oracle_f16_to_f64(((const uint16_t *)x)[m * ldx + k]);
    case ORACLE_X_BF16:
        return oracle_bf16_to_f64(((const uint16_t *)x)[m * ldx + k]);
    default:
        return (double)((const float *)x)[m * ldx + k];
    }
}

/* The four weight encodings. */
enum { ORACLE_W_INT4 = 0, ORACLE_W_Q4K = 1, ORACLE_W_Q4K_PLANE = 2,
       ORACLE_W_BF16 = 3 };

typedef struct {
    int kind;
    const uint8_t *w;        /* int4 codes, q4_K blocks, or bf16 bits */
    const uint16_t *scales;  /* int4 */
    const uint8_t *zp;       /* int4, may be NULL */
    const float *plane;      /* q4_K via plane */
    int64_t block_size;      /* int4 */
    int64_t ldw;             /* bf16 row stride in elements */
    int64_t N, K;
} weights_t;

static double weight_at(const weights_t *W, int64_t n, int64_t k)
{
    switch (W->kind) {
    case ORACLE_W_INT4:
        return oracle_int4_weight(W->w, W->scales, W->zp, W->K, W->block_size,
                                  n, k);
    case ORACLE_W_Q4K:
        return oracle_q4k_weight(W->w, W->K, n, k);
    case ORACLE_W_Q4K_PLANE:
        return oracle_q4k_weight_plane(W->w, W->plane, W->N, W->K, n, k);
    default:
        return oracle_bf16_to_f64(((const uint16_t *)W->w)[n * W->ldw + k]);
    }
}

/* y_ref[m, j] = sum_k x[m,k] * w[cols[j], k] and S[m, j] = sum_k |x*w| for
 * every row m < M and every listed column (all N columns when cols is NULL).
 * Each product is exact in double (at most 11 + 24 significant bits); only the
 * sums round, with an error far below the tolerance.  Outputs are [M][ncols]. */
static void gemv(const void *x, int xtype, int64_t ldx, const weights_t *W,
                 int64_t M, const int64_t *cols, int64_t ncols, double *y_ref,
                 double *s_abs)
{
    for (int64_t j = 0; j < ncols; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t k = 0; k < W->K; k++) {
                double p = x_at(x, xtype, ldx, m, k) * weight_at(W, n, k);
                acc += p;
                acc_abs += fabs(p);
            }
            y_ref[m * ncols + j] = acc;
            s_abs[m * ncols + j] = acc_abs;
        }
    }
}

void oracle_int4_gemv(const uint16_t *x_f16, int64_t ldx, const uint8_t *w,
                      const uint16_t *scales, const uint8_t *zp, int64_t M,
                      int64_t N, int64_t K, int64_t block_size,
                      const int64_t *cols, int64_t ncols, double *y_ref,
                      double *s_abs)
{
    weights_t W = {ORACLE_W_INT4, w, scales, zp, NULL, block_size, 0, N, K};
    gemv(x_f16, ORACLE_X_F16, ldx, &W, M, cols, cols ? ncols : N, y_ref, s_abs);
}

void oracle_q4k_gemv(const float *x, int64_t ldx, const uint8_t *w, int64_t M,
                     int64_t N, int64_t K, const int64_t *cols, int64_t ncols,
                     double *y_ref, double *s_abs)
{
    weights_t W = {ORACLE_W_Q4K, w, NULL, NULL, NULL, 0, 0, N, K};
    gemv(x, ORACLE_X_F32, ldx, &W, M, cols, cols ? ncols : N, y_ref, s_abs);
}

void oracle_q4k_plane_gemv(const float *x, int64_t ldx, const uint8_t *w,
                           const float *plane, int64_t M, int64_t N, int64_t K,
                           const int64_t *cols, int64_t ncols, double *y_ref,
                           double *s_abs)
{
    weights_t W = {ORACLE_W_Q4K_PLANE, w, NULL, NULL, plane, 0, 0, N, K};
    gemv(x, ORACLE_X_F32, ldx, &W, M, cols, cols ? ncols : N, y_ref, s_abs);
}

void oracle_bf16_gemv(const uint16_t *x, int64_t ldx, const uint16_t *w,
                      int64_t ldw, int64_t M, int64_t N, int64_t K,
                      const int64_t *cols, int64_t ncols, double *y_ref,
                      double *s_abs)
{
    weights_t W = {ORACLE_W_BF16, (const uint8_t *)w, NULL, NULL, NULL, 0, ldw,
                   N, K};
    gemv(x, ORACLE_X_BF16, ldx, &W, M, cols, cols ? ncols : N, y_ref, s_abs);
}

/* ------------------------------------------------------------------------ */
/* q4_K prefill with 8-bit activations.                                      */
/* ------------------------------------------------------------------------ */

/* One block of 32 activations -> 32 signed 8-bit codes and the block scale
 * (see the file header for the rule).  Every operation is a single binary32
 * operation: the division amax / 127, the division x / d, and the rounding of
 * the quotient half away from zero to an integer (|x / d| <= 127 up to a few
 * binary32 ulps, so the code fits in 8 bits). */
void oracle_q8_quantize_block(const float *x, int8_t *q, float *d_out)
{
    float amax = 0.0f;
    for (int i = 0; i < 32; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float d = amax / 127.0f;
    *d_out = d;
    for (int i = 0; i < 32; i++) {
        if (d == 0.0f) {
            q[i] = 0;
        } else {
            float v = x[i] / d;
            q[i] = (int8_t)roundf(v);
        }
    }
}

/* Rows of x[T][ldx] (K a multiple of 32) -> codes q[T][K] and scales
 * d[T][K/32]. */
void oracle_q8_quantize_rows(const float *x, int64_t ldx, int64_t T, int64_t K,
                             int8_t *q, float *d)
{
    for (int64_t t = 0; t < T; t++)
        for (int64_t b = 0; b < K / 32; b++)
            oracle_q8_quantize_block(x + t * ldx + 32 * b, q + t * K + 32 * b,
                                     d + t * (K / 32) + b);
}

/* y_ref[t, j] for every activation row t < T and listed weight row n =
 * cols[j] (all N when cols is NULL): the sum over chunks c of
 *     d_a[t,c] * (dv[n,c] * D + mv[n,c] * Sa)
 * with the exact integers D = sum_{k in c} q_w[n,k] * q_a[t,k] and
 * Sa = sum_{k in c} q_a[t,k]; S[t, j] sums the magnitudes of the two terms.
 * The coefficients come from the super-block (oracle_q4k_coeffs) and the
 * quants in GGUF order (oracle_q4k_code).  Outputs are [T][ncols]. */
void oracle_q4k_mmq(const float *x, int64_t ldx, const uint8_t *w, int64_t T,
                    int64_t N, int64_t K, const int64_t *cols, int64_t ncols,
                    int8_t *qa, float *da, int *qw, double *y_ref,
                    double *s_abs)
{
    /* qa [T][K], da [T][K/32] and qw [K] are caller-provided scratch. */
    int64_t nchunk = K / 32;
    int64_t nc = cols ? ncols : N;
    oracle_q8_quantize_rows(x, ldx, T, K, qa, da);
    for (int64_t j = 0; j < nc; j++) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t k = 0; k < K; k++)
            qw[k] = oracle_q4k_code(w, K, n, k);
        for (int64_t t = 0; t < T; t++) {
            double acc = 0.0, acc_abs = 0.0;
            for (int64_t c = 0; c < nchunk; c++) {
                float dv, mv;
                oracle_q4k_coeffs(w, K, n, c, &dv, &mv); /* chunk c of row n */
                int64_t dot = 0, sum = 0;
                for (int64_t k = 32 * c; k < 32 * c + 32; k++) {
                    dot += (int64_t)qw[k] * (int64_t)qa[t * K + k];
                    sum += (int64_t)qa[t * K + k];
                }
                double a = (double)da[t * nchunk + c];
                double term_d = a * ((double)dv * (double)dot);
                double term_m = a * ((double)mv * (double)sum);
                acc += term_d + term_m;
                acc_abs += fabs(term_d) + fabs(term_m);
            }
            y_ref[t * nc + j] = acc;
            s_abs[t * nc + j] = acc_abs;
        }
    }
}
