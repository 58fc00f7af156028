/*
 * qgemv.h -- C ABI of libqgemv.so: decode-time weight-only quantized GEMV /
 * small-M GEMM on AMD Instinct MI355X (gfx950).
 *
 *     y[M,N] = x[M,K] . dequant(W[N,K])^T,      1 <= M <= 8
 *
 * for three weight encodings: MatMulNBits-style blockwise int4, llama.cpp-style
 * q4_K super-blocks (decoded in the kernel, or through a pre-decoded
 * chunk-major "W_dsc" coefficient plane), and plain bf16.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers.  Every array argument is a DEVICE pointer (HBM, e.g. from a
 *    PyTorch tensor) owned by the caller.  The library allocates nothing,
 *    keeps no state between calls and never frees anything.  Buffers must
 *    stay valid until the enqueued work has finished on `stream`.
 *  - Streams.  `stream` is a hipStream_t passed as `void*`; NULL means the
 *    null stream.  All work is enqueued asynchronously on that stream; no
 *    entry point synchronises the host.
 *  - Layouts.  Row-major.  Leading dimensions (ld*) are in ELEMENTS of the
 *    array's own type.  x is [M][ldx] (row m at x + m*ldx), y is [M][ldy].
 *    The weight matrix has one row per output column n (N rows of K).
 *  - Arithmetic.  Every weight is dequantized exactly (the value is an exact
 *    binary32 number; see each entry point), products are accumulated in
 *    binary32, and y is rounded to nearest-even to its type once.  The result
 *    satisfies |y - y_ref| <= 2e-3 * sum_k |x[m,k] w[n,k]| + 1 ulp of y's type,
 *    where y_ref is the exact dot product.  The summation order is fixed for
 *    a given (entry point, shape), so repeated calls are bitwise identical.
 *  - Errors.  Arguments are validated on the host before anything is
 *    enqueued; a non-QG_OK status means nothing was enqueued (except
 *    QG_ERR_HIP, returned when the HIP runtime rejects a launch).  A
 *    human-readable detail of the last failure on the calling thread is
 *    available from qg_last_error().  N == 0 is a valid empty problem:
 *    QG_OK, nothing enqueued.
 *  - Aliasing.  y must not overlap any input (QG_ERR_ALIAS).
 *  - Thread safety.  All entry points are reentrant.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qg_status {
    QG_OK = 0,
    QG_ERR_NULL_POINTER = 1, /* a required pointer is NULL                    */
    QG_ERR_BAD_SHAPE = 2,    /* M not in 1..8, N < 0, K < 1, ld < extent,
                                K not a multiple of the block / super-block   */
    QG_ERR_UNSUPPORTED = 3,  /* block size or dtype not provided             */
    QG_ERR_MISALIGNED = 4,   /* a pointer or stride breaks its alignment rule */
    QG_ERR_ALIAS = 5,        /* y overlaps an input                           */
    QG_ERR_HIP = 6           /* the HIP runtime reported an error             */
} qg_status;

typedef enum qg_dtype {
    QG_F16 = 0,  /* IEEE binary16                 */
    QG_BF16 = 1, /* bfloat16 (top half of binary32) */
    QG_F32 = 2   /* IEEE binary32                 */
} qg_dtype;

/*
 * qgemv_int4_blockwise -- MatMulNBits-style int4 GEMV.
 *
 * Operation: the M = 1 int4 MatMulNBits decode GEMV with per-column fp32
 * accumulation of the onnx-genai pull request #1000 ("Summary", "What it
 * does"), generalised to M = 1..8.  For column n and reduction index k, with
 * b = k / block_size:
 *     q  = 4-bit code of (n,k)    : byte  w[n*(K/2) + k/2], low nibble for
 *                                   even k, high nibble for odd k
 *     zp = 4-bit zero point (n,b) : byte  zero_points[n*ZR + b/2], low nibble
 *                                   for even b, ZR = ceil((K/block_size)/2);
 *                                   8 when zero_points == NULL
 *     s  = scales[n*(K/block_size) + b]  (fp16 bits)
 *     w[n,k] = float(s) * (q - zp)       (exact in binary32)
 *     y[m,n] = sum_k x[m,k] * w[n,k]
 *
 * x           : [M][ldx] of x_type, 2-byte aligned.
 * x_type      : QG_F16 (IEEE binary16).  QG_BF16 activations are not
 *               provided and return QG_ERR_UNSUPPORTED (nothing enqueued);
 *               any other value is QG_ERR_UNSUPPORTED as well.
 * w           : [N][K/2] bytes, 16-byte aligned.
 * scales      : fp16 bits, [N][K/block_size], 2-byte aligned.
 * zero_points : [N][ZR] bytes or NULL (symmetric, zero point 8).  In a row
 *               with an odd block count the last high nibble is ignored.
 * y           : [M][ldy] of y_type (QG_F16, QG_BF16 or QG_F32), aligned to
 *               its element size.
 * block_size  : 32, 64, 128 or 256 (QG_ERR_UNSUPPORTED otherwise); K must be
 *               a positive multiple of it (QG_ERR_BAD_SHAPE otherwise).
 */
qg_status qgemv_int4_blockwise(const void *x, int64_t ldx, int32_t x_type,
                               const uint8_t *w, const uint16_t *scales,
                               const uint8_t *zero_points, void *y, int64_t ldy,
                               int32_t y_type, int64_t M, int64_t N, int64_t K,
                               int32_t block_size, void *stream);

/*
 * int4 weights in a load-time packed layout for the matrix-core GEMV.
 *
 * Operation: the offline weight repack with a versioned layout flag that the
 * onnx-genai pull request #1000 proposes ("Roadmap recommendation"), for the
 * MatMulNBits int4 weights of qgemv_int4_blockwise.  The packed buffer holds
 * the same codes, scales and zero points, bit for bit, in another order;
 * qgemv_int4_packed on it computes the product qgemv_int4_blockwise defines
 * (same tolerance; the summation order is that of the packed kernel).
 *
 * Layout QG_INT4_LAYOUT_TILE16_V1 (K a positive multiple of 128 and of the
 * block size bs in {32, 64, 128, 256}; NBI = max(1, 128/bs)):
 *   rows in tiles of 16 (T = ceil(N/16), the last tile padded with zero
 *   rows), each row's weights in items of 128 (C = K/128); tile t's item c
 *   is a record of RB bytes at byte offset (t*C + c)*RB, RB = 1184 (bs 32),
 *   1104 (bs 64) or 1072 (bs 128, 256):
 *   bytes [0, 1024)     16 bytes per lane l = 16g + n (n, g = 0..15, 0..3):
 *                       4-byte word j (j = 0..3) at 16l + 4j is the original
 *                       4-byte word of row 16t + n at byte 64c + 16j + 4g
 *                       (weights k = 128c + 32j + 8g .. +7);
 *   [1024, 1024+32NBI)  fp16 scales [16][NBI]: entry (n, b) is the scale of
 *                       row 16t + n, block 128c/bs + b (bs = 256: block c/2);
 *   next 16 bytes (32 when NBI = 4)  zero points: max(1, NBI/2) bytes per
 *                       row n; bits 4b..4b+3 hold the zero point of the
 *                       same block (8 when zero_points was NULL), other
 *                       bits 0.
 *   Padding rows hold zero codes, scales and zero points.
 * A layout flag other than QG_INT4_LAYOUT_TILE16_V1 returns
 * QG_ERR_UNSUPPORTED, so a buffer written by a later layout version cannot
 * be read as this one.
 */
#define QG_INT4_LAYOUT_TILE16_V1 1

/* Bytes of the packed form of an N x K matrix with block size block_size in
 * `layout`; 0 when the layout, block size or shape is not provided (N < 0,
 * K not a positive multiple of 128 and of block_size). */
size_t int4_packed_bytes(int64_t N, int64_t K, int32_t block_size,
                         int32_t layout);

/*
 * int4_repack -- write the packed form of (w, scales, zero_points), whose
 * layout and meaning are those of qgemv_int4_blockwise, into `packed`.  Run
 * once per weight, on `stream`.
 * w : [N][K/2] bytes, 4-byte aligned.  scales : fp16 bits [N][K/bs],
 * 2-byte aligned.  zero_points : [N][ceil((K/bs)/2)] bytes or NULL
 * (zero point 8).  packed : packed_bytes >= int4_packed_bytes(N, K,
 * block_size, layout) bytes, 16-byte aligned, not overlapping an input
 * (QG_ERR_BAD_SHAPE when too small, QG_ERR_ALIAS on overlap).  N == 0
 * enqueues nothing.
 */
qg_status int4_repack(const uint8_t *w, const uint16_t *scales,
                      const uint8_t *zero_points, uint8_t *packed,
                      size_t packed_bytes, int64_t N, int64_t K,
                      int32_t block_size, int32_t layout, void *stream);

/*
 * qgemv_int4_packed -- y = x . dequant(W)^T with W in the packed layout
 * written by int4_repack (the same N, K, block_size and layout).
 * x, x_type, y, y_type, ldx, ldy, M, N : as in qgemv_int4_blockwise.
 * packed, packed_bytes : the packed weights (16-byte aligned) and the size
 *                        of that buffer (QG_ERR_BAD_SHAPE when below
 *                        int4_packed_bytes).
 * Rows of x beyond what one launch keeps in LDS are run as groups of rows,
 * each reading the weights again; K above about 80000 (one row of x no
 * longer fits) returns QG_ERR_UNSUPPORTED.
 */
qg_status qgemv_int4_packed(const void *x, int64_t ldx, int32_t x_type,
                            const uint8_t *packed, size_t packed_bytes,
                            int32_t layout, void *y, int64_t ldy,
                            int32_t y_type, int64_t M, int64_t N, int64_t K,
                            int32_t block_size, void *stream);

/*
 * qgemv_q4k -- q4_K GEMV, scale/min decoded inside the kernel.
 *
 * Operation: "62 . r59 -- q4_K W_dsc plane + riders", sections 2.1 and 3.2.
 * Row n of W is K/256 super-blocks of 144 bytes.  Super-block sb of row n
 * starts at w + (n*(K/256) + sb)*144 and holds: d (fp16, bytes 0..1), dmin
 * (fp16, bytes 2..3), twelve bytes of packed 6-bit scales and mins (4..15),
 * and 128 bytes of 4-bit quants qs (16..143).  For element e = k mod 256,
 * chunk cc = e/32, l = e%32, g = cc/2:
 *     q = low nibble of qs[32g + l] for even cc, high nibble for odd cc
 *     (sc, m) = get_scale_min_k4(cc):  cc < 4: sc = b[cc] & 63,
 *               m = b[cc+4] & 63;  cc >= 4: sc = (b[cc+4] & 15) |
 *               ((b[cc-4] >> 6) << 4),  m = (b[cc+4] >> 4) | ((b[cc] >> 6) << 4)
 *     dv = float(d) * sc,  mv = -(float(dmin) * m)       (exact binary32)
 *     w[n,k] = dv*q + mv                                  (binary32)
 *     y[m,n] = sum_k x[m,k] * w[n,k]
 *
 * x : binary32, [M][ldx], 4-byte aligned.
 * w : [N][K/256][144] bytes, 16-byte aligned.  K must be a positive multiple
 *     of 256.
 * y : binary32, [M][ldy].
 */
qg_status qgemv_q4k(const float *x, int64_t ldx, const uint8_t *w, float *y,
                    int64_t ldy, int64_t M, int64_t N, int64_t K, void *stream);

/*
 * qgemv_q4k_dsc -- q4_K GEMV reading (dv, mv) from a W_dsc plane.
 *
 * Operation: "62 . r59 -- q4_K W_dsc plane + riders", section 2.2: the same
 * result as qgemv_q4k, with the coefficients of chunk c = k/32 of row n read
 * from dsc[(c*N + n)*2 + 0] (dv) and dsc[(c*N + n)*2 + 1] (mv) instead of
 * being decoded from the super-block header.  The quants are read from `w`
 * exactly as in qgemv_q4k (the header bytes are not read).  With a plane
 * built by q4k_build_dsc_plane from the same `w`, the result is bitwise equal
 * to qgemv_q4k's (the two share one kernel and one summation order).
 *
 * dsc : binary32 pairs, [(K/32)*N][2], 16-byte aligned.  NULL is an error
 *       (QG_ERR_NULL_POINTER); the library never falls back silently.
 * other arguments as in qgemv_q4k.
 */
qg_status qgemv_q4k_dsc(const float *x, int64_t ldx, const uint8_t *w,
                        const float *dsc, float *y, int64_t ldy, int64_t M,
                        int64_t N, int64_t K, void *stream);

/*
 * gemv_bf16 -- dense bf16 GEMV, any K >= 1 and any 2-byte storage offset.
 *
 * Operation: the bf16 GEMV primitive of the AstrAI backend commit list
 * (M = 1..8, M = 9 rejected; 128-bit weight loads anchored at each row's first
 * 16-byte-aligned address with scalar head/tail sweeps, so that any positive
 * K and any storage offset is correct).
 *     y[m,n] = sum_k x[m,k] * w[n,k]
 *
 * x : bfloat16 bits, [M][ldx], 2-byte aligned, ldx >= K.
 * w : bfloat16 bits, [N][ldw], 2-byte aligned, ldw >= K.
 * y : [M][ldy] of y_type (QG_BF16, QG_F32 or QG_F16).
 */
qg_status gemv_bf16(const uint16_t *x, int64_t ldx, const uint16_t *w,
                    int64_t ldw, void *y, int64_t ldy, int32_t y_type,
                    int64_t M, int64_t N, int64_t K, void *stream);

/*
 * q4k_dsc_plane_bytes -- size in bytes of the W_dsc plane of an N x K q4_K
 * matrix: (K/32) chunks * N rows * 8 bytes = N*K/4 ("62 . r59 -- q4_K W_dsc
 * plane + riders", section 2.2).  Returns 0 when N < 0, K < 1 or K is not a
 * multiple of 256.
 */
size_t q4k_dsc_plane_bytes(int64_t N, int64_t K);

/*
 * q4k_build_dsc_plane -- load-time repack of raw q4_K weights into the
 * chunk-major W_dsc plane ("62 . r59 -- q4_K W_dsc plane + riders", sections
 * 2.2, 2.3 and 3.2): for every row n and global chunk c = sb*8 + cc,
 *     dsc_out[(c*N + n)*2 + 0] = float(d) * sc      (one binary32 multiply)
 *     dsc_out[(c*N + n)*2 + 1] = -(float(dmin) * m) (exact negation: -0.0
 *                                                   when m == 0 or dmin == 0)
 * The plane is byte-identical to the definition.  Run once per weight.
 *
 * w       : [N][K/256][144] bytes, 16-byte aligned; K a positive multiple of
 *           256; any N >= 0.
 * dsc_out : q4k_dsc_plane_bytes(N, K) bytes, 16-byte aligned, must not
 *           overlap w.
 */
qg_status q4k_build_dsc_plane(const uint8_t *w, float *dsc_out, int64_t N,
                              int64_t K, void *stream);

/*
 * q4_K prefill with 8-bit activations ("62 . r59 -- q4_K W_dsc plane +
 * riders", section 2.1: the rank-1 rescale of each (chunk, row) integer dot
 * product by (d*sc, -dmin*m) read from the W_dsc plane; section 3.2: the
 * activations are quantized to 8 bits in a prepass before the integer matrix
 * product).  For any number T of activation rows:
 *     y[t,n] = sum_c d_a[t,c] * (dv[n,c] * sum_{k in c} q_w[n,k] * q_a[t,k]
 *                               + mv[n,c] * sum_{k in c} q_a[t,k])
 * The activation rule is not given on the page; this library uses, per block
 * of 32 consecutive k of one row (one weight chunk): d_a = amax / 127 and
 * q_a = x / d_a rounded half away from zero, both correctly rounded binary32
 * operations; an all-zero block has d_a = 0 and q_a = 0.
 */

/* Workspace bytes qgemm_q4k_mmq needs for T activation rows of length K: the
 * codes (T*K bytes, rounded up to 256) followed by T*(K/32) float2 (d_a,
 * d_a * sum q_a).  0 when T < 1 or K is not a positive multiple of 256. */
size_t q4k_mmq_workspace_bytes(int64_t T, int64_t K);

/*
 * q8_quantize_rows -- the activation prepass alone.
 * x   : float32 [T][ldx], 4-byte aligned, ldx >= K; K a positive multiple of
 *       32; T >= 0 (T == 0 enqueues nothing).
 * qa  : int8 [T][K] codes out, 4-byte aligned.
 * sda : float32 [T][K/32][2] out, 8-byte aligned: (d_a, d_a * sum of the
 *       block's codes), the product rounded to binary32.
 * qa, sda and x must not overlap.
 */
qg_status q8_quantize_rows(const float *x, int64_t ldx, int8_t *qa, float *sda,
                           int64_t T, int64_t K, void *stream);

/*
 * qgemm_q4k_mmq -- the prefill product: prepass into `workspace`, then the
 * int8 matrix-core product rescaled with the plane.  Two kernels on `stream`.
 * x         : float32 [T][ldx], 4-byte aligned, ldx >= K.
 * w         : raw q4_K [N][K/256][144] bytes, 16-byte aligned, < 4 GiB.
 * dsc       : the W_dsc plane of w (q4k_build_dsc_plane), 16-byte aligned;
 *             NULL is an error (QG_ERR_NULL_POINTER), never a silent fallback.
 * y         : float32 [T][ldy] out, ldy >= N, 4-byte aligned.
 * workspace : caller-owned device scratch of at least
 *             q4k_mmq_workspace_bytes(T, K) bytes, 256-byte aligned; its
 *             contents are overwritten; calls that share one workspace on
 *             different streams race.
 * T, N >= 0 (either 0 enqueues nothing), K a positive multiple of 256.
 * y must not overlap x, w, dsc or the workspace, nor the workspace an input.
 */
qg_status qgemm_q4k_mmq(const float *x, int64_t ldx, const uint8_t *w,
                        const float *dsc, float *y, int64_t ldy, int64_t T,
                        int64_t N, int64_t K, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * qgemm_q4k_mmq_noalloc -- qgemm_q4k_mmq for callers that cannot allocate
 * device memory (code recorded under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same two kernels and the same result,
 * bit for bit, with the workspace taken from a static device array of the
 * library instead of a caller-owned buffer.  It calls no allocating routine.
 *
 * The array holds QG_MMQ_NOALLOC_SCRATCH_BYTES bytes; every GPU the library
 * runs on keeps its own copy from the library's load until the process ends.
 * Problems whose q4k_mmq_workspace_bytes(T, K) exceeds it return
 * QG_ERR_UNSUPPORTED with nothing enqueued (use qgemm_q4k_mmq).  The prepass
 * overwrites every workspace byte the product reads, so nothing has to start
 * at zero, but all calls on one GPU share the array: calls that overlap on
 * one GPU (different streams, or host threads) race and must be serialised
 * by the caller.
 * Arguments as in qgemm_q4k_mmq, without the workspace; y must not overlap
 * x, w or dsc.
 */
#define QG_MMQ_NOALLOC_SCRATCH_BYTES (32u << 20)
qg_status qgemm_q4k_mmq_noalloc(const float *x, int64_t ldx, const uint8_t *w,
                                const float *dsc, float *y, int64_t ldy,
                                int64_t T, int64_t N, int64_t K, void *stream);

/* Static English name of a status code ("QG_OK", ...). */
const char *qg_status_string(qg_status s);

/* Detail of the last non-QG_OK status returned on the calling thread, or ""
 * when the last call succeeded.  The string lives until the next call on the
 * same thread. */
const char *qg_last_error(void);

/*
 * Liveness and explain trace (for callers that dispatch on top of this
 * library).  Which kernel path produced a result cannot be told from the
 * result, so every launch is counted and described by name; a caller that
 * falls back from a fast path can then report it ("62 . r59 -- q4_K W_dsc
 * plane + riders", section 3.1, on failures that must not go unnoticed;
 * section 4, liveness).
 *
 * qg_last_launch   : the kernels enqueued by the calling thread's last library
 *                    call, as "path M=.. grid=.. block=.. lds=.." entries
 *                    separated by "; " ("" if it enqueued nothing).  The
 *                    string is thread-local storage owned by the library,
 *                    valid until the thread's next call.
 * qg_path_count    : number of kernel paths.
 * qg_path_name     : the name of path i (NULL when out of range); static
 *                    storage.
 * qg_path_launches : launches of path i since the library was loaded (all
 *                    threads; 0 when out of range).
 * Host-only; none of these touches the GPU.
 */
const char *qg_last_launch(void);
int32_t qg_path_count(void);
const char *qg_path_name(int32_t path);
uint64_t qg_path_launches(int32_t path);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_H */
