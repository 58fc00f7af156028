// qgemv_api.cpp -- the C ABI of libqgemv.so (declared in include/qgemv.h).
//
// Every entry point validates its arguments on the host -- pointers, shapes,
// strides, alignment, dtype, aliasing -- and only then enqueues exactly one
// kernel on the caller's stream.  Nothing is allocated and nothing is
// synchronised.  A failed validation enqueues nothing and records a
// human-readable detail for qg_last_error() in thread-local storage.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qgemv.h"
#include "qgemv_launch.h"

namespace {

thread_local char g_last_error[512];

// Liveness: per-path launch counts (process-wide) and the kernels launched by
// the calling thread's last library call.
std::atomic<uint64_t> g_path_launches[qg::kPathCount];
thread_local char g_last_launch[512];
thread_local int g_last_launch_count;

const char* const kPathNames[qg::kPathCount] = {
    "int4_dot2_persistent", "int4_dot2_tiled",      "int4_mfma_tiles", "int4_mfma_split",
    "int4_mfma_phased",     "q4k_persistent",       "q4k_persistent_plane", "q4k_tiled",
    "q4k_tiled_plane",      "q4k_plane_build",      "bf16_aligned",    "bf16_mfma_tiles",
    "bf16_mfma_split",      "bf16_general",         "q8_quantize",     "q4k_mmq",
    "int4_span",            "int4_repack",          "int4_packed"};

void begin_call() {
  g_last_launch[0] = '\0';
  g_last_launch_count = 0;
}

qg_status ok() {
  g_last_error[0] = '\0';
  return QG_OK;
}

__attribute__((format(printf, 2, 3))) qg_status fail(qg_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

qg_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QG_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Kernels address every tensor with 32-bit byte offsets.
constexpr int64_t kMaxTensorBytes = int64_t(1) << 32;

int dtype_size(int32_t t) { return t == QG_F32 ? 4 : 2; }

bool valid_out_dtype(int32_t t) { return t == QG_F16 || t == QG_BF16 || t == QG_F32; }

// Common shape checks.  Returns QG_OK or the failure already recorded.
qg_status check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 8) return fail(QG_ERR_BAD_SHAPE, "%s: M = %lld, must be in 1..8", fn, (long long)M);
  if (N < 0) return fail(QG_ERR_BAD_SHAPE, "%s: N = %lld < 0", fn, (long long)N);
  if (K < 1) return fail(QG_ERR_BAD_SHAPE, "%s: K = %lld < 1", fn, (long long)K);
  if (N > INT32_MAX || K > INT32_MAX)
    return fail(QG_ERR_BAD_SHAPE, "%s: N or K exceeds 2^31-1", fn);
  return QG_OK;
}

qg_status check_ld(const char* fn, const char* name, int64_t ld, int64_t need) {
  if (ld < need)
    return fail(QG_ERR_BAD_SHAPE, "%s: %s = %lld < %lld", fn, name, (long long)ld, (long long)need);
  return QG_OK;
}

}  // namespace

namespace qg {

void note_launch(Path path, int M, int grid, int block, size_t lds) {
  if (path < 0 || path >= kPathCount) return;
  g_path_launches[path].fetch_add(1, std::memory_order_relaxed);
  const size_t used = strlen(g_last_launch);
  if (used + 1 < sizeof(g_last_launch))
    snprintf(g_last_launch + used, sizeof(g_last_launch) - used, "%s%s M=%d grid=%d block=%d lds=%zu",
             g_last_launch_count ? "; " : "", kPathNames[path], M, grid, block, lds);
  ++g_last_launch_count;
}

}  // namespace qg

// The library is built with hidden visibility; only the C ABI is exported.
#pragma GCC visibility push(default)
extern "C" {

const char* qg_status_string(qg_status s) {
  switch (s) {
    case QG_OK: return "QG_OK";
    case QG_ERR_NULL_POINTER: return "QG_ERR_NULL_POINTER";
    case QG_ERR_BAD_SHAPE: return "QG_ERR_BAD_SHAPE";
    case QG_ERR_UNSUPPORTED: return "QG_ERR_UNSUPPORTED";
    case QG_ERR_MISALIGNED: return "QG_ERR_MISALIGNED";
    case QG_ERR_ALIAS: return "QG_ERR_ALIAS";
    case QG_ERR_HIP: return "QG_ERR_HIP";
  }
  return "QG_ERR_UNKNOWN";
}

const char* qg_last_error(void) { return g_last_error; }

const char* qg_last_launch(void) { return g_last_launch; }

int32_t qg_path_count(void) { return (int32_t)qg::kPathCount; }

const char* qg_path_name(int32_t path) {
  return path >= 0 && path < qg::kPathCount ? kPathNames[path] : nullptr;
}

uint64_t qg_path_launches(int32_t path) {
  return path >= 0 && path < qg::kPathCount
             ? g_path_launches[path].load(std::memory_order_relaxed)
             : 0;
}

qg_status qgemv_int4_blockwise(const void* xv, int64_t ldx, int32_t x_type, const uint8_t* w,
                               const uint16_t* scales, const uint8_t* zero_points, void* y,
                               int64_t ldy, int32_t y_type, int64_t M, int64_t N, int64_t K,
                               int32_t block_size, void* stream) {
  begin_call();
  static const char fn[] = "qgemv_int4_blockwise";
  const uint16_t* x = static_cast<const uint16_t*>(xv);
  if (!x || !w || !scales || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, w, scales and y are required", fn);
  if (x_type != QG_F16)
    return fail(QG_ERR_UNSUPPORTED, "%s: x_type %d (only QG_F16 activations are provided)", fn,
                x_type);
  if (qg_status s = check_mnk(fn, M, N, K)) return s;
  if (block_size != 32 && block_size != 64 && block_size != 128 && block_size != 256)
    return fail(QG_ERR_UNSUPPORTED, "%s: block_size %d not in {32, 64, 128, 256}", fn, block_size);
  if (K % block_size != 0)
    return fail(QG_ERR_BAD_SHAPE, "%s: K = %lld is not a multiple of block_size %d", fn,
                (long long)K, block_size);
  if (!valid_out_dtype(y_type)) return fail(QG_ERR_UNSUPPORTED, "%s: y_type %d", fn, y_type);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (qg_status s = check_ld(fn, "ldy", ldy, N)) return s;
  if (!aligned(w, 16)) return fail(QG_ERR_MISALIGNED, "%s: w must be 16-byte aligned", fn);
  if (!aligned(x, 2) || !aligned(scales, 2))
    return fail(QG_ERR_MISALIGNED, "%s: x and scales must be 2-byte aligned", fn);
  const int ysz = dtype_size(y_type);
  if (!aligned(y, ysz)) return fail(QG_ERR_MISALIGNED, "%s: y must be %d-byte aligned", fn, ysz);
  const int64_t nb = K / block_size;
  const int64_t zrow = (nb + 1) / 2;
  if (N * (K / 2) >= kMaxTensorBytes)
    return fail(QG_ERR_UNSUPPORTED, "%s: w is 4 GiB or larger (kernels use 32-bit offsets)", fn);
  const Range ry = range_of(y, ((M - 1) * ldy + N) * ysz);
  if (N > 0 && (overlap(ry, range_of(x, ((M - 1) * ldx + K) * 2)) ||
                overlap(ry, range_of(w, N * (K / 2))) || overlap(ry, range_of(scales, N * nb * 2)) ||
                (zero_points && overlap(ry, range_of(zero_points, N * zrow)))))
    return fail(QG_ERR_ALIAS, "%s: y overlaps an input", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_int4_gemv(x, ldx, w, scales, zero_points, y, ldy, y_type, (int)M,
                                         (int)N, (int)K, block_size,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

size_t int4_packed_bytes(int64_t N, int64_t K, int32_t block_size, int32_t layout) {
  if (layout != QG_INT4_LAYOUT_TILE16_V1 || N < 0 || K < 128 || K % 128 != 0 ||
      (block_size != 32 && block_size != 64 && block_size != 128 && block_size != 256) ||
      K % block_size != 0 || N > INT32_MAX || K > INT32_MAX)
    return 0;
  return (size_t)((N + 15) / 16) * (size_t)(K / 128) * (size_t)qg::int4_packed_record_bytes(block_size);
}

// Shape and layout checks shared by the repack and the packed GEMV.
static qg_status packed_checks(const char* fn, int64_t N, int64_t K, int32_t block_size,
                               int32_t layout, size_t packed_bytes, size_t* need) {
  if (layout != QG_INT4_LAYOUT_TILE16_V1)
    return fail(QG_ERR_UNSUPPORTED, "%s: layout %d (only QG_INT4_LAYOUT_TILE16_V1 = %d)", fn,
                layout, QG_INT4_LAYOUT_TILE16_V1);
  if (block_size != 32 && block_size != 64 && block_size != 128 && block_size != 256)
    return fail(QG_ERR_UNSUPPORTED, "%s: block_size %d not in {32, 64, 128, 256}", fn, block_size);
  if (N < 0 || N > INT32_MAX) return fail(QG_ERR_BAD_SHAPE, "%s: N = %lld", fn, (long long)N);
  if (K < 128 || K > INT32_MAX || K % 128 != 0 || K % block_size != 0)
    return fail(QG_ERR_BAD_SHAPE, "%s: K = %lld is not a positive multiple of 128 and of block_size %d",
                fn, (long long)K, block_size);
  *need = int4_packed_bytes(N, K, block_size, layout);
  if (packed_bytes < *need)
    return fail(QG_ERR_BAD_SHAPE, "%s: packed buffer of %zu bytes, the layout needs %zu", fn,
                packed_bytes, *need);
  return QG_OK;
}

qg_status int4_repack(const uint8_t* w, const uint16_t* scales, const uint8_t* zero_points,
                      uint8_t* packed, size_t packed_bytes, int64_t N, int64_t K,
                      int32_t block_size, int32_t layout, void* stream) {
  begin_call();
  static const char fn[] = "int4_repack";
  if (!w || !scales || !packed) return fail(QG_ERR_NULL_POINTER, "%s: w, scales and packed are required", fn);
  size_t need = 0;
  if (qg_status s = packed_checks(fn, N, K, block_size, layout, packed_bytes, &need)) return s;
  if (!aligned(w, 4) || !aligned(scales, 2) || !aligned(packed, 16))
    return fail(QG_ERR_MISALIGNED, "%s: w must be 4-, scales 2- and packed 16-byte aligned", fn);
  const int64_t nb = K / block_size;
  const int64_t zrow = (nb + 1) / 2;
  const Range rp = range_of(packed, (int64_t)need);
  if (N > 0 && (overlap(rp, range_of(w, N * (K / 2))) || overlap(rp, range_of(scales, N * nb * 2)) ||
                (zero_points && overlap(rp, range_of(zero_points, N * zrow)))))
    return fail(QG_ERR_ALIAS, "%s: packed overlaps an input", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_int4_repack(w, scales, zero_points, packed, (int)N, (int)K,
                                           block_size, static_cast<hipStream_t>(stream)),
                    fn);
}

qg_status qgemv_int4_packed(const void* xv, int64_t ldx, int32_t x_type, const uint8_t* packed,
                            size_t packed_bytes, int32_t layout, void* y, int64_t ldy,
                            int32_t y_type, int64_t M, int64_t N, int64_t K, int32_t block_size,
                            void* stream) {
  begin_call();
  static const char fn[] = "qgemv_int4_packed";
  const uint16_t* x = static_cast<const uint16_t*>(xv);
  if (!x || !packed || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, packed and y are required", fn);
  if (x_type != QG_F16)
    return fail(QG_ERR_UNSUPPORTED, "%s: x_type %d (only QG_F16 activations are provided)", fn,
                x_type);
  if (qg_status s = check_mnk(fn, M, N, K)) return s;
  size_t need = 0;
  if (qg_status s = packed_checks(fn, N, K, block_size, layout, packed_bytes, &need)) return s;
  if (qg::int4_packed_max_rows_of_x((int)K) < 1)
    return fail(QG_ERR_UNSUPPORTED, "%s: K = %lld: one row of x does not fit in LDS", fn, (long long)K);
  if (!valid_out_dtype(y_type)) return fail(QG_ERR_UNSUPPORTED, "%s: y_type %d", fn, y_type);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (qg_status s = check_ld(fn, "ldy", ldy, N)) return s;
  if (!aligned(packed, 16)) return fail(QG_ERR_MISALIGNED, "%s: packed must be 16-byte aligned", fn);
  if (!aligned(x, 2)) return fail(QG_ERR_MISALIGNED, "%s: x must be 2-byte aligned", fn);
  const int ysz = dtype_size(y_type);
  if (!aligned(y, ysz)) return fail(QG_ERR_MISALIGNED, "%s: y must be %d-byte aligned", fn, ysz);
  const Range ry = range_of(y, ((M - 1) * ldy + N) * ysz);
  if (N > 0 && (overlap(ry, range_of(x, ((M - 1) * ldx + K) * 2)) ||
                overlap(ry, range_of(packed, (int64_t)need))))
    return fail(QG_ERR_ALIAS, "%s: y overlaps an input", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_int4_gemv_packed(x, ldx, packed, y, ldy, y_type, (int)M, (int)N,
                                                (int)K, block_size, static_cast<hipStream_t>(stream)),
                    fn);
}

static qg_status q4k_common(const char* fn, const float* x, int64_t ldx, const uint8_t* w,
                            const float* dsc, float* y, int64_t ldy, int64_t M, int64_t N,
                            int64_t K, void* stream) {
  if (qg_status s = check_mnk(fn, M, N, K)) return s;
  if (K % 256 != 0)
    return fail(QG_ERR_BAD_SHAPE, "%s: K = %lld is not a multiple of 256", fn, (long long)K);
  if (N * (K / 256) * 144 >= kMaxTensorBytes)
    return fail(QG_ERR_UNSUPPORTED, "%s: w is 4 GiB or larger (kernels use 32-bit offsets)", fn);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (qg_status s = check_ld(fn, "ldy", ldy, N)) return s;
  if (!aligned(w, 16)) return fail(QG_ERR_MISALIGNED, "%s: w must be 16-byte aligned", fn);
  if (dsc && !aligned(dsc, 16)) return fail(QG_ERR_MISALIGNED, "%s: dsc must be 16-byte aligned", fn);
  if (!aligned(x, 4) || !aligned(y, 4))
    return fail(QG_ERR_MISALIGNED, "%s: x and y must be 4-byte aligned", fn);
  const Range ry = range_of(y, ((M - 1) * ldy + N) * 4);
  if (N > 0 && (overlap(ry, range_of(x, ((M - 1) * ldx + K) * 4)) ||
                overlap(ry, range_of(w, N * (K / 256) * 144)) ||
                (dsc && overlap(ry, range_of(dsc, N * K / 4)))))
    return fail(QG_ERR_ALIAS, "%s: y overlaps an input", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_q4k_gemv(x, ldx, w, dsc, y, ldy, (int)M, (int)N, (int)K,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

qg_status qgemv_q4k(const float* x, int64_t ldx, const uint8_t* w, float* y, int64_t ldy,
                    int64_t M, int64_t N, int64_t K, void* stream) {
  begin_call();
  static const char fn[] = "qgemv_q4k";
  if (!x || !w || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, w and y are required", fn);
  return q4k_common(fn, x, ldx, w, nullptr, y, ldy, M, N, K, stream);
}

qg_status qgemv_q4k_dsc(const float* x, int64_t ldx, const uint8_t* w, const float* dsc, float* y,
                        int64_t ldy, int64_t M, int64_t N, int64_t K, void* stream) {
  begin_call();
  static const char fn[] = "qgemv_q4k_dsc";
  if (!x || !w || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, w and y are required", fn);
  if (!dsc) return fail(QG_ERR_NULL_POINTER, "%s: dsc plane is NULL (no silent fallback)", fn);
  return q4k_common(fn, x, ldx, w, dsc, y, ldy, M, N, K, stream);
}

qg_status gemv_bf16(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                    int64_t ldy, int32_t y_type, int64_t M, int64_t N, int64_t K, void* stream) {
  begin_call();
  static const char fn[] = "gemv_bf16";
  if (!x || !w || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, w and y are required", fn);
  if (qg_status s = check_mnk(fn, M, N, K)) return s;
  if (!valid_out_dtype(y_type)) return fail(QG_ERR_UNSUPPORTED, "%s: y_type %d", fn, y_type);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (qg_status s = check_ld(fn, "ldw", ldw, K)) return s;
  if (qg_status s = check_ld(fn, "ldy", ldy, N)) return s;
  if (N > 0 && ((N - 1) * ldw + K) * 2 >= kMaxTensorBytes)
    return fail(QG_ERR_UNSUPPORTED, "%s: w spans 4 GiB or more (kernels use 32-bit offsets)", fn);
  if (!aligned(x, 2) || !aligned(w, 2))
    return fail(QG_ERR_MISALIGNED, "%s: x and w must be 2-byte aligned", fn);
  const int ysz = dtype_size(y_type);
  if (!aligned(y, ysz)) return fail(QG_ERR_MISALIGNED, "%s: y must be %d-byte aligned", fn, ysz);
  const Range ry = range_of(y, ((M - 1) * ldy + N) * ysz);
  if (N > 0 && (overlap(ry, range_of(x, ((M - 1) * ldx + K) * 2)) ||
                overlap(ry, range_of(w, ((N - 1) * ldw + K) * 2))))
    return fail(QG_ERR_ALIAS, "%s: y overlaps an input", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_bf16_gemv(x, ldx, w, ldw, y, ldy, y_type, (int)M, (int)N, (int)K,
                                         static_cast<hipStream_t>(stream)),
                    fn);
}

size_t q4k_dsc_plane_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 1 || K % 256 != 0) return 0;
  return (size_t)N * (size_t)K / 4;
}

qg_status q4k_build_dsc_plane(const uint8_t* w, float* dsc_out, int64_t N, int64_t K,
                              void* stream) {
  begin_call();
  static const char fn[] = "q4k_build_dsc_plane";
  if (!w || !dsc_out) return fail(QG_ERR_NULL_POINTER, "%s: w and dsc_out are required", fn);
  if (N < 0 || K < 1 || K % 256 != 0)
    return fail(QG_ERR_BAD_SHAPE, "%s: N = %lld, K = %lld (need N >= 0, K a positive multiple of 256)",
                fn, (long long)N, (long long)K);
  if (N > INT32_MAX || K > INT32_MAX) return fail(QG_ERR_BAD_SHAPE, "%s: N or K exceeds 2^31-1", fn);
  if (!aligned(w, 16) || !aligned(dsc_out, 16))
    return fail(QG_ERR_MISALIGNED, "%s: w and dsc_out must be 16-byte aligned", fn);
  if (N * (K / 256) * 144 >= kMaxTensorBytes)
    return fail(QG_ERR_UNSUPPORTED, "%s: w is 4 GiB or larger (kernels use 32-bit offsets)", fn);
  if (N > 0 && overlap(range_of(dsc_out, N * K / 4), range_of(w, N * (K / 256) * 144)))
    return fail(QG_ERR_ALIAS, "%s: dsc_out overlaps w", fn);
  if (N == 0) return ok();
  return hip_status(qg::launch_q4k_build_plane(w, dsc_out, (int)N, (int)K,
                                               static_cast<hipStream_t>(stream)),
                    fn);
}

size_t q4k_mmq_workspace_bytes(int64_t T, int64_t K) {
  if (T < 1 || K < 256 || K % 256 != 0 || T > INT32_MAX || K > INT32_MAX) return 0;
  return qg::q8_workspace_codes_bytes(T, K) + (size_t)T * (size_t)(K / 32) * 8;
}

qg_status q8_quantize_rows(const float* x, int64_t ldx, int8_t* qa, float* sda, int64_t T,
                           int64_t K, void* stream) {
  begin_call();
  static const char fn[] = "q8_quantize_rows";
  if (!x || !qa || !sda) return fail(QG_ERR_NULL_POINTER, "%s: x, qa and sda are required", fn);
  if (T < 0 || K < 32 || K % 32 != 0)
    return fail(QG_ERR_BAD_SHAPE, "%s: T = %lld, K = %lld (need T >= 0, K a positive multiple of 32)",
                fn, (long long)T, (long long)K);
  if (T > INT32_MAX || K > INT32_MAX) return fail(QG_ERR_BAD_SHAPE, "%s: T or K exceeds 2^31-1", fn);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (!aligned(x, 4) || !aligned(qa, 4) || !aligned(sda, 8))
    return fail(QG_ERR_MISALIGNED, "%s: x and qa must be 4-byte, sda 8-byte aligned", fn);
  if (T == 0) return ok();
  const Range rx = range_of(x, ((T - 1) * ldx + K) * 4), rq = range_of(qa, T * K),
              rs = range_of(sda, T * (K / 32) * 8);
  if (overlap(rq, rx) || overlap(rs, rx) || overlap(rq, rs))
    return fail(QG_ERR_ALIAS, "%s: qa, sda and x must not overlap", fn);
  return hip_status(qg::launch_q8_quantize(x, ldx, qa, sda, (int)T, (int)K,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

static qg_status mmq_common(const char* fn, const float* x, int64_t ldx, const uint8_t* w,
                            const float* dsc, float* y, int64_t ldy, int64_t T, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes, bool static_ws,
                            void* stream) {
  if (!x || !w || !y) return fail(QG_ERR_NULL_POINTER, "%s: x, w and y are required", fn);
  if (!dsc) return fail(QG_ERR_NULL_POINTER, "%s: dsc plane is NULL (no silent fallback)", fn);
  if (T < 0 || N < 0 || K < 256 || K % 256 != 0)
    return fail(QG_ERR_BAD_SHAPE,
                "%s: T = %lld, N = %lld, K = %lld (need T, N >= 0, K a positive multiple of 256)", fn,
                (long long)T, (long long)N, (long long)K);
  if (T > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(QG_ERR_BAD_SHAPE, "%s: T, N or K exceeds 2^31-1", fn);
  if (qg_status s = check_ld(fn, "ldx", ldx, K)) return s;
  if (qg_status s = check_ld(fn, "ldy", ldy, N)) return s;
  if (T == 0 || N == 0) return ok();
  const size_t need = q4k_mmq_workspace_bytes(T, K);
  if (static_ws) {
    if (need > (size_t)QG_MMQ_NOALLOC_SCRATCH_BYTES)
      return fail(QG_ERR_UNSUPPORTED,
                  "%s: T = %lld rows of K = %lld need %zu bytes of workspace, the static scratch "
                  "holds %zu (use qgemm_q4k_mmq with a workspace)",
                  fn, (long long)T, (long long)K, need, (size_t)QG_MMQ_NOALLOC_SCRATCH_BYTES);
  } else {
    if (!workspace) return fail(QG_ERR_NULL_POINTER, "%s: workspace is required", fn);
    if (workspace_bytes < need)
      return fail(QG_ERR_BAD_SHAPE, "%s: workspace of %zu bytes, need %zu (q4k_mmq_workspace_bytes)",
                  fn, workspace_bytes, need);
  }
  const int64_t wbytes = N * (K / 256) * 144;
  if (wbytes >= kMaxTensorBytes)
    return fail(QG_ERR_UNSUPPORTED, "%s: w is 4 GiB or larger (kernels use 32-bit offsets)", fn);
  if (!aligned(w, 16) || !aligned(dsc, 16) || !aligned(x, 4) || !aligned(y, 4))
    return fail(QG_ERR_MISALIGNED, "%s: w and dsc must be 16-byte, x and y 4-byte aligned", fn);
  if (static_ws) {
    // The first call on a device looks the array's address up (no
    // allocation); later calls reuse it.
    const hipError_t e = qg::mmq_static_scratch(&workspace);
    if (e != hipSuccess) return hip_status(e, fn);
  } else if (!aligned(workspace, 256)) {
    return fail(QG_ERR_MISALIGNED, "%s: workspace must be 256-byte aligned", fn);
  }
  const Range rx = range_of(x, ((T - 1) * ldx + K) * 4), rw = range_of(w, wbytes),
              rd = range_of(dsc, N * K / 4), rws = range_of(workspace, (int64_t)need),
              ry = range_of(y, ((T - 1) * ldy + N) * 4);
  if (overlap(ry, rx) || overlap(ry, rw) || overlap(ry, rd) || overlap(ry, rws))
    return fail(QG_ERR_ALIAS, "%s: y overlaps an input or the workspace", fn);
  if (overlap(rws, rx) || overlap(rws, rw) || overlap(rws, rd))
    return fail(QG_ERR_ALIAS, "%s: the workspace overlaps an input", fn);
  int8_t* qa = static_cast<int8_t*>(workspace);
  float* sda = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        qg::q8_workspace_codes_bytes(T, K));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = qg::launch_q8_quantize(x, ldx, qa, sda, (int)T, (int)K, st);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(qg::launch_q4k_mmq(qa, sda, w, dsc, y, ldy, (int)T, (int)N, (int)K, st), fn);
}

qg_status qgemm_q4k_mmq(const float* x, int64_t ldx, const uint8_t* w, const float* dsc, float* y,
                        int64_t ldy, int64_t T, int64_t N, int64_t K, void* workspace,
                        size_t workspace_bytes, void* stream) {
  begin_call();
  return mmq_common("qgemm_q4k_mmq", x, ldx, w, dsc, y, ldy, T, N, K, workspace, workspace_bytes,
                    false, stream);
}

qg_status qgemm_q4k_mmq_noalloc(const float* x, int64_t ldx, const uint8_t* w, const float* dsc,
                                float* y, int64_t ldy, int64_t T, int64_t N, int64_t K,
                                void* stream) {
  begin_call();
  return mmq_common("qgemm_q4k_mmq_noalloc", x, ldx, w, dsc, y, ldy, T, N, K, nullptr, 0, true,
                    stream);
}

}  // extern "C"
#pragma GCC visibility pop
