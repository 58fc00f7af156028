// qgemv_launch.h -- internal launchers (host side), one per kernel family.
// Arguments have already been validated by qgemv_api.cpp; each launcher picks
// a launch geometry, enqueues one kernel on `stream` and returns the HIP status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace qg {

// Kernel paths, for the liveness record of every launch (note_launch):
// which kernel family ran, counted per process and described per thread.
enum Path : int {
  kPathInt4Dot2Persistent = 0,
  kPathInt4Dot2Tiled,
  kPathInt4MfmaTiles,
  kPathInt4MfmaSplit,
  kPathInt4MfmaPhased,
  kPathQ4kPersistent,
  kPathQ4kPersistentPlane,
  kPathQ4kTiled,
  kPathQ4kTiledPlane,
  kPathQ4kPlaneBuild,
  kPathBf16Aligned,
  kPathBf16MfmaTiles,
  kPathBf16MfmaSplit,
  kPathBf16General,
  kPathQ8Quantize,
  kPathQ4kMmq,
  kPathInt4Span,
  kPathInt4Repack,
  kPathInt4Packed,
    kPathCount
};

// Record one launch: counted for `path` and appended to the calling thread's
// description of its current library call (M rows of x, grid, workgroup
// size, dynamic LDS bytes).  Defined in qgemv_api.cpp.
void note_launch(Path path, int M, int grid, int block, size_t lds);

hipError_t launch_int4_gemv(const uint16_t* x, int64_t ldx, const uint8_t* w,
                            const uint16_t* scales, const uint8_t* zp, void* y,
                            int64_t ldy, int y_type, int M, int N, int K,
                            int block_size, hipStream_t stream);

// int4 packed layout (int4_packed.hip): bytes of one record (16 rows x 128
// weights with their scales and zero points), the rows of x one launch of the
// packed GEMV holds in LDS for rows of K, the load-time repack, and the GEMV.
int64_t int4_packed_record_bytes(int block_size);
size_t int4_packed_max_rows_of_x(int K);
hipError_t launch_int4_repack(const uint8_t* w, const uint16_t* scales, const uint8_t* zp,
                              uint8_t* out, int N, int K, int block_size, hipStream_t stream);
hipError_t launch_int4_gemv_packed(const uint16_t* x, int64_t ldx, const uint8_t* wp, void* y,
                                   int64_t ldy, int y_type, int M, int N, int K, int block_size,
                                   hipStream_t stream);

hipError_t launch_q4k_gemv(const float* x, int64_t ldx, const uint8_t* w,
                           const float* dsc, float* y, int64_t ldy, int M, int N,
                           int K, hipStream_t stream);

hipError_t launch_q4k_build_plane(const uint8_t* w, float* dsc, int N, int K,
                                  hipStream_t stream);

// q4_K prefill (q4k_mmq.hip): the 8-bit activation prepass, the bytes its
// codes take in a workspace (rounded up to 256), and the integer product.
size_t q8_workspace_codes_bytes(int64_t T, int64_t K);
hipError_t launch_q8_quantize(const float* x, int64_t ldx, int8_t* qa, float* sda, int T, int K,
                              hipStream_t stream);
hipError_t launch_q4k_mmq(const int8_t* qa, const float* sda, const uint8_t* w, const float* dsc,
                          float* y, int64_t ldy, int T, int N, int K, hipStream_t stream);
// Device address of the static workspace of qgemm_q4k_mmq_noalloc on the
// current device (QG_MMQ_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned),
// looked up on the first call per device; allocates nothing.
hipError_t mmq_static_scratch(void** ptr);

hipError_t launch_bf16_gemv(const uint16_t* x, int64_t ldx, const uint16_t* w,
                            int64_t ldw, void* y, int64_t ldy, int y_type, int M,
                            int N, int K, hipStream_t stream);

// LDS budget per workgroup for staged activations (bytes).
constexpr int kLdsBudget = 64 * 1024;
// gfx950 gives a workgroup up to 160 KB of LDS; a kernel must raise its
// dynamic-LDS limit (allow_lds) before it is launched with more than 64 KB.
constexpr int kLdsMax = 160 * 1024;
// The same budget less 1 KB for the static reduction buffers of the tiled
// kernels (the workgroup total stays within 64 KB).
constexpr int kLdsXBudget = kLdsBudget - 1024;

// Lanes that keep every CU busy: 256 CUs x 8 wavefronts x 64 lanes.
constexpr int64_t kLanesToFill = 256LL * 8 * 64;

// Lanes per row: start from `lpr` and double it (up to 256, and not past the
// row's piece count) until the N rows occupy `fill` lanes, so that short,
// wide matrices still launch enough wavefronts to hide HBM latency.  With
// `whole_strides` a doubling must also leave no lane without a piece.
inline int widen_lanes_per_row(int lpr, int N, int pieces, int64_t fill = kLanesToFill,
                               bool whole_strides = false) {
  while ((int64_t)N * lpr < fill && lpr < 256 &&
         (whole_strides ? 2 * lpr <= pieces : lpr < pieces))
    lpr *= 2;
  return lpr;
}

// Workgroups of `kernel` that fit on the whole device at once: a host-side
// occupancy calculation (no GPU work), remembered per (kernel, device, LDS).
template <typename F>
inline int resident_workgroups(F kernel, int threads, size_t shmem) {
  struct Entry {
    const void* fn;
    int dev;
    int threads;
    size_t shmem;
    int value;
  };
  static std::mutex mu;
  static Entry table[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (table[i].fn == fn && table[i].dev == dev && table[i].threads == threads &&
          table[i].shmem == shmem)
        return table[i].value;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, shmem) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 1;
  const int value = per_cu * cus;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 256) table[used++] = Entry{fn, dev, threads, shmem, value};
  return value;
}

// CUs of the current device (cached per device).
inline int device_cus() {
  static std::mutex mu;
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// k parts of a split matrix-core kernel (16 x 16 MFMA tiles whose columns
// may carry 16 / ks weight rows in ks parts of their k range): 1, or 2 (4)
// while 16-row (8-row) tiles number fewer than the CUs, the parts divide the
// row's 128-weight items, each of the `waves` wavefronts keeps at least one
// step, and M fits the A rows of a part.
inline int mfma_k_parts(int M, int N, int K, int waves) {
  const int C = K / 128, cus = device_cus();
  int ks = 1;
  while (ks < 4 && (N + 16 / ks - 1) / (16 / ks) < cus && M <= 8 / ks && C % (2 * ks) == 0 &&
         C / (2 * ks) >= waves)
    ks *= 2;
  return ks;
}

// Raise `kernel`'s dynamic-LDS limit to `bytes` when that is above 64 KB
// (once per kernel, device and size).
template <typename F>
inline hipError_t allow_lds(F kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  struct Entry {
    const void* fn;
    int dev;
    size_t bytes;
  };
  static std::mutex mu;
  static Entry table[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const void* fn = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (table[i].fn == fn && table[i].dev == dev && table[i].bytes >= bytes) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && used < 256) table[used++] = Entry{fn, dev, bytes};
  return e;
}

}  // namespace qg
