// int4_packed.hip -- MatMulNBits int4 weights repacked once at load time for
// the matrix-core GEMV, and the GEMV that reads them (gfx950, M = 1..8).
//
// Operation: the int4 MatMulNBits GEMV of the onnx-genai pull request #1000
// ("Summary", "What it does"), y[m,n] = sum_k x[m,k] * s[n,k/bs] * (q[n,k] -
// zp[n,k/bs]), on weights that an offline repack has put into a versioned
// layout (the page's "Roadmap recommendation": offline weight repack plus a
// layout flag).  The values are those of the original layout, bit for bit;
// only their order in memory changes.
//
// Layout QG_INT4_LAYOUT_TILE16_V1 (block size bs in {32, 64, 128, 256}, K a
// multiple of 128; NBI = max(1, 128 / bs) scale blocks per 128 weights):
//   rows are grouped in tiles of 16 (the last tile padded with zero rows), a
//   row's K weights in items of 128, and tile t's item c is one record of
//   RB = 1024 + 32 * NBI + ZB bytes (ZB = 32 for NBI = 4, else 16) at byte
//   (t * K/128 + c) * RB:
//   [0, 1024)   lane l = (n = l % 16, g = l / 16) owns bytes 16 l .. 16 l + 15:
//               32-bit word j (j = 0..3) is the original word of row 16t + n
//               at byte 64c + 16j + 4g, i.e. weights k = 128c + 32j + 8g + e
//               (e = 0..7), nibbles in their original order;
//   [1024, +32 NBI)  fp16 scales, [16 rows][NBI]: scale b of row n is the
//               original scale of block (128c) / bs + b (bs <= 128) or c / 2
//               (bs = 256);
//   [1024 + 32 NBI, +ZB)  zero points, max(1, NBI / 2) bytes per row: nibble
//               b (bits 4b..4b+3) of row n's bytes is the zero point of the
//               same block (8 when the original has none); other bits 0.
//   Padding rows have zero weights, scales and zero points.
// Why: lane (n, g) then holds, in word j, exactly the B operand of the j-th
// v_mfma_f32_16x16x32_f16 of the item (no lane exchanges), its scales and
// zero points are one small load each, and a wavefront's consecutive items
// are consecutive 1 KB runs of HBM.
#include <type_traits>

#include "int4_device.h"
#include "qgemv_launch.h"

namespace qg {
namespace {

template <int NBI>
struct PackedGeom {
  static constexpr int kScaleBytes = 32 * NBI;
  static constexpr int kZpBytes = NBI == 4 ? 32 : 16;
  static constexpr int kRecord = 1024 + kScaleBytes + kZpBytes;
  static constexpr int kZpRowBytes = NBI == 4 ? 2 : 1;
};

// One thread per (record, lane): lane l writes its 16 weight bytes; lanes
// 0..15 also write row l's scales and zero points.  Any N >= 1.
template <int NBI>
__global__ __launch_bounds__(kBlock) void int4_repack_kernel(
    const uint8_t* __restrict__ w, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zp, uint8_t* __restrict__ out, int N, int K, int bs_log2,
    int zrow, int64_t nrec) {
  using Geo = PackedGeom<NBI>;
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t r = t >> 6;  // record
  if (r >= nrec) return;
  const int l = (int)(t & 63);
  const int C = K >> 7;
  const int tile = (int)(r / C), c = (int)(r - (int64_t)tile * C);
  const int n = l & 15, g = l >> 4;
  const int row = tile * 16 + n;
  uint8_t* rec = out + r * Geo::kRecord;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < N) {
    const uint32_t* wr = reinterpret_cast<const uint32_t*>(w + (size_t)row * (size_t)(K >> 1));
    // word j at byte 64c + 16j + 4g
    v.x = wr[(64 * c + 0 + 4 * g) >> 2];
    v.y = wr[(64 * c + 16 + 4 * g) >> 2];
    v.z = wr[(64 * c + 32 + 4 * g) >> 2];
    v.w = wr[(64 * c + 48 + 4 * g) >> 2];
  }
  *reinterpret_cast<uint4*>(rec + 16 * l) = v;
  if (l < 16) {
    const int nb = K >> bs_log2;
    const int blk0 = (128 * c) >> bs_log2;  // the item's first block
    uint16_t* sd = reinterpret_cast<uint16_t*>(rec + 1024) + n * NBI;
    uint32_t zbits = 0;
#pragma unroll
    for (int b = 0; b < NBI; ++b) {
      const int blk = blk0 + b;
      uint16_t s = 0;
      uint32_t z = 0;
      if (row < N) {
        s = scales[(size_t)row * nb + blk];
        z = zp ? (zp[(size_t)row * zrow + (blk >> 1)] >> ((blk & 1) << 2)) & 15u : 8u;
      }
      sd[b] = s;
      zbits |= z << (4 * b);
    }
    uint8_t* zd = rec + 1024 + Geo::kScaleBytes + n * Geo::kZpRowBytes;
    zd[0] = (uint8_t)(zbits & 0xFFu);
    if (Geo::kZpRowBytes == 2) zd[1] = (uint8_t)(zbits >> 8);
    // 16 rows x kZpRowBytes = kZpBytes: every zero-point byte is written.
  }
}

// GEMV on the packed layout.  A workgroup of NW wavefronts takes tiles b,
// b + G, ... (G = grid); its wavefronts split each tile's K/128 items into
// NW contiguous ranges (every wavefront gets at least one item), and each
// stages in LDS the part of x its own items read.  Each lane
// keeps a ring of DG items in flight (weights, scales and zero points),
// reloaded as soon as an item is consumed.  Per item: four MFMAs
// v_mfma_f32_16x16x32_f16 with x (rows >= M repeat real rows; those outputs
// are not stored) as A and the unpacked exact (q - zp) as B; the fp32 result
// of each scale block is scaled once (the fp16 scale is exact in binary32).
// At a tile's end the wavefronts' partial sums meet in LDS and wavefront 0
// adds them in wavefront order (deterministic) and stores the tile's 16
// columns.
// XG: x is not staged in LDS; each item's four A operands are loaded from
// global memory (16 bytes per lane, 16-byte aligned rows of x) together with
// the item's weights, into the same ring.  Used for rows of x that LDS cannot
// hold at once, instead of one launch (and one pass over the weights) per
// group of rows: 4096 x 11008 at M = 8 takes 13.3 us cold against 19.5 in
// two groups.  Where x fits, staging it is faster (1536 x 6912, M = 8: 7.8
// against 10.3 us; on the 151936-row lm_head more than twice as fast): each
// workgroup reads x from L2 once instead of once per wavefront.
template <int M, int NBI, int NW, bool XG>
__global__ __launch_bounds__(NW * kWave) void int4_gemv_packed(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ wp,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int ntiles, int x_vec16) {
  using Geo = PackedGeom<NBI>;
  constexpr int DG = XG ? 2 : 4;                        // items in flight per lane
  constexpr int PPB = NBI == 4 ? 1 : NBI == 2 ? 2 : 4;  // MFMAs per scale block
  extern __shared__ uint4 xs[];  // [M][K/8] swizzled x slots, then [NW][64] partials
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g = lane >> 4;
  const int C = K >> 7;
  const int S8 = K >> 3;
  const int i0 = wave * C / NW;
  const int i1 = (wave + 1) * C / NW;
  const int G = (int)gridDim.x;
  const int mytiles = ((int)blockIdx.x < ntiles) ? (ntiles - (int)blockIdx.x + G - 1) / G : 0;
  const int total = mytiles * (i1 - i0);
  const uint32_t magic = vreg_const(0x64006400u);

  using SType = std::conditional_t<NBI == 4, uint2, uint32_t>;
  struct Item {
    uint4 w;
    SType s;
    uint32_t z;
    uint4 a[4];  // XG: the item's x operands, as loaded
  };
  struct Cursor {
    int tile, c;
  };
  auto advance = [&](Cursor& cu) {
    if (++cu.c == i1) {
      cu.c = i0;
      cu.tile += G;
    }
  };
  // Rows of x for the A operand: rows >= M repeat real rows (their outputs
  // are not stored).
  const int arow = n < M ? n : n % M;
  const uint16_t* xrow = x + (size_t)arow * (size_t)ldx + 8 * g;
  auto load = [&](Item& it, const Cursor& cu) {
    const uint8_t* rec = wp + ((size_t)cu.tile * (size_t)C + (size_t)cu.c) * Geo::kRecord;
    it.w = load_stream16(rec + 16 * lane);
    if constexpr (XG) {
#pragma unroll
      for (int t = 0; t < 4; ++t) it.a[t] = load16(xrow + (cu.c * 128 + 32 * t));
    }
    const uint8_t* sp = rec + 1024 + n * (2 * NBI);
    if constexpr (NBI == 4) it.s = *reinterpret_cast<const uint2*>(sp);
    else if constexpr (NBI == 2) it.s = *reinterpret_cast<const uint32_t*>(sp);
    else it.s = *reinterpret_cast<const uint16_t*>(sp);
    const uint8_t* zq = rec + 1024 + Geo::kScaleBytes + n * Geo::kZpRowBytes;
    it.z = NBI == 4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(zq) : (uint32_t)*zq;
  };

  // Stage x: slot gi of row m holds x[m, 8 gi .. 8 gi + 7] (pair order),
  // XOR-swizzled on the bits that select the MFMA within an item.
  Item ring[DG];
  Cursor lc = {(int)blockIdx.x, i0};
  auto fill_ring = [&] {
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      if (k < total) load(ring[k], lc);
      advance(lc);
    }
  };
  if constexpr (XG) {
    fill_ring();
  } else {
    // Each wavefront stages only the x slots of its own items [i0, i1) (16
    // slots of 8 halves per item and row of x), the same for every tile it
    // takes, and reads no others: no workgroup barrier precedes the first
    // item, and a wavefront waits for its own x only (measured against the
    // whole workgroup staging all of x: 1536 x 6912 at M = 8 7.8 -> 6.7 us,
    // M = 2 6.4 -> 5.5; 4096^2 M = 8 6.7 -> 6.1; 11008 x 4096 M = 8 10.0 ->
    // 9.1; the lm_head 1% faster).  Its first weight loads go out between
    // its x loads and their LDS stores.
    const int ns = 16 * (i1 - i0);
    bool pending = true;
    for (int r0 = 0; r0 < ns; r0 += kWave) {
      const int r = r0 + lane < ns ? r0 + lane : ns - 1;
      const int gi = 16 * i0 + r;
      uint4 v[M];
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] = load_x8(x + m * ldx + gi * 8, x_vec16);
      if (pending) {
        __builtin_amdgcn_sched_barrier(0);
        fill_ring();
        __builtin_amdgcn_sched_barrier(0);
        pending = false;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) xs[m * S8 + (gi ^ ((m & 3) << 2))] = pair_halves(v[m]);
    }
    // The wavefront's lanes read slots that other lanes of it wrote: keep
    // the reads behind the writes (LDS serves one wavefront in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  uint32_t aoff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    aoff[t] = (uint32_t)((arow * S8 + ((4 * t + g) ^ ((arow & 3) << 2))) * 16);
  const char* xs_bytes = reinterpret_cast<const char*>(xs);
  f32x4* red = reinterpret_cast<f32x4*>(xs + (XG ? 0 : M * S8));  // [NW][64]

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  auto consume = [&](const Item& it, const Cursor& cu) {
    const uint32_t ibase = (uint32_t)cu.c * 256u;  // 16 slots of 16 bytes per item
    uint4 av[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      av[t] = XG ? pair_halves(it.a[t])
                 : *reinterpret_cast<const uint4*>(xs_bytes + (aoff[t] + ibase));
    f32x4 d = zero4;
    uint32_t bias_lo = 0, bias_hi = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int bi = t / PPB;
      if (t % PPB == 0) {
        const uint32_t z = (it.z >> (4 * bi)) & 15u;
        bias_lo = 0xE400E400u + z * 0x00010001u;  // -(1024 + zp) in both halves
        bias_hi = 0xD400D400u + z * 0x00100010u;  // -(64 + zp) in both halves
      }
      const Pairs8 q = unpack8(word_of(it.w, t), magic, bias_lo, bias_hi);
      const f16x8 bop = {q.a.x, q.a.y, q.b.x, q.b.y, q.c.x, q.c.y, q.d.x, q.d.y};
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(av[t]), bop,
                                                 t % PPB == 0 ? zero4 : d, 0, 0, 0);
      if (t % PPB == PPB - 1) {
        uint32_t sbits;
        if constexpr (NBI == 4) sbits = ((bi < 2 ? it.s.x : it.s.y) >> (16 * (bi & 1))) & 0xFFFFu;
        else if constexpr (NBI == 2) sbits = (it.s >> (16 * bi)) & 0xFFFFu;
        else sbits = it.s & 0xFFFFu;
        const float sc = f16_to_f32(sbits);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, d[i], acc[i]);
      }
    }
    if (cu.c == i1 - 1) {
      // Tile finished: lane (n, g) holds rows 4g..4g+3 of column n of this
      // wavefront's share; add the shares in wavefront order.
      red[wave * kWave + lane] = acc;
      __syncthreads();
      if (wave == 0) {
        f32x4 sum = red[lane];
        auto add_share = [&](int v) {
          const f32x4 o = red[v * kWave + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[i] += o[i];
        };
        // 16 wavefronts with x in LDS (small matrices, one workgroup per CU):
        // a full unroll (measured faster, 1536 x 6912 at M = 8: 7.8 against
        // 8.1 us).  Otherwise a partial one: holding every wavefront's
        // partials at once raises the register count, so that fewer
        // workgroups stay resident (the lm_head at M = 4: 72.4 against 68.5
        // us) or, with x from global memory, registers spill.
        if constexpr (NW >= 16 && !XG) {
#pragma unroll
          for (int v = 1; v < NW; ++v) add_share(v);
        } else {
#pragma unroll 4
          for (int v = 1; v < NW; ++v) add_share(v);
        }
        const int col = cu.tile * 16 + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * g + i;
          if (m < M && col < N) store_out(y, m * ldy + col, sum[i], y_type);
        }
      }
      __syncthreads();
      acc = zero4;
    }
    // Keep the next item's A reads (and their registers) below this item.
    __builtin_amdgcn_sched_barrier(0);
  };

  Cursor pc = {(int)blockIdx.x, i0};
  int u = 0;
  // Steady state: every consumed slot is reloaded unconditionally; the last
  // items are finished below with the reload under a (wave-uniform) bound.
#pragma unroll 1
  for (; u + 2 * DG <= total; u += DG) {
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      consume(ring[k], pc);
      advance(pc);
      load(ring[k], lc);
      advance(lc);
    }
  }
#pragma unroll 1
  for (; u < total; u += DG) {
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      if (u + k < total) {
        consume(ring[k], pc);
        advance(pc);
        if (u + k + DG < total) load(ring[k], lc);
        advance(lc);
      }
    }
  }
}

template <int NBI>
hipError_t launch_repack_nbi(const uint8_t* w, const uint16_t* scales, const uint8_t* zp,
                             uint8_t* out, int N, int K, int block_size, hipStream_t stream) {
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int64_t nrec = (int64_t)((N + 15) / 16) * (K / 128);
  const int64_t threads = nrec * 64;
  const int grid = (int)((threads + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(int4_repack_kernel<NBI>, dim3(grid), dim3(kBlock), 0, stream, w, scales, zp,
                     out, N, K, bs_log2, zrow, nrec);
  note_launch(kPathInt4Repack, 0, grid, kBlock, 0);
  return hipGetLastError();
}

// Waves per workgroup: 8, or fewer when a row has fewer than 8 items (every
// wavefront must get at least one item of each tile); 16 when the matrix has
// fewer tiles than the GPU has CUs, so that each tile's CU keeps more of its
// bytes in flight.
constexpr bool kPackedWide = true;
constexpr int kPackedWideTiles = 256;
// When x is read from global memory (XG) instead of LDS: 0 never, 1 for rows
// of x that LDS cannot hold, 2 always (x 16-byte aligned rows in every case).
constexpr int kPackedXg = 1;

template <int M, int NBI, int NW, bool XG>
hipError_t launch_packed_nw(const uint16_t* x, int64_t ldx, const uint8_t* wp, void* y,
                            int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  const size_t shmem = (XG ? 0 : (size_t)M * K * 2) + (size_t)NW * kWave * 16;
  auto kern = int4_gemv_packed<M, NBI, NW, XG>;
  const hipError_t e = allow_lds(kern, shmem);
  if (e != hipSuccess) return e;
  const int ntiles = (N + 15) / 16;
  const int cap = resident_workgroups(kern, NW * kWave, shmem);
  const int grid = ntiles < cap ? ntiles : cap;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * kWave), shmem, stream, x, ldx, wp, y, ldy,
                     y_type, N, K, ntiles, x_vec16);
  note_launch(kPathInt4Packed, M, grid, NW * kWave, shmem);
  return hipGetLastError();
}

template <int M, int NBI, bool XG>
hipError_t launch_packed_m(const uint16_t* x, int64_t ldx, const uint8_t* wp, void* y,
                           int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  const int C = K / 128;
  const size_t xbytes = XG ? 0 : (size_t)M * K * 2;
  const int ntiles = (N + 15) / 16;
  if (kPackedWide && C >= 16 && ntiles < kPackedWideTiles &&
      xbytes + 16 * kWave * 16 <= (size_t)kLdsMax)
    return launch_packed_nw<M, NBI, 16, XG>(x, ldx, wp, y, ldy, y_type, N, K, stream);
  if (C >= 8) return launch_packed_nw<M, NBI, 8, XG>(x, ldx, wp, y, ldy, y_type, N, K, stream);
  if (C >= 4) return launch_packed_nw<M, NBI, 4, XG>(x, ldx, wp, y, ldy, y_type, N, K, stream);
  if (C >= 2) return launch_packed_nw<M, NBI, 2, XG>(x, ldx, wp, y, ldy, y_type, N, K, stream);
  return launch_packed_nw<M, NBI, 1, XG>(x, ldx, wp, y, ldy, y_type, N, K, stream);
}

template <int NBI>
hipError_t launch_packed_nbi(const uint16_t* x, int64_t ldx, const uint8_t* wp, void* y,
                             int64_t ldy, int y_type, int M, int N, int K, bool xg,
                             hipStream_t stream) {
  switch (M) {
#define QG_CASE(MM) \
  case MM:          \
    return xg ? launch_packed_m<MM, NBI, true>(x, ldx, wp, y, ldy, y_type, N, K, stream) \
              : launch_packed_m<MM, NBI, false>(x, ldx, wp, y, ldy, y_type, N, K, stream);
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t int4_packed_record_bytes(int block_size) {
  const int nbi = block_size >= 128 ? 1 : 128 / block_size;
  return nbi == 4 ? PackedGeom<4>::kRecord : nbi == 2 ? PackedGeom<2>::kRecord
                                                      : PackedGeom<1>::kRecord;
}

size_t int4_packed_max_rows_of_x(int K) {
  // x of all M rows plus the 8-wavefront partials within the LDS limit
  const size_t room = (size_t)kLdsMax - 8 * kWave * 16;
  return room / ((size_t)K * 2);
}

hipError_t launch_int4_repack(const uint8_t* w, const uint16_t* scales, const uint8_t* zp,
                              uint8_t* out, int N, int K, int block_size, hipStream_t stream) {
  if (block_size == 32) return launch_repack_nbi<4>(w, scales, zp, out, N, K, block_size, stream);
  if (block_size == 64) return launch_repack_nbi<2>(w, scales, zp, out, N, K, block_size, stream);
  return launch_repack_nbi<1>(w, scales, zp, out, N, K, block_size, stream);
}

hipError_t launch_int4_gemv_packed(const uint16_t* x, int64_t ldx, const uint8_t* wp, void* y,
                                   int64_t ldy, int y_type, int M, int N, int K, int block_size,
                                   hipStream_t stream) {
  // Rows of x beyond what LDS holds: x from global memory, or (x not 16-byte
  // aligned) groups of rows, each a launch that re-reads the weights.
  const int mfit = (int)int4_packed_max_rows_of_x(K);
  const bool x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const bool xg = x_vec16 && (kPackedXg == 2 || (kPackedXg == 1 && M > mfit));
  if (!xg && mfit < 1) return hipErrorInvalidValue;
  if (!xg && M > mfit) {
    for (int m0 = 0; m0 < M; m0 += mfit) {
      const int mm = M - m0 < mfit ? M - m0 : mfit;
      const size_t ysz = y_type == 2 ? 4 : 2;
      const hipError_t e = launch_int4_gemv_packed(
          x + m0 * ldx, ldx, wp, static_cast<char*>(y) + (size_t)m0 * ldy * ysz, ldy, y_type, mm,
          N, K, block_size, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (block_size == 32)
    return launch_packed_nbi<4>(x, ldx, wp, y, ldy, y_type, M, N, K, xg, stream);
  if (block_size == 64)
    return launch_packed_nbi<2>(x, ldx, wp, y, ldy, y_type, M, N, K, xg, stream);
  return launch_packed_nbi<1>(x, ldx, wp, y, ldy, y_type, M, N, K, xg, stream);
}

}  // namespace qg
