// int4_gemv.hip -- MatMulNBits-style blockwise int4 GEMV for gfx950, M = 1..8.
//
// Operation (onnx-genai pull request #1000, "Summary" and "What it does": the
// M = 1 int4 MatMulNBits decode GEMV with per-column fp32 accumulation):
//     y[m,n] = sum_k x[m,k] * s[n,k/bs] * (q[n,k] - zp[n,k/bs])
//
// Design (MI355X-first; the page's multicol NC=4 CUDA kernel is prior art only):
//  * The weight matrix is one contiguous byte stream ([N][K/2]).  A
//    workgroup (256 threads = 4 wavefronts) owns a tile of rows; inside it a
//    group of LPR consecutive lanes owns one row and walks that row's 16-byte
//    pieces (32 nibbles = 32 weights) with a stride of LPR pieces, so every
//    wavefront load instruction reads 64/LPR contiguous runs of LPR*16 bytes.
//    Each lane owns R rows at once so that every x value read from LDS is
//    used R times.
//  * x is staged in LDS (once per workgroup), pre-permuted within every group of
//    8 elements to (x0,x4 | x1,x5 | x2,x6 | x3,x7) so that it lines up with the
//    nibble pairs below.  Each 64-byte piece of x is followed by 16 bytes of
//    padding: the lanes of a row read pieces 80 bytes apart, which spreads
//    their 16-byte LDS reads over distinct banks.
//  * Unpack: OR-ing a nibble into the mantissa of fp16 1024.0 gives 1024+q
//    exactly; a nibble sitting 4 bits higher gives 1024+16q.  One packed fp16
//    add (or fma by 1/16) with -(1024+zp) (or -(64+zp)) then yields q-zp
//    exactly as a pair of fp16 values: 9 VALU ops per 8 weights.  The zero
//    point is subtracted per weight, so all-zero-point weights give y = 0
//    exactly.
//  * MAC: v_dot2_f32_f16 multiplies an exact (q-zp) pair by an x pair and
//    accumulates in fp32 (the products are exact).  The per-block fp16 scale
//    (exact in fp32) is applied once per 32-weight piece with one fp32 FMA, so
//    dequantized weights never leave registers and a one-hot x reproduces
//    s*(q-zp) bit-exactly.
//  * Reduction: the LPR lanes of a row reduce with cross-lane shuffles; no
//    atomics and no cross-workgroup split-K (the AstrAI commit list measured
//    split-K as a regression).
//  * At M = 1, rows of 2048, 4096 or 8192 weights (the lm_head and the
//    4096-wide layers) and the rows of matrices too short for the persistent
//    kernel (128 < K/32 <= 512) take the span kernel instead: each wavefront
//    streams whole runs of about 4 KB of consecutive rows, one contiguous 1 KB
//    access per load instruction, and reloads each piece's registers with the
//    next run as soon as they are consumed.
//  * M >= 2 takes the matrix cores (int4_gemv_mfma below), except a few
//    M = 2 shapes.
#include <type_traits>

#include "int4_device.h"
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qg {
namespace {

// Everything one lane loads for one 16-byte piece of R rows.
template <int R>
struct Piece {
  uint4 w[R];
  uint32_t s[R];  // fp16 scale bits
  uint32_t z[R];  // zero-point byte (both nibbles)
};

template <int M, int LPR, int R, bool ZP>
__global__ __launch_bounds__(kBlock) void int4_gemv_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zp, int zrow,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int bs_log2, int KC,
    int x_vec16) {
  extern __shared__ uint4 xs[];  // [M][KC/32][5]: 4 permuted groups of 8 halves + pad
  constexpr int S = kBlock / LPR;  // row slots per workgroup
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int j = tid % LPR;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int nb = K >> bs_log2;
  const int PS = (KC >> 5) * 5;  // uint4 slots per x row in LDS
  const uint32_t magic = vreg_const(0x64006400u);

  // Rows past the end are clamped to the last row for loading (no branches in
  // the stream); their results are never stored.  Offsets are 32-bit (the
  // host rejects tensors of 4 GiB or more), so every load is a uniform base
  // address plus one VGPR offset.
  int rows[R];
  uint32_t wo[R], so[R], zo[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    rows[i] = (tile * R + i) * S + slot;
    const uint32_t nl = (uint32_t)(rows[i] < N ? rows[i] : N - 1);
    wo[i] = nl * (uint32_t)(K >> 1);
    so[i] = nl * (uint32_t)nb;
    zo[i] = nl * (uint32_t)zrow;
  }

  auto load = [&](Piece<R>& st, int gp) {
    const uint32_t blk = (uint32_t)((gp << 5) >> bs_log2);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      st.w[i] = load_stream16(w + (wo[i] + (uint32_t)gp * 16u));
      st.s[i] = scales[so[i] + blk];
      st.z[i] = ZP ? zp[zo[i] + (blk >> 1)] : 0x88u;
    }
  };

  float acc[R][M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;

#pragma unroll 1
  for (int kc = 0; kc < K; kc += KC) {
    const int kn = min(KC, K - kc);
    const int P = kn >> 5;
    const int gp0 = kc >> 5;
    // The first piece's loads go out right behind the x loads: their latency
    // overlaps the staging and the barrier.
    Piece<R> cur;
    __syncthreads();
    const int groups = kn >> 3;
    stage_slots<4>(
        tid, kBlock, M * groups,
        [&](int t) {
          const int m = t / groups;
          return load_x8(x + m * ldx + kc + (t - m * groups) * 8, x_vec16);
        },
        [&](int t, uint4 v) {
          const int m = t / groups;
          const int gi = t - m * groups;
          xs[m * PS + (gi >> 2) * 5 + (gi & 3)] = pair_halves(v);
        },
        [&] {
          if (j < P) load(cur, gp0 + j);
        });
    __syncthreads();

#pragma unroll 1
    for (int p = j; p < P; p += LPR) {
      // Prefetch the next piece while this one is computed.
      Piece<R> nxt;
      const bool more = p + LPR < P;
      if (more) load(nxt, gp0 + p + LPR);

      const int gp = gp0 + p;
      const int zsh = (((gp << 5) >> bs_log2) & 1) << 2;
      float sc[R];
      uint32_t blo[R], bhi[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        sc[i] = f16_to_f32(cur.s[i]);
        const uint32_t z = (cur.z[i] >> zsh) & 15u;
        blo[i] = (0xE400u + z) * 0x00010001u;         // -(1024 + zp) in both halves
        bhi[i] = (0xD400u + (z << 4)) * 0x00010001u;  // -(64 + zp) in both halves
      }
      float part[R][M];
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) part[i][m] = 0.f;

      const uint4* xp = xs + p * 5;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = xp[m * PS + d];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const Pairs8 q = unpack8(word_of(cur.w[i], d), magic, blo[i], bhi[i]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float t = part[i][m];
            t = __builtin_amdgcn_fdot2(q.a, bitcast<f16x2>(xv[m].x), t, false);
            t = __builtin_amdgcn_fdot2(q.b, bitcast<f16x2>(xv[m].y), t, false);
            t = __builtin_amdgcn_fdot2(q.c, bitcast<f16x2>(xv[m].z), t, false);
            t = __builtin_amdgcn_fdot2(q.d, bitcast<f16x2>(xv[m].w), t, false);
            part[i][m] = t;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = __builtin_fmaf(sc[i], part[i][m], acc[i][m]);
      if (more) cur = nxt;
    }
  }

  __shared__ float red[(kBlock / kWave) * R * M];
  float tot[R * M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) tot[i * M + m] = acc[i][m];
  group_sum_wide<LPR, R * M>(tot, red);
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (j == 0 && rows[i] < N) store_out(y, m * ldy + rows[i], tot[i * M + m], y_type);
}

// Persistent variant, used whenever all of x fits in LDS: one resident round
// of workgroups, each staging x once and then streaming row tiles.  A lane's
// work is a flat sequence of (tile, item) pairs; an item is PB adjacent
// 16-byte pieces of each of the lane's R rows (PB = 2: 32 contiguous bytes,
// one zero-point byte for both 32-weight blocks).  A one-item register
// prefetch runs across tile boundaries; when a tile's last item is done its
// rows are reduced and stored.
template <int R, int PB>
struct Item {
  uint4 w[R][PB];
  uint32_t s[R][PB];  // fp16 scale bits per piece
  uint32_t z[R][PB];  // zero-point byte per piece
};

template <int M, int LPR, int R, int PB, bool ZP, bool STRIDED, int NT>
__global__ __launch_bounds__(NT) void int4_gemv_persistent(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zp, int zrow,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int bs_log2, int ntiles,
    int x_vec16) {
  extern __shared__ uint4 xs[];  // [M][K/32][5]: 4 permuted groups of 8 halves + pad
  constexpr int S = NT / LPR;  // row slots per workgroup
  constexpr int RT = S * R;        // rows per tile
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int j = tid % LPR;
  // Tile order: STRIDED walks tiles b, b+G, b+2G, ... so that the resident
  // workgroups sweep one compact window of the matrix together; otherwise
  // workgroup b takes a contiguous range of tiles.
  const int b = STRIDED ? (int)blockIdx.x : xcd_tile(blockIdx.x, gridDim.x);
  const int G = (int)gridDim.x;
  const int t_begin = STRIDED ? b : (int)((int64_t)b * ntiles / G);
  const int t_end = STRIDED ? ntiles : (int)((int64_t)(b + 1) * ntiles / G);
  const int t_step = STRIDED ? G : 1;
  const int my_tiles = STRIDED ? (ntiles - b + G - 1) / G : t_end - t_begin;
  const int nb = K >> bs_log2;
  const int P = K >> 5;                              // pieces per row
  const int PPI = (P + LPR * PB - 1) / (LPR * PB);   // items per lane per tile
  const int PS = P * 5;
  const uint32_t magic = vreg_const(0x64006400u);

  auto load = [&](Item<R, PB>& st, int tile, int it) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int row = tile * RT + i * S + slot;
      const uint32_t nl = (uint32_t)(row < N ? row : N - 1);
      const uint32_t wrow = nl * (uint32_t)(K >> 1);
      const uint32_t srow = nl * (uint32_t)nb;
      const uint32_t zr = nl * (uint32_t)zrow;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        int p = PB * (j + LPR * it) + q;
        p = p < P ? p : P - 1;  // idle lanes of a ragged last stride re-read a valid piece
        const uint32_t blk = (uint32_t)((p << 5) >> bs_log2);
        st.w[i][q] = load_stream16(w + (wrow + (uint32_t)p * 16u));
        st.s[i][q] = scales[srow + blk];
        st.z[i][q] = ZP ? zp[zr + (blk >> 1)] : 0x88u;
      }
    }
  };

  const int nitems = my_tiles * PPI;
  Item<R, PB> cur;
  const int groups = K >> 3;
  stage_slots<4>(
      tid, NT, M * groups,
      [&](int t) {
        const int m = t / groups;
        return load_x8(x + m * ldx + (t - m * groups) * 8, x_vec16);
      },
      [&](int t, uint4 v) {
        const int m = t / groups;
        const int gi = t - m * groups;
        xs[m * PS + (gi >> 2) * 5 + (gi & 3)] = pair_halves(v);
      },
      [&] { load(cur, t_begin, 0); });  // rows past the end are clamped
  __syncthreads();

  float acc[R][M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;

  int tile = t_begin, it = 0;
#pragma unroll 1
  for (int u = 0; u < nitems; ++u) {
    int ntile = tile, nit = it + 1;
    if (nit == PPI) {
      nit = 0;
      ntile += t_step;
    }
    Item<R, PB> nxt;
    const bool more = u + 1 < nitems;
    if (more) load(nxt, ntile, nit);

#pragma unroll
    for (int q = 0; q < PB; ++q) {
      const int p = PB * (j + LPR * it) + q;
      if (p < P) {
        const int zsh = (((p << 5) >> bs_log2) & 1) << 2;
        float sc[R];
        uint32_t blo[R], bhi[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          sc[i] = f16_to_f32(cur.s[i][q]);
          const uint32_t z = (cur.z[i][q] >> zsh) & 15u;
          blo[i] = 0xE400E400u + z * 0x00010001u;          // -(1024 + zp) in both halves
          bhi[i] = 0xD400D400u + z * 0x00100010u;          // -(64 + zp) in both halves
        }
        float part[R][M];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int m = 0; m < M; ++m) part[i][m] = 0.f;
        const uint4* xp = xs + p * 5;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint4 xv[M];
#pragma unroll
          for (int m = 0; m < M; ++m) xv[m] = xp[m * PS + d];
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const Pairs8 qq = unpack8(word_of(cur.w[i][q], d), magic, blo[i], bhi[i]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              float t = part[i][m];
              t = __builtin_amdgcn_fdot2(qq.a, bitcast<f16x2>(xv[m].x), t, false);
              t = __builtin_amdgcn_fdot2(qq.b, bitcast<f16x2>(xv[m].y), t, false);
              t = __builtin_amdgcn_fdot2(qq.c, bitcast<f16x2>(xv[m].z), t, false);
              t = __builtin_amdgcn_fdot2(qq.d, bitcast<f16x2>(xv[m].w), t, false);
              part[i][m] = t;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[i][m] = __builtin_fmaf(sc[i], part[i][m], acc[i][m]);
      }
    }

    if (it == PPI - 1) {  // tile finished (uniform across the workgroup)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int row = tile * RT + i * S + slot;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = group_sum<LPR>(acc[i][m]);
          acc[i][m] = 0.f;
          if (j == 0 && row < N) store_out(y, m * ldy + row, v, y_type);
        }
      }
    }
    if (more) cur = nxt;
    tile = ntile;
    it = nit;
  }
}

// Sums over the 64 lanes of a wavefront for NV = 1, 2 or 4 values at once.
// Lane swaps (v_permlane32_swap, v_permlane16_swap) fold the values into one
// register, value k ending in a quarter or half of the lanes, and four DPP
// steps finish each 16-lane row: the lane-row r (lane / 16) then holds the
// total of value span_value<NV>(r) in every lane.  No LDS round trip.
template <int NV>
__device__ __forceinline__ float span_reduce(const float (&v)[NV]) {
  static_assert(NV == 1 || NV == 2 || NV == 4, "values per reduction");
  float t;
  if constexpr (NV == 1) {
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[0]),
                                                    false, false);
    t = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t),
                                                    false, false);
    t = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  } else if constexpr (NV == 2) {
    // Lanes 0-31: value 0 (its two halves added); lanes 32-63: value 1.
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                    false, false);
    t = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t),
                                                    false, false);
    t = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  } else {
    const auto q01 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]),
                                                      __float_as_uint(v[1]), false, false);
    const auto q23 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2]),
                                                      __float_as_uint(v[3]), false, false);
    const float a = __uint_as_float(q01[0]) + __uint_as_float(q01[1]);  // rows 0,1: v0; 2,3: v1
    const float c = __uint_as_float(q23[0]) + __uint_as_float(q23[1]);  // rows 0,1: v2; 2,3: v3
    // Odd rows of a <-> even rows of c: rows 0..3 then hold v0, v2, v1, v3.
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(c),
                                                    false, false);
    t = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
  return group_sum<16>(t);
}

// Which value of span_reduce<NV> lane-row r (0..3) holds.
template <int NV>
__device__ __forceinline__ int span_value(int r) {
  if constexpr (NV == 1) return 0;
  else if constexpr (NV == 2) return r >> 1;
  else return ((r & 1) << 1) | (r >> 1);
}

// Span variant, M = 1, for rows of P = K/32 pieces of 32 weights.  Lane l
// takes pieces l + 64u (u < U) of a row, so each weight load of a lane is one
// contiguous 1 KB wavefront access.  Rows of exactly 64U pieces (K = 2048,
// 4096, 8192: U = 1, 2, 4) are cut into spans of R = 4/U consecutive rows,
// i.e. 4 KB of contiguous weight bytes.  RAGGED rows, 64(U-1) < P < 64U
// (U = 3..8), make spans of one row: in the last u the lanes past the row's
// end read its last piece and add it with scale 0.  Each wavefront streams
// whole spans (gw, gw + GW, ... for global wavefront gw of GW), which keeps
// runs of about 4 KB of HBM in flight per wavefront (measured: such runs
// stream about 9% faster than the same bytes read with a grid-wide stride).
// The span index is wave-uniform, so row offsets are scalar and each load is
// a scalar base plus a fixed per-lane offset.  PIPE picks how loads overlap
// the compute (below).  A span's R row sums are reduced together across the
// wavefront and stored by one lane each.  Unpack, zero point, scale and MAC
// are those of the kernels above; x is staged once per workgroup in LDS and
// each lane reads the same x slots for every span.
#ifdef QG_WAVE_TIMES
// Bench-only build (libqgemv_wavetimes.so, never the product library): the
// span kernel records, per wavefront, the 100 MHz real-time counter at its
// start, once x is staged and at its end, and the number of spans it
// streamed, for the last launch.
constexpr int kWaveTimesMax = 16384;
__device__ uint64_t wave_times[kWaveTimesMax * 4];

__device__ __forceinline__ void wave_times_record(int gw, uint64_t t0, uint64_t t1, int spans) {
  const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x % kWave == 0 && gw < kWaveTimesMax) {
    uint64_t* r = wave_times + 4 * (size_t)gw;
    r[0] = t0;
    r[1] = t1;
    r[2] = t2;
    r[3] = (uint64_t)spans;
  }
}
#endif

// How a span kernel keeps loads in flight while it computes.
enum SpanPipe : int {
  kSpanSerial = 0,  // load a span, then compute it (occupancy hides latency)
  kSpanDouble = 1,  // two register sets: the next span loads while one computes
  kSpanRing = 2,    // one register set: each piece is reloaded with the next
                    // span's piece as soon as it has been consumed
  kSpanRing2 = 3,   // two register sets used in turn, each piece reloaded with
                    // the piece of the span after next
};

template <int M, int R, int U, bool ZP, int PIPE, bool RAGGED>
__global__ __launch_bounds__(kBlock) void int4_gemv_span(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zp, int zrow,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int bs_log2, int nspans,
    int x_vec16) {
  static_assert(R * M == 1 || R * M == 2 || R * M == 4, "row sums per span");
  extern __shared__ uint4 xs[];  // [M][K/32][5]: 4 permuted groups of 8 halves + pad
  constexpr int NWV = kBlock / kWave;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int gw = (int)blockIdx.x * NWV + __builtin_amdgcn_readfirstlane(tid / kWave);
  const int GW = (int)gridDim.x * NWV;
#ifdef QG_WAVE_TIMES
  const uint64_t wt_start = __builtin_amdgcn_s_memrealtime();
#endif
  const int nb = K >> bs_log2;
  const int PS = (K >> 5) * 5;
  const uint32_t magic = vreg_const(0x64006400u);
  // Per-lane parts of the offsets (fixed for the whole kernel).
  // Rows of P = K/32 pieces with 64(U-1) < P <= 64U: in the last u, lanes
  // past the row's end read its last piece and add it with scale 0.
  const int P = K >> 5;
  int pc[U];
  uint32_t lblk[U], zoff[U], woff[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    pc[u] = !RAGGED || lane + kWave * u < P ? lane + kWave * u : P - 1;
    lblk[u] = ((uint32_t)pc[u] << 5) >> bs_log2;
    zoff[u] = lblk[u] >> 1;
    woff[u] = (uint32_t)pc[u] * 16u;
  }

  struct Span {
    uint4 w[R][U];
    uint32_t s[R][U];  // fp16 scale bits per piece
    uint32_t z[R][U];  // zero-point byte per piece
  };
  // Piece u of row i of span s.  Rows past the end are clamped to the last
  // row (their sums are not stored).
  auto load_piece = [&](Span& sp, int s, int i, int u) {
    const int row = s * R + i < N ? s * R + i : N - 1;  // wave-uniform
    // scalar row bases, 32-bit lane offsets: base + offset addressing
    const uint8_t* wr = w + (size_t)row * (size_t)(K >> 1);
    const uint16_t* sr = scales + (size_t)row * (size_t)nb;
    const uint8_t* zr = zp + (size_t)row * (size_t)zrow;
    sp.w[i][u] = load_stream16(wr + woff[u]);
    sp.s[i][u] = sr[lblk[u]];
    sp.z[i][u] = ZP ? zr[zoff[u]] : 0x88u;
  };
  auto load = [&](Span& sp, int s) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u) load_piece(sp, s, i, u);
  };

  const int groups = K >> 3;
  Span bufA, bufB;
  stage_slots<4>(
      tid, kBlock, M * groups,
      [&](int t) {
        const int m = t / groups;
        return load_x8(x + m * ldx + (t - m * groups) * 8, x_vec16);
      },
      [&](int t, uint4 v) {
        const int m = t / groups;
        const int gi = t - m * groups;
        xs[m * PS + (gi >> 2) * 5 + (gi & 3)] = pair_halves(v);
      },
      [&] { load(bufA, gw < nspans ? gw : nspans - 1); });
  __syncthreads();
#ifdef QG_WAVE_TIMES
  const uint64_t wt_x = __builtin_amdgcn_s_memrealtime();
#endif

  // Computes span s from `cur`; after the pieces u of every row have been
  // consumed, `done(u)` runs (the ring reloads them there).
  auto compute = [&](Span& cur, int s, auto done) {
    float acc[R * M];
#pragma unroll
    for (int k = 0; k < R * M; ++k) acc[k] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = pc[u];
      const bool live = !RAGGED || u < U - 1 || lane + kWave * u < P;
      const int zsh = (int)(lblk[u] & 1) << 2;
      float sc[R];
      uint32_t blo[R], bhi[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        sc[i] = live ? f16_to_f32(cur.s[i][u]) : 0.f;
        const uint32_t z = (cur.z[i][u] >> zsh) & 15u;
        blo[i] = 0xE400E400u + z * 0x00010001u;  // -(1024 + zp) in both halves
        bhi[i] = 0xD400D400u + z * 0x00100010u;  // -(64 + zp) in both halves
      }
      float part[R][M];
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m) part[i][m] = 0.f;
      const uint4* xp = xs + p * 5;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint4 xv[M];
#pragma unroll
        for (int m = 0; m < M; ++m) xv[m] = xp[m * PS + d];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const Pairs8 q = unpack8(word_of(cur.w[i][u], d), magic, blo[i], bhi[i]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float t = part[i][m];
            t = __builtin_amdgcn_fdot2(q.a, bitcast<f16x2>(xv[m].x), t, false);
            t = __builtin_amdgcn_fdot2(q.b, bitcast<f16x2>(xv[m].y), t, false);
            t = __builtin_amdgcn_fdot2(q.c, bitcast<f16x2>(xv[m].z), t, false);
            t = __builtin_amdgcn_fdot2(q.d, bitcast<f16x2>(xv[m].w), t, false);
            part[i][m] = t;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
          acc[i * M + m] = __builtin_fmaf(sc[i], part[i][m], acc[i * M + m]);
      done(u);
    }
    const float tot = span_reduce<R * M>(acc);
    if ((lane & 15) == 0 && (R * M == 4 || (lane & 31) == 0) && (R * M > 1 || lane == 0)) {
      const int k = span_value<R * M>(lane >> 4);  // value index i * M + m
      const int row = s * R + k / M;
      if (row < N) store_out(y, (k % M) * ldy + row, tot, y_type);
    }
  };
  auto nothing = [](int) {};

  if constexpr (PIPE == kSpanDouble) {
    // bufA holds span s; the loop alternates the two register sets.
#pragma unroll 1
    for (int s = gw; s < nspans;) {
      if (s + GW < nspans) load(bufB, s + GW);
      compute(bufA, s, nothing);
      s += GW;
      if (s >= nspans) break;
      if (s + GW < nspans) load(bufA, s + GW);
      compute(bufB, s, nothing);
      s += GW;
    }
  } else if constexpr (PIPE == kSpanRing) {
    // Every span but the wave's last reloads its registers (the last is
    // peeled off so that no reload is conditional).
    int s = gw;
#pragma unroll 1
    for (; s + GW < nspans; s += GW) {
      compute(bufA, s, [&](int u) {
#pragma unroll
        for (int i = 0; i < R; ++i) load_piece(bufA, s + GW, i, u);
        // Keep the reloads behind the last use of the registers they fill.
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    if (s < nspans) compute(bufA, s, nothing);
  } else if constexpr (PIPE == kSpanRing2) {
    // bufA holds span s, bufB span s + GW; every consumed piece is reloaded
    // with the same piece of the span two steps on (unconditionally while
    // three more spans follow, then under a wave-uniform bound).
    if (gw + GW < nspans) load(bufB, gw + GW);
    int s = gw;
#pragma unroll 1
    for (; s + 3 * GW < nspans; s += 2 * GW) {
      compute(bufA, s, [&](int u) {
#pragma unroll
        for (int i = 0; i < R; ++i) load_piece(bufA, s + 2 * GW, i, u);
        __builtin_amdgcn_sched_barrier(0);
      });
      compute(bufB, s + GW, [&](int u) {
#pragma unroll
        for (int i = 0; i < R; ++i) load_piece(bufB, s + 3 * GW, i, u);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    if (s < nspans) {
      const bool third = s + 2 * GW < nspans;
      compute(bufA, s, [&](int u) {
        if (third) {
#pragma unroll
          for (int i = 0; i < R; ++i) load_piece(bufA, s + 2 * GW, i, u);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      if (s + GW < nspans) compute(bufB, s + GW, nothing);
      if (third) compute(bufA, s + 2 * GW, nothing);
    }
  } else {
#pragma unroll 1
    for (int s = gw; s < nspans; s += GW) {
      if (s != gw) load(bufA, s);
      compute(bufA, s, nothing);
    }
  }
#ifdef QG_WAVE_TIMES
  wave_times_record(gw, wt_start, wt_x, gw < nspans ? (nspans - gw + GW - 1) / GW : 0);
#endif
}

// Matrix-core variant for M >= 2 (where the v_dot2 path turns VALU-bound;
// the launcher keeps some M = 2 shapes on v_dot2, where it measured faster):
// v_mfma_f32_16x16x32_f16 with x as the A operand and 16 weight rows as the B
// operand, so one MFMA contracts 32 k for 16 rows.  A rows M..15 repeat real
// rows (their D rows are never stored), so every A read is unconditional.
// Work is cut into items: 4 consecutive 32-weight pieces (128 weights) of a
// 16-row tile; lane l (n = l % 16, g = l / 16) holds 16 bytes = piece 4c+g of
// row n of item c.  (q - zp) enters the MFMA exactly as fp16, as in the
// v_dot2 path, and the fp32 MFMA result is scaled once per scale block (the
// fp16 scale is exact in fp32).
//  * PPB (pieces per scale block) = 4 (block >= 128): the item shares one
//    scale and zero point, so its 4 MFMAs chain their accumulator and need
//    no data exchange: MFMA t pairs k-group g with word t of every lane's own
//    16 bytes, i.e. k = (4c+g)*32 + 8t + e.
//  * PPB = 1 or 2: a 4x4 transpose across the lane groups (two
//    v_permlane32_swap, two v_permlane16_swap) leaves lane (n, g) holding
//    8-weight group g of pieces 4c..4c+3, so MFMA t covers exactly piece 4c+t.
// Memory: items travel in groups of 4.  Per group a lane issues its 4 weight
// loads back to back (256 contiguous bytes per row across the row's lanes)
// and one load each of the scales and zero points of item g of the group;
// three swaps then give every lane those of all 4 items.  (Per-item scale
// loads touch 16 rows for a few bytes each and cost more than the weights.)
// DG groups are in flight per lane (a register ring; each slot is refilled as
// soon as it is consumed, unconditionally: past the last item the row and item
// indices are clamped, so surplus loads re-read cached bytes).
// x is staged in LDS in natural order (16-byte slots of 8 halves,
// pre-permuted like the nibble pairs; with SPLIT each wave stages the slots
// of its own items, otherwise the workgroup stages all); each row's slots are XOR-
// swizzled by (row & 3) on the slot bits that the 4 lanes of a row vary, so
// the A reads of rows 0..3 fall in distinct banks.  SPLIT: all NW waves of a
// workgroup share one tile and split its items; the partial sums are added in
// LDS in wave order (deterministic).  Otherwise each wave owns whole tiles.
// PHASED (with SPLIT, one tile per workgroup): x is staged in chunks of `cp`
// items when all of it does not fit in LDS; the waves split each chunk's
// items, keep their accumulators across chunks, and the workgroup restages x
// between chunks.
// D needs no cross-lane reduction: lane (n, g) ends with rows 4g..4g+3 of
// column n.
// KS (k parts, with SPLIT and x wholly staged; M <= 16 / KS): A rows M..15
// would idle, so the 16 MFMA columns carry TR = 16 / KS weight rows in KS
// parts of their k range instead of 16 rows: column n is tile row n % TR,
// part h = n / TR, and A row r holds x row r % TR (repeated past M) of part
// r / TR.  A step s of a tile covers items KS * s + h of its rows (the host
// takes KS only where it divides the row's item count), and D[r][n] is a
// partial sum of output (r % TR, n % TR) exactly where r / TR = h; the other
// entries are computed and never read.  A short matrix then spreads over KS
// times as many workgroups (1536 rows: 96 tiles of 16 rows, 192 of 8 rows),
// with no data shared between workgroups; the tile-end sum adds the KS parts
// after the waves, in a fixed order.
// x slots each thread loads before it stores them (matrix-core kernel;
// measured on the 4096-row 7B layers: 12 and 16 are slower).
constexpr int kMfmaStageUnroll = 4;

template <int M, bool ZP, int PPB, bool SPLIT, int NW, int DG, bool PHASED = false, int KS = 1>
__global__ __launch_bounds__(NW * kWave) void int4_gemv_mfma(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zp, int zrow,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int bs_log2, int ntiles,
    int x_vec16, int cp) {
  static_assert(!PHASED || SPLIT, "chunks of x are staged per tile: split mode only");
  static_assert(PPB == 1 || PPB == 2 || PPB == 4, "pieces per scale block");
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && SPLIT && !PHASED && M <= 16 / KS),
                "k parts: split tiles with x wholly staged, M rows per part");
  constexpr int TR = 16 / KS;  // weight rows per tile
  extern __shared__ uint4 xs[];  // [M][CP*16] slots, swizzled; then the SPLIT partials
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g = lane >> 4;
  const int ti = n % TR, h = n / TR;  // tile row and k part of column n
  const int nb = K >> bs_log2;
  const int C = K >> 7;                                // items per row
  const int CS = C / KS;                               // steps per tile
  const int CP = PHASED ? cp : CS;                     // steps per staged chunk of x
  const int nph = PHASED ? (CS + CP - 1) / CP : 1;     // chunks
  const int S8 = (CP * KS) << 4;                       // 16-byte slots per staged x row
  // This wave's stream of tiles (t0, t0 + TS, ...) and its step range
  // [item_begin(p), item_end(p)) in chunk p of each tile (with KS = 1 a step
  // is an item).
  const int t0 = SPLIT ? (int)blockIdx.x : (int)blockIdx.x * NW + wave;
  const int TS = SPLIT ? (int)gridDim.x : (int)gridDim.x * NW;
  auto item_begin = [&](int p) {
    const int base = p * CP, len = (CS - base < CP ? CS - base : CP);
    return SPLIT ? base + wave * len / NW : base;
  };
  auto item_end = [&](int p) {
    const int base = p * CP, len = (CS - base < CP ? CS - base : CP);
    return SPLIT ? base + (wave + 1) * len / NW : base + len;
  };
  const int my_tiles = t0 < ntiles ? (ntiles - t0 + TS - 1) / TS : 0;
  int groups_per_tile = 0;
  for (int p = 0; p < nph; ++p) groups_per_tile += (item_end(p) - item_begin(p) + 3) >> 2;
  const int ngroups = my_tiles * groups_per_tile;
  const uint32_t magic = vreg_const(0x64006400u);
  // Slot swizzle of x row n: PPB = 4 reads slots 16c + 4g + t, the others
  // 16c + 4t + g; the swizzle flips the bits that t selects.
  constexpr int kSwzShift = PPB == 4 ? 0 : 2;

  // Scale bytes of one item: 8 (PPB 1: four blocks), 4 (two) or 2 (one).
  using SType = std::conditional_t<PPB == 1, uint2, uint32_t>;
  struct Group {
    uint4 w[4];  // step j: piece 4(KS(gc+j)+h)+g of tile row ti
    SType s;     // scales of step gc+g
    uint32_t z;  // zero-point bytes of step gc+g (PPB 1: 2 bytes, else 1)
  };
  // Position in the stream: tile, chunk, first item of the group, end of the
  // wave's items in that chunk.
  struct Cursor {
    int tile, p, gc, e;
  };
  const char* sbytes = reinterpret_cast<const char*>(scales);
  auto issue = [&](Group& gr, const Cursor& cu) {
    const int gc = cu.gc, ce = cu.e;
    const int row = cu.tile * TR + ti;
    const uint32_t nl = (uint32_t)(row < N ? row : N - 1);
    const uint32_t wrow = nl * (uint32_t)(K >> 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = KS * (gc + j < ce ? gc + j : ce - 1) + h;
      gr.w[j] = load16(w + (wrow + (uint32_t)(4 * c + g) * 16u));
    }
    const int cg = KS * (gc + g < ce ? gc + g : ce - 1) + h;
    const uint32_t blk0 = (uint32_t)((cg << 7) >> bs_log2);  // first block of item cg
    const char* sp = sbytes + (nl * (uint32_t)nb + blk0) * 2u;
    if constexpr (PPB == 1) gr.s = *reinterpret_cast<const uint2*>(sp);
    else if constexpr (PPB == 2) gr.s = *reinterpret_cast<const uint32_t*>(sp);
    else gr.s = *reinterpret_cast<const uint16_t*>(sp);
    if constexpr (ZP) {
      const uint8_t* zq = zp + (nl * (uint32_t)zrow + (blk0 >> 1));
      gr.z = PPB == 1 ? (uint32_t)*reinterpret_cast<const uint16_t*>(zq) : (uint32_t)*zq;
    } else {
      gr.z = 0x8888u;
    }
  };
  auto advance = [&](Cursor& cu) {
    cu.gc += 4;
    if (cu.gc >= cu.e) {
      if (++cu.p == nph) {
        cu.p = 0;
        cu.tile += TS;
      }
      cu.gc = item_begin(cu.p);
      cu.e = item_end(cu.p);
    }
  };

  // Chunk p of x: L8 slots of each row, from slot p * CP * 16 of the row.
  auto stage_load = [&](int p, int L8, int t) {
    const int m = t / L8;
    return load_x8(x + m * ldx + (p * S8 + (t - m * L8)) * 8, x_vec16);
  };
  auto stage_store = [&](int L8, int t, uint4 v) {
    const int m = t / L8;
    const int gi = t - m * L8;
    xs[m * S8 + (gi ^ ((m & 3) << kSwzShift))] = pair_halves(v);
  };
  auto chunk_slots = [&](int p) { return (CS - p * CP < CP ? CS - p * CP : CP) << 4; };

  Group ring[DG];
  Cursor lc = {t0, 0, item_begin(0), item_end(0)};  // next group to load
  auto fill_ring = [&] {  // unconditional: rows past the end are clamped
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      issue(ring[k], lc);
      advance(lc);
    }
  };
  if constexpr (SPLIT && !PHASED) {
    // Each wavefront stages only the x slots of its own items (16 per item
    // and row of x), the same for every tile it takes, and reads no others:
    // no workgroup barrier precedes the first item and a wavefront waits for
    // its own x only (measured against the whole workgroup staging all of x:
    // 1536 x 6912 M = 8 9.0 -> 7.7 us, M = 4 7.6 -> 6.9; 4096^2 M = 8 7.2 ->
    // 6.2; 11008 x 4096 M = 8 10.5 -> 9.2; bitwise the same results).
    const int ib = KS * item_begin(0), ns = 16 * KS * (item_end(0) - item_begin(0));
    bool pending = true;
    for (int r0 = 0; r0 < ns; r0 += kWave) {
      const int r = r0 + lane < ns ? r0 + lane : ns - 1;
      const int gi = 16 * ib + r;
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
      for (int m = 0; m < M; ++m) xs[m * S8 + (gi ^ ((m & 3) << kSwzShift))] = pair_halves(v[m]);
    }
    // The wavefront's lanes read slots that other lanes of it wrote: keep
    // the reads behind the writes (LDS serves one wavefront in order).
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  } else {
    const int L8 = chunk_slots(0);
    stage_slots<kMfmaStageUnroll>(
        tid, NW * kWave, M * L8, [&](int t) { return stage_load(0, L8, t); },
        [&](int t, uint4 v) { stage_store(L8, t, v); }, fill_ring);
    __syncthreads();
  }

  // LDS byte address of the A slot that MFMA t of step 0 reads: A row n is
  // x row n % TR (rows >= M read row (n % TR) % M) at item h.
  uint32_t aoff[4];
  const int arow = ti < M ? ti : ti % M;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int slot = PPB == 4 ? 4 * g + t : 4 * t + g;
    aoff[t] = (uint32_t)((arow * S8 + 16 * h + (slot ^ ((arow & 3) << kSwzShift))) * 16);
  }
  const char* xs_bytes = reinterpret_cast<const char*>(xs);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // out[j] = v of lane (n, j): the 32-lane swap pairs lane groups (0,2) and
  // (1,3), the 16-lane swaps then pair neighbouring groups.
  auto gather4 = [](uint32_t v, uint32_t (&out)[4]) {
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // v(g&1), v(g&1 | 2)
    const auto e01 = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto e23 = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    out[0] = e01[0]; out[1] = e01[1]; out[2] = e23[0]; out[3] = e23[1];
  };

  auto consume = [&](const Group& gr, const Cursor& cu) {
    const int tile = cu.tile, gc = cu.gc, ce = cu.e;
    // Scales and zero points of items gc..gc+3, in every lane.
    uint32_t s_lo[4], s_hi[4], zb[4];
    if constexpr (PPB == 1) {
      gather4(gr.s.x, s_lo);
      gather4(gr.s.y, s_hi);
    } else {
      gather4(gr.s, s_lo);
    }
    if constexpr (ZP) gather4(gr.z, zb);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = gc + j;
      if (c >= ce) break;  // partial last group of a tile (uniform)
      const uint32_t ibase = (uint32_t)(KS * (c - cu.p * CP)) * 256u;
      uint4 av[4];  // A operands of the item's 4 MFMAs
#pragma unroll
      for (int t = 0; t < 4; ++t)
        av[t] = *reinterpret_cast<const uint4*>(xs_bytes + (aoff[t] + ibase));
      uint32_t words[4];
      if constexpr (PPB == 4) {
        words[0] = gr.w[j].x; words[1] = gr.w[j].y; words[2] = gr.w[j].z; words[3] = gr.w[j].w;
      } else {
        // The swaps overwrite their operands: copy the ring slot out first so
        // that its registers stay free for the refill load.
        uint32_t d0 = vreg_copy(gr.w[j].x), d1 = vreg_copy(gr.w[j].y),
                 d2 = vreg_copy(gr.w[j].z), d3 = vreg_copy(gr.w[j].w);
        // 4x4 transpose (lane group g <-> register t): afterwards word t
        // holds 8-weight group g of piece 4c+t.
        const auto r02 = __builtin_amdgcn_permlane32_swap(d0, d2, false, false);
        const auto r13 = __builtin_amdgcn_permlane32_swap(d1, d3, false, false);
        d0 = r02[0]; d2 = r02[1]; d1 = r13[0]; d3 = r13[1];
        const auto r01 = __builtin_amdgcn_permlane16_swap(d0, d1, false, false);
        const auto r23 = __builtin_amdgcn_permlane16_swap(d2, d3, false, false);
        words[0] = r01[0]; words[1] = r01[1]; words[2] = r23[0]; words[3] = r23[1];
      }
      // Zero-point nibble and fp16 scale bits of block b of item c.
      auto zero_point = [&](int b) -> uint32_t {
        if constexpr (!ZP) {
          return 8u;
        } else if constexpr (PPB == 4) {
          const uint32_t blk0 = (uint32_t)(((KS * c + h) << 7) >> bs_log2);
          return (zb[j] >> ((blk0 & 1u) << 2)) & 15u;
        } else {
          return (zb[j] >> (4 * b)) & 15u;
        }
      };
      auto scale_bits = [&](int b) -> uint32_t {
        if constexpr (PPB == 1) return ((b < 2 ? s_lo[j] : s_hi[j]) >> (16 * (b & 1))) & 0xFFFFu;
        else if constexpr (PPB == 2) return (s_lo[j] >> (16 * b)) & 0xFFFFu;
        else return s_lo[j] & 0xFFFFu;
      };
      f32x4 d = zero4;
      uint32_t bias_lo = 0, bias_hi = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t % PPB == 0) {
          const uint32_t z = zero_point(t / PPB);
          bias_lo = 0xE400E400u + z * 0x00010001u;
          bias_hi = 0xD400D400u + z * 0x00100010u;
        }
        const Pairs8 q = unpack8(words[t], magic, bias_lo, bias_hi);
        const f16x8 b = {q.a.x, q.a.y, q.b.x, q.b.y, q.c.x, q.c.y, q.d.x, q.d.y};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(av[t]), b,
                                                   t % PPB == 0 ? zero4 : d, 0, 0, 0);
        if (t % PPB == PPB - 1) {
          const float sc = f16_to_f32(scale_bits(t / PPB));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, d[i], acc[i]);
        }
      }
      if (PHASED && c == ce - 1 && cu.p < nph - 1) {
        // Chunk finished: once every wave is done with it, stage the next.
        __syncthreads();
        const int L8 = chunk_slots(cu.p + 1);
        stage_slots<kMfmaStageUnroll>(
            tid, NW * kWave, M * L8, [&](int t) { return stage_load(cu.p + 1, L8, t); },
            [&](int t, uint4 v) { stage_store(L8, t, v); });
        __syncthreads();
      } else if (c == ce - 1) {  // tile finished: lane (n, g) holds rows 4g..4g+3 of column n
        const int row = tile * TR + ti;
        if constexpr (SPLIT) {
          f32x4* red = reinterpret_cast<f32x4*>(xs + M * S8);  // [NW][64]
          red[wave * kWave + lane] = acc;
          __syncthreads();
          // Part 0's lanes (n < TR, rows 4g.. < TR) add each part's sum over
          // the waves, parts in order; part h of the same outputs sits in
          // lane (n + h * TR, g + h * TR / 4).
          if (wave == 0 && (KS == 1 || (h == 0 && 4 * g < TR))) {
            auto part_sum = [&](int src) {
              f32x4 ps = red[src];
#pragma unroll
              for (int v = 1; v < NW; ++v) {
                const f32x4 o = red[v * kWave + src];
#pragma unroll
                for (int i = 0; i < 4; ++i) ps[i] += o[i];
              }
              return ps;
            };
            f32x4 sum = part_sum(lane);
            // a loop, so that one part's reads are in registers at a time
            // (with two parts the compiler peels its one pass, which holds
            // both parts' reads: 106 instead of 68 VGPRs, and measured
            // faster than a loop it cannot peel, 1536 x 6912 at M = 8: 6.2
            // against 6.5 us)
#pragma unroll 1
            for (int hp = 1; hp < KS; ++hp) {
              const f32x4 ps = part_sum(lane + hp * (TR + 16 * (TR / 4)));
#pragma unroll
              for (int i = 0; i < 4; ++i) sum[i] += ps[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = 4 * g + i;
              if (m < M && row < N) store_out(y, m * ldy + row, sum[i], y_type);
            }
          }
          __syncthreads();
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = 4 * g + i;
            if (m < M && row < N) store_out(y, m * ldy + row, acc[i], y_type);
          }
        }
        acc = zero4;
      }
      // Keep the scheduler from hoisting the next item's A reads (and their
      // 16 registers) above this item.
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  Cursor pc = {t0, 0, item_begin(0), item_end(0)};  // next group to consume
  int u = 0;
#pragma unroll 1
  for (; u + DG <= ngroups; u += DG) {
#pragma unroll
    for (int k = 0; k < DG; ++k) {
      consume(ring[k], pc);
      advance(pc);
      issue(ring[k], lc);
      advance(lc);
    }
  }
#pragma unroll
  for (int k = 0; k < DG; ++k) {
    if (u + k < ngroups) {
      consume(ring[k], pc);
      advance(pc);
    }
  }
}

// Measured on the 151936 x 4096 lm_head shape: a grid-stride tile order over a
// full resident grid beats contiguous per-workgroup ranges and beats an
// equal-share (smaller) grid.
constexpr bool kStrided = true;
constexpr bool kBalanced = false;

// Threads per workgroup of the persistent kernel at M = 1: 512 for long rows,
// where staging x once per workgroup costs as much as a tile of weights
// (measured: 4096 x 11008 and 4096 x 14336 gain a third; the 4096-wide
// lm_head and 11008 x 4096 lose a few percent at 512), else 256.
constexpr int kLongRowK = 8192;

template <int M, int LPR, int R, int PB, int NT>
hipError_t launch_persistent(const uint16_t* x, int64_t ldx, const uint8_t* w,
                             const uint16_t* scales, const uint8_t* zp, void* y, int64_t ldy,
                             int y_type, int N, int K, int block_size, size_t shmem,
                             hipStream_t stream) {
  constexpr int RT = (NT / LPR) * R;
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int ntiles = (N + RT - 1) / RT;
  auto kern = zp ? int4_gemv_persistent<M, LPR, R, PB, true, kStrided, NT>
                 : int4_gemv_persistent<M, LPR, R, PB, false, kStrided, NT>;
  const int cap = resident_workgroups(kern, NT, shmem);
  // Equal tile counts per workgroup: the fewest rounds that fit, then the
  // smallest grid that still covers every tile in that many rounds.
  const int rounds = (ntiles + cap - 1) / cap;
  const int grid = kBalanced ? (ntiles + rounds - 1) / rounds : (ntiles < cap ? ntiles : cap);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), shmem, stream, x, ldx, w, scales, zp, zrow, y,
                     ldy, y_type, N, K, bs_log2, ntiles, x_vec16);
  note_launch(kPathInt4Dot2Persistent, M, grid, NT, shmem);
  return hipGetLastError();
}

// Largest M that takes the span kernel (rows of 2048, 4096 or 8192 weights),
// and how it overlaps loads with compute.
constexpr int kSpanMaxM = 1;
constexpr int kSpanPipe = kSpanRing;
// Pieces per lane and span (rows per span x pieces per row and lane).
constexpr int kSpanRows = 4;

// Span kernel launch: two resident rounds of workgroups (or fewer when the
// spans run out first).  Wavefronts of the workgroups dispatched first on a
// CU run ahead of the later ones (per-wave timestamps of the lm_head: with
// one round the first wavefronts end after 22 us, the last after 57); with
// two rounds the second round's workgroups take the CU slots of the ones that
// end early, which measured 1% faster on the lm_head (55.9 -> 55.3 us); four
// rounds 56.1 us, one span per wavefront (16 rounds) 65 us.
constexpr int kSpanRounds = 2;

template <int M, int R, int U, bool RAGGED>
hipError_t launch_span(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                       const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                       int block_size, hipStream_t stream) {
  const size_t shmem = (size_t)M * (K / 32) * 80;
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int nspans = (N + R - 1) / R;
  auto kern = zp ? int4_gemv_span<M, R, U, true, kSpanPipe, RAGGED>
                 : int4_gemv_span<M, R, U, false, kSpanPipe, RAGGED>;
  const int cap = resident_workgroups(kern, kBlock, shmem);
  const int want = (nspans + kBlock / kWave - 1) / (kBlock / kWave);
  const int grid = want < cap * kSpanRounds ? want : cap * kSpanRounds;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), shmem, stream, x, ldx, w, scales, zp, zrow, y,
                     ldy, y_type, N, K, bs_log2, nspans, x_vec16);
  note_launch(kPathInt4Span, M, grid, kBlock, shmem);
  return hipGetLastError();
}

template <int M, int LPR, int R, int PB = 1>
hipError_t launch_cfg(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                      const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                      int block_size, hipStream_t stream) {
  // x takes 80 bytes of LDS per 32 elements and row.
  const size_t full = (size_t)M * (K / 32) * 80;
  if constexpr (LPR <= kWave) {
    if (full <= (size_t)kLdsBudget) {
      if constexpr (M == 1) {
        if (K >= kLongRowK)
          return launch_persistent<M, LPR, R, PB, 512>(x, ldx, w, scales, zp, y, ldy, y_type, N,
                                                      K, block_size, full, stream);
      }
      return launch_persistent<M, LPR, R, PB, kBlock>(x, ldx, w, scales, zp, y, ldy, y_type, N,
                                                      K, block_size, full, stream);
    }
  }
  constexpr int RT = (kBlock / LPR) * R;
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int ntiles = (N + RT - 1) / RT;
  const int grid = ntiles;
  int KC = (kLdsXBudget / (80 * M)) * 32;
  if (KC > K) KC = K;
  const size_t shmem = (size_t)M * (KC / 32) * 80;
  if (zp)
    hipLaunchKernelGGL((int4_gemv_kernel<M, LPR, R, true>), dim3(grid), dim3(kBlock), shmem,
                       stream, x, ldx, w, scales, zp, zrow, y, ldy, y_type, N, K, bs_log2, KC,
                       x_vec16);
  else
    hipLaunchKernelGGL((int4_gemv_kernel<M, LPR, R, false>), dim3(grid), dim3(kBlock), shmem,
                       stream, x, ldx, w, scales, zp, zrow, y, ldy, y_type, N, K, bs_log2, KC,
                       x_vec16);
  note_launch(kPathInt4Dot2Tiled, M, grid, kBlock, shmem);
  return hipGetLastError();
}

// Smallest M that takes the matrix-core kernel.
constexpr int kMfmaMinM = 2;


// Matrix-core launch shape: waves per workgroup and register groups (of 4
// items) in flight per lane.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaDepth = 1;
// The same for the split kernel (the waves of a workgroup share each tile;
// measured on the 4096-row 7B layers: 16 waves, or 2 to 4 groups in flight,
// are slower).
constexpr int kSplitWaves = 8;
constexpr int kSplitDepth = 1;

template <int M, int PPB, bool SPLIT, bool PHASED = false, int KS = 1, int NWS = kSplitWaves>
hipError_t launch_mfma_cfg(const uint16_t* x, int64_t ldx, const uint8_t* w,
                           const uint16_t* scales, const uint8_t* zp, void* y, int64_t ldy,
                           int y_type, int N, int K, int block_size, size_t shmem, int cp,
                           hipStream_t stream) {
  constexpr int NW = SPLIT ? NWS : kMfmaWaves;
  constexpr int DG = SPLIT ? kSplitDepth : kMfmaDepth;
  constexpr int TR = 16 / KS;
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int ntiles = (N + TR - 1) / TR;
  auto kern = zp ? int4_gemv_mfma<M, true, PPB, SPLIT, NW, DG, PHASED, KS>
                 : int4_gemv_mfma<M, false, PPB, SPLIT, NW, DG, PHASED, KS>;
  const hipError_t e = allow_lds(kern, shmem);
  if (e != hipSuccess) return e;
  // Phased: one tile per workgroup (the chunks of x are staged per tile).
  const int cap = PHASED ? ntiles : resident_workgroups(kern, NW * kWave, shmem);
  const int want = SPLIT ? ntiles : (ntiles + NW - 1) / NW;
  const int grid = want < cap ? want : cap;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * kWave), shmem, stream, x, ldx, w, scales, zp,
                     zrow, y, ldy, y_type, N, K, bs_log2, ntiles, x_vec16, cp);
  note_launch(PHASED ? kPathInt4MfmaPhased : SPLIT ? kPathInt4MfmaSplit : kPathInt4MfmaTiles, M,
              grid, NW * kWave, shmem);
  return hipGetLastError();
}

// Chunks of x for the phased matrix-core kernel: the fewest chunks of equal
// item counts (the last one shorter) whose x fits in LDS beside the split
// partials.  Returns the items per chunk, or 0 when a chunk would leave some
// wave without an item.
inline int mfma_chunk_items(int M, int K) {
  constexpr int NW = kSplitWaves;
  const int C = K / 128;
  const int64_t room = (int64_t)kLdsMax - (int64_t)NW * kWave * 16;
  const int fit = (int)(room / ((int64_t)M * 256));
  if (fit < NW) return 0;
  const int nph = (C + fit - 1) / fit;
  const int cp = (C + nph - 1) / nph;
  return C - (nph - 1) * cp >= NW ? cp : 0;
}

// Whole tiles per wave when the tiles fill at least half of the resident
// wavefront slots; otherwise (and when every wave gets at least one item and
// the partial sums fit in LDS) the waves of a workgroup split each tile.
// When x itself does not fit in LDS, the split kernel stages it in chunks.
template <int M, int PPB>
hipError_t launch_mfma_ppb(const uint16_t* x, int64_t ldx, const uint8_t* w,
                           const uint16_t* scales, const uint8_t* zp, void* y, int64_t ldy,
                           int y_type, int N, int K, int block_size, hipStream_t stream) {
  constexpr int NW = kMfmaWaves;
  const size_t xbytes = (size_t)M * K * 2;
  const size_t partials = (size_t)kSplitWaves * kWave * 16;
  const size_t split_bytes = xbytes + partials;
  const int ntiles = (N + 15) / 16;
  const bool x_fits = xbytes <= (size_t)kLdsMax;
  int64_t waves = 0;
  if (x_fits) {
    auto whole = int4_gemv_mfma<M, true, PPB, false, NW, kMfmaDepth>;
    const hipError_t e = allow_lds(whole, xbytes);
    if (e != hipSuccess) return e;
    waves = (int64_t)resident_workgroups(whole, NW * kWave, xbytes) * NW;
  }
  const bool few_tiles = !x_fits || 2LL * ntiles < waves;
  if (few_tiles && K / 128 >= kSplitWaves) {
    if (split_bytes <= (size_t)kLdsMax) {
      // k parts: tiles of 8 (4) rows when 16-row tiles leave CUs idle (8
      // wavefronts per workgroup: 16 measured slower, 1536 x 6912 at M = 8
      // 7.9 against 6.2 us; so did k parts in the packed layout's kernel,
      // 7.0 against 6.8 us for its 16-row tiles over 16 wavefronts)
      switch (mfma_k_parts(M, N, K, kSplitWaves)) {
        case 4:
          if constexpr (M <= 4)
            return launch_mfma_cfg<M, PPB, true, false, 4>(x, ldx, w, scales, zp, y, ldy, y_type,
                                                           N, K, block_size, split_bytes, 0,
                                                           stream);
          break;
        case 2:
          return launch_mfma_cfg<M, PPB, true, false, 2>(x, ldx, w, scales, zp, y, ldy, y_type, N,
                                                         K, block_size, split_bytes, 0, stream);
        default: {
          // rows too short for 8 wavefronts a step each in parts (e.g. 12
          // items): 4 wavefronts per workgroup
          const size_t bytes4 = xbytes + (size_t)4 * kWave * 16;
          switch (mfma_k_parts(M, N, K, 4)) {
            case 4:
              if constexpr (M <= 4)
                return launch_mfma_cfg<M, PPB, true, false, 4, 4>(
                    x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, bytes4, 0, stream);
              break;
            case 2:
              return launch_mfma_cfg<M, PPB, true, false, 2, 4>(
                  x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, bytes4, 0, stream);
            default:
              break;
          }
        }
      }
      return launch_mfma_cfg<M, PPB, true>(x, ldx, w, scales, zp, y, ldy, y_type, N, K,
                                           block_size, split_bytes, K / 128, stream);
    }
    const int cp = mfma_chunk_items(M, K);
    if (cp != 0)
      return launch_mfma_cfg<M, PPB, true, true>(x, ldx, w, scales, zp, y, ldy, y_type, N, K,
                                                 block_size, (size_t)M * cp * 256 + partials, cp,
                                                 stream);
  }
  if (!x_fits) return hipErrorInvalidValue;  // launch_m checks this first
  return launch_mfma_cfg<M, PPB, false>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size,
                                        xbytes, K / 128, stream);
}

template <int M>
hipError_t launch_mfma(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                       const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                       int block_size, hipStream_t stream) {
  if (block_size >= 128)
    return launch_mfma_ppb<M, 4>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
  if (block_size == 64)
    return launch_mfma_ppb<M, 2>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
  return launch_mfma_ppb<M, 1>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
}

template <int M>
hipError_t launch_m(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                    const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                    int block_size, hipStream_t stream) {
  if constexpr (M >= kMfmaMinM) {
    // The matrix-core kernel reads an item's scales with one load of
    // 8 * 32 / block_size bytes (at least 2) and, for block 32, its zero
    // points with one 2-byte load: both need matching base alignment.
    const uintptr_t salign = block_size >= 128 ? 2 : (size_t)8 * 32 / block_size;
    const bool aligned = (reinterpret_cast<uintptr_t>(scales) % salign == 0) &&
                         (block_size != 32 || reinterpret_cast<uintptr_t>(zp) % 2 == 0);
    // Two rows of x stay on v_dot2 (measured cold, in us, v_dot2 / matrix
    // cores) with blocks of 32 along rows of at most 4096 weights, where the
    // matrix-core kernel's per-block scaling and lane swaps cost more than
    // v_dot2 spends on a second row (4096 x 4096 6.0 / 6.8, 14336 x 4096
    // 11.7 / 12.4, 32000 x 4096 18.7 / 19.8, 11008 x 4096 10.1 / 10.4).  With
    // longer rows, or blocks of 64 or more, the matrix cores win, on short
    // matrices through the k parts of the split kernel (1536 x 6912, blocks
    // of 128: v_dot2 6.3, matrix cores in 16-row tiles 7.1, in parts 5.1;
    // 1536 x 1536: 4.4 against 3.4).
    const bool dot2_pair = M == 2 && block_size == 32 && K <= 4096;
    if (K % 128 == 0 && aligned && !dot2_pair &&
        ((size_t)M * K * 2 <= (size_t)kLdsMax || mfma_chunk_items(M, K) != 0))
      return launch_mfma<M>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
  }
  if constexpr (M <= kSpanMaxM) {
    if (K == 2048)
      return launch_span<M, kSpanRows / 1, 1, false>(x, ldx, w, scales, zp, y, ldy, y_type, N, K,
                                                      block_size, stream);
    if (K == 4096)
      return launch_span<M, kSpanRows / 2, 2, false>(x, ldx, w, scales, zp, y, ldy, y_type, N, K,
                                                      block_size, stream);
    if (K == 8192)
      return launch_span<M, kSpanRows / 4, 4, false>(x, ldx, w, scales, zp, y, ldy, y_type, N, K,
                                                      block_size, stream);
  }
  // Lanes per row (measured on the 151936 x 4096 lm_head shape): 32 is best at
  // small M, 8 at large M (more rows share each x read).  Take the first
  // preference that divides the row's piece count, so no lane idles in the
  // last stride of a row; then widen it for short matrices, up to twice the
  // lanes of one full round of wavefronts (measured on the 4096-row layers of
  // a 7B model: 4096 x 4096, 4096 x 11008, 4096 x 14336).
  const int P = K / 32;  // 16-byte pieces per row
  constexpr int pref[3] = {M <= 2 ? 32 : 8, 16, M <= 2 ? 8 : 32};
  int lpr = pref[0];
  for (int c : pref)
    if (P % c == 0) {
      lpr = c;
      break;
    }
  lpr = widen_lanes_per_row(lpr, N, P, 2 * kLanesToFill, true);
  if constexpr (M <= kSpanMaxM) {
    // Matrices too short for the persistent kernel (rows widened past one
    // wavefront, which takes the tiled kernel, so P >= 128 and, rows of
    // exactly 128 pieces taking the span kernel above, U >= 3): the span
    // kernel with a row per wavefront (measured faster than the tiled kernel
    // also with up to 40 of the last u's 64 lanes idle: 896 x 4864, 1536 x
    // 6912).
    const int U = (P + kWave - 1) / kWave;
    if (lpr > kWave && U >= 3 && U <= 8 &&
        (size_t)M * P * 80 <= (size_t)kLdsBudget) {
#define QG_SPAN(UU) \
  case UU:          \
    return launch_span<M, 1, UU, true>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
      switch (U) {
        QG_SPAN(3) QG_SPAN(4) QG_SPAN(5) QG_SPAN(6) QG_SPAN(7) QG_SPAN(8)
        default: break;
      }
#undef QG_SPAN
    }
  }
#define QG_LAUNCH(L, RR) \
  return launch_cfg<M, L, RR>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream)
  switch (lpr) {
    case 8: QG_LAUNCH(8, 2);
    case 16: QG_LAUNCH(16, 2);
    case 32: QG_LAUNCH(32, 2);
    case 64: QG_LAUNCH(64, 1);
    case 128: QG_LAUNCH(128, 1);
    default: QG_LAUNCH(256, 1);
  }
#undef QG_LAUNCH
}

}  // namespace

#ifdef QG_WAVE_TIMES
// Copies the wave records of the last span-kernel launch (4 x uint64 per
// wavefront: start, x staged, end, spans) to host memory; returns the number
// of wavefronts copied, or -1.
extern "C" __attribute__((visibility("default"))) int qg_wave_times_read(uint64_t* host,
                                                                          int max_waves) {
  const int n = max_waves < kWaveTimesMax ? max_waves : kWaveTimesMax;
  if (host == nullptr || n <= 0) return -1;
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(wave_times), (size_t)n * 4 * sizeof(uint64_t), 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return -1;
  return n;
}
#endif

hipError_t launch_int4_gemv(const uint16_t* x, int64_t ldx, const uint8_t* w,
                            const uint16_t* scales, const uint8_t* zp, void* y, int64_t ldy,
                            int y_type, int M, int N, int K, int block_size,
                            hipStream_t stream) {
  switch (M) {
#define QG_CASE(MM) \
  case MM:          \
    return launch_m<MM>(x, ldx, w, scales, zp, y, ldy, y_type, N, K, block_size, stream);
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace qg
