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
//  * x is staged once per workgroup in LDS, pre-permuted within every group of
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
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qg {
namespace {

struct Pairs8 {
  f16x2 a, b, c, d;  // (e0,e4)-zp, (e1,e5)-zp, (e2,e6)-zp, (e3,e7)-zp
};

// Eight 4-bit codes of one 32-bit word (element 2i in the low nibble of byte
// i) -> four exact fp16 pairs of (code - zero point).  `magic` is fp16 1024.0
// in both halves, held in a VGPR so that each mask-and-or is one v_and_or_b32.
__device__ __forceinline__ Pairs8 unpack8(uint32_t word, uint32_t magic, uint32_t bias_lo,
                                          uint32_t bias_hi) {
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = word >> 8;
  Pairs8 r;
  r.a = bitcast<f16x2>((word & 0x000F000Fu) | magic) + bitcast<f16x2>(bias_lo);
  r.b = __builtin_elementwise_fma(bitcast<f16x2>((word & 0x00F000F0u) | magic), sixteenth,
                                  bitcast<f16x2>(bias_hi));
  r.c = bitcast<f16x2>((w8 & 0x000F000Fu) | magic) + bitcast<f16x2>(bias_lo);
  r.d = __builtin_elementwise_fma(bitcast<f16x2>((w8 & 0x00F000F0u) | magic), sixteenth,
                                  bitcast<f16x2>(bias_hi));
  return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

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
    // Issue the first piece's loads before staging x: their latency overlaps
    // the staging and the barrier.
    Piece<R> cur;
    if (j < P) load(cur, gp0 + j);

    __syncthreads();
    const int groups = kn >> 3;
    for (int t = tid; t < M * groups; t += kBlock) {
      const int m = t / groups;
      const int gi = t - m * groups;
      const uint16_t* src = x + m * ldx + kc + gi * 8;
      uint32_t h[8];
      if (x_vec16) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        h[0] = v.x & 0xFFFFu; h[1] = v.x >> 16; h[2] = v.y & 0xFFFFu; h[3] = v.y >> 16;
        h[4] = v.z & 0xFFFFu; h[5] = v.z >> 16; h[6] = v.w & 0xFFFFu; h[7] = v.w >> 16;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = src[e];
      }
      xs[m * PS + (gi >> 2) * 5 + (gi & 3)] = make_uint4(
          h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16));
    }
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

template <int M, int LPR, int R, int PB, bool ZP, bool STRIDED>
__global__ __launch_bounds__(kBlock) void int4_gemv_persistent(
    const uint16_t* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zp, int zrow,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int bs_log2, int ntiles,
    int x_vec16) {
  extern __shared__ uint4 xs[];  // [M][K/32][5]: 4 permuted groups of 8 halves + pad
  constexpr int S = kBlock / LPR;  // row slots per workgroup
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
  if (nitems > 0) load(cur, t_begin, 0);

  const int groups = K >> 3;
  for (int t = tid; t < M * groups; t += kBlock) {
    const int m = t / groups;
    const int gi = t - m * groups;
    const uint16_t* src = x + m * ldx + gi * 8;
    uint32_t h[8];
    if (x_vec16) {
      const uint4 v = *reinterpret_cast<const uint4*>(src);
      h[0] = v.x & 0xFFFFu; h[1] = v.x >> 16; h[2] = v.y & 0xFFFFu; h[3] = v.y >> 16;
      h[4] = v.z & 0xFFFFu; h[5] = v.z >> 16; h[6] = v.w & 0xFFFFu; h[7] = v.w >> 16;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = src[e];
    }
    xs[m * PS + (gi >> 2) * 5 + (gi & 3)] = make_uint4(
        h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16));
  }
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

// Measured on the 151936 x 4096 lm_head shape: a grid-stride tile order over a
// full resident grid beats contiguous per-workgroup ranges and beats an
// equal-share (smaller) grid.
constexpr bool kStrided = true;
constexpr bool kBalanced = false;

template <int M, int LPR, int R, int PB = 1>
hipError_t launch_cfg(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                      const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                      int block_size, hipStream_t stream) {
  constexpr int RT = (kBlock / LPR) * R;
  const int bs_log2 = __builtin_ctz((unsigned)block_size);
  const int zrow = ((K / block_size) + 1) / 2;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int ntiles = (N + RT - 1) / RT;
  // x takes 80 bytes of LDS per 32 elements and row.
  const size_t full = (size_t)M * (K / 32) * 80;
  if constexpr (LPR <= kWave) {
   if (full <= (size_t)kLdsBudget) {
    auto kern = zp ? int4_gemv_persistent<M, LPR, R, PB, true, kStrided>
                   : int4_gemv_persistent<M, LPR, R, PB, false, kStrided>;
    const int cap = resident_workgroups(kern, kBlock, full);
    // Equal tile counts per workgroup: the fewest rounds that fit, then the
    // smallest grid that still covers every tile in that many rounds.
    const int rounds = (ntiles + cap - 1) / cap;
    const int grid = kBalanced ? (ntiles + rounds - 1) / rounds : (ntiles < cap ? ntiles : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), full, stream, x, ldx, w, scales, zp, zrow,
                       y, ldy, y_type, N, K, bs_log2, ntiles, x_vec16);
    return hipGetLastError();
   }
  }
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
  return hipGetLastError();
}

template <int M>
hipError_t launch_m(const uint16_t* x, int64_t ldx, const uint8_t* w, const uint16_t* scales,
                    const uint8_t* zp, void* y, int64_t ldy, int y_type, int N, int K,
                    int block_size, hipStream_t stream) {
  // Lanes per row (measured on the 151936 x 4096 lm_head shape): 32 is best at
  // small M, 8 at large M (more rows share each x read).  Take the first
  // preference that divides the row's piece count, so no lane idles in the
  // last stride of a row; then widen it for short matrices.
  const int P = K / 32;  // 16-byte pieces per row
  constexpr int pref[3] = {M <= 2 ? 32 : 8, 16, M <= 2 ? 8 : 32};
  int lpr = pref[0];
  for (int c : pref)
    if (P % c == 0) {
      lpr = c;
      break;
    }
  lpr = widen_lanes_per_row(lpr, N, P);
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
