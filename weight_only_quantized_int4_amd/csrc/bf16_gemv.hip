// bf16_gemv.hip -- dense bf16 GEMV for gfx950, M = 1..8, any K >= 1 and any
// 2-byte storage offset of x and W.
//
// Operation (the bf16 GEMV primitive of the AstrAI backend commit list):
//     y[m,n] = sum_k x[m,k] * w[n,k]
//
// Three kernels, chosen per call on the host:
//  * aligned: x and W rows 16-byte aligned and K a multiple of 8 (the
//    production case with allocator-aligned tensors).  Pure 128-bit weight
//    loads, x staged as bf16 in LDS, v_dot2_f32_bf16 (exact bf16 products,
//    fp32 accumulation) -- no branch inside the loop.
//  * general: any alignment.  Each row's 128-bit loads are anchored at the
//    row's first 16-byte-aligned element h (0..7); the h head elements and
//    the < 8 tail elements are swept one at a time.  x is staged in LDS as
//    fp32 (so it can be read at any element offset) in K-chunks with an
//    8-element halo, and every product is one fp32 FMA.
// Both keep one row per group of LPR lanes and reduce with cross-lane
// shuffles; no split-K (measured as a regression on the page).
//  * matrix core (M >= 2, aligned, K a multiple of 128): see bf16_gemv_mfma.
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qg {
namespace {

template <int M, int LPR, int R, int DG>
__global__ __launch_bounds__(kBlock) void bf16_gemv_aligned(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int KC) {
  extern __shared__ uint4 xs[];  // [M][KC/8] bf16
  constexpr int S = kBlock / LPR;
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int j = tid % LPR;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int G = KC >> 3;

  // Rows past the end load the last row (results never stored): no branches.
  int rows[R];
  uint32_t wo[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    rows[i] = (tile * R + i) * S + slot;
    wo[i] = (uint32_t)(rows[i] < N ? rows[i] : N - 1) * (uint32_t)ldw;
  }
  float acc[R][M];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.f;

#pragma unroll 1
  for (int kc = 0; kc < K; kc += KC) {
    const int kn = min(KC, K - kc);
    const int P = kn >> 3;
    auto load = [&](uint4 (&v)[R], int p) {
#pragma unroll
      for (int i = 0; i < R; ++i) v[i] = load_stream16(w + (wo[i] + (uint32_t)(kc + 8 * p)));
    };
    // A ring of DG pieces per lane: piece p + DG*LPR reloads the slot of
    // piece p as soon as p is consumed, so DG 16-byte loads per row stay in
    // flight.
    uint4 ring[DG][R];
    __syncthreads();
    stage_slots<4>(
        tid, kBlock, M * P,
        [&](int t) {
          const int m = t / P;
          return *reinterpret_cast<const uint4*>(x + m * ldx + kc + 8 * (t - m * P));
        },
        [&](int t, uint4 v) {
          const int m = t / P;
          xs[m * G + (t - m * P)] = v;
        },
        [&] {
#pragma unroll
          for (int k = 0; k < DG; ++k)
            if (j + k * LPR < P) load(ring[k], j + k * LPR);
        });
    __syncthreads();
    auto consume = [&](const uint4 (&wv)[R], int p) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint4 xv = xs[m * G + p];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          float t = acc[i][m];
          t = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(wv[i].x), bitcast<bf16x2>(xv.x), t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(wv[i].y), bitcast<bf16x2>(xv.y), t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(wv[i].z), bitcast<bf16x2>(xv.z), t, false);
          t = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(wv[i].w), bitcast<bf16x2>(xv.w), t, false);
          acc[i][m] = t;
        }
      }
    };
#pragma unroll 1
    for (int p = j; p < P; p += DG * LPR) {
#pragma unroll
      for (int k = 0; k < DG; ++k) {
        const int pk = p + k * LPR;
        if (pk < P) {
          consume(ring[k], pk);
          if (pk + DG * LPR < P) load(ring[k], pk + DG * LPR);
        }
      }
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

constexpr int kGenStage = 8;
constexpr int kGenShortRow = 128;  // elements

// LDS layout of the general kernel's staged x: a pad float after every 8.
__host__ __device__ constexpr int gen_x_index(int e) { return e + (e >> 3); }
__host__ __device__ constexpr int gen_x_stride(int KC) { return gen_x_index(KC + 8) + 1; }

template <int M, int LPR>
__global__ __launch_bounds__(kBlock) void bf16_gemv_general(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int KC) {
  // [M][gen_x_stride(KC)] fp32, chunk plus halo; element e of a row sits at
  // e + e / 8 (one pad float after every 8), so the lanes of a row, whose
  // pieces start 8 elements apart, read banks 9 floats apart (no conflicts;
  // unpadded, every read of a wavefront hit 4 banks).
  extern __shared__ float xf[];
  const int XS = gen_x_stride(KC);
  constexpr int S = kBlock / LPR;
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int j = tid % LPR;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int n = tile * S + slot;
  const bool live = n < N;
  const uint16_t* wr = w + (int64_t)(live ? n : 0) * ldw;
  // Anchor: first element of the row whose address is 16-byte aligned.
  int h = (int)(((16u - (uint32_t)(reinterpret_cast<uintptr_t>(wr) & 15u)) & 15u) >> 1);
  if (h > K) h = K;
  const int nbody = (K - h) >> 3;
  const int t0 = h + (nbody << 3);

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;

  auto body_piece = [&](const uint4 v, int s0, int kc) {
    const float wv[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                         bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float* xp = xf + m * XS;
      float a = acc[m];
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaf(wv[e], xp[gen_x_index(s0 - kc + e)], a);
      acc[m] = a;
    }
  };
  // The first chunk's first body piece of this lane is loaded behind the
  // first round of x loads, so the two latencies overlap.
  uint4 pre = {0u, 0u, 0u, 0u};
  const int e_hi0 = min(KC, K) - h;
  const bool have_pre = live && j < min(nbody, e_hi0 > 0 ? (e_hi0 + 7) >> 3 : 0);

#pragma unroll 1
  for (int kc = 0; kc < K; kc += KC) {
    const int kn = min(KC, K - kc);
    const int ext = min(kn + 8, K - kc);
    __syncthreads();
    // x rows are read as aligned 16-byte words (8 elements each; a word that
    // holds an element of the row lies in the same page as that element, so
    // its other bytes are readable), kGenStage words in flight per thread
    // before the first wait.  Slot q of a thread is word tid + r * kBlock of
    // row m, q = m * per + r (the same for the whole workgroup, counted
    // without divisions).
    const int per = ((ext + 14) / 8 + kBlock - 1) / kBlock;  // >= words of any row
    // Short rows (a few words) are staged one element per thread: cheaper
    // than kGenStage word slots per thread that mostly hold nothing.
    const int nq = ext <= kGenShortRow ? 0 : M * per;
    if (nq == 0) {
      for (int t = tid; t < M * ext; t += kBlock) {
        const int m = t / ext, e = t - m * ext;
        xf[m * XS + gen_x_index(e)] = __uint_as_float((uint32_t)x[m * ldx + kc + e] << 16);
      }
      if (kc == 0 && have_pre) pre = load_stream16(wr + h + 8 * j);
    }
    int m0 = 0, r0 = 0;      // (m, r) of slot q0
    for (int q0 = 0; q0 < nq; q0 += kGenStage) {
      uint4 v[kGenStage];
      int mu[kGenStage], wu[kGenStage];
      {
        int m = m0, r = r0;
#pragma unroll
        for (int u = 0; u < kGenStage; ++u) {
          const int mc = min(m, M - 1);
          const uintptr_t rb = reinterpret_cast<uintptr_t>(x + mc * ldx + kc);
          const int skip = (int)((rb & 15u) >> 1);  // elements before the row in its first word
          const int nw = (skip + ext + 7) >> 3;     // words holding the row
          const int wi = tid + r * kBlock;
          mu[u] = m < M && wi < nw ? m : -1;         // -1: nothing to store
          wu[u] = 8 * wi - skip;                     // element of the word's first half-word
          v[u] = *reinterpret_cast<const uint4*>((rb & ~(uintptr_t)15) +
                                                 16 * (uintptr_t)min(wi, nw - 1));
          if (++r == per) { r = 0; ++m; }
        }
        m0 = m;
        r0 = r;
      }
      if (kc == 0 && q0 == 0 && have_pre) {
        __builtin_amdgcn_sched_barrier(0);
        pre = load_stream16(wr + h + 8 * j);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < kGenStage; ++u) {
        if (mu[u] >= 0) {  // (whole wavefronts skip the words past short rows)
          const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int e = wu[u] + k;
            if (e >= 0 && e < ext)
              xf[mu[u] * XS + gen_x_index(e)] =
                  __uint_as_float(k & 1 ? wd[k >> 1] & 0xFFFF0000u : wd[k >> 1] << 16);
          }
        }
      }
    }
    __syncthreads();
    if (!live) continue;

    // head: k in [0, h)
    for (int k = kc + j; k < min(h, kc + kn); k += LPR) {
      const float wf = __uint_as_float((uint32_t)wr[k] << 16);
#pragma unroll
      for (int m = 0; m < M; ++m)
        acc[m] = __builtin_fmaf(wf, xf[m * XS + gen_x_index(k - kc)], acc[m]);
    }
    // body: 16-byte pieces starting at h + 8i that begin inside this chunk
    const int i_lo = (kc > h) ? (kc - h + 7) >> 3 : 0;
    const int e_hi = kc + kn - h;
    const int i_hi = min(nbody, e_hi > 0 ? (e_hi + 7) >> 3 : 0);
    int i = i_lo + j;
    if (kc == 0 && have_pre) {  // i == j here
      body_piece(pre, h + 8 * j, kc);
      i += LPR;
    }
    for (; i < i_hi; i += LPR) body_piece(load_stream16(wr + h + 8 * i), h + 8 * i, kc);
    // tail: k in [t0, K)
    for (int k = max(kc, t0) + j; k < kc + kn; k += LPR) {
      const float wf = __uint_as_float((uint32_t)wr[k] << 16);
#pragma unroll
      for (int m = 0; m < M; ++m)
        acc[m] = __builtin_fmaf(wf, xf[m * XS + gen_x_index(k - kc)], acc[m]);
    }
  }

  __shared__ float red[(kBlock / kWave) * M];
  group_sum_wide<LPR, M>(acc, red);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (j == 0 && live) store_out(y, m * ldy + n, acc[m], y_type);
}

// Matrix-core variant for M >= 2 (16-byte aligned rows, K a multiple of 128):
// v_mfma_f32_16x16x32_bf16 with x as the A operand (M rows; A rows M..15
// repeat real rows and their D rows are never stored) and 16 weight rows as
// the B operand.  An item is 128 k of a 16-row tile; lane (n, g) loads
// k = 128c + 32t + 8g .. +8 of row n for t = 0..3 (each load instruction
// reads 64 contiguous bytes of 16 rows), which is exactly the B operand of
// MFMA t over k = 128c + 32t .. +32.  bf16 products are exact and the 4
// MFMAs of every item chain into one fp32 accumulator, so the loop carries no
// vector ALU work beyond LDS addressing.  x is staged in LDS (16-byte slots
// of 8 elements, XOR-swizzled by 4 * (row & 3) so the A
// reads of rows 0..3 fall in distinct banks; with SPLIT each wave stages the
// slots of its own items).  Tiles, the D-item register ring and the SPLIT
// partial sums follow the int4 matrix-core kernel, and so do the k parts
// (KS, with SPLIT): where 16-row tiles leave CUs idle, the 16 MFMA columns
// carry TR = 16 / KS rows in KS parts of their k range (column n: tile row
// n % TR, part h = n / TR; A row r: x row r % TR of part r / TR; step c
// covers items KS * c + h), and the tile-end sum adds the parts after the
// wavefronts, in a fixed order.
template <int M, bool SPLIT, int NW, int D, int KS = 1>
__global__ __launch_bounds__(NW * kWave) void bf16_gemv_mfma(
    const uint16_t* __restrict__ x, int64_t ldx, const uint16_t* __restrict__ w, int64_t ldw,
    void* __restrict__ y, int64_t ldy, int y_type, int N, int K, int ntiles, int x_vec16) {
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && SPLIT && M <= 16 / KS),
                "k parts: split tiles, M rows per part");
  constexpr int TR = 16 / KS;  // weight rows per tile
  extern __shared__ uint4 xs[];  // [M][K/8] slots, swizzled; then the SPLIT partials
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = lane & 15, g = lane >> 4;
  const int ti = n % TR, h = n / TR;  // tile row and k part of column n
  const int S8 = K >> 3;
  const int C = K >> 7;
  const int CS = C / KS;  // steps per tile
  const int t0 = SPLIT ? (int)blockIdx.x : (int)blockIdx.x * NW + wave;
  const int TS = SPLIT ? (int)gridDim.x : (int)gridDim.x * NW;
  const int cb = SPLIT ? wave * CS / NW : 0;
  const int ce = SPLIT ? (wave + 1) * CS / NW : CS;
  const int my_tiles = t0 < ntiles ? (ntiles - t0 + TS - 1) / TS : 0;
  const int nitems = my_tiles * (ce - cb);

  struct Item {
    uint4 w[4];
  };
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(w);
  auto issue = [&](Item& it, int tile, int c) {
    const int row = tile * TR + ti;
    // byte offset (tensors are below 4 GiB): a 32-bit offset off a uniform
    // base keeps each load to one address register
    const uint32_t base = ((uint32_t)(row < N ? row : N - 1) * (uint32_t)ldw +
                           (uint32_t)(128 * (KS * c + h) + 8 * g)) * 2u;
#pragma unroll
    for (int t = 0; t < 4; ++t) it.w[t] = load16(wb + (base + 64u * t));
  };
  auto advance = [&](int& tile, int& c) {
    c = c + 1 == ce ? cb : c + 1;
    tile = c == cb ? tile + TS : tile;
  };

  Item ring[D];
  int lt = t0, lc = cb;
  auto load_slot = [&](const uint16_t* src) {
    if (x_vec16) return *reinterpret_cast<const uint4*>(src);
    return make_uint4(src[0] | ((uint32_t)src[1] << 16), src[2] | ((uint32_t)src[3] << 16),
                      src[4] | ((uint32_t)src[5] << 16), src[6] | ((uint32_t)src[7] << 16));
  };
  auto fill_ring = [&] {  // unconditional: rows past the end are clamped
#pragma unroll
    for (int k = 0; k < D; ++k) {
      issue(ring[k], lt, lc);
      advance(lt, lc);
    }
  };
  // SPLIT: each wavefront stages only the x slots of its own items [cb, ce)
  // (16 per item and row of x) and reads no others, as in the int4 kernel
  // (1536 x 6912 M = 8 12.2 -> 10.6 us, M = 3 10.9 -> 9.9; 4096^2 M = 8
  // 10.2 -> 9.4), except for more than 4 rows of x over fewer than 2 items
  // per wavefront, where most lanes would idle in it (6912 x 1536 M = 8:
  // 7.4 against 7.8 us).
  if (SPLIT && !(M > 4 && C < 2 * NW)) {
    const int ns = 16 * KS * (ce - cb);
    bool pending = true;
    for (int r0 = 0; r0 < ns; r0 += kWave) {
      const int r = r0 + lane < ns ? r0 + lane : ns - 1;
      const int gi = 16 * KS * cb + r;
      uint4 v[M];
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] = load_slot(x + m * ldx + gi * 8);
      if (pending) {
        __builtin_amdgcn_sched_barrier(0);
        fill_ring();
        __builtin_amdgcn_sched_barrier(0);
        pending = false;
      }
#pragma unroll
      for (int m = 0; m < M; ++m) xs[m * S8 + (gi ^ ((m & 3) << 2))] = v[m];
    }
    // Lanes read slots that other lanes of the wavefront wrote.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  } else {
    stage_slots<4>(
        tid, NW * kWave, M * S8, [&](int t) { return load_slot(x + (t / S8) * ldx + (t % S8) * 8); },
        [&](int t, uint4 v) {
          const int m = t / S8;
          xs[m * S8 + ((t - m * S8) ^ ((m & 3) << 2))] = v;
        },
        fill_ring);
    __syncthreads();
  }

  uint32_t aoff[4];
  const int arow = ti < M ? ti : ti % M;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    aoff[t] = (uint32_t)((arow * S8 + 16 * h + ((4 * t + g) ^ ((arow & 3) << 2))) * 16);
  const char* xs_bytes = reinterpret_cast<const char*>(xs);

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc = zero4;
  auto consume = [&](const Item& cur, int tile, int c) {
    const uint32_t ibase = (uint32_t)(KS * c) * 256u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 a = *reinterpret_cast<const uint4*>(xs_bytes + (aoff[t] + ibase));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(cur.w[t]),
                                                    acc, 0, 0, 0);
    }
    if (c == ce - 1) {  // tile finished: lane (n, g) holds rows 4g..4g+3 of column n
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
          // a loop (its count hidden from the compiler, which would otherwise
          // peel a single pass), so that one part's reads are in registers at
          // a time
          if constexpr (KS > 1) {
            int nparts = KS;
            asm volatile("" : "+s"(nparts));
#pragma unroll 1
            for (int hp = 1; hp < nparts; ++hp) {
              const f32x4 ps = part_sum(lane + hp * (TR + 16 * (TR / 4)));
#pragma unroll
              for (int i = 0; i < 4; ++i) sum[i] += ps[i];
            }
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
    // Keep the scheduler from hoisting later items' A reads (16 registers
    // each) above this one.
    __builtin_amdgcn_sched_barrier(0);
  };

  int pt = t0, pc = cb;
  int u = 0;
#pragma unroll 1
  for (; u + D <= nitems; u += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      consume(ring[k], pt, pc);
      advance(pt, pc);
      issue(ring[k], lt, lc);
      advance(lt, lc);
    }
  }
#pragma unroll
  for (int k = 0; k < D; ++k) {
    if (u + k < nitems) {
      consume(ring[k], pt, pc);
      advance(pt, pc);
    }
  }
}

// Launch shapes (waves per workgroup, items in flight per lane) for whole
// tiles per wave and for tiles split over the waves of a workgroup (short
// matrices); measured on the 1536 x 6912, 6912 x 1536 and 1536 x 1536 shapes.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaDepth = 2;
constexpr int kSplitWaves = 8;
constexpr int kSplitDepth = 2;

template <int M, bool SPLIT, int NW, int D, int KS = 1>
hipError_t launch_mfma_cfg(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                           int64_t ldy, int y_type, int N, int K, size_t shmem,
                           hipStream_t stream) {
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0);
  const int ntiles = (N + 16 / KS - 1) / (16 / KS);
  auto kern = bf16_gemv_mfma<M, SPLIT, NW, D, KS>;
  const hipError_t e = allow_lds(kern, shmem);
  if (e != hipSuccess) return e;
  const int cap = resident_workgroups(kern, NW * kWave, shmem);
  const int want = SPLIT ? ntiles : (ntiles + NW - 1) / NW;
  const int grid = want < cap ? want : cap;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * kWave), shmem, stream, x, ldx, w, ldw, y, ldy,
                     y_type, N, K, ntiles, x_vec16);
  note_launch(SPLIT ? kPathBf16MfmaSplit : kPathBf16MfmaTiles, M, grid, NW * kWave, shmem);
  return hipGetLastError();
}

// Whole tiles per wave when the tiles fill at least half of the resident
// wavefront slots; otherwise the waves of a workgroup split each tile.
template <int M>
hipError_t launch_mfma(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                       int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  const size_t xbytes = (size_t)M * K * 2;
  const int ntiles = (N + 15) / 16;
  auto whole = bf16_gemv_mfma<M, false, kMfmaWaves, kMfmaDepth>;
  const hipError_t e = allow_lds(whole, xbytes);
  if (e != hipSuccess) return e;
  const int64_t waves = (int64_t)resident_workgroups(whole, kMfmaWaves * kWave, xbytes) * kMfmaWaves;
  // Split: every wave needs at least one item of the tile, and the partial
  // sums (16 bytes per lane) share LDS with x.
  const size_t split_bytes = xbytes + (size_t)kSplitWaves * kWave * 16;
  if (2LL * ntiles < waves && K / 128 >= kSplitWaves && split_bytes <= (size_t)kLdsMax) {
    // k parts: tiles of 8 (4) rows when 16-row tiles leave CUs idle
    switch (mfma_k_parts(M, N, K, kSplitWaves)) {
      case 4:
        if constexpr (M <= 4)
          return launch_mfma_cfg<M, true, kSplitWaves, kSplitDepth, 4>(x, ldx, w, ldw, y, ldy,
                                                                      y_type, N, K, split_bytes,
                                                                      stream);
        break;
      case 2:
        return launch_mfma_cfg<M, true, kSplitWaves, kSplitDepth, 2>(x, ldx, w, ldw, y, ldy,
                                                                    y_type, N, K, split_bytes,
                                                                    stream);
      default: {
        // rows too short for 8 wavefronts a step each in parts (e.g. 12
        // items): 4 wavefronts per workgroup
        const size_t bytes4 = xbytes + (size_t)4 * kWave * 16;
        switch (mfma_k_parts(M, N, K, 4)) {
          case 4:
            if constexpr (M <= 4)
              return launch_mfma_cfg<M, true, 4, kSplitDepth, 4>(x, ldx, w, ldw, y, ldy, y_type,
                                                                 N, K, bytes4, stream);
            break;
          case 2:
            return launch_mfma_cfg<M, true, 4, kSplitDepth, 2>(x, ldx, w, ldw, y, ldy, y_type, N,
                                                               K, bytes4, stream);
          default:
            break;
        }
      }
    }
    return launch_mfma_cfg<M, true, kSplitWaves, kSplitDepth>(x, ldx, w, ldw, y, ldy, y_type, N,
                                                             K, split_bytes, stream);
  }
  return launch_mfma_cfg<M, false, kMfmaWaves, kMfmaDepth>(x, ldx, w, ldw, y, ldy, y_type, N, K,
                                                          xbytes, stream);
}

// 16-byte weight loads in flight per lane and row in the aligned kernel.
constexpr int kAlignedDepth = 4;
// Wavefronts per SIMD the v_dot2 kernels' rows should occupy (lanes per row
// are widened up to that).
constexpr int kBf16FillWaves = 8;
constexpr int kBf16LongRowK = 4096;

template <int M, int LPR, int R>
hipError_t launch_aligned(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                          int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  constexpr int RT = (kBlock / LPR) * R;
  const int grid = (N + RT - 1) / RT;
  int KC = (kLdsXBudget / (2 * M)) & ~7;
  if (KC > K) KC = K;
  const size_t shmem = (size_t)M * KC * 2;
  hipLaunchKernelGGL((bf16_gemv_aligned<M, LPR, R, kAlignedDepth>), dim3(grid), dim3(kBlock), shmem, stream, x,
                     ldx, w, ldw, y, ldy, y_type, N, K, KC);
  note_launch(kPathBf16Aligned, M, grid, kBlock, shmem);
  return hipGetLastError();
}

template <int M, int LPR>
hipError_t launch_general(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                          int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  constexpr int S = kBlock / LPR;
  const int grid = (N + S - 1) / S;
  // largest multiple of 8 whose padded rows fit the budget
  int KC = ((kLdsXBudget / (4 * M) - 10) * 8 / 9) & ~7;
  if (KC > K) KC = K;
  const size_t shmem = (size_t)M * gen_x_stride(KC) * 4;
  hipLaunchKernelGGL((bf16_gemv_general<M, LPR>), dim3(grid), dim3(kBlock), shmem, stream, x, ldx,
                     w, ldw, y, ldy, y_type, N, K, KC);
  note_launch(kPathBf16General, M, grid, kBlock, shmem);
  return hipGetLastError();
}

// Smallest M that takes the matrix-core kernel.
constexpr int kMfmaMinM = 2;

template <int M>
hipError_t launch_m(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw, void* y,
                    int64_t ldy, int y_type, int N, int K, hipStream_t stream) {
  const bool aligned = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 8 == 0) &&
                       ((reinterpret_cast<uintptr_t>(w) & 15) == 0) && (ldw % 8 == 0) &&
                       (K % 8 == 0);
  if constexpr (M >= kMfmaMinM) {
    if (aligned && K % 128 == 0 && (size_t)M * K * 2 <= (size_t)kLdsMax)
      return launch_mfma<M>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
  }
  // 16 lanes per row, widened for short matrices (see widen_lanes_per_row).
  // Rows of at least kBf16LongRowK weights are widened until they occupy
  // kBf16FillWaves wavefronts per SIMD: a 16-byte piece holds 8 bf16 weights
  // (32 int4 ones), so HBM needs more of them in flight.  Shorter rows keep
  // the int4 kernels' target: wider rows there leave each lane about one
  // piece, and each workgroup stages x for one or two rows (measured: 1536²
  // 3.6 -> 4.3 us, 6912 x 1536 6.2 -> 7.8 us when widened).
  const int64_t fill = K >= kBf16LongRowK ? kLanesToFill * kBf16FillWaves / 2 : kLanesToFill;
  const int lpr = widen_lanes_per_row(16, N, (K + 7) / 8, fill);
  constexpr int R = (M <= 4) ? 2 : 1;
  if (aligned) {
    switch (lpr) {
      case 16: return launch_aligned<M, 16, R>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
      case 32: return launch_aligned<M, 32, R>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
      case 64: return launch_aligned<M, 64, 1>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
      case 128: return launch_aligned<M, 128, 1>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
      default: return launch_aligned<M, 256, 1>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    }
  }
  switch (lpr) {
    case 16: return launch_general<M, 16>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    case 32: return launch_general<M, 32>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    case 64: return launch_general<M, 64>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    case 128: return launch_general<M, 128>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    default: return launch_general<M, 256>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
  }
}

}  // namespace

hipError_t launch_bf16_gemv(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                            void* y, int64_t ldy, int y_type, int M, int N, int K,
                            hipStream_t stream) {
  switch (M) {
#define QG_CASE(MM) \
  case MM:          \
    return launch_m<MM>(x, ldx, w, ldw, y, ldy, y_type, N, K, stream);
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace qg
