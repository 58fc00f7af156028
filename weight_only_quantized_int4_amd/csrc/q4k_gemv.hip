// q4k_gemv.hip -- q4_K GEMV for gfx950 (coefficients decoded in the kernel or
// read from a W_dsc plane), and the load-time W_dsc plane builder.
//
// Operation ("62 . r59 -- q4_K W_dsc plane + riders", sections 2.1-2.3 and 3.2):
// a q4_K row is K/256 super-blocks of 144 bytes (fp16 d, fp16 dmin, twelve
// bytes of packed 6-bit scales/mins, 128 bytes of 4-bit quants).  Chunk c of
// 32 weights has the rank-1 coefficients dv = d*sc(c), mv = -(dmin*m(c)), and
// its weights are w = dv*q + mv.  The W_dsc plane stores (dv, mv) chunk-major:
// entry (c, n) at float2 index c*N + n.
//
// Design:
//  * One kernel template serves both entry points: DSC=false decodes (dv, mv)
//    from the super-block header, DSC=true loads them from the plane.  Every
//    other instruction, and so the summation order, is shared, which makes
//    the two results bitwise equal whenever the plane matches the weights
//    (the same structural argument the page makes for its two kernel
//    instances).
//  * A "piece" is 32 quant bytes of one super-block = chunks 2g and 2g+1
//    (64 weights).  A whole wavefront owns a row (LPR = 64 lanes); lane j
//    always has the same g = j % 4, so its half-pair of the 6-bit decode is
//    loop-invariant and branch-free.  A K = 4096 row is 64 pieces, one per
//    lane, so every lane's 48 bytes are in flight at once; a workgroup of 16
//    wavefronts covers 16 rows and shares one staged copy of x.
//  * Rank-1 factorisation per chunk: sum_l (dv*q_l + mv) x_l is evaluated as
//    dv * (sum_l q_l x_l) + mv * (sum_l x_l).  The chunk sums of x are computed
//    once per workgroup while x is staged in LDS, so the inner loop spends one
//    fp32 FMA per weight (v_fma_mix_f32 on an exact fp16 quant).  With a one-hot
//    x this still reproduces w = RN(dv*q + mv) bit-exactly.
//  * Quants are converted with the fp16 1024.0 mantissa trick (exact), as in
//    the int4 kernel.
//  * Weights are read with plain (cached) loads: a super-block's header and
//    quants share cache lines and are read by different instructions
//    (measured faster than non-temporal loads here).
//  * x lives in LDS as fp32 with 4 floats of padding after every 64: the
//    lanes of a row read pieces 272 bytes apart, so their 16-byte LDS reads
//    fall in distinct banks (without the padding all of them would hit the
//    same bank).
#include "qgemv_device.h"
#include "qgemv_launch.h"

namespace qg {
namespace {

constexpr int kQ4kBlockBytes = 144;

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// (sc, m) of chunks 2g and 2g+1 from the twelve packed bytes (words A = bytes
// 0..3, B = 4..7, C = 8..11), as two bytes each: s2 = sc(2g) | sc(2g+1) << 8.
// get_scale_min_k4, branch-free over the lane's g:
//   chunk < 4 : sc = A.byte[c] & 63,  m = B.byte[c] & 63
//   chunk >= 4: sc = (C.byte[c-4] & 15) | ((A.byte[c-4] >> 6) << 4)
//               m  = (C.byte[c-4] >> 4) | ((B.byte[c-4] >> 6) << 4)
// For both halves the two bytes sit at byte offset 2*(g&1) of their words.
__device__ __forceinline__ void scale_min_pair(uint32_t A, uint32_t B, uint32_t C, int g,
                                               uint32_t& s2, uint32_t& m2) {
  const int sh = (g & 1) << 4;
  const uint32_t a = A >> sh, b = B >> sh, c = C >> sh;
  if (g < 2) {
    s2 = a & 0x3F3Fu;
    m2 = b & 0x3F3Fu;
  } else {
    s2 = (c & 0x0F0Fu) | ((a >> 2) & 0x3030u);
    m2 = ((c >> 4) & 0x0F0Fu) | ((b >> 2) & 0x3030u);
  }
}

// What one lane loads for one piece: 32 quant bytes and either the 16-byte
// header (decoded in the kernel) or the two plane entries.
struct Q4kPiece {
  uint4 q0, q1;
  uint4 h;      // header (DSC = false)
  float2 ea, eb;  // plane entries of chunks 2g and 2g+1 (DSC = true)
};

template <int M, int LPR, int NT, bool DSC>
__global__ __launch_bounds__(NT) void q4k_gemv_kernel(
    const float* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const float2* __restrict__ dsc, float* __restrict__ y, int64_t ldy, int N, int K, int KC,
    int x_vec16) {
  static_assert(LPR % 4 == 0, "a lane's pair index g must be fixed");
  extern __shared__ float smem[];
  const int XSTR = (KC >> 6) * 68;  // floats per x row in LDS (64 + 4 pad per piece)
  float* xs = smem;                 // [M][KC/64][68]
  float* sx = smem + M * XSTR;      // [M][KC/32] chunk sums of x
  const int KC32 = KC >> 5;
  constexpr int S = NT / LPR;
  const int tid = threadIdx.x;
  const int slot = tid / LPR;
  const int j = tid % LPR;
  const int g = j & 3;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int n = tile * S + slot;
  // Rows past the end load the last row (results never stored): no branches.
  const uint32_t nl = (uint32_t)(n < N ? n : N - 1);
  const int nsb = K >> 8;
  const uint32_t wo = nl * (uint32_t)nsb * (uint32_t)kQ4kBlockBytes;

  const uint32_t magic = vreg_const(0x64006400u);
  const f16x2 m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const f16x2 m64 = {(_Float16)-64.0f, (_Float16)-64.0f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};

  auto load = [&](Q4kPiece& st, int sb) {
    const uint32_t bo = wo + (uint32_t)sb * kQ4kBlockBytes;
    st.q0 = load16(w + (bo + 16u + 32u * g));
    st.q1 = load16(w + (bo + 32u + 32u * g));
    if constexpr (DSC) {
      const uint32_t c = (uint32_t)sb * 8u + 2u * g;
      st.ea = load8f(dsc + (c * (uint32_t)N + nl));
      st.eb = load8f(dsc + ((c + 1u) * (uint32_t)N + nl));
    } else {
      st.h = load16(w + bo);
    }
  };

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;

#pragma unroll 1
  for (int kc = 0; kc < K; kc += KC) {
    const int kn = min(KC, K - kc);
    const int P = kn >> 6;  // (super-block, g) pieces in this chunk
    const int sb0 = kc >> 8;
    // The first piece's loads go out right behind the first x loads.
    Q4kPiece cur;
    auto first_piece = [&] {
      if (j < P) load(cur, sb0 + (j >> 2));
    };

    __syncthreads();
    if (x_vec16) {
      const int v4 = kn >> 2;
      // one slot in flight: this kernel's M accumulators per row already use
      // the register file
      stage_slots<1>(
          tid, NT, M * v4,
          [&](int t) {
            const int m = t / v4;
            return *reinterpret_cast<const uint4*>(x + m * ldx + kc + 4 * (t - m * v4));
          },
          [&](int t, uint4 v) {
            const int m = t / v4;
            const int e = 4 * (t - m * v4);
            *reinterpret_cast<uint4*>(xs + m * XSTR + (e >> 6) * 68 + (e & 63)) = v;
          },
          first_piece);
    } else {
      first_piece();
      for (int t = tid; t < M * kn; t += NT) {
        const int m = t / kn, i = t - m * kn;
        xs[m * XSTR + (i >> 6) * 68 + (i & 63)] = x[m * ldx + kc + i];
      }
    }
    __syncthreads();
    const int nch = kn >> 5;
    for (int t = tid; t < M * nch; t += NT) {
      const int m = t / nch, c = t - m * nch;
      const float* src = xs + m * XSTR + (c >> 1) * 68 + 32 * (c & 1);
      float s = 0.f;
#pragma unroll
      for (int l = 0; l < 32; ++l) s += src[l];
      sx[m * KC32 + c] = s;
    }
    __syncthreads();

#pragma unroll 1
    for (int p = j; p < P; p += LPR) {
      Q4kPiece nxt;
      const bool more = p + LPR < P;
      if (more) load(nxt, sb0 + ((p + LPR) >> 2));

      float dva, mva, dvb, mvb;
      if constexpr (DSC) {
        dva = cur.ea.x; mva = cur.ea.y; dvb = cur.eb.x; mvb = cur.eb.y;
      } else {
        uint32_t s2, m2;
        scale_min_pair(cur.h.y, cur.h.z, cur.h.w, g, s2, m2);
        const float d = f16_to_f32(cur.h.x & 0xFFFFu);
        const float dmin = f16_to_f32(cur.h.x >> 16);
        dva = d * (float)(s2 & 0xFFu);
        dvb = d * (float)(s2 >> 8);
        mva = -(dmin * (float)(m2 & 0xFFu));
        mvb = -(dmin * (float)(m2 >> 8));
      }

      float pa[M], pb[M];
#pragma unroll
      for (int m = 0; m < M; ++m) pa[m] = pb[m] = 0.f;
      const float* xa = xs + p * 68;  // chunk 2g; chunk 2g+1 at +32
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t word = t < 4 ? word_of(cur.q0, t) : word_of(cur.q1, t - 4);
        const uint32_t w8 = word >> 8;
        // chunk 2g: low nibbles of bytes (0,2) and (1,3); chunk 2g+1: high nibbles
        const f16x2 A = bitcast<f16x2>((word & 0x000F000Fu) | magic) + m1024;
        const f16x2 C = bitcast<f16x2>((w8 & 0x000F000Fu) | magic) + m1024;
        const f16x2 B =
            __builtin_elementwise_fma(bitcast<f16x2>((word & 0x00F000F0u) | magic), sixteenth, m64);
        const f16x2 D =
            __builtin_elementwise_fma(bitcast<f16x2>((w8 & 0x00F000F0u) | magic), sixteenth, m64);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float4 xa4 = *reinterpret_cast<const float4*>(xa + m * XSTR + 4 * t);
          const float4 xb4 = *reinterpret_cast<const float4*>(xa + m * XSTR + 32 + 4 * t);
          float u = pa[m], v = pb[m];
          u = __builtin_fmaf((float)A.x, xa4.x, u);
          u = __builtin_fmaf((float)C.x, xa4.y, u);
          u = __builtin_fmaf((float)A.y, xa4.z, u);
          u = __builtin_fmaf((float)C.y, xa4.w, u);
          v = __builtin_fmaf((float)B.x, xb4.x, v);
          v = __builtin_fmaf((float)D.x, xb4.y, v);
          v = __builtin_fmaf((float)B.y, xb4.z, v);
          v = __builtin_fmaf((float)D.y, xb4.w, v);
          pa[m] = u;
          pb[m] = v;
        }
      }
      const int ca = 2 * p;  // chunk index within this K-chunk (= 8*(p/4) + 2g)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = acc[m];
        a = __builtin_fmaf(dva, pa[m], a);
        a = __builtin_fmaf(mva, sx[m * KC32 + ca], a);
        a = __builtin_fmaf(dvb, pb[m], a);
        a = __builtin_fmaf(mvb, sx[m * KC32 + ca + 1], a);
        acc[m] = a;
      }
      if (more) cur = nxt;
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float v = group_sum<LPR>(acc[m]);
    if (j == 0 && n < N) y[m * ldy + n] = v;
  }
}

// Persistent variant, used whenever x and its chunk sums fit in LDS: one
// resident round of workgroups; each stages x once and splits an equal,
// contiguous share of rows among its wavefronts.  A wavefront owns one row at
// a time (LPR = 64) and walks a flat sequence of (row, piece) items with a
// register ring of D items that crosses row boundaries.
// M = 1 with 1024-thread workgroups and a ring of at most 2 items asks for 64
// VGPRs (8 wavefronts per SIMD), so that two workgroups share a CU.
template <int M, int NT, bool DSC, bool STRIDED, int D>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(M == 1 && NT == 1024 && D <= 2 ? 8 : 1)))
void q4k_gemv_persistent(
    const float* __restrict__ x, int64_t ldx, const uint8_t* __restrict__ w,
    const float2* __restrict__ dsc, float* __restrict__ y, int64_t ldy, int N, int K,
    int x_vec16) {
  constexpr int NW = NT / kWave;  // wavefronts (rows in flight) per workgroup
  extern __shared__ float smem[];
  const int XSTR = (K >> 6) * 68;  // floats per x row in LDS (64 + 4 pad per piece)
  float* xs = smem;                // [M][K/64][68]
  float* sx = smem + M * XSTR;     // [M][K/32] chunk sums of x
  const int K32 = K >> 5;
  const int tid = threadIdx.x;
  const int wv = tid / kWave;
  const int j = tid % kWave;
  const int g = j & 3;
  // Row order: STRIDED gives wavefront gw rows gw, gw + GW, ... (GW = all
  // wavefronts of the grid), so the resident wavefronts sweep one compact
  // window; otherwise a workgroup takes a contiguous range of rows.
  const int b = STRIDED ? (int)blockIdx.x : xcd_tile(blockIdx.x, gridDim.x);
  const int r_begin = STRIDED ? 0 : (int)((int64_t)b * N / gridDim.x);
  const int r_end = STRIDED ? N : (int)((int64_t)(b + 1) * N / gridDim.x);
  const int first = STRIDED ? b * NW + wv : r_begin + wv;
  const int rstep = STRIDED ? (int)gridDim.x * NW : NW;
  const int nsb = K >> 8;
  const int P = K >> 6;                  // pieces per row
  const int PPI = (P + kWave - 1) / kWave;  // pieces per lane per row
  const int span = r_end - first;
  const int nrows = span > 0 ? (span + rstep - 1) / rstep : 0;  // rows of this wavefront
  const int nitems = nrows * PPI;

  const uint32_t magic = vreg_const(0x64006400u);
  const f16x2 m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const f16x2 m64 = {(_Float16)-64.0f, (_Float16)-64.0f};
  const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};

  auto load = [&](Q4kPiece& st, int row, int it) {
    row = row < N ? row : N - 1;  // a bound only: loaded items never pass the last row
    int p = j + kWave * it;
    p = p < P ? p : P - 1;  // idle lanes of a ragged last stride re-read a valid piece
    const uint32_t sb = (uint32_t)(p >> 2);
    const uint32_t bo = ((uint32_t)row * (uint32_t)nsb + sb) * (uint32_t)kQ4kBlockBytes;
    st.q0 = load16(w + (bo + 16u + 32u * g));
    st.q1 = load16(w + (bo + 32u + 32u * g));
    if constexpr (DSC) {
      const uint32_t c = sb * 8u + 2u * g;
      st.ea = load8f(dsc + (c * (uint32_t)N + (uint32_t)row));
      st.eb = load8f(dsc + ((c + 1u) * (uint32_t)N + (uint32_t)row));
    } else {
      st.h = load16(w + bo);
    }
  };
  auto advance = [&](int& row, int& it) {
    it = it + 1 == PPI ? 0 : it + 1;
    row = it == 0 ? row + rstep : row;
  };

  // D items in flight per lane: a register ring, each slot refilled as soon
  // as it is consumed, as long as items remain (the branch is uniform across
  // the wavefront).
  Q4kPiece ring[D];
  int lrow = first, lit = 0;  // next item to load
  auto fill_ring = [&] {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      if (k < nitems) load(ring[k], lrow, lit);
      advance(lrow, lit);
    }
  };

  // Stage x; the chunk sums come out of the same pass when x is 16-byte
  // aligned (8 consecutive lanes hold one 32-element chunk).  Decoding in
  // the kernel, a thread issues its weight loads once its x slots are in:
  // behind the weight stream of the whole grid, x would arrive late (measured
  // 0.2-0.5 us per call on the 7B layer shapes).  With the plane, the ring's
  // first loads go out right behind the x loads (measured better there).
  if (x_vec16) {
    // K is a multiple of 256, so M * K / 4 is a multiple of 64: whole
    // wavefronts stage together and the 8-lane DPP sum is well defined.
    const int v4 = K >> 2;
    stage_slots<2>(
        tid, NT, M * v4,
        [&](int t) {
          const int m = t / v4;
          return *reinterpret_cast<const uint4*>(x + m * ldx + 4 * (t - m * v4));
        },
        [&](int t, uint4 u) {
          const int m = t / v4, i = t - m * v4;
          const int e = 4 * i;
          const float4 v = bitcast<float4>(u);
          *reinterpret_cast<float4*>(xs + m * XSTR + (e >> 6) * 68 + (e & 63)) = v;
          const float part = group_sum<8>((v.x + v.y) + (v.z + v.w));
          if ((i & 7) == 0) sx[m * K32 + (i >> 3)] = part;
        },
        [&] {
          if constexpr (DSC) fill_ring();
        });
    if constexpr (!DSC) {
      __builtin_amdgcn_sched_barrier(0);
      fill_ring();
    }
    __syncthreads();
  } else {
    fill_ring();
    for (int t = tid; t < M * K; t += NT) {
      const int m = t / K, i = t - m * K;
      xs[m * XSTR + (i >> 6) * 68 + (i & 63)] = x[m * ldx + i];
    }
    __syncthreads();
    for (int t = tid; t < M * K32; t += NT) {
      const int m = t / K32, c = t - m * K32;
      const float* src = xs + m * XSTR + (c >> 1) * 68 + 32 * (c & 1);
      float sum = 0.f;
#pragma unroll
      for (int l = 0; l < 32; ++l) sum += src[l];
      sx[m * K32 + c] = sum;
    }
    __syncthreads();
  }

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.f;

  auto consume = [&](const Q4kPiece& cur, int row, int it) {
    const int p = j + kWave * it;
    if (p < P) {
      float dva, mva, dvb, mvb;
      if constexpr (DSC) {
        dva = cur.ea.x; mva = cur.ea.y; dvb = cur.eb.x; mvb = cur.eb.y;
      } else {
        uint32_t s2, m2;
        scale_min_pair(cur.h.y, cur.h.z, cur.h.w, g, s2, m2);
        const float d = f16_to_f32(cur.h.x & 0xFFFFu);
        const float dmin = f16_to_f32(cur.h.x >> 16);
        dva = d * (float)(s2 & 0xFFu);
        dvb = d * (float)(s2 >> 8);
        mva = -(dmin * (float)(m2 & 0xFFu));
        mvb = -(dmin * (float)(m2 >> 8));
      }
      float pa[M], pb[M];
#pragma unroll
      for (int m = 0; m < M; ++m) pa[m] = pb[m] = 0.f;
      const float* xa = xs + p * 68;  // chunk 2g; chunk 2g+1 at +32
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t word = t < 4 ? word_of(cur.q0, t) : word_of(cur.q1, t - 4);
        const uint32_t w8 = word >> 8;
        const f16x2 A = bitcast<f16x2>((word & 0x000F000Fu) | magic) + m1024;
        const f16x2 C = bitcast<f16x2>((w8 & 0x000F000Fu) | magic) + m1024;
        const f16x2 B = __builtin_elementwise_fma(
            bitcast<f16x2>((word & 0x00F000F0u) | magic), sixteenth, m64);
        const f16x2 D2 = __builtin_elementwise_fma(
            bitcast<f16x2>((w8 & 0x00F000F0u) | magic), sixteenth, m64);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float4 xa4 = *reinterpret_cast<const float4*>(xa + m * XSTR + 4 * t);
          const float4 xb4 = *reinterpret_cast<const float4*>(xa + m * XSTR + 32 + 4 * t);
          float u0 = pa[m], v0 = pb[m];
          u0 = __builtin_fmaf((float)A.x, xa4.x, u0);
          u0 = __builtin_fmaf((float)C.x, xa4.y, u0);
          u0 = __builtin_fmaf((float)A.y, xa4.z, u0);
          u0 = __builtin_fmaf((float)C.y, xa4.w, u0);
          v0 = __builtin_fmaf((float)B.x, xb4.x, v0);
          v0 = __builtin_fmaf((float)D2.x, xb4.y, v0);
          v0 = __builtin_fmaf((float)B.y, xb4.z, v0);
          v0 = __builtin_fmaf((float)D2.y, xb4.w, v0);
          pa[m] = u0;
          pb[m] = v0;
        }
      }
      const int ca = 2 * p;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a = acc[m];
        a = __builtin_fmaf(dva, pa[m], a);
        a = __builtin_fmaf(mva, sx[m * K32 + ca], a);
        a = __builtin_fmaf(dvb, pb[m], a);
        a = __builtin_fmaf(mvb, sx[m * K32 + ca + 1], a);
        acc[m] = a;
      }
    }
    if (it == PPI - 1) {  // row finished (uniform across the wavefront)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = group_sum<kWave>(acc[m]);
        acc[m] = 0.f;
        if (j == 0) y[m * ldy + row] = v;
      }
    }
  };

  int prow = first, pit = 0;  // next item to consume
  int u = 0;
#pragma unroll 1
  for (; u + D <= nitems; u += D) {
#pragma unroll
    for (int k = 0; k < D; ++k) {
      consume(ring[k], prow, pit);
      advance(prow, pit);
      if (u + k + D < nitems) load(ring[k], lrow, lit);
      advance(lrow, lit);
    }
  }
#pragma unroll
  for (int k = 0; k < D; ++k) {
    if (u + k < nitems) {
      consume(ring[k], prow, pit);
      advance(prow, pit);
    }
  }
}

// One thread per (super-block sb, row n), n fastest: decode the header once,
// write the eight (dv, mv) pairs of the super-block.  For a fixed chunk the
// writes of consecutive threads are consecutive float2s.
__global__ __launch_bounds__(kBlock) void q4k_plane_kernel(const uint8_t* __restrict__ w,
                                                           float2* __restrict__ dsc, int N,
                                                           int nsb) {
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (int64_t)N * nsb) return;
  const int n = (int)(t % N);
  const int sb = (int)(t / N);
  const uint4 h = *reinterpret_cast<const uint4*>(w + ((int64_t)n * nsb + sb) * kQ4kBlockBytes);
  const float d = f16_to_f32(h.x & 0xFFFFu);
  const float dmin = f16_to_f32(h.x >> 16);
  uint32_t sc[12];
  const uint32_t words[3] = {h.y, h.z, h.w};
#pragma unroll
  for (int i = 0; i < 12; ++i) sc[i] = (words[i >> 2] >> ((i & 3) * 8)) & 0xFFu;
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    uint32_t s, m;
    if (cc < 4) {
      s = sc[cc] & 63u;
      m = sc[cc + 4] & 63u;
    } else {
      s = (sc[cc + 4] & 15u) | ((sc[cc - 4] >> 6) << 4);
      m = (sc[cc + 4] >> 4) | ((sc[cc] >> 6) << 4);
    }
    const float dv = d * (float)s;        // one binary32 multiply (exact)
    const float mv = -(dmin * (float)m);  // exact negation: -0.0 when the product is 0
    dsc[((int64_t)sb * 8 + cc) * N + n] = make_float2(dv, mv);
  }
}

constexpr bool kQ4kStrided = false;

// One persistent launch with a ring of D items per lane: each wavefront gets
// D / PPI rows (at least one), so that all of its items can be in flight at
// once; the grid is capped at one resident round.
template <int M, int NT, int D>
hipError_t launch_persistent(const float* x, int64_t ldx, const uint8_t* w, const float2* dsc2,
                             float* y, int64_t ldy, int N, int K, int x_vec16, size_t full, int PPI,
                             hipStream_t stream) {
  auto kern = dsc2 ? q4k_gemv_persistent<M, NT, true, kQ4kStrided, D>
                   : q4k_gemv_persistent<M, NT, false, kQ4kStrided, D>;
  const hipError_t e = allow_lds(kern, full);
  if (e != hipSuccess) return e;
  const int cap = resident_workgroups(kern, NT, full);
  const int rows_per_wave = D / PPI > 1 ? D / PPI : 1;
  const int rows_per_wg = (NT / kWave) * rows_per_wave;
  const int want = (N + rows_per_wg - 1) / rows_per_wg;
  const int grid = want < cap ? want : cap;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), full, stream, x, ldx, w, dsc2, y, ldy, N, K,
                     x_vec16);
  note_launch(dsc2 ? kPathQ4kPersistentPlane : kPathQ4kPersistent, M, grid, NT, full);
  return hipGetLastError();
}

// Persistent kernel (1024 threads: 16 rows in flight per workgroup, x staged
// once) whenever x and its chunk sums fit in a workgroup's LDS (up to 160 KB);
// otherwise the K-chunked tiled kernel (256 threads: it keeps the full
// register file for its M accumulators per row).
template <int M>
hipError_t launch_m(const float* x, int64_t ldx, const uint8_t* w, const float* dsc, float* y,
                    int64_t ldy, int N, int K, hipStream_t stream) {
  constexpr int NT = 1024, LPR = 64, NT_TILED = 256;
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 4 == 0);
  const float2* dsc2 = reinterpret_cast<const float2*>(dsc);
  // x (68 floats per 64 elements) plus its chunk sums (2 floats per 64), fp32.
  const size_t full = (size_t)M * ((K / 64) * 68 + K / 32) * 4;
  if (full <= (size_t)kLdsMax) {
    // One item per lane in flight over a full grid measured faster than
    // deeper rings on fewer workgroups (4096 x 11008 and 11008 x 4096, M = 1).
    return launch_persistent<M, NT, 1>(x, ldx, w, dsc2, y, ldy, N, K, x_vec16, full, 1, stream);
  }
  // The tiled kernel is launched for at most 4 rows of x (launch_q4k_gemv
  // splits larger M into row groups), so only M <= 4 is instantiated.
  if constexpr (M > 4) {
    return hipErrorInvalidValue;
  } else {
    constexpr int S = NT_TILED / LPR;
    const int grid = (N + S - 1) / S;
    // KC a multiple of 256 (whole super-blocks) within the LDS budget.
    int KC = (kLdsBudget / (4 * 70 * M)) * 64 & ~255;
    if (KC > K) KC = K;
    const size_t shmem = (size_t)M * ((KC / 64) * 68 + KC / 32) * 4;
    if (dsc)
      hipLaunchKernelGGL((q4k_gemv_kernel<M, LPR, NT_TILED, true>), dim3(grid), dim3(NT_TILED),
                         shmem, stream, x, ldx, w, dsc2, y, ldy, N, K, KC, x_vec16);
    else
      hipLaunchKernelGGL((q4k_gemv_kernel<M, LPR, NT_TILED, false>), dim3(grid), dim3(NT_TILED),
                         shmem, stream, x, ldx, w, nullptr, y, ldy, N, K, KC, x_vec16);
    note_launch(dsc ? kPathQ4kTiledPlane : kPathQ4kTiled, M, grid, NT_TILED, shmem);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_q4k_gemv(const float* x, int64_t ldx, const uint8_t* w, const float* dsc,
                           float* y, int64_t ldy, int M, int N, int K, hipStream_t stream) {
  // When x (all M rows) does not fit in a workgroup's LDS but a few rows do,
  // run the persistent kernel on groups of rows: each group re-reads the
  // weights, which beats restaging x for every 4 rows in the tiled kernel.
  // Rows too long for LDS go to the K-chunked tiled kernel, at most 4 rows of
  // x at a time (its per-row accumulators would spill beyond that).
  const size_t per_row = ((size_t)(K / 64) * 68 + K / 32) * 4;
  const int mfit = (size_t)kLdsMax >= per_row ? (int)((size_t)kLdsMax / per_row) : (M < 4 ? M : 4);
  if (M > mfit) {
    for (int m0 = 0; m0 < M; m0 += mfit) {
      const int mm = M - m0 < mfit ? M - m0 : mfit;
      const hipError_t e = launch_q4k_gemv(x + m0 * ldx, ldx, w, dsc, y + m0 * ldy, ldy, mm, N,
                                           K, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  switch (M) {
#define QG_CASE(MM) \
  case MM:          \
    return launch_m<MM>(x, ldx, w, dsc, y, ldy, N, K, stream);
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_q4k_build_plane(const uint8_t* w, float* dsc, int N, int K, hipStream_t stream) {
  const int nsb = K / 256;
  const int64_t total = (int64_t)N * nsb;
  const int grid = (int)((total + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(q4k_plane_kernel, dim3(grid), dim3(kBlock), 0, stream, w,
                     reinterpret_cast<float2*>(dsc), N, nsb);
  note_launch(kPathQ4kPlaneBuild, 0, grid, kBlock, 0);
  return hipGetLastError();
}

}  // namespace qg
