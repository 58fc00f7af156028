// q4k_mmq.hip -- q4_K prefill on the int8 matrix cores (gfx950).
//
// "62 . r59 -- q4_K W_dsc plane + riders": the prefill path quantizes the
// activations to 8 bits in a prepass (section 3.2, the dispatch arm), takes
// integer dot products of the raw 4-bit quants with them, and rescales each
// (chunk, row) product with the pre-decoded coefficients of the W_dsc plane,
// (d*sc, -dmin*m) (sections 2.1 and 2.2):
//     y[t,n] = sum_c d_a[t,c] * (dv[n,c] * sum_{k in c} q_w[n,k]*q_a[t,k]
//                               + mv[n,c] * sum_{k in c} q_a[t,k])
// The page leaves the activation rule open; the reading used here is the
// plain symmetric one per block of 32 (one weight chunk): d = amax/127 and
// q = x/d rounded half away from zero, both in binary32 (correctly rounded
// divisions), and an all-zero block gives d = 0 and q = 0.
//
// Prepass: 8 lanes per block of 32 activations (4 each), group max and sum
// by lane shuffles; writes the codes [T][K] and (d, d * sum q) per block.
//
// Product: v_mfma_i32_16x16x32_i8 -- A = 16 activation rows x 32 k (one
// chunk), B = 32 k x 16 weight rows, D = 16 x 16 exact int32 sums.  Lane l
// holds A[l%16][8(l/16)..+8], B[8(l/16)..+8][l%16] and D[4(l/16)+i][l%16].
// The 4-bit quants need no reordering: chunk 2g (2g+1) of a super-block is the
// low (high) nibble of quant bytes 32g..32g+31, so lane group j takes bytes
// 32g+8j..+8 for both chunks, and the A operand takes the activations of the
// same k.  A wavefront owns 16 activation rows x 64 weight rows (1 x 4 MFMA
// blocks); a workgroup of 4 x 2 wavefronts covers 64 activation rows x 128
// weight rows, stages one super-block (256 k) of its codes, quant bytes (split
// into low and high nibbles on the way into LDS), plane entries and activation
// scales in LDS and prefetches the next super-block into registers meanwhile.
// The dv term is rescaled in fp32 per chunk and output on the vector ALUs; the
// mv term, a product over chunks of (d_a * sum q_a) and mv, runs on the fp32
// matrix cores (v_mfma_f32_16x16x4f32, four chunks per instruction) into
// accumulators of its own, added at the end.  Vector-ALU issue is the limit of
// this kernel; both moves take work off it (measured 3-11% faster each).
#include <mutex>

#include "qgemv.h"
#include "qgemv_device.h"
#include "qgemv_launch.h"

// Workspace of the prefill entry point that allocates nothing
// (qgemm_q4k_mmq_noalloc): the 8-bit codes and activation scales live in this
// file-scope device array instead of a caller-owned buffer.  Every GPU the
// library runs on holds its own copy, from the library's load until the
// process ends.  Host code must never pass the array's name to a kernel (on
// the host it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns for the current device (mmq_static_scratch).
static __device__ __align__(256) uint8_t scratch[QG_MMQ_NOALLOC_SCRATCH_BYTES];

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ4kBlockBytes = 144;  // d, dmin (f16), 12 scale bytes, 128 quant bytes
constexpr int kPrepassThreads = 256;

// ---------------------------------------------------------------------------
// Prepass
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kPrepassThreads) void q8_quantize_kernel(
    const float* __restrict__ x, int64_t ldx, int8_t* __restrict__ qa, float2* __restrict__ sda,
    int T, int K, int x_vec16) {
  const int64_t nblk = (int64_t)T * (K >> 5);
  const int64_t blk = ((int64_t)blockIdx.x * kPrepassThreads + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  // Whole groups of 8 lanes are in or out of range (8 divides the block).
  if (blk >= nblk) return;
  const int bpr = K >> 5;
  const int t = (int)(blk / bpr);
  const int b = (int)(blk - (int64_t)t * bpr);
  const float* src = x + (int64_t)t * ldx + 32 * b + 4 * j;
  float v[4];
  if (x_vec16) {
    const float4 f = *reinterpret_cast<const float4*>(src);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[i];
  }
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 8));
  const float d = amax / 127.0f;  // correctly rounded binary32 division
  int q[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[i] = d == 0.0f ? 0 : (int)roundf(v[i] / d);  // half away from zero
    sum += q[i];
  }
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) sum += __shfl_xor(sum, s, 8);
  const uint32_t packed = (uint32_t)(q[0] & 0xFF) | ((uint32_t)(q[1] & 0xFF) << 8) |
                          ((uint32_t)(q[2] & 0xFF) << 16) | ((uint32_t)(q[3] & 0xFF) << 24);
  *reinterpret_cast<uint32_t*>(qa + (int64_t)t * K + 32 * b + 4 * j) = packed;
  if (j == 0) sda[blk] = make_float2(d, d * (float)sum);
}

// ---------------------------------------------------------------------------
// Product
// ---------------------------------------------------------------------------

constexpr int kWaveRows = 64;      // weight rows per wavefront (4 MFMA blocks)
constexpr int kRowWaves = 2;       // wavefronts along the weight rows
constexpr int kBN = kWaveRows * kRowWaves;  // weight rows per workgroup
constexpr int kAStride = 256 + 16;  // LDS bytes per staged activation row (one super-block)
constexpr int kBStride = 256 + 16;  // LDS bytes per staged weight row (128 low, 128 high nibbles)

// WT wavefronts along the activation rows, each with TB blocks of 16 rows.
template <int WT, int TB>
struct MmqShape {
  static constexpr int kWaveTokens = 16 * TB;  // activation rows per wavefront
  static constexpr int kThreads = WT * kRowWaves * kWave;
  static constexpr int kBT = WT * kWaveTokens;  // activation rows per workgroup
  static constexpr int kABytes = kBT * kAStride;
  static constexpr int kBBytes = kBN * kBStride;
  static constexpr int kPBytes = 8 * kBN * 8;   // plane: [chunk][row] float2
  static constexpr int kSBytes = 8 * kBT * 8;   // activation scales: [chunk][token] float2
  static constexpr int kLds = kABytes + kBBytes + kPBytes + kSBytes;
  // Register prefetch per thread: 16-byte pieces of A and B, 8-byte plane
  // entries, 16-byte pieces of the activation scales (two chunks each).
  static constexpr int kAPieces = kBT * 16 / kThreads;
  static constexpr int kBPieces = kBN * 8 / kThreads;
  static constexpr int kPEntries = 8 * kBN / kThreads;
  static constexpr int kSPieces = (kBT * 4 + kThreads - 1) / kThreads;
  static_assert(kBT * 16 % kThreads == 0 && kBN * 8 % kThreads == 0 && 8 * kBN % kThreads == 0,
                "staging pieces must divide evenly");
};

template <int WT, int TB>
__global__ __launch_bounds__((MmqShape<WT, TB>::kThreads)) void q4k_mmq_kernel(
    const int8_t* __restrict__ qa, const float2* __restrict__ sda, const uint8_t* __restrict__ w,
    const float2* __restrict__ dsc, float* __restrict__ y, int64_t ldy, int T, int N, int K) {
  using S = MmqShape<WT, TB>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char* As = lds;
  char* Bs = As + S::kABytes;
  float2* Ps = reinterpret_cast<float2*>(Bs + S::kBBytes);
  float2* Ss = reinterpret_cast<float2*>(reinterpret_cast<char*>(Ps) + S::kPBytes);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wt = wave / kRowWaves, wn = wave % kRowWaves;
  const int n16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kBN;        // first weight row of the tile
  const int t0 = blockIdx.y * S::kBT;     // first activation row of the tile
  const int nsb = K >> 8;                 // super-blocks
  const int nchunk = K >> 5;
  const uint32_t wrow = (uint32_t)nsb * kQ4kBlockBytes;

  // ---- global -> registers (one super-block), rows and tokens clamped ----
  // (native vector types: arrays of the HIP uint4 struct were placed in
  // scratch memory, which serialized every prefetch load)
  u32x4 ra[S::kAPieces], rb[S::kBPieces], rs[S::kSPieces];
  float2 rp[S::kPEntries];
  auto fetch = [&](int sb) {
#pragma unroll
    for (int i = 0; i < S::kAPieces; ++i) {
      const int p = tid + i * S::kThreads;
      const int tok = min(t0 + (p >> 4), T - 1);
      ra[i] = *reinterpret_cast<const u32x4*>(qa + (int64_t)tok * K + sb * 256 + (p & 15) * 16);
    }
#pragma unroll
    for (int i = 0; i < S::kBPieces; ++i) {
      const int p = tid + i * S::kThreads;
      const int row = min(n0 + (p >> 3), N - 1);
      rb[i] = *reinterpret_cast<const u32x4*>(w + (row * wrow + sb * kQ4kBlockBytes + 16 + (p & 7) * 16));
    }
#pragma unroll
    for (int i = 0; i < S::kPEntries; ++i) {
      const int p = tid + i * S::kThreads;  // p = cc * kBN + r
      const int row = min(n0 + (p % kBN), N - 1);
      rp[i] = dsc[(int64_t)(sb * 8 + p / kBN) * N + row];
    }
#pragma unroll
    for (int i = 0; i < S::kSPieces; ++i) {
      const int p = min(tid + i * S::kThreads, S::kBT * 4 - 1);  // p = token * 4 + pair
      const int tok = min(t0 + (p >> 2), T - 1);
      rs[i] = *reinterpret_cast<const u32x4*>(sda + (int64_t)tok * nchunk + sb * 8 + (p & 3) * 2);
    }
  };
  // ---- registers -> LDS ----
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < S::kAPieces; ++i) {
      const int p = tid + i * S::kThreads;
      *reinterpret_cast<u32x4*>(As + (p >> 4) * kAStride + (p & 15) * 16) = ra[i];
    }
    // the quant bytes split once per super-block into their low nibbles
    // (chunks 2g) and high nibbles (chunks 2g+1), one byte per 4-bit value
#pragma unroll
    for (int i = 0; i < S::kBPieces; ++i) {
      const int p = tid + i * S::kThreads;
      char* dst = Bs + (p >> 3) * kBStride + (p & 7) * 16;
      *reinterpret_cast<u32x4*>(dst) = rb[i] & 0x0F0F0F0Fu;
      *reinterpret_cast<u32x4*>(dst + 128) = (rb[i] >> 4) & 0x0F0F0F0Fu;
    }
#pragma unroll
    for (int i = 0; i < S::kPEntries; ++i) Ps[tid + i * S::kThreads] = rp[i];
#pragma unroll
    for (int i = 0; i < S::kSPieces; ++i) {
      const int p = tid + i * S::kThreads;
      if (p < S::kBT * 4) {
        const int tok = p >> 2, c = (p & 3) * 2;
        Ss[c * S::kBT + tok] = make_float2(__uint_as_float(rs[i][0]), __uint_as_float(rs[i][1]));
        Ss[(c + 1) * S::kBT + tok] = make_float2(__uint_as_float(rs[i][2]), __uint_as_float(rs[i][3]));
      }
    }
  };

  f32x4 acc[TB][4], accm[TB][4];
#pragma unroll
  for (int a = 0; a < TB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
      accm[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const i32x4 zero = {0, 0, 0, 0};

  // LDS byte offsets of this lane's operands
  const int a_off0 = (wt * S::kWaveTokens + n16) * kAStride + 8 * g;  // + 16 * tb rows, + 32 * cc
  const int b_off0 = (wn * kWaveRows + n16) * kBStride + 8 * g;      // + 16 * rb rows, + 32 * pair
  const int s_tok0 = wt * S::kWaveTokens + 4 * g;                     // + 16 * tb, tokens +0..3
  const int p_row0 = wn * kWaveRows + n16;                            // + 16 * rb

  fetch(0);
  stash();
  __syncthreads();
#pragma unroll 1
  for (int sb = 0; sb < nsb; ++sb) {
    fetch(sb + 1 < nsb ? sb + 1 : sb);  // unconditional: the last round re-reads its own
    // mv term: sum over the super-block's chunks c of (d_a * sum q_a)[t, c] *
    // mv[n, c], four chunks per fp32 MFMA (A[t][k] = chunk 4hh+k of token t,
    // B[k][n] = the same chunk of weight row n), accumulated apart from the
    // integer products' rescale
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c = 4 * hh + g;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const float am = Ss[c * S::kBT + wt * S::kWaveTokens + tb * 16 + n16].y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float bm = Ps[c * kBN + p_row0 + r * 16].y;
          accm[tb][r] = __builtin_amdgcn_mfma_f32_16x16x4f32(am, bm, accm[tb][r], 0, 0, 0);
        }
      }
    }
#pragma unroll 1
    for (int pair = 0; pair < 4; ++pair) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int cc = pair * 2 + h;
        int64_t av[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          av[tb] = *reinterpret_cast<const int64_t*>(As + a_off0 + tb * 16 * kAStride + cc * 32);
        int64_t bv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          bv[r] = *reinterpret_cast<const int64_t*>(Bs + b_off0 + r * 16 * kBStride + h * 128 + pair * 32);
        i32x4 dd[TB][4];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            dd[tb][r] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[tb], bv[r], zero, 0, 0, 0);
        float2 pc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pc[r] = Ps[cc * kBN + p_row0 + r * 16];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const float4* sp = reinterpret_cast<const float4*>(Ss + cc * S::kBT + s_tok0 + tb * 16);
          const float4 s01 = sp[0], s23 = sp[1];
          const float da[4] = {s01.x, s01.z, s23.x, s23.z};
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[tb][r][i] = __builtin_fmaf(da[i] * pc[r].x, (float)dd[tb][r][i], acc[tb][r][i]);
        }
        // keep the next chunk's operands and products from being hoisted here
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // every wavefront is done with this super-block
    if (sb + 1 < nsb) {
      stash();
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds activation rows 4g..4g+3 of weight row n16 ----
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = n0 + wn * kWaveRows + r * 16 + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + wt * S::kWaveTokens + tb * 16 + 4 * g + i;
        if (tok < T && row < N) y[(int64_t)tok * ldy + row] = acc[tb][r][i] + accm[tb][r][i];
      }
    }
}

template <int WT, int TB>
hipError_t launch_mmq_wt(const int8_t* qa, const float2* sda, const uint8_t* w, const float2* dsc,
                         float* y, int64_t ldy, int T, int N, int K, hipStream_t stream) {
  using S = MmqShape<WT, TB>;
  const dim3 grid((N + kBN - 1) / kBN, (T + S::kBT - 1) / S::kBT);
  auto kern = q4k_mmq_kernel<WT, TB>;
  const hipError_t e = allow_lds(kern, S::kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(S::kThreads), S::kLds, stream, qa, sda, w, dsc, y, ldy, T, N,
                     K);
  note_launch(kPathQ4kMmq, T, (int)(grid.x * grid.y), S::kThreads, S::kLds);
  return hipGetLastError();
}

}  // namespace

hipError_t mmq_static_scratch(void** ptr) {
  // Looked up once per device, with that device current; kept per device
  // (each GPU has the array at an address of its own).
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t q8_workspace_codes_bytes(int64_t T, int64_t K) {
  return ((size_t)T * (size_t)K + 255) & ~(size_t)255;
}

hipError_t launch_q8_quantize(const float* x, int64_t ldx, int8_t* qa, float* sda, int T, int K,
                              hipStream_t stream) {
  const int64_t threads = (int64_t)T * (K / 32) * 8;
  const int grid = (int)((threads + kPrepassThreads - 1) / kPrepassThreads);
  const int x_vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0) && (ldx % 4 == 0);
  hipLaunchKernelGGL(q8_quantize_kernel, dim3(grid), dim3(kPrepassThreads), 0, stream, x, ldx, qa,
                     reinterpret_cast<float2*>(sda), T, K, x_vec16);
  note_launch(kPathQ8Quantize, T, grid, kPrepassThreads, 0);
  return hipGetLastError();
}

hipError_t launch_q4k_mmq(const int8_t* qa, const float* sda, const uint8_t* w, const float* dsc,
                          float* y, int64_t ldy, int T, int N, int K, hipStream_t stream) {
  const float2* s2 = reinterpret_cast<const float2*>(sda);
  const float2* p2 = reinterpret_cast<const float2*>(dsc);
  // One block of 16 activation rows per wavefront (TB = 1) and 4 wavefronts
  // along the activation rows measured fastest for T = 8 .. 2048 on the 7B
  // layer shapes (against 2 blocks per wavefront and 2 wavefronts: twice the
  // wavefronts for the same work, ~115 instead of 157-184 VGPRs, and the stalls
  // of one wavefront overlap another's; 4096 x 4096 at T = 512: 81 -> 61 us).
  return launch_mmq_wt<4, 1>(qa, s2, w, p2, y, ldy, T, N, K, stream);
}

}  // namespace qg
