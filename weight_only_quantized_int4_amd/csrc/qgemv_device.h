// qgemv_device.h -- device-side helpers shared by the gfx950 GEMV kernels.
//
// Everything here is CDNA4 code: 64-wide wavefronts, packed-f16 VOP3P math,
// v_dot2 instructions, DPP and lane-swap cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // threads per workgroup (4 wavefronts)
constexpr int kXcds = 8;     // MI355X: 8 accelerator complex dies, 32 CUs each

template <typename T, typename U>
__device__ __forceinline__ T bitcast(U u) {
  static_assert(sizeof(T) == sizeof(U), "size");
  return __builtin_bit_cast(T, u);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)bitcast<_Float16>((uint16_t)bits16);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Workgroups are handed to the XCDs round-robin (workgroup id mod 8).  Give
// each XCD one contiguous range of tiles instead, so that tiles which share
// cache lines (neighbouring rows of a plane, the tail of one row and the head
// of the next) are served by the same L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_tile(int bid, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return xcd * q + (xcd < r ? xcd : r) + idx;
}

// A 32-bit constant the compiler must keep in a VGPR.  gfx9 VOP3 encodings
// cannot carry a literal, so (word & mask) | magic only becomes a single
// v_and_or_b32 when one of the two constants already lives in a register.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(c));
  return v;
}

// A register-to-register copy the compiler cannot fold away: gives a value a
// register of its own (for instructions that overwrite their operands).
__device__ __forceinline__ uint32_t vreg_copy(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// Stage `count` 16-byte slots into LDS: slot t is read by load(t) and
// written by store(t, v).  Each thread keeps up to U independent loads in
// flight before its first wait, so staging costs one memory round trip per U
// slots of a thread instead of one per slot.
//
// `first` runs once per thread right after the first round of x loads is
// issued and before anything waits on them: kernels issue their first weight
// loads there.  Loads complete in issue order as far as the wait counter is
// concerned, so weight loads issued before the x loads would make the first
// x store wait for the weights (a full HBM round trip) as well.
//
// Loads and stores are unconditional (a slot index past `count` re-reads and
// rewrites the last slot with the same value; count >= 1): no branch sits
// between the x loads and `first`'s loads and nothing sinks the x loads
// behind them, so the wait before the first store covers the x loads only.
// A store that combines lanes (DPP) sees whole wavefronts either in range or
// all clamped when `count` is a multiple of 64.
template <int U, typename Load, typename Store, typename First>
__device__ __forceinline__ void stage_slots(int tid, int nthreads, int count, Load load,
                                            Store store, First first) {
  bool pending = true;
  for (int t0 = tid; t0 < count || pending; t0 += nthreads * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * nthreads;
      v[u] = load(t < count ? t : count - 1);
    }
    if (pending) {
      // keep the scheduler from moving x loads behind `first`'s loads (or
      // x stores ahead of them)
      __builtin_amdgcn_sched_barrier(0);
      first();
      __builtin_amdgcn_sched_barrier(0);
      pending = false;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * nthreads;
      store(t < count ? t : count - 1, v[u]);
    }
  }
}

template <int U, typename Load, typename Store>
__device__ __forceinline__ void stage_slots(int tid, int nthreads, int count, Load load,
                                            Store store) {
  stage_slots<U>(tid, nthreads, count, load, store, [] {});
}

// DPP lane permutes within a row of 16 lanes.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// v + the value of lane (lane ^ S), S = 16 or 32, in every lane: one
// v_permlane16_swap / v_permlane32_swap (a VALU lane exchange, no LDS) and
// one add.  The swap of v with itself leaves each lane's own value in one
// result and its partner's in the other; their sum is the same in both lanes
// of a pair (addition commutes).
template <int S>
__device__ __forceinline__ float swap_add(float v) {
  static_assert(S == 16 || S == 32, "lane distance");
  const uint32_t u = __float_as_uint(v);
  if constexpr (S == 16) {
    const auto h = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
  } else {
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
}

// Sum over aligned groups of G consecutive lanes (G a power of two <= 64);
// every lane of the group receives the group total.  Steps inside a 16-lane
// row use DPP (fused into v_add_f32_dpp); larger groups finish with lane
// swaps.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f32<kDppMirror>(v);
  if constexpr (G >= 32) v = swap_add<16>(v);
  if constexpr (G >= 64) v = swap_add<32>(v);
  return v;
}

// Sums NV values per thread over aligned groups of G consecutive threads of a
// kBlock-thread workgroup.  G <= 64: cross-lane DPP/shuffles, every lane of a
// group gets the totals.  G = 128 or 256 (a row spread over 2 or 4
// wavefronts): wavefront totals meet in `red` (LDS, kBlock/64 * NV floats);
// only the first thread of each group gets the totals.  Every thread of the
// workgroup must call it (it contains barriers when G > 64).
template <int G, int NV>
__device__ __forceinline__ void group_sum_wide(float (&v)[NV], float* red) {
  if constexpr (G <= kWave) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = group_sum<G>(v[i]);
  } else {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = group_sum<kWave>(v[i]);
    __syncthreads();  // red may still be read from a previous call
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < NV; ++i) red[wave * NV + i] = v[i];
    __syncthreads();
    if (threadIdx.x % G == 0)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < G / kWave; ++k) t += red[(wave + k) * NV + i];
        v[i] = t;
      }
  }
}

// Round-to-nearest-even store of an fp32 result in the output type.
// y_type: 0 = fp16, 1 = bf16, 2 = fp32 (the qg_dtype values).
__device__ __forceinline__ void store_out(void* y, int64_t idx, float v, int y_type) {
  if (y_type == 0)
    static_cast<_Float16*>(y)[idx] = (_Float16)v;
  else if (y_type == 1)
    static_cast<__bf16*>(y)[idx] = (__bf16)v;
  else
    static_cast<float*>(y)[idx] = v;
}

// 128-bit weight-stream load.  The weights are read exactly once per call, so
// they are loaded non-temporally: they should not displace x, the scales or
// the output in the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Plain 128-bit load, for streams whose cache lines are touched by more than
// one load instruction (the q4_K header and quants share lines).
__device__ __forceinline__ uint4 load16(const void* p) {
  const u32x4 v = *static_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float2 load8f(const float2* p) {
  const f32x2 v = *reinterpret_cast<const f32x2*>(p);
  return make_float2(v.x, v.y);
}

}  // namespace qg
