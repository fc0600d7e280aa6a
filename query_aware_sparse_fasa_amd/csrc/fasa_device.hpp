// Device helpers shared by the FASA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fasa {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Load 8 consecutive cache elements (16-byte aligned for bf16, 32-byte for fp32)
// and widen them to fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Eight cache elements as loaded (before widening): one 16-byte vector for bf16,
// two for fp32.  Keeping loads raw halves the registers held while they are in flight.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  // Streaming load: data read once (the slab, K/V rows no other workgroup
  // reads) is marked non-temporal so it does not displace reused lines.
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const u4v t = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
    v = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  // fp32 caches keep ordinary loads (the non-temporal form measured slower
  // on the small fp32 workloads).
  __device__ __forceinline__ void load_nt(const float* p) { load(p); }
  __device__ __forceinline__ void unpack(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

__device__ __forceinline__ float to_f32(uint16_t h) { return bf16_to_f32(h); }
__device__ __forceinline__ float to_f32(float f) { return f; }

// Order-preserving map of an fp32 score to an unsigned key: a larger score
// gives a larger key; -0.0 is first turned into +0.0 so the two tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// t_b clamped into what the buffers can hold.
__device__ __forceinline__ int clamp_len(int t, int max_t, int max_blocks) {
  t = t < 0 ? 0 : t;
  t = t > max_t ? max_t : t;
  const int lim = max_blocks * 256;
  return t > lim ? lim : t;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of m in lanes below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
}

// DPP (data-parallel primitive) lane moves: a VALU operand modifier, no LDS
// round trip.  update_dpp(old, src, ctrl, row_mask, bank_mask, bound_ctrl)
// returns old in lanes whose source lane is out of range or masked off.
constexpr int kDppRowShr = 0x110;      // + n: lane i reads lane i-n of its 16-lane row
constexpr int kDppRowRor = 0x120;      // + n: rotate right by n inside the row
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row feeds the next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 feeds rows 2 and 3

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each
// 16-lane row (shifts 1, 2, 4, 8), then row totals carried across rows.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr + 1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr + 2, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr + 4, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr + 8, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// Value of lane 63 (the wave total after an inclusive scan), as a scalar.
__device__ __forceinline__ uint32_t wave_last(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the 16 lanes of each row, returned in every lane of the row
// (rotations by 8, 4, 2, 1 inside the row).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor + 8, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor + 4, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor + 2, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor + 1, 0xF, 0xF, false));
  return v;
}

// Workgroup coordinates in XCD-aware order.  The dispatcher hands the
// workgroup with linear id L (x fastest) to XCD L mod 8, so consecutive
// workgroups land on different XCDs and each XCD has its own L2.  Renumbering
// L to l = (L mod 8) * (N / 8) + L / 8 (N workgroups; the last N mod 8 keep
// their number) gives every XCD one contiguous run of logical ids.  Every
// launch of a step orders its grid with the (sequence, kv head) unit as the
// slow index, so a unit's workgroups share one L2 (the query heads of a group
// reading the same rows, the chunks of one score row), and with N a multiple
// of 8 a unit stays on the same XCD from launch to launch.  A bijection on
// [0, N): every logical workgroup still runs exactly once.
struct WgCoord {
  int x, y, z;
};
__device__ __forceinline__ WgCoord xcd_grouped() {
  const uint32_t X = gridDim.x, Y = gridDim.y;
  const uint32_t n = X * Y * gridDim.z;
  const uint32_t L = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
  const uint32_t per = n >> 3;
  const uint32_t l = L < (per << 3) ? (L & 7u) * per + (L >> 3) : L;
  const uint32_t yz = l / X;
  return WgCoord{int(l - yz * X), int(yz % Y), int(yz / Y)};
}

// Hand-off between the workgroups of one launch: the last one to arrive on
// `counter` (which must start at zero) sees everything the others stored before
// arriving.  Every wave waits until its own stores are acknowledged, the
// workgroup meets at a barrier, then one thread writes the XCD's L2 back
// (agent-scope release), waits for that, and moves the counter; the thread that
// moves it to n invalidates its stale cached lines (agent-scope acquire) before
// the barrier that hands the verdict to the rest of the workgroup.  One L2
// write-back per workgroup, and one invalidate per hand-off.  Returns true in
// every thread of the last workgroup.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n, uint32_t* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
    const bool last = atomicAdd(counter, 1u) == n - 1u;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *lds_flag = last ? 1u : 0u;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

}  // namespace fasa
