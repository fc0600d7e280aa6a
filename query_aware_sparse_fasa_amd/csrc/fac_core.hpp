// Per-wave core of FAC (Focused Attention Computation): online softmax over a run
// of selected rows for up to HG query heads of one kv head.
//
// out_h = softmax(q_h K_T^T * scale) V_T over the selected rows at their original
// positions (paper-graph-ui review of FASA, section 3.4 "Online Stage 2: Focused
// Attention Computation (FAC)").  A wave takes four rows per step: 16 lanes per
// row, 8 channels per lane.  Every K/V row is loaded once and serves all HG
// heads.  The state per head is (running max m, running sum l, acc[8 channels])
// in each of the four 16-lane row groups; fold_row_groups() combines them.
//
// Precision: bf16 caches accumulate in fp32 (logits pre-scaled by log2(e),
// exponentiated with exp2); fp32 caches run logits, softmax and the weighted sum
// in fp64 (fp32 logits of magnitude ~30 carry ~2e-6 absolute error, enough to
// move a fp32 output by more than 1e-5).
#pragma once

#include <math.h>

#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {

template <typename Acc>
__device__ __forceinline__ Acc fexp(Acc x);
template <>
__device__ __forceinline__ float fexp<float>(float x) { return exp2f(x); }
template <>
__device__ __forceinline__ double fexp<double>(double x) { return exp(x); }

template <typename Acc>
__device__ __forceinline__ Acc neg_inf();
template <>
__device__ __forceinline__ float neg_inf<float>() { return -INFINITY; }
template <>
__device__ __forceinline__ double neg_inf<double>() { return -(double)INFINITY; }

__device__ __forceinline__ float shfl_xor_acc(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shfl_xor_acc(double v, int m) { return __shfl_xor(v, m, 64); }

// Sum over the 16 lanes of a row group, in every lane of it: DPP rotations for
// fp32, cross-lane shuffles for fp64.
__device__ __forceinline__ float row_sum(float v) { return row16_sum(v); }
__device__ __forceinline__ double row_sum(double v) {
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Merge weight of a partial state with max mi against the global max M
// (0 for an empty partial).
template <typename Acc>
__device__ __forceinline__ Acc merge_weight(Acc mi, Acc M) {
  return (mi == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(mi - M);
}

template <typename T, typename Acc, int HG>
struct FacWave {
  Acc qv[HG][8];
  Acc m[HG], l[HG], acc[HG][8];

  // Query slices of heads h_first .. h_first+nh-1 (rows of q, each kHeadDim long),
  // pre-scaled; unused head slots are zero.  Loads are unconditional.
  __device__ __forceinline__ void init(const T* q_head0, int nh, float scale) {
    const int sub = threadIdx.x & 15;
    Raw8<T> qr[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) qr[hh].load(q_head0 + int64_t(min(hh, nh - 1)) * kHeadDim + 8 * sub);
    const Acc qscale = sizeof(Acc) == 4 ? Acc(scale) * Acc(1.4426950408889634) : Acc(scale);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      m[hh] = neg_inf<Acc>();
      l[hh] = Acc(0);
      float x[8];
      qr[hh].unpack(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[hh][e] = Acc(0);
        qv[hh][e] = (hh < nh) ? Acc(x[e]) * qscale : Acc(0);
      }
    }
  }

  // Rows r0 .. r1-1 of the selection.  lane_offset(r) returns the element offset
  // of row r inside the kv head's pool slice, or -1 for an invalid row; it is
  // called once per 64 rows with r = base + lane (two dependent loads at most).
  // Invalid rows load a valid row of the wave instead and are then ignored, so
  // the row loads need no branch and go out together.
  template <typename LaneOffset>
  __device__ __forceinline__ void run(int r0, int r1, LaneOffset lane_offset, const T* kbase,
                                      const T* vbase) {
    const int lane = threadIdx.x & 63, rg = lane >> 4, sub = lane & 15;
    kbase += 8 * sub;
    vbase += 8 * sub;
    constexpr int U = 2;   // row quads whose loads are in flight together
    for (int base = r0; base < r1; base += 64) {   // wave-uniform
      const int64_t my_off = lane_offset(base + lane);
      const uint64_t ok = __ballot(my_off >= 0);
      if (ok == 0) continue;
      const int64_t dummy = __shfl(my_off, __ffsll((unsigned long long)ok) - 1, 64);
      const int nrows = min(64, r1 - base);
      for (int q4 = 0; q4 < nrows; q4 += 4 * U) {
        Raw8<T> kr[U], vr[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int src = q4 + 4 * u + rg;   // lane holding this row's offset
          const int64_t off = __shfl(my_off, src < 64 ? src : 0, 64);
          valid[u] = (src < nrows) && off >= 0;
          const int64_t o = valid[u] ? off : dummy;
          kr[u].load(kbase + o);
          vr[u].load(vbase + o);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float kx[8], vx[8];
          kr[u].unpack(kx);
          vr[u].unpack(vx);
          Acc z[HG];
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            Acc s = Acc(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fma(qv[hh][e], Acc(kx[e]), s);
            z[hh] = row_sum(s);
          }
          if (valid[u]) {
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
              const Acc mn = fmax(m[hh], z[hh]);
              const Acc corr = fexp<Acc>(m[hh] - mn);
              const Acc pz = fexp<Acc>(z[hh] - mn);
              m[hh] = mn;
              l[hh] = fma(l[hh], corr, pz);
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[hh][e] = fma(acc[hh][e], corr, pz * Acc(vx[e]));
            }
          }
        }
      }
    }
  }

  // Fold the four row groups (lanes sub, sub+16, sub+32, sub+48 own the same
  // channels); afterwards every lane holds the wave's state for its channels.
  __device__ __forceinline__ void fold_row_groups() {
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const Acc mo = shfl_xor_acc(m[hh], o);
        const Acc lo = shfl_xor_acc(l[hh], o);
        const Acc mn = fmax(m[hh], mo);
        const Acc ca = merge_weight(m[hh], mn);
        const Acc cb = merge_weight(mo, mn);
        l[hh] = l[hh] * ca + lo * cb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const Acc ao = shfl_xor_acc(acc[hh][e], o);
          acc[hh][e] = acc[hh][e] * ca + ao * cb;
        }
        m[hh] = mn;
      }
    }
  }
};

}  // namespace fasa
