// Per-wave core of FAC (Focused Attention Computation): online softmax over a run
// of selected rows for up to HG query heads of one kv head.
//
// out_h = softmax(q_h K_T^T * scale) V_T over the selected rows at their original
// positions (paper-graph-ui review of FASA, section 3.4 "Online Stage 2: Focused
// Attention Computation (FAC)").  A wave takes four rows per step: 16 lanes per
// row, 8 channels per lane.  Every K/V row is loaded once and serves all HG
// heads.  The state per head is (running max m, running sum l, acc[8 channels])
// in each of the four 16-lane row groups; fold_row_groups() combines them.
// FacWaveOct (bf16, long one-head lists) takes eight rows per step with 8 lanes
// of 16 channels per row; FacWaveMfma (bf16, several heads) runs the same
// softmax on the matrix cores.
//
// Precision: bf16 caches accumulate in fp32 (logits pre-scaled by log2(e),
// exponentiated with exp2); fp32 caches run logits, softmax and the weighted sum
// in fp64 (fp32 logits of magnitude ~30 carry ~2e-6 absolute error, enough to
// move a fp32 output by more than 1e-5).
#pragma once

#include <math.h>

#include <type_traits>

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

// An fp64 value moved by a DPP lane pattern (both 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = uint32_t(__builtin_amdgcn_update_dpp(0, int(uint32_t(u >> 32)), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}

// Sum over the 16 lanes of a row group, in every lane of it: DPP rotations by
// 8, 4, 2, 1 inside the row.
__device__ __forceinline__ float row_sum(float v) { return row16_sum(v); }
__device__ __forceinline__ double row_sum(double v) {
  v += dpp_f64<kDppRowRor + 8>(v);
  v += dpp_f64<kDppRowRor + 4>(v);
  v += dpp_f64<kDppRowRor + 2>(v);
  v += dpp_f64<kDppRowRor + 1>(v);
  return v;
}

// Merge weight of a partial state with max mi against the global max M
// (0 for an empty partial).
template <typename Acc>
__device__ __forceinline__ Acc merge_weight(Acc mi, Acc M) {
  return (mi == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(mi - M);
}

// The values of a lane pair that differ in lane bit 4 (PAIR 16) or bit 5
// (PAIR 32), returned in every lane of the pair as (lower-lane value,
// upper-lane value): v_permlane16_swap exchanges the odd 16-lane rows of one
// operand with the even rows of the other, v_permlane32_swap the upper half of
// one with the lower half of the other -- VALU moves, no LDS round trip.
template <int PAIR>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto r = PAIR == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                            : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
}
template <int PAIR>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  uint32_t a, b;
  lane_pair<PAIR>(__float_as_uint(v), a, b);
  lo = __uint_as_float(a);
  hi = __uint_as_float(b);
}
template <int PAIR>
__device__ __forceinline__ void lane_pair(double v, double& lo, double& hi) {
  const uint64_t u = __double_as_longlong(v);
  uint32_t a0, b0, a1, b1;
  lane_pair<PAIR>(uint32_t(u), a0, b0);
  lane_pair<PAIR>(uint32_t(u >> 32), a1, b1);
  lo = __longlong_as_double(int64_t((uint64_t(a1) << 32) | a0));
  hi = __longlong_as_double(int64_t((uint64_t(b1) << 32) | b0));
}

// q.k of one lane's 8 channels.  bf16 caches: four v_dot2_f32_bf16 on the raw
// bf16 pairs of q and k (bf16 products are exact in fp32; sums round in fp32),
// no widening of k; fp32 caches: eight fp64 FMAs.
__device__ __forceinline__ float dot8(const uint4& q, const Raw8<uint16_t>& k) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  auto h = [](uint32_t x) { return __builtin_bit_cast(bf16x2, x); };
  const float a = __builtin_amdgcn_fdot2_f32_bf16(h(k.v.x), h(q.x), 0.f, false);
  const float b = __builtin_amdgcn_fdot2_f32_bf16(h(k.v.y), h(q.y), 0.f, false);
  const float c = __builtin_amdgcn_fdot2_f32_bf16(h(k.v.z), h(q.z), a, false);
  const float d = __builtin_amdgcn_fdot2_f32_bf16(h(k.v.w), h(q.w), b, false);
  return c + d;
}

// N consecutive fp32 values of a row.
template <int N>
struct RawF {
  typedef float fv __attribute__((ext_vector_type(N)));
  fv v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const fv*>(p); }
  __device__ __forceinline__ void unpack(float (&x)[N]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = v[i];
  }
};

// VS > 1 (fp32 caches, one head over TIP's lists): the workgroup takes 1/VS of
// each V row (channels (128/VS) vpart onwards; the logits still use all of K),
// one 16- or 8-byte load a lane per row instead of two 16-byte ones; each lane
// then holds 8/VS channels.
template <typename T, typename Acc, int HG, int VS = 1>
struct FacWave {
  static_assert(VS == 1 || (sizeof(T) == 4 && (VS == 2 || VS == 4)), "fp32 caches split V in halves or quarters");
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kLanesPerRow = 16;   // lanes per row; each holds kCh channels
  static constexpr int kCh = 8 / VS;
  using QRaw = Raw8<T>;
  using VRaw = std::conditional_t<VS == 1, Raw8<T>, RawF<8 / VS>>;
  int vofs = 0;                             // VS > 1: the first channel of this workgroup's part
  __device__ __forceinline__ int chan(int sub, int e) const { return vofs + kCh * sub + e; }
  // Query slices: raw bf16 pairs (logits scaled afterwards by zscale), or
  // pre-scaled fp64 values for fp32 caches.
  uint4 q2[kBf16 ? HG : 1];
  Acc qv[kBf16 ? 1 : HG][8];
  Acc zscale;
  Acc m[HG], l[HG], acc[HG][kCh];

  // This lane's raw query slices of heads 0 .. nh-1 from q_head0 (rows of q,
  // each kHeadDim long); loads are unconditional (slots past nh repeat the last).
  static __device__ __forceinline__ void load_q(const T* q_head0, int nh, Raw8<T> (&qr)[HG]) {
    const int sub = threadIdx.x & 15;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) qr[hh].load(q_head0 + int64_t(min(hh, nh - 1)) * kHeadDim + 8 * sub);
  }

  // Query slices of heads h_first .. h_first+nh-1; unused head slots are zero.
  // Logits come out scaled by scale (and by log2(e) for fp32 accumulation,
  // whose exponentials are exp2).
  __device__ __forceinline__ void init(const T* q_head0, int nh, float scale) {
    Raw8<T> qr[HG];
    load_q(q_head0, nh, qr);
    init_raw(qr, nh, scale);
  }
  __device__ __forceinline__ void init_raw(const Raw8<T> (&qr)[HG], int nh, float scale, int vpart = 0) {
    vofs = VS > 1 ? (kHeadDim / VS) * vpart : 0;
    const Acc qscale = sizeof(Acc) == 4 ? Acc(scale) * Acc(1.4426950408889634) : Acc(scale);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      m[hh] = neg_inf<Acc>();
      l[hh] = Acc(0);
#pragma unroll
      for (int e = 0; e < kCh; ++e) acc[hh][e] = Acc(0);
      if constexpr (kBf16) {
        const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
        q2[hh] = (hh < nh) ? reinterpret_cast<const uint4&>(qr[hh]) : z4;
      } else {
        float x[8];
        qr[hh].unpack(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[hh][e] = (hh < nh) ? Acc(x[e]) * qscale : Acc(0);
      }
    }
    zscale = kBf16 ? qscale : Acc(1);
  }

  // Rows r0 .. r1-1 of the selection.  lane_offset(r) returns the element offset
  // of row r inside the kv head's pool slice, or -1 for an invalid row; it is
  // called once per 64 rows with r = base + lane (two dependent loads at most).
  // Invalid rows load a valid row of the wave instead and are then ignored, so
  // the row loads need no branch and go out together.
  // U: row quads whose loads are in flight together (2 U raw registers of 4 or 8
  // VGPRs each).  The online softmax is updated once per U quads: the logits of
  // all U quads first, then one rescale of each head's state to the new
  // maximum, then the U weighted rows added.
  // NT: non-temporal row loads, for rows that no other workgroup reads.
  // FAST: batches whose rows all exist and are valid take an unmasked copy of
  // the batch (measured 0.7 us faster over 1024-row lists, 0.1 us slower over
  // 256-row lists, where each wave sees one batch and fetches both copies; the
  // 8-lane FacWaveOct gains over both).
  template <int U = 2, bool NT = false, bool FAST = false, typename LaneOffset>
  __device__ __forceinline__ void run(int r0, int r1, LaneOffset lane_offset, const T* kbase,
                                      const T* vbase) {
    const int lane = threadIdx.x & 63, rg = lane >> 4, sub = lane & 15;
    kbase += 8 * sub;
    vbase += kCh * sub + vofs;
    for (int base = r0; base < r1; base += 64) {   // wave-uniform
      const int64_t my_off = lane_offset(base + lane);
      const uint64_t ok = __ballot(my_off >= 0);
      if (ok == 0) continue;
      const int64_t dummy = __shfl(my_off, __ffsll((unsigned long long)ok) - 1, 64);
      const int nrows = min(64, r1 - base);
      for (int q4 = 0; q4 < nrows; q4 += 4 * U) {
        Raw8<T> kr[U];
        VRaw vr[U];
        // A batch whose 4 U rows all exist and are valid skips every mask.
        static_assert(4 * U < 64, "a batch within one 64-row window");
        const bool full = FAST && q4 + 4 * U <= nrows &&
                          ((ok >> q4) & ((uint64_t(1) << (4 * U)) - 1)) == ((uint64_t(1) << (4 * U)) - 1);
        if constexpr (FAST) if (full) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t o = __shfl(my_off, q4 + 4 * u + rg, 64);
            if constexpr (NT) {
              kr[u].load_nt(kbase + o);
              vr[u].load_nt(vbase + o);
            } else {
              kr[u].load(kbase + o);
              vr[u].load(vbase + o);
            }
          }
          const bool all[U] = {};
          absorb<U, false>(kr, vr, all);
          continue;
        }
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int src = q4 + 4 * u + rg;   // lane holding this row's offset
          const int64_t off = __shfl(my_off, src < 64 ? src : 0, 64);
          valid[u] = (src < nrows) && off >= 0;
          const int64_t o = valid[u] ? off : dummy;
          if constexpr (NT) {
            kr[u].load_nt(kbase + o);
            vr[u].load_nt(vbase + o);
          } else {
            kr[u].load(kbase + o);
            vr[u].load(vbase + o);
          }
        }
        absorb<U>(kr, vr, valid);
      }
    }
  }

  // Fold U row quads already loaded (kr, vr: this row group's row of each
  // quad; valid[u] false drops quad u's row) into the online softmax: the
  // logits of all U quads first, then one rescale of each head's state to the
  // new maximum, then the U weighted rows added.  MASKED false: every row is
  // valid (valid is not read), so no logit is -inf and the batch's maximum is
  // finite.
  template <int U, bool MASKED = true>
  __device__ __forceinline__ void absorb(const Raw8<T> (&kr)[U], const VRaw (&vr)[U], const bool (&valid)[U]) {
    Acc z[U][HG], mn[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) mn[hh] = m[hh];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kx[8];
      if constexpr (!kBf16) kr[u].unpack(kx);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        Acc sdot;
        if constexpr (kBf16) {
          sdot = Acc(dot8(q2[hh], reinterpret_cast<const Raw8<uint16_t>&>(kr[u])));
        } else {
          sdot = Acc(0);
#pragma unroll
          for (int e = 0; e < 8; ++e) sdot = fma(qv[hh][e], Acc(kx[e]), sdot);
        }
        const Acc zz = row_sum(sdot) * zscale;
        z[u][hh] = (!MASKED || valid[u]) ? zz : neg_inf<Acc>();
        mn[hh] = fmax(mn[hh], z[u][hh]);
      }
    }
    // Rescale each head's state to its new maximum once.
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const Acc corr = merge_weight(m[hh], mn[hh]);
      l[hh] *= corr;
#pragma unroll
      for (int e = 0; e < kCh; ++e) acc[hh][e] *= corr;
      m[hh] = mn[hh];
    }
    // Add the weighted rows.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vx[kCh];
      vr[u].unpack(vx);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const Acc pz = MASKED ? merge_weight(z[u][hh], mn[hh]) : fexp<Acc>(z[u][hh] - mn[hh]);
        l[hh] += pz;
#pragma unroll
        for (int e = 0; e < kCh; ++e) acc[hh][e] = fma(pz, Acc(vx[e]), acc[hh][e]);
      }
    }
  }

  // Fold the four row groups (lanes sub, sub+16, sub+32, sub+48 own the same
  // channels) with the log-sum-exp rule, row pairs (0,1), (2,3) first, then the
  // two halves; afterwards every lane holds the wave's state for its channels.
  template <int PAIR>
  __device__ __forceinline__ void fold_pairs() {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      Acc ma, mb, la, lb;
      lane_pair<PAIR>(m[hh], ma, mb);
      lane_pair<PAIR>(l[hh], la, lb);
      const Acc mn = fmax(ma, mb);
      const Acc wa = merge_weight(ma, mn);
      const Acc wb = merge_weight(mb, mn);
      l[hh] = la * wa + lb * wb;
#pragma unroll
      for (int e = 0; e < kCh; ++e) {
        Acc aa, ab;
        lane_pair<PAIR>(acc[hh][e], aa, ab);
        acc[hh][e] = aa * wa + ab * wb;
      }
      m[hh] = mn;
    }
  }
  __device__ __forceinline__ void fold_row_groups() {
    fold_pairs<16>();
    fold_pairs<32>();
  }
};

// DPP patterns inside each 8-lane half of a 16-lane row.
constexpr int kDppHalfMirror = 0x141;   // lane i reads lane 7 - i of its half row
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2, 3, 0, 1]: lane i reads lane i ^ 2
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1, 0, 3, 2]: lane i reads lane i ^ 1
constexpr int kDppRowRor8 = 0x128;      // lane i reads lane i ^ 8 of its 16-lane row

// Sum over the 8 lanes of a half row, the same value in all 8: the pair sums
// v_i + v_(7-i), then pairs of those, then the two halves of the quad (every
// lane adds the same two pair-of-pair sums, so the results agree bit for bit).
__device__ __forceinline__ float oct_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppHalfMirror, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadSwap2, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadSwap1, 0xF, 0xF, false));
  return v;
}

// 16 bf16 values of a row: channels c .. c+7 and 64+c .. 64+c+7 (from p = row + c),
// so that the 8 lanes of a row read its first 128 bytes with one instruction
// and the other 128 with the next.
struct Raw16 {
  uint4 a, b;
  __device__ __forceinline__ void load(const uint16_t* p) {
    a = *reinterpret_cast<const uint4*>(p);
    b = *reinterpret_cast<const uint4*>(p + 64);
  }
  __device__ __forceinline__ void unpack(float (&x)[16]) const {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};

// The same online softmax as FacWave for bf16 caches, with 8 lanes per row and
// 16 channels per lane: a wave takes eight rows per step.  Per row that halves
// the lanes running the logit reduction, the exponentials and the row
// addresses, and takes one DPP step less for the sum; the V unpack and FMAs stay
// one per channel.  exp2 is the hardware instruction: arguments below -126 (a
// weight under 2^-126 of the running maximum's) give 0 instead of a denormal.
// 4 bf16 values (8 bytes) of a row.
struct Raw4 {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void unpack(float (&x)[4]) const {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  }
};

template <int HG, int VS = 1>
struct FacWaveOct {
  // VS > 1: this wave's workgroup takes only 1/VS of each V row (channels
  // (128/VS) vpart onwards; the logits still use all of K), so V costs one
  // load instruction per 8 rows (of 16 or 8 bytes a lane) instead of two, and
  // VS workgroups per head share the rows; each lane then holds 16/VS channels.
  static_assert(VS == 1 || VS == 2 || VS == 4, "whole, half or quarter V rows");
  static constexpr int kLanesPerRow = 8;
  static constexpr int kCh = 16 / VS;
  using QRaw = Raw16;
  using VRaw = std::conditional_t<VS == 1, Raw16, std::conditional_t<VS == 2, Raw8<uint16_t>, Raw4>>;
  uint4 q2[HG][2];
  float zscale;
  float m[HG], l[HG], acc[HG][kCh];
  int vofs;                                 // VS > 1: the first channel of this workgroup's part

  // Channel of a lane's value e (sub = lane % 8).
  __device__ __forceinline__ int chan(int sub, int e) const {
    return VS > 1 ? vofs + kCh * sub + e : (e < 8 ? 0 : 64) + 8 * sub + (e & 7);
  }

  static __device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
  static __device__ __forceinline__ float weight(float mi, float M) {
    return mi == -INFINITY ? 0.f : ex2(mi - M);
  }

  static __device__ __forceinline__ void load_q(const uint16_t* q_head0, int nh, Raw16 (&qr)[HG]) {
    const int sub = threadIdx.x & 7;
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) qr[hh].load(q_head0 + int64_t(min(hh, nh - 1)) * kHeadDim + 8 * sub);
  }

  __device__ __forceinline__ void init_raw(const Raw16 (&qr)[HG], int nh, float scale, int vpart = 0) {
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < kCh; ++e) acc[hh][e] = 0.f;
      q2[hh][0] = hh < nh ? qr[hh].a : z4;
      q2[hh][1] = hh < nh ? qr[hh].b : z4;
    }
    zscale = scale * 1.4426950408889634f;
    vofs = VS > 1 ? (kHeadDim / VS) * vpart : 0;
  }

  // Rows r0 .. r1-1, as FacWave::run; U: rows per lane in flight (8 U per wave).
  template <int U = 4, bool NT = false, bool FAST = false, typename LaneOffset>
  __device__ __forceinline__ void run(int r0, int r1, LaneOffset lane_offset, const uint16_t* kbase,
                                      const uint16_t* vbase) {
    static_assert(!NT, "ordinary row loads");
    const int lane = threadIdx.x & 63, rg = lane >> 3, sub = lane & 7;
    kbase += 8 * sub;
    vbase += (VS > 1 ? kCh * sub : 8 * sub) + vofs;
    for (int base = r0; base < r1; base += 64) {   // wave-uniform
      const int64_t my_off = lane_offset(base + lane);
      const uint64_t ok = __ballot(my_off >= 0);
      if (ok == 0) continue;
      const int64_t dummy = __shfl(my_off, __ffsll((unsigned long long)ok) - 1, 64);
      const int nrows = min(64, r1 - base);
      for (int q8 = 0; q8 < nrows; q8 += 8 * U) {
        Raw16 kr[U];
        VRaw vr[U];
        static_assert(8 * U < 64, "a batch within one 64-row window");
        constexpr uint64_t kAll = (uint64_t(1) << (8 * U)) - 1;
        const bool full = FAST && q8 + 8 * U <= nrows && ((ok >> q8) & kAll) == kAll;
        if constexpr (FAST) if (full) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t o = __shfl(my_off, q8 + 8 * u + rg, 64);
            kr[u].load(kbase + o);
            vr[u].load(vbase + o);
          }
          const bool all[U] = {};
          absorb<U, false>(kr, vr, all);
          continue;
        }
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int src = q8 + 8 * u + rg;
          const int64_t off = __shfl(my_off, src < 64 ? src : 0, 64);
          valid[u] = (src < nrows) && off >= 0;
          const int64_t o = valid[u] ? off : dummy;
          kr[u].load(kbase + o);
          vr[u].load(vbase + o);
        }
        absorb<U>(kr, vr, valid);
      }
    }
  }

  template <int U, bool MASKED = true>
  __device__ __forceinline__ void absorb(const Raw16 (&kr)[U], const VRaw (&vr)[U], const bool (&valid)[U]) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    auto h = [](uint32_t x) { return __builtin_bit_cast(bf16x2, x); };
    float z[U][HG], mn[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) mn[hh] = m[hh];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const uint4 &qa = q2[hh][0], &qb = q2[hh][1];
        float s0 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].a.x), h(qa.x), 0.f, false);
        float s1 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].a.y), h(qa.y), 0.f, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].a.z), h(qa.z), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].a.w), h(qa.w), s1, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].b.x), h(qb.x), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].b.y), h(qb.y), s1, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].b.z), h(qb.z), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(h(kr[u].b.w), h(qb.w), s1, false);
        const float zz = oct_sum(s0 + s1) * zscale;
        z[u][hh] = (!MASKED || valid[u]) ? zz : -INFINITY;
        mn[hh] = fmaxf(mn[hh], z[u][hh]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const float corr = weight(m[hh], mn[hh]);
      l[hh] *= corr;
#pragma unroll
      for (int e = 0; e < kCh; ++e) acc[hh][e] *= corr;
      m[hh] = mn[hh];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vx[kCh];
      vr[u].unpack(vx);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float pz = MASKED ? weight(z[u][hh], mn[hh]) : ex2(z[u][hh] - mn[hh]);
        l[hh] += pz;
#pragma unroll
        for (int e = 0; e < kCh; ++e) acc[hh][e] = fmaf(pz, vx[e], acc[hh][e]);
      }
    }
  }

  // The pair of row groups that differ in lane bit 3 (PAIR 8, a DPP rotation by
  // 8 inside the 16-lane row), bit 4 or bit 5, merged by the log-sum-exp rule in
  // (lower, upper) order in both lanes of the pair.
  template <int PAIR>
  static __device__ __forceinline__ void pair_of(float v, float& lo, float& hi) {
    if constexpr (PAIR == 8) {
      const float o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor8, 0xF, 0xF, false));
      const bool upper = threadIdx.x & 8;
      lo = upper ? o : v;
      hi = upper ? v : o;
    } else {
      lane_pair<PAIR>(v, lo, hi);
    }
  }
  template <int PAIR>
  __device__ __forceinline__ void fold_pairs() {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float ma, mb, la, lb;
      pair_of<PAIR>(m[hh], ma, mb);
      pair_of<PAIR>(l[hh], la, lb);
      const float mn = fmaxf(ma, mb);
      const float wa = weight(ma, mn), wb = weight(mb, mn);
      l[hh] = la * wa + lb * wb;
#pragma unroll
      for (int e = 0; e < kCh; ++e) {
        float aa, ab;
        pair_of<PAIR>(acc[hh][e], aa, ab);
        acc[hh][e] = aa * wa + ab * wb;
      }
      m[hh] = mn;
    }
  }
  // Afterwards lanes 0 .. 7 (and every other half row) hold the wave's state
  // for their 16 channels.
  __device__ __forceinline__ void fold_row_groups() {
    fold_pairs<8>();
    fold_pairs<16>();
    fold_pairs<32>();
  }
};

// ---------------------------------------------------------------------------
// Matrix-core variant for bf16 caches, the same online softmax over 16-row
// blocks.  With G query heads per kv head the per-row work is a G x 128
// contraction with K and a G-wide P times V; on the vector ALUs it costs more
// issue time than the rows take to arrive from HBM, on the matrix cores a small
// part of it.
//
// Lane l, g = l / 16, n = l % 16.  Both instructions give the 16 x 16 result as
// D[4 g + i][n], i < 4.
//   Logits: S = K Q^T with v_mfma_f32_16x16x32_bf16 (A[n][8 g + j],
//     B[8 g + j][n], j < 8), heads padded to 16 columns (n >= HG are zero).
//     A = K rows: lane l loads 16 bytes of block row n, channels 32 s + 8 g .. +7
//     for step s < 4; B = Q^T in the same channel order (loaded once).  Lane l
//     ends up with the logits of block rows 4 g .. 4 g + 3 for head n.
//   Weighted sum: O^T += V^T P with v_mfma_f32_16x16x16bf16_1k (A[n][4 g + j],
//     B[4 g + j][n], j < 4).  B = P: lane l's own four logits' weights.  A = V^T:
//     lane l needs channel 16 dt + n of block rows 4 g .. 4 g + 3, a transposed
//     access, so each wave first writes its 16 V rows into its own LDS tile
//     (rows padded to 264 bytes) and reads each 16-channel tile back with one
//     transposing LDS read (ds_read_b64_tr_b16).  P enters as a
//     bf16 high part and a bf16 low part (the rounding error of a single bf16
//     P, about 2^-9 of |v|, would exceed the 2e-3 bound on outputs with large
//     channels); the two products add up to P within about 2^-17.  D: lane l
//     holds channels 16 dt + 4 g + i of head n.
// Lane l keeps the running max of head n (the same in the four lanes of the
// column), its own partial sum, and the 32 channels of O^T above, so the
// rescale to a new maximum is lane-local.  fold_row_groups() moves the result
// into FacWave's layout (lane sub holds channels 8 sub .. +7 of every head)
// through the same LDS tile.
constexpr int kMfmaTilePitch = 132;                  // bf16 per LDS row (264 bytes)
constexpr int kMfmaTileElems = 16 * kMfmaTilePitch;  // one wave's tile

template <int HG>
struct FacWaveMfma {
  // Channel of a lane's value e after fold_row_groups (lanes 0 .. 15 hold 8 each).
  __device__ __forceinline__ int chan(int sub, int e) const { return 8 * sub + e; }
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  typedef __attribute__((ext_vector_type(4))) short s16x4;
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  static_assert(HG <= 16, "heads are padded to 16 columns");
  static_assert(HG * kHeadDim * 4 + 2 * HG * 4 <= kMfmaTileElems * 2, "the fold fits in the LDS tile");
  // The result, in FacWave's layout, after fold_row_groups().
  float m[HG], l[HG], acc[HG][8];
  bf16x8 qb[4];       // Q^T operand for channel steps 0..3
  float zscale;
  float mrun, lrun;   // head lane % 16
  f32x4 o[8];         // O^T channels 16 dt + 4 g + i, head lane % 16
  uint16_t* tile;     // this wave's LDS tile (kMfmaTileElems)

  // This lane's query slices (head lane % 16, channels 32 s + 8 g .. +7),
  // loaded unconditionally (heads past nh repeat the last; init zeroes them).
  static __device__ __forceinline__ void load_q(const uint16_t* q_head0, int nh, uint4 (&qm)[4]) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const uint16_t* qh = q_head0 + int64_t(min(n, nh - 1)) * kHeadDim + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      Raw8<uint16_t> x;
      x.load(qh + 32 * s);
      qm[s] = x.v;
    }
  }
  __device__ __forceinline__ void init(const uint16_t* q_head0, int nh, float scale, uint16_t* lds_tile) {
    uint4 qm[4];
    load_q(q_head0, nh, qm);
    init_raw(qm, nh, scale, lds_tile);
  }
  __device__ __forceinline__ void init_raw(const uint4 (&qm)[4], int nh, float scale, uint16_t* lds_tile) {
    const int n = threadIdx.x & 15;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = __builtin_bit_cast(bf16x8, n < nh ? qm[s] : make_uint4(0u, 0u, 0u, 0u));
    zscale = scale * 1.4426950408889634f;
    mrun = -INFINITY;
    lrun = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    tile = lds_tile;
  }

  // Rows r0 .. r1-1; lane_offset as for FacWave::run (called once per 64 rows
  // with r = base + lane).  Invalid rows load a valid row of the batch and get
  // a -inf logit.  NT: non-temporal row loads.  One 16-row block's loads are in
  // flight per wave at a time.
  template <bool NT = false, typename LaneOffset>
  __device__ __forceinline__ void run(int r0, int r1, LaneOffset lane_offset, const uint16_t* kbase,
                                      const uint16_t* vbase) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    for (int base = r0; base < r1; base += 64) {   // wave-uniform
      const int64_t my_off = lane_offset(base + lane);
      const int nrows = min(64, r1 - base);
      const uint64_t in_range = nrows >= 64 ? ~uint64_t(0) : ((uint64_t(1) << nrows) - 1);
      const uint64_t ok = __ballot(my_off >= 0) & in_range;
      if (ok == 0) continue;
      const int64_t dummy = __shfl(my_off, __ffsll((unsigned long long)ok) - 1, 64);
      auto row_off = [&](int x) -> int64_t {   // x < 64
        const int64_t o = __shfl(my_off, x, 64);
        return ((ok >> x) & 1) ? o : dummy;
      };
      for (int b = 0; b < nrows; b += 16) {   // wave-uniform
        // K: block row n; V: rows 4 k + g, channels 8 n .. +7.
        const int64_t k0 = row_off(b + n);
        uint4 ka[4], va[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = load16<NT>(kbase + k0 + 32 * s + 8 * g);
#pragma unroll
        for (int k = 0; k < 4; ++k) va[k] = load16<NT>(vbase + row_off(b + 4 * k + g) + 8 * n);
        block(ka, va, uint32_t(ok >> (b + 4 * g)) & 0xFu);
      }
    }
  }

  // Rows r0 .. r1-1 with the next block's loads in flight while a block is
  // computed (two 16-row blocks, 16 KB per wave).  The row offsets of up to
  // kPfRows rows are resolved first -- all of lane_offset's dependent loads in
  // one go -- into this wave's LDS area `offs` (kPfRows entries; negative:
  // invalid row, which loads the chunk's first valid row and gets a -inf logit).
  static constexpr int kPfRows = 512;
  template <bool NT, typename LaneOffset>
  __device__ __forceinline__ void run_pipelined(int r0, int r1, LaneOffset lane_offset, const uint16_t* kbase,
                                                const uint16_t* vbase, int64_t* offs) {
    const int lane = threadIdx.x & 63;
    for (int cb = r0; cb < r1; cb += kPfRows) {   // wave-uniform
      int64_t o[kPfRows / 64];
#pragma unroll
      for (int k = 0; k < kPfRows / 64; ++k) o[k] = lane_offset(cb + 64 * k + lane);
      int64_t dummy = -1;
#pragma unroll
      for (int k = kPfRows / 64 - 1; k >= 0; --k) {   // the lowest valid row wins
        const uint64_t m = __ballot(o[k] >= 0);
        if (m != 0) dummy = __shfl(o[k], __ffsll((unsigned long long)m) - 1, 64);
      }
      if (dummy < 0) continue;                       // no valid row in this chunk
      __builtin_amdgcn_wave_barrier();               // the previous chunk's reads of offs are done
#pragma unroll
      for (int k = 0; k < kPfRows / 64; ++k) offs[64 * k + lane] = o[k];
      __builtin_amdgcn_wave_barrier();
      const int nb = (min(kPfRows, r1 - cb) + 15) >> 4;
      uint4 ka[4], va[4];
      uint32_t ra;
      load_block<NT>(offs, 0, dummy, kbase, vbase, ka, va, ra);
      for (int i = 1; i < nb; ++i) {                 // wave-uniform
        uint4 kb[4], vb[4];
        uint32_t rb;
        load_block<NT>(offs, 16 * i, dummy, kbase, vbase, kb, vb, rb);
        block(ka, va, ra);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          ka[s] = kb[s];
          va[s] = vb[s];
        }
        ra = rb;
      }
      block(ka, va, ra);
    }
  }

  // Loads of the 16-row block at row b of `offs` (see run_pipelined); rv bit i:
  // block row 4 g + i is valid.
  template <bool NT>
  static __device__ __forceinline__ void load_block(const int64_t* offs, int b, int64_t dummy, const uint16_t* kbase,
                                                    const uint16_t* vbase, uint4 (&ka)[4], uint4 (&va)[4],
                                                    uint32_t& rv) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const int64_t kr = offs[b + n];
    const uint16_t* kp = kbase + (kr >= 0 ? kr : dummy) + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[s] = load16<NT>(kp + 32 * s);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t vr = offs[b + 4 * k + g];
      va[k] = load16<NT>(vbase + (vr >= 0 ? vr : dummy) + 8 * n);
    }
    rv = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) rv |= offs[b + 4 * g + i] >= 0 ? (1u << i) : 0u;
  }

  // One 16-row block: ka holds K block row n (channels 32 s + 8 g .. +7), va V
  // rows 4 k + g (channels 8 n .. +7); rv bit i: block row 4 g + i is valid.
  __device__ __forceinline__ void block(const uint4 (&ka)[4], const uint4 (&va)[4], uint32_t rv) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    f32x4 st = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[s]), qb[s], st, 0, 0, 0);
    // V rows into the LDS tile (8-byte writes; the tile rows are 8-byte aligned).
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint2* dst = reinterpret_cast<uint2*>(tile + (4 * k + g) * kMfmaTilePitch + 8 * n);
      dst[0] = make_uint2(va[k].x, va[k].y);
      dst[1] = make_uint2(va[k].z, va[k].w);
    }
    // Logits of block rows 4 g + i, head n; the block maximum of the column.
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = ((rv >> i) & 1u) != 0u ? st[i] * zscale : -INFINITY;
      mx = fmaxf(mx, z[i]);
    }
    float xa, xb;
    lane_pair<16>(mx, xa, xb);
    mx = fmaxf(xa, xb);
    lane_pair<32>(mx, xa, xb);
    mx = fmaxf(xa, xb);
    const float mn = fmaxf(mrun, mx);
    const float corr = merge_weight(mrun, mn);
    mrun = mn;
    s16x4 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = merge_weight(z[i], mn);
      psum += p;
      const __bf16 h = (__bf16)p;
      phi[i] = __builtin_bit_cast(short, h);
      plo[i] = __builtin_bit_cast(short, (__bf16)(p - (float)h));
    }
    lrun = lrun * corr + psum;
    __builtin_amdgcn_wave_barrier();
    // V^T operand of channel tile dt: lane (g, n) needs rows 4 g .. 4 g + 3 of
    // channel 16 dt + n.  The transposing LDS read gives it in one instruction:
    // within each 16-lane group, lane 4 r + q supplies 4 channels (4 q .. 4 q + 3
    // of the tile) of row 4 g + r, and lane n receives channel n of the four rows.
    const uint16_t* vsrc = tile + (4 * g + (n >> 2)) * kMfmaTilePitch + 4 * (n & 3);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      typedef short s16x4_lds __attribute__((ext_vector_type(4)));
      const s16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4_lds __attribute__((address_space(3)))*)(vsrc + 16 * dt));
      o[dt] = o[dt] * corr;
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, o[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  template <bool NT>
  static __device__ __forceinline__ uint4 load16(const uint16_t* p) {
    Raw8<uint16_t> x;
    if constexpr (NT) x.load_nt(p);
    else x.load(p);
    return x.v;
  }

  // The wave's state in FacWave's layout, through the LDS tile: O^T into
  // [head][channel] floats, the column sums and maxima after it.
  __device__ __forceinline__ void fold_row_groups() {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15, sub = lane & 15;
    float la, lb;
    lane_pair<16>(lrun, la, lb);
    lrun = la + lb;
    lane_pair<32>(lrun, la, lb);
    lrun = la + lb;
    float* f = reinterpret_cast<float*>(tile);
    __builtin_amdgcn_wave_barrier();
    if (n < HG) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[n * kHeadDim + 16 * dt + 4 * g + i] = o[dt][i];
      }
      if (g == 0) {
        f[HG * kHeadDim + n] = mrun;
        f[HG * kHeadDim + HG + n] = lrun;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = f[hh * kHeadDim + 8 * sub + e];
      m[hh] = f[HG * kHeadDim + hh];
      l[hh] = f[HG * kHeadDim + HG + hh];
    }
    __builtin_amdgcn_wave_barrier();
  }
};

}  // namespace fasa
