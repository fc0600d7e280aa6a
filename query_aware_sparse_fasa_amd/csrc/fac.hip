// FAC: Focused Attention Computation over the selected rows.
//
// For every query head h of kv head g: out_h = softmax(q_h K_T^T * scale) V_T,
// where K_T, V_T are the cached rows at the selected token indices, used in
// place at their original positions (paper-graph-ui review of FASA, section 3.4
// "Online Stage 2: Focused Attention Computation (FAC)", gather and attention
// equations).  The gather is never materialised: each selected row is read
// straight from the paged pool through the block table.
//
// Split-K flash decode.  A workgroup is 4 waves; each wave walks its own run of
// selected rows, four rows at a time (16 lanes per row, 8 channels per lane),
// and keeps a running (max m, sum l, acc[128]) per query head -- the online
// softmax.  Every K/V row is loaded once per kv head and reused by all query
// heads of the group (GQA).  A wave's logits need a 16-lane reduction; the four
// row groups of a wave are folded together with cross-lane shuffles at the end
// and the wave writes one partial.  A second kernel merges the partials of a
// head with the log-sum-exp rule.  With at most 8 query heads per pass the q.K
// product is an 8 x 128 by 128 x rows contraction at a few flops per loaded
// byte -- HBM/latency bound, so it runs on the vector ALUs, not MFMA.
//
// Precision: bf16 caches accumulate in fp32 (logits pre-scaled by log2(e) and
// exponentiated with exp2); fp32 caches run the logits, softmax and weighted
// sum in fp64 and round once at the end (fp32 logits of magnitude ~30 carry
// ~2e-6 absolute error, enough to move a fp32 output by more than 1e-5).
#include <math.h>

#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

struct FacArgs {
  Common c;
  FacPlan p;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* sel_idx;
  const int32_t* sel_count;
  void* part_acc;   // [b][H_q][P][128] Acc
  void* part_ml;    // [b][H_q][P][2]   Acc (running max, running sum)
  float* out;
};

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

template <typename T, typename Acc, int HG>
__global__ __launch_bounds__(256) void fac_split_kernel(FacArgs a) {
  const Common& c = a.c;
  const FacPlan& p = a.p;
  const int b = blockIdx.z;
  const int g = blockIdx.y / p.head_chunks;
  const int h0 = (blockIdx.y % p.head_chunks) * HG;      // first head of this pass, within the group
  const int nh = min(HG, c.group - h0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane >> 4, sub = lane & 15;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;
  int count = a.sel_count[unit];
  count = count < 0 ? 0 : (count > c.cap ? c.cap : count);   // contents are preconditions; stay in bounds
  const int pidx = blockIdx.x * kFacWaves + wave;
  const int r0 = pidx * p.rows_per_wave;
  const int r1 = min(r0 + p.rows_per_wave, count);
  const int32_t* sel = a.sel_idx + unit * c.cap;
  const int32_t* btab = a.block_table + int64_t(b) * c.max_blocks;

  // Query slices of this pass's heads, pre-scaled (by scale*log2(e) for exp2 in fp32).
  const Acc qscale = sizeof(Acc) == 4 ? Acc(c.scale) * Acc(1.4426950408889634) : Acc(c.scale);
  Acc qv[HG][8];
  Acc m[HG], l[HG], acc[HG][8];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = neg_inf<Acc>();
    l[hh] = Acc(0);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = Acc(0);
    if (hh < nh) {
      const int h = g * c.group + h0 + hh;
      float x[8];
      load8(static_cast<const T*>(a.q) + (int64_t(b) * c.n_q_heads + h) * kHeadDim + 8 * sub, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = Acc(x[e]) * qscale;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = Acc(0);
    }
  }

  const T* kbase = static_cast<const T*>(a.k_pool) + int64_t(g) * c.kv_head_stride + 8 * sub;
  const T* vbase = static_cast<const T*>(a.v_pool) + int64_t(g) * c.kv_head_stride + 8 * sub;
  for (int r4 = r0; r4 < r1; r4 += 4) {                  // wave-uniform trip count
    const int r = r4 + rg;
    const int j = r < r1 ? sel[r] : -1;
    const bool valid = j >= 0 && j < c.max_blocks * kBlock;
    float kx[8], vx[8];
    if (valid) {
      const int64_t off = int64_t(btab[j >> 8]) * c.kv_block_stride + int64_t(j & (kBlock - 1)) * kHeadDim;
      load8(kbase + off, kx);
      load8(vbase + off, vx);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kx[e] = vx[e] = 0.f;
    }
    Acc z[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      Acc s = Acc(0);
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fma(qv[hh][e], Acc(kx[e]), s);
      z[hh] = s;
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) z[hh] += shfl_xor_acc(z[hh], o);
    }
    if (valid) {
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

  // Fold the four row groups (lanes sub, sub+16, sub+32, sub+48 own the same channels).
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const Acc mo = shfl_xor_acc(m[hh], o);
      const Acc lo = shfl_xor_acc(l[hh], o);
      const Acc mn = fmax(m[hh], mo);
      const Acc ca = (m[hh] == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(m[hh] - mn);
      const Acc cb = (mo == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(mo - mn);
      l[hh] = l[hh] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const Acc ao = shfl_xor_acc(acc[hh][e], o);
        acc[hh][e] = acc[hh][e] * ca + ao * cb;
      }
      m[hh] = mn;
    }
  }

  if (rg == 0) {
    Acc* pacc = static_cast<Acc*>(a.part_acc);
    Acc* pml = static_cast<Acc*>(a.part_ml);
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      if (hh < nh) {
        const int64_t h = int64_t(b) * c.n_q_heads + g * c.group + h0 + hh;
        const int64_t slot = h * p.n_partials + pidx;
#pragma unroll
        for (int e = 0; e < 8; ++e) pacc[slot * kHeadDim + 8 * sub + e] = acc[hh][e];
        if (sub == 0) {
          pml[slot * 2 + 0] = m[hh];
          pml[slot * 2 + 1] = l[hh];
        }
      }
    }
  }
}

template <typename Acc>
__global__ __launch_bounds__(kHeadDim) void fac_merge_kernel(FacArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int P = a.p.n_partials;
  const int64_t base = (int64_t(b) * a.c.n_q_heads + h) * P;
  const Acc* pacc = static_cast<const Acc*>(a.part_acc) + base * kHeadDim + d;
  const Acc* pml = static_cast<const Acc*>(a.part_ml) + base * 2;
  Acc M = neg_inf<Acc>();
  for (int i = 0; i < P; ++i) M = fmax(M, pml[2 * i]);
  float res = 0.f;
  if (M != neg_inf<Acc>()) {
    Acc L = Acc(0), O = Acc(0);
    for (int i = 0; i < P; ++i) {
      const Acc mi = pml[2 * i];
      if (mi == neg_inf<Acc>()) continue;
      const Acc w = fexp<Acc>(mi - M);
      L = fma(pml[2 * i + 1], w, L);
      O = fma(pacc[int64_t(i) * kHeadDim], w, O);
    }
    res = float(O / L);
  }
  a.out[(int64_t(b) * a.c.n_q_heads + h) * kHeadDim + d] = res;
}

template <typename T, typename Acc>
hipError_t launch_fac_t(FacArgs& a, hipStream_t s) {
  const FacPlan& p = a.p;
  const dim3 grid(p.n_split, a.c.n_kv_heads * p.head_chunks, a.c.batch);
  switch (p.heads_per_pass) {
    case 1: hipLaunchKernelGGL((fac_split_kernel<T, Acc, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((fac_split_kernel<T, Acc, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((fac_split_kernel<T, Acc, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((fac_split_kernel<T, Acc, 8>), grid, dim3(256), 0, s, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fac_merge_kernel<Acc>, dim3(a.c.n_q_heads, a.c.batch), dim3(kHeadDim), 0, s, a);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

FacPlan fac_plan(const Common& c) {
  FacPlan p;
  const int g8 = c.group < 8 ? c.group : 8;
  int hg = 1;
  while (hg < g8) hg <<= 1;
  p.heads_per_pass = hg;
  p.head_chunks = (c.group + hg - 1) / hg;
  const int64_t units = int64_t(c.batch) * c.n_kv_heads * p.head_chunks;
  const int64_t rows = units * int64_t(c.cap);
  int64_t rpw = (rows + 4095) / 4096;             // aim at ~4096 waves in flight
  if (rpw < 2 * g8) rpw = 2 * g8;                 // keep partial traffic below ~1/2 of row traffic
  rpw = (rpw + 3) & ~int64_t(3);
  if (rpw < 4) rpw = 4;
  if (rpw > 128) rpw = 128;
  p.rows_per_wave = int(rpw);
  const int per_wg = kFacWaves * p.rows_per_wave;
  p.n_split = c.cap > 0 ? (c.cap + per_wg - 1) / per_wg : 1;
  p.n_partials = p.n_split * kFacWaves;
  return p;
}

size_t fac_workspace_bytes(const Common& c, const FacPlan& p) {
  const size_t acc_sz = c.bf16 ? sizeof(float) : sizeof(double);
  const size_t slots = size_t(c.batch) * c.n_q_heads * p.n_partials;
  return align256(slots * kHeadDim * acc_sz) + align256(slots * 2 * acc_sz);
}

size_t scores_bytes(const Common& c) {
  return align256(size_t(c.batch) * c.n_kv_heads * size_t(c.max_t) * sizeof(float));
}

hipError_t launch_fac(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, const int32_t* sel_idx,
                      const int32_t* sel_count, float* out, void* ws, hipStream_t s) {
  const size_t acc_sz = c.bf16 ? sizeof(float) : sizeof(double);
  const size_t slots = size_t(c.batch) * c.n_q_heads * p.n_partials;
  char* w = static_cast<char*>(ws);
  FacArgs a{c, p, q, k_pool, v_pool, block_table, sel_idx, sel_count,
            w, w + align256(slots * kHeadDim * acc_sz), out};
  if (c.bf16) return launch_fac_t<uint16_t, float>(a, s);
  return launch_fac_t<float, double>(a, s);
}

}  // namespace fasa
