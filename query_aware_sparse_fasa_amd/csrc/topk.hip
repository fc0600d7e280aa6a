// TOP-B: per (sequence, kv head), the B highest-scoring candidate tokens plus the
// forced tokens, as an ascending index list.
//
// T_t = TopK-I(S_t, N_fac) (paper-graph-ui review of FASA, section 3.4, token
// selection after TIP): the indices of the B largest scores.  Largest is signed;
// equal scores go to the lower token index; -0.0 equals +0.0.  The first n_sink
// and last n_recent cached tokens are always kept and the budget is spent on the
// rest, so the candidates are the contiguous range [c_lo, c_hi).
//
// Method: exact radix select on order-preserving 32-bit keys, 8 bits per pass
// from the top, one workgroup (16 waves) per unit.  Each pass histograms the
// keys that still match the chosen prefix (one LDS histogram per wave, so only
// lanes of one wave contend), then the digit holding the B-th largest key is
// found by a suffix scan of the 256 bins.  A pass stops early when the whole
// boundary bin is taken.  The result is a key prefix P (under mask M) and the
// number r of keys equal to P under M that are still needed.  A final pass in
// index order keeps every key above P and the first r keys equal to P -- that
// is the lower-index tie rule, and it emits the indices already ascending.
// Candidates are staged once in LDS (160 KB per CU on gfx950) when they fit;
// longer contexts re-read the fp32 scores from L2 on every pass.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

constexpr int NT = kTopkThreads;
constexpr int NW = NT / 64;

struct TopkArgs {
  Common c;
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_idx;
  int32_t* sel_count;
};

// Exclusive scan of one value per wave (NW values) held by lane 0 of each wave;
// every thread gets its wave's exclusive prefix and the total.
__device__ __forceinline__ void wave_values_scan(uint32_t* sh, int wave, uint32_t mine,
                                                 uint32_t& excl, uint32_t& total) {
  if ((threadIdx.x & 63) == 0) sh[wave] = mine;
  __syncthreads();
  uint32_t e = 0, s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t v = sh[w];
    e += (w < wave) ? v : 0u;
    s += v;
  }
  excl = e;
  total = s;
  __syncthreads();
}

template <bool STAGED>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = clamp_len(a.seq_lens[b], c.max_t, c.max_blocks);
  const int c_lo = min(c.n_sink, t);
  const int c_hi = max(c_lo, t - c.n_recent);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  const int count = (t - nC) + Bc;          // forced + chosen, always <= cap
  int32_t* out = a.sel_idx + (int64_t(b) * c.n_kv_heads + g) * c.cap;

  // Forced prefix [0, c_lo), forced suffix [c_hi, t) placed after the Bc chosen,
  // and -1 padding.  When every candidate is kept the chosen part is [c_lo, c_hi)
  // itself, so the whole list is 0..count-1.
  const bool keep_all = (Bc == nC);
  for (int i = tid; i < c.cap; i += NT) {
    int v;
    if (i >= count) v = -1;
    else if (i < c_lo || keep_all) v = i;
    else if (i >= c_lo + Bc) v = c_hi + (i - c_lo - Bc);
    else continue;
    out[i] = v;
  }
  if (tid == 0) a.sel_count[int64_t(b) * c.n_kv_heads + g] = count;
  if (keep_all) return;

  __shared__ uint32_t hist[NW][256];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t sh_scan[NW];
  __shared__ uint32_t sh_digit, sh_rem, sh_full;
  __shared__ uint32_t keys[STAGED ? kTopkLdsKeys : 1];

  const float* row = a.scores + (int64_t(b) * c.n_kv_heads + g) * c.max_t + c_lo;
  if constexpr (STAGED) {
    for (int i = tid; i < nC; i += NT) keys[i] = score_key(row[i]);
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (STAGED) return keys[i];
    else return score_key(row[i]);
  };

  uint32_t prefix = 0, pmask = 0, rem = uint32_t(Bc);
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NW * 256; i += NT) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < nC; i += NT) {
      const uint32_t k = key_at(i);
      if ((k & pmask) == prefix) atomicAdd(&hist[wave][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      // Bins in descending digit order: thread tid looks at digit 255 - tid.
      const int d = 255 - tid;
      uint32_t n = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) n += hist[w][d];
      tot[d] = n;
      const uint32_t incl = wave_inclusive_scan(n);
      if (lane == 63) sh_scan[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      const int d = 255 - tid;
      uint32_t base = 0;
      for (int w = 0; w < wave; ++w) base += sh_scan[w];
      const uint32_t n = tot[d];
      const uint32_t incl = wave_inclusive_scan(n) + base;   // keys with digit >= d
      const uint32_t above = incl - n;                       // keys with digit > d
      if (above < rem && rem <= incl) {
        sh_digit = uint32_t(d);
        sh_rem = rem - above;
        sh_full = (n == rem - above) ? 1u : 0u;
      }
    }
    __syncthreads();
    const uint32_t d = sh_digit;
    rem = sh_rem;
    prefix |= d << shift;
    pmask |= 0xFFu << shift;
    if (sh_full) break;
  }

  // Index-order compaction: wave w owns a contiguous run of candidates.
  const int per_wave = ((nC + NW - 1) / NW + 63) & ~63;
  const int w0 = min(nC, wave * per_wave), w1 = min(nC, w0 + per_wave);
  uint32_t n_gt = 0, n_eq = 0;
  for (int base = w0; base < w1; base += 64) {
    const int i = base + lane;
    const bool valid = i < w1;
    const uint32_t k = valid ? (key_at(i) & pmask) : 0u;
    n_gt += __popcll(__ballot(valid && k > prefix));
    n_eq += __popcll(__ballot(valid && k == prefix));
  }
  uint32_t eq_before, eq_total;
  wave_values_scan(sh_scan, wave, n_eq, eq_before, eq_total);
  const uint32_t take_eq = (rem > eq_before) ? min(rem - eq_before, n_eq) : 0u;
  uint32_t sel_before, sel_total;
  wave_values_scan(sh_scan, wave, n_gt + take_eq, sel_before, sel_total);

  int pos = c_lo + int(sel_before);
  uint32_t eq_seen = eq_before;
  for (int base = w0; base < w1; base += 64) {
    const int i = base + lane;
    const bool valid = i < w1;
    const uint32_t k = valid ? (key_at(i) & pmask) : 0u;
    const bool gt = valid && k > prefix;
    const bool eq = valid && k == prefix;
    const uint64_t eq_mask = __ballot(eq);
    const bool take = gt || (eq && (eq_seen + uint32_t(lanes_below(eq_mask))) < rem);
    const uint64_t take_mask = __ballot(take);
    const int at = pos + lanes_below(take_mask);
    if (take && at < c_lo + Bc) out[at] = c_lo + i;   // the guard never fails when the counts agree
    pos += __popcll(take_mask);
    eq_seen += __popcll(eq_mask);
  }
}

}  // namespace

hipError_t launch_topk(const Common& c, const float* scores, const int32_t* seq_lens,
                       int32_t* sel_idx, int32_t* sel_count, hipStream_t s) {
  TopkArgs a{c, scores, seq_lens, sel_idx, sel_count};
  const dim3 grid(c.n_kv_heads, c.batch);
  if (c.max_t <= kTopkLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace fasa
