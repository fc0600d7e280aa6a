// TOP-B: per (sequence, kv head), the B highest-scoring candidate tokens plus the
// forced tokens, as an ascending index list.
//
// T_t = TopK-I(S_t, N_fac) (paper-graph-ui review of FASA, section 3.4, token
// selection after TIP): the indices of the B largest scores.  Largest is signed;
// equal scores go to the lower token index; -0.0 equals +0.0.  The first n_sink
// and last n_recent cached tokens are always kept and the budget is spent on the
// rest, so the candidates are the contiguous range [c_lo, c_hi).
//
// Exact radix select on order-preserving 32-bit keys, in three stages.
//
// Stage 1, spread over the whole GPU: a coarse histogram of key bits 31..21
// (2048 bins) per unit.  In a decode step TIP builds it while its scores are
// still in registers; the standalone select builds it with hist_kernel.
//
// Stage 2, filter_kernel, one 256-thread workgroup per 2048 tokens of a unit:
// every workgroup reads the histogram and finds the bin b1 that holds the Bc-th
// largest key (Bc = budget capped by the candidates).  Every key in a bin >= b1
// is kept -- typically B plus a few hundred per unit -- and written with its
// token index, in index order, into the chunk's slot array; the chunk's count
// goes next to it, and b1 into a per-unit word.
//
// Stage 3, the exact select of one unit by one workgroup (select_core.hpp):
// the kept pairs are gathered into LDS, the second and third digits of the
// Bc-th largest key are found by radix passes over them, and a final pass
// keeps every key above it and, among keys equal to it, the lowest indices
// first.  Here that is finish_kernel (1024 threads per unit), which also writes
// the forced part of the list and zeroes the unit's histogram for the next
// call.  In a decode step with a small budget the FAC workgroups run stage 3
// themselves on their way to the attention (fac.hip), so no launch is spent on it.
//
// The histogram only narrows the search: any b1 keeps every key in bins >= b1,
// so whenever at least Bc keys are kept the Bc-th largest is among them.  If
// fewer than Bc are kept (a stale histogram) or more than LDS holds, stage 3
// falls back to a radix select over the whole row, so results never depend on
// the histogram's contents.
#include "select_core.hpp"

namespace fasa {
namespace {

using namespace sel;

constexpr int FNT = 256;                    // filter threads (8 tokens each)
constexpr int BIG = kTopkThreads;           // 1024 threads of finish_kernel
constexpr int64_t kFilterLateGrid = 2048;   // filter grids above which a chunk reads the length before its scores

struct TopkArgs {
  Common c;
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_idx;
  int32_t* sel_count;
  SelectBuffers w;
  uint32_t* fac_arrive;      // [units][head_chunks] FAC arrival counters to zero, or nullptr
  int head_chunks;
};

// The 8 scores of filter thread tid in the 2048-token chunk at `base`: two
// coalesced 1 KB-per-wave loads, slot e is token base + 1024 (e / 4) + 4 tid + e % 4.
// lim and VEC as in load_steps.
template <bool VEC>
__device__ __forceinline__ void load_chunk8(const float* row, int lim, int base, float (&v)[8]) {
  const int j0 = base + int(threadIdx.x) * 4;
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(row + min(j0 + 1024 * q, lim - 4));
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = row[min(j0 + 1024 * q + r, lim - 1)];
    }
  }
}
// Readable elements of a scores row for the loaders.
template <bool VEC>
__device__ __forceinline__ int row_lim(const Common& c) { return VEC ? c.score_stride : c.max_t; }
__device__ __forceinline__ int chunk8_index(int base, int e) {
  return base + (e >> 2) * 1024 + int(threadIdx.x) * 4 + (e & 3);
}

// The arrival counters of the FAC that follows this launch (one per head chunk).
__device__ __forceinline__ void zero_fac_arrive(const TopkArgs& a, int64_t unit) {
  if (a.fac_arrive != nullptr && int(threadIdx.x) < a.head_chunks) a.fac_arrive[unit * a.head_chunks + threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// Stage 1 for the standalone select: the unit histogram of given scores.
// Grid (ceil(max_t / 2048), kv heads, batch), 256 threads with 8 slots each.
// LATE as for filter_kernel: the length first, chunks without candidates leave
// before loading their scores.
template <bool VEC, bool LATE>
__global__ __launch_bounds__(FNT) void hist_kernel(TopkArgs a) {
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z;
  const int64_t unit = int64_t(b) * c.n_kv_heads + wg.y;
  const float* row = a.scores + unit * c.score_stride;
  const int base = wg.x * FCH;
  float v[8];
  if constexpr (!LATE) load_chunk8<VEC>(row, row_lim<VEC>(c), base, v);
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  if constexpr (LATE) {
    if (base >= c_hi || base + FCH <= c_lo) return;    // no candidate here: nothing to count
    load_chunk8<VEC>(row, row_lim<VEC>(c), base, v);
  }
  __shared__ uint32_t h[HB];
  for (int i = threadIdx.x; i < HB; i += FNT) h[i] = 0u;
  __syncthreads();
  RunHist rh;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = chunk8_index(base, e);
    rh.add(h, j >= c_lo && j < c_hi, score_key(v[e]) >> kHistShift);
  }
  rh.flush(h);
  __syncthreads();
  uint32_t* hg = a.w.hist + unit * HB;
  for (int i = threadIdx.x; i < HB; i += FNT) {
    const uint32_t x = h[i];
    if (x != 0u) atomicAdd(&hg[i], x);
  }
}

// ---------------------------------------------------------------------------
// Stage 2.  Grid (ceil(max_t / 2048), kv heads, batch), 256 threads.
// LATE (grids of several rounds): the sequence length comes first, and a chunk
// with no candidate (past a short sequence's end) writes its zero count and
// leaves without loading its scores; with several rounds of workgroups per CU
// the extra round trip is hidden by the others, and ragged batches stop reading
// the unused ends of their score rows.
template <bool VEC, bool LATE>
__global__ __launch_bounds__(FNT) void filter_kernel(TopkArgs a) {
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t unit = int64_t(b) * c.n_kv_heads + wg.y;
  const int nfa = filter_chunks(c);
  const float* row = a.scores + unit * c.score_stride;
  const int base = wg.x * FCH;

  // Independent loads: this thread's 8 scores and its 8 histogram bins.  Thread
  // t owns bins 2047-8t down to 2040-8t, so a scan over threads counts from the top.
  float v[8];
  if constexpr (!LATE) load_chunk8<VEC>(row, row_lim<VEC>(c), base, v);
  const uint32_t* hg = a.w.hist + unit * HB;
  const uint4 hlo = *reinterpret_cast<const uint4*>(hg + HB - 8 - 8 * tid);
  const uint4 hhi = *reinterpret_cast<const uint4*>(hg + HB - 4 - 8 * tid);
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  if (wg.x == 0) zero_fac_arrive(a, unit);
  if (Bc == nC) return;                // every candidate is kept: no kept-pair list
  if constexpr (LATE) {
    // Chunk 0 always finds b1 (it publishes it); any other chunk without a
    // candidate only records that it keeps nothing.
    if (wg.x != 0 && (base >= c_hi || base + FCH <= c_lo)) {
      if (tid == 0) a.w.counts[unit * nfa + wg.x] = 0;
      return;
    }
    load_chunk8<VEC>(row, row_lim<VEC>(c), base, v);
  }

  __shared__ uint32_t s_w[FNT / 64];
  __shared__ uint32_t s_b1;
  const uint32_t h[8] = {hhi.w, hhi.z, hhi.y, hhi.x, hlo.w, hlo.z, hlo.y, hlo.x};   // descending bins
  uint32_t hs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) hs += h[i];
  const uint32_t incl = wave_inclusive_scan(hs);
  if (lane == 63) s_w[wave] = incl;
  if (tid == 0) s_b1 = 0u;             // fewer than Bc keys counted: keep every candidate
  __syncthreads();
  uint32_t above = incl - hs;          // keys in bins above 2047-8t
#pragma unroll
  for (int w = 0; w < FNT / 64; ++w) above += (w < wave) ? s_w[w] : 0u;
  const uint32_t bc = uint32_t(Bc);
  // A consistent histogram has one crossing.  One that is not (stale counts,
  // whose 32-bit sums may wrap) can have several: the largest crossing bin wins,
  // so every chunk of the unit -- all reading the same histogram -- keeps from
  // the same b1, the one chunk 0 publishes.
  if (above < bc && bc <= above + hs) {
    uint32_t cum = above;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (cum < bc && bc <= cum + h[i]) atomicMax(&s_b1, uint32_t(HB - 1 - 8 * tid - i));
      cum += h[i];
    }
  }
  __syncthreads();
  const uint32_t b1 = s_b1;

  // Keep keys in bins >= b1; positions in index order (q, thread, slot) from one
  // packed block scan of the two per-step counts (each total <= 1024 fits 16 bits).
  uint32_t key[8];
  bool keep[8];
  uint32_t c0 = 0, c1 = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = chunk8_index(base, e);
    key[e] = score_key(v[e]);
    keep[e] = j >= c_lo && j < c_hi && (key[e] >> kHistShift) >= b1;
    if (e < 4) c0 += keep[e] ? 1u : 0u;
    else c1 += keep[e] ? 1u : 0u;
  }
  const uint32_t packed = c0 | (c1 << 16);
  const uint32_t pin = wave_inclusive_scan(packed);
  if (lane == 63) s_w[wave] = pin;     // the reads of s_w above all precede the last barrier
  __syncthreads();
  uint32_t ex = pin - packed, tot = 0;
#pragma unroll
  for (int w = 0; w < FNT / 64; ++w) {
    const uint32_t x = s_w[w];
    ex += (w < wave) ? x : 0u;
    tot += x;
  }
  const uint32_t tot0 = tot & 0xffffu, tot1 = tot >> 16;
  uint32_t pos0 = ex & 0xffffu, pos1 = tot0 + (ex >> 16);
  uint2* out = static_cast<uint2*>(a.w.slots) + (unit * nfa + wg.x) * int64_t(FCH);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t& pos = e < 4 ? pos0 : pos1;
    if (keep[e]) out[pos] = make_uint2(key[e], uint32_t(chunk8_index(base, e)));
    pos += keep[e] ? 1u : 0u;
  }
  if (tid == 0) {
    a.w.counts[unit * nfa + wg.x] = int32_t(tot0 + tot1);
    if (wg.x == 0) a.w.b1[unit] = int32_t(b1);
  }
}

// ---------------------------------------------------------------------------
// Stage 3 as its own launch: one 1024-thread workgroup per unit.  Grid (kv
// heads, batch).  Also the whole select when max_t == 0 (every unit keep-all).
struct FinishShared {
  SelState<BIG> sel;
  int32_t chunk_off[CPT * BIG + 1];
  uint32_t key[kCandLds];
  int32_t idx[kCandLds];
};

template <bool VEC>
__global__ __launch_bounds__(BIG) void finish_kernel(TopkArgs a) {
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.y, tid = threadIdx.x;
  const int64_t unit = int64_t(b) * c.n_kv_heads + wg.x;
  const int nfa = filter_chunks(c);
  const uint2* unit_slots = static_cast<const uint2*>(a.w.slots) + unit * nfa * int64_t(FCH);
  // Loads that do not depend on t_b go out first (clamped into the arrays),
  // among them the first 512 slots of this wave's chunk: large budgets keep
  // hundreds of pairs per chunk, which then need no second round trip.
  constexpr int DEEP = 8;
  uint2 pre[DEEP];
  prefetch_kept<BIG, 1, DEEP>(unit_slots, nfa, pre);
  int cnt[CPT];
  load_counts(a.w.counts + unit * nfa, nfa, cnt);
  const int b1 = a.w.b1[unit];
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  const int count = (t - nC) + Bc;          // forced + chosen, always <= cap
  const bool keep_all = Bc == nC;           // also every unit when max_t == 0
  int32_t* out = a.sel_idx + unit * c.cap;
  zero_fac_arrive(a, unit);
  if (!keep_all) {
    __shared__ FinishShared sm;
    select_from_kept<BIG, 1, VEC, DEEP>(sm.sel, sm.chunk_off, sm.key, sm.idx, kCandLds, unit_slots,
                                  a.scores + unit * c.score_stride, row_lim<VEC>(c), c.max_t, nfa, cnt, pre, c_lo,
                                  c_hi, Bc, b1, out + c_lo);
  }
  // Outputs that nothing above waits on go last: the forced part of the list,
  // its padding and count, and the consumed histogram (zero for the next step).
  for (int i = tid; i < c.cap; i += BIG) {
    if (i >= c_lo && i < c_lo + Bc && !keep_all) continue;
    out[i] = (i >= count) ? -1 : ((i < c_lo || keep_all) ? i : c_hi + (i - c_lo - Bc));
  }
  if (tid == 0) a.sel_count[unit] = count;
  uint4* hg = reinterpret_cast<uint4*>(a.w.hist + unit * HB);
  for (int i = tid; i < HB / 4; i += BIG) hg[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

size_t hist_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * HB * sizeof(uint32_t) + 255) & ~size_t(255);
}
size_t slots_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * filter_chunks(c) * FCH * sizeof(uint2) + 255) & ~size_t(255);
}
size_t counts_bytes(const Common& c) {
  // Per-chunk counts of the filter (4 bytes per 2048-token chunk) or the
  // summaries of TIP's emitted lists (8 bytes per 1024-token chunk).
  const size_t fb = size_t(filter_chunks(c)) * sizeof(int32_t), eb = size_t(emit_chunks(c)) * sizeof(uint2);
  return (size_t(c.batch) * c.n_kv_heads * (eb > fb ? eb : fb) + 255) & ~size_t(255);
}

hipError_t launch_filter(const Common& c, const float* scores, const int32_t* seq_lens, const SelectBuffers& w,
                         bool have_hist, uint32_t* fac_arrive, int head_chunks, hipStream_t s, bool rows_full) {
  if (c.max_t == 0) return hipSuccess;
  const TopkArgs a{c, scores, seq_lens, nullptr, nullptr, w, fac_arrive, head_chunks};
  const dim3 grid(filter_chunks(c), c.n_kv_heads, c.batch);
  const bool vec = (c.score_stride & 3) == 0;
  // Grids of more than one round of workgroups (8 per CU): load the length
  // first and skip chunks without candidates (measured on the ragged batch),
  // unless the caller expects every row to run to max_t, where there is
  // nothing to skip (one calibration sequence of 32768 tokens, 8320
  // workgroups: 135.2 -> 134.7 us per call).
  const bool late = !rows_full && int64_t(grid.x) * grid.y * grid.z > kFilterLateGrid;
  if (!have_hist) {
    if (vec) {
      if (late) hipLaunchKernelGGL((hist_kernel<true, true>), grid, dim3(FNT), 0, s, a);
      else hipLaunchKernelGGL((hist_kernel<true, false>), grid, dim3(FNT), 0, s, a);
    } else {
      if (late) hipLaunchKernelGGL((hist_kernel<false, true>), grid, dim3(FNT), 0, s, a);
      else hipLaunchKernelGGL((hist_kernel<false, false>), grid, dim3(FNT), 0, s, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (vec) {
    if (late) hipLaunchKernelGGL((filter_kernel<true, true>), grid, dim3(FNT), 0, s, a);
    else hipLaunchKernelGGL((filter_kernel<true, false>), grid, dim3(FNT), 0, s, a);
  } else {
    if (late) hipLaunchKernelGGL((filter_kernel<false, true>), grid, dim3(FNT), 0, s, a);
    else hipLaunchKernelGGL((filter_kernel<false, false>), grid, dim3(FNT), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_finish(const Common& c, const float* scores, const int32_t* seq_lens, int32_t* sel_idx,
                         int32_t* sel_count, const SelectBuffers& w, uint32_t* fac_arrive, int head_chunks,
                         hipStream_t s) {
  const TopkArgs a{c, scores, seq_lens, sel_idx, sel_count, w, fac_arrive, head_chunks};
  if ((c.score_stride & 3) == 0)
    hipLaunchKernelGGL(finish_kernel<true>, dim3(c.n_kv_heads, c.batch), dim3(BIG), 0, s, a);
  else
    hipLaunchKernelGGL(finish_kernel<false>, dim3(c.n_kv_heads, c.batch), dim3(BIG), 0, s, a);
  return hipGetLastError();
}

}  // namespace fasa
