// TOP-B: per (sequence, kv head), the B highest-scoring candidate tokens plus the
// forced tokens, as an ascending index list.
//
// T_t = TopK-I(S_t, N_fac) (paper-graph-ui review of FASA, section 3.4, token
// selection after TIP): the indices of the B largest scores.  Largest is signed;
// equal scores go to the lower token index; -0.0 equals +0.0.  The first n_sink
// and last n_recent cached tokens are always kept and the budget is spent on the
// rest, so the candidates are the contiguous range [c_lo, c_hi).
//
// Exact radix select on order-preserving 32-bit keys, in two stages.
//
// Stage 1, spread over the whole GPU: a coarse histogram of key bits 31..21
// (2048 bins) per unit.  In a decode step TIP builds it while its scores are
// still in registers; the standalone select builds it with hist_kernel.
//
// Stage 2, one workgroup of 1024 threads per unit (select_kernel): the bin b1
// that holds the Bc-th largest key is read off the histogram.  Every key in a
// bin >= b1 is a candidate -- typically B plus a few hundred -- and is copied,
// in index order, with its index into LDS.  Three radix passes (11, 11, 10 bits)
// over the LDS candidates find the exact Bc-th largest key; a final pass keeps
// every key above it and, among keys equal to it, the lowest indices first (the
// tie rule), writing the indices ascending.  The unit's histogram is zeroed for
// the next call.
//
// The histogram only narrows the search: if the candidates found are fewer than
// Bc (a stale histogram) or more than LDS holds, the workgroup falls back to a
// radix select over the whole row, so results never depend on it.
//
// Layout inside the workgroup: a row is walked in chunks of 32768 tokens; in a
// chunk, wave w owns the 2048 tokens from 2048 w, and at step q (0..7) lane l
// holds the 4 consecutive tokens from 256 q + 4 l.  Every load instruction thus
// reads 1 KB of consecutive scores (one 16-byte vector per lane), and index
// order is (chunk, wave, q, lane, slot): ranks come from one 64-lane scan per
// step and one scan over the 16 waves.  Rows of at most 32768 tokens are loaded
// once (eight 16-byte loads per thread, all in flight before the sequence
// length is known) and stay in registers; longer rows are re-read from L2
// chunk by chunk.  A key of 0 marks a slot that is not a candidate.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

constexpr int NT = kTopkThreads;            // 1024
constexpr int NW = NT / 64;                 // 16 waves
constexpr int KPT = kTopkLdsKeys / NT;      // 32 consecutive slots per thread per chunk
constexpr int CHUNK = NT * KPT;             // 32768 tokens
constexpr int HB = kHistBins;               // 2048

struct TopkArgs {
  Common c;
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_idx;
  int32_t* sel_count;
  uint32_t* hist;            // [units][2048]
};

struct Shared {
  uint32_t hist[HB];
  uint32_t wave_sum[NW];
  uint32_t digit, rem, full;
  uint32_t cand_key[kCandLds];
  int32_t cand_idx[kCandLds];
};

// Block-wide exclusive scan of one value per thread; returns the exclusive
// prefix and writes the block total.
__device__ __forceinline__ uint32_t block_excl_scan(Shared& s, uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) s.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = s.wave_sum[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Exclusive prefix over the 16 waves of a per-wave value (the same in every lane
// of a wave); also returns the block total.
__device__ __forceinline__ uint32_t wave_base(Shared& s, uint32_t wave_val, uint32_t& total) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s.wave_sum[wave] = wave_val;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t x = s.wave_sum[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base;
}

// Find the digit d of a histogram with nb <= 2048 bins such that fewer than rem
// keys lie in bins above d and at least rem in bins >= d.  Thread t owns bins
// nb-1-2t and nb-2-2t (descending order), so an inclusive scan over threads
// counts keys from the top.  Leaves s.digit untouched when there are fewer
// than rem keys in total.
__device__ __forceinline__ void find_digit(Shared& s, int nb, uint32_t rem) {
  const int tid = threadIdx.x;
  const int hi = nb - 1 - 2 * tid, lo = hi - 1;
  const uint32_t ch = hi >= 0 ? s.hist[hi] : 0u;
  const uint32_t cl = lo >= 0 ? s.hist[lo] : 0u;
  uint32_t total;
  const uint32_t incl = block_excl_scan(s, ch + cl, total) + ch + cl;   // keys in bins >= lo
  const uint32_t above_hi = incl - ch - cl;                            // keys in bins > hi
  if (hi >= 0 && above_hi < rem && rem <= above_hi + ch) {
    s.digit = uint32_t(hi);
    s.rem = rem - above_hi;
    s.full = (ch == rem - above_hi) ? 1u : 0u;
  } else if (lo >= 0 && above_hi + ch < rem && rem <= incl) {
    s.digit = uint32_t(lo);
    s.rem = rem - above_hi - ch;
    s.full = (cl == rem - above_hi - ch) ? 1u : 0u;
  }
  __syncthreads();
}

// Run-length histogram of one lane's slots: consecutive active slots in the same
// bin are counted in a register and added once, so tied or skewed scores do not
// serialise on one LDS address.
struct RunHist {
  uint32_t bin = 0u, cnt = 0u;
  __device__ __forceinline__ void add(uint32_t* hist, bool active, uint32_t b) {
    const bool brk = active && b != bin;
    if (brk && cnt != 0u) atomicAdd(&hist[bin], cnt);
    cnt = brk ? 1u : cnt + (active ? 1u : 0u);
    bin = brk ? b : bin;
  }
  __device__ __forceinline__ void flush(uint32_t* hist) {
    if (cnt != 0u) atomicAdd(&hist[bin], cnt);
  }
};

// Keeps the scheduler from hoisting the per-slot comparisons of the unrolled
// slot loops above each other (each is a 64-bit lane mask in scalar registers).
__device__ __forceinline__ void slot_fence() { __builtin_amdgcn_sched_barrier(0); }

// Token index of slot (q, r) of this lane in the tile that starts at `base`.
__device__ __forceinline__ int tile_index(int base, int q, int r) {
  return base + (threadIdx.x >> 6) * 2048 + q * 256 + (threadIdx.x & 63) * 4 + r;
}

// Raw scores of this lane's 32 slots of the tile at `base`, loaded without
// branches (indices clamped into the row).
__device__ __forceinline__ void load_tile(const float* row, int max_t, int base, float (&v)[KPT]) {
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    const int j = tile_index(base, q, 0);
    if ((max_t & 3) == 0) {
      // A clamped vector only ever covers slots >= max_t, which are never used.
      const float4 x = *reinterpret_cast<const float4*>(row + min(j, max_t - 4));
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = row[min(j + r, max_t - 1)];
    }
  }
}

// Index-order placement of flagged slots of a tile.  For each step q, lane l's
// offset of its first flagged slot among the wave's flagged slots, and the
// wave's total.  Uses one 64-lane scan per step.
template <typename Flag>
__device__ __forceinline__ uint32_t tile_offsets(Flag flag, uint32_t (&qoff)[KPT / 4]) {
  uint32_t run = 0;
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    uint32_t cq = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) cq += flag(4 * q + r) ? 1u : 0u;
    const uint32_t incl = wave_inclusive_scan(cq);
    qoff[q] = run + incl - cq;
    run += wave_last(incl);
  }
  return run;
}

__device__ __forceinline__ void unit_range(const Common& c, int t_raw, int& t, int& c_lo, int& c_hi) {
  t = clamp_len(t_raw, c.max_t, c.max_blocks);
  c_lo = min(c.n_sink, t);
  c_hi = max(c_lo, t - c.n_recent);
}

// ---------------------------------------------------------------------------
// Stage 1 for the standalone select: the unit histogram of given scores.
// Grid (ceil(max_t / 2048), kv heads, batch), 256 threads with 8 slots each.
__global__ __launch_bounds__(256) void hist_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.z;
  const int64_t unit = int64_t(b) * c.n_kv_heads + blockIdx.y;
  const float* row = a.scores + unit * c.max_t;
  float v[8];
#pragma unroll
  for (int q = 0; q < 2; ++q) {          // two coalesced 1 KB-per-wave loads
    const int j = blockIdx.x * 2048 + q * 1024 + threadIdx.x * 4;
    if ((c.max_t & 3) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(row + min(j, c.max_t - 4));
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = row[min(j + r, c.max_t - 1)];
    }
  }
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  __shared__ uint32_t h[HB];
  for (int i = threadIdx.x; i < HB; i += 256) h[i] = 0u;
  __syncthreads();
  RunHist rh;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = blockIdx.x * 2048 + (e >> 2) * 1024 + threadIdx.x * 4 + (e & 3);
    rh.add(h, j >= c_lo && j < c_hi, score_key(v[e]) >> kHistShift);
  }
  rh.flush(h);
  __syncthreads();
  uint32_t* hg = a.hist + unit * HB;
  for (int i = threadIdx.x; i < HB; i += 256) {
    const uint32_t x = h[i];
    if (x != 0u) atomicAdd(&hg[i], x);
  }
}

// ---------------------------------------------------------------------------
// Stage 2.
template <bool RESIDENT>
__global__ __launch_bounds__(NT) void select_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;
  const float* row = a.scores + unit * c.max_t;
  uint32_t* hg = a.hist + unit * HB;
  const int nchunks = RESIDENT ? 1 : (c.max_t + CHUNK - 1) / CHUNK;

  // Loads that do not depend on t_b go out first: the histogram and, for
  // resident rows, the whole row.
  const uint32_t h0 = hg[tid], h1 = hg[tid + NT];
  float pre[RESIDENT ? KPT : 1];
  if constexpr (RESIDENT) load_tile(row, c.max_t, 0, pre);

  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  const int count = (t - nC) + Bc;          // forced + chosen, always <= cap
  int32_t* out = a.sel_idx + unit * c.cap;

  // The histogram is consumed: leave it zero for the next step.
  hg[tid] = 0u;
  hg[tid + NT] = 0u;

  // Forced prefix [0, c_lo), forced suffix [c_hi, t) placed after the Bc chosen,
  // and -1 padding.  When every candidate is kept the list is 0..count-1.
  const bool keep_all = (Bc == nC);
  for (int i = tid; i < c.cap; i += NT) {
    int val;
    if (i >= count) val = -1;
    else if (i < c_lo || keep_all) val = i;
    else if (i >= c_lo + Bc) val = c_hi + (i - c_lo - Bc);
    else continue;
    out[i] = val;
  }
  if (tid == 0) a.sel_count[unit] = count;
  if (keep_all) return;

  __shared__ Shared s;
  uint32_t k[KPT];
  if constexpr (RESIDENT) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = tile_index(0, e >> 2, e & 3);
      k[e] = (j >= c_lo && j < c_hi) ? score_key(pre[e]) : 0u;
    }
  }
  // This thread's keys of chunk ch (loaded again for streamed rows).
  auto keys_of = [&](int ch) {
    if constexpr (!RESIDENT) {
      float v[KPT];
      load_tile(row, c.max_t, ch * CHUNK, v);
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const int j = tile_index(ch * CHUNK, e >> 2, e & 3);
        k[e] = (j >= c_lo && j < c_hi) ? score_key(v[e]) : 0u;
      }
    }
  };

  // ---- bin b1 of the Bc-th largest key, from the histogram
  s.hist[tid] = h0;
  s.hist[tid + NT] = h1;
  if (tid == 0) s.digit = 0u;
  __syncthreads();
  find_digit(s, HB, uint32_t(Bc));
  const uint32_t b1 = s.digit;

  // ---- candidates (bin >= b1) into LDS, in index order
  uint32_t n_cand = 0;
  for (int ch = 0; ch < nchunks; ++ch) {
    keys_of(ch);
    auto in = [&](int e) { return k[e] != 0u && (k[e] >> kHistShift) >= b1; };
    uint32_t qoff[KPT / 4];
    const uint32_t wtot = tile_offsets(in, qoff);
    uint32_t tot;
    const uint32_t wbase = n_cand + wave_base(s, wtot, tot);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      uint32_t pos = wbase + qoff[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * q + r;
        const bool f = in(e);
        if (f && pos < uint32_t(kCandLds)) {
          s.cand_key[pos] = k[e];
          s.cand_idx[pos] = tile_index(ch * CHUNK, q, r);
        }
        pos += f ? 1u : 0u;
      }
      slot_fence();
    }
    n_cand += tot;
  }
  __syncthreads();

  uint32_t prefix = 0, pmask = 0, rem = uint32_t(Bc);
  if (n_cand >= uint32_t(Bc) && n_cand <= uint32_t(kCandLds)) {
    // ---- exact select among the LDS candidates.  Thread t owns a contiguous run.
    const int N = int(n_cand);
    const int per = (N + NT - 1) / NT;
    const int i0 = min(N, tid * per), i1 = min(N, i0 + per);
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      const uint32_t dmask = uint32_t(nb - 1);
      for (int i = tid; i < nb; i += NT) s.hist[i] = 0u;
      __syncthreads();
      RunHist rh;
      for (int i = i0; i < i1; ++i) {
        const uint32_t key = s.cand_key[i];
        rh.add(s.hist, (key & pmask) == prefix, (key >> shift) & dmask);
      }
      rh.flush(s.hist);
      __syncthreads();
      find_digit(s, nb, rem);
      const uint32_t d = s.digit, full = s.full;
      rem = s.rem;
      prefix |= d << shift;
      pmask |= dmask << shift;
      if (full) break;
    }
    uint32_t n_gt = 0, n_eq = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t m = s.cand_key[i] & pmask;
      n_gt += m > prefix ? 1u : 0u;
      n_eq += m == prefix ? 1u : 0u;
    }
    uint32_t eq_tot, sel_tot;
    const uint32_t eq_base = block_excl_scan(s, n_eq, eq_tot);
    const uint32_t take_eq = (rem > eq_base) ? min(rem - eq_base, n_eq) : 0u;
    int pos = c_lo + int(block_excl_scan(s, n_gt + take_eq, sel_tot));
    uint32_t eq_seen = eq_base;
    for (int i = i0; i < i1; ++i) {
      const uint32_t m = s.cand_key[i] & pmask;
      const bool eq = m == prefix;
      const bool take = m > prefix || (eq && eq_seen < rem);
      eq_seen += eq ? 1u : 0u;
      if (take && pos < c_lo + Bc) out[pos] = s.cand_idx[i];   // the guard never fails when the counts agree
      pos += take ? 1 : 0;
    }
    return;
  }

  // ---- fallback: radix select over the whole row (a stale histogram, or more
  // candidates than LDS holds).  A bound from group maxima prunes the first pass:
  // the Bc-th largest of the maxima of >= Bc disjoint slot groups is <= the Bc-th
  // largest key.
  uint32_t b_lo = 0;
  {
    const int64_t groups_needed = (int64_t(Bc) + int64_t(NT) * nchunks - 1) / (int64_t(NT) * nchunks);
    int gpt = 1;                               // groups per thread per chunk, a power of two
    while (gpt < KPT && gpt < groups_needed) gpt <<= 1;
    const int G = KPT / gpt;
    for (int i = tid; i < HB; i += NT) s.hist[i] = 0u;
    if (tid == 0) s.digit = 0u;
    __syncthreads();
    RunHist rh;
    for (int ch = 0; ch < nchunks; ++ch) {
      keys_of(ch);
      uint32_t gmax = 0;
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        gmax = max(gmax, k[e]);
        const bool end = ((e + 1) & (G - 1)) == 0;
        rh.add(s.hist, end, gmax >> kHistShift);
        gmax = end ? 0u : gmax;
        slot_fence();
      }
    }
    rh.flush(s.hist);
    __syncthreads();
    find_digit(s, HB, uint32_t(Bc));          // digit stays 0 with fewer than Bc groups
    b_lo = s.digit;
  }
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    const uint32_t dmask = uint32_t(nb - 1);
    const uint32_t lo_bin = pass == 0 ? b_lo : 0u;
    for (int i = tid; i < nb; i += NT) s.hist[i] = 0u;
    __syncthreads();
    RunHist rh;
    for (int ch = 0; ch < nchunks; ++ch) {
      keys_of(ch);
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const uint32_t key = k[e];
        const bool act = key != 0u && (key & pmask) == prefix && (key >> kHistShift) >= lo_bin;
        rh.add(s.hist, act, (key >> shift) & dmask);
        slot_fence();
      }
    }
    rh.flush(s.hist);
    __syncthreads();
    find_digit(s, nb, rem);
    const uint32_t d = s.digit, full = s.full;
    rem = s.rem;
    prefix |= d << shift;
    pmask |= dmask << shift;
    if (full) break;
  }
  // Index-order compaction.  First the rank of every key equal to the prefix
  // among the equal keys (the first rem of them are taken), then the output
  // position of every taken key.
  uint32_t eq_run = 0, sel_run = 0;
  for (int ch = 0; ch < nchunks; ++ch) {
    keys_of(ch);
    auto is_gt = [&](int e) { return k[e] != 0u && (k[e] & pmask) > prefix; };
    auto is_eq = [&](int e) { return k[e] != 0u && (k[e] & pmask) == prefix; };
    uint32_t eoff[KPT / 4];
    const uint32_t ewt = tile_offsets(is_eq, eoff);
    uint32_t eq_tot;
    const uint32_t ebase = eq_run + wave_base(s, ewt, eq_tot);
    // take(e): above the prefix, or equal with an equal-rank below rem
    uint32_t take_bits = 0;
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      uint32_t er = ebase + eoff[q];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = 4 * q + r;
        const bool eq = is_eq(e);
        const bool take = is_gt(e) || (eq && er < rem);
        er += eq ? 1u : 0u;
        take_bits |= take ? (1u << e) : 0u;
      }
      slot_fence();
    }
    auto taken = [&](int e) { return ((take_bits >> e) & 1u) != 0u; };
    uint32_t toff[KPT / 4];
    const uint32_t twt = tile_offsets(taken, toff);
    uint32_t sel_tot;
    const uint32_t tbase = sel_run + wave_base(s, twt, sel_tot);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      int pos = c_lo + int(tbase + toff[q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool tk = taken(4 * q + r);
        if (tk && pos < c_lo + Bc) out[pos] = tile_index(ch * CHUNK, q, r);   // the guard never fails when the counts agree
        pos += tk ? 1 : 0;
      }
      slot_fence();
    }
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
}

}  // namespace

size_t hist_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * HB * sizeof(uint32_t) + 255) & ~size_t(255);
}

hipError_t launch_topk(const Common& c, const float* scores, const int32_t* seq_lens,
                       int32_t* sel_idx, int32_t* sel_count, uint32_t* hist, bool have_hist,
                       hipStream_t s) {
  TopkArgs a{c, scores, seq_lens, sel_idx, sel_count, hist};
  if (!have_hist && c.max_t > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3((c.max_t + 2047) / 2048, c.n_kv_heads, c.batch), dim3(256), 0, s,
                       a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(c.n_kv_heads, c.batch);
  if (c.max_t <= CHUNK)
    hipLaunchKernelGGL(select_kernel<true>, grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(select_kernel<false>, grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace fasa
