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
// goes next to it.
//
// Stage 3, the exact select of one unit by one workgroup: the kept pairs of all
// chunks are gathered into LDS (still in index order).  Three radix passes (11,
// 11, 10 bits) over them find the exact Bc-th largest key; a final pass keeps
// every key above it and, among keys equal to it, the lowest indices first (the
// tie rule), writing the indices ascending.  The unit's histogram is zeroed for
// the next call.  For small budgets the last filter workgroup of a unit to
// finish (counted with an atomic arrival counter) runs stage 3 itself, so no
// further launch is needed; for large budgets finish_kernel, 1024 threads per
// unit with a larger LDS area, runs it.
//
// The histogram only narrows the search: any b1 keeps every key in bins >= b1,
// so whenever at least Bc keys are kept the Bc-th largest is among them.  If
// fewer than Bc are kept (a stale histogram) or more than LDS holds, stage 3
// falls back to a radix select over the whole row, so results never depend on
// the histogram's contents.  The arrival counters are zeroed by the kernel
// that runs before the filter (TIP, or hist_kernel), never assumed zero.
//
// Fallback layout: a row is walked in tiles of 16 slots per thread; in a tile,
// wave w owns 1024 consecutive tokens and at step q (0..3) lane l holds the 4
// consecutive tokens from 256 q + 4 l.  Every load instruction thus reads 1 KB
// of consecutive scores, and index order is (tile, wave, q, lane, slot): ranks
// come from one 64-lane scan per step and one scan over the waves.
#include <type_traits>

#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

constexpr int HB = kHistBins;               // 2048
constexpr int FCH = kFilterChunk;           // 2048 tokens per filter workgroup
constexpr int FNT = 256;                    // filter threads (8 tokens each)
constexpr int BIG = kTopkThreads;           // 1024 threads of finish_kernel
constexpr int KPT = 16;                     // fallback slots per thread per tile
constexpr int CPT = 4;                      // chunk counts summed per thread in the gather

struct TopkArgs {
  Common c;
  const float* scores;
  const int32_t* seq_lens;
  int32_t* sel_idx;
  int32_t* sel_count;
  uint32_t* hist;            // [units][2048]
  uint2* slots;              // [units][nfa * 2048] kept (key, token) pairs per chunk
  int32_t* counts;           // [units][nfa] kept pairs per chunk
  uint32_t* arrive;          // [units] filter workgroups done (zeroed before the filter)
  uint32_t* fac_arrive;      // [units][head_chunks] FAC arrival counters to zero, or nullptr
  int head_chunks;
};

// Filter chunks of a row (at least one, so that slot and count arrays are never
// empty and clamped loads from them stay in bounds).
__host__ __device__ __forceinline__ int filter_chunks(const Common& c) {
  const int n = (c.max_t + FCH - 1) / FCH;
  return n > 0 ? n : 1;
}

template <int NTH>
struct SelState {
  alignas(16) uint32_t hist[HB];
  uint32_t wave_sum[NTH / 64];
  uint32_t digit, rem, full, above;
};

// Block-wide exclusive scan of one value per thread; returns the exclusive
// prefix and writes the block total.
template <int NTH>
__device__ __forceinline__ uint32_t block_excl_scan(SelState<NTH>& s, uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) s.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const uint32_t x = s.wave_sum[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// Exclusive prefix over the waves of a per-wave value (the same in every lane
// of a wave); also returns the block total.
template <int NTH>
__device__ __forceinline__ uint32_t wave_base(SelState<NTH>& s, uint32_t wave_val, uint32_t& total) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s.wave_sum[wave] = wave_val;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const uint32_t x = s.wave_sum[w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base;
}

// Find the digit d of a histogram with NB bins (1024 or 2048) such that fewer
// than rem keys lie in bins above d and at least rem in bins >= d.  Thread t
// owns the BPT bins below NB - BPT t (read as 16-byte vectors when BPT >= 4);
// an exclusive scan over threads counts the keys above them, and the thread
// whose bins hold the crossing walks them in registers.  Leaves s.digit
// untouched when there are fewer than rem keys in total.
template <int NTH, int NB>
__device__ __forceinline__ void find_digit(SelState<NTH>& s, uint32_t rem) {
  constexpr int BPT = NB > NTH ? NB / NTH : 1;
  const int lo = NB - BPT * (int(threadIdx.x) + 1);     // lowest owned bin
  uint32_t h[BPT];
  if constexpr (BPT >= 4) {
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) {
      const uint4 x = reinterpret_cast<const uint4*>(s.hist + lo)[v];
      h[4 * v + 0] = x.x; h[4 * v + 1] = x.y; h[4 * v + 2] = x.z; h[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BPT; ++i) h[i] = lo + i >= 0 ? s.hist[lo + i] : 0u;
  }
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += h[i];
  uint32_t total;
  const uint32_t above = block_excl_scan(s, sum, total);    // keys in bins above the owned ones
  if (above < rem && rem <= above + sum) {
    uint32_t cum = above;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (cum < rem && rem <= cum + h[i]) {
        s.digit = uint32_t(lo + i);
        s.rem = rem - cum;
        s.full = (h[i] == rem - cum) ? 1u : 0u;
      }
      cum += h[i];
    }
  }
  __syncthreads();
}

template <int NTH, int NB>
__device__ __forceinline__ void zero_bins(SelState<NTH>& s) {
  for (int i = threadIdx.x; i < NB / 4; i += NTH) reinterpret_cast<uint4*>(s.hist)[i] = make_uint4(0u, 0u, 0u, 0u);
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

// Token index of slot (q, r) of this lane in the fallback tile that starts at `base`.
__device__ __forceinline__ int tile_index(int base, int q, int r) {
  return base + (threadIdx.x >> 6) * (64 * KPT) + q * 256 + (threadIdx.x & 63) * 4 + r;
}

// Raw scores of this lane's KPT slots of the tile at `base`, loaded without
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

// The 8 scores of filter thread tid in the 2048-token chunk at `base`: two
// coalesced 1 KB-per-wave loads, slot e is token base + 1024 (e / 4) + 4 tid + e % 4.
__device__ __forceinline__ void load_chunk8(const float* row, int max_t, int base, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = base + q * 1024 + threadIdx.x * 4;
    if ((max_t & 3) == 0) {
      const float4 x = *reinterpret_cast<const float4*>(row + min(j, max_t - 4));
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = row[min(j + r, max_t - 1)];
    }
  }
}
__device__ __forceinline__ int chunk8_index(int base, int e) {
  return base + (e >> 2) * 1024 + int(threadIdx.x) * 4 + (e & 3);
}

// The fixed part of a unit's list: forced prefix [0, c_lo), forced suffix
// [c_hi, t) placed after the Bc chosen, -1 padding up to cap, and the count.
// When every candidate is kept the list is 0..count-1.
template <int NTH>
__device__ __forceinline__ void write_fixed(const TopkArgs& a, int64_t unit, int t, int c_lo, int c_hi,
                                            int Bc) {
  const Common& c = a.c;
  const int nC = c_hi - c_lo;
  const int count = (t - nC) + Bc;          // forced + chosen, always <= cap
  const bool keep_all = (Bc == nC);
  int32_t* out = a.sel_idx + unit * c.cap;
  for (int i = threadIdx.x; i < c.cap; i += NTH) {
    int val;
    if (i >= count) val = -1;
    else if (i < c_lo || keep_all) val = i;
    else if (i >= c_lo + Bc) val = c_hi + (i - c_lo - Bc);
    else continue;
    out[i] = val;
  }
  if (threadIdx.x == 0) a.sel_count[unit] = count;
}

// The unit's histogram is consumed: leave it zero for the next step.
template <int NTH>
__device__ __forceinline__ void zero_hist(const TopkArgs& a, int64_t unit) {
  uint4* hg = reinterpret_cast<uint4*>(a.hist + unit * HB);
  for (int i = threadIdx.x; i < HB / 4; i += NTH) hg[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The arrival counters of the FAC that follows this kernel (one per head chunk).
__device__ __forceinline__ void zero_fac_arrive(const TopkArgs& a, int64_t unit) {
  if (a.fac_arrive != nullptr && int(threadIdx.x) < a.head_chunks) a.fac_arrive[unit * a.head_chunks + threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// Stage 3 pieces.

// Gather the kept pairs of the nfc chunks into LDS, in index order.  Thread t
// sums the counts of chunks CPT t .. CPT t + CPT - 1; wave w copies chunks w,
// w + waves, ...  pre[k] holds the first 64 pairs of chunk w + k * waves
// (loaded early by the caller, unconditionally).  Returns the number of kept
// pairs, or -1 when they do not fit (then nothing is gathered).
template <int NTH, int PRE>
__device__ int gather_kept(SelState<NTH>& s, int32_t* chunk_off, const uint2* slots, const int32_t* counts,
                           int nfc, int cap_lds, const uint2 (&pre)[PRE], uint32_t* key, int32_t* idx) {
  constexpr int NW = NTH / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (nfc > CPT * NTH) return -1;           // uniform
  int cnt[CPT];
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int ch = CPT * tid + k;
    cnt[k] = counts[min(ch, nfc - 1)];
    cnt[k] = ch < nfc ? cnt[k] : 0;
    sum += uint32_t(cnt[k]);
  }
  uint32_t N;
  uint32_t off = block_excl_scan(s, sum, N);
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int ch = CPT * tid + k;
    if (ch < nfc) chunk_off[ch] = int32_t(off);
    off += uint32_t(cnt[k]);
  }
  if (tid == 0) chunk_off[nfc] = int32_t(N);
  if (N > uint32_t(cap_lds)) return -1;     // uniform
  __syncthreads();
  for (int ch = wave; ch < nfc; ch += NW) {
    const int o = chunk_off[ch], n = chunk_off[ch + 1] - o;
    const int kpre = (ch - wave) / NW;
    for (int k = lane; k < n; k += 64) {
      uint2 e;
      if (k < 64 && kpre < PRE) {
        e = pre[0];
#pragma unroll
        for (int p = 1; p < PRE; ++p) e = (kpre == p) ? pre[p] : e;
      } else {
        e = slots[int64_t(ch) * FCH + k];
      }
      key[o + k] = e.x;
      idx[o + k] = int32_t(e.y);
    }
  }
  __syncthreads();
  return int(N);
}

// Exact select of the Bc largest of the N keys key[0..N) (index order, with token
// indices idx) held in LDS; writes the chosen tokens ascending to out[0..Bc).
// Thread t owns a contiguous run of the keys.  With b1 >= 0 every key is known
// to lie in a coarse bin >= b1 (the filter kept exactly those): the first digit
// is then b1 itself unless more than Bc keys lie above it, and only the keys
// above b1 are counted instead of a first histogram pass.
template <int NTH>
__device__ void lds_select(SelState<NTH>& s, const uint32_t* key, const int32_t* idx, int N, int Bc, int b1,
                           int32_t* out) {
  const int tid = threadIdx.x;
  const int per = (N + NTH - 1) / NTH;
  const int i0 = min(N, tid * per), i1 = min(N, i0 + per);
  uint32_t prefix = 0, pmask = 0, rem = uint32_t(Bc);
  int pass = 0;
  if (b1 >= 0) {
    // Second-digit histogram of the keys in bin b1, and the count above b1.
    zero_bins<NTH, HB>(s);
    if (tid == 0) s.above = 0u;
    __syncthreads();
    RunHist rh;
    uint32_t n_above = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key[i];
      const uint32_t bin = k >> kHistShift;
      n_above += bin > uint32_t(b1) ? 1u : 0u;
      rh.add(s.hist, bin == uint32_t(b1), (k >> 10) & 2047u);
    }
    rh.flush(s.hist);
    if (n_above != 0u) atomicAdd(&s.above, n_above);
    __syncthreads();
    const uint32_t above = s.above;
    if (above < rem) {               // uniform; otherwise start from the first digit
      rem -= above;
      prefix = uint32_t(b1) << 21;
      pmask = 0x7ffu << 21;
      find_digit<NTH, 2048>(s, rem);
      const uint32_t d = s.digit, full = s.full;
      rem = s.rem;
      prefix |= d << 10;
      pmask |= 0x7ffu << 10;
      pass = full ? 3 : 2;
    }
  }
#pragma unroll 1
  for (; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    if (pass == 2) zero_bins<NTH, 1024>(s);
    else zero_bins<NTH, 2048>(s);
    __syncthreads();
    RunHist rh;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key[i];
      rh.add(s.hist, (k & pmask) == prefix, (k >> shift) & dmask);
    }
    rh.flush(s.hist);
    __syncthreads();
    if (pass == 2) find_digit<NTH, 1024>(s, rem);
    else find_digit<NTH, 2048>(s, rem);
    const uint32_t d = s.digit, full = s.full;
    rem = s.rem;
    prefix |= d << shift;
    pmask |= dmask << shift;
    if (full) break;
  }
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t m = key[i] & pmask;
    n_gt += m > prefix ? 1u : 0u;
    n_eq += m == prefix ? 1u : 0u;
  }
  uint32_t eq_tot, sel_tot;
  const uint32_t eq_base = block_excl_scan(s, n_eq, eq_tot);
  const uint32_t take_eq = (rem > eq_base) ? min(rem - eq_base, n_eq) : 0u;
  int pos = int(block_excl_scan(s, n_gt + take_eq, sel_tot));
  uint32_t eq_seen = eq_base;
  for (int i = i0; i < i1; ++i) {
    const uint32_t m = key[i] & pmask;
    const bool eq = m == prefix;
    const bool take = m > prefix || (eq && eq_seen < rem);
    eq_seen += eq ? 1u : 0u;
    if (take && pos < Bc) out[pos] = idx[i];   // the guard never fails when the counts agree
    pos += take ? 1 : 0;
  }
}

// Fallback: radix select over the whole candidate range [c_lo, c_hi) of a row,
// streamed from memory in tiles.  A bound from group maxima prunes the first
// pass: the Bc-th largest of the maxima of >= Bc disjoint slot groups is <= the
// Bc-th largest key.
template <int NTH>
__device__ void row_select(SelState<NTH>& s, const float* row, int max_t, int c_lo, int c_hi, int Bc,
                           int32_t* out) {
  constexpr int TILE = NTH * KPT;
  const int tid = threadIdx.x;
  const int ntiles = (max_t + TILE - 1) / TILE;
  uint32_t k[KPT];
  auto keys_of = [&](int ch) {
    float v[KPT];
    load_tile(row, max_t, ch * TILE, v);
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = tile_index(ch * TILE, e >> 2, e & 3);
      k[e] = (j >= c_lo && j < c_hi) ? score_key(v[e]) : 0u;
    }
  };
  uint32_t prefix = 0, pmask = 0, rem = uint32_t(Bc);
  uint32_t b_lo = 0;
  {
    const int64_t groups_needed = (int64_t(Bc) + int64_t(NTH) * ntiles - 1) / (int64_t(NTH) * ntiles);
    int gpt = 1;                               // groups per thread per tile, a power of two
    while (gpt < KPT && gpt < groups_needed) gpt <<= 1;
    const int G = KPT / gpt;
    zero_bins<NTH, HB>(s);
    if (tid == 0) s.digit = 0u;
    __syncthreads();
    RunHist rh;
    for (int ch = 0; ch < ntiles; ++ch) {
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
    find_digit<NTH, HB>(s, uint32_t(Bc));     // digit stays 0 with fewer than Bc groups
    b_lo = s.digit;
  }
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    const uint32_t lo_bin = pass == 0 ? b_lo : 0u;
    if (pass == 2) zero_bins<NTH, 1024>(s);
    else zero_bins<NTH, 2048>(s);
    __syncthreads();
    RunHist rh;
    for (int ch = 0; ch < ntiles; ++ch) {
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
    if (pass == 2) find_digit<NTH, 1024>(s, rem);
    else find_digit<NTH, 2048>(s, rem);
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
  for (int ch = 0; ch < ntiles; ++ch) {
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
      int pos = int(tbase + toff[q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool tk = taken(4 * q + r);
        if (tk && pos < Bc) out[pos] = tile_index(ch * TILE, q, r);   // the guard never fails when the counts agree
        pos += tk ? 1 : 0;
      }
      slot_fence();
    }
    eq_run += eq_tot;
    sel_run += sel_tot;
  }
}

// Stage 3 for one unit that is not keep-all: gather, then select from LDS, or
// fall back to the whole row.
// b1 >= 0: the coarse bin the filter kept keys from (known to the filter's own
// workgroups), else -1.
template <int NTH, int PRE>
__device__ void select_unit(const TopkArgs& a, SelState<NTH>& s, int32_t* chunk_off, uint32_t* key,
                            int32_t* idx, int cap_lds, int64_t unit, int c_lo, int c_hi, int Bc, int b1,
                            const uint2 (&pre)[PRE]) {
  const Common& c = a.c;
  const int nfa = filter_chunks(c);
  int32_t* out = a.sel_idx + unit * c.cap + c_lo;
  const int N = gather_kept<NTH, PRE>(s, chunk_off, a.slots + unit * nfa * int64_t(FCH), a.counts + unit * nfa,
                                      nfa, cap_lds, pre, key, idx);
  if (N >= Bc) lds_select<NTH>(s, key, idx, N, Bc, b1, out);
  else row_select<NTH>(s, a.scores + unit * c.max_t, c.max_t, c_lo, c_hi, Bc, out);
}

// First 64 kept pairs of chunks wave, wave + waves, ... (clamped into the unit's slots).
template <int NTH, int PRE>
__device__ __forceinline__ void prefetch_kept(const TopkArgs& a, int64_t unit, uint2 (&pre)[PRE]) {
  const int nfa = filter_chunks(a.c);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < PRE; ++p)
    pre[p] = a.slots[(unit * nfa + min(wave + p * (NTH / 64), nfa - 1)) * int64_t(FCH) + lane];
}

// ---------------------------------------------------------------------------
// Stage 1 for the standalone select: the unit histogram of given scores; also
// zeroes the unit's arrival counter for the filter that follows.
// Grid (ceil(max_t / 2048), kv heads, batch), 256 threads with 8 slots each.
__global__ __launch_bounds__(FNT) void hist_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.z;
  const int64_t unit = int64_t(b) * c.n_kv_heads + blockIdx.y;
  const float* row = a.scores + unit * c.max_t;
  const int base = blockIdx.x * FCH;
  float v[8];
  load_chunk8(row, c.max_t, base, v);
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.arrive[unit] = 0u;
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
  uint32_t* hg = a.hist + unit * HB;
  for (int i = threadIdx.x; i < HB; i += FNT) {
    const uint32_t x = h[i];
    if (x != 0u) atomicAdd(&hg[i], x);
  }
}

// ---------------------------------------------------------------------------
// Stage 2 (and, with LAST, stage 3 in the unit's last workgroup).
// Grid (ceil(max_t / 2048), kv heads, batch), 256 threads.
struct FilterSmall {
  uint32_t w[FNT / 64];
  uint32_t b1, last;
};
struct FilterLast {
  SelState<FNT> sel;
  int32_t chunk_off[CPT * FNT + 1];
  uint32_t key[kSmallCand];
  int32_t idx[kSmallCand];
  FilterSmall f;
};

template <bool LAST>
__global__ __launch_bounds__(FNT) void filter_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t unit = int64_t(b) * c.n_kv_heads + blockIdx.y;
  const int nfa = filter_chunks(c);
  const float* row = a.scores + unit * c.max_t;
  const int base = blockIdx.x * FCH;

  // Independent loads: this thread's 8 scores and its 8 histogram bins.  Thread
  // t owns bins 2047-8t down to 2040-8t, so a scan over threads counts from the top.
  float v[8];
  load_chunk8(row, c.max_t, base, v);
  const uint32_t* hg = a.hist + unit * HB;
  const uint4 hlo = *reinterpret_cast<const uint4*>(hg + HB - 8 - 8 * tid);
  const uint4 hhi = *reinterpret_cast<const uint4*>(hg + HB - 4 - 8 * tid);
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  if (LAST && blockIdx.x == 0) zero_fac_arrive(a, unit);
  if (Bc == nC) {                      // every candidate is kept: no kept-pair list
    if (LAST && blockIdx.x == 0) {
      zero_hist<FNT>(a, unit);
      write_fixed<FNT>(a, unit, t, c_lo, c_hi, Bc);
    }
    return;
  }

  using Smem = typename std::conditional<LAST, FilterLast, FilterSmall>::type;
  __shared__ Smem sm;
  FilterSmall& fs = [&]() -> FilterSmall& {
    if constexpr (LAST) return sm.f; else return sm;
  }();
  const uint32_t h[8] = {hhi.w, hhi.z, hhi.y, hhi.x, hlo.w, hlo.z, hlo.y, hlo.x};   // descending bins
  uint32_t hs = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) hs += h[i];
  const uint32_t incl = wave_inclusive_scan(hs);
  if (lane == 63) fs.w[wave] = incl;
  if (tid == 0) fs.b1 = 0u;            // fewer than Bc keys counted: keep every candidate
  __syncthreads();
  uint32_t above = incl - hs;          // keys in bins above 2047-8t
#pragma unroll
  for (int w = 0; w < FNT / 64; ++w) above += (w < wave) ? fs.w[w] : 0u;
  const uint32_t bc = uint32_t(Bc);
  if (above < bc && bc <= above + hs) {
    uint32_t cum = above;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (cum < bc && bc <= cum + h[i]) fs.b1 = uint32_t(HB - 1 - 8 * tid - i);
      cum += h[i];
    }
  }
  __syncthreads();
  const uint32_t b1 = fs.b1;

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
  if (lane == 63) fs.w[wave] = pin;    // the reads of fs.w above all precede the last barrier
  __syncthreads();
  uint32_t ex = pin - packed, tot = 0;
#pragma unroll
  for (int w = 0; w < FNT / 64; ++w) {
    const uint32_t x = fs.w[w];
    ex += (w < wave) ? x : 0u;
    tot += x;
  }
  const uint32_t tot0 = tot & 0xffffu, tot1 = tot >> 16;
  uint32_t pos0 = ex & 0xffffu, pos1 = tot0 + (ex >> 16);
  uint2* out = a.slots + (unit * nfa + blockIdx.x) * int64_t(FCH);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t& pos = e < 4 ? pos0 : pos1;
    if (keep[e]) out[pos] = make_uint2(key[e], uint32_t(chunk8_index(base, e)));
    pos += keep[e] ? 1u : 0u;
  }
  if (tid == 0) a.counts[unit * nfa + blockIdx.x] = int32_t(tot0 + tot1);

  if constexpr (LAST) {
    // The workgroup that completes the unit runs stage 3.
    if (!arrive_last(&a.arrive[unit], uint32_t(nfa), &fs.last)) return;
    uint2 pre[4];
    prefetch_kept<FNT, 4>(a, unit, pre);
    zero_hist<FNT>(a, unit);
    write_fixed<FNT>(a, unit, t, c_lo, c_hi, Bc);
    select_unit<FNT, 4>(a, sm.sel, sm.chunk_off, sm.key, sm.idx, kSmallCand, unit, c_lo, c_hi, Bc, int(b1), pre);
  }
}

// ---------------------------------------------------------------------------
// Stage 3 as its own launch (large budgets, and max_t == 0): one 1024-thread
// workgroup per unit.  Grid (kv heads, batch).
struct FinishShared {
  SelState<BIG> sel;
  int32_t chunk_off[CPT * BIG + 1];
  uint32_t key[kCandLds];
  int32_t idx[kCandLds];
};

__global__ __launch_bounds__(BIG) void finish_kernel(TopkArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.y;
  const int64_t unit = int64_t(b) * c.n_kv_heads + blockIdx.x;
  uint2 pre[1];
  prefetch_kept<BIG, 1>(a, unit, pre);     // independent of t_b: goes out first
  int t, c_lo, c_hi;
  unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  zero_fac_arrive(a, unit);
  zero_hist<BIG>(a, unit);
  write_fixed<BIG>(a, unit, t, c_lo, c_hi, Bc);
  if (Bc == nC) return;                     // keep-all (also every unit when max_t == 0)
  __shared__ FinishShared sm;
  select_unit<BIG, 1>(a, sm.sel, sm.chunk_off, sm.key, sm.idx, kCandLds, unit, c_lo, c_hi, Bc, -1, pre);
}

}  // namespace

size_t hist_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * HB * sizeof(uint32_t) + 255) & ~size_t(255);
}
size_t slots_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * filter_chunks(c) * FCH * sizeof(uint2) + 255) & ~size_t(255);
}
size_t counts_bytes(const Common& c) {
  return (size_t(c.batch) * c.n_kv_heads * filter_chunks(c) * sizeof(int32_t) + 255) & ~size_t(255);
}

hipError_t launch_topk(const Common& c, const float* scores, const int32_t* seq_lens,
                       int32_t* sel_idx, int32_t* sel_count, const SelectBuffers& w, bool have_hist,
                       uint32_t* fac_arrive, int head_chunks, hipStream_t s) {
  const TopkArgs a{c, scores, seq_lens, sel_idx, sel_count, w.hist, static_cast<uint2*>(w.slots), w.counts,
                   w.arrive, fac_arrive, head_chunks};
  const dim3 fgrid(filter_chunks(c), c.n_kv_heads, c.batch);
  if (c.max_t > 0 && !have_hist) {
    hipLaunchKernelGGL(hist_kernel, fgrid, dim3(FNT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (c.max_t > 0 && c.budget <= kSmallBudget) {
    hipLaunchKernelGGL(filter_kernel<true>, fgrid, dim3(FNT), 0, s, a);
    return hipGetLastError();
  }
  if (c.max_t > 0) {
    hipLaunchKernelGGL(filter_kernel<false>, fgrid, dim3(FNT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(finish_kernel, dim3(c.n_kv_heads, c.batch), dim3(BIG), 0, s, a);
  return hipGetLastError();
}

}  // namespace fasa
