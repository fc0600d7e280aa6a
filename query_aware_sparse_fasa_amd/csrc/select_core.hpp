// Exact top-B selection machinery shared by the select launches (topk.hip)
// and the FAC launch that selects its own rows (fac.hip): block-wide scans,
// radix digit search over LDS histograms, the gather of the filter's kept
// (key, token) pairs into LDS, the exact select over them, and the whole-row
// fallback.  NTH is the workgroup size (a multiple of 64).
//
// Keys are the order-preserving 32-bit images of fp32 scores (score_key);
// digits are bits 31..21, 20..10 and 9..0 (11, 11, 10 bits).  The selection
// rule (paper-graph-ui review of FASA, section 3.4, TopK-I over the TIP
// scores): the Bc largest keys, equal keys going to the lower token index,
// written as ascending token indices.
#pragma once

#include <type_traits>

#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace sel {

constexpr int HB = kHistBins;               // 2048
constexpr int FCH = kFilterChunk;           // 2048 tokens per filter chunk
constexpr int KPT = 16;                     // fallback slots per thread per tile
constexpr int CPT = 4;                      // chunk counts summed per thread in the gather

// Filter chunks of a row (at least one, so that slot and count arrays are never
// empty and clamped loads from them stay in bounds).
__host__ __device__ __forceinline__ int filter_chunks(const Common& c) {
  const int n = (c.max_t + FCH - 1) / FCH;
  return n > 0 ? n : 1;
}

template <int NTH>
struct SelState {
  alignas(16) uint32_t hist[HB];
  alignas(16) uint32_t hist2[HB];   // the exact select's passes alternate between hist2 and hist
  uint32_t wave_sum[2][NTH / 64];   // two buffers: back-to-back scans alternate
  uint32_t digit, rem, full;
  uint32_t cut;                     // emitted lists: largest threshold of a chunk that left a candidate out, or 0
};

// Block-wide exclusive scan of one value per thread; returns the exclusive
// prefix and writes the block total.  One barrier: the wave totals go through
// buffer BUF, so a scan may only follow another scan on the same buffer once a
// barrier has passed since that one returned (scans with nothing between them
// alternate buffers).
template <int BUF = 0, int NTH>
__device__ __forceinline__ uint32_t block_excl_scan(SelState<NTH>& s, uint32_t v, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) s.wave_sum[BUF][wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const uint32_t x = s.wave_sum[BUF][w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  total = tot;
  return base + incl - v;
}

// block_excl_scan of v, and the block total of w, behind one barrier (the wave
// totals of v go through buffer 0, those of w through buffer 1).  Both buffers
// must be free: a barrier has passed since the last scan returned.
template <int NTH>
__device__ __forceinline__ uint32_t block_excl_scan_and_sum(SelState<NTH>& s, uint32_t v, uint32_t& total, uint32_t w,
                                                           uint32_t& w_total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v), incl_w = wave_inclusive_scan(w);
  if (lane == 63) {
    s.wave_sum[0][wave] = incl;
    s.wave_sum[1][wave] = incl_w;
  }
  __syncthreads();
  uint32_t base = 0, tot = 0, tot_w = 0;
#pragma unroll
  for (int i = 0; i < NTH / 64; ++i) {
    const uint32_t x = s.wave_sum[0][i];
    base += (i < wave) ? x : 0u;
    tot += x;
    tot_w += s.wave_sum[1][i];
  }
  total = tot;
  w_total = tot_w;
  return base + incl - v;
}

// Largest value over the wave's 64 lanes (all active), as a scalar: rotations
// by 8, 4, 2 and 1 inside each 16-lane row, then the four rows' results -- no
// LDS round trips.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kDppRowRor + 8, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kDppRowRor + 4, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kDppRowRor + 2, 0xF, 0xF, false)));
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kDppRowRor + 1, 0xF, 0xF, false)));
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(v), 0)), r1 = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
  const uint32_t r2 = uint32_t(__builtin_amdgcn_readlane(int(v), 32)), r3 = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
  return max(max(r0, r1), max(r2, r3));
}

// Lane Q of the lane's quad (DPP quad_perm [Q, Q, Q, Q]).
template <int Q>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x55 * Q, 0xF, 0xF, false));
}

// Exclusive prefix over the waves of a per-wave value (the same in every lane
// of a wave); also returns the block total.
template <int NTH>
__device__ __forceinline__ uint32_t wave_base(SelState<NTH>& s, uint32_t wave_val, uint32_t& total) {
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s.wave_sum[0][wave] = wave_val;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    const uint32_t x = s.wave_sum[0][w];
    base += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return base;
}

template <int NTH, int NB, int BPT>
__device__ __forceinline__ void find_digit_held(SelState<NTH>& s, uint32_t rem, const uint32_t (&h)[BPT]);

// Find the digit d of a histogram with NB bins (1024 or 2048) such that fewer
// than rem keys lie in bins above d and at least rem in bins >= d.  Thread t
// owns the BPT bins below NB - BPT t (read as 16-byte vectors when BPT >= 4);
// an exclusive scan over threads counts the keys above them, and the thread
// whose bins hold the crossing walks them in registers.  Leaves s.digit
// untouched when there are fewer than rem keys in total.  hist: the histogram
// (s.hist unless given).
template <int NTH, int NB>
__device__ __forceinline__ void find_digit(SelState<NTH>& s, uint32_t rem, const uint32_t* hist = nullptr) {
  constexpr int BPT = NB > NTH ? NB / NTH : 1;
  const uint32_t* hb = hist ? hist : s.hist;
  const int lo = NB - BPT * (int(threadIdx.x) + 1);     // lowest owned bin
  uint32_t h[BPT];
  if constexpr (BPT >= 4) {
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) {
      const uint4 x = reinterpret_cast<const uint4*>(hb + lo)[v];
      h[4 * v + 0] = x.x; h[4 * v + 1] = x.y; h[4 * v + 2] = x.z; h[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BPT; ++i) h[i] = lo + i >= 0 ? hb[lo + i] : 0u;
  }
  find_digit_held<NTH, NB, BPT>(s, rem, h);
}

// find_digit over bins the threads already hold: h[i] is bin NB - BPT (t + 1) + i
// of thread t.  The scan's barrier orders any write to s.digit, s.rem or s.full
// made before the call ahead of the search's own.
template <int NTH, int NB, int BPT>
__device__ __forceinline__ void find_digit_held(SelState<NTH>& s, uint32_t rem, const uint32_t (&h)[BPT]) {
  const int lo = NB - BPT * (int(threadIdx.x) + 1);     // lowest owned bin
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += h[i];
  uint32_t total;
  const uint32_t above = block_excl_scan<1>(s, sum, total);  // keys in bins above the owned ones
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
// The exact select's first buffer, zeroed by every gather that precedes it
// (published by the gather's barriers).
template <int NTH>
__device__ __forceinline__ void zero_hist2(SelState<NTH>& s) {
  for (int i = threadIdx.x; i < HB / 4; i += NTH) reinterpret_cast<uint4*>(s.hist2)[i] = make_uint4(0u, 0u, 0u, 0u);
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
// Scores row[j0 + 256 q + r] for q < Q, r < 4 (4 consecutive per step; steps
// 256 apart; j0 a multiple of 4), clamped into the row's lim readable elements.
// VEC (lim a multiple of 4, the row 16-byte aligned): one 16-byte load per
// step -- a clamped vector only ever covers slots past the valid tokens, which
// are never used; otherwise 4 scalar loads per step.  The choice is a template
// parameter, not a branch, so every load is in flight before the first wait.
template <int Q, bool VEC>
__device__ __forceinline__ void load_steps(const float* row, int lim, int j0, float (&v)[4 * Q]) {
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(row + min(j0 + 256 * q, lim - 4));
      v[4 * q + 0] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = row[min(j0 + 256 * q + r, lim - 1)];
    }
  }
}

template <bool VEC>
__device__ __forceinline__ void load_tile(const float* row, int lim, int base, float (&v)[KPT]) {
  load_steps<KPT / 4, VEC>(row, lim, tile_index(base, 0, 0), v);
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

// Copy the kept pairs of chunks 0 .. nfc-1 (chunk k at slots + k * CHUNK, its
// pairs at offsets chunk_off[k] .. chunk_off[k+1] of the LDS arrays, already
// published) through put(at, pair), in index order: wave w copies chunks w,
// w + waves, ...; pre[p * D + d] holds pairs 64 d .. 64 d + 63 of chunk
// w + p * waves (loaded early by the caller, unconditionally).  No barrier.
template <int NTH, int PRE, int D, int CHUNK, typename Put>
__device__ __forceinline__ void copy_kept(const int32_t* chunk_off, const uint2* slots, int nfc,
                                          const uint2 (&pre)[PRE * D], Put put) {
  constexpr int NW = NTH / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bool more = false;
#pragma unroll
  for (int p = 0; p < PRE; ++p) {
    const int ch = wave + p * NW;
    if (ch < nfc) {
      const int o = chunk_off[ch], n = chunk_off[ch + 1] - o;
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (64 * d + lane < n) put(o + 64 * d + lane, pre[p * D + d]);
      more = more || n > 64 * D;
    }
  }
  more = more || nfc > PRE * NW;
  if (__builtin_amdgcn_readfirstlane(int(more)) != 0) {
    // The first 64 pairs of the chunks past the prefetched ones, 8 chunks of
    // this wave at a time: their loads go out together (clamped chunk, always
    // readable), then they are copied.
    for (int c0 = wave + PRE * NW; c0 < nfc; c0 += 8 * NW) {   // wave-uniform
      uint2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = slots[int64_t(min(c0 + u * NW, nfc - 1)) * CHUNK + lane];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ch = c0 + u * NW;
        if (ch < nfc) {
          const int o = chunk_off[ch], n = chunk_off[ch + 1] - o;
          if (lane < n) put(o + lane, v[u]);
        }
      }
    }
    // Pairs past the first 64 of a chunk (a chunk keeps up to CHUNK), U x 64 of
    // them per wave at a time: the loads go out together (clamped to the
    // chunk's last kept pair, so loads past the end all read one line), then
    // the valid ones are copied.  U is 8 while more than 128 pairs remain, 2
    // for the last few (each width is straight-line code with its own wait).
    auto copy_run = [&](auto width, const uint2* cs, int o, int n, int k0) {
      constexpr int U = decltype(width)::value;
      uint2 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = cs[min(k0 + 64 * u + lane, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = k0 + 64 * u + lane;
        if (k < n) put(o + k, v[u]);
      }
    };
    for (int ch = wave; ch < nfc; ch += NW) {
      const int o = chunk_off[ch], n = chunk_off[ch + 1] - o;
      const uint2* cs = slots + int64_t(ch) * CHUNK;
      int k0 = ch < PRE * NW ? 64 * D : 64;         // pairs already prefetched
      for (; n - k0 > 128; k0 += 8 * 64) copy_run(std::integral_constant<int, 8>(), cs, o, n, k0);   // wave-uniform
      if (k0 < n) copy_run(std::integral_constant<int, 2>(), cs, o, n, k0);
    }
  }
}

// Gather the kept pairs of the nfc chunks into LDS, in index order.  cnt_raw[k]
// is the count of chunk CPT t + k (loaded by the caller, clamped); wave w
// copies chunks w, w + waves, ...; pre[p * D + d] holds pairs 64 d .. 64 d + 63
// of chunk w + p * waves (loaded early by the caller, unconditionally).  Returns
// the number of kept pairs, or -1 when they do not fit (then nothing is gathered).
template <int NTH, int PRE, int D = 1>
__device__ __forceinline__ int gather_kept(SelState<NTH>& s, int32_t* chunk_off, const uint2* slots, int nfc, int cap_lds,
                           const int (&cnt_raw)[CPT], const uint2 (&pre)[PRE * D], uint32_t* key, int32_t* idx,
                           int b1, uint32_t& above) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (nfc > CPT * NTH) return -1;           // uniform
  int cnt[CPT];
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    cnt[k] = (CPT * tid + k < nfc) ? cnt_raw[k] : 0;
    sum += uint32_t(cnt[k]);
  }
  uint32_t N;
  if (nfc <= 64 * CPT) {
    // Up to 256 chunks (every selecting FAC launch): wave 0 holds all the
    // counts, scans them itself and writes the chunk offsets and the total; one
    // barrier publishes them.
    if (wave == 0) {
      const uint32_t incl = wave_inclusive_scan(sum);
      uint32_t off = incl - sum;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int ch = CPT * tid + k;
        if (ch < nfc) chunk_off[ch] = int32_t(off);
        off += uint32_t(cnt[k]);
      }
      if (lane == 63) chunk_off[nfc] = int32_t(incl);
    }
    __syncthreads();
    N = uint32_t(chunk_off[nfc]);
    if (N > uint32_t(cap_lds)) return -1;   // uniform
  } else {
    uint32_t off = block_excl_scan(s, sum, N);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ch = CPT * tid + k;
      if (ch < nfc) chunk_off[ch] = int32_t(off);
      off += uint32_t(cnt[k]);
    }
    if (tid == 0) chunk_off[nfc] = int32_t(N);
    if (N > uint32_t(cap_lds)) return -1;   // uniform
    __syncthreads();
  }
  // The prefetched pairs first (no memory access), then whatever is beyond them.
  // With b1 >= 0 every copied key also goes into the second-digit histogram
  // (bits 20..10) if it lies in bin b1, or is counted if it lies above b1 (the
  // histogram was zeroed by the caller before this call).
  uint32_t n_above = 0;
  auto put = [&](int at, uint2 e) {
    key[at] = e.x;
    idx[at] = int32_t(e.y);
    if (b1 >= 0) {
      const uint32_t bin = e.x >> kHistShift;
      n_above += bin > uint32_t(b1) ? 1u : 0u;
      if (bin == uint32_t(b1)) atomicAdd(&s.hist[(e.x >> 10) & 2047u], 1u);
    }
  };
  copy_kept<NTH, PRE, D, FCH>(chunk_off, slots, nfc, pre, put);
  // The barrier inside the scan also publishes the copied pairs and the histogram.
  (void)block_excl_scan(s, n_above, above);
  return int(N);
}

// The radix passes of an exact select from pass `pass` on (0: bits 31..21, 1:
// bits 20..10, 2: bits 9..0), given the digits found so far (prefix under
// pmask) and the rem keys still to take among those equal to the prefix, then
// the index-order compaction: the Bc largest of the N <= kCandLds keys key[0..N) (index
// order, token indices idx) in LDS are written ascending to out[0..Bc).
// all_eq: every key equal to the prefix is taken (skip to one scan).  Thread t
// owns a contiguous run of the keys.
// Returns the determined digits of the Bc-th largest key with the others zero
// (a lower bound of that key).  The passes alternate histogram buffers: the
// first pass counts into s.hist2, which the caller's gather zeroed, and each
// pass zeroes the next one's buffer (free since the previous digit search
// ended) while it counts, so no pass waits on its own zeroing.
template <int NTH>
__device__ __forceinline__ uint32_t lds_select_from(SelState<NTH>& s, const uint32_t* key, const int32_t* idx,
                                                    int N, int Bc, uint32_t prefix, uint32_t pmask, uint32_t rem,
                                                    int pass, bool all_eq, int32_t* out) {
  const int tid = threadIdx.x;
  const int per = (N + NTH - 1) / NTH;
  const int i0 = min(N, tid * per), i1 = min(N, i0 + per);
  uint32_t* cur = s.hist2;
  uint32_t* nxt = s.hist;
#pragma unroll 1
  for (; !all_eq && pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    if (pass < 2) {
      for (int i = tid; i < (pass == 1 ? 1024 : 2048) / 4; i += NTH)
        reinterpret_cast<uint4*>(nxt)[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    RunHist rh;
    for (int i = i0; i < i1; ++i) {
      const uint32_t k = key[i];
      rh.add(cur, (k & pmask) == prefix, (k >> shift) & dmask);
    }
    rh.flush(cur);
    __syncthreads();                        // the counts, and the next buffer's zeros
    if (pass == 2) find_digit<NTH, 1024>(s, rem, cur);
    else find_digit<NTH, 2048>(s, rem, cur);
    const uint32_t d = s.digit, full = s.full;
    rem = s.rem;
    prefix |= d << shift;
    pmask |= dmask << shift;
    all_eq = full != 0u;
    uint32_t* t = cur;
    cur = nxt;
    nxt = t;
  }
  if (all_eq) {
    // Every key at or above the prefix is taken: one scan places them.
    uint32_t n_take = 0;
    for (int i = i0; i < i1; ++i) n_take += (key[i] & pmask) >= prefix ? 1u : 0u;
    uint32_t tot;
    int pos = int(block_excl_scan(s, n_take, tot));
    for (int i = i0; i < i1; ++i) {
      const bool take = (key[i] & pmask) >= prefix;
      if (take && pos < Bc) out[pos] = idx[i];   // the guard never fails when the counts agree
      pos += take ? 1 : 0;
    }
    return prefix;
  }
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t m = key[i] & pmask;
    n_gt += m > prefix ? 1u : 0u;
    n_eq += m == prefix ? 1u : 0u;
  }
  // The keys equal to the prefix are taken in index order, the first rem of
  // them: the threads before this one take min(rem, eq_base) of theirs.
  // Both counts fit 16 bits (N is at most the LDS capacity), so one scan
  // carries them.
  static_assert(kCandLds < 65536 && kSmallCand < 65536, "the keys' counts fit 16 bits");
  uint32_t tot;
  const uint32_t base = block_excl_scan(s, n_gt | (n_eq << 16), tot);
  const uint32_t eq_base = base >> 16;
  int pos = int((base & 0xffffu) + min(rem, eq_base));
  uint32_t eq_seen = eq_base;
  for (int i = i0; i < i1; ++i) {
    const uint32_t m = key[i] & pmask;
    const bool eq = m == prefix;
    const bool take = m > prefix || (eq && eq_seen < rem);
    eq_seen += eq ? 1u : 0u;
    if (take && pos < Bc) out[pos] = idx[i];   // the guard never fails when the counts agree
    pos += take ? 1 : 0;
  }
  return prefix;
}

// Exact select of the Bc largest of the N keys key[0..N) held in LDS (index
// order, token indices idx); writes the chosen tokens ascending to out[0..Bc).
// With b1 >= 0 every key is known to lie in a coarse bin >= b1 (the filter kept
// exactly those), `above` keys lie above it and s.hist holds the second-digit
// histogram of the keys in b1 (both built by the gather): the first digit is
// then b1 itself unless at least Bc keys lie above it.  When a digit's bin
// holds exactly the keys still needed, the remaining digits are skipped and
// one scan places every key at or above the prefix.
template <int NTH>
__device__ __forceinline__ void lds_select(SelState<NTH>& s, const uint32_t* key, const int32_t* idx, int N, int Bc, int b1,
                           uint32_t above, int32_t* out) {
  uint32_t prefix = 0, pmask = 0, rem = uint32_t(Bc);
  bool all_eq = false;
  int pass = 0;
  if (b1 >= 0 && above < rem) {        // uniform; otherwise start from the first digit
    // The second-digit histogram of the keys in bin b1 was built by the gather.
    rem -= above;
    prefix = uint32_t(b1) << 21;
    pmask = 0x7ffu << 21;
    find_digit<NTH, 2048>(s, rem);
    const uint32_t d = s.digit, full = s.full;
    rem = s.rem;
    prefix |= d << 10;
    pmask |= 0x7ffu << 10;
    all_eq = full != 0u;
    pass = 2;
  }
  (void)lds_select_from<NTH>(s, key, idx, N, Bc, prefix, pmask, rem, pass, all_eq, out);
}

// Gather the candidate lists TIP emitted for the unit's nfc chunks (chunk k at
// slots + k * kEmitChunk; meta_raw[k] is the summary (emit_word, tau) of chunk
// CPT t + k, loaded by the caller, clamped) into LDS in index order, and build
// the histogram of their first digits (bits 31..21) in s.hist (zeroed by the
// caller).  s.cut gets the largest threshold tau of a chunk that left some
// candidate out (0 if none did).  Returns the number of pairs, or -1 when they
// do not fit cap_lds or there are more than 256 chunks (then nothing is
// gathered).
template <int NTH, int PRE, int D = 1>
__device__ __forceinline__ int gather_emitted(SelState<NTH>& s, int32_t* chunk_off, const uint2* slots, int nfc,
                                              int cap_lds, const uint2 (&meta_raw)[CPT], const uint2 (&pre)[PRE * D],
                                              uint32_t* key, int32_t* idx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (nfc > 64 * CPT) return -1;            // uniform
  if (wave == 0) {
    // Wave 0 holds every chunk's summary: it scans the counts, writes the
    // chunk offsets and the total, and finds the largest threshold of a cut chunk.
    uint32_t cnt[CPT], sum = 0, cut = 0;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const bool in = CPT * tid + k < nfc;
      const uint32_t w = in ? meta_raw[k].x : 0u;
      cnt[k] = emit_count(w);
      sum += cnt[k];
      cut = (in && emit_cut(w)) ? max(cut, meta_raw[k].y) : cut;
    }
    cut = wave_max_u32(cut);
    const uint32_t incl = wave_inclusive_scan(sum);
    uint32_t off = incl - sum;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ch = CPT * tid + k;
      if (ch < nfc) chunk_off[ch] = int32_t(off);
      off += cnt[k];
    }
    if (lane == 63) chunk_off[nfc] = int32_t(incl);
    if (lane == 0) s.cut = cut;
  }
  __syncthreads();
  const uint32_t N = uint32_t(chunk_off[nfc]);
  if (N > uint32_t(cap_lds)) return -1;     // uniform
  auto put = [&](int at, uint2 e) {
    key[at] = e.x;
    idx[at] = int32_t(e.y);
    atomicAdd(&s.hist[e.x >> kHistShift], 1u);
  };
  copy_kept<NTH, PRE, D, kEmitChunk>(chunk_off, slots, nfc, pre, put);
  __syncthreads();                          // publishes the pairs and the histogram
  return int(N);
}

// Lists of at most B1_LISTS chunks, each read up to B1_LIST pairs, by the
// histogram-filtered gather below.
constexpr int B1_LISTS = 128;
constexpr int B1_LIST = 128;

// The pairs of TIP's lists that thread t holds: list (chunk) t / TPC, and of
// it, with j = t mod TPC, the uint4 (two pairs) TPC i + j for i < VPT -- the
// TPC threads of a chunk read adjacent 16-byte pieces, so one load instruction
// of a wave covers whole 64-byte runs of 64 / TPC lists.  Steps i < EARLY are
// read before the list's length is known (early, for nfa chunks); the others
// (late) only below the list's length n, taken from the chunk's summary m (0
// past the unit's nfc chunks).
template <int NTH, int EARLY = 0>
struct B1Slice {
  static constexpr int TPC = NTH / B1_LISTS;         // threads per chunk
  static constexpr int VPT = B1_LIST / (2 * TPC);    // uint4 per thread
  static_assert(TPC * B1_LISTS == NTH && VPT * 2 * TPC == B1_LIST && VPT <= 16 && EARLY <= VPT,
                "whole chunks per block; a kept mask fits 32 bits");
  uint4 pr[VPT];
  int n = 0;                                         // the list's length
  __device__ __forceinline__ int j() const { return int(threadIdx.x) % TPC; }
  __device__ __forceinline__ const uint4* src(const uint2* slots, int nch) const {
    return reinterpret_cast<const uint4*>(slots + int64_t(min(int(threadIdx.x) / TPC, nch - 1)) * kEmitChunk) + j();
  }
  // Position of the h-th pair of step i in the list.
  __device__ __forceinline__ int pos(int i, int h) const { return 2 * (TPC * i + j()) + h; }
  __device__ __forceinline__ void early(const uint2* slots, int nfa) {
    const uint4* p = src(slots, nfa);
#pragma unroll
    for (int i = 0; i < EARLY; ++i) pr[i] = p[TPC * i];
  }
  __device__ __forceinline__ void late(const uint2* slots, int nfc, uint2 m) {
    const int ch = int(threadIdx.x) / TPC;
    n = ch < nfc ? int(emit_count(m.x)) : 0;
    const uint4* p = src(slots, nfc);
#pragma unroll
    for (int i = EARLY; i < VPT; ++i) pr[i] = pos(i, 0) < n ? p[TPC * i] : make_uint4(0u, 0u, 0u, 0u);
  }
};

// Gather from TIP's per-chunk lists only the keys in coarse bins >= b1 (the
// unit histogram's bin of the Bc-th largest key), in index order, into LDS: the
// filter's kept set without a filter launch.  Each thread holds its pieces of
// one list (sl, with the summary m of that chunk); the kept pairs of a list
// are placed from the masks of its TPC threads (which pieces each keeps), the
// lists one after another by a block scan of their kept counts, so the keys
// land in index order (chunk by chunk, each list ascending).  Builds the
// second-digit histogram (bits 20..10) of the keys in bin b1 in s.hist (zeroed
// by the caller) and counts the keys above b1.  The lists hold every key of bin
// >= b1 when no chunk that left candidates out has its threshold tau above b1's
// lower edge (a chunk leaves out only keys below its tau).  Returns the number
// of pairs, or -1 (nothing gathered) when that does not hold, a list is longer
// than B1_LIST, or the kept keys exceed cap_lds.
template <int NTH, int EARLY>
__device__ __forceinline__ int gather_lists_b1(SelState<NTH>& s, const B1Slice<NTH, EARLY>& sl, uint2 m, int nfc,
                                               int cap_lds, uint32_t* key, int32_t* idx, uint32_t b1, uint32_t& above) {
  using S = B1Slice<NTH, EARLY>;
  constexpr int TPC = S::TPC, VPT = S::VPT;
  static_assert(2 * TPC <= 15, "a step's kept count of a list fits 4 bits");
  const int lane = int(threadIdx.x) & 63, j = sl.j();
  const int ch = int(threadIdx.x) / TPC;
  const bool unusable = sl.n > B1_LIST || (ch < nfc && emit_cut(m.x) && m.y > (b1 << kHistShift));
  // Steps that hold a pair of some list of this wave (the longest list decides).
  const int steps = int((min(wave_max_u32(uint32_t(sl.n)), uint32_t(B1_LIST)) + 2 * TPC - 1) / (2 * TPC));
  // Bit 2 i + h: the h-th pair of step i lies in the list (its position
  // 2 (TPC i + j) + h is below n): i < ceil((n - 2 j - h) / (2 TPC)).
  const int r = sl.n - 2 * j;
  const int a0 = min((max(r, 0) + 2 * TPC - 1) / (2 * TPC), VPT);
  const int a1 = min((max(r - 1, 0) + 2 * TPC - 1) / (2 * TPC), VPT);
  const uint32_t valid = (0x55555555u & (a0 >= 16 ? ~0u : (1u << (2 * a0)) - 1u)) |
                         (0xAAAAAAAAu & (a1 >= 16 ? ~0u : (1u << (2 * a1)) - 1u));
  // Bit 2 i + h of mask: that pair is kept (bin >= b1); of amask: its bin is above b1.
  const uint32_t lo_key = b1 << kHistShift, hi_key = lo_key | ((1u << kHistShift) - 1u);
  uint32_t mask = 0, amask = 0;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (i < steps) {                        // uniform; no break, so pr keeps static indices
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k = h == 0 ? sl.pr[i].x : sl.pr[i].z;
        mask |= k >= lo_key ? (1u << (2 * i + h)) : 0u;
        amask |= k > hi_key ? (1u << (2 * i + h)) : 0u;
      }
    }
  }
  mask &= valid;
  const uint32_t n_above = uint32_t(__popc(amask & valid));
  // The masks of the list's TPC threads, and their kept counts per step, 4 bits
  // a step: step 2 k in bits 4 k .. 4 k + 3 of *_e, step 2 k + 1 in those of
  // *_o; tot_* over the list's TPC threads, pre_* over those before this one.
  uint32_t mg[TPC];
  if constexpr (TPC == 4) {                 // the list is the lane's quad: quad broadcasts
    mg[0] = quad_bcast<0>(mask);
    mg[1] = quad_bcast<1>(mask);
    mg[2] = quad_bcast<2>(mask);
    mg[3] = quad_bcast<3>(mask);
  } else {
#pragma unroll
    for (int q = 0; q < TPC; ++q) mg[q] = uint32_t(__shfl(int(mask), (lane & ~(TPC - 1)) + q, 64));
  }
  uint32_t list_kept = 0, tot_e = 0, tot_o = 0, pre_e = 0, pre_o = 0;
#pragma unroll
  for (int q = 0; q < TPC; ++q) {
    const uint32_t mq = mg[q];
    list_kept += uint32_t(__popc(mq));
    const uint32_t c2 = (mq & 0x55555555u) + ((mq >> 1) & 0x55555555u);   // 2 bits a step
    const uint32_t e = c2 & 0x33333333u, o = (c2 >> 2) & 0x33333333u;
    tot_e += e;
    tot_o += o;
    pre_e += q < j ? e : 0u;
    pre_o += q < j ? o : 0u;
  }
  // The list's count rides on its last thread; a flag on any thread adds more
  // than any block could keep.
  const uint32_t v = (j == TPC - 1 ? list_kept : 0u) + (unusable ? uint32_t(cap_lds) + 1u : 0u);
  uint32_t tot;
  uint32_t run = block_excl_scan_and_sum(s, v, tot, n_above, above);
  if (tot > uint32_t(cap_lds)) return -1;   // uniform
  auto put = [&](uint32_t at, uint32_t k, uint32_t t) {
    key[at] = k;
    idx[at] = int32_t(t);
    if ((k >> kHistShift) == b1) atomicAdd(&s.hist[(k >> 10) & 2047u], 1u);
  };
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (i < steps) {                        // uniform
      const int sh = 4 * (i >> 1);
      const uint32_t at = run + ((((i & 1) ? pre_o : pre_e) >> sh) & 15u);   // the list's kept pairs before this thread's
      run += (((i & 1) ? tot_o : tot_e) >> sh) & 15u;
      const uint32_t mine = mask >> (2 * i);
      if (mine & 1u) put(at, sl.pr[i].x, sl.pr[i].y);
      if (mine & 2u) put(at + (mine & 1u), sl.pr[i].z, sl.pr[i].w);
    }
  }
  __syncthreads();                          // the pairs and the histogram
  return int(tot);
}

// Exact select of the Bc largest of the N (>= Bc) emitted keys in LDS, whose
// first-digit histogram gather_emitted built, into out[0..Bc) ascending.
// The emitted lists are the whole story only if no chunk left out a key that
// could belong: every key a chunk left out lies below that chunk's threshold
// tau, so if no cut chunk's tau lies above the Bc-th largest emitted key K,
// every key left out is smaller than K, and the Bc largest of the union are
// the Bc largest of the unit.  Returns false otherwise (out is then not a
// valid result): early, when a tau's coarse bin lies above K's, or after the
// select, when a tau exceeds the digits of K that the select determined.
template <int NTH>
__device__ __forceinline__ bool select_emitted(SelState<NTH>& s, const uint32_t* key, const int32_t* idx, int N,
                                               int Bc, int32_t* out) {
  find_digit<NTH, 2048>(s, uint32_t(Bc));
  const uint32_t d = s.digit, full = s.full, rem = s.rem, cut = s.cut;
  if ((cut >> 21) > d) return false;        // uniform
  const uint32_t k_low = lds_select_from<NTH>(s, key, idx, N, Bc, d << 21, 0x7ffu << 21, rem, 1, full != 0u, out);
  return cut <= k_low;                      // uniform
}

// Fallback: radix select over the whole candidate range [c_lo, c_hi) of a row,
// streamed from memory in tiles.  A bound from group maxima prunes the first
// pass: the Bc-th largest of the maxima of >= Bc disjoint slot groups is <= the
// Bc-th largest key.
// lim: readable elements of the row (see load_steps); the tokens are [0, max_t).
template <int NTH, bool VEC>
__device__ __forceinline__ void row_select(SelState<NTH>& s, const float* row, int lim, int max_t, int c_lo, int c_hi, int Bc,
                           int32_t* out) {
  constexpr int TILE = NTH * KPT;
  const int tid = threadIdx.x;
  const int ntiles = (max_t + TILE - 1) / TILE;
  uint32_t k[KPT];
  auto keys_of = [&](int ch) {
    float v[KPT];
    load_tile<VEC>(row, lim, ch * TILE, v);
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

// First 64 kept pairs of chunks wave, wave + waves, ... of a unit's slots
// (clamped to the unit's nfa chunks; loaded unconditionally).
// D > 1: also pairs 64 .. 64 D - 1 of each of those chunks (read whatever the
// slots hold; only the first count of them are used).
template <int NTH, int PRE, int D = 1, int CHUNK = FCH>
__device__ __forceinline__ void prefetch_kept(const uint2* unit_slots, int nfa, uint2 (&pre)[PRE * D]) {
  static_assert(64 * D <= CHUNK, "a chunk holds CHUNK slots");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < PRE; ++p) {
    const uint2* cs = unit_slots + int64_t(min(wave + p * (NTH / 64), nfa - 1)) * CHUNK;
#pragma unroll
    for (int d = 0; d < D; ++d) pre[p * D + d] = cs[64 * d + lane];
  }
}

// Chunk summaries of TIP's lists, CPT per thread (chunk CPT t + k), loaded unconditionally.
__device__ __forceinline__ void load_meta(const uint2* unit_meta, int nfa, uint2 (&m)[CPT]) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) m[k] = unit_meta[min(CPT * int(threadIdx.x) + k, nfa - 1)];
}

// Chunk counts of a unit, CPT per thread (chunk CPT t + k), loaded unconditionally.
__device__ __forceinline__ void load_counts(const int32_t* unit_counts, int nfa, int (&cnt)[CPT]) {
#pragma unroll
  for (int k = 0; k < CPT; ++k) cnt[k] = unit_counts[min(CPT * int(threadIdx.x) + k, nfa - 1)];
}

// The exact select from TIP's lists filtered by the unit histogram (see
// gather_lists_b1): thread t holds the unit histogram's bins HB - 4 (t + 1) ..
// HB - 4 t - 1 in hv (the digit search's order), whose bin of the Bc-th largest
// key is b1; sl holds the thread's slice of the lists, m its chunk's summary.
// Falls back to the whole scores row when the lists cannot be used.
template <int NTH, bool VEC, int EARLY>
__device__ void select_from_lists_b1(SelState<NTH>& s, uint32_t* key, int32_t* idx, int cap_lds,
                                     const B1Slice<NTH, EARLY>& sl, uint2 m, uint4 hv, const float* row, int lim,
                                     int max_t, int nfc, int c_lo, int c_hi, int Bc, int32_t* out) {
  static_assert(HB == 4 * NTH, "four bins per thread");
  if (threadIdx.x == 0) {
    s.digit = 0u;                            // fewer than Bc keys counted: keep every candidate
    s.rem = uint32_t(Bc);
    s.full = 0u;
  }
  const uint32_t h[4] = {hv.x, hv.y, hv.z, hv.w};
  find_digit_held<NTH, HB>(s, uint32_t(Bc), h);   // ends with a barrier
  const uint32_t b1 = s.digit;
  zero_bins<NTH, HB>(s);                     // the second-digit histogram; published by the gather's first barrier
  zero_hist2<NTH>(s);
  uint32_t above = 0;
  const int N = gather_lists_b1<NTH, EARLY>(s, sl, m, nfc, cap_lds, key, idx, b1, above);
  if (N >= Bc) {
    lds_select<NTH>(s, key, idx, N, Bc, int(b1), above, out);
    return;
  }
  row_select<NTH, VEC>(s, row, lim, max_t, c_lo, c_hi, Bc, out);
}

// Exact select of one unit that is not keep-all, from the filter's kept pairs
// (nfc chunks, counts cnt and first pairs pre already loaded), into out[0..Bc)
// -- global or LDS.  b1: the coarse bin the filter kept keys from.  Falls back
// to the whole score row when the kept pairs are fewer than Bc or do not fit.
template <int NTH, int PRE, bool VEC, int D = 1>
__device__ void select_from_kept(SelState<NTH>& s, int32_t* chunk_off, uint32_t* key, int32_t* idx, int cap_lds,
                                 const uint2* unit_slots, const float* row, int lim, int max_t, int nfc,
                                 const int (&cnt)[CPT],
                                 const uint2 (&pre)[PRE * D], int c_lo, int c_hi, int Bc, int b1, int32_t* out) {
  zero_bins<NTH, HB>(s);               // the gather's second-digit histogram; published by its first barrier
  zero_hist2<NTH>(s);
  uint32_t above = 0;
  const int N = gather_kept<NTH, PRE, D>(s, chunk_off, unit_slots, nfc, cap_lds, cnt, pre, key, idx, b1, above);
  if (N >= Bc) lds_select<NTH>(s, key, idx, N, Bc, b1, above, out);
  else row_select<NTH, VEC>(s, row, lim, max_t, c_lo, c_hi, Bc, out);
}

// Exact select of one unit that is not keep-all from the lists TIP emitted
// (nfc chunks, summaries meta and first pairs pre already loaded), into
// out[0..Bc) -- global or LDS.  Falls back to the whole score row when the
// lists cannot be shown to hold the top-Bc, hold fewer than Bc keys, or do not
// fit.
template <int NTH, int PRE, bool VEC, int D = 1>
__device__ void select_from_emitted(SelState<NTH>& s, int32_t* chunk_off, uint32_t* key, int32_t* idx, int cap_lds,
                                    const uint2* unit_slots, const float* row, int lim, int max_t, int nfc,
                                    const uint2 (&meta)[CPT], const uint2 (&pre)[PRE * D], int c_lo, int c_hi, int Bc,
                                    int32_t* out) {
  zero_bins<NTH, HB>(s);               // the gather's first-digit histogram; published by its first barrier
  zero_hist2<NTH>(s);
  const int N = gather_emitted<NTH, PRE, D>(s, chunk_off, unit_slots, nfc, cap_lds, meta, pre, key, idx);
  if (N >= Bc && select_emitted<NTH>(s, key, idx, N, Bc, out)) return;
  row_select<NTH, VEC>(s, row, lim, max_t, c_lo, c_hi, Bc, out);
}

}  // namespace sel
}  // namespace fasa
