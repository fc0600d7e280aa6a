// TIP: Token Importance Prediction over the dominant frequency chunks.
//
// For every sequence b, kv head g and cached token j < t_b:
//   S[j] = sum_{h in group(g)} sum_{f < F} q_h[2 I_g[f]] k_j[2 I_g[f]] + q_h[2 I_g[f]+1] k_j[2 I_g[f]+1]
// (paper-graph-ui review of FASA, section 3.4 "Online Stage 1: Token Importance
// Predictor (TIP)", S_t as the sum of the single-FC score vectors alpha^(i) over
// I_dom; keys are cached after RoPE, so each alpha^(i) entry is the FC-i dot
// product of the post-RoPE vectors, section 3.4 "RoPE from a Frequency-Chunk
// Perspective").  The score is linear in q, so the G query heads of the group
// are first summed per dominant column (the "folded" query, 2F fp32 values, a
// wave reduction in wave 0: a few heads per lane, then butterfly shuffles
// across the lanes of a column -- measured level with a per-thread serial sum
// over all heads at 1-8 sequences and 1.3 us faster at 64); each token then
// costs 2F fused multiply-adds on 2F cache elements.
//
// Mapping (gfx950, wave64): one workgroup = 4 waves = 4 cache blocks of one
// (b, g) = one 1024-token chunk; lane l of a wave owns tokens 4l..4l+3 of its
// block.  Reading the slab, FC f of the block is one contiguous 1 KB (bf16) run
// and each lane issues one 16-byte load per FC -- F independent loads in flight
// per lane, no cross-lane traffic, and the folded query is a wave-uniform LDS
// broadcast.  The slab is indexed by (sequence, logical block), so its
// addresses need nothing but the workgroup's coordinates: the slab loads go
// out at kernel entry, beside the query and length loads.  Scores leave as one
// 16-byte store per lane.  The kernel is a pure HBM stream (2 flops per 2-byte
// element), so there is nothing for MFMA to do.
//
// Four epilogues (MODE):
//   kTipScores: scores only (fasa_tip);
//   kTipHist:   also the unit's coarse key histogram for the filter launch of
//               the three-launch select (global atomics);
//   kTipEmit:   also this chunk's candidates for the exact select that the
//               FAC launch finishes: every candidate key of the chunk at or
//               above tau, the lower edge of the coarse bin (key bits 31..21)
//               that holds the chunk's k-th largest key (k from the unit's
//               budget and length), written as (key, token) pairs in index
//               order, with the chunk's count, tau, and whether any candidate
//               of the chunk was left out.  Keys left out are all below tau,
//               which is what lets the FAC launch prove that the union of the
//               chunks' lists holds the unit's top-B (or fall back to the
//               whole scores row).  (An exact k-th largest found by ballot
//               binary searches, 32 dependent rounds per wave, measured 10 us
//               slower per launch than this LDS histogram.)
//   kTipEmitHist: the list and the unit histogram both (the chunk's LDS
//               histogram added to the unit's); the FAC launch keeps only the
//               list keys in bins at or above the unit histogram's bin of the
//               B-th key.
// One chunk per workgroup: workgroups that walked 2-8 chunks of a unit, with
// the next chunk's slab loads in flight during the current one's arithmetic and
// one histogram flush at the end (91-178 VGPRs), streamed slower than these
// light workgroups (56 VGPRs, many resident per CU): TIP 51.8 -> 54.0 us at
// batch 16, 15.1 -> 15.4 us at 128K tokens, 224 -> 260 us on the ragged batch.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

struct TipArgs {
  Common c;
  const void* q;
  const void* src;      // slab, or k_pool when gathering in place
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* fc_idx;
  float* scores;
  uint32_t* hist;       // [units][kHistBins] coarse key histogram (kTipHist)
  uint2* slots;         // [units][emit chunks][kEmitChunk] (key, token) pairs (kTipEmit)
  uint2* meta;          // [units][emit chunks] chunk summary: (emit_word, tau) (kTipEmit)
  uint32_t* arrive;     // [units] counters of the FAC launch, zeroed by chunk 0 (kTipEmitHist)
};

// Column slots of the query fold for F dominant FCs: 2F rounded up to a power of two.
__host__ __device__ constexpr int fold_slots(int F) {
  int p = 2;
  while (p < 2 * F) p <<= 1;
  return p;
}

// Folded query of unit (b, g) into qf[0..2F) and cols[0..F), summed over the
// group's query heads by a wave reduction (run by wave 0): column slot
// sl = 2f + comp (column 2 I_g[f] + comp) of P slots, P = 2F rounded up to a
// power of two.  With P <= 64, lane l takes slot l % P and heads l / P,
// l / P + 64 / P, ...; the 64 / P lanes of a slot then add their sums with
// butterfly shuffles.  With P = 128 (F > 32) a lane takes slots l and l + 64 and
// all the heads.  Slots past 2F, and unused FC slots (index < 0, a head with
// fewer FCs), contribute nothing.  sl0 / fi0: the lane's first slot and its FC
// index, loaded by the caller at kernel entry.
template <typename T, int FT>
__device__ __forceinline__ void fold_query(const TipArgs& a, int b, int g, int F, int P, int sl0, int fi0,
                                           float* qf, int* cols) {
  const Common& c = a.c;
  const int lane = threadIdx.x & 63;
  const T* qg = static_cast<const T*>(a.q) + (int64_t(b) * c.n_q_heads + int64_t(g) * c.group) * kHeadDim;
  // Heads per lane: at most NH (known when F is), loads clamped to the group
  // and issued together, terms past the group masked to +0.
  constexpr int NH = FT > 0 ? (16 + 64 / fold_slots(FT) - 1) / (64 / fold_slots(FT)) : 16;
  const int hs = P <= 64 ? 64 / P : 1;
  const int per = P <= 64 ? 1 : 2;
  for (int k = 0; k < per; ++k) {
    const int sl = k == 0 ? sl0 : lane + 64;
    const int fi = k == 0 ? fi0 : (sl < 2 * F ? a.fc_idx[g * F + (sl >> 1)] : -1);
    const int col = 2 * (fi < 0 ? 0 : fi) + (sl & 1);
    const int h0 = P <= 64 ? lane / P : 0;
    T qv[NH];
#pragma unroll
    for (int u = 0; u < NH; ++u) qv[u] = qg[min(h0 + u * hs, c.group - 1) * kHeadDim + col];
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < NH; ++u) s += (h0 + u * hs < c.group) ? to_f32(qv[u]) : 0.f;
    for (int o = P; o < 64; o <<= 1) s += __shfl_xor(s, o, 64);
    if ((P <= 64 ? lane : sl) < 2 * F && (P > 64 || lane < P)) {
      qf[sl] = fi < 0 ? 0.f : s;
      if ((sl & 1) == 0) cols[sl >> 1] = col;
    }
  }
}

// Adds the chunk's histogram to the unit's.
__device__ __forceinline__ void hist_flush(const uint32_t* hist_s, uint32_t* hg) {
  for (int i = threadIdx.x; i < kHistBins; i += 256) {
    const uint32_t v = hist_s[i];
    if (v != 0u) atomicAdd(&hg[i], v);
  }
}

// Adds a lane's 4 consecutive tokens j0 .. j0+3 (candidates in [c_lo, c_hi)
// only) to the LDS histogram of coarse key bins; equal bins are merged first.
__device__ __forceinline__ void hist_add4(uint32_t* hist_s, const float (&acc)[4], int j0, bool live, int c_lo,
                                          int c_hi) {
  uint32_t run_bin = 0u, run_cnt = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = j0 + r;
    const bool act = live && j >= c_lo && j < c_hi;
    const uint32_t bin = score_key(acc[r]) >> kHistShift;
    const bool brk = act && bin != run_bin;
    if (brk && run_cnt != 0u) atomicAdd(&hist_s[run_bin], run_cnt);
    run_cnt = brk ? 1u : run_cnt + (act ? 1u : 0u);
    run_bin = brk ? bin : run_bin;
  }
  if (run_cnt != 0u) atomicAdd(&hist_s[run_bin], run_cnt);
}

// FT > 0: compile-time F (all loads of a block issued back to back); FT == 0: runtime F.
template <typename T, int FT, bool FROM_SLAB, int MODE>
__global__ __launch_bounds__(256) void tip_kernel(TipArgs a) {
  constexpr bool HIST = MODE == kTipHist, EMIT = MODE == kTipEmit || MODE == kTipEmitHist, LDS_HIST = HIST || EMIT;
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z, g = wg.y;
  const int F = FT > 0 ? FT : c.n_fc;
  // The wave index is made explicitly uniform so the block-table entry (row
  // gather only) is a scalar load, issued at once and waited on its own counter.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int blk = wg.x * 4 + wave;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;

  // Independent loads: (sequence length, the slab), then (wave 0) the FC
  // indices and the query values the fold needs; the fold waits for them while
  // the slab stream is in flight.  The row-gather path also needs the
  // block-table entry before its key loads.
  const int e = threadIdx.x;
  const int t_raw = a.seq_lens[b];
  // The fold's column slots (used by wave 0; see below): P = 2F rounded up to
  // a power of two; a lane's first slot and its FC index.
  const int P = fold_slots(F);
  const int sl0 = P <= 64 ? (lane & (P - 1)) : lane;
  const int fi0 = sl0 < 2 * F ? a.fc_idx[g * F + (sl0 >> 1)] : -1;
  const int blk_c = min(blk, c.max_blocks - 1);
  Raw8<T> x[FROM_SLAB && FT > 0 ? FT : 1];
  const T* sbase = static_cast<const T*>(a.src) + (int64_t(b) * c.max_blocks + blk_c) * c.slab_block_stride +
                   int64_t(g) * c.slab_head_stride + lane * 8;
  if constexpr (FROM_SLAB && FT > 0) {
    // Unconditional (a block past the sequence's end is within the slab and
    // its values are not used), so nothing waits for the length first.
#pragma unroll
    for (int f = 0; f < FT; ++f) x[f].load_nt(sbase + f * kSlabFcStride);
  }
  const int64_t phys_raw = FROM_SLAB ? 0 : a.block_table[int64_t(b) * c.max_blocks + blk_c];
  const int t = clamp_len(t_raw, c.max_t, c.max_blocks);
  // A workgroup whose four blocks all lie past the end of a short sequence has
  // nothing to do (the whole workgroup leaves together, before any barrier).
  if (wg.x * 4 * kBlock >= t) return;

  __shared__ float qf[kHeadDim];   // folded query, [f][2]
  __shared__ int cols[kHeadDim / 2];
  __shared__ __align__(16) uint32_t hist_s[LDS_HIST ? kHistBins : 1];
  if constexpr (LDS_HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) hist_s[i] = 0u;
  }
  const bool live = blk * kBlock < t;          // wave-uniform
  const int64_t phys = live ? phys_raw : 0;

  if (wave == 0) fold_query<T, FT>(a, b, g, F, P, sl0, fi0, qf, cols);
  __syncthreads();
  if (!LDS_HIST && !live) return;              // otherwise every wave reaches the later barriers

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
  if constexpr (FROM_SLAB) {
    if constexpr (FT > 0) {
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        float y[8];
        x[f].unpack(y);
        const float q0 = qf[2 * f], q1 = qf[2 * f + 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(q1, y[2 * r + 1], fmaf(q0, y[2 * r], acc[r]));
      }
    } else {
#pragma unroll 4
      for (int f = 0; f < F; ++f) {
        float y[8];
        load8(sbase + f * kSlabFcStride, y);
        const float q0 = qf[2 * f], q1 = qf[2 * f + 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(q1, y[2 * r + 1], fmaf(q0, y[2 * r], acc[r]));
      }
    }
  } else {
    // Same arithmetic, reading the dominant pairs from the row-major key cache.
    const T* base = static_cast<const T*>(a.src) + phys * c.kv_block_stride +
                    int64_t(g) * c.kv_head_stride + int64_t(lane) * 4 * kHeadDim;
#pragma unroll 4
    for (int f = 0; f < F; ++f) {
      const int col = cols[f];
      const float q0 = qf[2 * f], q1 = qf[2 * f + 1];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const T* row = base + r * kHeadDim + col;
        acc[r] = fmaf(q1, to_f32(row[1]), fmaf(q0, to_f32(row[0]), acc[r]));
      }
    }
  }

  }   // live

  const int j0 = blk * kBlock + lane * 4;
  if (live) {
    float* dst = a.scores + unit * c.score_stride + j0;
    if (j0 + 3 < t && (c.score_stride & 3) == 0) {
      if constexpr (EMIT) {
        // Only the select's fallback reads these scores back: streaming
        // stores, which leave no dirty lines for the kernel's end to write back.
        typedef float f4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f4v{acc[0], acc[1], acc[2], acc[3]}, reinterpret_cast<f4v*>(dst));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (j0 + r < t) dst[r] = acc[r];
    }
  }
  if constexpr (HIST) {
    // Candidates exclude the forced tokens [0, c_lo) and [c_hi, t).
    const int c_lo = min(c.n_sink, t);
    const int c_hi = max(c_lo, t - c.n_recent);
    hist_add4(hist_s, acc, j0, live, c_lo, c_hi);
    __syncthreads();
    hist_flush(hist_s, a.hist + unit * kHistBins);
  }
  if constexpr (EMIT) {
    // This chunk's candidates [max(c_lo, k0), min(c_hi, k0 + 1024)) and the
    // unit's target (the same in every chunk of the unit).
    const int c_lo = min(c.n_sink, t);
    const int c_hi = max(c_lo, t - c.n_recent);
    const int k0 = wg.x * kEmitChunk;
    const int n_in = max(0, min(c_hi, k0 + kEmitChunk) - max(c_lo, k0));
    const int nC = c_hi - c_lo;
    const uint32_t want = uint32_t(emit_target(min(c.budget, nC), nC));
    uint32_t key[4];
    bool act[4];
    uint32_t run_bin = 0u, run_cnt = 0u;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = j0 + r;
      act[r] = live && j >= c_lo && j < c_hi;
      key[r] = score_key(acc[r]);
      const uint32_t bin = key[r] >> kHistShift;
      const bool brk = act[r] && bin != run_bin;
      if (brk && run_cnt != 0u) atomicAdd(&hist_s[run_bin], run_cnt);
      run_cnt = brk ? 1u : run_cnt + (act[r] ? 1u : 0u);
      run_bin = brk ? bin : run_bin;
    }
    if (run_cnt != 0u) atomicAdd(&hist_s[run_bin], run_cnt);
    __syncthreads();
    // The bin where the count from the top first reaches `want`: thread e owns
    // bins 2047 - 8e down to 2040 - 8e; an exclusive scan over threads counts
    // the keys above them.  With want >= n_in every candidate is written (bin 0).
    // (Each wave finding the bin itself from the whole histogram, one barrier
    // instead of two, measured 0.4 us slower.)
    __shared__ uint32_t s_w[4], s_w2[4];
    __shared__ uint32_t s_bin;
    const uint4 hlo = *reinterpret_cast<const uint4*>(hist_s + kHistBins - 8 - 8 * e);
    const uint4 hhi = *reinterpret_cast<const uint4*>(hist_s + kHistBins - 4 - 8 * e);
    const uint32_t h[8] = {hhi.w, hhi.z, hhi.y, hhi.x, hlo.w, hlo.z, hlo.y, hlo.x};   // descending bins
    uint32_t hs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) hs += h[i];
    const uint32_t incl = wave_inclusive_scan(hs);
    if (lane == 63) s_w[wave] = incl;
    if (e == 0) s_bin = 0u;
    __syncthreads();
    uint32_t above = incl - hs;
#pragma unroll
    for (int w = 0; w < 4; ++w) above += (w < wave) ? s_w[w] : 0u;
    if (want < uint32_t(n_in) && above < want && want <= above + hs) {
      uint32_t cum = above;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (cum < want && want <= cum + h[i]) s_bin = uint32_t(kHistBins - 1 - 8 * e - i);
        cum += h[i];
      }
    }
    __syncthreads();
    const uint32_t tau = s_bin << kHistShift;
    // Every candidate key at or above the bin's lower edge tau, in index order
    // (lanes in order, then slots).
    bool keep[4];
    uint32_t cnt = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      keep[r] = act[r] && key[r] >= tau;
      cnt += keep[r] ? 1u : 0u;
    }
    const uint32_t pin = wave_inclusive_scan(cnt);
    if (lane == 63) s_w2[wave] = pin;
    __syncthreads();
    uint32_t pos = pin - cnt, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t v = s_w2[w];
      pos += (w < wave) ? v : 0u;
      tot += v;
    }
    uint2* out = a.slots + (unit * emit_chunks(c) + wg.x) * int64_t(kEmitChunk);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (keep[r]) out[pos] = make_uint2(key[r], uint32_t(j0 + r));
      pos += keep[r] ? 1u : 0u;
    }
    if (e == 0) a.meta[unit * emit_chunks(c) + wg.x] = make_uint2(emit_word(tot, tot < uint32_t(n_in)), tau);
    if constexpr (MODE == kTipEmitHist) {
      // The chunk's histogram (still intact: the bin search only read it) into
      // the unit's, for the FAC launch's global threshold.
      hist_flush(hist_s, a.hist + unit * kHistBins);
      if (wg.x == 0 && e == 0) a.arrive[unit] = 0u;
    }
  }
}

template <typename T, bool FROM_SLAB, int MODE>
hipError_t launch_t(const TipArgs& a, dim3 grid, hipStream_t s) {
  switch (a.c.n_fc) {
    case 8: hipLaunchKernelGGL((tip_kernel<T, 8, FROM_SLAB, MODE>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((tip_kernel<T, 16, FROM_SLAB, MODE>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((tip_kernel<T, 32, FROM_SLAB, MODE>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((tip_kernel<T, 0, FROM_SLAB, MODE>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <typename T, int MODE>
hipError_t launch_src(const TipArgs& a, dim3 grid, bool slab, hipStream_t s) {
  return slab ? launch_t<T, true, MODE>(a, grid, s) : launch_t<T, false, MODE>(a, grid, s);
}

template <typename T>
hipError_t launch_mode(const TipArgs& a, dim3 grid, bool slab, int mode, hipStream_t s) {
  if (mode == kTipHist) return launch_src<T, kTipHist>(a, grid, slab, s);
  if (mode == kTipEmit) return launch_src<T, kTipEmit>(a, grid, slab, s);
  if (mode == kTipEmitHist) return launch_src<T, kTipEmitHist>(a, grid, slab, s);
  return launch_src<T, kTipScores>(a, grid, slab, s);
}

}  // namespace

hipError_t launch_tip(const Common& c, const void* q, const void* slab, const void* k_pool,
                      const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                      float* scores, const TipOutputs& o, hipStream_t s) {
  TipArgs a{c, q, slab ? slab : k_pool, block_table, seq_lens, fc_idx, scores, o.hist, o.slots, o.meta, o.arrive};
  const int nblk = (c.max_t + kBlock - 1) / kBlock;
  const dim3 grid((nblk + 3) / 4, c.n_kv_heads, c.batch);
  const bool sl = slab != nullptr;
  return c.bf16 ? launch_mode<uint16_t>(a, grid, sl, o.mode, s) : launch_mode<float>(a, grid, sl, o.mode, s);
}

}  // namespace fasa
