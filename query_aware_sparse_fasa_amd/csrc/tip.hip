// TIP: Token Importance Prediction over the dominant frequency chunks.
//
// For every sequence b, kv head g and cached token j < t_b:
//   S[j] = sum_{h in group(g)} sum_{f < F} q_h[2 I_g[f]] k_j[2 I_g[f]] + q_h[2 I_g[f]+1] k_j[2 I_g[f]+1]
// (paper-graph-ui review of FASA, section 3.4 "Online Stage 1: Token Importance
// Predictor (TIP)", S_t as the sum of the single-FC score vectors alpha^(i) over
// I_dom; keys are cached after RoPE, so each alpha^(i) entry is the FC-i dot
// product of the post-RoPE vectors, section 3.4 "RoPE from a Frequency-Chunk
// Perspective").  The score is linear in q, so the G query heads of the group
// are first summed per dominant column (the "folded" query, 2F fp32 values);
// each token then costs 2F fused multiply-adds on 2F cache elements.
//
// Mapping (gfx950, wave64): one workgroup = 4 waves = 4 cache blocks of one
// (b, g); lane l of a wave owns tokens 4l..4l+3 of its block.  Reading the slab,
// FC f of the block is one contiguous 1 KB (bf16) run and each lane issues one
// 16-byte load per FC -- F independent loads in flight per lane, no cross-lane
// traffic, and the folded query is a wave-uniform LDS broadcast.  Scores leave
// as one 16-byte store per lane.  The kernel is a pure HBM stream
// (2 flops per 2-byte element), so there is nothing for MFMA to do.
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
  uint32_t* hist;       // [units][kHistBins] coarse key histogram (HIST only)
};

// FT > 0: compile-time F (all loads of a block issued back to back); FT == 0: runtime F.
// HIST: also add this workgroup's candidate scores to the unit's coarse histogram
// of key bits 31..21 (the first radix digit of the top-B select), while the
// scores are still in registers.
template <typename T, int FT, bool FROM_SLAB, bool HIST>
__global__ __launch_bounds__(256) void tip_kernel(TipArgs a) {
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z, g = wg.y;
  const int F = FT > 0 ? FT : c.n_fc;
  // The wave index is made explicitly uniform so the block-table entry is a
  // scalar load, issued at once and waited on its own counter.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int blk = wg.x * 4 + wave;

  // Dependency chain kept to two memory round trips: (sequence length, block
  // table entry, FC index) are independent loads; then the slab loads and the
  // query loads go out together.
  const int e = threadIdx.x;
  const int ec = e < 2 * F ? e : 0;
  const int f_q = ec >> 1, comp = ec & 1;
  const int t_raw = a.seq_lens[b];
  const int64_t phys_raw = a.block_table[int64_t(b) * c.max_blocks + min(blk, c.max_blocks - 1)];
  const int fi = a.fc_idx[g * F + f_q];          // < 0: unused slot (a head with fewer FCs)
  const int col = 2 * (fi < 0 ? 0 : fi) + comp;
  const int t = clamp_len(t_raw, c.max_t, c.max_blocks);
  // A workgroup whose four blocks all lie past the end of a short sequence has
  // nothing to do (the whole workgroup leaves together, before any barrier).
  // The slab loads need the length and the block-table entry anyway, so this
  // adds no wait for the others.
  if (wg.x * 4 * kBlock >= t) return;

  __shared__ float qf[kHeadDim];   // folded query, [f][2]
  __shared__ int cols[kHeadDim / 2];
  __shared__ uint32_t hist_s[HIST ? kHistBins : 1];
  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) hist_s[i] = 0u;
  }
  const bool live = blk * kBlock < t;          // wave-uniform
  const int64_t phys = live ? phys_raw : 0;

  // Query loads first (unconditional, head index clamped), then this block's slab
  // loads; the fold only waits for the query values.
  const T* qh = static_cast<const T*>(a.q) +
                (int64_t(b) * c.n_q_heads + int64_t(g) * c.group) * kHeadDim + col;
  T qv[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) qv[h] = qh[min(h, c.group - 1) * kHeadDim];

  Raw8<T> x[FROM_SLAB && FT > 0 ? FT : 1];
  const T* sbase = static_cast<const T*>(a.src) + phys * c.slab_block_stride +
                   int64_t(g) * c.slab_head_stride + lane * 8;
  if constexpr (FROM_SLAB && FT > 0) {
    if (live) {
#pragma unroll
      for (int f = 0; f < FT; ++f) x[f].load_nt(sbase + f * kSlabFcStride);
    }
  }
  {
    // Folded query: thread e < 2F sums column 2 I_g[f] + comp over the group's
    // heads in head order (terms past the group are masked to +0).
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < 16; ++h) s += (h < c.group) ? to_f32(qv[h]) : 0.f;
    if (e < 2 * F) {
      qf[e] = fi < 0 ? 0.f : s;                  // an unused slot scores nothing
      if (comp == 0) cols[f_q] = col;
    }
  }
  __syncthreads();
  if (!HIST && !live) return;                  // with HIST every wave reaches the second barrier

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
    float* dst = a.scores + (int64_t(b) * c.n_kv_heads + g) * c.score_stride + j0;
    if (j0 + 3 < t && (c.score_stride & 3) == 0) {
      *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (j0 + r < t) dst[r] = acc[r];
    }
  }
  if constexpr (HIST) {
    // Candidates exclude the forced tokens [0, c_lo) and [c_hi, t).  A lane's 4
    // tokens are consecutive: equal bins are merged before the LDS add.
    const int c_lo = min(c.n_sink, t);
    const int c_hi = max(c_lo, t - c.n_recent);
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
    __syncthreads();
    uint32_t* hg = a.hist + (int64_t(b) * c.n_kv_heads + g) * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += 256) {
      const uint32_t v = hist_s[i];
      if (v != 0u) atomicAdd(&hg[i], v);
    }
  }
}

template <typename T, bool FROM_SLAB, bool HIST>
hipError_t launch_t(const TipArgs& a, dim3 grid, hipStream_t s) {
  switch (a.c.n_fc) {
    case 8: hipLaunchKernelGGL((tip_kernel<T, 8, FROM_SLAB, HIST>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((tip_kernel<T, 16, FROM_SLAB, HIST>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((tip_kernel<T, 32, FROM_SLAB, HIST>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((tip_kernel<T, 0, FROM_SLAB, HIST>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <typename T, bool HIST>
hipError_t launch_src(const TipArgs& a, dim3 grid, bool slab, hipStream_t s) {
  return slab ? launch_t<T, true, HIST>(a, grid, s) : launch_t<T, false, HIST>(a, grid, s);
}

}  // namespace

hipError_t launch_tip(const Common& c, const void* q, const void* slab, const void* k_pool,
                      const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                      float* scores, uint32_t* hist, hipStream_t s) {
  TipArgs a{c, q, slab ? slab : k_pool, block_table, seq_lens, fc_idx, scores, hist};
  const int nblk = (c.max_t + kBlock - 1) / kBlock;
  const dim3 grid((nblk + 3) / 4, c.n_kv_heads, c.batch);
  const bool sl = slab != nullptr;
  if (c.bf16)
    return hist ? launch_src<uint16_t, true>(a, grid, sl, s) : launch_src<uint16_t, false>(a, grid, sl, s);
  return hist ? launch_src<float, true>(a, grid, sl, s) : launch_src<float, false>(a, grid, sl, s);
}

}  // namespace fasa
