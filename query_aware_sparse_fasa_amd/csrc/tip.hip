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
};

// FT > 0: compile-time F (all loads of a block issued back to back); FT == 0: runtime F.
template <typename T, int FT, bool FROM_SLAB>
__global__ __launch_bounds__(256) void tip_kernel(TipArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.z, g = blockIdx.y;
  const int F = FT > 0 ? FT : c.n_fc;
  const int t = clamp_len(a.seq_lens[b], c.max_t, c.max_blocks);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + wave;
  if (blockIdx.x * 4 * kBlock >= t) return;   // whole workgroup past the end

  __shared__ float qf[kHeadDim];   // folded query, [f][2]
  __shared__ int cols[kHeadDim / 2];
  {
    const int e = threadIdx.x;
    if (e < 2 * F) {
      const int f = e >> 1, comp = e & 1;
      const int col = 2 * a.fc_idx[g * F + f] + comp;
      const T* qh = static_cast<const T*>(a.q) +
                    (int64_t(b) * c.n_q_heads + int64_t(g) * c.group) * kHeadDim + col;
      float s = 0.f;
      for (int h = 0; h < c.group; ++h) s += to_f32(qh[h * kHeadDim]);
      qf[e] = s;
      if (comp == 0) cols[f] = col;
    }
  }
  __syncthreads();
  if (blk * kBlock >= t) return;

  const int64_t phys = a.block_table[int64_t(b) * c.max_blocks + blk];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FROM_SLAB) {
    const T* base = static_cast<const T*>(a.src) + phys * c.slab_block_stride +
                    int64_t(g) * c.slab_head_stride + lane * 8;
    if constexpr (FT > 0) {
      float x[FT][8];
#pragma unroll
      for (int f = 0; f < FT; ++f) load8(base + f * kSlabFcStride, x[f]);
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const float q0 = qf[2 * f], q1 = qf[2 * f + 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(q1, x[f][2 * r + 1], fmaf(q0, x[f][2 * r], acc[r]));
      }
    } else {
#pragma unroll 4
      for (int f = 0; f < F; ++f) {
        float x[8];
        load8(base + f * kSlabFcStride, x);
        const float q0 = qf[2 * f], q1 = qf[2 * f + 1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(q1, x[2 * r + 1], fmaf(q0, x[2 * r], acc[r]));
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

  const int j0 = blk * kBlock + lane * 4;
  float* dst = a.scores + (int64_t(b) * c.n_kv_heads + g) * c.max_t + j0;
  if (j0 + 3 < t && (c.max_t & 3) == 0) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (j0 + r < t) dst[r] = acc[r];
  }
}

template <typename T, bool FROM_SLAB>
hipError_t launch_t(const TipArgs& a, dim3 grid, hipStream_t s) {
  switch (a.c.n_fc) {
    case 8: hipLaunchKernelGGL((tip_kernel<T, 8, FROM_SLAB>), grid, dim3(256), 0, s, a); break;
    case 16: hipLaunchKernelGGL((tip_kernel<T, 16, FROM_SLAB>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((tip_kernel<T, 32, FROM_SLAB>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((tip_kernel<T, 0, FROM_SLAB>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tip(const Common& c, const void* q, const void* slab, const void* k_pool,
                      const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                      float* scores, hipStream_t s) {
  TipArgs a{c, q, slab ? slab : k_pool, block_table, seq_lens, fc_idx, scores};
  const int nblk = (c.max_t + kBlock - 1) / kBlock;
  const dim3 grid((nblk + 3) / 4, c.n_kv_heads, c.batch);
  if (c.bf16)
    return slab ? launch_t<uint16_t, true>(a, grid, s) : launch_t<uint16_t, false>(a, grid, s);
  return slab ? launch_t<float, true>(a, grid, s) : launch_t<float, false>(a, grid, s);
}

}  // namespace fasa
