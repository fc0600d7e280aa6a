// Dominant-key cache ("slab") maintenance.
//
// FASA's TIP stage only ever reads the dimensions of the dominant FCs of the
// cached keys; the pages keep exactly those dimensions GPU-resident as the
// dominant key cache C_key^dom (paper-graph-ui review of FASA, section 3.4,
// "Hardware-Aware Variants", FASA-M component 1 and FASA-C).  Read in place
// from a row-major key cache, 16 scattered FC pairs of a 256-byte bf16 row
// still touch almost every 32-byte sector, so TIP would pay for the whole key
// row.  The slab stores those columns FC-major per 256-token block, indexed by
// the sequence and the block's logical position in it (not by the physical
// block of the pool),
//   [sequence][logical block][kv head][F][256 tokens][2],
// so one FC of one block is a contiguous 1 KB (bf16) run that a wave reads
// with one 16-byte load per lane, and TIP finds it without reading the block
// table.  It is written once per token (append) or once per prefix (build),
// never per decode step.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

template <typename T>
struct Pair;
template <>
struct Pair<uint16_t> { using type = uint32_t; };
template <>
struct Pair<float> { using type = uint2; };

template <typename T>
__global__ __launch_bounds__(256) void slab_build_kernel(Common c, const T* __restrict__ k_pool,
                                                         const int32_t* __restrict__ block_table,
                                                         const int32_t* __restrict__ seq_lens,
                                                         const int32_t* __restrict__ fc_idx,
                                                         T* __restrict__ slab) {
  using P = typename Pair<T>::type;
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = clamp_len(seq_lens[b], c.max_t, c.max_blocks);
  if (blk * kBlock >= t) return;
  const int64_t phys = block_table[int64_t(b) * c.max_blocks + blk];
  const int s = threadIdx.x;
  const T* src = k_pool + phys * c.kv_block_stride + int64_t(g) * c.kv_head_stride + int64_t(s) * kHeadDim;
  T* dst = slab + (int64_t(b) * c.max_blocks + blk) * c.slab_block_stride + int64_t(g) * c.slab_head_stride + 2 * s;
  for (int f = 0; f < c.n_fc; ++f) {
    const int fi = fc_idx[g * c.n_fc + f];     // < 0: an unused slot of a head with fewer FCs, kept zero
    *reinterpret_cast<P*>(dst + int64_t(f) * kSlabFcStride) =
        fi >= 0 ? *reinterpret_cast<const P*>(src + 2 * fi) : P{};
  }
}

template <typename T>
__global__ __launch_bounds__(64) void slab_append_kernel(Common c, const T* __restrict__ k_pool,
                                                         const int32_t* __restrict__ block_table,
                                                         const int32_t* __restrict__ positions,
                                                         const int32_t* __restrict__ fc_idx,
                                                         T* __restrict__ slab) {
  using P = typename Pair<T>::type;
  const int b = blockIdx.x, g = blockIdx.y;
  const int pos = positions[b];
  if (pos < 0 || pos >= c.max_blocks * kBlock) return;
  const int64_t phys = block_table[int64_t(b) * c.max_blocks + (pos >> 8)];
  const int s = pos & (kBlock - 1);
  const T* src = k_pool + phys * c.kv_block_stride + int64_t(g) * c.kv_head_stride + int64_t(s) * kHeadDim;
  T* dst = slab + (int64_t(b) * c.max_blocks + (pos >> 8)) * c.slab_block_stride + int64_t(g) * c.slab_head_stride +
           2 * s;
  for (int f = threadIdx.x; f < c.n_fc; f += 64) {
    const int fi = fc_idx[g * c.n_fc + f];
    *reinterpret_cast<P*>(dst + int64_t(f) * kSlabFcStride) =
        fi >= 0 ? *reinterpret_cast<const P*>(src + 2 * fi) : P{};
  }
}

}  // namespace

hipError_t launch_slab_build(const Common& c, const void* k_pool, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* fc_idx, void* slab,
                             hipStream_t s) {
  const dim3 grid(c.max_blocks, c.n_kv_heads, c.batch);
  if (c.bf16)
    hipLaunchKernelGGL(slab_build_kernel<uint16_t>, grid, dim3(256), 0, s, c,
                       static_cast<const uint16_t*>(k_pool), block_table, seq_lens, fc_idx,
                       static_cast<uint16_t*>(slab));
  else
    hipLaunchKernelGGL(slab_build_kernel<float>, grid, dim3(256), 0, s, c,
                       static_cast<const float*>(k_pool), block_table, seq_lens, fc_idx,
                       static_cast<float*>(slab));
  return hipGetLastError();
}

hipError_t launch_slab_append(const Common& c, const void* k_pool, const int32_t* block_table,
                              const int32_t* positions, const int32_t* fc_idx, void* slab,
                              hipStream_t s) {
  const dim3 grid(c.batch, c.n_kv_heads);
  if (c.bf16)
    hipLaunchKernelGGL(slab_append_kernel<uint16_t>, grid, dim3(64), 0, s, c,
                       static_cast<const uint16_t*>(k_pool), block_table, positions, fc_idx,
                       static_cast<uint16_t*>(slab));
  else
    hipLaunchKernelGGL(slab_append_kernel<float>, grid, dim3(64), 0, s, c,
                       static_cast<const float*>(k_pool), block_table, positions, fc_idx,
                       static_cast<float*>(slab));
  return hipGetLastError();
}

}  // namespace fasa
