// FASA-M: the memory-optimised placement of the cache (paper-graph-ui review of
// FASA, section 3.4 "Hardware-Aware Variants", FASA-M and Equation 10).  The GPU
// keeps the dominant-key cache (the slab) and per-step buffers only; the
// non-dominant key columns and all value rows live in pinned host memory.  TIP
// needs only the slab; after the selection, the selected rows' non-dominant key
// columns and values are read from host memory (the GPU reads the pinned pages
// directly, over the host link) and put back together with the dominant
// columns from the slab into full rows in a device staging area, which FAC then
// reads.
//
// Host layouts (element type = the cache type), indexed by the pool's physical
// block like the pool and the slab:
//   k_nd [block][H_kv][256][nd_stride]: the 128 - 2F non-dominant key columns of
//        every token in ascending column order, each row padded with zeros to
//        nd_stride elements (a multiple of 16 bytes);
//   v    [block][H_kv][256][128]: the value rows.
// Staging (device workspace): [b][H_kv][cap][128] for K and for V; row r of a
// unit is its r-th selected token.
//
// Prefetch (the latency mitigation of the same section: while TIP runs, the
// keys and values that the previous query needed are loaded in advance): the
// previous step's selection is gathered, the same way, into a second pair of
// staging arrays (the prefetch area) on another stream, concurrently with
// TIP and the select; the step's own gather then takes every selected row that
// the previous step also selected from the prefetch area (device memory) and
// only the others from the host.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

struct MArgs {
  Common c;
  const void* k_pool;       // offload: device pools
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* fc_idx;    // [H_kv][F]
  void* k_nd;               // host (device-visible alias)
  void* v_host;
  const void* slab;         // gather: dominant pairs
  const int32_t* sel_idx;   // gather: the selection
  const int32_t* sel_count;
  void* stage_k;            // gather: device staging
  void* stage_v;
  int nd_stride;            // elements per k_nd row
  // Gather with reuse: the previous selection and its rows in the prefetch area.
  const int32_t* prev_idx;  // [b][H_kv][cap], ascending
  const int32_t* prev_count;
  const void* pf_k;         // [b][H_kv][cap][128], row p = token prev_idx[p]
  const void* pf_v;
  int32_t* hits;            // nullable: rows taken from the prefetch area, added per unit
};

// Raw element of the cache type.
template <typename T>
struct Bits;
template <>
struct Bits<uint16_t> { typedef uint16_t type; };
template <>
struct Bits<float> { typedef uint32_t type; };

// Column map of kv head g in LDS: dom_f[p] = f when FC pair p is the f-th
// dominant one, else -1; nd_pos[c] = position of channel c among the
// non-dominant columns (unused for dominant channels).  Wave 0, lane p, handles
// pair p.  Published by the caller's next barrier.
__device__ __forceinline__ void column_map(const Common& c, const int32_t* fc_idx, int g, int* dom_f, int* nd_pos) {
  if (threadIdx.x < 64) {
    const int p = threadIdx.x;
    int f_of = -1;
    for (int f = 0; f < c.n_fc; ++f) f_of = (fc_idx[g * c.n_fc + f] == p) ? f : f_of;
    const uint64_t nd_mask = __ballot(f_of < 0);
    const int rank = __popcll(nd_mask & ((uint64_t(1) << p) - 1));
    dom_f[p] = f_of;
    nd_pos[2 * p] = 2 * rank;
    nd_pos[2 * p + 1] = 2 * rank + 1;
  }
}

// Offload of whole blocks: grid (max_blocks, H_kv, batch), 256 threads, 64
// tokens per pass; 4 threads per token, 32 channels each, moved in 16-byte
// pieces.  Blocks at or past ceil(t_b / 256) leave at once.
template <typename T>
__global__ __launch_bounds__(256) void fasam_offload_kernel(MArgs a) {
  typedef typename Bits<T>::type E;
  constexpr int PER = 16 / int(sizeof(E));          // elements per 16-byte piece
  constexpr int NP = 32 / PER;                      // pieces per thread
  const Common& c = a.c;
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = clamp_len(a.seq_lens[b], c.max_t, c.max_blocks);
  if (blk * kBlock >= t) return;
  const int64_t pb = a.block_table[int64_t(b) * c.max_blocks + blk];
  __shared__ int dom_f[64];
  __shared__ int nd_pos[kHeadDim];
  __shared__ __align__(16) E nd[64 * kHeadDim];
  column_map(c, a.fc_idx, g, dom_f, nd_pos);
  const int nd_n = kHeadDim - 2 * c.n_fc;
  const int tok = threadIdx.x >> 2, q = threadIdx.x & 3;
  const E* kp = static_cast<const E*>(a.k_pool) + pb * c.kv_block_stride + int64_t(g) * c.kv_head_stride;
  const E* vp = static_cast<const E*>(a.v_pool) + pb * c.kv_block_stride + int64_t(g) * c.kv_head_stride;
  E* knd = static_cast<E*>(a.k_nd) + ((pb * c.n_kv_heads + g) * kBlock) * int64_t(a.nd_stride);
  E* vh = static_cast<E*>(a.v_host) + ((pb * c.n_kv_heads + g) * kBlock) * int64_t(kHeadDim);
  for (int pass = 0; pass < kBlock / 64; ++pass) {
    const int s = pass * 64 + tok;
    const int64_t o = int64_t(s) * kHeadDim + 32 * q;
    uint4 kx[NP], vx[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      kx[k] = reinterpret_cast<const uint4*>(kp + o)[k];
      vx[k] = reinterpret_cast<const uint4*>(vp + o)[k];
    }
    __syncthreads();                       // the map is published; the previous pass has left LDS
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      reinterpret_cast<uint4*>(vh + o)[k] = vx[k];
      const E* xe = reinterpret_cast<const E*>(&kx[k]);
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int ch = 32 * q + PER * k + e;
        if (dom_f[ch >> 1] < 0) nd[tok * a.nd_stride + nd_pos[ch]] = xe[e];
      }
    }
    if (q == 3)
      for (int e = nd_n; e < a.nd_stride; ++e) nd[tok * a.nd_stride + e] = E(0);
    __syncthreads();
    // The 64 rows are one contiguous run of the host array: 16-byte stores.
    const int words = 64 * a.nd_stride * int(sizeof(E)) / 16;
    const uint4* src = reinterpret_cast<const uint4*>(nd);
    uint4* dst = reinterpret_cast<uint4*>(knd + int64_t(pass * 64) * a.nd_stride);
    for (int i = threadIdx.x; i < words; i += 256) dst[i] = src[i];
  }
}

// Gather of the selected rows: grid (ceil(cap / 16), H_kv, batch), 256 threads,
// 16 rows per workgroup and 16 lanes per row (8 channels each).  A row's
// non-dominant key columns come over in 16-byte pieces into LDS, its value
// channels straight into registers (16-byte pieces too: host reads are not
// cached, so every piece is one transfer), its dominant pairs from the slab;
// the full key row is then written in channel order.
// REUSE: the gather with reuse (see the head of the file): the previous
// selection (at most kPrevLds entries) is staged in LDS and searched for each
// row's token; a row found there is copied from the prefetch area.
constexpr int kPrevLds = 8192;
template <typename T, bool REUSE>
__global__ __launch_bounds__(256) void fasam_gather_kernel(MArgs a) {
  typedef typename Bits<T>::type E;
  constexpr int EPL = 8;                                   // channels per lane
  constexpr int LP = EPL * int(sizeof(E)) / 16;            // 16-byte pieces per lane and row
  const Common& c = a.c;
  const int g = blockIdx.y, b = blockIdx.z;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;
  const int i = threadIdx.x >> 4, lane = threadIdx.x & 15;
  const int r = blockIdx.x * 16 + i;
  __shared__ int dom_f[64];
  __shared__ int nd_pos[kHeadDim];
  __shared__ __align__(16) E nd[16 * kHeadDim];
  __shared__ int prev_s[REUSE ? kPrevLds : 1];
  column_map(c, a.fc_idx, g, dom_f, nd_pos);

  int count = a.sel_count[unit];
  count = count < 0 ? 0 : (count > c.cap ? c.cap : count);
  const bool live = r < count;
  int j = live ? a.sel_idx[unit * c.cap + r] : 0;
  j = (j < 0 || j >= c.max_blocks * kBlock) ? 0 : j;
  const int64_t pb = a.block_table[int64_t(b) * c.max_blocks + (j >> 8)];
  const int s = j & (kBlock - 1);
  const int64_t hrow = (pb * c.n_kv_heads + g) * kBlock + s;

  // REUSE: where the row's token sits in the previous selection, or -1.
  int hit = -1;
  if constexpr (REUSE) {
    int np = a.prev_count[unit];
    np = np < 0 ? 0 : (np > c.cap ? c.cap : np);
    for (int k = threadIdx.x; k < np; k += 256) prev_s[k] = a.prev_idx[unit * c.cap + k];
    __syncthreads();                                        // the list (and the column map)
    int lo = 0, hi = np;                                    // first position with prev_s[pos] >= j
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (prev_s[mid] < j) lo = mid + 1;
      else hi = mid;
    }
    hit = (live && lo < np && prev_s[lo] == j) ? lo : -1;
    if (a.hits != nullptr) {
      const uint64_t m = __ballot(hit >= 0 && lane == 0);
      if ((threadIdx.x & 63) == 0 && m != 0u) atomicAdd(&a.hits[unit], int32_t(__popcll(m)));
    }
  }
  const bool from_host = live && hit < 0;

  // Host reads: this row's non-dominant pieces (lane l takes pieces l, l + 16)
  // and the lane's value channels.  A row found in the prefetch area reads its
  // whole key and value rows from there instead.
  const int nd_pieces = a.nd_stride * int(sizeof(E)) / 16;
  const uint4* knd = reinterpret_cast<const uint4*>(static_cast<const E*>(a.k_nd) + hrow * a.nd_stride);
  const uint4* vh = reinterpret_cast<const uint4*>(static_cast<const E*>(a.v_host) + hrow * kHeadDim + EPL * lane);
  uint4 piece[LP], vx[LP], pk[LP];
#pragma unroll
  for (int k = 0; k < LP; ++k) {
    const int pc = lane + 16 * k;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    piece[k] = (from_host && pc < nd_pieces) ? knd[pc] : z;
    vx[k] = from_host ? vh[k] : z;
    pk[k] = z;
  }
  if constexpr (REUSE) {
    if (hit >= 0) {
      const int64_t prow = (unit * c.cap + hit) * int64_t(kHeadDim) + EPL * lane;
      const uint4* fk = reinterpret_cast<const uint4*>(static_cast<const E*>(a.pf_k) + prow);
      const uint4* fv = reinterpret_cast<const uint4*>(static_cast<const E*>(a.pf_v) + prow);
#pragma unroll
      for (int k = 0; k < LP; ++k) {
        pk[k] = fk[k];
        vx[k] = fv[k];
      }
    }
  }
  if constexpr (!REUSE) __syncthreads();                    // the column map
  // Dominant pairs of the lane's 4 FC pairs, from the slab (device; indexed by
  // the sequence and the logical block).
  const E* sl = static_cast<const E*>(a.slab) + (int64_t(b) * c.max_blocks + (j >> 8)) * c.slab_block_stride +
                int64_t(g) * c.slab_head_stride + s * 2;
  E dv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int f = dom_f[(EPL * lane + e) >> 1];
    dv[e] = (from_host && f >= 0) ? sl[int64_t(f) * kSlabFcStride + (e & 1)] : E(0);
  }
#pragma unroll
  for (int k = 0; k < LP; ++k) {
    const int pc = lane + 16 * k;
    if (pc < nd_pieces) reinterpret_cast<uint4*>(nd + i * kHeadDim)[pc] = piece[k];
  }
  __syncthreads();
  if (!live) return;
  uint4 kx[LP];
  E* ke = reinterpret_cast<E*>(kx);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int ch = EPL * lane + e;
    ke[e] = dom_f[ch >> 1] >= 0 ? dv[e] : nd[i * kHeadDim + nd_pos[ch]];
  }
  if (hit >= 0) {
#pragma unroll
    for (int k = 0; k < LP; ++k) kx[k] = pk[k];
  }
  const int64_t row = (unit * c.cap + r) * int64_t(kHeadDim) + EPL * lane;
  uint4* sk = reinterpret_cast<uint4*>(static_cast<E*>(a.stage_k) + row);
  uint4* sv = reinterpret_cast<uint4*>(static_cast<E*>(a.stage_v) + row);
#pragma unroll
  for (int k = 0; k < LP; ++k) {
    sk[k] = kx[k];
    sv[k] = vx[k];
  }
}

}  // namespace

int m_nd_stride(const Common& c) {
  const int e = c.bf16 ? 2 : 4;
  const int bytes = (kHeadDim - 2 * c.n_fc) * e;
  return ((bytes + 15) / 16) * 16 / e;
}

hipError_t launch_m_offload(const Common& c, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* fc_idx, void* k_nd, void* v_host,
                            hipStream_t s) {
  MArgs a{c, k_pool, v_pool, block_table, seq_lens, fc_idx, k_nd, v_host, nullptr, nullptr, nullptr,
          nullptr, nullptr, m_nd_stride(c)};
  const dim3 grid(c.max_blocks, c.n_kv_heads, c.batch);
  if (c.bf16) hipLaunchKernelGGL(fasam_offload_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fasam_offload_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_m_gather(const Common& c, const void* k_nd, const void* v_host, const void* slab,
                           const int32_t* block_table, const int32_t* fc_idx, const int32_t* sel_idx,
                           const int32_t* sel_count, void* stage_k, void* stage_v, const MReuse& reuse,
                           hipStream_t s) {
  if (c.cap == 0) return hipSuccess;
  MArgs a{c, nullptr, nullptr, block_table, nullptr, fc_idx, const_cast<void*>(k_nd), const_cast<void*>(v_host),
          slab, sel_idx, sel_count, stage_k, stage_v, m_nd_stride(c),
          reuse.prev_idx, reuse.prev_count, reuse.pf_k, reuse.pf_v, reuse.hits};
  const dim3 grid((c.cap + 15) / 16, c.n_kv_heads, c.batch);
  const bool re = reuse.prev_idx != nullptr && m_reuses(c);
  if (c.bf16) {
    if (re) hipLaunchKernelGGL((fasam_gather_kernel<uint16_t, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((fasam_gather_kernel<uint16_t, false>), grid, dim3(256), 0, s, a);
  } else {
    if (re) hipLaunchKernelGGL((fasam_gather_kernel<float, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((fasam_gather_kernel<float, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool m_reuses(const Common& c) { return c.cap <= kPrevLds; }

}  // namespace fasa
