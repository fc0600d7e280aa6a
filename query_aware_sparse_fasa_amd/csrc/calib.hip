// Offline calibration: Contextual Agreement (CA) of every frequency chunk with
// its head, and the dominant FCs that follow from it (paper-graph-ui review of
// FASA, section 3.4: the CA metric, and the offline calibration that keeps the
// N_tip FCs of highest mean CA).
//
// One calibration row is one decode query (sequence b, position t_b) against
// the keys 0..t_b-1 of the paged cache.  For every kv head g (the group's
// queries summed per column, as TIP scores them):
//   alpha_j     = q~ . k_j                                  (the full head)
//   alpha^(i)_j = q~_2i k_j,2i + q~_2i+1 k_j,2i+1            (FC i alone)
//   hits[b][g][i] = |TopK-I(alpha, K) n TopK-I(alpha^(i), K)|, CA = hits / K.
// Since the top-K sets decide integers, the scores are computed in float32 in
// one fixed order with no fused multiply-add: q~ summed over the group's heads
// in head order, each pair as fl(fl(q x k) + fl(q x k)), alpha as the FC terms
// added in FC order.
//
// Kernels: ca_scores_kernel writes the 65 score rows of every unit (alpha, then
// alpha^(0..63)) into the workspace; the library's exact top-K (filter and
// finish launches, run with 65 * H_kv "units" per sequence) selects every row;
// ca_hits_kernel intersects the 64 FC lists with the head's list.
// ca_dominant_kernel sums the hits over calibration rows and keeps the N_tip
// largest sums per kv head (lower FC index on ties), in ascending FC order.
#include "fasa_device.hpp"
#include "fasa_internal.hpp"

namespace fasa {
namespace {

constexpr int kFcAll = kHeadDim / 2;   // 64 FCs
constexpr int kCaRows = kFcAll + 1;    // alpha and the 64 alpha^(i)

struct CaArgs {
  Common c;
  const void* q;
  const void* k_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* scores;           // [b][H_kv][65][score_stride]
  const int32_t* sel_idx;  // [b][H_kv * 65][cap]
  const int32_t* sel_count;
  int32_t* hits;           // [b][H_kv][64]
  int32_t* topk;           // nullable: [b][H_kv][65][cap] copies of the lists, -1 padded
};

// Grid (ceil(max_t / 256), H_kv, batch), one thread per token.
template <typename T>
__global__ __launch_bounds__(256) void ca_scores_kernel(CaArgs a) {
  const Common& c = a.c;
  const int b = blockIdx.z, g = blockIdx.y;
  const int j = blockIdx.x * kBlock + threadIdx.x;
  __shared__ float qf[kHeadDim];
  if (threadIdx.x < kHeadDim) {
    const T* qh = static_cast<const T*>(a.q) + (int64_t(b) * c.n_q_heads + int64_t(g) * c.group) * kHeadDim;
    float s = 0.f;
    for (int h = 0; h < c.group; ++h) s = __fadd_rn(s, to_f32(qh[int64_t(h) * kHeadDim + threadIdx.x]));
    qf[threadIdx.x] = s;
  }
  __syncthreads();
  const int t = clamp_len(a.seq_lens[b], c.max_t, c.max_blocks);
  if (j >= t) return;
  const int64_t pb = a.block_table[int64_t(b) * c.max_blocks + (j >> 8)];
  const T* kr = static_cast<const T*>(a.k_pool) + pb * c.kv_block_stride + int64_t(g) * c.kv_head_stride +
                int64_t(j & (kBlock - 1)) * kHeadDim;
  float* out = a.scores + ((int64_t(b) * c.n_kv_heads + g) * kCaRows) * c.score_stride + j;
  float full = 0.f;
#pragma unroll 4
  for (int p = 0; p < kHeadDim / 8; ++p) {
    Raw8<T> x;
    x.load(kr + 8 * p);
    float k8[8];
    x.unpack(k8);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * p + u;
      const float fc = __fadd_rn(__fmul_rn(qf[2 * i], k8[2 * u]), __fmul_rn(qf[2 * i + 1], k8[2 * u + 1]));
      out[int64_t(1 + i) * c.score_stride] = fc;
      full = __fadd_rn(full, fc);
    }
  }
  out[0] = full;
}

// Grid (H_kv, batch), 256 threads.  The head's list (ascending) is staged in
// LDS; every FC list element is looked up there by binary search.
__global__ __launch_bounds__(256) void ca_hits_kernel(CaArgs a) {
  const Common& c = a.c;
  const int g = blockIdx.x, b = blockIdx.y;
  const int64_t u0 = (int64_t(b) * c.n_kv_heads + g) * kCaRows;   // the unit of alpha
  __shared__ int32_t full[kCaMaxK];
  __shared__ uint32_t cnt[kFcAll];
  const int nf = min(max(a.sel_count[u0], 0), min(c.cap, kCaMaxK));
  for (int e = threadIdx.x; e < nf; e += 256) full[e] = a.sel_idx[u0 * c.cap + e];
  if (threadIdx.x < kFcAll) cnt[threadIdx.x] = 0u;
  __syncthreads();
  // Thread t walks FC (t & 63)'s list from element t >> 6 in steps of 4.
  const int i = threadIdx.x & (kFcAll - 1);
  const int64_t ui = u0 + 1 + i;
  const int ni = min(max(a.sel_count[ui], 0), c.cap);
  uint32_t h = 0;
  for (int e = threadIdx.x >> 6; e < ni; e += 256 / kFcAll) {
    const int x = a.sel_idx[ui * c.cap + e];
    int lo = 0, hi = nf;                   // first position with full[pos] >= x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (full[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    h += (lo < nf && full[lo] == x) ? 1u : 0u;
  }
  atomicAdd(&cnt[i], h);
  if (a.topk != nullptr) {
    // The 65 lists behind the counts, each padded with -1 to cap entries.
    for (int r = 0; r < kCaRows; ++r) {
      const int64_t ur = u0 + r;
      const int n = min(max(a.sel_count[ur], 0), c.cap);
      for (int e = threadIdx.x; e < c.cap; e += 256) a.topk[ur * c.cap + e] = e < n ? a.sel_idx[ur * c.cap + e] : -1;
    }
  }
  __syncthreads();
  if (threadIdx.x < kFcAll) a.hits[(int64_t(b) * c.n_kv_heads + g) * kFcAll + threadIdx.x] = int32_t(cnt[threadIdx.x]);
}

// Grid (H_kv), 64 threads (one wave): FC i = lane.  Sums the hits of n_rows
// calibration rows, ranks the FCs (more hits first, lower index on ties) and
// writes the n_tip best in ascending order.
__global__ __launch_bounds__(64) void ca_dominant_kernel(const int32_t* hits, int n_rows, int n_kv, int n_tip,
                                                         int32_t* fc_idx) {
  const int g = blockIdx.x, i = threadIdx.x;
  __shared__ int64_t tot[kFcAll];
  int64_t s = 0;
  for (int r = 0; r < n_rows; ++r) s += hits[(int64_t(r) * n_kv + g) * kFcAll + i];
  tot[i] = s;
  __syncthreads();
  int rank = 0;
  for (int k = 0; k < kFcAll; ++k) rank += (tot[k] > s || (tot[k] == s && k < i)) ? 1 : 0;
  const bool take = rank < n_tip;
  const uint64_t m = __ballot(take);
  const int pos = __popcll(m & ((uint64_t(1) << i) - 1));
  if (take) fc_idx[int64_t(g) * n_tip + pos] = i;
}

}  // namespace

hipError_t launch_ca_scores(const Common& c, const void* q, const void* k_pool, const int32_t* block_table,
                            const int32_t* seq_lens, float* scores, hipStream_t s) {
  CaArgs a{c, q, k_pool, block_table, seq_lens, scores, nullptr, nullptr, nullptr, nullptr};
  const dim3 grid((c.max_t + kBlock - 1) / kBlock, c.n_kv_heads, c.batch);
  if (c.bf16) hipLaunchKernelGGL(ca_scores_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(ca_scores_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ca_hits(const Common& c, const int32_t* sel_idx, const int32_t* sel_count, int32_t* hits,
                          int32_t* topk, hipStream_t s) {
  CaArgs a{c, nullptr, nullptr, nullptr, nullptr, nullptr, sel_idx, sel_count, hits, topk};
  hipLaunchKernelGGL(ca_hits_kernel, dim3(c.n_kv_heads, c.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ca_dominant(const int32_t* hits, int n_rows, int n_kv, int n_tip, int32_t* fc_idx,
                              hipStream_t s) {
  hipLaunchKernelGGL(ca_dominant_kernel, dim3(n_kv), dim3(kFcAll), 0, s, hits, n_rows, n_kv, n_tip, fc_idx);
  return hipGetLastError();
}

}  // namespace fasa
