// FAC: Focused Attention Computation over the selected rows.
//
// For every query head h of kv head g: out_h = softmax(q_h K_T^T * scale) V_T,
// where K_T, V_T are the cached rows at the selected token indices, used in
// place at their original positions (paper-graph-ui review of FASA, section 3.4
// "Online Stage 2: Focused Attention Computation (FAC)", gather and attention
// equations).  The gather is never materialised: each selected row is read
// straight from the paged pool through the block table.
//
// Split-K flash decode.  A workgroup is 4 waves; each wave walks its own run of
// selected rows and keeps a running (max m, sum l, acc[128]) per query head --
// the online softmax.  Every K/V row is loaded once per kv head and reused by
// all query heads of the group (GQA).  The workgroup folds its waves into one
// partial.  The partials of a head are merged with the log-sum-exp rule, in a
// decode step with a small grid by the last workgroup of the head's split to
// finish (an arrival counter decides which), otherwise by a second launch.
// Per wave, bf16 caches run on the matrix cores (FacWaveMfma: 16-row blocks,
// logits and the weighted sum as 16 x 16 matrix products with the heads padded
// to 16): with G query heads per row the vector-ALU version spent more issue
// time than the rows take to arrive, and dense decode over every row was
// bound by it.  fp32 caches keep the vector path (FacWave: four rows at a
// time, 16 lanes per row, fp64 arithmetic).
//
// The same split kernel also runs full attention over every cached row (the
// dense decode) and FAC over rows already gathered into a staging area
// (FASA-M).  In a decode step with a small budget a different launch,
// fac_select_kernel, finishes the selection itself and needs no partials.
//
// Precision: bf16 caches accumulate in fp32 (logits from v_dot2 on the raw
// bf16 pairs, scaled by scale * log2(e) and exponentiated with exp2); fp32
// caches run the logits, softmax and weighted sum in fp64 and round once at
// the end (fp32 logits of magnitude ~30 carry ~2e-6 absolute error, enough to
// move a fp32 output by more than 1e-5).
#include <math.h>

#include <atomic>

#include "fac_core.hpp"
#include "fasa_device.hpp"
#include "fasa_internal.hpp"
#include "select_core.hpp"

namespace fasa {
namespace {

struct FacArgs {
  Common c;
  FacPlan p;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  int32_t* sel_idx;       // read by the split launch; written by the selecting launch
  int32_t* sel_count;
  void* part_acc;   // [b][H_q][P][128] Acc
  void* part_ml;    // [b][H_q][P][2]   Acc (running max, running sum)
  float* out;
  uint32_t* arrive; // [b][H_kv][head_chunks] arrival counters (zeroed by the preceding launch), merge in split
  // Selecting launch only: the filter's output and the scores behind it.
  const float* scores;
  const int32_t* seq_lens;
  SelectBuffers w;
};

// Log-sum-exp merge of the P partials of query heads head0 .. head0+nh-1 by one
// 256-thread workgroup: thread t owns V consecutive output channels (V = HG/2,
// at least 1) and streams the (max, sum, acc) of all P partials -- 8 partials'
// loads in flight at a time, all independent -- folding them with a running
// maximum.
template <typename Acc, int HG>
__device__ void merge_heads(const FacArgs& a, int64_t head0, int nh) {
  constexpr int V = HG >= 2 ? HG / 2 : 1;
  const int P = a.p.n_partials;
  const int o0 = int(threadIdx.x) * V;
  const int hh = o0 / kHeadDim, ch = o0 % kHeadDim;
  if (hh >= nh) return;
  const Acc* pml = static_cast<const Acc*>(a.part_ml);
  const Acc* pacc = static_cast<const Acc*>(a.part_acc);
  const int64_t base = (head0 + hh) * P;
  Acc M = neg_inf<Acc>(), L = Acc(0), O[V];
#pragma unroll
  for (int v = 0; v < V; ++v) O[v] = Acc(0);
  for (int p0 = 0; p0 < P; p0 += 8) {
    Acc m[8], l[8], o[8][V];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t sl = base + min(p0 + u, P - 1);
      m[u] = pml[sl * 2 + 0];
      l[u] = pml[sl * 2 + 1];
#pragma unroll
      for (int v = 0; v < V; ++v) o[u][v] = pacc[sl * kHeadDim + ch + v];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const Acc mu = (p0 + u < P) ? m[u] : neg_inf<Acc>();
      const Acc mn = fmax(M, mu);
      const Acc cs = merge_weight(M, mn), cu = merge_weight(mu, mn);
      L = L * cs + l[u] * cu;
#pragma unroll
      for (int v = 0; v < V; ++v) O[v] = O[v] * cs + o[u][v] * cu;
      M = mn;
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) a.out[(head0 + hh) * kHeadDim + ch + v] = L > Acc(0) ? float(O[v] / L) : 0.f;
}

// LDS area in which the 4 waves of a workgroup fold their states.
template <typename Acc, int HG, int NWV = kFacWaves>
struct WaveFold {
  Acc acc[NWV][HG][kHeadDim];
  Acc m[NWV][HG], l[NWV][HG];
};

// Fold the 4 wave states of heads head0 .. head0+nh-1 (after fold_row_groups)
// through LDS into one partial (m, l, acc[128]) per head, stored in slot
// `split` of the head's partials.
template <typename Acc, int HG, typename W>
__device__ __forceinline__ void store_partial(const FacArgs& a, const W& w, WaveFold<Acc, HG>& f, int64_t head0,
                                              int nh, int split) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, sub = lane & 15;
  if (lane < 16) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f.acc[wave][hh][8 * sub + e] = w.acc[hh][e];
      if (sub == 0) {
        f.m[wave][hh] = w.m[hh];
        f.l[wave][hh] = w.l[hh];
      }
    }
  }
  __syncthreads();
  Acc* pacc = static_cast<Acc*>(a.part_acc);
  Acc* pml = static_cast<Acc*>(a.part_ml);
  for (int idx = threadIdx.x; idx < nh * kHeadDim; idx += 256) {
    const int hh = idx / kHeadDim, ch = idx % kHeadDim;
    Acc M = neg_inf<Acc>();
#pragma unroll
    for (int v = 0; v < kFacWaves; ++v) M = fmax(M, f.m[v][hh]);
    Acc L = Acc(0), O = Acc(0);
    if (M != neg_inf<Acc>()) {
#pragma unroll
      for (int v = 0; v < kFacWaves; ++v) {
        const Acc wgt = merge_weight(f.m[v][hh], M);
        L = fma(f.l[v][hh], wgt, L);
        O = fma(f.acc[v][hh][ch], wgt, O);
      }
    }
    const int64_t slot = (head0 + hh) * a.p.n_partials + split;
    pacc[slot * kHeadDim + ch] = O;
    if (ch == 0) {
      pml[slot * 2 + 0] = M;
      pml[slot * 2 + 1] = L;
    }
  }
}

// MERGE: the last workgroup of a (sequence, kv head, head chunk) to finish --
// counted on an arrival counter -- merges the partials of its heads, so no
// second launch is needed (used when n_split <= kFacMergeMax).
// ROWS picks where row r of a unit comes from:
//   kSelRows:    token sel_idx[unit][r] of the paged pool, r < sel_count[unit];
//   kDenseRows:  token r of the paged pool, every r < t_b (full attention; the
//                selection is not read);
//   kStagedRows: row r of the unit's contiguous staging area, rows
//                [unit * cap, unit * cap + sel_count[unit]) of k_pool / v_pool
//                (selected rows already gathered there).
enum { kSelRows = 0, kDenseRows = 1, kStagedRows = 2 };
template <typename T, typename Acc, int HG, bool MERGE, int ROWS>
__device__ __forceinline__ void fac_split_body(const FacArgs& a) {
  constexpr bool DENSE = ROWS == kDenseRows;
  const Common& c = a.c;
  const FacPlan& p = a.p;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z;
  const int g = wg.y / p.head_chunks;
  const int h0 = (wg.y % p.head_chunks) * HG;      // first head of this pass, within the group
  const int nh = min(HG, c.group - h0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;
  const int r0 = (wg.x * kFacWaves + wave) * p.rows_per_wave;
  const int32_t* sel = a.sel_idx + unit * c.cap;
  const int32_t* btab = a.block_table + int64_t(b) * c.max_blocks;

  // Three memory round trips: (count, query slices, this wave's first 64
  // selected indices) are independent; the block-table entries depend on the
  // indices; the K/V rows depend on those.  Loads are unconditional with clamped
  // indices -- validity is applied afterwards -- so nothing serialises them.
  int count = DENSE ? clamp_len(a.seq_lens[b], c.max_t, c.max_blocks) : a.sel_count[unit];
  const int cap1 = c.cap > 0 ? c.cap - 1 : 0;
  const int j_first = (ROWS == kSelRows && c.cap > 0) ? sel[min(r0 + lane, cap1)] : -1;
  // bf16 caches run the logits and the weighted sum on the matrix cores
  // (FacWaveMfma, one LDS tile per wave); fp32 caches keep the fp64 vector path.
  constexpr bool kMfma = sizeof(T) == 2;
  __shared__ __attribute__((aligned(16))) uint16_t mfma_tile[kMfma ? kFacWaves : 1][kMfma ? kMfmaTileElems : 1];
  std::conditional_t<kMfma, FacWaveMfma<HG>, FacWave<T, Acc, HG>> w;
  const T* q_head0 = static_cast<const T*>(a.q) + (int64_t(b) * c.n_q_heads + g * c.group + h0) * kHeadDim;
  if constexpr (kMfma) w.init(q_head0, nh, c.scale, mfma_tile[wave]);
  else w.init(q_head0, nh, c.scale);
  count = count < 0 ? 0 : (count > c.cap ? c.cap : count);   // contents are preconditions; stay in bounds
  const int r1 = min(r0 + p.rows_per_wave, count);
  auto lane_offset = [&](int r) -> int64_t {
    if constexpr (ROWS == kStagedRows) {
      return r < r1 ? (unit * c.cap + r) * int64_t(kHeadDim) : -1;
    } else {
      const int j = DENSE ? r : ((r - lane == r0) ? j_first : sel[min(r, cap1)]);
      const bool ok = r < r1 && j >= 0 && j < c.max_blocks * kBlock;
      const int64_t pb = btab[ok ? (j >> 8) : 0];
      return ok ? pb * c.kv_block_stride + int64_t(j & (kBlock - 1)) * kHeadDim : -1;
    }
  };
  const int64_t head_off = ROWS == kStagedRows ? 0 : int64_t(g) * c.kv_head_stride;
  const T* kbase = static_cast<const T*>(a.k_pool) + head_off;
  const T* vbase = static_cast<const T*>(a.v_pool) + head_off;
  // Row quads of loads in flight per wave: as many as the registers allow at
  // two waves per SIMD (about 64 KB in flight per CU hides HBM latency).
  constexpr int U = (sizeof(Acc) == 4 && HG <= 4) ? 8 : (HG <= 2 ? 4 : (HG <= 4 || sizeof(Acc) == 4 ? 2 : 1));
  // All heads of a chunk share this workgroup's rows, and no other workgroup
  // of the launch reads them unless the group spans several chunks.
  if constexpr (kMfma && HG >= 4) {
    // Waves with more than 128 rows resolve their row offsets up front and keep
    // the next block's loads in flight while they compute one; shorter ones
    // take the plain loop, whose one or two batches of lookups cost less than
    // the up-front pass (measured at 8 and 128 rows per wave).  Groups of 1 or
    // 2 heads keep the plain loop only: the pipelined one would make them spill.
    __shared__ int64_t row_offs[kFacWaves][FacWaveMfma<HG>::kPfRows];
    if (r1 - r0 > 128) w.template run_pipelined<true>(r0, r1, lane_offset, kbase, vbase, row_offs[wave]);
    else w.template run<true>(r0, r1, lane_offset, kbase, vbase);
  }
  else if constexpr (kMfma) w.template run<true>(r0, r1, lane_offset, kbase, vbase);
  else w.template run<U, true>(r0, r1, lane_offset, kbase, vbase);
  w.fold_row_groups();

  __shared__ WaveFold<Acc, HG> fold;
  store_partial<Acc, HG>(a, w, fold, int64_t(b) * c.n_q_heads + g * c.group + h0, nh, wg.x);
  if constexpr (MERGE) {
    // The workgroup that completes the head chunk's split merges it.
    __shared__ uint32_t s_last;
    if (!arrive_last(&a.arrive[int64_t(wg.z) * gridDim.y + wg.y], uint32_t(p.n_split), &s_last))
      return;
    merge_heads<Acc, HG>(a, int64_t(b) * c.n_q_heads + g * c.group + h0, nh);
  }
}

// fp32 caches (fp64 vector arithmetic).
template <int HG, bool MERGE, int ROWS>
__global__ __launch_bounds__(256) void fac_split_kernel(FacArgs a) {
  fac_split_body<float, double, HG, MERGE, ROWS>(a);
}

// bf16 caches (matrix-core waves), held to at least three waves per SIMD: each
// wave waits for a whole block before it computes, so the waves of a SIMD
// overlap each other's loads (three measured faster than two; forcing four
// spilled registers and measured much slower).
template <int HG, bool MERGE, int ROWS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void fac_split_mfma_kernel(FacArgs a) {
  fac_split_body<uint16_t, float, HG, MERGE, ROWS>(a);
}

constexpr int kSelThreads = 512;            // workgroup of the selecting launch
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelWideUnits = 256;          // units from which a workgroup covers several heads
constexpr int kB1Early = 0;                 // list pieces read before the lengths are known (per thread)

// The selecting launch of a decode step (budgets up to kSmallBudget).  One
// workgroup per (sequence, query head chunk): it first makes its unit's exact
// top-B selection itself, from the filter's kept pairs (select_core.hpp), into
// LDS -- redundantly across the head chunks of the unit, since a unit keeps
// only a few hundred pairs -- then runs FAC for its heads over every row of the
// list with kSelWaves waves, and writes the heads' outputs directly: no
// partials and no merge.  With one head per workgroup (few units) the G
// workgroups of a unit read the same K/V rows; the XCD-aware order puts them on
// one XCD, so after the first they mostly come from its L2.  Over TIP's lists
// with bf16 caches each head takes VS = 4 or 2 workgroups (as many as keep one
// workgroup per CU), one per part of the V channels: each computes every logit
// from all of K but loads, weighs and writes only its part of V, so a CU
// issues fewer row loads and more CUs share the rows, still with nothing to
// merge.  Workgroup 0 of each unit also publishes the list and its count and
// clears the unit's histogram for the next step.
// Grid (head chunks, or VS x heads for the bf16 lists, kv heads, batch).
template <typename Acc, int HG>
struct FacSelShared {
  union {
    struct {
      sel::SelState<kSelThreads> st;
      int32_t chunk_off[sel::CPT * kSelThreads + 1];
      uint32_t key[kSmallCand];
      int32_t idx[kSmallCand];
    } s;
    WaveFold<Acc, HG, kSelWaves> fold;
    alignas(16) uint16_t tiles[kSelWaves][kMfmaTileElems];   // bf16 FAC: one LDS tile per wave
  } u;
  int32_t chosen[kSmallBudget];
  int32_t btab[kBtabLds];
};

// HG query heads per workgroup (the x coordinate picks the head chunk): 1 when there
// are few units and latency rules, up to 8 when many units fill the chip and
// each K/V row should be read once.  DEEP (one head per workgroup and rows of
// more than 16 filter chunks, or more than 32 emitted chunks): the first kept
// pairs of up to 64 chunks are prefetched at kernel start instead of 16 (32).
// EMIT: the candidates are the lists TIP emitted per 1024-token chunk (the
// two-launch step, no filter launch); otherwise the filter's kept pairs.  B1
// (with EMIT): only the list keys in bins >= the unit histogram's bin of the
// B-th key, each thread holding a slice of one list; the unit's last
// workgroup to read the histogram clears it.
template <typename T, typename Acc, int HG, bool DEEP = false, bool EMIT = false, bool B1 = false, int VS = 1>
__global__ __launch_bounds__(kSelThreads) void fac_select_kernel(FacArgs a) {
  static_assert(!B1 || (EMIT && HG == 1), "the histogram filter reads TIP's lists, one head per workgroup");
  static_assert(VS == 1 || (EMIT && HG == 1), "V is split over one-head list workgroups");
  const Common& c = a.c;
  const WgCoord wg = xcd_grouped();
  const int b = wg.z, g = wg.y, hc = wg.x;
  // VS > 1 (TIP's lists, one head per workgroup): VS workgroups per head,
  // each over 1/VS of the V channels: x = VS head + part.
  const int vpart = VS > 1 ? hc % VS : 0;
  const int h0 = (hc / VS) * HG, nh = min(HG, c.group - h0);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t unit = int64_t(b) * c.n_kv_heads + g;
  constexpr int CHUNK = EMIT ? kEmitChunk : sel::FCH;
  const int nfa = EMIT ? emit_chunks(c) : sel::filter_chunks(c);
  const uint2* unit_slots = static_cast<const uint2*>(a.w.slots) + unit * nfa * int64_t(CHUNK);
  const float* row = a.scores + unit * c.score_stride;   // a decode step's rows: 16-byte aligned, padded
  const int lim = c.score_stride;
  __shared__ FacSelShared<Acc, HG> sm;

  // Independent loads first: the first kept pairs of every chunk (up to 16
  // chunks -- 32 emitted ones -- or 64 with DEEP; the gather fetches the rest 8
  // chunks per wave at a time), the chunk counts (summaries) and b1; the query
  // slices, the block-table row and the length.
  constexpr int PRE = (DEEP ? 64 : (EMIT ? 32 : 16)) / kSelWaves;
  uint2 pre[PRE];
  int cnt[sel::CPT];
  uint2 meta[sel::CPT];
  uint4 hv = make_uint4(0u, 0u, 0u, 0u);
  uint2 m1 = make_uint2(0u, 0u);
  sel::B1Slice<kSelThreads, kB1Early> sl;
  if constexpr (B1) {
    // The unit histogram (thread t: bins HB - 4 (t + 1) .. HB - 4 t - 1, the
    // order of the digit search) and the summary of the chunk
    // whose list slice this thread takes; the slice itself once the length is known.
    static_assert(kSelThreads * 4 == sel::HB, "one uint4 of bins per thread");
    hv = reinterpret_cast<const uint4*>(a.w.hist + unit * sel::HB)[kSelThreads - 1 - tid];
    m1 = reinterpret_cast<const uint2*>(a.w.counts)[unit * nfa + min(tid / sel::B1Slice<kSelThreads>::TPC, nfa - 1)];
    sl.early(unit_slots, nfa);
  } else {
    if constexpr (EMIT) sel::prefetch_kept<kSelThreads, PRE, 1, kEmitChunk>(unit_slots, nfa, pre);
    else sel::prefetch_kept<kSelThreads, PRE>(unit_slots, nfa, pre);
    if constexpr (EMIT) sel::load_meta(reinterpret_cast<const uint2*>(a.w.counts) + unit * nfa, nfa, meta);
    else sel::load_counts(a.w.counts + unit * nfa, nfa, cnt);
  }
  const int b1 = EMIT ? -1 : a.w.b1[unit];
  const int64_t head0 = int64_t(b) * c.n_q_heads + g * c.group + h0;
  // bf16 caches with 4 or more heads per workgroup run the FAC on the matrix
  // cores (FacWaveMfma, 16-row blocks, whose LDS tiles take the select area
  // once the select is done).  With fewer heads the vector path wins (measured:
  // the matrix tiles mostly idle, and its 32 rows per wave in one round trip
  // against two 16-row blocks); fp32 caches always take the vector path.
  constexpr bool kMfma = sizeof(T) == 2 && HG >= 4;
  // One head over TIP's lists with V split: 8 lanes per row (FacWaveOct) for
  // bf16 caches, 16 for fp32 ones.
  constexpr bool kOct = VS > 1 && sizeof(T) == 2;
  using VecWave = std::conditional_t<kOct, FacWaveOct<HG, VS>, FacWave<T, Acc, HG, VS>>;
  typename VecWave::QRaw qraw[kMfma ? 1 : HG];
  uint4 qm[kMfma ? 4 : 1];
  if constexpr (kMfma) FacWaveMfma<HG>::load_q(static_cast<const T*>(a.q) + head0 * kHeadDim, nh, qm);
  else VecWave::load_q(static_cast<const T*>(a.q) + head0 * kHeadDim, nh, qraw);
  // The sequence's block-table row (at most kBtabLds entries), held in
  // registers through the select and moved to LDS after it.
  const int32_t* btab = a.block_table + int64_t(b) * c.max_blocks;
  int32_t bt[kBtabLds / kSelThreads];
#pragma unroll
  for (int k = 0; k < kBtabLds / kSelThreads; ++k) bt[k] = btab[min(tid + kSelThreads * k, c.max_blocks - 1)];
  int t, c_lo, c_hi;
  sel::unit_range(c, a.seq_lens[b], t, c_lo, c_hi);
  const int nC = c_hi - c_lo;
  const int Bc = min(c.budget, nC);
  const int count = (t - nC) + Bc;          // forced + chosen, <= cap
  const bool keep_all = Bc == nC;

  if constexpr (B1) {
    if (!keep_all) sl.late(unit_slots, emit_chunks_of(t), m1);
  }
  if (!keep_all) {
    if constexpr (B1)
      sel::select_from_lists_b1<kSelThreads, true, kB1Early>(sm.u.s.st, sm.u.s.key, sm.u.s.idx, kSmallCand, sl, m1, hv, row, lim,
                                                   c.max_t, emit_chunks_of(t), c_lo, c_hi, Bc, sm.chosen);
    else if constexpr (EMIT)
      sel::select_from_emitted<kSelThreads, PRE, true>(sm.u.s.st, sm.u.s.chunk_off, sm.u.s.key, sm.u.s.idx,
                                                       kSmallCand, unit_slots, row, lim, c.max_t,
                                                       emit_chunks_of(t), meta, pre, c_lo, c_hi, Bc, sm.chosen);
    else
      sel::select_from_kept<kSelThreads, PRE, true>(sm.u.s.st, sm.u.s.chunk_off, sm.u.s.key, sm.u.s.idx, kSmallCand,
                                                    unit_slots, row, lim, c.max_t, nfa, cnt, pre, c_lo, c_hi, Bc, b1,
                                                    sm.chosen);
  }
#pragma unroll
  for (int k = 0; k < kBtabLds / kSelThreads; ++k)
    if (tid + kSelThreads * k < c.max_blocks) sm.btab[tid + kSelThreads * k] = bt[k];
  __syncthreads();                          // the list and the block table are in LDS; the select area is free
  if constexpr (B1) {
    // Every wave of this workgroup is done with its histogram bins (the digit
    // search has used them; a keep-all workgroup never uses them); the unit's
    // last workgroup to get here leaves the histogram zero for the next step's
    // TIP.  The counter was zeroed by TIP.
    if (wave == 0) {
      uint32_t old = 0;
      if (tid == 0) old = atomicAdd(&a.arrive[unit], 1u);
      old = uint32_t(__shfl(int(old), 0, 64));
      if (old == gridDim.x - 1) {
        uint4* hg = reinterpret_cast<uint4*>(a.w.hist + unit * sel::HB);
        for (int i = tid; i < sel::HB / 4; i += 64) hg[i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  // Row r of the list: the forced prefix, the chosen, then the forced suffix.
  std::conditional_t<kMfma, FacWaveMfma<HG>, VecWave> w;
  if constexpr (kMfma) w.init_raw(qm, nh, c.scale, sm.u.tiles[wave]);
  else w.init_raw(qraw, nh, c.scale, vpart);
  auto token = [&](int r) -> int {
    const int ch = sm.chosen[min(max(r - c_lo, 0), kSmallBudget - 1)];
    return (keep_all || r < c_lo) ? r : (r < c_lo + Bc ? ch : c_hi + (r - c_lo - Bc));
  };
  const int rpw = ((count + kSelWaves - 1) / kSelWaves + 3) & ~3;
  const int r0 = wave * rpw;
  const int r1 = min(r0 + rpw, count);
  auto lane_offset = [&](int r) -> int64_t {
    const int j = token(r);
    const bool ok = r < r1 && j >= 0 && j < c.max_blocks * kBlock;
    const int64_t pb = sm.btab[ok ? (j >> 8) : 0];
    return ok ? pb * c.kv_block_stride + int64_t(j & (kBlock - 1)) * kHeadDim : -1;
  };
  const T* kbase = static_cast<const T*>(a.k_pool) + int64_t(g) * c.kv_head_stride;
  const T* vbase = static_cast<const T*>(a.v_pool) + int64_t(g) * c.kv_head_stride;
  // Row quads in flight per wave: 8 (a whole 32-row share of a 256-row list in
  // one round trip) for one head; fewer as the per-head state grows.
  constexpr int U = kOct ? 4 : (HG == 1 ? 8 : (HG <= 4 && sizeof(Acc) == 4 ? 4 : 2));
  if constexpr (kMfma) {
    w.template run<false>(r0, r1, lane_offset, kbase, vbase);
    w.fold_row_groups();
    __syncthreads();                        // the fold area below overlaps the other waves' tiles
  } else {
    w.template run<U, false, B1 || kOct>(r0, r1, lane_offset, kbase, vbase);
    w.fold_row_groups();
  }

  // Fold the waves through LDS and write the heads' outputs.
  WaveFold<Acc, HG, kSelWaves>& f = sm.u.fold;
  constexpr int kLpr = kMfma ? 16 : VecWave::kLanesPerRow, kCh = kMfma ? kHeadDim / 16 : VecWave::kCh;
  const int lane = tid & 63, sub = lane & (kLpr - 1);
  if (lane < kLpr) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
      for (int e = 0; e < kCh; ++e) f.acc[wave][hh][w.chan(sub, e)] = w.acc[hh][e];
      if (sub == 0) {
        f.m[wave][hh] = w.m[hh];
        f.l[wave][hh] = w.l[hh];
      }
    }
  }
  __syncthreads();
  constexpr int kOutCh = kHeadDim / VS;    // this workgroup's output channels
  for (int idx = tid; idx < nh * kOutCh; idx += kSelThreads) {
    const int hh = idx / kOutCh, ch = kOutCh * vpart + idx % kOutCh;
    Acc M = neg_inf<Acc>();
#pragma unroll
    for (int v = 0; v < kSelWaves; ++v) M = fmax(M, f.m[v][hh]);
    Acc L = Acc(0), O = Acc(0);
    if (M != neg_inf<Acc>()) {
#pragma unroll
      for (int v = 0; v < kSelWaves; ++v) {
        const Acc wgt = merge_weight(f.m[v][hh], M);
        L = fma(f.l[v][hh], wgt, L);
        O = fma(f.acc[v][hh][ch], wgt, O);
      }
    }
    a.out[(head0 + hh) * kHeadDim + ch] = L > Acc(0) ? float(O / L) : 0.f;
  }
  if (hc == 0) {
    // Workgroup 0 of the unit publishes the list and (after a filter launch)
    // leaves the consumed histogram zero for the next step.
    int32_t* list = a.sel_idx + unit * c.cap;
    for (int i = tid; i < c.cap; i += kSelThreads) list[i] = i < count ? token(i) : -1;
    if (tid == 0) a.sel_count[unit] = count;
    if constexpr (!EMIT) {
      uint4* hg = reinterpret_cast<uint4*>(a.w.hist + unit * sel::HB);
      for (int i = tid; i < sel::HB / 4; i += kSelThreads) hg[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// One workgroup per (sequence, query head): log-sum-exp merge of the partials.
// Up to 8 partials: one round trip, merged in registers.  More: the weights
// e^(m_i - M) and l_i e^(m_i - M) go through LDS; each thread then streams its
// channel of every partial with 8 loads in flight.
template <typename Acc>
__global__ __launch_bounds__(kHeadDim) void fac_merge_kernel(FacArgs a) {
  constexpr int MAXP = 512;
  __shared__ Acc s_w[MAXP], s_lw[MAXP];
  __shared__ Acc s_red[2];
  const WgCoord wg = xcd_grouped();
  const int h = wg.x, b = wg.y, d = threadIdx.x;
  const int P = a.p.n_partials;
  const int64_t base = (int64_t(b) * a.c.n_q_heads + h) * P;
  const Acc* pacc = static_cast<const Acc*>(a.part_acc) + base * kHeadDim + d;
  const Acc* pml = static_cast<const Acc*>(a.part_ml) + base * 2;
  if (P >= 1 && P <= 8) {
    // Few partials: every (m, l) and this channel of every accumulator in one
    // round trip (indices clamped; the extra slots are masked), merged in
    // registers in partial order.
    Acc m[8], l[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = min(i, P - 1);
      m[i] = pml[2 * k];
      l[i] = pml[2 * k + 1];
      o[i] = pacc[int64_t(k) * kHeadDim];
    }
    Acc M = neg_inf<Acc>();
#pragma unroll
    for (int i = 0; i < 8; ++i) M = i < P ? fmax(M, m[i]) : M;
    float res = 0.f;
    if (M != neg_inf<Acc>()) {
      Acc L = Acc(0), O = Acc(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const Acc w = (i >= P || m[i] == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(m[i] - M);
        O = fma(o[i], w, O);
        L += l[i] * w;
      }
      res = float(O / L);
    }
    a.out[(int64_t(b) * a.c.n_q_heads + h) * kHeadDim + d] = res;
    return;
  }
  Acc M = neg_inf<Acc>();
  for (int i = d; i < P; i += kHeadDim) M = fmax(M, pml[2 * i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmax(M, shfl_xor_acc(M, o));
  if ((d & 63) == 0) s_red[d >> 6] = M;
  __syncthreads();
  M = fmax(s_red[0], s_red[1]);
  float res = 0.f;
  if (M != neg_inf<Acc>()) {
    Acc L = Acc(0), O = Acc(0);
    for (int p0 = 0; p0 < P; p0 += MAXP) {
      const int n = min(MAXP, P - p0);
      __syncthreads();
      for (int i = d; i < n; i += kHeadDim) {
        const Acc mi = pml[2 * (p0 + i)];
        const Acc w = (mi == neg_inf<Acc>()) ? Acc(0) : fexp<Acc>(mi - M);
        s_w[i] = w;
        s_lw[i] = pml[2 * (p0 + i) + 1] * w;
      }
      __syncthreads();
      int i = 0;
      for (; i + 8 <= n; i += 8) {
        Acc v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pacc[int64_t(p0 + i + u) * kHeadDim];
#pragma unroll
        for (int u = 0; u < 8; ++u) O = fma(v[u], s_w[i + u], O);
      }
      for (; i < n; ++i) O = fma(pacc[int64_t(p0 + i) * kHeadDim], s_w[i], O);
      for (int k = 0; k < n; ++k) L += s_lw[k];
    }
    res = float(O / L);
  }
  a.out[(int64_t(b) * a.c.n_q_heads + h) * kHeadDim + d] = res;
}

template <int HG, bool MERGE, int ROWS>
void launch_split_hg(bool bf16, const FacArgs& a, const dim3& grid, hipStream_t s) {
  if (bf16) hipLaunchKernelGGL((fac_split_mfma_kernel<HG, MERGE, ROWS>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((fac_split_kernel<HG, MERGE, ROWS>), grid, dim3(256), 0, s, a);
}

template <typename T, typename Acc, bool MERGE, int ROWS = kSelRows>
void launch_split(const FacArgs& a, const dim3& grid, hipStream_t s) {
  constexpr bool bf16 = sizeof(T) == 2;
  switch (a.p.heads_per_pass) {
    case 1: launch_split_hg<1, MERGE, ROWS>(bf16, a, grid, s); break;
    case 2: launch_split_hg<2, MERGE, ROWS>(bf16, a, grid, s); break;
    case 4: launch_split_hg<4, MERGE, ROWS>(bf16, a, grid, s); break;
    default: launch_split_hg<8, MERGE, ROWS>(bf16, a, grid, s); break;
  }
}

// Full attention: the split launch over every cached row, then the merge launch.
template <typename T, typename Acc>
hipError_t launch_dense_t(const FacArgs& a, hipStream_t s) {
  const FacPlan& p = a.p;
  const dim3 grid(p.n_split, a.c.n_kv_heads * p.head_chunks, a.c.batch);
  launch_split<T, Acc, false, kDenseRows>(a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fac_merge_kernel<Acc>, dim3(a.c.n_q_heads, a.c.batch), dim3(kHeadDim), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename Acc, int ROWS = kSelRows>
hipError_t launch_fac_t(FacArgs& a, hipStream_t s) {
  const FacPlan& p = a.p;
  const dim3 grid(p.n_split, a.c.n_kv_heads * p.head_chunks, a.c.batch);
  const int64_t n_wg = int64_t(grid.x) * grid.y * grid.z;
  if (a.arrive != nullptr && p.n_split <= kFacMergeMax && n_wg <= kFacMergeGrid) {
    launch_split<T, Acc, true, ROWS>(a, grid, s);
    return hipGetLastError();
  }
  launch_split<T, Acc, false, ROWS>(a, grid, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fac_merge_kernel<Acc>, dim3(a.c.n_q_heads, a.c.batch), dim3(kHeadDim), 0, s, a);
  return hipGetLastError();
}

// Heads per workgroup of the selecting launch: one while the (sequence, kv
// head) units are fewer than the CUs; otherwise the whole group, up to 8.
// (fp64 state for fp32 caches: at most 2 heads, which keeps the registers.)
int select_heads(const Common& c) {
  if (int64_t(c.batch) * c.n_kv_heads < kSelWideUnits) return 1;
  const int most = c.bf16 ? 8 : 2;
  int hg = 1;
  while (hg < c.group && hg < most) hg <<= 1;
  return hg;
}

// Compute units of the current device, asked once per device (256, the whole
// chip, if the query fails).
int64_t device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, typename Acc>
hipError_t launch_fac_select_t(const FacArgs& a, int lists, hipStream_t s) {
  const int hg = select_heads(a.c);
  const dim3 grid((a.c.group + hg - 1) / hg, a.c.n_kv_heads, a.c.batch);
  const bool emitted = lists != kFromFilter;
  // One-head workgroups over TIP's lists with bf16 caches split V over VS
  // workgroups per head, as many as keep one workgroup per CU (measured at the
  // 8B layer: halves 17.54 -> 17.41 us, quarters 16.8 us, eighths no better;
  // the Qwen shape's 224 half workgroups 34.1 -> 33.0 us, 448 quarters 36.3 us).
  const int64_t heads = int64_t(a.c.batch) * a.c.n_kv_heads * a.c.group;
  const int64_t cus = hg == 1 && emitted ? device_cus() : 0;
  const int vs = cus == 0 ? 1 : (heads * 4 <= cus ? 4 : (heads * 2 <= cus ? 2 : 1));
  const dim3 gv(grid.x * vs, grid.y, grid.z);
  if (lists == kFromListsB1) {
    if (vs == 4) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true, true, 4>), gv, dim3(kSelThreads), 0, s, a);
    else if (vs == 2) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true, true, 2>), gv, dim3(kSelThreads), 0, s, a);
    else hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true, true>), gv, dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
  }
  // One head per workgroup has the registers for a deeper prefetch; it pays only
  // when the rows span more than 16 filter chunks (measured: 128K-token rows
  // gain 0.7 us, 32K-token rows lose 0.4 us to the redundant loads), or more
  // than 32 emitted chunks.  TIP's lists are only used with one head per
  // workgroup (decode_lists).
  if (emitted) {
    const bool deep = emit_chunks(a.c) > 32;
    if (vs == 4) {
      if (deep) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, true, true, false, 4>), gv, dim3(kSelThreads), 0, s, a);
      else hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true, false, 4>), gv, dim3(kSelThreads), 0, s, a);
      return hipGetLastError();
    }
    if (vs == 2) {
      if (deep) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, true, true, false, 2>), gv, dim3(kSelThreads), 0, s, a);
      else hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true, false, 2>), gv, dim3(kSelThreads), 0, s, a);
      return hipGetLastError();
    }
    if (deep) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, true, true>), gv, dim3(kSelThreads), 0, s, a);
    else hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, false, true>), gv, dim3(kSelThreads), 0, s, a);
    return hipGetLastError();
  }
  const bool deep = sel::filter_chunks(a.c) > 16;
  if (hg == 1 && deep) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1, true>), grid, dim3(kSelThreads), 0, s, a);
  else if (hg == 1) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 1>), grid, dim3(kSelThreads), 0, s, a);
  else if (hg == 2) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 2>), grid, dim3(kSelThreads), 0, s, a);
  else if constexpr (sizeof(Acc) == 4) {
    if (hg == 4) hipLaunchKernelGGL((fac_select_kernel<T, Acc, 4>), grid, dim3(kSelThreads), 0, s, a);
    else hipLaunchKernelGGL((fac_select_kernel<T, Acc, 8>), grid, dim3(kSelThreads), 0, s, a);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

FacArgs make_args(const Common& c, const FacPlan& p, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_table, int32_t* sel_idx, int32_t* sel_count, float* out, void* ws,
                  uint32_t* arrive) {
  const size_t acc_sz = c.bf16 ? sizeof(float) : sizeof(double);
  const size_t slots = size_t(c.batch) * c.n_q_heads * p.n_partials;
  char* w = static_cast<char*>(ws);
  FacArgs a{c, p, q, k_pool, v_pool, block_table, sel_idx, sel_count,
            w, w + align256(slots * kHeadDim * acc_sz), out, arrive, nullptr, nullptr, {}};
  return a;
}

}  // namespace

bool fac_selects(const Common& c, const FacPlan& p) {
  (void)p;
  return c.max_t > 0 && c.budget <= kSmallBudget && c.max_blocks <= kBtabLds && (c.score_stride & 3) == 0;
}

int decode_lists(const Common& c, const FacPlan& p) {
  // Few units (one-head selecting workgroups): there the filter launch and its
  // launch gap are a large part of the step.  Many units keep the filter
  // launch, whose cost they share, and whose global threshold does not depend
  // on how the top keys cluster along the row (measured: the ragged batch of
  // 64 sequences x 8 kv heads on TIP's lists, four heads per workgroup, took
  // 350 us against 292 us).
  if (c.max_t <= 0 || !fac_selects(c, p) || select_heads(c) != 1 || emit_chunks(c) > 64 * sel::CPT)
    return kFromFilter;
  // Every chunk writes emit_target() keys (more only with ties): at the longest
  // row about 2 Bc + 18 per chunk; a quarter more for ties and short rows.
  // Lists expected to overflow the selecting launch's LDS are cut down to the
  // filter's kept set with the unit histogram, when a list's target leaves
  // room for ties within what the gather reads of a list (a longer list sends
  // its unit to the scores row: measured 20 -> 32 us at a 4096-token row whose
  // chunks target 144 keys each).
  const int64_t bc = c.budget < c.max_t ? c.budget : c.max_t;
  const int64_t expect = 5 * (2 * bc + 18 * int64_t(emit_chunks(c))) / 4;
  if (expect <= kSmallCand) return kFromLists;
  if (emit_chunks(c) <= sel::B1_LISTS && 2 * emit_target(int(bc), c.max_t) <= sel::B1_LIST) return kFromListsB1;
  return kFromFilter;
}

FacPlan fac_plan(const Common& c) {
  FacPlan p;
  const int g8 = c.group < 8 ? c.group : 8;
  int hg = 1;
  while (hg < g8) hg <<= 1;
  p.heads_per_pass = hg;
  p.head_chunks = (c.group + hg - 1) / hg;
  const int64_t units = int64_t(c.batch) * c.n_kv_heads * p.head_chunks;
  const int64_t rows = units * int64_t(c.cap);
  // Aim at about 2048 waves (512 workgroups, two per CU): with the matrix-core
  // waves, fewer and longer runs measured faster than 4096 waves of at most 128
  // rows (batch 16, B = 6193: 86 -> 81 us).
  int64_t rpw = (rows + 2047) / 2048;
  if (rpw < 2 * g8) rpw = 2 * g8;                 // keep partial traffic below ~1/2 of row traffic
  rpw = (rpw + 3) & ~int64_t(3);
  if (rpw < 4) rpw = 4;
  if (rpw > 512) rpw = 512;
  p.rows_per_wave = int(rpw);
  const int per_wg = kFacWaves * p.rows_per_wave;
  p.n_split = c.cap > 0 ? (c.cap + per_wg - 1) / per_wg : 1;
  p.n_partials = p.n_split;
  return p;
}

FacPlan dense_plan(const Common& c) {
  // Every cached row is read: aim at about 512 workgroups (two per CU, all
  // resident at once) for short contexts, and give each wave up to 256 rows as
  // the context grows (fewer partials).  Longer runs per wave measured slower
  // on ragged batches, whose short sequences leave many workgroups idle.
  FacPlan p = fac_plan(c);
  const int64_t rows = int64_t(c.batch) * c.n_kv_heads * p.head_chunks * int64_t(c.cap);
  int64_t rpw = (rows + 512 * kFacWaves - 1) / (512 * kFacWaves);
  rpw = (rpw + 3) & ~int64_t(3);
  if (rpw < 32) rpw = 32;
  if (rpw > 256) rpw = 256;
  p.rows_per_wave = int(rpw);
  const int per_wg = kFacWaves * p.rows_per_wave;
  p.n_split = c.cap > 0 ? (c.cap + per_wg - 1) / per_wg : 1;
  p.n_partials = p.n_split;
  return p;
}

size_t fac_workspace_bytes(const Common& c, const FacPlan& p) {
  const size_t acc_sz = c.bf16 ? sizeof(float) : sizeof(double);
  const size_t slots = size_t(c.batch) * c.n_q_heads * p.n_partials;
  return align256(slots * kHeadDim * acc_sz) + align256(slots * 2 * acc_sz);
}

size_t scores_bytes(const Common& c) {
  // Rows padded to a multiple of 4 (a decode step's stride).
  return align256(size_t(c.batch) * c.n_kv_heads * size_t((c.max_t + 3) & ~3) * sizeof(float));
}

hipError_t launch_fac(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, const int32_t* sel_idx,
                      const int32_t* sel_count, float* out, void* ws, uint32_t* arrive, hipStream_t s) {
  FacArgs a = make_args(c, p, q, k_pool, v_pool, block_table, const_cast<int32_t*>(sel_idx),
                        const_cast<int32_t*>(sel_count), out, ws, arrive);
  if (c.bf16) return launch_fac_t<uint16_t, float>(a, s);
  return launch_fac_t<float, double>(a, s);
}

hipError_t launch_fac_staged(const Common& c, const FacPlan& p, const void* q, const void* stage_k,
                             const void* stage_v, const int32_t* sel_count, float* out, void* ws, uint32_t* arrive,
                             hipStream_t s) {
  FacArgs a = make_args(c, p, q, stage_k, stage_v, nullptr, nullptr, const_cast<int32_t*>(sel_count), out, ws,
                        arrive);
  if (c.bf16) return launch_fac_t<uint16_t, float, kStagedRows>(a, s);
  return launch_fac_t<float, double, kStagedRows>(a, s);
}

hipError_t launch_dense(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seq_lens, float* out,
                        void* ws, hipStream_t s) {
  FacArgs a = make_args(c, p, q, k_pool, v_pool, block_table, nullptr, nullptr, out, ws, nullptr);
  a.seq_lens = seq_lens;
  if (c.bf16) return launch_dense_t<uint16_t, float>(a, s);
  return launch_dense_t<float, double>(a, s);
}

hipError_t launch_fac_select(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table, const float* scores,
                             const int32_t* seq_lens, const SelectBuffers& sb, int lists, uint32_t* arrive,
                             int32_t* sel_idx, int32_t* sel_count, float* out, hipStream_t s) {
  FacArgs a = make_args(c, p, q, k_pool, v_pool, block_table, sel_idx, sel_count, out, nullptr, arrive);
  a.scores = scores;
  a.seq_lens = seq_lens;
  a.w = sb;
  if (c.bf16) return launch_fac_select_t<uint16_t, float>(a, lists, s);
  return launch_fac_select_t<float, double>(a, lists, s);
}

}  // namespace fasa
