// Internal interface between the C-ABI layer (fasa_api.cpp) and the kernel
// translation units.  Every launcher enqueues on the given stream and returns
// the launch status; the API layer has validated all arguments before.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fasa {

constexpr int kHeadDim = 128;
constexpr int kBlock = 256;            // tokens per cache block
constexpr int kSlabFcStride = 512;     // elements between FCs inside a slab block (256 tokens x 2)

// Top-B: a filter workgroup per 2048 tokens keeps the keys at or above the
// coarse-histogram bin of the B-th largest (one bin per value of key bits
// 31..21); then one workgroup per unit selects exactly among the kept keys in
// LDS: a 1024-thread finish workgroup (up to kCandLds keys), or, in a decode
// step with a budget up to kSmallBudget, each FAC workgroup itself (up to
// kSmallCand keys).
constexpr int kTopkThreads = 1024;
constexpr int kHistBins = 2048;
constexpr int kHistShift = 21;
constexpr int kCandLds = 12288;
constexpr int kFilterChunk = 2048;
constexpr int kSmallBudget = 1024;
constexpr int kSmallCand = 4096;

// Candidate emission by TIP (the two-launch step): every 1024-token chunk (one
// TIP workgroup) writes its candidate keys at or above tau, the lower edge of
// the coarse bin that holds its k-th largest key, k = emit_target(), as (key,
// token) pairs in index order, and a summary (count | (some candidate left
// out) << 31, tau).
constexpr int kEmitChunk = 1024;
__host__ __device__ __forceinline__ int emit_chunks_of(int max_t) {
  const int n = (max_t + kEmitChunk - 1) / kEmitChunk;
  return n > 0 ? n : 1;
}
// Per-chunk target for a unit choosing Bc of nC candidates: twice the chunk's
// expected share of the top-Bc plus 16, at most a chunk.  The lists fail to
// cover the top-Bc only if some chunk holds at least this many keys above the
// Bc-th largest; the select then falls back to the whole scores row.
__host__ __device__ __forceinline__ int emit_target(int Bc, int nC) {
  if (nC <= 0) return kEmitChunk;
  const int64_t share = (int64_t(Bc) * kEmitChunk + nC - 1) / nC;
  const int64_t k = 2 * share + 16;
  return int(k < kEmitChunk ? k : kEmitChunk);
}
__host__ __device__ __forceinline__ uint32_t emit_word(uint32_t count, bool cut) {
  return count | (cut ? 0x80000000u : 0u);
}
__host__ __device__ __forceinline__ uint32_t emit_count(uint32_t w) { return w & 0xffffu; }
__host__ __device__ __forceinline__ bool emit_cut(uint32_t w) { return (w & 0x80000000u) != 0u; }

// FAC: 4 waves per workgroup; the waves' states are folded in LDS into one
// partial.  Up to kFacMergeMax partials per head are merged by the last
// workgroup of the split launch, when the launch has at most kFacMergeGrid
// workgroups; otherwise a separate merge launch runs.  (Each workgroup's
// device-scope release writes back its XCD's L2; a few of those cost less
// than a launch, thousands cost far more.)
constexpr int kFacWaves = 4;
constexpr int kFacMergeMax = 64;
constexpr int kFacMergeGrid = 128;
// The selecting FAC launch keeps the sequence's block-table row in LDS (up to
// kBtabLds blocks, 512K tokens).
constexpr int kBtabLds = 2048;

struct Common {
  int batch, n_q_heads, n_kv_heads, group, n_fc, budget, n_sink, n_recent;
  int max_blocks, max_t, cap;
  int score_stride;   // elements per row of the scores array (>= max_t; a multiple of 4 in a decode step)
  int64_t kv_block_stride, kv_head_stride, slab_block_stride, slab_head_stride;
  int bf16;     // 1: bf16 storage, 0: fp32 storage
  float scale;
};

__host__ __device__ __forceinline__ int emit_chunks(const Common& c) { return emit_chunks_of(c.max_t); }

// FAC work split, derived on the host from the shape (workspace size depends on it).
struct FacPlan {
  int rows_per_wave;   // multiple of 4
  int n_split;         // workgroups per (sequence, kv head, head chunk)
  int n_partials;      // one partial (m, l, acc[128]) per workgroup: n_split
  int heads_per_pass;  // 1, 2, 4 or 8 (>= min(group, 8)), a power of two
  int head_chunks;     // ceil(group / heads_per_pass)
};

FacPlan fac_plan(const Common& c);
FacPlan dense_plan(const Common& c);   // full attention: c.cap == max_t
size_t fac_workspace_bytes(const Common& c, const FacPlan& p);
size_t scores_bytes(const Common& c);

hipError_t launch_slab_build(const Common& c, const void* k_pool, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* fc_idx, void* slab,
                             hipStream_t s);
hipError_t launch_slab_append(const Common& c, const void* k_pool, const int32_t* block_table,
                              const int32_t* positions, const int32_t* fc_idx, void* slab,
                              hipStream_t s);
size_t hist_bytes(const Common& c);
size_t slots_bytes(const Common& c);    // kept (key, token) pairs: 8 bytes per token of max_t
size_t counts_bytes(const Common& c);

// Select state inside the workspace: unit histograms (zero between calls),
// per-chunk kept pairs and their counts, and the coarse bin b1 of every unit.
struct SelectBuffers {
  uint32_t* hist;
  void* slots;
  int32_t* counts;
  int32_t* b1;
};

// TIP epilogues: scores only; + the unit's coarse histogram (global atomics,
// for the filter launch); + this chunk's candidate list for the select that
// the FAC launch finishes (no filter launch); + both the list and the unit
// histogram (the FAC launch keeps only the list keys in bins >= the
// histogram's bin of the B-th largest key).
enum { kTipScores = 0, kTipHist = 1, kTipEmit = 2, kTipEmitHist = 3 };
struct TipOutputs {
  int mode;
  uint32_t* hist;   // kTipHist, kTipEmitHist: [units][kHistBins], holding the counts of nothing else
  uint2* slots;     // kTipEmit, kTipEmitHist: [units][emit_chunks][kEmitChunk] (key, token) pairs
  uint2* meta;      // kTipEmit, kTipEmitHist: [units][emit_chunks] (emit_word, tau)
  uint32_t* arrive = nullptr;   // kTipEmitHist: [units] counters, zeroed (by chunk 0's workgroup)
};
hipError_t launch_tip(const Common& c, const void* q, const void* slab, const void* k_pool,
                      const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* fc_idx, float* scores, const TipOutputs& o, hipStream_t s);
// Top-B stages 1-2: the unit histograms (unless have_hist: TIP filled them) and
// the filter's kept pairs, counts and b1.  Nothing when max_t == 0.
// fac_arrive (nullable): FAC arrival counters, [units][head_chunks], zeroed here
// for the FAC launch that follows.  rows_full: the caller expects every row to
// run to max_t (a speed hint; any lengths stay correct).
hipError_t launch_filter(const Common& c, const float* scores, const int32_t* seq_lens, const SelectBuffers& w,
                         bool have_hist, uint32_t* fac_arrive, int head_chunks, hipStream_t s,
                         bool rows_full = false);
// Top-B stage 3 as its own launch: the selection lists and counts; zeroes the
// histograms (and fac_arrive when given).
hipError_t launch_finish(const Common& c, const float* scores, const int32_t* seq_lens, int32_t* sel_idx,
                         int32_t* sel_count, const SelectBuffers& w, uint32_t* fac_arrive, int head_chunks,
                         hipStream_t s);
// FAC over given selections.  arrive (nullable): zeroed FAC arrival counters;
// the merge then runs in the split launch when the plan allows it.
hipError_t launch_fac(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, const int32_t* sel_idx,
                      const int32_t* sel_count, float* out, void* ws, uint32_t* arrive, hipStream_t s);
// Full attention over rows 0 .. t_b-1 of every sequence (no selection): the
// split launch with row r = token r, then the merge launch.  c.cap must be
// max_t and p = dense_plan(c); ws holds the partials (fac_workspace_bytes).
hipError_t launch_dense(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                        const void* v_pool, const int32_t* block_table, const int32_t* seq_lens, float* out,
                        void* ws, hipStream_t s);
// FAC over rows staged contiguously per unit: row r of unit u at
// stage_k / stage_v + (u * c.cap + r) * 128, for r < sel_count[u].
hipError_t launch_fac_staged(const Common& c, const FacPlan& p, const void* q, const void* stage_k,
                             const void* stage_v, const int32_t* sel_count, float* out, void* ws, uint32_t* arrive,
                             hipStream_t s);

// FASA-M (fasam.hip): host-resident non-dominant key columns and values.
// Elements per row of the host non-dominant key array (128 - 2F, padded to 16 bytes).
int m_nd_stride(const Common& c);
// Copy tokens' blocks [0, ceil(t_b / 256)) of the device pools into the host arrays.
hipError_t launch_m_offload(const Common& c, const void* k_pool, const void* v_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* fc_idx, void* k_nd, void* v_host,
                            hipStream_t s);
// Reuse of the previous step's rows by the gather: its selection (ascending,
// [b][H_kv][cap]) and its rows in the prefetch area ([b][H_kv][cap][128], K and
// V); hits (nullable) counts per unit the rows taken from there.  prev_idx ==
// nullptr: no reuse.
struct MReuse {
  const int32_t* prev_idx = nullptr;
  const int32_t* prev_count = nullptr;
  const void* pf_k = nullptr;
  const void* pf_v = nullptr;
  int32_t* hits = nullptr;
};
// Whether the gather can search the previous selection on chip (cap <= 8192);
// otherwise every row comes from the host.
bool m_reuses(const Common& c);
// Rebuild the selected rows (non-dominant columns and values from the host,
// dominant pairs from the slab; with reuse, the rows the previous step selected
// from the prefetch area) into the staging arrays [b][H_kv][cap][128].
hipError_t launch_m_gather(const Common& c, const void* k_nd, const void* v_host, const void* slab,
                           const int32_t* block_table, const int32_t* fc_idx, const int32_t* sel_idx,
                           const int32_t* sel_count, void* stage_k, void* stage_v, const MReuse& reuse,
                           hipStream_t s);

// Offline calibration (calib.hip).  kCaMaxK: largest calibration window K.
constexpr int kCaMaxK = 4096;
// The 65 score rows (alpha, alpha^(0..63)) of every unit into scores
// [b][H_kv][65][c.score_stride].
hipError_t launch_ca_scores(const Common& c, const void* q, const void* k_pool, const int32_t* block_table,
                            const int32_t* seq_lens, float* scores, hipStream_t s);
// hits[b][g][i] from the top-K lists of the 65 rows of each unit; c is the
// selection's Common (cap = the lists' row length; c.n_kv_heads = H_kv).
hipError_t launch_ca_hits(const Common& c, const int32_t* sel_idx, const int32_t* sel_count, int32_t* hits,
                          int32_t* topk, hipStream_t s);
hipError_t launch_ca_dominant(const int32_t* hits, int n_rows, int n_kv, int n_tip, int32_t* fc_idx, hipStream_t s);

// Whether a decode step may use launch_fac_select (small budget, block-table
// rows that fit in LDS).
bool fac_selects(const Common& c, const FacPlan& p);
// Top-B stage 3 and FAC in one launch: writes the selection lists and counts,
// leaves the unit histograms zero, and computes out (one workgroup per query
// head, no merge).  lists: where the candidates come from --
//   kFromFilter: the filter's kept pairs (after launch_filter);
//   kFromLists:  TIP's per-chunk lists (TIP ran with kTipEmit; sb.slots /
//                sb.counts hold its pairs and summaries);
//   kFromListsB1: the same lists, keeping the keys in bins >= the unit
//                histogram's bin of the B-th largest key (TIP ran with
//                kTipEmitHist; arrive holds its per-unit counters).
enum { kFromFilter = 0, kFromLists = 1, kFromListsB1 = 2 };
hipError_t launch_fac_select(const Common& c, const FacPlan& p, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table, const float* scores,
                             const int32_t* seq_lens, const SelectBuffers& sb, int lists, uint32_t* arrive,
                             int32_t* sel_idx, int32_t* sel_count, float* out, hipStream_t s);
// Where a decode step's candidates come from (kFrom*): TIP's lists (two
// launches) when fac_selects() and few units; with the unit histogram's filter
// when the plain lists are not expected to fit the selecting launch's LDS; the
// filter launch otherwise.
int decode_lists(const Common& c, const FacPlan& p);

}  // namespace fasa
