// C ABI of libfasa.so (declared in include/fasa.h): host-side validation, then
// kernel launches on the caller's stream.  Nothing here allocates, synchronises
// or keeps state between calls.
#include <stdint.h>
#include <string.h>

#include <limits>

#include "fasa.h"
#include "fasa_internal.hpp"

using fasa::Common;
using fasa::FacPlan;

namespace {

constexpr int64_t kMaxGrid = 65535;   // limit of gridDim.y / gridDim.z

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

fasa_status check_shape(const fasa_shape* s) {
  if (!s) return FASA_ERR_INVALID_ARG;
  if (s->kv_dtype != FASA_F32 && s->kv_dtype != FASA_BF16) return FASA_ERR_INVALID_ARG;
  if (s->batch < 1 || s->batch > kMaxGrid) return FASA_ERR_INVALID_ARG;
  if (s->n_kv_heads < 1 || s->n_q_heads < 1) return FASA_ERR_INVALID_ARG;
  if (s->n_q_heads % s->n_kv_heads != 0) return FASA_ERR_INVALID_ARG;
  if (s->head_dim < 2 || (s->head_dim & 1)) return FASA_ERR_INVALID_ARG;
  if (s->head_dim != fasa::kHeadDim) return FASA_ERR_UNSUPPORTED;
  if (s->block_size != fasa::kBlock) return FASA_ERR_UNSUPPORTED;
  const int group = s->n_q_heads / s->n_kv_heads;
  if (group > 16) return FASA_ERR_UNSUPPORTED;
  if (int64_t(s->n_kv_heads) * ((group + 7) / 8) > kMaxGrid) return FASA_ERR_UNSUPPORTED;
  if (s->n_q_heads > kMaxGrid) return FASA_ERR_UNSUPPORTED;
  if (s->n_fc < 1 || s->n_fc > s->head_dim / 2) return FASA_ERR_INVALID_ARG;
  if (s->budget < 1) return FASA_ERR_INVALID_ARG;
  if (s->n_sink < 0 || s->n_recent < 0) return FASA_ERR_INVALID_ARG;
  if (s->max_blocks_per_seq < 1 || s->max_blocks_per_seq > (std::numeric_limits<int32_t>::max() / 256))
    return FASA_ERR_INVALID_ARG;
  const int64_t row = int64_t(fasa::kBlock) * s->head_dim;
  if (s->kv_head_stride < row || (s->kv_head_stride & 7)) return FASA_ERR_INVALID_ARG;
  if (s->kv_block_stride < row || (s->kv_block_stride & 7)) return FASA_ERR_INVALID_ARG;
  if (s->slab_head_stride < int64_t(fasa::kSlabFcStride) * s->n_fc || (s->slab_head_stride & 7))
    return FASA_ERR_INVALID_ARG;
  if (s->slab_block_stride < int64_t(fasa::kSlabFcStride) * s->n_fc || (s->slab_block_stride & 7))
    return FASA_ERR_INVALID_ARG;
  if (!(s->scale >= 0.f) || s->scale == std::numeric_limits<float>::infinity()) return FASA_ERR_INVALID_ARG;
  return FASA_OK;
}

fasa_status check_max_t(const fasa_shape* s, int32_t max_t) {
  if (max_t < 0) return FASA_ERR_INVALID_ARG;
  // The last block of a sequence is read whole; scores rows must fit an int.
  if (int64_t(max_t) > int64_t(s->max_blocks_per_seq) * fasa::kBlock) return FASA_ERR_INVALID_ARG;
  return FASA_OK;
}

int32_t capacity(const fasa_shape* s, int32_t max_t) {
  const int64_t want = int64_t(s->budget) + s->n_sink + s->n_recent;
  return int32_t(want < max_t ? want : max_t);
}

Common make_common(const fasa_shape* s, int32_t max_t) {
  Common c;
  c.batch = s->batch;
  c.n_q_heads = s->n_q_heads;
  c.n_kv_heads = s->n_kv_heads;
  c.group = s->n_q_heads / s->n_kv_heads;
  c.n_fc = s->n_fc;
  c.budget = s->budget;
  c.n_sink = s->n_sink;
  c.n_recent = s->n_recent;
  c.max_blocks = s->max_blocks_per_seq;
  c.max_t = max_t;
  c.cap = capacity(s, max_t);
  c.score_stride = max_t;
  c.kv_block_stride = s->kv_block_stride;
  c.kv_head_stride = s->kv_head_stride;
  c.slab_block_stride = s->slab_block_stride;
  c.slab_head_stride = s->slab_head_stride;
  c.bf16 = s->kv_dtype == FASA_BF16 ? 1 : 0;
  c.scale = s->scale > 0.f ? s->scale : 1.0f / 11.313708498984761f;   // 1/sqrt(128)
  return c;
}

// Workspace layout shared by every entry point:
//   [unit histograms | FAC arrival counters | unit b1 | scores | kept pairs | kept counts | FAC partials]
// The histograms come first so that no other entry point ever writes over them:
// the select leaves them zero for the next call (a workspace that starts zeroed
// takes the fast path from the first call; other contents only slow it down).
// The FAC arrival counters (one per unit and head chunk) are zeroed by the
// launch before the FAC launch that counts on them.
struct Layout {
  size_t hist, fac_arrive, b1, scores, slots, counts, fac, total;
};
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
Layout layout(const Common& c, const FacPlan& p) {
  const size_t units = size_t(c.batch) * c.n_kv_heads;
  Layout l;
  l.hist = 0;
  l.fac_arrive = fasa::hist_bytes(c);
  l.b1 = l.fac_arrive + align256(units * p.head_chunks * sizeof(uint32_t));
  l.scores = l.b1 + align256(units * sizeof(int32_t));
  l.slots = l.scores + fasa::scores_bytes(c);
  l.counts = l.slots + fasa::slots_bytes(c);
  l.fac = l.counts + fasa::counts_bytes(c);
  l.total = l.fac + fasa::fac_workspace_bytes(c, p);
  return l;
}
fasa::SelectBuffers select_buffers(void* workspace, const Layout& l) {
  char* w = static_cast<char*>(workspace);
  return {reinterpret_cast<uint32_t*>(w + l.hist), w + l.slots, reinterpret_cast<int32_t*>(w + l.counts),
          reinterpret_cast<int32_t*>(w + l.b1)};
}
size_t decode_workspace(const Common& c, const FacPlan& p) { return layout(c, p).total; }

// Full attention: every cached token is a row, so the FAC plan is made for
// cap = max_t; the workspace holds the split partials only.
Common dense_common(const fasa_shape* s, int32_t max_t) {
  Common c = make_common(s, max_t);
  c.cap = max_t;
  return c;
}
size_t dense_workspace(const Common& c, const FacPlan& p) {
  const size_t n = fasa::fac_workspace_bytes(c, p);
  return n > 0 ? n : 256;
}

fasa_status hip_status(hipError_t e) { return e == hipSuccess ? FASA_OK : FASA_ERR_HIP; }

// Calibration: the selection runs over 65 rows per (sequence, kv head) --
// alpha and the 64 single-FC vectors -- as if they were 65 * H_kv kv heads.
// Workspace: [scores | unit histograms | b1 | kept pairs | kept counts |
// lists | list counts].
Common ca_select_common(const fasa_shape* s, int32_t max_t, int32_t k_top) {
  Common c = make_common(s, max_t);
  c.n_kv_heads = s->n_kv_heads * (fasa::kHeadDim / 2 + 1);
  c.n_q_heads = c.n_kv_heads * c.group;
  c.budget = k_top;
  c.n_sink = 0;
  c.n_recent = 0;
  c.cap = k_top < max_t ? k_top : max_t;
  c.score_stride = (max_t + 3) & ~3;
  return c;
}
struct CaLayout {
  size_t scores, hist, b1, slots, counts, sel_idx, sel_count, total;
};
CaLayout ca_layout(const Common& cs) {
  const size_t units = size_t(cs.batch) * cs.n_kv_heads;
  CaLayout l;
  l.scores = 0;
  l.hist = l.scores + align256(units * size_t(cs.score_stride) * sizeof(float));
  l.b1 = l.hist + fasa::hist_bytes(cs);
  l.slots = l.b1 + align256(units * sizeof(int32_t));
  l.counts = l.slots + fasa::slots_bytes(cs);
  l.sel_idx = l.counts + fasa::counts_bytes(cs);
  l.sel_count = l.sel_idx + align256(units * size_t(cs.cap > 0 ? cs.cap : 1) * sizeof(int32_t));
  l.total = l.sel_count + align256(units * sizeof(int32_t));
  return l;
}

// FASA-M: the decode workspace followed by the two staging arrays
// [b][H_kv][cap][128] (K, then V).
// Two row areas (K and V staging each): a step of parity p stages its rows in
// area p and finds the previous step's rows in area 1 - p.
struct MLayout {
  Layout d;
  size_t rows_k[2], rows_v[2], total;
};
MLayout m_layout(const Common& c, const FacPlan& p) {
  MLayout m;
  m.d = layout(c, p);
  const size_t e = c.bf16 ? 2 : 4;
  const size_t st = align256(size_t(c.batch) * c.n_kv_heads * size_t(c.cap) * fasa::kHeadDim * e);
  size_t o = m.d.total;
  for (int a = 0; a < 2; ++a) {
    m.rows_k[a] = o;
    m.rows_v[a] = o + st;
    o += 2 * st;
  }
  m.total = o;
  return m;
}

// Host arrays of FASA-M (element counts, for n_blocks physical blocks).
int64_t m_knd_elems(const fasa_shape* s, int64_t n_blocks) {
  const Common c = make_common(s, 0);
  return n_blocks * s->n_kv_heads * int64_t(fasa::kBlock) * fasa::m_nd_stride(c);
}
int64_t m_v_elems(const fasa_shape* s, int64_t n_blocks) {
  return n_blocks * s->n_kv_heads * int64_t(fasa::kBlock) * fasa::kHeadDim;
}

// The device-visible address of pinned host memory, or nullptr when ptr is not
// page-locked host memory known to the HIP runtime.
void* host_alias(const void* ptr) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type != hipMemoryTypeHost) return nullptr;
  if (at.devicePointer == nullptr) return const_cast<void*>(ptr);
  // The attributes describe the allocation that holds ptr: keep ptr's offset.
  if (at.hostPointer != nullptr)
    return static_cast<char*>(at.devicePointer) + (static_cast<const char*>(ptr) - static_cast<char*>(at.hostPointer));
  return at.devicePointer;
}

// Largest block-table / slab / pool pointers are only checked for null and
// alignment; their extents are preconditions.
size_t elem_align(const fasa_shape*) { return 16; }   // 16-byte vector loads

}  // namespace

extern "C" {

const char* fasa_status_str(fasa_status s) {
  switch (s) {
    case FASA_OK: return "FASA_OK";
    case FASA_ERR_INVALID_ARG: return "FASA_ERR_INVALID_ARG: null pointer, size, stride or alignment out of range";
    case FASA_ERR_UNSUPPORTED: return "FASA_ERR_UNSUPPORTED: shape not implemented (head_dim must be 128, block_size 256, group <= 16)";
    case FASA_ERR_WORKSPACE: return "FASA_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case FASA_ERR_HIP: return "FASA_ERR_HIP: a kernel launch failed";
    case FASA_ERR_SCRATCH:
      return "FASA_ERR_SCRATCH: the call needs more workspace than fasa_decode_scratch's fixed 64 MiB per device";
  }
  return "FASA: unknown status";
}

fasa_status fasa_validate_shape(const fasa_shape* shape) { return check_shape(shape); }

fasa_status fasa_selection_capacity(const fasa_shape* shape, int32_t max_t, int32_t* cap) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!cap) return FASA_ERR_INVALID_ARG;
  *cap = capacity(shape, max_t);
  return FASA_OK;
}

fasa_status fasa_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!bytes) return FASA_ERR_INVALID_ARG;
  const Common c = make_common(shape, max_t);
  *bytes = decode_workspace(c, fasa::fac_plan(c));
  return FASA_OK;
}

fasa_status fasa_decode_path(const fasa_shape* shape, int32_t max_t, int32_t* path) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!path) return FASA_ERR_INVALID_ARG;
  Common c = make_common(shape, max_t);
  c.score_stride = (max_t + 3) & ~3;   // as the decode step lays out its workspace
  const FacPlan p = fasa::fac_plan(c);
  const int lists = fasa::decode_lists(c, p);
  if (max_t <= 0) *path = FASA_PATH_NONE;
  else if (lists == fasa::kFromLists) *path = FASA_PATH_LISTS;
  else if (lists == fasa::kFromListsB1) *path = FASA_PATH_FILTERED_LISTS;
  else if (fasa::fac_selects(c, p)) *path = FASA_PATH_FILTER;
  else *path = FASA_PATH_SPLIT;
  return FASA_OK;
}

fasa_status fasa_check_fc_idx(const fasa_shape* shape, const int32_t* fc_idx_host) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (!fc_idx_host) return FASA_ERR_INVALID_ARG;
  const int nfc_all = shape->head_dim / 2;
  for (int g = 0; g < shape->n_kv_heads; ++g) {
    uint64_t seen[2] = {0, 0};   // head_dim/2 <= 64 when head_dim == 128
    bool padding = false;
    for (int f = 0; f < shape->n_fc; ++f) {
      const int32_t i = fc_idx_host[int64_t(g) * shape->n_fc + f];
      if (i == -1 && f > 0) {    // unused slots: only after at least one FC, to the end of the row
        padding = true;
        continue;
      }
      if (padding || i < 0 || i >= nfc_all) return FASA_ERR_INVALID_ARG;
      uint64_t& w = seen[i >> 6];
      const uint64_t bit = uint64_t(1) << (i & 63);
      if (w & bit) return FASA_ERR_INVALID_ARG;
      w |= bit;
    }
  }
  return FASA_OK;
}

fasa_status fasa_slab_build(const fasa_shape* shape, const void* k_pool, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* fc_idx, void* slab,
                            hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (!k_pool || !block_table || !seq_lens || !fc_idx || !slab) return FASA_ERR_INVALID_ARG;
  if (!aligned(k_pool, elem_align(shape)) || !aligned(slab, elem_align(shape))) return FASA_ERR_INVALID_ARG;
  if (shape->max_blocks_per_seq > std::numeric_limits<int32_t>::max() / 256) return FASA_ERR_INVALID_ARG;
  Common c = make_common(shape, shape->max_blocks_per_seq * fasa::kBlock);
  return hip_status(fasa::launch_slab_build(c, k_pool, block_table, seq_lens, fc_idx, slab, stream));
}

fasa_status fasa_slab_append(const fasa_shape* shape, const void* k_pool, const int32_t* block_table,
                             const int32_t* positions, const int32_t* fc_idx, void* slab,
                             hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (!k_pool || !block_table || !positions || !fc_idx || !slab) return FASA_ERR_INVALID_ARG;
  if (!aligned(k_pool, elem_align(shape)) || !aligned(slab, elem_align(shape))) return FASA_ERR_INVALID_ARG;
  Common c = make_common(shape, shape->max_blocks_per_seq * fasa::kBlock);
  return hip_status(fasa::launch_slab_append(c, k_pool, block_table, positions, fc_idx, slab, stream));
}

fasa_status fasa_tip(const fasa_shape* shape, const void* q, const void* slab, const void* k_pool,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                     float* scores, int32_t max_t, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!q || !block_table || !seq_lens || !fc_idx || !scores) return FASA_ERR_INVALID_ARG;
  if (!slab && !k_pool) return FASA_ERR_INVALID_ARG;
  const void* src = slab ? slab : k_pool;
  if (!aligned(src, elem_align(shape)) || !aligned(scores, 16)) return FASA_ERR_INVALID_ARG;
  if (max_t == 0) return FASA_OK;
  Common c = make_common(shape, max_t);
  return hip_status(fasa::launch_tip(c, q, slab, k_pool, block_table, seq_lens, fc_idx, scores,
                                     fasa::TipOutputs{fasa::kTipScores, nullptr, nullptr, nullptr}, stream));
}

fasa_status fasa_topk(const fasa_shape* shape, const float* scores, const int32_t* seq_lens,
                      int32_t max_t, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!scores || !seq_lens || !sel_count) return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(scores, 16)) return FASA_ERR_INVALID_ARG;
  Common c = make_common(shape, max_t);
  const Layout l = layout(c, fasa::fac_plan(c));
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < l.total) return FASA_ERR_WORKSPACE;
  const fasa::SelectBuffers sb = select_buffers(workspace, l);
  if ((st = hip_status(fasa::launch_filter(c, scores, seq_lens, sb, false, nullptr, 0, stream))) != FASA_OK) return st;
  return hip_status(fasa::launch_finish(c, scores, seq_lens, sel_idx, sel_count, sb, nullptr, 0, stream));
}

fasa_status fasa_fac(const fasa_shape* shape, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* sel_idx, const int32_t* sel_count,
                     int32_t max_t, float* out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !sel_count || !out) return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)) return FASA_ERR_INVALID_ARG;
  Common c = make_common(shape, max_t);
  const FacPlan p = fasa::fac_plan(c);
  const Layout l = layout(c, p);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < l.total) return FASA_ERR_WORKSPACE;
  return hip_status(fasa::launch_fac(c, p, q, k_pool, v_pool, block_table, sel_idx, sel_count, out,
                                     static_cast<char*>(workspace) + l.fac, nullptr, stream));
}

namespace {

// The per-call plan of a decode step, shared by its two stages: the layout of
// the workspace and whether TIP emits per-chunk candidates (two launches) or
// builds the unit histograms for a filter launch.
struct DecodePlan {
  Common c;
  FacPlan p;
  Layout l;
  int lists;        // where the select's candidates come from (fasa::kFrom*)
};

fasa_status decode_plan(const fasa_shape* shape, int32_t max_t, const void* workspace, size_t workspace_bytes,
                        DecodePlan& d) {
  d.c = make_common(shape, max_t);
  d.c.score_stride = (max_t + 3) & ~3;   // the workspace's scores rows: 16-byte loads throughout
  d.p = fasa::fac_plan(d.c);
  d.l = layout(d.c, d.p);
  d.lists = fasa::decode_lists(d.c, d.p);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < d.l.total) return FASA_ERR_WORKSPACE;
  return FASA_OK;
}

// Stage 1: TIP, with the outputs stage 2 reads (candidate lists or histograms).
fasa_status decode_tip_stage(const DecodePlan& d, const void* q, const void* k_pool, const void* slab,
                             const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                             void* workspace, hipStream_t stream) {
  if (d.c.max_t <= 0) return FASA_OK;
  char* w = static_cast<char*>(workspace);
  const fasa::SelectBuffers sb = select_buffers(workspace, d.l);
  float* scores = reinterpret_cast<float*>(w + d.l.scores);
  uint32_t* fac_arrive = reinterpret_cast<uint32_t*>(w + d.l.fac_arrive);
  const int mode = d.lists == fasa::kFromLists ? fasa::kTipEmit
                   : (d.lists == fasa::kFromListsB1 ? fasa::kTipEmitHist : fasa::kTipHist);
  const fasa::TipOutputs to{mode, sb.hist, static_cast<uint2*>(sb.slots), reinterpret_cast<uint2*>(sb.counts),
                            fac_arrive};
  return hip_status(fasa::launch_tip(d.c, q, slab, k_pool, block_table, seq_lens, fc_idx, scores, to, stream));
}

// Stage 2: the exact top-B from stage 1's outputs, then FAC.
fasa_status decode_rest_stage(const DecodePlan& d, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens, float* out, int32_t* sel_idx,
                              int32_t* sel_count, void* workspace, hipStream_t stream) {
  const Common& c = d.c;
  const FacPlan& p = d.p;
  char* w = static_cast<char*>(workspace);
  const fasa::SelectBuffers sb = select_buffers(workspace, d.l);
  float* scores = reinterpret_cast<float*>(w + d.l.scores);
  uint32_t* fac_arrive = reinterpret_cast<uint32_t*>(w + d.l.fac_arrive);
  if (d.lists != fasa::kFromFilter)
    return hip_status(fasa::launch_fac_select(c, p, q, k_pool, v_pool, block_table, scores, seq_lens, sb, d.lists,
                                              fac_arrive, sel_idx, sel_count, out, stream));
  fasa_status st;
  if ((st = hip_status(fasa::launch_filter(c, scores, seq_lens, sb, true, fac_arrive, p.head_chunks, stream))) !=
      FASA_OK)
    return st;
  if (fasa::fac_selects(c, p))
    return hip_status(fasa::launch_fac_select(c, p, q, k_pool, v_pool, block_table, scores, seq_lens, sb,
                                              fasa::kFromFilter, nullptr, sel_idx, sel_count, out, stream));
  if ((st = hip_status(fasa::launch_finish(c, scores, seq_lens, sel_idx, sel_count, sb, fac_arrive, p.head_chunks,
                                           stream))) != FASA_OK)
    return st;
  return hip_status(fasa::launch_fac(c, p, q, k_pool, v_pool, block_table, sel_idx, sel_count, out,
                                     w + d.l.fac, fac_arrive, stream));
}

fasa_status check_decode_inputs(const fasa_shape* shape, int32_t max_t, const void* q, const void* k_pool,
                                const void* slab, const int32_t* block_table, const int32_t* seq_lens) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!q || !k_pool || !block_table || !seq_lens) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16)) return FASA_ERR_INVALID_ARG;
  if (slab && !aligned(slab, 16)) return FASA_ERR_INVALID_ARG;
  return FASA_OK;
}

fasa_status check_decode_outputs(const fasa_shape* shape, int32_t max_t, const void* v_pool, const float* out,
                                 const int32_t* sel_idx, const int32_t* sel_count) {
  if (!v_pool || !out || !sel_count) return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(v_pool, 16)) return FASA_ERR_INVALID_ARG;
  return FASA_OK;
}

}  // namespace

fasa_status fasa_decode(const fasa_shape* shape, const void* q, const void* k_pool, const void* v_pool,
                        const void* slab, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t max_t, const int32_t* fc_idx, float* out, int32_t* sel_idx,
                        int32_t* sel_count, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  // Small budgets and rows whose candidate lists fit on chip: TIP (+ each
  // chunk's candidates) -> FAC that finishes the exact select from them and
  // writes out directly; two launches.  Otherwise TIP (+ unit histograms) ->
  // filter (+ FAC counters zeroed) -> the same FAC over the filter's kept keys
  // (small budgets), or for large budgets the exact select as a launch of its
  // own, followed by a split-K FAC merged in its last workgroups.
  fasa_status st = check_decode_inputs(shape, max_t, q, k_pool, slab, block_table, seq_lens);
  if (st != FASA_OK) return st;
  if (!fc_idx) return FASA_ERR_INVALID_ARG;
  if ((st = check_decode_outputs(shape, max_t, v_pool, out, sel_idx, sel_count)) != FASA_OK) return st;
  DecodePlan d;
  if ((st = decode_plan(shape, max_t, workspace, workspace_bytes, d)) != FASA_OK) return st;
  if ((st = decode_tip_stage(d, q, k_pool, slab, block_table, seq_lens, fc_idx, workspace, stream)) != FASA_OK)
    return st;
  return decode_rest_stage(d, q, k_pool, v_pool, block_table, seq_lens, out, sel_idx, sel_count, workspace, stream);
}

fasa_status fasa_decode_tip(const fasa_shape* shape, const void* q, const void* k_pool, const void* slab,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t max_t,
                            const int32_t* fc_idx, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = check_decode_inputs(shape, max_t, q, k_pool, slab, block_table, seq_lens);
  if (st != FASA_OK) return st;
  if (!fc_idx) return FASA_ERR_INVALID_ARG;
  DecodePlan d;
  if ((st = decode_plan(shape, max_t, workspace, workspace_bytes, d)) != FASA_OK) return st;
  return decode_tip_stage(d, q, k_pool, slab, block_table, seq_lens, fc_idx, workspace, stream);
}

fasa_status fasa_decode_rest(const fasa_shape* shape, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t max_t, float* out,
                             int32_t* sel_idx, int32_t* sel_count, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  fasa_status st = check_decode_inputs(shape, max_t, q, k_pool, nullptr, block_table, seq_lens);
  if (st != FASA_OK) return st;
  if ((st = check_decode_outputs(shape, max_t, v_pool, out, sel_idx, sel_count)) != FASA_OK) return st;
  DecodePlan d;
  if ((st = decode_plan(shape, max_t, workspace, workspace_bytes, d)) != FASA_OK) return st;
  return decode_rest_stage(d, q, k_pool, v_pool, block_table, seq_lens, out, sel_idx, sel_count, workspace, stream);
}

fasa_status fasa_m_host_sizes(const fasa_shape* shape, int64_t n_blocks, size_t* k_nd_bytes, size_t* v_bytes) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (n_blocks < 1 || !k_nd_bytes || !v_bytes) return FASA_ERR_INVALID_ARG;
  const size_t e = shape->kv_dtype == FASA_BF16 ? 2 : 4;
  *k_nd_bytes = size_t(m_knd_elems(shape, n_blocks)) * e;
  *v_bytes = size_t(m_v_elems(shape, n_blocks)) * e;
  return FASA_OK;
}

fasa_status fasa_m_offload(const fasa_shape* shape, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* seq_lens, const int32_t* fc_idx,
                           void* k_nd_host, void* v_host, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (!k_pool || !v_pool || !block_table || !seq_lens || !fc_idx || !k_nd_host || !v_host)
    return FASA_ERR_INVALID_ARG;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_nd_host, 16) || !aligned(v_host, 16))
    return FASA_ERR_INVALID_ARG;
  void* knd = host_alias(k_nd_host);
  void* vh = host_alias(v_host);
  if (!knd || !vh) return FASA_ERR_INVALID_ARG;
  const Common c = make_common(shape, shape->max_blocks_per_seq * fasa::kBlock);
  return hip_status(fasa::launch_m_offload(c, k_pool, v_pool, block_table, seq_lens, fc_idx, knd, vh, stream));
}

fasa_status fasa_m_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!bytes) return FASA_ERR_INVALID_ARG;
  const Common c = make_common(shape, max_t);
  *bytes = m_layout(c, fasa::fac_plan(c)).total;
  return FASA_OK;
}

namespace {

// Shared checks and plan of the FASA-M entry points.
struct MPlan {
  Common c;
  FacPlan p;
  MLayout m;
};

fasa_status m_plan(const fasa_shape* shape, int32_t max_t, const void* workspace, size_t workspace_bytes,
                   MPlan& mp) {
  mp.c = make_common(shape, max_t);
  mp.c.score_stride = (max_t + 3) & ~3;
  mp.p = fasa::fac_plan(mp.c);
  mp.m = m_layout(mp.c, mp.p);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < mp.m.total) return FASA_ERR_WORKSPACE;
  return FASA_OK;
}

fasa_status m_check(const fasa_shape* shape, int32_t max_t) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  return check_max_t(shape, max_t);
}

// TIP on the slab -> filter -> exact select (the list is needed to gather).
fasa_status m_select_stage(const MPlan& mp, const void* q, const void* slab, const int32_t* block_table,
                           const int32_t* seq_lens, const int32_t* fc_idx, int32_t* sel_idx, int32_t* sel_count,
                           void* workspace, hipStream_t stream) {
  const Common& c = mp.c;
  char* w = static_cast<char*>(workspace);
  const fasa::SelectBuffers sb = select_buffers(workspace, mp.m.d);
  float* scores = reinterpret_cast<float*>(w + mp.m.d.scores);
  uint32_t* fac_arrive = reinterpret_cast<uint32_t*>(w + mp.m.d.fac_arrive);
  fasa_status st;
  if (c.max_t > 0) {
    if ((st = hip_status(fasa::launch_tip(c, q, slab, nullptr, block_table, seq_lens, fc_idx, scores,
                                          fasa::TipOutputs{fasa::kTipHist, sb.hist, nullptr, nullptr}, stream))) !=
        FASA_OK)
      return st;
  }
  if ((st = hip_status(fasa::launch_filter(c, scores, seq_lens, sb, true, fac_arrive, mp.p.head_chunks, stream))) !=
      FASA_OK)
    return st;
  return hip_status(fasa::launch_finish(c, scores, seq_lens, sel_idx, sel_count, sb, fac_arrive, mp.p.head_chunks,
                                        stream));
}

// Rows from the host (and, with reuse, the other row area) into row area
// `area` -> FAC.
fasa_status m_finish_stage(const MPlan& mp, const void* q, const void* slab, const void* knd, const void* vh,
                           const int32_t* block_table, const int32_t* fc_idx, const int32_t* sel_idx,
                           const int32_t* sel_count, const fasa::MReuse& reuse, int area, float* out,
                           void* workspace, hipStream_t stream) {
  char* w = static_cast<char*>(workspace);
  uint32_t* fac_arrive = reinterpret_cast<uint32_t*>(w + mp.m.d.fac_arrive);
  fasa_status st;
  if ((st = hip_status(fasa::launch_m_gather(mp.c, knd, vh, slab, block_table, fc_idx, sel_idx, sel_count,
                                             w + mp.m.rows_k[area], w + mp.m.rows_v[area], reuse, stream))) !=
      FASA_OK)
    return st;
  return hip_status(fasa::launch_fac_staged(mp.c, mp.p, q, w + mp.m.rows_k[area], w + mp.m.rows_v[area], sel_count,
                                            out, w + mp.m.d.fac, fac_arrive, stream));
}

}  // namespace

fasa_status fasa_m_decode(const fasa_shape* shape, const void* q, const void* slab, const void* k_nd_host,
                          const void* v_host, const int32_t* block_table, const int32_t* seq_lens, int32_t max_t,
                          const int32_t* fc_idx, float* out, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = m_check(shape, max_t);
  if (st != FASA_OK) return st;
  if (!q || !slab || !k_nd_host || !v_host || !block_table || !seq_lens || !fc_idx || !out || !sel_count)
    return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(slab, 16) || !aligned(k_nd_host, 16) || !aligned(v_host, 16))
    return FASA_ERR_INVALID_ARG;
  const void* knd = host_alias(k_nd_host);
  const void* vh = host_alias(v_host);
  if (!knd || !vh) return FASA_ERR_INVALID_ARG;
  MPlan mp;
  if ((st = m_plan(shape, max_t, workspace, workspace_bytes, mp)) != FASA_OK) return st;
  if ((st = m_select_stage(mp, q, slab, block_table, seq_lens, fc_idx, sel_idx, sel_count, workspace, stream)) !=
      FASA_OK)
    return st;
  return m_finish_stage(mp, q, slab, knd, vh, block_table, fc_idx, sel_idx, sel_count, fasa::MReuse{}, 0, out,
                        workspace, stream);
}

fasa_status fasa_m_decode_select(const fasa_shape* shape, const void* q, const void* slab,
                                 const int32_t* block_table, const int32_t* seq_lens, int32_t max_t,
                                 const int32_t* fc_idx, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = m_check(shape, max_t);
  if (st != FASA_OK) return st;
  if (!q || !slab || !block_table || !seq_lens || !fc_idx || !sel_count) return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(slab, 16)) return FASA_ERR_INVALID_ARG;
  MPlan mp;
  if ((st = m_plan(shape, max_t, workspace, workspace_bytes, mp)) != FASA_OK) return st;
  return m_select_stage(mp, q, slab, block_table, seq_lens, fc_idx, sel_idx, sel_count, workspace, stream);
}

fasa_status fasa_m_prefetch(const fasa_shape* shape, const void* slab, const void* k_nd_host, const void* v_host,
                            const int32_t* block_table, int32_t max_t, const int32_t* fc_idx,
                            const int32_t* prev_sel_idx, const int32_t* prev_sel_count, int32_t parity,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = m_check(shape, max_t);
  if (st != FASA_OK) return st;
  if (parity != 0 && parity != 1) return FASA_ERR_INVALID_ARG;
  if (!slab || !k_nd_host || !v_host || !block_table || !fc_idx || !prev_sel_count) return FASA_ERR_INVALID_ARG;
  if (!prev_sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if (!aligned(slab, 16) || !aligned(k_nd_host, 16) || !aligned(v_host, 16)) return FASA_ERR_INVALID_ARG;
  const void* knd = host_alias(k_nd_host);
  const void* vh = host_alias(v_host);
  if (!knd || !vh) return FASA_ERR_INVALID_ARG;
  MPlan mp;
  if ((st = m_plan(shape, max_t, workspace, workspace_bytes, mp)) != FASA_OK) return st;
  char* w = static_cast<char*>(workspace);
  return hip_status(fasa::launch_m_gather(mp.c, knd, vh, slab, block_table, fc_idx, prev_sel_idx, prev_sel_count,
                                          w + mp.m.rows_k[1 - parity], w + mp.m.rows_v[1 - parity],
                                          fasa::MReuse{}, stream));
}

fasa_status fasa_m_decode_finish(const fasa_shape* shape, const void* q, const void* slab, const void* k_nd_host,
                                 const void* v_host, const int32_t* block_table, int32_t max_t,
                                 const int32_t* fc_idx, const int32_t* prev_sel_idx,
                                 const int32_t* prev_sel_count, const int32_t* sel_idx, const int32_t* sel_count,
                                 int32_t parity, float* out, int32_t* hits, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = m_check(shape, max_t);
  if (st != FASA_OK) return st;
  if (parity != 0 && parity != 1) return FASA_ERR_INVALID_ARG;
  if (!q || !slab || !k_nd_host || !v_host || !block_table || !fc_idx || !out || !sel_count)
    return FASA_ERR_INVALID_ARG;
  if (!sel_idx && capacity(shape, max_t) > 0) return FASA_ERR_INVALID_ARG;
  if ((prev_sel_idx == nullptr) != (prev_sel_count == nullptr)) return FASA_ERR_INVALID_ARG;
  if (!prev_sel_idx && hits) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(slab, 16) || !aligned(k_nd_host, 16) || !aligned(v_host, 16))
    return FASA_ERR_INVALID_ARG;
  const void* knd = host_alias(k_nd_host);
  const void* vh = host_alias(v_host);
  if (!knd || !vh) return FASA_ERR_INVALID_ARG;
  MPlan mp;
  if ((st = m_plan(shape, max_t, workspace, workspace_bytes, mp)) != FASA_OK) return st;
  char* w = static_cast<char*>(workspace);
  fasa::MReuse reuse;
  if (prev_sel_idx) {
    reuse.prev_idx = prev_sel_idx;
    reuse.prev_count = prev_sel_count;
    reuse.pf_k = w + mp.m.rows_k[1 - parity];
    reuse.pf_v = w + mp.m.rows_v[1 - parity];
    reuse.hits = hits;
  }
  return m_finish_stage(mp, q, slab, knd, vh, block_table, fc_idx, sel_idx, sel_count, reuse, parity, out, workspace,
                        stream);
}

fasa_status fasa_ca_workspace_size(const fasa_shape* shape, int32_t max_t, int32_t k_top, size_t* bytes) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!bytes || k_top < 1 || k_top > fasa::kCaMaxK) return FASA_ERR_INVALID_ARG;
  *bytes = ca_layout(ca_select_common(shape, max_t, k_top)).total;
  return FASA_OK;
}

fasa_status fasa_ca_hits(const fasa_shape* shape, const void* q, const void* k_pool, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t max_t, int32_t k_top, int32_t* hits, int32_t* topk,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!q || !k_pool || !block_table || !seq_lens || !hits || k_top < 1 || k_top > fasa::kCaMaxK)
    return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16)) return FASA_ERR_INVALID_ARG;
  const Common cs = ca_select_common(shape, max_t, k_top);
  const CaLayout l = ca_layout(cs);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < l.total) return FASA_ERR_WORKSPACE;
  char* w = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(w + l.scores);
  int32_t* sel_idx = reinterpret_cast<int32_t*>(w + l.sel_idx);
  int32_t* sel_count = reinterpret_cast<int32_t*>(w + l.sel_count);
  const fasa::SelectBuffers sb{reinterpret_cast<uint32_t*>(w + l.hist), w + l.slots,
                               reinterpret_cast<int32_t*>(w + l.counts), reinterpret_cast<int32_t*>(w + l.b1)};
  Common c = make_common(shape, max_t);
  c.score_stride = cs.score_stride;
  if (max_t > 0) {
    if ((st = hip_status(fasa::launch_ca_scores(c, q, k_pool, block_table, seq_lens, scores, stream))) != FASA_OK)
      return st;
  }
  // One calibration sequence normally fills its rows to max_t: the filter
  // then loads its scores without waiting for the length.
  if ((st = hip_status(fasa::launch_filter(cs, scores, seq_lens, sb, false, nullptr, 0, stream,
                                           shape->batch == 1))) != FASA_OK)
    return st;
  if ((st = hip_status(fasa::launch_finish(cs, scores, seq_lens, sel_idx, sel_count, sb, nullptr, 0, stream))) !=
      FASA_OK)
    return st;
  Common ch = cs;
  ch.n_kv_heads = shape->n_kv_heads;
  return hip_status(fasa::launch_ca_hits(ch, sel_idx, sel_count, hits, topk, stream));
}

fasa_status fasa_ca_dominant(const fasa_shape* shape, const int32_t* hits, int32_t n_rows, int32_t n_tip,
                             int32_t* fc_idx, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if (!hits || !fc_idx || n_rows < 1 || n_tip < 1 || n_tip > fasa::kHeadDim / 2) return FASA_ERR_INVALID_ARG;
  return hip_status(fasa::launch_ca_dominant(hits, n_rows, shape->n_kv_heads, n_tip, fc_idx, stream));
}

fasa_status fasa_dense_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!bytes) return FASA_ERR_INVALID_ARG;
  const Common c = dense_common(shape, max_t);
  *bytes = dense_workspace(c, fasa::dense_plan(c));
  return FASA_OK;
}

fasa_status fasa_dense_decode(const fasa_shape* shape, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens, int32_t max_t, float* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fasa_status st = check_shape(shape);
  if (st != FASA_OK) return st;
  if ((st = check_max_t(shape, max_t)) != FASA_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out) return FASA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16)) return FASA_ERR_INVALID_ARG;
  const Common c = dense_common(shape, max_t);
  const FacPlan p = fasa::dense_plan(c);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < dense_workspace(c, p)) return FASA_ERR_WORKSPACE;
  return hip_status(fasa::launch_dense(c, p, q, k_pool, v_pool, block_table, seq_lens, out, workspace, stream));
}

}  // extern "C"
