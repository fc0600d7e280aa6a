/*
 * fasa.h -- C ABI of libfasa.so: the decode-time hot path of FASA
 * (Frequency-Aware Sparse Attention) for AMD Instinct MI355X (gfx950).
 *
 * One decode step, for every sequence b and kv head g (a "unit"):
 *   TIP  : S[j] = sum over the group's query heads h and the dominant FCs f of
 *          q_h[2 I_g[f]] k_j[2 I_g[f]] + q_h[2 I_g[f]+1] k_j[2 I_g[f]+1]
 *          for every cached token j < t_b  (paper-graph-ui review of FASA,
 *          section 3.4 "Online Stage 1: Token Importance Predictor (TIP)",
 *          score equation; FC i is the dimension pair (2i, 2i+1), section 3.4
 *          "RoPE from a Frequency-Chunk Perspective").
 *   TOP-B: sel = forced tokens  U  the B candidates with the largest S, where
 *          the forced tokens are j < n_sink and j >= t_b - n_recent, equal
 *          scores go to the lower index, and -0.0 equals +0.0 (section 3.4,
 *          token-selection equation T_t = TopK-I(S_t, N_fac)).
 *   FAC  : out_h = softmax(q_h K_sel^T * scale) V_sel for every query head of
 *          the group, over the selected rows at their original positions
 *          (section 3.4 "Online Stage 2: Focused Attention Computation",
 *          gather and attention equations).
 * Query head h belongs to kv head h / (n_q_heads / n_kv_heads).
 *
 * Memory layout (all element offsets are in units of the cache dtype):
 *   q         [batch][n_q_heads][head_dim]            post-RoPE query, kv dtype
 *   k_pool,   element (p, g, s, c) of physical block p, kv head g, slot s,
 *   v_pool      channel c at p*kv_block_stride + g*kv_head_stride + s*head_dim + c
 *               (a paged pool [n_blocks][H_kv][256][d] has strides
 *               (H_kv*256*d, 256*d); a dense [batch][H_kv][T][d] cache has
 *               strides (256*d, T*d) with block_table[b][k] = b*H_kv*T/256 + k)
 *   block_table [batch][max_blocks_per_seq] int32: token j of sequence b lives
 *               in physical block block_table[b][j/256], slot j%256
 *   seq_lens  [batch] int32, t_b: cached tokens 0..t_b-1 (the query is at t_b)
 *   fc_idx    [n_kv_heads][n_fc] int32: dominant FC indices I_g, distinct,
 *               each in [0, head_dim/2)
 *   slab      the dominant-key cache (FC-major side copy of the dominant key
 *               columns), indexed by sequence and logical block -- not by the
 *               pool's physical block, so TIP needs no block-table lookup:
 *               element (b, k, g, f, s, c) = K of token 256*k + s of sequence b,
 *               kv head g, column 2*fc_idx[g][f] + c, at
 *               (b*max_blocks_per_seq + k)*slab_block_stride
 *                 + g*slab_head_stride + f*512 + s*2 + c
 *               (default strides (H_kv*F*512, F*512): an array
 *               [batch][max_blocks_per_seq][H_kv][F][256][2])
 *   scores    [batch][n_kv_heads][max_t] fp32, S of token j at column j
 *   sel_idx   [batch][n_kv_heads][cap] int32, cap = fasa_selection_capacity():
 *               the selected token indices ascending, then -1 padding
 *   sel_count [batch][n_kv_heads] int32, number of valid entries of sel_idx
 *   out       [batch][n_q_heads][head_dim] fp32
 *
 * Ownership and threading: the caller owns every buffer; every pointer is a
 * device pointer except the fasa_shape and fc_idx_host arguments, which are
 * read during the call only.  The library allocates nothing, frees nothing,
 * never synchronises, and keeps no mutable global state, so calls are
 * thread-safe and may be captured into a HIP graph.  Work is enqueued on the
 * given stream (0 = the null stream).
 *
 * Errors: every argument is validated on the host before anything is enqueued;
 * on any error nothing is enqueued or written.  FASA_ERR_HIP reports a failed
 * kernel launch.  Faults inside kernels surface at the caller's next
 * synchronisation.  The *contents* of device arrays are preconditions:
 * seq_lens[b] <= min(max_t, 256*max_blocks_per_seq), block_table entries name
 * allocated blocks, fc_idx rows are distinct and in range (check them with
 * fasa_check_fc_idx), and scores are finite (non-finite scores give an
 * unspecified selection).  Kernels clamp t_b into range instead of faulting.
 * A sequence with t_b = 0 selects nothing and its output rows are zero.
 */
#ifndef FASA_H
#define FASA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fasa_status {
  FASA_OK = 0,
  FASA_ERR_INVALID_ARG = 1,  /* null pointer, size or stride out of range */
  FASA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim != 128, ...) */
  FASA_ERR_WORKSPACE = 3,    /* workspace too small or misaligned */
  FASA_ERR_HIP = 4,          /* a kernel launch failed */
  FASA_ERR_SCRATCH = 5       /* fasa_decode_scratch: the call needs more than its fixed scratch */
} fasa_status;

typedef enum fasa_dtype { FASA_F32 = 0, FASA_BF16 = 1 } fasa_dtype;

/* Problem description, read on the host at call time only. */
typedef struct fasa_shape {
  int32_t batch;              /* sequences, >= 1 */
  int32_t n_q_heads;          /* H_q, a multiple of n_kv_heads */
  int32_t n_kv_heads;         /* H_kv >= 1; group size G = H_q/H_kv <= 16 */
  int32_t head_dim;           /* d, must be 128 */
  int32_t n_fc;               /* F dominant FCs per kv head, 1..head_dim/2 */
  int32_t budget;             /* B >= 1; B >= candidates keeps them all */
  int32_t n_sink;             /* always-kept first tokens, >= 0 */
  int32_t n_recent;           /* always-kept last tokens, >= 0 */
  int32_t block_size;         /* tokens per cache block, must be 256 */
  int32_t max_blocks_per_seq; /* columns of block_table, >= 1 */
  int64_t kv_block_stride;    /* elements, multiple of 8, >= 256*head_dim */
  int64_t kv_head_stride;     /* elements, multiple of 8, >= 256*head_dim */
  int64_t slab_block_stride;  /* elements between logical blocks, multiple of 8 */
  int64_t slab_head_stride;   /* elements, multiple of 8, >= 512*n_fc */
  int32_t kv_dtype;           /* fasa_dtype of q, k_pool, v_pool and slab */
  float scale;                /* softmax scale; 0 means 1/sqrt(head_dim) */
} fasa_shape;

/* Text for a status code (static storage). */
const char* fasa_status_str(fasa_status s);

/* Host-side check of every field of *shape (no device work). */
fasa_status fasa_validate_shape(const fasa_shape* shape);

/* cap = min(max_t, budget + n_sink + n_recent): the row length of sel_idx. */
fasa_status fasa_selection_capacity(const fasa_shape* shape, int32_t max_t, int32_t* cap);

/* Bytes of workspace that fasa_decode, fasa_topk and fasa_fac need for contexts
 * up to max_t (one size for all three): about 12 bytes per token of max_t per
 * (sequence, kv head) -- scores and the select's kept (key, index) pairs --
 * plus 8 KB per (sequence, kv head) and the FAC partials.  The workspace must
 * be 256-byte aligned.
 * It carries one small per-unit histogram from call to call: the select leaves
 * it zero, and a workspace that starts zero-filled takes the fast path from the
 * first call.  Its contents never change any result (a non-zero histogram only
 * sends the select to its slower full-row path once).  Calls that share a
 * workspace must be ordered on one stream. */
fasa_status fasa_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes);

/* Host check of a HOST copy of fc_idx [n_kv_heads][n_fc]: every entry in
 * [0, head_dim/2) and no duplicate within a row (an FC is an indivisible unit
 * and is counted once: section 3.4, "FCs Are Indivisible Units").  A row may
 * end in -1 entries after at least one FC: kv head g then uses only its first
 * N_tip(g) FCs (per-head N_tip, an extension the pages leave to future work);
 * the slab keeps zeros in those slots and TIP still reads n_fc slots per
 * token.  FASA-M (fasa_m_*) needs rows without -1 entries. */
fasa_status fasa_check_fc_idx(const fasa_shape* shape, const int32_t* fc_idx_host);

/* Build the dominant-key cache for tokens 0..t_b-1 of every sequence from the
 * post-RoPE key pool (the GPU-resident dominant key cache of section 3.4,
 * "Hardware-Aware Variants": only the dominant dimensions of every key).
 * Writes logical blocks 0 .. ceil(t_b/256)-1 of each sequence whole (slots
 * past t_b in the last block are copied from the pool as they are); sequences
 * that share physical blocks get their own copies. */
fasa_status fasa_slab_build(const fasa_shape* shape, const void* k_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* fc_idx, void* slab, hipStream_t stream);

/* After the caller has written the post-RoPE key of token positions[b] of every
 * sequence into k_pool, copy its dominant columns into the slab (slot
 * positions[b] % 256 of logical block positions[b] / 256 of sequence b; the
 * dominant-key cache is kept current per token, section 3.4, "Hardware-Aware
 * Variants").  positions[b] < 0 skips sequence b; positions at or past
 * 256*max_blocks_per_seq are skipped too. */
fasa_status fasa_slab_append(const fasa_shape* shape, const void* k_pool,
                             const int32_t* block_table, const int32_t* positions,
                             const int32_t* fc_idx, void* slab, hipStream_t stream);

/* TIP (section 3.4, "Online Stage 1: Token Importance Predictor (TIP)", the
 * score equation: the importance of every cached token from the dominant FCs
 * only; FC i is the pair (2i, 2i+1), section 3.4 "RoPE from a Frequency-Chunk
 * Perspective"): scores[b][g][j] for j < t_b (columns past t_b are left
 * untouched).  Reads the slab when slab != NULL; with slab == NULL it gathers the dominant
 * columns straight from k_pool (same arithmetic, same bits, more bytes).
 * Scores accumulate in fp32: the query heads of the group are first summed per
 * dominant column (fp32), then each token's 2*n_fc products are added in FC
 * order with fused multiply-adds. */
fasa_status fasa_tip(const fasa_shape* shape, const void* q, const void* slab,
                     const void* k_pool, const int32_t* block_table,
                     const int32_t* seq_lens, const int32_t* fc_idx, float* scores,
                     int32_t max_t, hipStream_t stream);

/* TOP-B over given scores (section 3.4, the token-selection equation
 * T_t = TopK-I(S_t, N_fac): the indices of the N_fac largest scores, with the
 * forced tokens kept on top): sel_idx / sel_count as described above.  Exact:
 * the selection is a function of the fp32 score bits only.  The workspace is
 * sized by fasa_workspace_size. */
fasa_status fasa_topk(const fasa_shape* shape, const float* scores,
                      const int32_t* seq_lens, int32_t max_t, int32_t* sel_idx,
                      int32_t* sel_count, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* FAC over a given selection (section 3.4, "Online Stage 2: Focused Attention
 * Computation (FAC)", the gather and attention equations: softmax(q K_T^T *
 * scale) V_T over the selected rows, which keep their positions), with
 * sel_idx / sel_count laid out for max_t.  bf16 caches compute in fp32; fp32 caches compute logits, softmax and the
 * weighted sum in fp64 and round the result to fp32 once.  sel_count is
 * clamped into [0, cap]; entries of sel_idx[0..sel_count) below 0 or at or past
 * max_blocks_per_seq * block_size contribute nothing, and a head whose
 * selection holds no such valid entry gets an all-zero output.  Entries that
 * are in range but past t_b read whatever the cache holds there. */
fasa_status fasa_fac(const fasa_shape* shape, const void* q, const void* k_pool,
                     const void* v_pool, const int32_t* block_table,
                     const int32_t* sel_idx, const int32_t* sel_count, int32_t max_t,
                     float* out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* The whole step of section 3.4 (TIP, then the token selection T_t =
 * TopK-I(S_t, N_fac), then FAC over T_t; the online stages 1 and 2), enqueued
 * on one stream: the same results as fasa_tip -> fasa_topk -> fasa_fac.  slab
 * == NULL makes TIP read the dominant columns from k_pool.  sel_idx and
 * sel_count are outputs (the selection used). */
fasa_status fasa_decode(const fasa_shape* shape, const void* q, const void* k_pool,
                        const void* v_pool, const void* slab, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t max_t, const int32_t* fc_idx,
                        float* out, int32_t* sel_idx, int32_t* sel_count,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* fasa_decode in its two stages, for callers that time or schedule them apart
 * (section 3.4's online stage 1, TIP, and stage 2, the selection and FAC).
 * fasa_decode_tip enqueues the step's first launch only: TIP over every unit,
 * leaving in the workspace what the rest of the step reads (per-chunk
 * candidate lists or per-unit score histograms, chosen from shape and max_t as
 * fasa_decode chooses).  fasa_decode_rest enqueues the rest: the exact top-B
 * from those, then FAC; sel_idx, sel_count and out as in fasa_decode.  The two
 * calls, in order on one stream with the same shape, max_t, inputs and
 * workspace, and nothing else using that workspace between them, give exactly
 * fasa_decode's results.  Arguments and errors as in fasa_decode (the
 * arguments a stage does not read are left out). */
fasa_status fasa_decode_tip(const fasa_shape* shape, const void* q, const void* k_pool,
                            const void* slab, const int32_t* block_table, const int32_t* seq_lens,
                            int32_t max_t, const int32_t* fc_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
fasa_status fasa_decode_rest(const fasa_shape* shape, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, int32_t max_t, float* out, int32_t* sel_idx,
                             int32_t* sel_count, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* The launch structure fasa_decode (and its two stages) uses for a shape and
 * max_t, written to *path (host memory); the results never depend on it.  It
 * is reported for tests and tuning:
 *   FASA_PATH_NONE            max_t == 0: nothing is launched;
 *   FASA_PATH_LISTS           TIP writes per-chunk candidate lists, and one
 *                             selecting FAC launch finishes the top-B from them;
 *   FASA_PATH_FILTERED_LISTS  the same, TIP also building the unit histograms,
 *                             whose threshold cuts the lists down;
 *   FASA_PATH_FILTER          TIP's unit histograms, a filter launch, then the
 *                             selecting FAC launch;
 *   FASA_PATH_SPLIT           large budgets: filter, finish, and the split FAC
 *                             with its merge.
 * No device work.  Errors: as fasa_workspace_size (FASA_ERR_INVALID_ARG for a
 * NULL path). */
enum {
  FASA_PATH_NONE = 0,
  FASA_PATH_LISTS = 1,
  FASA_PATH_FILTERED_LISTS = 2,
  FASA_PATH_FILTER = 3,
  FASA_PATH_SPLIT = 4
};
fasa_status fasa_decode_path(const fasa_shape* shape, int32_t max_t, int32_t* path);

/* ---- FASA-M: the memory-optimised placement (section 3.4, "Hardware-Aware
 * Variants", FASA-M and Equation 10).  The GPU keeps only the dominant-key
 * cache (the slab) and per-step buffers; the non-dominant key columns and all
 * value rows live in pinned host memory, which the GPU reads directly after
 * the selection.  Host arrays (element type = the cache type), indexed by the
 * pool's physical block like the pool and the slab:
 *   k_nd [block][n_kv_heads][256][nd]: the 128 - 2*n_fc non-dominant key
 *        columns of every token, ascending, each row zero-padded to nd
 *        elements, nd = (128 - 2*n_fc) rounded up to a multiple of 16 bytes;
 *   v    [block][n_kv_heads][256][128]: the value rows.
 * Both must be page-locked host memory known to the HIP runtime (hipHostMalloc,
 * or a pinned torch tensor) and 16-byte aligned; anything else is
 * FASA_ERR_INVALID_ARG.  The caller owns them. */

/* Bytes of the two host arrays for a pool of n_blocks physical blocks. */
fasa_status fasa_m_host_sizes(const fasa_shape* shape, int64_t n_blocks, size_t* k_nd_bytes,
                              size_t* v_bytes);

/* Copy blocks 0 .. ceil(t_b/256)-1 of every sequence from the device pools
 * (post-RoPE keys, values) into the host arrays: the offload after prefill.
 * Whole blocks are copied; blocks past a sequence's end are left untouched.
 * The slab (fasa_slab_build) holds the dominant columns. */
fasa_status fasa_m_offload(const fasa_shape* shape, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* fc_idx, void* k_nd_host, void* v_host,
                           hipStream_t stream);

/* Workspace of fasa_m_decode and its stages: fasa_workspace_size's layout plus
 * two row areas, each two staging arrays of batch * n_kv_heads * cap rows of
 * 128 elements (K and V). */
fasa_status fasa_m_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes);

/* One FASA-M decode step: TIP on the slab, the exact top-B (sel_idx and
 * sel_count are outputs, as in fasa_decode), then the selected rows' key
 * (non-dominant columns from k_nd, dominant pairs from the slab) and value
 * rows are rebuilt into the workspace's staging arrays, and FAC runs over
 * them.  Same selection and the same FAC arithmetic as fasa_decode, so the
 * same results up to the order of the softmax sums; the device never reads
 * the full-cache K/V pools. */
fasa_status fasa_m_decode(const fasa_shape* shape, const void* q, const void* slab,
                          const void* k_nd_host, const void* v_host, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t max_t, const int32_t* fc_idx,
                          float* out, int32_t* sel_idx, int32_t* sel_count, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* FASA-M with the previous query's rows loaded in advance (section 3.4,
 * "Hardware-Aware Variants", the mitigation of FASA-M's CPU-GPU transfer
 * latency: the keys and values that the previous query needed are loaded
 * asynchronously, in advance, so that TIP overlaps the transfer).
 * fasa_m_decode in two stages around a pair of row areas in the workspace; a
 * step of parity p (0 or 1; consecutive steps alternate) stages its selected
 * rows in area p and takes every row whose token the previous selection also
 * holds from area 1 - p, so that only the others cross the host link:
 *   fasa_m_decode_select: TIP, then the exact top-B into sel_idx / sel_count;
 *   fasa_m_decode_finish: after it, the selected rows into area `parity` --
 *     from area 1 - parity where the token is in prev_sel_idx, from the host
 *     otherwise -- then FAC into out.  prev_sel_idx / prev_sel_count (laid out
 *     as sel_idx / sel_count) must be the selection whose rows area 1 - parity
 *     holds; pass NULL for both to take every row from the host (hits must
 *     then be NULL).  hits (nullable, int32 [batch][n_kv_heads]) is
 *     incremented by the rows taken from area 1 - parity.  Rows are reused
 *     only when cap <= 8192; above that every row comes from the host.
 *   Area 1 - parity holds the previous selection's rows when the previous
 *   step ran fasa_m_decode_finish with parity 1 - parity on this workspace
 *   (a workspace kept per layer: nothing crosses the link for those rows), or
 *   after fasa_m_prefetch:
 *   fasa_m_prefetch: the rows of prev_sel_idx / prev_sel_count rebuilt from
 *     the host arrays and the slab into area 1 - parity, for a step of parity
 *     `parity` (a workspace shared by several layers).  It touches nothing else
 *     of the workspace, so it may run on a second stream concurrently with
 *     fasa_m_decode_select on the same workspace.
 * The results (sel_idx, sel_count, out) equal fasa_m_decode's bit for bit,
 * whatever the previous selection was.  Order: fasa_m_prefetch and
 * fasa_m_decode_select after the previous step's finish; the finish after
 * both.  fasa_m_decode itself stages in area 0. */
fasa_status fasa_m_decode_select(const fasa_shape* shape, const void* q, const void* slab,
                                 const int32_t* block_table, const int32_t* seq_lens, int32_t max_t,
                                 const int32_t* fc_idx, int32_t* sel_idx, int32_t* sel_count,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
fasa_status fasa_m_prefetch(const fasa_shape* shape, const void* slab, const void* k_nd_host,
                            const void* v_host, const int32_t* block_table, int32_t max_t,
                            const int32_t* fc_idx, const int32_t* prev_sel_idx,
                            const int32_t* prev_sel_count, int32_t parity, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
fasa_status fasa_m_decode_finish(const fasa_shape* shape, const void* q, const void* slab,
                                 const void* k_nd_host, const void* v_host, const int32_t* block_table,
                                 int32_t max_t, const int32_t* fc_idx, const int32_t* prev_sel_idx,
                                 const int32_t* prev_sel_count, const int32_t* sel_idx,
                                 const int32_t* sel_count, int32_t parity, float* out, int32_t* hits,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Offline calibration: Contextual Agreement (section 3.4, the CA metric
 * and the offline calibration).  A calibration row is one decode query
 * (sequence b, its query at position t_b) against the keys 0..t_b-1 of the
 * paged cache; several steps of one calibration sample are several sequences
 * whose block tables share their prefix blocks.  Per kv head, the group's
 * queries are summed per column (as TIP scores them). */

/* Workspace of fasa_ca_hits: the 65 score rows of every (sequence, kv head)
 * and the exact top-K state for them.  1 <= k_top <= 4096. */
fasa_status fasa_ca_workspace_size(const fasa_shape* shape, int32_t max_t, int32_t k_top,
                                   size_t* bytes);

/* hits[b][g][i] (int32, [batch][n_kv_heads][64]) = the size of the
 * intersection of TopK-I(alpha, K) and TopK-I(alpha^(i), K), where alpha_j is
 * the full q.k_j score and alpha^(i)_j the score of FC i alone, over tokens
 * j < t_b; CA of FC i is hits / k_top (section 3.4, the CA metric, Eq. 4).
 * TopK-I takes the largest values, the lower index on ties, and every token
 * when t_b < k_top.  The scores are float32 in one fixed order without fused
 * multiply-adds (the group's heads summed in head order; each FC as
 * fl(fl(q x k) + fl(q x k)); alpha as the 64 FC terms added in FC order), so
 * the sets are reproducible bit for bit.  topk (nullable, int32,
 * [batch][n_kv_heads][65][min(k_top, max_t)]) receives the lists behind the
 * counts: row 0 is TopK-I(alpha), row 1 + i TopK-I(alpha^(i)), each ascending
 * and padded with -1.  fc_idx, budget, n_sink and n_recent are not used. */
fasa_status fasa_ca_hits(const fasa_shape* shape, const void* q, const void* k_pool,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t max_t,
                         int32_t k_top, int32_t* hits, int32_t* topk, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* The dominant FCs from n_rows calibration rows of hits ([n_rows][n_kv_heads][64]):
 * per kv head, the n_tip FCs with the largest total hits (the largest mean
 * CA), the lower FC index on ties, written ascending to fc_idx
 * [n_kv_heads][n_tip] -- a valid fc_idx for the other entry points when
 * n_tip == n_fc.  1 <= n_tip <= 64. */
fasa_status fasa_ca_dominant(const fasa_shape* shape, const int32_t* hits, int32_t n_rows,
                             int32_t n_tip, int32_t* fc_idx, hipStream_t stream);

/* Bytes of workspace that fasa_dense_decode needs for contexts up to max_t:
 * the split partials, about 4 * (128 + 2) bytes per query head per 512 tokens
 * of max_t (fp32 caches: twice that).  256-byte aligned; contents are
 * scratch. */
fasa_status fasa_dense_workspace_size(const fasa_shape* shape, int32_t max_t, size_t* bytes);

/* Full attention over every cached token, the dense decode that FASA replaces:
 * out[b][h] = softmax(q_h K^T * scale) V over tokens 0..t_b-1 of kv head g(h)
 * (the full-KV reference of the review's experimental section, and the
 * standard attention whose 2*t*d loaded elements Equation 8 of section 3.4,
 * "Hardware-Aware Variants", compares with).  It is FAC with the selection
 * "every token": same kernels, same per-row arithmetic and precision as
 * fasa_fac.  Reads q, k_pool, v_pool, block_table, seq_lens (t_b is clamped
 * into [0, max_t]); writes out [batch][n_q_heads][128] fp32 (zeros for
 * t_b == 0).  fc_idx, budget, n_sink and n_recent are not used. */
fasa_status fasa_dense_decode(const fasa_shape* shape, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t max_t, float* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- Allocation-free decode, for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it).
 * fasa_decode_scratch is fasa_decode with the workspace taken from a fixed
 * device array that the library owns: fasa_scratch_capacity() bytes (64 MiB)
 * on every device the library runs on, held until the process ends.  The
 * caller passes inputs and outputs only; nothing is allocated or freed.  A call
 * whose fasa_workspace_size exceeds the capacity returns FASA_ERR_SCRATCH
 * before anything is enqueued.  The stream must belong to the current device
 * (FASA_ERR_INVALID_ARG otherwise).  All calls on one device share its array:
 * calls that may overlap (unordered streams) race and must not be issued;
 * calls ordered on one stream are safe.  Results equal fasa_decode's. */
size_t fasa_scratch_capacity(void);
fasa_status fasa_decode_scratch(const fasa_shape* shape, const void* q, const void* k_pool,
                                const void* v_pool, const void* slab, const int32_t* block_table,
                                const int32_t* seq_lens, int32_t max_t, const int32_t* fc_idx,
                                float* out, int32_t* sel_idx, int32_t* sel_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FASA_H */
