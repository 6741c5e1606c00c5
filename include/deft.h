/*
 * deft.h - C ABI of libdeft: DeFT-style tree attention for one decode step on
 * one AMD Instinct MI355X (gfx950).
 *
 * A decode step's queries each sit on a node of a prefix tree whose nodes own
 * KV segments; a query attends to the KV of its node and of all the node's
 * ancestors.  Sources (the DeFT pages: arXiv 2404.00242, abstract, and "DeFT
 * Guide: Flash Tree-Attention for LLM Serving"):
 *   - the result: "Tree-Constrained Attention Formulation" (masked softmax
 *     over prefix and ancestor tokens, scale 1/sqrt(d));
 *   - KV-Guided Grouping: each KV chunk is read once for every query that
 *     needs it ("1. KV-Guided Grouping");
 *   - Flattened Tree KV Splitting: the tree's KV is laid out as one linear
 *     index space cut into equal token chunks ("2. Flattened Tree KV
 *     Splitting");
 *   - per-chunk partials with a running max m and sum l, combined by the
 *     online-softmax rule ("The Online Softmax Tile Accumulation");
 *   - paged KV: flattened indices map onto non-contiguous pages through a
 *     block table ("Integration with Paged KV Caches", "2. Paged KV-Cache
 *     Compatibility").
 *
 * Conventions for every call:
 *   - integers are int32 unless stated; arrays are contiguous and row-major;
 *   - "host" pointers are ordinary CPU memory, "device" pointers are HIP
 *     device memory of the current device;
 *   - streams are hipStream_t passed as void* (NULL = the null stream);
 *   - every device-side call is asynchronous on its stream and never
 *     synchronises the host, with the exceptions each call states
 *     (deft_plan_upload and deft_plan_destroy wait for the plan's previous
 *     upload copy; DEFT_VALIDATE=1 synchronises the attention calls);
 *   - the library never allocates device memory: plan images, workspaces,
 *     KV pools and outputs all belong to the caller;
 *   - a call returns DEFT_OK or a negative code; deft_last_error() then
 *     describes the failure (per thread).  Nothing aborts or throws across
 *     this boundary.
 *
 * Tree encoding (borrowed, read during the call only):
 *   parents[i]     parent of node i, or -1 for a root; must lie in [-1, i)
 *                  (a forest is allowed)
 *   seg_lens[i]    KV tokens owned by node i, >= 1
 *   query_nodes[q] node that query q sits on (several queries may share a
 *                  node; internal nodes are allowed)
 * Logical KV order: node segments concatenated in node-id order, so node i
 * owns logical tokens [node_start[i], node_start[i] + seg_lens[i]) with
 * node_start the exclusive prefix sum of seg_lens.
 *
 * Tensor layouts:
 *   q, out        [num_queries][num_q_heads][head_dim], dtype of desc
 *   k_cache,      [num_pages][page_size][num_kv_heads][head_dim], dtype of desc;
 *   v_cache       logical token t is at page block_table[t / page_size],
 *                 row t % page_size
 *   block_table   [ceil(total_tokens / page_size)] int32 physical page ids
 *   query head h reads KV head h / (num_q_heads / num_kv_heads)
 *   scale 1/sqrt(head_dim); output is the exact softmax-weighted mean of V,
 *   rounded to the output dtype (round to nearest even for bf16).
 */
#ifndef DEFT_H
#define DEFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DEFT_OK                     0
#define DEFT_ERR_INVALID_ARGUMENT  -1  /* null pointer, bad count, buffer too small, plan/desc mismatch */
#define DEFT_ERR_INVALID_TREE      -2  /* parents/seg_lens/query_nodes break the encoding above */
#define DEFT_ERR_UNSUPPORTED       -3  /* valid request outside what the kernels implement */
#define DEFT_ERR_HIP               -4  /* a HIP call or kernel launch failed */
#define DEFT_ERR_NO_MEMORY         -5  /* host allocation failed */

/* Element types of q, k_cache, v_cache and out. */
#define DEFT_DTYPE_F32   0
#define DEFT_DTYPE_BF16  1

/* Formats of the per-slot partial O (see deft_partial_attention). */
#define DEFT_PARTIAL_F32        0  /* fp32, unnormalised: sum exp(s - m) v */
#define DEFT_PARTIAL_BF16_NORM  1  /* bf16, divided by l: the softmax-weighted mean over the slot */

typedef struct deft_plan deft_plan;   /* opaque, host-owned */

/*
 * Read-only view of a plan's arrays (host memory owned by the plan, valid
 * until deft_plan_destroy).  Definitions, with T = total_tokens, C =
 * chunk_tokens, W = mask_words = ceil(C / 32), S = num_slots:
 *   node_start[N]          logical start of each node's segment
 *   flat_node_order[N]     depth-first pre-order of the nodes: roots in
 *                          ascending id, then each node's children in
 *                          ascending id (the flattened index space of
 *                          "2. Flattened Tree KV Splitting")
 *   node_flat_start[N]     flat index of each node's first token
 *   flat_to_logical[T]     logical token stored at each flat index
 *   chunk_start[nc+1]      chunk c covers flat [c*C, min((c+1)*C, T))
 *   group_offsets[nc+1]    CSR over chunks into slot_query
 *   slot_query[S]          the query of each (chunk, query) slot: per chunk,
 *                          the queries that see >= 1 of its tokens, in
 *                          ascending query index ("1. KV-Guided Grouping")
 *   slot_mask[S*W]         bit (t & 31) of word (t >> 5) of a slot's row is set
 *                          iff the chunk's t-th token lies on the query's
 *                          root-to-node path; bits at t >= chunk length are 0
 *   chunk_full[nc]         1 iff the chunk has slots and all their bits are set
 *   query_slot_offsets[Nq+1], query_slots[S]
 *                          each query's slots in ascending chunk order (the
 *                          operands of its log-sum-exp merge)
 */
typedef struct {
  int32_t num_nodes;
  int32_t num_queries;
  int32_t chunk_tokens;
  int32_t total_tokens;
  int32_t num_chunks;
  int32_t num_slots;
  int32_t mask_words;
  const int32_t*  node_start;
  const int32_t*  flat_node_order;
  const int32_t*  node_flat_start;
  const int32_t*  flat_to_logical;
  const int32_t*  chunk_start;
  const int32_t*  group_offsets;
  const int32_t*  slot_query;
  const uint32_t* slot_mask;
  const uint8_t*  chunk_full;
  const int32_t*  query_slot_offsets;
  const int32_t*  query_slots;
} deft_plan_view;

/* Shapes of one attention call. */
typedef struct {
  int32_t dtype;         /* DEFT_DTYPE_F32 or DEFT_DTYPE_BF16 */
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t page_size;     /* tokens per KV page: 16 */
  int32_t num_pages;     /* pages in k_cache and v_cache (each) */
  int32_t f32_partials;  /* 0: the workspace holds each dtype's internal partial format (bf16 O / l
                            for bf16 inputs, fp32 unnormalised O for fp32); 1: fp32 unnormalised
                            O for every dtype (twice the partial bytes for bf16, no rounding of
                            the per-slot results before the merge) */
} deft_attn_desc;

/*
 * Build a plan on the host (flattening, chunking, grouping, bitmasks, merge
 * lists).  The tree arrays are host pointers read during the call only.
 * chunk_tokens >= 1 (the attention calls support chunk_tokens <= 4096).
 * Errors: INVALID_ARGUMENT for null pointers, num_nodes < 1,
 * num_queries < 1 or chunk_tokens < 1; INVALID_TREE for parents[i] outside
 * [-1, i), seg_lens[i] < 1, query_nodes[q] outside [0, num_nodes), or more
 * than 2^31 - 1 tokens in total; UNSUPPORTED for more than 2^31 - 1
 * (chunk, query) slots; NO_MEMORY.  *out_plan is set on success.
 */
int deft_plan_create(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                     const int32_t* query_nodes, int32_t num_queries, int32_t chunk_tokens,
                     deft_plan** out_plan);

/*
 * Query-centric baseline plan, for measuring what KV-Guided Grouping saves
 * on the same hardware (the pages contrast DeFT with per-query attention
 * that reloads the shared prefix for every query: abstract; Guide, "The
 * Tree-Attention Bottleneck: Redundant Memory IO and Severe Load
 * Imbalances", "1. Massive Redundant Memory Access (IO)").  Same arguments and errors as
 * deft_plan_create (plus INVALID_TREE if the summed path lengths exceed
 * 2^31 - 1).  Each query's root-to-node path tokens (root segment first, each
 * segment in order) form their own run of the flat index space, queries in
 * order; each run is cut into chunk_tokens windows from its start and every
 * chunk has exactly one slot, its query, with all bits set, so the attention
 * calls stream every query's whole path by itself.  In the view,
 * total_tokens is the summed path length and flat_to_logical maps that
 * space; node_start, flat_node_order and node_flat_start are those of
 * deft_plan_create.  Results of the attention calls are those of the tree
 * plan up to rounding.
 */
int deft_plan_create_query_centric(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                   const int32_t* query_nodes, int32_t num_queries,
                                   int32_t chunk_tokens, deft_plan** out_plan);

/*
 * Node-granularity plan, the ablation of Flattened Tree KV Splitting (the
 * Guide's "2. Flattened Tree KV Splitting" sets its equal flat chunks against
 * node-sized work units): the same depth-first flat layout as
 * deft_plan_create, but every node's segment is cut into chunk_tokens
 * windows from its own start, so no chunk crosses a node boundary and only
 * nodes longer than chunk_tokens are split.  A chunk's group is every query
 * whose root-to-node path holds the chunk's node (ascending), each slot with
 * all of the chunk's bits set; chunk_full is 1 for every chunk with a group.
 * Same arguments and errors as deft_plan_create; results of the attention
 * calls are those of the tree plan up to rounding.
 */
int deft_plan_create_node_chunks(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                 const int32_t* query_nodes, int32_t num_queries, int32_t chunk_tokens,
                                 deft_plan** out_plan);

/*
 * Tree plan with multi-token query nodes (tree prefill, speculative nodes
 * holding several draft tokens).  The pages' mask (DeFT Guide, "Deep Dive:
 * Mathematical Formulation", "Tree-Constrained Attention Formulation") is
 * defined by ancestry alone; the causal rule inside one node is a reading
 * that keeps ordinary causal attention along a chain: query q sits at a
 * position inside its node and sees its ancestors' segments plus the first
 * query_lens[q] tokens of its own node (it sees its own token).  Grouping,
 * flattening and chunking are those of deft_plan_create; a chunk's group
 * holds only the queries that see at least one of its tokens.
 *   query_lens  host int32 [num_queries], each in [1, seg_lens[query_nodes[q]]];
 *               NULL means the whole segment (exactly deft_plan_create).
 * Errors: those of deft_plan_create; DEFT_ERR_INVALID_TREE for a query_lens
 * entry outside its range.
 */
int deft_plan_create_multi_token(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                 const int32_t* query_nodes, const int32_t* query_lens,
                                 int32_t num_queries, int32_t chunk_tokens, deft_plan** out_plan);

/*
 * Chunk size for deft_plan_create (or deft_plan_create_multi_token, with
 * query_lens; NULL means whole nodes) chosen by one rule: the smallest
 * multiple of 32 tokens, up to 4096, for which the partial-attention kernel
 * of this tree under `desc` has at most `num_cus` work-groups, so every chunk
 * of every KV head runs in one round on a device of num_cus compute units
 * (one work-group per compute unit); 4096 when even that needs more rounds
 * (long chunks then amortise each work-group's fixed cost).  Work-groups are
 * counted as items of 64 rows for bf16 groups of 16 or more rows and of 8
 * rows otherwise, times num_kv_heads, from each chunk's group size ("2.
 * Flattened Tree KV Splitting" cuts the flat token space into equal chunks;
 * "1. KV-Guided Grouping" gives each chunk one group).  num_cus = 0 takes the
 * current device's count (256 when it cannot be queried).
 * *out_chunk_tokens is set on success.  Errors: those of deft_plan_create for
 * the tree arrays, INVALID_ARGUMENT for a NULL out pointer or num_cus < 0,
 * and the desc errors of deft_plan_device_bytes.
 */
int deft_plan_auto_chunk_tokens(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                const int32_t* query_nodes, const int32_t* query_lens, int32_t num_queries,
                                const deft_attn_desc* desc, int32_t num_cus, int32_t* out_chunk_tokens);

/* Free a plan (NULL is ignored); waits for its last upload's copy to have
 * run.  The caller must first let every stream that consumes its device
 * image get past that work (the image is caller memory and stays). */
void deft_plan_destroy(deft_plan* plan);

/* Fill *out_view with the plan's arrays (see deft_plan_view). */
int deft_plan_export(const deft_plan* plan, deft_plan_view* out_view);

/*
 * Sizes the caller must allocate for a given attention shape:
 *   *plan_bytes       device image of the plan (deft_plan_upload)
 *   *workspace_bytes  per-slot partial results of deft_tree_attention: part_o
 *                     in the format desc->f32_partials selects, then part_m
 *                     and part_l, each padded to 256 bytes
 * Either output pointer may be NULL.  UNSUPPORTED if desc is outside this
 * build (head_dim not 64/128, page_size != 16, Hq % Hkv != 0, chunk_tokens
 * > 4096), if num_queries * num_q_heads reaches 2^28, or if the work items
 * times num_kv_heads exceed 2^23 - 1 (one launch's grid; a larger
 * chunk_tokens makes fewer items); INVALID_ARGUMENT for non-positive shapes
 * or f32_partials other than 0 and 1.
 */
int deft_plan_device_bytes(deft_plan* plan, const deft_attn_desc* desc,
                           size_t* plan_bytes, size_t* workspace_bytes);

/*
 * Build the plan's device image for desc (chunk metadata, masks, the
 * flattened-to-logical map, merge lists and the kernels' work lists) and copy
 * it into dev_plan (device memory of at least plan_bytes, 256-byte aligned)
 * on `stream`.  The plan remembers dev_plan and desc; later attention calls
 * read the image from there.  The copy's source is a host staging buffer
 * owned by the plan: a later upload of the same plan, and deft_plan_destroy,
 * first wait (on the host) for the previous copy to have run, so the caller
 * need not synchronise for it.  The copy is from pageable memory: not for
 * use under stream capture.
 */
int deft_plan_upload(deft_plan* plan, const deft_attn_desc* desc, void* dev_plan,
                     size_t dev_plan_bytes, void* stream);

/*
 * Tree attention for one decode step: the partial-attention kernel (every
 * chunk's KV streamed once per KV head for all its grouped queries and their
 * query heads, bitmask applied, per-slot partials written to the workspace in
 * format DEFT_PARTIAL_BF16_NORM for bf16 inputs, DEFT_PARTIAL_F32 for fp32
 * inputs or when desc->f32_partials is 1) followed by the log-sum-exp merge
 * kernel.  q, k_cache, v_cache, block_table, out, workspace: device pointers.
 * desc must equal the desc of the last deft_plan_upload (f32_partials aside:
 * the image does not depend on it, so each call may choose).  workspace_bytes
 * must be at least the size from deft_plan_device_bytes.  block_table
 * entries are not range-checked on the device; an entry outside
 * [0, num_pages) is undefined behaviour.  With the environment variable
 * DEFT_VALIDATE=1, this call, deft_tree_attention_fused and
 * deft_partial_attention first copy the entries of the tree's logical pages
 * to the host on `stream` and synchronise it (so not under graph capture),
 * and return DEFT_ERR_INVALID_ARGUMENT, launching nothing, if one is out of
 * range.
 */
/*
 * Work items (deft_plan_device_bytes, deft_plan_upload): bf16 groups of 16
 * or more rows take the matrix-core kernel in items of 64 rows, or of 128
 * rows for groups of more than 64 when the 64-row items would fill the
 * current device's compute units at least twice (each chunk is then streamed
 * by half as many work-groups).  DEFT_MFMA_WIDE=1 or 0 in the environment
 * forces 128-row items on or off (tests); the choice is made at upload.
 */
int deft_tree_attention(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_table, const deft_plan* plan, void* out,
                        const deft_attn_desc* desc, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * deft_tree_attention in one dispatch per partial kernel: the per-chunk
 * partials are merged by the partial kernel itself instead of a second
 * kernel (the Guide's "3. Fused In-SRAM Online Softmax Merging" describes
 * merging partial results where they are produced; "The Online Softmax Tile
 * Accumulation" gives the rule).  Unlike that description, partials still
 * pass through memory: the workspace holds them as for deft_tree_attention
 * (4.46 MB written and read back on the 4K-prefix / 64-node tree), because
 * the chunks of one query run on different compute units.  The one grid
 * holds the partial work-groups followed by merge work-groups (16 (query,
 * head) rows each while that needs at most 128 of them, else 32).  A
 * partial work-group writes its partials with
 * device-coherent stores, waits for them, and adds one to a device-scope
 * ticket per (query, head) row it wrote; a merge work-group waits until its
 * rows' tickets count every slot of their query, subtracts that count,
 * merges the rows and writes `out`.  Its wait is bounded (as deft_plan_status
 * describes): past the limit it reports a give-up and merges what it finds.
 * The tickets live in the plan's device image (zero after upload and after
 * every completed call), so calls that share a plan must not overlap and the
 * plan is not const here.  Arguments, layouts, workspace and errors as for
 * deft_tree_attention; results are bitwise equal to it.
 */
int deft_tree_attention_fused(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, deft_plan* plan, void* out,
                              const deft_attn_desc* desc, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Whether the attention calls on this plan since the last check ran
 * correctly.  The matrix-core partial kernels synchronise the waves that
 * share an LDS ring through flags with a bounded wait (2^20 checks, about
 * 30 ms; DEFT_SPIN_LIMIT in the environment lowers it, for tests), and the
 * merge work-groups of deft_tree_attention_fused wait for their rows'
 * tickets with the same number of checks (each a device-scope load, so
 * about a second); a wait that runs out never hangs the GPU but leaves that
 * work-group's results invalid, and sets a status word in the plan's device
 * image.  This call
 * copies that word to the host on `stream`, synchronises the stream, and
 * returns DEFT_ERR_HIP (with a message) if it was set, clearing it; else
 * DEFT_OK.  INVALID_ARGUMENT if the plan is NULL or has no device image.
 * It synchronises, so it is meant for periodic checks and tests, not for
 * every step or for graph capture.
 */
int deft_plan_status(deft_plan* plan, void* stream);

/*
 * Size of the device scratch that deft_tree_attention_noalloc uses for the
 * partial results (one copy per GPU the library runs on, held until the
 * process ends).
 */
#define DEFT_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * deft_tree_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same two kernels and results, bit for bit, but the
 * per-slot partials go to a library-owned device scratch of
 * DEFT_NOALLOC_SCRATCH_BYTES instead of a caller workspace, and the call
 * allocates nothing.  The caller still passes q, the KV pool, block_table,
 * the uploaded plan and out (device pointers, layouts as for
 * deft_tree_attention).  The scratch's device address is looked up on the
 * first call on each device (with that device current) and kept.  Every
 * call on one GPU shares that GPU's scratch, so calls that overlap on one
 * GPU (on different streams, or from several threads) race and must be
 * ordered by the caller; nothing in the scratch needs to start at zero.
 * DEFT_VALIDATE is not honoured here (that check copies to host memory and
 * synchronises).  Errors: those of deft_tree_attention, and
 * DEFT_ERR_UNSUPPORTED when the plan's workspace size (deft_plan_device_bytes)
 * exceeds DEFT_NOALLOC_SCRATCH_BYTES (a larger chunk_tokens means fewer
 * slots), before anything is launched.
 */
int deft_tree_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const deft_plan* plan, void* out,
                                const deft_attn_desc* desc, void* stream);

/*
 * The partial-attention kernel on its own ("The Online Softmax Tile
 * Accumulation" applied per chunk).  For every slot s (chunk c, query q) and
 * query head h, over the chunk's tokens visible to q:
 *   part_m[s*Hq + h]          max of the scaled scores (natural-log domain)
 *   part_l[s*Hq + h]          sum of exp(score - m)
 *   part_o[(s*Hq + h)*d + e]  partial_format DEFT_PARTIAL_F32: fp32
 *                             sum of exp(score - m) * v[e] (unnormalised);
 *                             DEFT_PARTIAL_BF16_NORM: that sum divided by l,
 *                             rounded to bf16 (bf16 inputs only; this is the
 *                             format deft_tree_attention uses for them)
 * part_m and part_l are fp32 arrays of S*Hq floats, part_o holds S*Hq*d
 * elements of the chosen format; all device pointers.
 */
int deft_partial_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const deft_plan* plan,
                           const deft_attn_desc* desc, void* part_o, float* part_m,
                           float* part_l, int32_t partial_format, void* stream);

/*
 * The merge kernel on its own: for every query q and head h, over q's slots
 * M = max m_s, L = sum l_s exp(m_s - M), out = sum o_s exp(m_s - M) / L
 * (with bf16-normalised partials: out = sum l_s exp(m_s - M) o_s / L),
 * rounded to desc->dtype.  Partials in the layout of deft_partial_attention.
 */
int deft_lse_merge(const deft_plan* plan, const deft_attn_desc* desc, const void* part_o,
                   const float* part_m, const float* part_l, int32_t partial_format, void* out,
                   void* stream);

/* Message for the calling thread's last failed call ("" if none). */
const char* deft_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DEFT_H */
