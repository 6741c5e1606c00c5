// Host tree planner: Flattened Tree KV Splitting and KV-Guided Grouping.
//
// Sources (DeFT, arXiv 2404.00242, abstract; "DeFT Guide: Flash Tree-Attention
// for LLM Serving", sections "1. KV-Guided Grouping", "2. Flattened Tree KV
// Splitting", "Tree-Constrained Attention Formulation").  The tree's KV is
// laid out in one linear (flat) index space, cut into equal chunks of
// chunk_tokens, and for every chunk the queries that need any of its tokens
// form one group, so the chunk is loaded once for all of them.  Readings
// where the pages leave the details open:
//   - flat order is a depth-first pre-order, roots and children by ascending
//     id, so every subtree (and every node's segment) is one flat interval;
//   - chunks are fixed windows from flat index 0 and may cross node
//     boundaries; only the last one may be short;
//   - a chunk's group is every query that sees at least one of its tokens,
//     in ascending query index; one "slot" per (chunk, query);
//   - bit t of a slot's mask row is set iff the chunk's t-th token belongs to
//     a node on the query's root-to-node path (its own node included).
//
// Method: a query's visible tokens are the segments of its path nodes, and
// in pre-order those segments appear at increasing flat positions.  Walking
// each path from the root down therefore touches chunks in ascending order,
// which yields the groups, the per-query merge lists and the mask bit runs
// in one pass over the paths, with no per-token visibility test.

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>

#include "deft_internal.h"

namespace deft {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

// Depth-first pre-order of the nodes (roots, then each node's children, in
// ascending id) and the flat index of each node's first token.
static void flatten(const int32_t* parents, const int32_t* seg_lens, int32_t n, std::vector<int32_t>* order,
                    std::vector<int32_t>* flat_start) {
  // Children in CSR form; filling in ascending i keeps each list ascending.
  std::vector<int32_t> child_off(n + 1, 0), child(n), roots;
  for (int32_t i = 0; i < n; ++i) {
    if (parents[i] < 0) roots.push_back(i); else child_off[parents[i] + 1]++;
  }
  for (int32_t i = 0; i < n; ++i) child_off[i + 1] += child_off[i];
  {
    std::vector<int32_t> fill(child_off.begin(), child_off.end() - 1);
    for (int32_t i = 0; i < n; ++i)
      if (parents[i] >= 0) child[fill[parents[i]]++] = i;
  }
  // Explicit stack (push in reverse to pop ascending).
  order->clear();
  order->reserve(n);
  std::vector<int32_t> stack(roots.rbegin(), roots.rend());
  while (!stack.empty()) {
    int32_t x = stack.back();
    stack.pop_back();
    order->push_back(x);
    for (int32_t k = child_off[x + 1] - 1; k >= child_off[x]; --k) stack.push_back(child[k]);
  }
  flat_start->resize(n);
  int64_t f = 0;
  for (int32_t x : *order) {
    (*flat_start)[x] = static_cast<int32_t>(f);
    f += seg_lens[x];
  }
}

// The tree encoding's checks shared by every entry point that takes a tree.
static int validate_tree(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                         const int32_t* query_nodes, int32_t num_queries, const int32_t* query_lens) {
  if (num_nodes < 1 || num_queries < 1)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "need at least one node and one query");
  if (!parents || !seg_lens || !query_nodes)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "tree arrays must not be NULL");
  for (int32_t i = 0; i < num_nodes; ++i) {
    if (parents[i] < -1 || parents[i] >= i)
      return fail(DEFT_ERR_INVALID_TREE,
                  "parents[" + std::to_string(i) + "] must be -1 or in [0, " + std::to_string(i) + ")");
    if (seg_lens[i] < 1)
      return fail(DEFT_ERR_INVALID_TREE, "seg_lens[" + std::to_string(i) + "] must be >= 1");
  }
  for (int32_t q = 0; q < num_queries; ++q)
    if (query_nodes[q] < 0 || query_nodes[q] >= num_nodes)
      return fail(DEFT_ERR_INVALID_TREE, "query_nodes[" + std::to_string(q) + "] out of range");
  if (query_lens)
    for (int32_t q = 0; q < num_queries; ++q)
      if (query_lens[q] < 1 || query_lens[q] > seg_lens[query_nodes[q]])
        return fail(DEFT_ERR_INVALID_TREE, "query_lens[" + std::to_string(q) + "] must be in [1, seg_lens[node]]");
  int64_t total = 0;
  for (int32_t i = 0; i < num_nodes; ++i) total += seg_lens[i];
  if (total > INT32_MAX) return fail(DEFT_ERR_INVALID_TREE, "total tokens exceed 2^31 - 1");
  return DEFT_OK;
}

// query_lens (may be null): leading tokens of its own node each query sees.
static int build_plan(deft_plan* p, const int32_t* parents, const int32_t* seg_lens,
                      int32_t n, const int32_t* query_nodes, int32_t nq, int32_t c,
                      const int32_t* query_lens = nullptr) {
  // Logical layout: segments in node-id order.
  p->node_start.resize(n);
  int64_t run = 0;
  for (int32_t i = 0; i < n; ++i) {
    p->node_start[i] = static_cast<int32_t>(run);
    run += seg_lens[i];
  }
  const int32_t total = static_cast<int32_t>(run);

  flatten(parents, seg_lens, n, &p->flat_node_order, &p->node_flat_start);
  p->flat_to_logical.resize(total);
  for (int32_t x : p->flat_node_order)
    for (int32_t i = 0; i < seg_lens[x]; ++i) p->flat_to_logical[p->node_flat_start[x] + i] = p->node_start[x] + i;

  // Equal chunks from flat index 0.
  const int32_t nc = static_cast<int32_t>((static_cast<int64_t>(total) + c - 1) / c);
  p->chunk_start.resize(nc + 1);
  for (int32_t k = 0; k <= nc; ++k)
    p->chunk_start[k] = static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(k) * c, total));
  const int32_t words = (c + 31) / 32;

  // Pass 1: for every query (ascending), the chunks its path touches, in
  // ascending chunk order; a query's position inside each chunk's group is
  // the number of lower queries already placed there.
  std::vector<int32_t> group_count(nc, 0);
  std::vector<int32_t> touch_off(nq + 1, 0);
  std::vector<int32_t> touch_chunk, touch_pos;
  std::vector<int32_t> path;
  for (int32_t q = 0; q < nq; ++q) {
    path.clear();
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) path.push_back(x);
    int32_t last = -1;
    for (auto it = path.rbegin(); it != path.rend(); ++it) {
      const int64_t a = p->node_flat_start[*it];
      const int64_t b = a + (query_lens && *it == query_nodes[q] ? query_lens[q] : seg_lens[*it]);
      for (int64_t k = a / c; k <= (b - 1) / c; ++k) {
        if (static_cast<int32_t>(k) == last) continue;
        last = static_cast<int32_t>(k);
        touch_chunk.push_back(last);
        touch_pos.push_back(group_count[last]++);
      }
    }
    if (touch_chunk.size() > static_cast<size_t>(INT32_MAX))
      return fail(DEFT_ERR_UNSUPPORTED, "more than 2^31 - 1 (chunk, query) slots");
    touch_off[q + 1] = static_cast<int32_t>(touch_chunk.size());
  }
  p->group_offsets.assign(nc + 1, 0);
  for (int32_t k = 0; k < nc; ++k) p->group_offsets[k + 1] = p->group_offsets[k] + group_count[k];
  const int32_t S = p->group_offsets[nc];

  // Pass 2: slots, merge lists, mask bit runs.
  p->slot_query.assign(S, 0);
  p->slot_mask.assign(static_cast<size_t>(S) * words, 0u);
  p->query_slot_offsets.assign(touch_off.begin(), touch_off.end());
  p->query_slots.assign(S, 0);
  std::vector<int64_t> slot_bits(S, 0);
  for (int32_t q = 0; q < nq; ++q) {
    for (int32_t t = touch_off[q]; t < touch_off[q + 1]; ++t) {
      const int32_t s = p->group_offsets[touch_chunk[t]] + touch_pos[t];
      p->slot_query[s] = q;
      p->query_slots[t] = s;
    }
    path.clear();
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) path.push_back(x);
    int32_t t = touch_off[q];
    for (auto it = path.rbegin(); it != path.rend(); ++it) {
      const int64_t a = p->node_flat_start[*it];
      const int64_t b = a + (query_lens && *it == query_nodes[q] ? query_lens[q] : seg_lens[*it]);
      while (t < touch_off[q + 1] && static_cast<int64_t>(touch_chunk[t] + 1) * c <= a) ++t;
      for (int32_t u = t; u < touch_off[q + 1]; ++u) {
        const int64_t cs = static_cast<int64_t>(touch_chunk[u]) * c;
        if (cs >= b) break;
        const int64_t lo = std::max(a, cs) - cs, hi = std::min(b, cs + c) - cs;  // [lo, hi) in chunk
        const int32_t s = p->group_offsets[touch_chunk[u]] + touch_pos[u];
        uint32_t* row = &p->slot_mask[static_cast<size_t>(s) * words];
        for (int64_t bit = lo; bit < hi;) {
          const int64_t w = bit >> 5, off = bit & 31;
          const int64_t take = std::min<int64_t>(32 - off, hi - bit);
          const uint32_t ones = take == 32 ? 0xffffffffu : ((1u << take) - 1u);
          row[w] |= ones << off;
          bit += take;
        }
        slot_bits[s] += hi - lo;
      }
    }
  }
  p->chunk_full.assign(nc, 0);
  for (int32_t k = 0; k < nc; ++k) {
    const int64_t len = p->chunk_start[k + 1] - p->chunk_start[k];
    bool full = p->group_offsets[k + 1] > p->group_offsets[k];
    for (int32_t s = p->group_offsets[k]; s < p->group_offsets[k + 1] && full; ++s)
      full = slot_bits[s] == len;
    p->chunk_full[k] = full ? 1 : 0;
  }

  p->num_nodes = n;
  p->num_queries = nq;
  p->chunk_tokens = c;
  p->total_tokens = total;
  p->num_chunks = nc;
  p->num_slots = S;
  p->mask_words = words;
  return DEFT_OK;
}

// Query-centric baseline plan: no KV sharing.  Each query's root-to-node
// path tokens (root segment first, each segment in order) form its own run of
// the flat index space, queries one after another; each run is cut into
// chunk_tokens windows from its start, every chunk has one slot (its query)
// with every bit set.  The same kernels then stream every query's whole path
// by itself, which is the per-query reading the pages compare DeFT against.
// node_start / flat_node_order / node_flat_start keep the tree plan's values.
static int build_query_centric(deft_plan* p, const int32_t* parents, const int32_t* seg_lens,
                               int32_t n, const int32_t* query_nodes, int32_t nq, int32_t c) {
  int rc = build_plan(p, parents, seg_lens, n, query_nodes, nq, c);   // tree fields
  if (rc) return rc;
  std::vector<int32_t> path;
  int64_t total = 0;
  for (int32_t q = 0; q < nq; ++q)
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) total += seg_lens[x];
  if (total > INT32_MAX) return fail(DEFT_ERR_INVALID_TREE, "total path tokens exceed 2^31 - 1");
  p->flat_to_logical.assign(static_cast<size_t>(total), 0);
  p->chunk_start.clear();
  p->slot_query.clear();
  p->query_slot_offsets.assign(nq + 1, 0);
  int64_t f = 0;
  for (int32_t q = 0; q < nq; ++q) {
    path.clear();
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) path.push_back(x);
    const int64_t q0 = f;
    for (auto it = path.rbegin(); it != path.rend(); ++it)
      for (int32_t i = 0; i < seg_lens[*it]; ++i) p->flat_to_logical[f++] = p->node_start[*it] + i;
    for (int64_t a = q0; a < f; a += c) {
      p->chunk_start.push_back(static_cast<int32_t>(a));
      p->slot_query.push_back(q);
    }
    p->query_slot_offsets[q + 1] = static_cast<int32_t>(p->slot_query.size());
  }
  const int32_t nc = static_cast<int32_t>(p->slot_query.size());
  p->chunk_start.push_back(static_cast<int32_t>(total));
  const int32_t words = (c + 31) / 32;
  p->group_offsets.resize(nc + 1);
  p->query_slots.resize(nc);
  for (int32_t k = 0; k <= nc; ++k) p->group_offsets[k] = k;
  for (int32_t k = 0; k < nc; ++k) p->query_slots[k] = k;
  p->slot_mask.assign(static_cast<size_t>(nc) * words, 0u);
  for (int32_t k = 0; k < nc; ++k) {
    const int32_t len = p->chunk_start[k + 1] - p->chunk_start[k];
    uint32_t* row = &p->slot_mask[static_cast<size_t>(k) * words];
    for (int32_t w = 0; w < words; ++w) {
      const int32_t bits = std::min(32, std::max(0, len - 32 * w));
      row[w] = bits == 32 ? 0xffffffffu : ((1u << bits) - 1u);
    }
  }
  p->chunk_full.assign(nc, 1);
  p->total_tokens = static_cast<int32_t>(total);
  p->num_chunks = nc;
  p->num_slots = nc;
  p->mask_words = words;
  p->query_centric = true;
  return DEFT_OK;
}

// Node-granularity plan (ablation of Flattened Tree KV Splitting): the same
// depth-first flat layout, but chunks never cross a node boundary; each
// node's segment is cut into chunk_tokens windows from its own start (only
// nodes longer than chunk_tokens are split).  A chunk's group is every query
// whose path holds the chunk's node, in ascending query index, each with all
// bits of the chunk set.
static int build_node_chunks(deft_plan* p, const int32_t* parents, const int32_t* seg_lens,
                             int32_t n, const int32_t* query_nodes, int32_t nq, int32_t c) {
  int rc = build_plan(p, parents, seg_lens, n, query_nodes, nq, c);   // flat layout
  if (rc) return rc;
  // chunk list in flat order, and the first chunk of every node
  std::vector<int32_t> node_first_chunk(n, 0);
  p->chunk_start.clear();
  for (int32_t x : p->flat_node_order) {
    node_first_chunk[x] = static_cast<int32_t>(p->chunk_start.size());
    for (int32_t a = 0; a < seg_lens[x]; a += c) p->chunk_start.push_back(p->node_flat_start[x] + a);
  }
  const int32_t nc = static_cast<int32_t>(p->chunk_start.size());
  p->chunk_start.push_back(p->total_tokens);
  auto n_chunks_of = [&](int32_t x) { return (seg_lens[x] + c - 1) / c; };
  // slots: chunk by chunk, its node's queries ascending
  std::vector<std::vector<int32_t>> node_queries(n);
  std::vector<int32_t> path;
  for (int32_t q = 0; q < nq; ++q)
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) node_queries[x].push_back(q);
  const int32_t words = (c + 31) / 32;
  p->group_offsets.assign(nc + 1, 0);
  for (int32_t x : p->flat_node_order)
    for (int32_t k = 0; k < n_chunks_of(x); ++k)
      p->group_offsets[node_first_chunk[x] + k + 1] = static_cast<int32_t>(node_queries[x].size());
  for (int32_t k = 0; k < nc; ++k) p->group_offsets[k + 1] += p->group_offsets[k];
  const int32_t S = p->group_offsets[nc];
  p->slot_query.assign(S, 0);
  p->slot_mask.assign(static_cast<size_t>(S) * words, 0u);
  p->chunk_full.assign(nc, 0);
  for (int32_t x : p->flat_node_order)
    for (int32_t k = 0; k < n_chunks_of(x); ++k) {
      const int32_t ch = node_first_chunk[x] + k;
      const int32_t len = p->chunk_start[ch + 1] - p->chunk_start[ch];
      for (size_t j = 0; j < node_queries[x].size(); ++j) {
        const int32_t s = p->group_offsets[ch] + static_cast<int32_t>(j);
        p->slot_query[s] = node_queries[x][j];
        uint32_t* row = &p->slot_mask[static_cast<size_t>(s) * words];
        for (int32_t w = 0; w < words; ++w) {
          const int32_t bits = std::min(32, std::max(0, len - 32 * w));
          row[w] = bits == 32 ? 0xffffffffu : ((1u << bits) - 1u);
        }
      }
      p->chunk_full[ch] = node_queries[x].empty() ? 0 : 1;
    }
  // merge lists: each query's slots in ascending chunk (= slot) order
  p->query_slot_offsets.assign(nq + 1, 0);
  for (int32_t s = 0; s < S; ++s) p->query_slot_offsets[p->slot_query[s] + 1]++;
  for (int32_t q = 0; q < nq; ++q) p->query_slot_offsets[q + 1] += p->query_slot_offsets[q];
  p->query_slots.assign(S, 0);
  {
    std::vector<int32_t> fill(p->query_slot_offsets.begin(), p->query_slot_offsets.end() - 1);
    for (int32_t s = 0; s < S; ++s) p->query_slots[fill[p->slot_query[s]]++] = s;
  }
  p->num_chunks = nc;
  p->num_slots = S;
  p->mask_words = words;
  return DEFT_OK;
}

int check_desc(const deft_plan* p, const deft_attn_desc* d) {
  if (!d) return fail(DEFT_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->page_size < 1 ||
      d->num_pages < 1)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "desc shapes must be positive");
  if (d->dtype != DEFT_DTYPE_F32 && d->dtype != DEFT_DTYPE_BF16)
    return fail(DEFT_ERR_UNSUPPORTED, "dtype must be DEFT_DTYPE_F32 or DEFT_DTYPE_BF16");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DEFT_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->page_size != kPageSize) return fail(DEFT_ERR_UNSUPPORTED, "page_size must be 16");
  if (d->f32_partials != 0 && d->f32_partials != 1)
    return fail(DEFT_ERR_INVALID_ARGUMENT, "f32_partials must be 0 or 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(DEFT_ERR_UNSUPPORTED, "num_q_heads must be a multiple of num_kv_heads");
  if (p && p->chunk_tokens > kMaxChunkTokens)
    return fail(DEFT_ERR_UNSUPPORTED, "chunk_tokens above 4096 is not supported by the kernels");
  // (query, query head) rows are indexed in 32 bits on the device, and the
  // merge launch covers them with 16 rows per 256-thread work-group
  if (p && static_cast<int64_t>(p->num_queries) * d->num_q_heads >= kMaxQueryRows)
    return fail(DEFT_ERR_UNSUPPORTED, "num_queries * num_q_heads must be below 2^28");
  return DEFT_OK;
}

static size_t align_words(size_t w) { return (w + 63) & ~static_cast<size_t>(63); }  // 256 B

size_t partial_o_words(const deft_plan* p, const deft_attn_desc* d) {
  const size_t n = static_cast<size_t>(p->num_slots) * d->num_q_heads * d->head_dim;
  return bf16_partials(d) ? (n + 1) / 2 : n;
}

size_t workspace_bytes_for(const deft_plan* p, const deft_attn_desc* d) {
  const size_t sh = static_cast<size_t>(p->num_slots) * d->num_q_heads;
  return 4 * (align_words(partial_o_words(p, d)) + 2 * align_words(sh));
}

// Which work items a chunk's group of `rows` (slot, query head) rows takes.
// MFMA when the group fills a tile (the query-centric baseline, groups of one
// query, takes MFMA for every bf16 group, its faster kernel).  Items of
// kMfmaWideRows rows (groups of more than kMfmaRows rows) halve the KV
// traffic of a group, since each chunk is streamed by half as many
// work-groups, but also halve the number of work-groups: worth it only when
// the 64-row items would fill the device at least twice over.  Whole-group
// items (kMfmaGroupRows, no token split) are taken only on request.
// DEFT_MFMA_WIDE / DEFT_MFMA_GROUP = 1 or 0 in the environment force either
// choice (tests).
// Rows a bf16 chunk needs to run on the matrix-core bodies: kMfmaMinRows
// (every chunk: a few-row item pads its rows on the matrix cores, which the
// latency-bound step loop has time for, where the VALU body spends its
// instruction stream on the same rows and ran about twice as long on the
// parallel-sampling tree's 512-token branches), or DEFT_MFMA_MIN_ROWS from
// the environment when it lies in [1, 4096] (tests send small chunks to the
// VALU body with it).
static int32_t mfma_min_rows() {
  const char* env = std::getenv("DEFT_MFMA_MIN_ROWS");
  if (env && env[0]) {
    const long v = std::strtol(env, nullptr, 10);
    if (v >= 1 && v <= 4096) return static_cast<int32_t>(v);
  }
  return kMfmaMinRows;
}

struct ItemPolicy {
  bool bf16, query_centric, wide_on, group_on;
  int32_t min_rows;
  bool mfma(int32_t rows) const { return bf16 && (rows >= min_rows || query_centric); }
  int32_t block(int32_t rows) const {
    if (!mfma(rows)) return kValuRows;
    if (group_on) return kMfmaGroupRows;
    if (wide_on && rows > kMfmaRows) return kMfmaWideRows;
    return kMfmaRows;
  }
};

static ItemPolicy item_policy(const std::vector<int32_t>& chunk_rows, const deft_attn_desc* d, bool query_centric,
                              int cus) {
  ItemPolicy pol{d->dtype == DEFT_DTYPE_BF16, query_centric, false, false, mfma_min_rows()};
  int64_t n64 = 0;
  for (int32_t rows : chunk_rows) {
    const int32_t b = pol.mfma(rows) ? kMfmaRows : kValuRows;
    n64 += (rows + b - 1) / b;
  }
  const char* force = std::getenv("DEFT_MFMA_WIDE");
  pol.wide_on = force && (force[0] == '0' || force[0] == '1') ? force[0] == '1'
                                                              : n64 * d->num_kv_heads >= 2 * static_cast<int64_t>(cus);
  const char* gforce = std::getenv("DEFT_MFMA_GROUP");
  pol.group_on = gforce && (gforce[0] == '0' || gforce[0] == '1') ? gforce[0] == '1' : false;
  return pol;
}

// Partial-kernel work-groups for chunks with these group row counts.
static int64_t work_groups(const std::vector<int32_t>& chunk_rows, const ItemPolicy& pol, int32_t hkv) {
  int64_t items = 0;
  for (int32_t rows : chunk_rows) {
    const int32_t b = pol.block(rows);
    items += (rows + b - 1) / b;
  }
  return items * hkv;
}

int build_image(deft_plan* p, const deft_attn_desc* d, std::vector<int32_t>* image,
                ImageLayout* L) {
  int rc = check_desc(p, d);
  if (rc) return rc;
  const int32_t G = d->num_q_heads / d->num_kv_heads;
  std::vector<WorkItem> group, wide, mfma, valu;
  std::vector<int32_t> chunk_rows(p->num_chunks);
  for (int32_t k = 0; k < p->num_chunks; ++k) chunk_rows[k] = (p->group_offsets[k + 1] - p->group_offsets[k]) * G;
  const ItemPolicy pol = item_policy(chunk_rows, d, p->query_centric, device_cu_count());
  for (int32_t k = 0; k < p->num_chunks; ++k) {
    const int32_t rows = (p->group_offsets[k + 1] - p->group_offsets[k]) * G;
    if (rows == 0) continue;
    const bool use_mfma = pol.mfma(rows);
    const int32_t blk = pol.block(rows);
    const bool use_group = blk == kMfmaGroupRows, use_wide = blk == kMfmaWideRows;
    const int32_t cs = p->chunk_start[k], len = p->chunk_start[k + 1] - cs;
    int32_t lstart = p->flat_to_logical[cs];
    for (int32_t t = 1; t < len && lstart >= 0; ++t)
      if (p->flat_to_logical[cs + t] != lstart + t) lstart = -1;
    for (int32_t r = 0; r < rows; r += blk)
      (use_group ? group : use_wide ? wide : use_mfma ? mfma : valu)
          .push_back({k, r, std::min(blk, rows - r), cs, len, p->group_offsets[k], p->chunk_full[k] ? 1 : 0, lstart});
  }
  // one launch of 512-thread work-groups covers every item for every KV head
  if (static_cast<int64_t>(group.size() + wide.size() + mfma.size() + valu.size()) * d->num_kv_heads >
      kMaxPartialBlocks)
    return fail(DEFT_ERR_UNSUPPORTED,
                "work items x num_kv_heads above 2^23 - 1, the partial kernel's grid limit (raise chunk_tokens)");
  size_t w = 0;
  auto take = [&](size_t n) { size_t at = w; w = align_words(w + n); return at; };
  const int32_t nc = p->num_chunks, S = p->num_slots, W = p->mask_words;
  L->chunk_start = take(nc + 1);
  L->group_offsets = take(nc + 1);
  L->chunk_full = take(nc);
  L->slot_query = take(S);
  L->slot_mask = take(static_cast<size_t>(S) * W);
  L->flat_to_logical = take(p->total_tokens);
  L->query_slot_offsets = take(p->num_queries + 1);
  L->query_slots = take(S);
  L->mfma_items = take(8 * (group.size() + wide.size() + mfma.size()));
  L->valu_items = take(8 * valu.size());
  // fused-merge tickets, one per (query, query head); zero in the uploaded
  // image and reset to zero by the kernels after use
  L->tickets = take(static_cast<size_t>(p->num_queries) * d->num_q_heads);
  // status word: 1 once a kernel's bounded inter-wave wait gave up (zero in
  // the uploaded image; deft_plan_status reads and clears it)
  L->status = take(1);
  // fixed-stride merge lists when padding costs at most about 4x the slots
  int32_t max_slots = 0;
  for (int32_t q = 0; q < p->num_queries; ++q)
    max_slots = std::max(max_slots, p->query_slot_offsets[q + 1] - p->query_slot_offsets[q]);
  const int64_t padded = static_cast<int64_t>(p->num_queries) * max_slots;
  L->merge_stride = (max_slots > 0 && padded <= 4 * static_cast<int64_t>(S) + 4096) ? max_slots : 0;
  L->merge_slots = take(L->merge_stride ? static_cast<size_t>(padded) : 0);
  L->total_words = w;
  L->n_mfma_group = static_cast<int32_t>(group.size());
  L->n_mfma_wide = static_cast<int32_t>(wide.size());
  L->n_mfma = static_cast<int32_t>(mfma.size());
  L->n_valu = static_cast<int32_t>(valu.size());
  L->max_valu_rows = 0;
  for (const WorkItem& it : valu) L->max_valu_rows = std::max(L->max_valu_rows, it.row_count);
  if (!image) return DEFT_OK;
  try {
    image->assign(w, 0);
  } catch (const std::bad_alloc&) {
    return fail(DEFT_ERR_NO_MEMORY, "host allocation of the plan image failed");
  }
  int32_t* im = image->data();
  std::copy(p->chunk_start.begin(), p->chunk_start.end(), im + L->chunk_start);
  std::copy(p->group_offsets.begin(), p->group_offsets.end(), im + L->group_offsets);
  for (int32_t k = 0; k < nc; ++k) im[L->chunk_full + k] = p->chunk_full[k];
  std::copy(p->slot_query.begin(), p->slot_query.end(), im + L->slot_query);
  std::memcpy(im + L->slot_mask, p->slot_mask.data(), 4 * p->slot_mask.size());
  std::copy(p->flat_to_logical.begin(), p->flat_to_logical.end(), im + L->flat_to_logical);
  std::copy(p->query_slot_offsets.begin(), p->query_slot_offsets.end(), im + L->query_slot_offsets);
  std::copy(p->query_slots.begin(), p->query_slots.end(), im + L->query_slots);
  std::memcpy(im + L->mfma_items, group.data(), sizeof(WorkItem) * group.size());
  std::memcpy(im + L->mfma_items + 8 * group.size(), wide.data(), sizeof(WorkItem) * wide.size());
  std::memcpy(im + L->mfma_items + 8 * (group.size() + wide.size()), mfma.data(), sizeof(WorkItem) * mfma.size());
  std::memcpy(im + L->valu_items, valu.data(), sizeof(WorkItem) * valu.size());
  if (L->merge_stride) {
    int32_t* ms = im + L->merge_slots;
    for (int32_t q = 0; q < p->num_queries; ++q) {
      const int32_t a = p->query_slot_offsets[q], b = p->query_slot_offsets[q + 1];
      int32_t* row = ms + static_cast<size_t>(q) * L->merge_stride;
      std::copy(p->query_slots.begin() + a, p->query_slots.begin() + b, row);
      std::fill(row + (b - a), row + L->merge_stride, -1);
    }
  }
  return DEFT_OK;
}

// Chunk-size rule: the smallest multiple of kAutoChunkStep tokens (up to
// kMaxChunkTokens) whose partial-kernel work-groups number at most `cus` (one
// round on the device), counting items of kMfmaRows rows for matrix-core
// groups and kValuRows rows otherwise; kMaxChunkTokens when none does.  (The
// wider items halve a chunk's work-groups but are taken for workloads that
// run several rounds anyway; a one-round size found by counting them gives
// more, shorter chunks, so more merge operands per query, and measured
// slower.)  A chunk's group size is counted from each
// query's visible flat intervals (its path's segments, in pre-order), as the
// planner's first pass does, without building the plan.
constexpr int32_t kAutoChunkStep = 32;

static int32_t auto_chunk_tokens(const int32_t* parents, const int32_t* seg_lens, int32_t n,
                                 const int32_t* query_nodes, const int32_t* query_lens, int32_t nq,
                                 const deft_attn_desc* d, int cus) {
  std::vector<int32_t> order, fstart;
  flatten(parents, seg_lens, n, &order, &fstart);
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) total += seg_lens[i];
  std::vector<int64_t> ia, ib;
  std::vector<int32_t> qoff(nq + 1, 0), path;
  for (int32_t q = 0; q < nq; ++q) {
    path.clear();
    for (int32_t x = query_nodes[q]; x >= 0; x = parents[x]) path.push_back(x);
    for (auto it = path.rbegin(); it != path.rend(); ++it) {
      const int64_t a = fstart[*it];
      ia.push_back(a);
      ib.push_back(a + (query_lens && *it == query_nodes[q] ? query_lens[q] : seg_lens[*it]));
    }
    qoff[q + 1] = static_cast<int32_t>(ia.size());
  }
  const int32_t G = d->num_q_heads / d->num_kv_heads;
  std::vector<int32_t> rows;
  for (int32_t c = kAutoChunkStep; c <= kMaxChunkTokens; c += kAutoChunkStep) {
    const int64_t nc = (total + c - 1) / c;
    rows.assign(static_cast<size_t>(nc), 0);
    for (int32_t q = 0; q < nq; ++q) {
      int64_t last = -1;
      for (int32_t t = qoff[q]; t < qoff[q + 1]; ++t)
        for (int64_t k = ia[t] / c; k <= (ib[t] - 1) / c; ++k)
          if (k != last) {
            rows[k] += G;
            last = k;
          }
    }
    ItemPolicy pol = item_policy(rows, d, false, cus);
    pol.wide_on = false;     // a one-round size is counted in 64-row items
    pol.group_on = false;
    if (work_groups(rows, pol, d->num_kv_heads) <= cus) return c;
  }
  return kMaxChunkTokens;
}

}  // namespace deft

using deft::fail;

extern "C" {

enum class PlanKind { kFlat, kQueryCentric, kNodeChunks };

static int plan_create(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                       const int32_t* query_nodes, int32_t num_queries, int32_t chunk_tokens,
                       PlanKind kind, deft_plan** out_plan, const int32_t* query_lens = nullptr) {
  deft::set_error("");
  if (!out_plan) return fail(DEFT_ERR_INVALID_ARGUMENT, "out_plan is NULL");
  *out_plan = nullptr;
  if (chunk_tokens < 1) return fail(DEFT_ERR_INVALID_ARGUMENT, "chunk_tokens must be >= 1");
  int rc = deft::validate_tree(parents, seg_lens, num_nodes, query_nodes, num_queries, query_lens);
  if (rc) return rc;
  deft_plan* p = new (std::nothrow) deft_plan();
  if (!p) return fail(DEFT_ERR_NO_MEMORY, "host allocation failed");
  try {
    if (kind == PlanKind::kQueryCentric)
      rc = deft::build_query_centric(p, parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens);
    else if (kind == PlanKind::kNodeChunks)
      rc = deft::build_node_chunks(p, parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens);
    else
      rc = deft::build_plan(p, parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens,
                            query_lens);
  } catch (const std::bad_alloc&) {
    rc = fail(DEFT_ERR_NO_MEMORY, "host allocation failed while planning");
  }
  if (rc) {
    delete p;
    return rc;
  }
  *out_plan = p;
  return DEFT_OK;
}

int deft_plan_create(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                     const int32_t* query_nodes, int32_t num_queries, int32_t chunk_tokens,
                     deft_plan** out_plan) {
  return plan_create(parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens, PlanKind::kFlat,
                     out_plan);
}

int deft_plan_create_query_centric(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                   const int32_t* query_nodes, int32_t num_queries,
                                   int32_t chunk_tokens, deft_plan** out_plan) {
  return plan_create(parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens,
                     PlanKind::kQueryCentric, out_plan);
}

int deft_plan_create_node_chunks(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                 const int32_t* query_nodes, int32_t num_queries, int32_t chunk_tokens,
                                 deft_plan** out_plan) {
  return plan_create(parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens,
                     PlanKind::kNodeChunks, out_plan);
}

int deft_plan_create_multi_token(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                 const int32_t* query_nodes, const int32_t* query_lens,
                                 int32_t num_queries, int32_t chunk_tokens, deft_plan** out_plan) {
  return plan_create(parents, seg_lens, num_nodes, query_nodes, num_queries, chunk_tokens, PlanKind::kFlat,
                     out_plan, query_lens);
}

void deft_plan_destroy(deft_plan* plan) {
  if (!plan) return;
  deft::release_upload(plan);
  delete plan;
}

int deft_plan_export(const deft_plan* p, deft_plan_view* v) {
  if (!p || !v) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan and view must not be NULL");
  v->num_nodes = p->num_nodes;
  v->num_queries = p->num_queries;
  v->chunk_tokens = p->chunk_tokens;
  v->total_tokens = p->total_tokens;
  v->num_chunks = p->num_chunks;
  v->num_slots = p->num_slots;
  v->mask_words = p->mask_words;
  v->node_start = p->node_start.data();
  v->flat_node_order = p->flat_node_order.data();
  v->node_flat_start = p->node_flat_start.data();
  v->flat_to_logical = p->flat_to_logical.data();
  v->chunk_start = p->chunk_start.data();
  v->group_offsets = p->group_offsets.data();
  v->slot_query = p->slot_query.data();
  v->slot_mask = p->slot_mask.data();
  v->chunk_full = p->chunk_full.data();
  v->query_slot_offsets = p->query_slot_offsets.data();
  v->query_slots = p->query_slots.data();
  return DEFT_OK;
}

int deft_plan_device_bytes(deft_plan* p, const deft_attn_desc* d, size_t* plan_bytes,
                           size_t* workspace_bytes) {
  if (!p) return fail(DEFT_ERR_INVALID_ARGUMENT, "plan is NULL");
  deft::ImageLayout L{};
  int rc = deft::build_image(p, d, nullptr, &L);
  if (rc) return rc;
  if (plan_bytes) *plan_bytes = 4 * L.total_words;
  if (workspace_bytes) *workspace_bytes = deft::workspace_bytes_for(p, d);
  return DEFT_OK;
}

int deft_plan_auto_chunk_tokens(const int32_t* parents, const int32_t* seg_lens, int32_t num_nodes,
                                const int32_t* query_nodes, const int32_t* query_lens, int32_t num_queries,
                                const deft_attn_desc* desc, int32_t num_cus, int32_t* out_chunk_tokens) {
  deft::set_error("");
  if (!out_chunk_tokens) return fail(DEFT_ERR_INVALID_ARGUMENT, "out_chunk_tokens is NULL");
  if (num_cus < 0) return fail(DEFT_ERR_INVALID_ARGUMENT, "num_cus must be >= 0");
  int rc = deft::validate_tree(parents, seg_lens, num_nodes, query_nodes, num_queries, query_lens);
  if (rc) return rc;
  rc = deft::check_desc(nullptr, desc);
  if (rc) return rc;
  try {
    *out_chunk_tokens = deft::auto_chunk_tokens(parents, seg_lens, num_nodes, query_nodes, query_lens, num_queries,
                                                desc, num_cus > 0 ? num_cus : deft::device_cu_count());
  } catch (const std::bad_alloc&) {
    return fail(DEFT_ERR_NO_MEMORY, "host allocation failed while choosing the chunk size");
  }
  return DEFT_OK;
}

const char* deft_last_error(void) { return deft::g_last_error.c_str(); }

}  // extern "C"
