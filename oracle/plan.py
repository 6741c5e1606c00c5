"""Reference tree planner (Python).  TEST INFRASTRUCTURE.

It writes out, from the DeFT pages, the bookkeeping a DeFT decode step needs,
so that the native planner can be compared with it array for array:

* Flattened Tree KV Splitting ("DeFT Guide ... The DeFT Architecture",
  "2. Flattened Tree KV Splitting"; the abstract of arXiv 2404.00242): the
  tree's KV is laid out as one contiguous linear index space and cut into
  equal-sized token chunks.  Reading: the linear order is a depth-first
  pre-order over the nodes (roots, then children, both by ascending id); the
  chunks are fixed C-token windows from flat index 0, so chunks cross node
  boundaries and only the last one may be short.
* KV-Guided Grouping ("1. KV-Guided Grouping"): the queries that need a
  chunk's KV are grouped so the chunk is loaded once for all of them.
  Reading: the group of a chunk is every query that sees at least one of its
  tokens, in ascending query index.
* Tree mask ("Tree-Constrained Attention Formulation"; the tiling sketch in
  the same "Deep Dive" section): per (chunk, query) a bit row, bit t set iff
  the chunk's t-th flat token belongs to a node on the query's root-to-node
  path (the node itself included).  Bits are packed LSB first into uint32
  words, ceil(C/32) words per row; bits past the chunk's end are zero.
* Multi-token query nodes (a reading; the pages define the mask by ancestry
  only): query_lens[i], when given, is how many leading tokens of its own
  node query i sees (1 .. seg_lens[node]), the causal mask inside a node that
  tree prefill needs; its node's later tokens are masked like another
  branch's.  Without query_lens every query sees its whole node.
* Merge lists: each query's (chunk, query) slots in ascending chunk order,
  the operands of its log-sum-exp merge ("3. Fused In-SRAM Online Softmax
  Merging" and "The Online Softmax Tile Accumulation").

Every array is int32 except slot_mask (uint32) and chunk_full (uint8).
"""
from __future__ import annotations

import numpy as np

INT32_MAX = 2**31 - 1


class PlanError(ValueError):
    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind          # "invalid_tree" or "invalid_argument"


def ref_plan(parents, seg_lens, query_nodes, chunk_tokens: int, query_lens=None) -> dict:
    parents = np.asarray(parents, dtype=np.int64)
    seg_lens = np.asarray(seg_lens, dtype=np.int64)
    query_nodes = np.asarray(query_nodes, dtype=np.int64)
    n = parents.shape[0]
    nq = query_nodes.shape[0]
    if chunk_tokens < 1:
        raise PlanError("invalid_argument", "chunk_tokens must be >= 1")
    if n < 1 or nq < 1 or seg_lens.shape[0] != n:
        raise PlanError("invalid_argument", "need at least one node and one query")
    for i in range(n):
        if not (-1 <= parents[i] < i):
            raise PlanError("invalid_tree", f"parents[{i}] must be -1 or in [0, {i})")
        if seg_lens[i] < 1:
            raise PlanError("invalid_tree", f"seg_lens[{i}] must be >= 1")
    for qi in range(nq):
        if not (0 <= query_nodes[qi] < n):
            raise PlanError("invalid_tree", f"query_nodes[{qi}] out of range")
    if query_lens is not None:
        query_lens = np.asarray(query_lens, dtype=np.int64)
        if query_lens.shape[0] != nq:
            raise PlanError("invalid_argument", "query_lens needs one entry per query")
        for qi in range(nq):
            if not (1 <= query_lens[qi] <= seg_lens[query_nodes[qi]]):
                raise PlanError("invalid_tree", f"query_lens[{qi}] must be in [1, seg_lens[node]]")
    total = int(seg_lens.sum())
    if total > INT32_MAX:
        raise PlanError("invalid_tree", "total tokens exceed int32")

    # logical layout: segments in node-id order
    node_start = np.zeros(n, dtype=np.int64)
    node_start[1:] = np.cumsum(seg_lens)[:-1]

    # children lists in ascending id; roots in ascending id
    children = [[] for _ in range(n)]
    roots = []
    for i in range(n):
        if parents[i] < 0:
            roots.append(i)
        else:
            children[parents[i]].append(i)

    # depth-first pre-order
    order = []
    stack = list(reversed(roots))
    while stack:
        x = stack.pop()
        order.append(x)
        stack.extend(reversed(children[x]))
    node_flat_start = np.zeros(n, dtype=np.int64)
    run = 0
    for x in order:
        node_flat_start[x] = run
        run += int(seg_lens[x])

    flat_to_logical = np.empty(total, dtype=np.int64)
    flat_node = np.empty(total, dtype=np.int64)
    flat_offset = np.empty(total, dtype=np.int64)     # position inside its node
    for x in range(n):
        a = node_flat_start[x]
        flat_to_logical[a:a + seg_lens[x]] = np.arange(node_start[x], node_start[x] + seg_lens[x])
        flat_node[a:a + seg_lens[x]] = x
        flat_offset[a:a + seg_lens[x]] = np.arange(seg_lens[x])

    c = int(chunk_tokens)
    n_chunks = -(-total // c)
    chunk_start = np.array([min(k * c, total) for k in range(n_chunks + 1)], dtype=np.int64)
    words = -(-c // 32)

    # per query: which nodes lie on its root-to-node path
    on_path = np.zeros((nq, n), dtype=bool)
    for qi in range(nq):
        x = int(query_nodes[qi])
        while x >= 0:
            on_path[qi, x] = True
            x = int(parents[x])

    group_offsets = [0]
    slot_query = []
    slot_mask = []
    chunk_full = np.zeros(n_chunks, dtype=np.uint8)
    for k in range(n_chunks):
        a, b = int(chunk_start[k]), int(chunk_start[k + 1])
        nodes = flat_node[a:b]
        full = True
        members = 0
        for qi in range(nq):
            vis = on_path[qi, nodes]
            if query_lens is not None:
                vis = vis & ~((nodes == query_nodes[qi]) & (flat_offset[a:b] >= query_lens[qi]))
            if not vis.any():
                continue
            members += 1
            full = full and bool(vis.all())
            bits = np.zeros(words * 32, dtype=np.uint8)
            bits[:b - a] = vis
            slot_mask.append(np.packbits(bits, bitorder="little").view("<u4"))
            slot_query.append(qi)
        group_offsets.append(group_offsets[-1] + members)
        chunk_full[k] = 1 if (full and members > 0) else 0

    s_tot = len(slot_query)
    slot_query = np.array(slot_query, dtype=np.int64)
    query_slot_offsets = np.zeros(nq + 1, dtype=np.int64)
    for qi in slot_query:
        query_slot_offsets[qi + 1] += 1
    query_slot_offsets = np.cumsum(query_slot_offsets)
    fill = query_slot_offsets[:-1].copy()
    query_slots = np.empty(s_tot, dtype=np.int64)
    for s in range(s_tot):          # slots are numbered in ascending chunk order
        qi = slot_query[s]
        query_slots[fill[qi]] = s
        fill[qi] += 1

    i32 = lambda a: np.asarray(a, dtype=np.int64).astype(np.int32)
    return {
        "num_nodes": n,
        "num_queries": nq,
        "chunk_tokens": c,
        "total_tokens": total,
        "num_chunks": n_chunks,
        "num_slots": s_tot,
        "mask_words": words,
        "node_start": i32(node_start),
        "flat_node_order": i32(order),
        "node_flat_start": i32(node_flat_start),
        "flat_to_logical": i32(flat_to_logical),
        "chunk_start": i32(chunk_start),
        "group_offsets": i32(group_offsets),
        "slot_query": i32(slot_query),
        "slot_mask": (np.stack(slot_mask) if s_tot else np.zeros((0, words), "<u4")).astype(np.uint32),
        "chunk_full": chunk_full,
        "query_slot_offsets": i32(query_slot_offsets),
        "query_slots": i32(query_slots),
    }


def ref_plan_query_centric(parents, seg_lens, query_nodes, chunk_tokens: int) -> dict:
    """The query-centric baseline plan (no KV sharing), the per-query reading
    of attention that DeFT's abstract and the Guide's "The Tree-Attention
    Bottleneck: Redundant Memory IO and Severe Load Imbalances" ("1. Massive
    Redundant Memory Access (IO)") contrast it with: each query's root-to-node path tokens
    (root segment first, every segment in order) form their own run of the
    flat index space, queries one after another; each run is cut into
    chunk_tokens windows from its own start; every chunk holds one slot (its
    query) with every bit of the chunk set.  node_start, flat_node_order and
    node_flat_start are those of the tree plan.
    """
    tree = ref_plan(parents, seg_lens, query_nodes, chunk_tokens)
    parents = np.asarray(parents, dtype=np.int64)
    seg_lens = np.asarray(seg_lens, dtype=np.int64)
    query_nodes = np.asarray(query_nodes, dtype=np.int64)
    node_start = tree["node_start"].astype(np.int64)
    nq = query_nodes.shape[0]
    c = int(chunk_tokens)
    words = -(-c // 32)
    flat, chunk_start, slot_query, qso = [], [], [], [0]
    for qi in range(nq):
        path = []
        x = int(query_nodes[qi])
        while x >= 0:
            path.append(x)
            x = int(parents[x])
        q0 = len(flat)
        for x in reversed(path):                 # root first
            flat.extend(range(int(node_start[x]), int(node_start[x] + seg_lens[x])))
        for a in range(q0, len(flat), c):
            chunk_start.append(a)
            slot_query.append(qi)
        qso.append(len(slot_query))
    total = len(flat)
    if total > INT32_MAX:
        raise PlanError("invalid_tree", "total path tokens exceed int32")
    chunk_start.append(total)
    nc = len(slot_query)
    slot_mask = np.zeros((nc, words), dtype=np.uint32)
    for k in range(nc):
        bits = np.zeros(words * 32, dtype=np.uint8)
        bits[:chunk_start[k + 1] - chunk_start[k]] = 1
        slot_mask[k] = np.packbits(bits, bitorder="little").view("<u4")
    i32 = lambda a: np.asarray(a, dtype=np.int64).astype(np.int32)
    out = dict(tree)
    out.update({
        "total_tokens": total,
        "num_chunks": nc,
        "num_slots": nc,
        "mask_words": words,
        "flat_to_logical": i32(flat),
        "chunk_start": i32(chunk_start),
        "group_offsets": i32(np.arange(nc + 1)),
        "slot_query": i32(slot_query),
        "slot_mask": slot_mask,
        "chunk_full": np.ones(nc, dtype=np.uint8),
        "query_slot_offsets": i32(qso),
        "query_slots": i32(np.arange(nc)),
    })
    return out


def ref_plan_node_chunks(parents, seg_lens, query_nodes, chunk_tokens: int) -> dict:
    """Node-granularity grouping (the ablation of Flattened Tree KV
    Splitting; the Guide's "2. Flattened Tree KV Splitting" contrasts it with
    node-sized work units): the tree plan's depth-first flat layout, but
    every node's segment is cut into chunk_tokens windows from its own start,
    so no chunk crosses a node boundary.  A chunk's group is every query whose
    root-to-node path holds the chunk's node, ascending, each slot with all of
    the chunk's bits set; the merge lists follow.
    """
    tree = ref_plan(parents, seg_lens, query_nodes, chunk_tokens)
    parents = np.asarray(parents, dtype=np.int64)
    seg_lens = np.asarray(seg_lens, dtype=np.int64)
    query_nodes = np.asarray(query_nodes, dtype=np.int64)
    n, nq, c = parents.shape[0], query_nodes.shape[0], int(chunk_tokens)
    words = -(-c // 32)
    sees = [set() for _ in range(n)]          # queries whose path holds node x
    for qi in range(nq):
        x = int(query_nodes[qi])
        while x >= 0:
            sees[x].add(qi)
            x = int(parents[x])
    chunk_start, group_offsets, slot_query, rows, full = [], [0], [], [], []
    for x in tree["flat_node_order"]:
        x = int(x)
        a0 = int(tree["node_flat_start"][x])
        for a in range(0, int(seg_lens[x]), c):
            length = min(c, int(seg_lens[x]) - a)
            chunk_start.append(a0 + a)
            members = sorted(sees[x])
            for qi in members:
                bits = np.zeros(words * 32, dtype=np.uint8)
                bits[:length] = 1
                rows.append(np.packbits(bits, bitorder="little").view("<u4"))
                slot_query.append(qi)
            group_offsets.append(group_offsets[-1] + len(members))
            full.append(1 if members else 0)
    chunk_start.append(int(tree["total_tokens"]))
    s_tot = len(slot_query)
    query_slots = [s for qi in range(nq) for s in range(s_tot) if slot_query[s] == qi]
    qso = np.concatenate([[0], np.cumsum(np.bincount(np.asarray(slot_query, dtype=np.int64), minlength=nq))])
    i32 = lambda v: np.asarray(v, dtype=np.int64).astype(np.int32)
    out = dict(tree)
    out.update({
        "num_chunks": len(chunk_start) - 1,
        "num_slots": s_tot,
        "mask_words": words,
        "chunk_start": i32(chunk_start),
        "group_offsets": i32(group_offsets),
        "slot_query": i32(slot_query),
        "slot_mask": (np.stack(rows) if s_tot else np.zeros((0, words), "<u4")).astype(np.uint32),
        "chunk_full": np.asarray(full, dtype=np.uint8),
        "query_slot_offsets": i32(qso),
        "query_slots": i32(query_slots),
    })
    return out
