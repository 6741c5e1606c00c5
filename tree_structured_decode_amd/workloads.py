"""Seeded synthetic workloads for tree-structured decode attention.

This module only builds inputs: tree topologies, query placements, paged-KV
pools with their block tables, and the Q/K/V values.  It holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can draw from it.

Workload shapes follow the tree-based decoding scenarios the DeFT pages
describe (DeFT, arXiv 2404.00242, abstract; DeFT Guide, "The Tree-Attention
Bottleneck" and "Empirical Benchmark Evaluation"): a long shared prompt prefix
with a speculative token tree below it, parallel sampling / beam branches over
a shared prompt, and an unbalanced multi-step reasoning tree.  No dataset is
used; every value is drawn from a seeded generator.

Tree encoding used throughout:
  parents[i]   parent node id, or -1 for a root; parents[i] < i
  seg_lens[i]  number of KV tokens owned by node i (>= 1)
  query_nodes  node id each decode query sits on (it sees that node and
               all of its ancestors)
  query_lens   optional, multi-token query nodes: how many leading tokens
               of its own node each query sees (its position in the node
               plus one); absent means the whole node
Logical KV token order is the node segments concatenated in node-id order, so
node i owns logical tokens [node_start[i], node_start[i] + seg_lens[i]) with
node_start the exclusive prefix sum of seg_lens.  Logical token t lives in
pool page block_table[t // page_size], row t % page_size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 16

# Names of the five standard workloads, in order.
WORKLOADS = {
    1: "tiny-f32-gqa4-d64-binary-tree",
    2: "spec-tree-4k-prefix-64-nodes-llama3-8b-bf16",
    3: "parallel-sampling-2k-prompt-32x512-bf16",
    4: "reasoning-tree-1k-root-depth6-100-leaves-bf16",
    5: "spec-tree-32k-prefix-256-nodes-llama3-70b-bf16",
    6: "multi-token-tree-2k-prompt-32-nodes-x8-bf16",
}


@dataclass
class Workload:
    name: str
    parents: np.ndarray          # int32 [N]
    seg_lens: np.ndarray         # int32 [N]
    query_nodes: np.ndarray      # int32 [Nq]
    chunk_tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype           # torch.float32 or torch.bfloat16
    num_pages: int               # physical pages in the pool
    block_table: np.ndarray      # int32 [ceil(T / PAGE_SIZE)]
    q: torch.Tensor              # [Nq, Hq, d] in `dtype`, CPU
    k_tokens: torch.Tensor       # [T, Hkv, d] in `dtype`, CPU, logical order
    v_tokens: torch.Tensor       # [T, Hkv, d] in `dtype`, CPU, logical order
    page_size: int = PAGE_SIZE
    meta: dict = field(default_factory=dict)
    query_lens: Optional[np.ndarray] = None   # int32 [Nq] or None

    @property
    def total_tokens(self) -> int:
        return int(self.seg_lens.astype(np.int64).sum())

    @property
    def num_queries(self) -> int:
        return int(self.query_nodes.shape[0])

    @property
    def used_pages(self) -> np.ndarray:
        """Sorted physical ids of the pages that hold logical tokens."""
        return np.unique(self.block_table)


# --------------------------------------------------------------------------
# Tree generators
# --------------------------------------------------------------------------

def binary_tree_4_leaves():
    """Root of 256 tokens, two children of 32, each with two children of 32.

    Node ids: 0 root, 1 and 2 its children, 3 and 4 under 1, 5 and 6 under 2.
    One decode query per leaf.
    """
    parents = np.array([-1, 0, 0, 1, 1, 2, 2], dtype=np.int32)
    seg = np.array([256, 32, 32, 32, 32, 32, 32], dtype=np.int32)
    queries = np.array([3, 4, 5, 6], dtype=np.int32)
    return parents, seg, queries


def medusa_token_tree(rng: np.random.Generator, branching, keep: int):
    """Medusa-style speculative token tree, pruned to `keep` nodes.

    The root token sits at depth 1.  Nodes are expanded breadth-first in
    creation order; every node at depth k receives branching[k-1] children.
    Each child's score is its parent's score times a uniform draw (the root
    has score 1), drawn in creation order.  The `keep` best nodes by
    (-score, creation id) are kept; that set is closed under ancestors
    because a child never outscores its parent.  Kept nodes are renumbered in
    creation order, so parent ids stay below child ids.

    Returns (parents, depths) over the kept nodes, parents -1 for the root.
    """
    par = [-1]
    score = [1.0]
    depth = [1]
    frontier = [0]
    for b in branching:
        nxt = []
        for p in frontier:
            for _ in range(b):
                par.append(p)
                score.append(score[p] * rng.uniform())
                depth.append(depth[p] + 1)
                nxt.append(len(par) - 1)
        frontier = nxt
    order = sorted(range(len(par)), key=lambda i: (-score[i], i))[:keep]
    kept = sorted(order)
    new_id = {old: i for i, old in enumerate(kept)}
    parents = np.array([-1 if par[o] < 0 else new_id[par[o]] for o in kept], dtype=np.int32)
    depths = np.array([depth[o] for o in kept], dtype=np.int32)
    assert all(p < i for i, p in enumerate(parents)), "pruned tree is not ancestor-closed"
    return parents, depths


def prefix_plus_token_tree(prefix_len: int, tree_parents: np.ndarray):
    """Node 0 is the shared prefix; tree node j becomes node j + 1."""
    k = tree_parents.shape[0]
    parents = np.empty(k + 1, dtype=np.int32)
    parents[0] = -1
    parents[1:] = np.where(tree_parents < 0, 0, tree_parents + 1)
    seg = np.ones(k + 1, dtype=np.int32)
    seg[0] = prefix_len
    queries = np.arange(1, k + 1, dtype=np.int32)
    return parents, seg, queries


def multi_token_nodes(parents: np.ndarray, seg_lens: np.ndarray, node_tokens: int):
    """Give every non-root node `node_tokens` tokens and put a query on each
    of them (tree prefill of multi-token speculative nodes): the query on a
    node's j-th token sees the ancestors and the node's first j + 1 tokens.
    Queries are ordered by node, then position.  Returns
    (parents, seg_lens, query_nodes, query_lens)."""
    seg = np.asarray(seg_lens, dtype=np.int32).copy()
    inner = np.nonzero(np.asarray(parents) >= 0)[0]
    seg[inner] = node_tokens
    qn = np.repeat(inner, node_tokens).astype(np.int32)
    ql = np.tile(np.arange(1, node_tokens + 1), inner.shape[0]).astype(np.int32)
    return np.asarray(parents, dtype=np.int32), seg, qn, ql


def shared_prompt_branches(prompt_len: int, n_branches: int, suffix_len: int):
    parents = np.array([-1] + [0] * n_branches, dtype=np.int32)
    seg = np.array([prompt_len] + [suffix_len] * n_branches, dtype=np.int32)
    queries = np.arange(1, n_branches + 1, dtype=np.int32)
    return parents, seg, queries


def reasoning_tree(rng: np.random.Generator, root_len=1000, depth=6, n_leaves=100,
                   branch_lo=1, branch_hi=5, seg_lo=20, seg_hi=400):
    """Unbalanced multi-step reasoning tree.

    The root (depth 0) owns `root_len` tokens.  Breadth-first, every node at
    depth < `depth` draws a child count uniform in [branch_lo, branch_hi] and
    then, per child, a segment length uniform in [seg_lo, seg_hi].  The first
    `n_leaves` depth-`depth` nodes in depth-first order (children in creation
    order) are kept with their ancestors and renumbered in creation order.
    One decode query per kept leaf, in ascending node id.
    """
    par = [-1]
    seg = [root_len]
    dep = [0]
    children = [[]]
    frontier = [0]
    for _ in range(depth):
        nxt = []
        for p in frontier:
            b = int(rng.integers(branch_lo, branch_hi + 1))
            for _ in range(b):
                par.append(p)
                seg.append(int(rng.integers(seg_lo, seg_hi + 1)))
                dep.append(dep[p] + 1)
                children.append([])
                children[p].append(len(par) - 1)
                nxt.append(len(par) - 1)
        frontier = nxt
    leaves = []
    stack = [0]
    while stack and len(leaves) < n_leaves:
        n = stack.pop()
        if dep[n] == depth:
            leaves.append(n)
            continue
        stack.extend(reversed(children[n]))
    keep = set()
    for leaf in leaves:
        n = leaf
        while n >= 0 and n not in keep:
            keep.add(n)
            n = par[n]
    kept = sorted(keep)
    new_id = {old: i for i, old in enumerate(kept)}
    parents = np.array([-1 if par[o] < 0 else new_id[par[o]] for o in kept], dtype=np.int32)
    seg_lens = np.array([seg[o] for o in kept], dtype=np.int32)
    queries = np.array(sorted(new_id[x] for x in leaves), dtype=np.int32)
    return parents, seg_lens, queries


# --------------------------------------------------------------------------
# Values and pools
# --------------------------------------------------------------------------

def draw_qkv(seed: int, nq: int, hq: int, hkv: int, d: int, total_tokens: int,
             dtype: torch.dtype, value_scale: float = 1.0):
    """Q [Nq,Hq,d], then K and V [T,Hkv,d] in logical order, i.i.d. N(0,1).

    Drawn in fp32 from torch's CPU generator, multiplied by `value_scale`,
    then rounded to `dtype` (round-to-nearest-even for bf16).
    """
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(nq, hq, d, generator=g, dtype=torch.float32)
    k = torch.randn(total_tokens, hkv, d, generator=g, dtype=torch.float32)
    v = torch.randn(total_tokens, hkv, d, generator=g, dtype=torch.float32)
    if value_scale != 1.0:
        q, k, v = q * value_scale, k * value_scale, v * value_scale
    return q.to(dtype), k.to(dtype), v.to(dtype)


def make_workload(name, parents, seg_lens, query_nodes, *, chunk_tokens, hq, hkv, d,
                  dtype, seed=0, placement="identity", pool_pages=None,
                  value_scale=1.0, meta=None, query_lens=None) -> Workload:
    """Assemble a workload: draw values, choose page placement.

    placement: "identity"  block_table[j] = j, pool = exactly the used pages
               "permuted"  pool = exactly the used pages, seeded permutation
               "scattered" pool of `pool_pages` pages, used pages at seeded
                           distinct random positions
    """
    parents = np.asarray(parents, dtype=np.int32)
    seg_lens = np.asarray(seg_lens, dtype=np.int32)
    query_nodes = np.asarray(query_nodes, dtype=np.int32)
    total = int(seg_lens.astype(np.int64).sum())
    n_lp = -(-total // PAGE_SIZE)
    prng = np.random.default_rng(seed + 7919)
    if placement == "identity":
        bt = np.arange(n_lp, dtype=np.int32)
        n_pages = n_lp if pool_pages is None else int(pool_pages)
    elif placement == "permuted":
        bt = prng.permutation(n_lp).astype(np.int32)
        n_pages = n_lp
    elif placement == "scattered":
        n_pages = int(pool_pages)
        if n_pages < n_lp:
            raise ValueError("pool smaller than the tree's pages")
        bt = np.sort(prng.choice(n_pages, size=n_lp, replace=False)).astype(np.int64)
        bt = prng.permutation(bt).astype(np.int32)
    else:
        raise ValueError(placement)
    q, k, v = draw_qkv(seed, query_nodes.shape[0], hq, hkv, d, total, dtype, value_scale)
    return Workload(name=name, parents=parents, seg_lens=seg_lens, query_nodes=query_nodes,
                    chunk_tokens=int(chunk_tokens), num_q_heads=hq, num_kv_heads=hkv,
                    head_dim=d, dtype=dtype, num_pages=n_pages, block_table=bt,
                    q=q, k_tokens=k, v_tokens=v, meta=dict(meta or {}),
                    query_lens=None if query_lens is None else np.asarray(query_lens, dtype=np.int32))


def hbm_pool_pages(total_bytes: int, hkv: int = 8, d: int = 128, elem_bytes: int = 2,
                   fraction: float = 0.6) -> int:
    """Pages that fill `fraction` of device memory with a K and a V pool."""
    page_bytes = 2 * PAGE_SIZE * hkv * d * elem_bytes
    return int(math.floor(fraction * total_bytes / page_bytes))


def standard_workload(cfg: int, seed: int = 0, *, chunk_tokens: Optional[int] = None,
                      pool_pages: Optional[int] = None, unscaled: bool = False,
                      placement: Optional[str] = None) -> Workload:
    """The standard workloads (see WORKLOADS for their names).

    1: fp32, 4 q heads / 1 KV head, d 64; binary tree 256 + 2x32 + 4x32,
       one query per leaf; chunks of 64 tokens.
    2: bf16, 32 q / 8 KV heads, d 128; 4096-token prefix plus a 64-node
       Medusa tree (branching 4/3/2/2), every tree node a query; values
       scaled by 1/sqrt(d) unless `unscaled`; chunks of 544 tokens.
    3: bf16, 32/8, d 128; 2048-token prompt with 32 branches of 512 tokens,
       one query per branch; the 1152 pages in a seeded random order.
    4: bf16, 32/8, d 128; 1000-token root and a depth-6 reasoning tree
       (branching 1..5, segments 20..400), first 100 leaves, one query each;
       chunks of 2176 tokens.
    5: bf16, 64 q / 8 KV heads, d 128; 32768-token prefix plus a 256-node
       Medusa tree (branching 8/4/2/2/1), every tree node a query; pages at
       random positions of a `pool_pages` pool (default: just the used pages).
    6: bf16, 32/8, d 128; multi-token query nodes: a 2048-token prompt and a
       32-node Medusa tree (branching 4/3/2) whose nodes hold 8 draft tokens
       each, every draft token a query (256 queries, causal inside a node);
       chunks of 1280 tokens; values scaled by 1/sqrt(d).
    """
    rng = np.random.default_rng(seed)
    if cfg == 1:
        p, s, qn = binary_tree_4_leaves()
        return make_workload(WORKLOADS[1], p, s, qn, chunk_tokens=chunk_tokens or 64,
                             hq=4, hkv=1, d=64, dtype=torch.float32, seed=seed,
                             placement=placement or "identity")
    if cfg == 2:
        tp, depths = medusa_token_tree(rng, (4, 3, 2, 2), 64)
        p, s, qn = prefix_plus_token_tree(4096, tp)
        scale = 1.0 if unscaled else 1.0 / math.sqrt(128)
        return make_workload(WORKLOADS[2], p, s, qn, chunk_tokens=chunk_tokens or 544,
                             hq=32, hkv=8, d=128, dtype=torch.bfloat16, seed=seed,
                             placement=placement or "identity", value_scale=scale,
                             meta={"depths": depths})
    if cfg == 3:
        p, s, qn = shared_prompt_branches(2048, 32, 512)
        return make_workload(WORKLOADS[3], p, s, qn, chunk_tokens=chunk_tokens or 512,
                             hq=32, hkv=8, d=128, dtype=torch.bfloat16, seed=seed,
                             placement=placement or "permuted")
    if cfg == 4:
        p, s, qn = reasoning_tree(rng)
        return make_workload(WORKLOADS[4], p, s, qn, chunk_tokens=chunk_tokens or 2176,
                             hq=32, hkv=8, d=128, dtype=torch.bfloat16, seed=seed,
                             placement=placement or "identity")
    if cfg == 5:
        tp, depths = medusa_token_tree(rng, (8, 4, 2, 2, 1), 256)
        p, s, qn = prefix_plus_token_tree(32768, tp)
        total = int(s.sum())
        pages = pool_pages if pool_pages is not None else -(-total // PAGE_SIZE)
        return make_workload(WORKLOADS[5], p, s, qn, chunk_tokens=chunk_tokens or 4096,
                             hq=64, hkv=8, d=128, dtype=torch.bfloat16, seed=seed,
                             placement=placement or "scattered", pool_pages=pages,
                             meta={"depths": depths})
    if cfg == 6:
        tp, depths = medusa_token_tree(rng, (4, 3, 2), 32)
        p, s, _ = prefix_plus_token_tree(2048, tp)
        p, s, qn, ql = multi_token_nodes(p, s, 8)
        return make_workload(WORKLOADS[6], p, s, qn, chunk_tokens=chunk_tokens or 1280,
                             hq=32, hkv=8, d=128, dtype=torch.bfloat16, seed=seed,
                             placement=placement or "permuted", value_scale=1.0 / math.sqrt(128),
                             meta={"depths": depths}, query_lens=ql)
    raise ValueError(f"unknown workload {cfg}")


def random_tree(rng: np.random.Generator, n_nodes: int, seg_lo: int, seg_hi: int,
                n_queries: int, forest_prob: float = 0.0):
    """Random tree (or forest) with parents[i] < i, for tests."""
    parents = np.empty(n_nodes, dtype=np.int32)
    parents[0] = -1
    for i in range(1, n_nodes):
        parents[i] = -1 if rng.uniform() < forest_prob else int(rng.integers(0, i))
    seg = rng.integers(seg_lo, seg_hi + 1, size=n_nodes).astype(np.int32)
    queries = rng.integers(0, n_nodes, size=n_queries).astype(np.int32)
    return parents, seg, queries


# --------------------------------------------------------------------------
# Placing the KV values into a paged pool
# --------------------------------------------------------------------------

def token_page_rows(wl: Workload):
    """(physical page, row) for every logical token."""
    t = np.arange(wl.total_tokens, dtype=np.int64)
    return wl.block_table[t // wl.page_size].astype(np.int64), t % wl.page_size


def build_pool(wl: Workload, device, poison: bool = True):
    """K and V pools [num_pages, page_size, Hkv, d] on `device`.

    Every row that holds no logical token (unused pages, the tail of the last
    page) is NaN when `poison`, so a stray read shows up in the output.
    """
    shape = (wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
    fill = float("nan") if poison else 0.0
    kc = torch.full(shape, fill, dtype=wl.dtype, device=device)
    vc = torch.full(shape, fill, dtype=wl.dtype, device=device)
    pages, rows = token_page_rows(wl)
    pi = torch.from_numpy(pages).to(device)
    ri = torch.from_numpy(rows).to(device)
    kc[pi, ri] = wl.k_tokens.to(device)
    vc[pi, ri] = wl.v_tokens.to(device)
    return kc, vc


def compact_pool(wl: Workload, poison: bool = True):
    """CPU copy of only the used pages: (page_ids, k_pages, v_pages).

    page_ids is sorted; k_pages[i] holds physical page page_ids[i].
    """
    ids = wl.used_pages
    shape = (ids.shape[0], wl.page_size, wl.num_kv_heads, wl.head_dim)
    fill = float("nan") if poison else 0.0
    kp = torch.full(shape, fill, dtype=wl.dtype)
    vp = torch.full(shape, fill, dtype=wl.dtype)
    pages, rows = token_page_rows(wl)
    idx = torch.from_numpy(np.searchsorted(ids, pages))
    ri = torch.from_numpy(rows)
    kp[idx, ri] = wl.k_tokens
    vp[idx, ri] = wl.v_tokens
    return ids, kp, vp
