"""KV read accounting.  TEST INFRASTRUCTURE.

What the DeFT pages count:
* The abstract of arXiv 2404.00242 reports the KV-cache IO that KV-Guided
  Grouping removes: the shared prefix is loaded once instead of once per
  query.  "DeFT Guide ... The Tree-Attention Bottleneck" describes the naive
  pattern: every branch's thread block re-reads the whole shared prefix.
* The simulator in "End-to-End Implementation: DeFT Flash Tree-Attention
  Simulator in PyTorch" counts token loads: +2 per token for its K and V,
  the prefix tiles once for all queries, then every ancestor-or-self tree
  token once per query; its baseline counts every query reading the whole
  prefix plus a fixed four tree tokens.

Byte accounting used for the MI355X measurements:
  ideal (grouped) KV bytes = T * 2 * Hkv * d * elem_bytes  (each token once)
  naive KV bytes           = sum over queries of path_len(q) * 2 * Hkv * d * eb
"""
from __future__ import annotations

import numpy as np

from .attention import path_nodes


def path_lengths(parents, seg_lens, query_nodes) -> np.ndarray:
    return np.array([sum(int(seg_lens[n]) for n in path_nodes(parents, int(x)))
                     for x in query_nodes], dtype=np.int64)


def ideal_kv_bytes(seg_lens, hkv: int, d: int, elem_bytes: int) -> int:
    return int(np.sum(seg_lens, dtype=np.int64)) * 2 * hkv * d * elem_bytes


def naive_kv_bytes(parents, seg_lens, query_nodes, hkv: int, d: int, elem_bytes: int) -> int:
    return int(path_lengths(parents, seg_lens, query_nodes).sum()) * 2 * hkv * d * elem_bytes


def simulator_grouped_reads(tree_parents, query_node_ids, prefix_len: int, tile: int) -> int:
    """Token loads the simulator counts for its grouped run.

    Prefix: tiles of `tile` tokens, each token counted twice (K and V), once
    for all queries.  Tree: one token per tree node; each query counts two
    loads per node on its ancestor-or-self list.
    """
    reads = 0
    for t0 in range(0, prefix_len, tile):
        reads += (min(t0 + tile, prefix_len) - t0) * 2
    for node in query_node_ids:
        reads += 2 * len(path_nodes(tree_parents, int(node)))
    return reads


def simulator_baseline_reads(num_queries: int, prefix_len: int, tree_tokens_per_query: int = 4) -> int:
    """The simulator's baseline: each query reads the prefix and a fixed
    number of tree tokens, two loads (K, V) per token."""
    return num_queries * prefix_len * 2 + num_queries * tree_tokens_per_query * 2


def reduction_percent(new: int, old: int) -> float:
    return (1.0 - new / old) * 100.0
