"""Tree-constrained attention, by definition, in fp64.  TEST INFRASTRUCTURE.

Source: "DeFT Guide: Flash Tree-Attention for LLM Serving", section "Deep
Dive: Mathematical Formulation", subsection "Tree-Constrained Attention
Formulation": for candidate query i, A_i = softmax((q_i K^T + M_i)/sqrt(d_k)) V,
with M_i zero on tokens of the prefix and of the query's ancestors and -inf
elsewhere.  The same page's simulator ("End-to-End Implementation") counts a
node as its own ancestor, so a query sees its own node too.

Readings where the pages leave a point open:
  * the prefix is the root node's segment; every node owns a KV segment;
    a query sees the segments of its node and of every ancestor;
  * the mask is applied as a selection (masked tokens are left out), which
    equals adding -inf before the softmax;
  * scale = 1/sqrt(d), d the head dimension;
  * grouped-query attention: query head h reads KV head h // (Hq / Hkv);
  * no epsilon in the normalisation (the simulator adds 1e-8; the formula
    does not, and the denominator is at least 1 after max subtraction).

Multi-token query nodes (tree prefill, speculative nodes that hold several
draft tokens): the pages define M_i only by ancestry, so the plainest reading
that keeps ordinary causal attention inside one node is taken: a query may sit
at a position inside its node and then sees the ancestors' segments and its
own node's tokens up to and including its position (query_lens[i] leading
tokens of the node).  With query_lens[i] = seg_lens[node] this is the decode
case above.

Paged KV ("Production Engineering ... Integration with Paged KV Caches"):
logical token t lives in pool page block_table[t // page_size], row
t % page_size.  Logical order is node segments concatenated in node-id order.

The partial convention (used to check per-chunk partial results) follows the
"Online Softmax Tile Accumulation" subsection: over a subset of the tokens,
m = max of the scaled scores, l = sum exp(s - m), O = sum exp(s - m) v
(unnormalised).  Partials over disjoint subsets combine by the log-sum-exp
merge that the same subsection's running-max update implies.
"""
from __future__ import annotations

import numpy as np


def node_starts(seg_lens) -> np.ndarray:
    """Logical start of each node's segment: exclusive prefix sum (int64)."""
    seg = np.asarray(seg_lens, dtype=np.int64)
    out = np.zeros_like(seg)
    if seg.size > 1:
        out[1:] = np.cumsum(seg)[:-1]
    return out


def path_nodes(parents, node: int) -> list:
    """The node and all its ancestors, walking parent links up to -1."""
    out = []
    n = int(node)
    while n >= 0:
        out.append(n)
        n = int(parents[n])
    return out


def path_tokens(parents, seg_lens, node: int, own_len=None) -> np.ndarray:
    """Logical token ids visible to a query on `node` (root segment first).

    own_len: how many leading tokens of `node` itself the query sees (None:
    the whole segment)."""
    starts = node_starts(seg_lens)
    nodes = path_nodes(parents, node)[::-1]
    if not nodes:
        return np.zeros(0, dtype=np.int64)
    lens = [int(seg_lens[n]) for n in nodes]
    if own_len is not None:
        if not 1 <= int(own_len) <= lens[-1]:
            raise ValueError("own_len must lie in [1, seg_lens[node]]")
        lens[-1] = int(own_len)
    return np.concatenate([np.arange(starts[n], starts[n] + ln, dtype=np.int64)
                           for n, ln in zip(nodes, lens)])


def gather_tokens(pool, tokens, block_table, page_size=16, page_ids=None) -> np.ndarray:
    """Rows of a paged pool for logical `tokens`, as fp64 [n, Hkv, d].

    pool is [P', page_size, Hkv, d]; page_ids (sorted) names the physical
    page each of its P' rows holds (default: row i holds page i).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    phys = np.asarray(block_table, dtype=np.int64)[tokens // page_size]
    row = phys if page_ids is None else np.searchsorted(np.asarray(page_ids), phys)
    if page_ids is not None and not np.array_equal(np.asarray(page_ids)[row], phys):
        raise KeyError("a logical token maps to a page missing from the pool copy")
    return np.asarray(pool, dtype=np.float64)[row, tokens % page_size]


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float() if str(x.dtype) == "torch.bfloat16" else x.detach().cpu()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def attend(qh: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(qh k^T * scale) v for one KV head: qh [G,d], k,v [n,d] -> [G,d]."""
    s = (qh @ k.T) * scale                      # [G, n]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def tree_attention(q, k_pool, v_pool, block_table, parents, seg_lens, query_nodes,
                   page_size: int = 16, page_ids=None, queries=None, query_lens=None) -> np.ndarray:
    """Reference output [len(queries), Hq, d] in fp64.

    q: [Nq, Hq, d]; k_pool, v_pool: [P', page_size, Hkv, d]; queries: indices
    into query_nodes to evaluate (default all of them); query_lens: per query,
    the leading tokens of its own node it sees (None: every token).
    """
    q = _as_f64(q)
    kp, vp = _as_f64(k_pool), _as_f64(v_pool)
    nq, hq, d = q.shape
    hkv = kp.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    grp = hq // hkv
    scale = 1.0 / np.sqrt(d)
    sel = range(nq) if queries is None else queries
    out = []
    for i in sel:
        own = None if query_lens is None else int(query_lens[i])
        toks = path_tokens(parents, seg_lens, int(query_nodes[i]), own)
        k = gather_tokens(kp, toks, block_table, page_size, page_ids)
        v = gather_tokens(vp, toks, block_table, page_size, page_ids)
        o = np.empty((hq, d))
        for g in range(hkv):
            hs = slice(g * grp, (g + 1) * grp)
            o[hs] = attend(q[i, hs], k[:, g], v[:, g], scale)
        out.append(o)
    return np.stack(out) if out else np.zeros((0, hq, d))


def partial(qh: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Unnormalised partial over one token subset: (O [G,d], m [G], l [G]).

    m is the max scaled score (natural-log domain), l = sum exp(s - m) and
    O = sum exp(s - m) v.  An empty subset gives m = -inf, l = 0, O = 0.
    """
    g, d = qh.shape
    if k.shape[0] == 0:
        return np.zeros((g, d)), np.full(g, -np.inf), np.zeros(g)
    s = (qh @ k.T) * scale
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    return p @ v, m, p.sum(axis=1)


def lse_merge(os_, ms, ls) -> np.ndarray:
    """Combine partials (O_j, m_j, l_j) over disjoint token sets.

    M = max_j m_j; weights w_j = exp(m_j - M); result = sum w_j O_j / sum w_j l_j.
    os_: [n, G, d]; ms, ls: [n, G].
    """
    os_ = np.asarray(os_, dtype=np.float64)
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    big = ms.max(axis=0)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - big[None, :]))
    num = (w[:, :, None] * os_).sum(axis=0)
    den = (w * ls).sum(axis=0)
    return num / den[:, None]


def chunk_partials(q, k_pool, v_pool, block_table, parents, seg_lens, query_nodes, plan,
                   page_size: int = 16, page_ids=None, query_lens=None):
    """Per-slot partials over the chunks of a reference plan.

    For slot s (chunk c, query qi): the chunk's flat tokens that qi sees (the
    path tokens of path_tokens), mapped to logical ids by the plan's
    flattening.  Visibility comes from the path walk, not from the plan's
    bitmasks.
    Returns O [S, Hq, d], m [S, Hq], l [S, Hq] in fp64.
    """
    q = _as_f64(q)
    kp, vp = _as_f64(k_pool), _as_f64(v_pool)
    nq, hq, d = q.shape
    hkv = kp.shape[2]
    grp = hq // hkv
    scale = 1.0 / np.sqrt(d)
    f2l = plan["flat_to_logical"].astype(np.int64)
    cs = plan["chunk_start"]
    go = plan["group_offsets"]
    sq = plan["slot_query"]
    s_tot = int(go[-1])
    o_out = np.zeros((s_tot, hq, d))
    m_out = np.full((s_tot, hq), -np.inf)
    l_out = np.zeros((s_tot, hq))
    for c in range(len(cs) - 1):
        f = np.arange(int(cs[c]), int(cs[c + 1]), dtype=np.int64)
        for s in range(int(go[c]), int(go[c + 1])):
            qi = int(sq[s])
            own = None if query_lens is None else int(query_lens[qi])
            seen = np.isin(f2l[f], path_tokens(parents, seg_lens, int(query_nodes[qi]), own))
            toks = f2l[f[seen]]
            k = gather_tokens(kp, toks, block_table, page_size, page_ids)
            v = gather_tokens(vp, toks, block_table, page_size, page_ids)
            for g in range(hkv):
                hs = slice(g * grp, (g + 1) * grp)
                o_out[s, hs], m_out[s, hs], l_out[s, hs] = partial(q[qi, hs], k[:, g], v[:, g], scale)
    return o_out, m_out, l_out
