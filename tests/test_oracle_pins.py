"""Pins for the fp64 oracle: each checks it against something other than itself.

  * a single chain of one-token nodes is ordinary causal attention, and one
    query at the end of a chain is ordinary decode attention (torch's
    scaled_dot_product_attention in float64, KV heads repeated per group);
  * partials over any split of a query's tokens, merged by log-sum-exp,
    equal the unsplit result (the online-softmax identity);
  * relabelling sibling nodes (which changes the flattening and the plan)
    leaves every query's output unchanged;
  * a brute-force scalar loop over every pool row with ancestor sets built
    by closure (not by walking parents) agrees on tiny trees, also with
    multi-token query nodes;
  * one multi-token node with a query per token is causal self-attention,
    and multi-token branches under a prefix are causal over their own path;
  * closed forms: zero keys make the softmax uniform, so the output is the
    token-count-weighted mean of per-node value patterns; constant values
    give that constant back;
  * the read counts printed by the DeFT Guide's simulator.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import io_model as IO
from oracle.plan import ref_plan
from tree_structured_decode_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _wl(parents, seg, queries, hq, hkv, d, seed, placement="permuted", dtype=torch.float32):
    return W.make_workload("t", parents, seg, queries, chunk_tokens=16, hq=hq, hkv=hkv, d=d,
                           dtype=dtype, seed=seed, placement=placement,
                           pool_pages=None if placement != "scattered" else 3 * (-(-int(np.sum(seg)) // 16)) + 5)


def _oracle(wl, **kw):
    ids, kp, vp = W.compact_pool(wl)
    return OA.tree_attention(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens, wl.query_nodes,
                             page_ids=ids, **kw)


def _sdpa(q, k, v, causal):
    """torch SDPA in float64; q [L,Hq,d], k/v [S,Hkv,d] -> [L,Hq,d]."""
    hq, hkv = q.shape[1], k.shape[1]
    k = k.repeat_interleave(hq // hkv, dim=1)
    v = v.repeat_interleave(hq // hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1).double(), k.transpose(0, 1).double(), v.transpose(0, 1).double(),
        is_causal=causal)
    return o.transpose(0, 1).numpy()


@pytest.mark.parametrize("seed", range(4))
def test_single_chain_of_one_token_nodes_is_causal_attention(seed):
    n = 37
    parents = np.arange(-1, n - 1, dtype=np.int32)
    seg = np.ones(n, dtype=np.int32)
    queries = np.arange(n, dtype=np.int32)
    wl = _wl(parents, seg, queries, hq=6, hkv=2, d=16, seed=seed)
    got = _oracle(wl)
    want = _sdpa(wl.q, wl.k_tokens, wl.v_tokens, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_query_at_end_of_chain_is_decode_attention(seed):
    rng = np.random.default_rng(seed)
    n = 6
    parents = np.arange(-1, n - 1, dtype=np.int32)
    seg = rng.integers(1, 40, size=n).astype(np.int32)
    wl = _wl(parents, seg, [n - 1, n - 1], hq=8, hkv=2, d=32, seed=seed, placement="scattered")
    got = _oracle(wl)
    want = _sdpa(wl.q, wl.k_tokens, wl.v_tokens, causal=False)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_split_then_merge_equals_unsplit(seed):
    rng = np.random.default_rng(100 + seed)
    p, s, qn = W.random_tree(rng, 12, 1, 30, 5)
    wl = _wl(p, s, qn, hq=4, hkv=2, d=16, seed=seed)
    ids, kp, vp = W.compact_pool(wl)
    full = OA.tree_attention(wl.q, kp, vp, wl.block_table, p, s, qn, page_ids=ids)
    q = wl.q.double().numpy()
    for i in range(len(qn)):
        toks = OA.path_tokens(p, s, qn[i])
        pieces = rng.integers(0, 5, size=toks.shape[0])       # arbitrary, non-contiguous split
        k = OA.gather_tokens(kp, toks, wl.block_table, 16, ids)
        v = OA.gather_tokens(vp, toks, wl.block_table, 16, ids)
        for g in range(2):
            parts = [OA.partial(q[i, 2 * g:2 * g + 2], k[pieces == j, g], v[pieces == j, g], 0.25)
                     for j in range(6)]                      # piece 5 is always empty
            merged = OA.lse_merge([x[0] for x in parts], [x[1] for x in parts], [x[2] for x in parts])
            np.testing.assert_allclose(merged, full[i, 2 * g:2 * g + 2], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", range(8))
def test_chunk_partials_merge_to_tree_attention(seed):
    """Per-slot partials over a plan's chunks, merged along each query's
    slot list, give the unsplit attention (with and without multi-token
    query nodes); every slot holds at least one token (finite m, l > 0)."""
    rng = np.random.default_rng(700 + seed)
    p, s, qn = W.random_tree(rng, int(rng.integers(2, 15)), 1, 40, int(rng.integers(1, 8)), forest_prob=0.2)
    ql = None if seed % 2 == 0 else np.array([int(rng.integers(1, s[x] + 1)) for x in qn], np.int32)
    wl = W.make_workload("cp", p, s, qn, chunk_tokens=16, hq=4, hkv=2, d=8, dtype=torch.float32,
                         seed=seed, placement="permuted", query_lens=ql)
    c = int(rng.choice([3, 16, 50]))
    plan = ref_plan(p, s, qn, c, query_lens=ql)
    ids, kp, vp = W.compact_pool(wl)
    o, m, l = OA.chunk_partials(wl.q, kp, vp, wl.block_table, p, s, qn, plan, page_ids=ids, query_lens=ql)
    assert np.isfinite(m).all() and (l > 0).all()
    full = OA.tree_attention(wl.q, kp, vp, wl.block_table, p, s, qn, page_ids=ids, query_lens=ql)
    qso, qs = plan["query_slot_offsets"], plan["query_slots"]
    for i in range(len(qn)):
        sl = qs[qso[i]:qso[i + 1]]
        np.testing.assert_allclose(OA.lse_merge(o[sl], m[sl], l[sl]), full[i], rtol=1e-12, atol=1e-12)


def _relabel_siblings(parents, seg, queries, rng):
    """Renumber nodes breadth-first with each node's children shuffled."""
    n = len(parents)
    kids = [[] for _ in range(n)]
    roots = []
    for i, par in enumerate(parents):
        (roots if par < 0 else kids[par]).append(i)
    rng.shuffle(roots)
    order, frontier = [], list(roots)
    while frontier:
        x = frontier.pop(0)
        order.append(x)
        ch = list(kids[x])
        rng.shuffle(ch)
        frontier.extend(ch)
    new = {old: i for i, old in enumerate(order)}
    np_ = np.array([-1 if parents[o] < 0 else new[int(parents[o])] for o in order], np.int32)
    ns = np.array([seg[o] for o in order], np.int32)
    nq = np.array([new[int(x)] for x in queries], np.int32)
    return np_, ns, nq, order


@pytest.mark.parametrize("seed", range(5))
def test_reordering_siblings_keeps_outputs(seed):
    rng = np.random.default_rng(200 + seed)
    p, s, qn = W.random_tree(rng, 15, 1, 20, 7, forest_prob=0.1)
    wl = _wl(p, s, qn, hq=4, hkv=1, d=8, seed=seed)
    base = _oracle(wl)
    p2, s2, q2, order = _relabel_siblings(p, s, qn, rng)
    # move each node's KV rows with it
    st = OA.node_starts(s)
    idx = np.concatenate([np.arange(st[o], st[o] + s[o]) for o in order])
    wl2 = W.make_workload("t2", p2, s2, q2, chunk_tokens=16, hq=4, hkv=1, d=8,
                          dtype=torch.float32, seed=seed, placement="permuted")
    wl2.q = wl.q.clone()
    wl2.k_tokens = wl.k_tokens[torch.from_numpy(idx)].clone()
    wl2.v_tokens = wl.v_tokens[torch.from_numpy(idx)].clone()
    got = _oracle(wl2)
    np.testing.assert_allclose(got, base, rtol=1e-12, atol=1e-12)
    # the relabelling really changes the flattened layout
    if seed == 0:
        assert not np.array_equal(ref_plan(p, s, qn, 7)["flat_to_logical"],
                                  ref_plan(p2, s2, q2, 7)["flat_to_logical"][np.argsort(idx)])


def _brute(wl):
    """Scalar loops over every pool row; ancestors by closure in id order."""
    n = len(wl.parents)
    anc = []
    for i in range(n):                      # parents[i] < i, so the parent's set is ready
        a = {i}
        if wl.parents[i] >= 0:
            a |= anc[wl.parents[i]]
        anc.append(a)
    bounds = []
    acc = 0
    for i in range(n):
        bounds.append((acc, acc + int(wl.seg_lens[i])))
        acc += int(wl.seg_lens[i])
    inv = {int(pg): j for j, pg in enumerate(wl.block_table)}
    ids, kp, vp = W.compact_pool(wl)
    kp, vp = kp.double().numpy(), vp.double().numpy()
    q = wl.q.double().numpy()
    nq, hq, d = q.shape
    hkv = kp.shape[2]
    out = np.zeros((nq, hq, d))
    for qi in range(nq):
        for h in range(hq):
            g = h // (hq // hkv)
            scores, vals = [], []
            for row, page in enumerate(ids):
                for r in range(wl.page_size):
                    if int(page) not in inv:
                        continue
                    t = inv[int(page)] * wl.page_size + r
                    if t >= acc:
                        continue
                    node = next(j for j, (a, b) in enumerate(bounds) if a <= t < b)
                    if node not in anc[int(wl.query_nodes[qi])]:
                        continue
                    if (wl.query_lens is not None and node == int(wl.query_nodes[qi])
                            and t - bounds[node][0] >= int(wl.query_lens[qi])):
                        continue
                    dot = 0.0
                    for x in range(d):
                        dot += q[qi, h, x] * kp[row, r, g, x]
                    scores.append(dot / math.sqrt(d))
                    vals.append(vp[row, r, g])
            mx = max(scores)
            w = [math.exp(sc - mx) for sc in scores]
            tot = sum(w)
            for x in range(d):
                out[qi, h, x] = sum(wi * vv[x] for wi, vv in zip(w, vals)) / tot
    return out


@pytest.mark.parametrize("seed", range(120))
def test_brute_force_tiny_trees(seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 9))
    p, s, qn = W.random_tree(rng, n, 1, 5, int(rng.integers(1, 5)), forest_prob=0.2)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2, 3]))
    d = int(rng.choice([1, 3, 8]))
    wl = W.make_workload("b", p, s, qn, chunk_tokens=4, hq=hq, hkv=hkv, d=d, dtype=torch.float32,
                         seed=seed, placement="scattered", pool_pages=int(rng.integers(2, 9)) + (-(-int(s.sum()) // 16)))
    np.testing.assert_allclose(_oracle(wl), _brute(wl), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(60))
def test_brute_force_tiny_trees_multi_token(seed):
    """Multi-token query nodes: the query at position j of its node sees the
    node's first j + 1 tokens (brute force, closure ancestor sets)."""
    rng = np.random.default_rng(350 + seed)
    n = int(rng.integers(1, 8))
    p, s, qn = W.random_tree(rng, n, 1, 6, int(rng.integers(1, 6)), forest_prob=0.2)
    ql = np.array([int(rng.integers(1, s[x] + 1)) for x in qn], dtype=np.int32)
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.choice([1, 2]))
    wl = W.make_workload("bm", p, s, qn, chunk_tokens=4, hq=hq, hkv=hkv, d=int(rng.choice([2, 5])),
                         dtype=torch.float32, seed=seed, placement="permuted", query_lens=ql)
    np.testing.assert_allclose(_oracle(wl, query_lens=ql), _brute(wl), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_one_multi_token_node_is_causal_attention(seed):
    """A single node of L tokens with a query on each token (tree prefill of
    one segment) is ordinary causal self-attention."""
    L = 45
    p, s, qn = np.array([-1]), np.array([L]), np.zeros(L, dtype=np.int32)
    ql = np.arange(1, L + 1, dtype=np.int32)
    wl = _wl(p, s, qn, hq=4, hkv=2, d=16, seed=seed)
    got = _oracle(wl, query_lens=ql)
    want = _sdpa(wl.q, wl.k_tokens, wl.v_tokens, causal=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_multi_token_branches_are_causal_over_their_path(seed):
    """Prefix plus two multi-token branches: each branch's queries give the
    last rows of causal attention over prefix ++ that branch, untouched by
    the sibling branch."""
    rng = np.random.default_rng(600 + seed)
    lp, la, lb = int(rng.integers(3, 30)), int(rng.integers(2, 20)), int(rng.integers(2, 20))
    p = np.array([-1, 0, 0], dtype=np.int32)
    s = np.array([lp, la, lb], dtype=np.int32)
    qn = np.array([1] * la + [2] * lb, dtype=np.int32)
    ql = np.concatenate([np.arange(1, la + 1), np.arange(1, lb + 1)]).astype(np.int32)
    wl = _wl(p, s, qn, hq=6, hkv=3, d=8, seed=seed, placement="scattered")
    got = _oracle(wl, query_lens=ql)
    for node, rows, (a, b) in ((1, slice(0, la), (lp, lp + la)), (2, slice(la, la + lb), (lp + la, lp + la + lb))):
        kk = torch.cat([wl.k_tokens[:lp], wl.k_tokens[a:b]])
        vv = torch.cat([wl.v_tokens[:lp], wl.v_tokens[a:b]])
        qq = torch.cat([torch.zeros_like(wl.q[:lp]), wl.q[rows]])
        want = _sdpa(qq, kk, vv, causal=True)[lp:]
        np.testing.assert_allclose(got[rows], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_zero_keys_give_segment_weighted_mean(seed):
    rng = np.random.default_rng(400 + seed)
    p, s, qn = W.random_tree(rng, 20, 1, 40, 10, forest_prob=0.1)
    d = 24
    wl = _wl(p, s, qn, hq=4, hkv=2, d=d, seed=seed, placement="scattered")
    wl.k_tokens.zero_()
    st = OA.node_starts(s)
    pattern = np.zeros((len(p), d))
    for node in range(len(p)):
        pattern[node, node % d] = node + 1.0
        wl.v_tokens[st[node]:st[node] + s[node]] = torch.from_numpy(pattern[node]).float()
    got = _oracle(wl)
    for i, node in enumerate(qn):
        path = OA.path_nodes(p, node)
        want = sum(s[x] * pattern[x] for x in path) / sum(s[x] for x in path)
        np.testing.assert_allclose(got[i], np.broadcast_to(want, got[i].shape), rtol=0, atol=1e-12)


def test_constant_values_return_the_constant():
    rng = np.random.default_rng(5)
    p, s, qn = W.random_tree(rng, 30, 1, 50, 12)
    wl = _wl(p, s, qn, hq=8, hkv=4, d=16, seed=1)
    c = torch.linspace(-3, 3, 16)
    wl.v_tokens[:] = c
    got = _oracle(wl)
    np.testing.assert_allclose(got, np.broadcast_to(c.double().numpy(), got.shape), rtol=0, atol=1e-14)


def test_simulator_printed_read_counts():
    with open(os.path.join(GOLDEN, "simulator_io.json")) as f:
        g = json.load(f)
    nq, prefix, tile = g["setup"]["num_queries"], g["setup"]["prefix_len"], g["setup"]["tile"]
    heap = np.array([-1] + [(i - 1) // 2 for i in range(1, nq)], dtype=np.int32)
    base = IO.simulator_baseline_reads(nq, prefix, g["setup"]["baseline_tree_tokens_per_query"])
    grouped = IO.simulator_grouped_reads(heap, range(nq), prefix, tile)
    assert base == g["printed"]["conventional_reads"]
    assert grouped == g["derived_from_the_listed_counting_rule"]["deft_reads"]
    assert round(IO.reduction_percent(grouped, base), 1) == g["printed"]["reduction_percent_one_decimal"]
    assert round(IO.reduction_percent(g["printed"]["deft_reads"], base), 1) == g["printed"]["reduction_percent_one_decimal"]


def test_kv_byte_accounting_closed_forms():
    # shared prompt of 2048 with 32 branches of 512, one query per branch
    p, s, qn = W.shared_prompt_branches(2048, 32, 512)
    assert IO.ideal_kv_bytes(s, 8, 128, 2) == (2048 + 32 * 512) * 2 * 8 * 128 * 2
    assert IO.naive_kv_bytes(p, s, qn, 8, 128, 2) == 32 * (2048 + 512) * 2 * 8 * 128 * 2
    assert round(IO.reduction_percent(IO.ideal_kv_bytes(s, 8, 128, 2), IO.naive_kv_bytes(p, s, qn, 8, 128, 2)), 2) == 77.5
    # the tiny binary tree: four leaf queries, each path 256 + 32 + 32
    p, s, qn = W.binary_tree_4_leaves()
    assert IO.naive_kv_bytes(p, s, qn, 1, 64, 4) == 4 * 320 * 2 * 64 * 4
    assert IO.ideal_kv_bytes(s, 1, 64, 4) == 448 * 2 * 64 * 4
