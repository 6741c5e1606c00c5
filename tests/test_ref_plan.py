"""Pins for the reference planner: a hand-worked example, brute-force masks
from ancestor sets built by closure, and the layout invariants."""
import json
import os

import numpy as np
import pytest

from oracle.plan import PlanError, ref_plan, ref_plan_node_chunks, ref_plan_query_centric
from tree_structured_decode_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_tiny_binary_tree():
    with open(os.path.join(GOLDEN, "plan_tiny_binary_tree_c64.json")) as f:
        g = json.load(f)
    t, e = g["tree"], g["expect"]
    pl = ref_plan(t["parents"], t["seg_lens"], t["query_nodes"], t["chunk_tokens"])
    for key in ("total_tokens", "num_chunks", "num_slots", "mask_words"):
        assert pl[key] == e[key], key
    for key in ("node_start", "flat_node_order", "node_flat_start", "chunk_start", "group_offsets",
                "slot_query", "chunk_full", "query_slot_offsets", "query_slots"):
        assert pl[key].tolist() == e[key], key
    assert pl["slot_mask"].tolist() == e["slot_mask"]
    f2l = np.empty(e["total_tokens"], dtype=np.int64)
    for fs, ls, n in e["flat_to_logical_runs"]:
        f2l[fs:fs + n] = np.arange(ls, ls + n)
    assert pl["flat_to_logical"].tolist() == f2l.tolist()
    lens = np.diff(pl["chunk_start"])
    go = pl["group_offsets"]
    assert int(sum(lens[c] * (go[c + 1] - go[c]) for c in range(pl["num_chunks"]))) == e["computed_token_query_pairs"]
    assert int(sum(bin(int(w)).count("1") for w in pl["slot_mask"].ravel())) == e["useful_token_query_pairs"]


def _ancestor_sets(parents):
    anc = []
    for i, p in enumerate(parents):
        a = {i}
        if p >= 0:
            a |= anc[p]
        anc.append(a)
    return anc


def check_plan_invariants(pl, parents, seg, queries, c, query_lens=None):
    n, nq = len(parents), len(queries)
    total = int(np.sum(seg))
    assert pl["total_tokens"] == total
    # flattening is a permutation and each node's segment stays contiguous and in order
    f2l = pl["flat_to_logical"].astype(np.int64)
    assert sorted(f2l.tolist()) == list(range(total))
    ns, nfs = pl["node_start"], pl["node_flat_start"]
    for x in range(n):
        assert (f2l[nfs[x]:nfs[x] + seg[x]] == np.arange(ns[x], ns[x] + seg[x])).all()
    # pre-order: a subtree occupies one flat interval starting at its root
    sub = np.array(seg, dtype=np.int64)
    for x in range(n - 1, -1, -1):
        if parents[x] >= 0:
            sub[parents[x]] += sub[x]
    for x in range(n):
        if parents[x] >= 0:
            p = parents[x]
            assert nfs[p] + seg[p] <= nfs[x] and nfs[x] + sub[x] <= nfs[p] + sub[p]
    # chunks: equal C except the last, covering [0, T)
    cs = pl["chunk_start"]
    assert cs[0] == 0 and cs[-1] == total
    lens = np.diff(cs)
    assert (lens[:-1] == c).all() and 1 <= lens[-1] <= c
    # masks against ancestor sets built by closure
    anc = _ancestor_sets(parents)
    flat_node = np.empty(total, dtype=np.int64)
    for x in range(n):
        flat_node[nfs[x]:nfs[x] + seg[x]] = x
    go, sq, sm = pl["group_offsets"], pl["slot_query"], pl["slot_mask"]
    words = -(-c // 32)
    assert sm.shape == (pl["num_slots"], words)
    own_len = list(seg[queries]) if query_lens is None else list(query_lens)

    def sees(qi, f):
        x = flat_node[f]
        return x in anc[queries[qi]] and (x != queries[qi] or f - nfs[x] < own_len[qi])

    for k in range(len(cs) - 1):
        members = []
        for qi in range(nq):
            vis = [sees(qi, f) for f in range(cs[k], cs[k + 1])]
            if any(vis):
                members.append((qi, vis))
        assert go[k + 1] - go[k] == len(members)
        full = bool(members) and all(all(v) for _, v in members)
        assert pl["chunk_full"][k] == int(full)
        for j, (qi, vis) in enumerate(members):
            s = go[k] + j
            assert sq[s] == qi
            bits = [(int(sm[s, t >> 5]) >> (t & 31)) & 1 for t in range(words * 32)]
            assert bits[:len(vis)] == [int(v) for v in vis]
            assert not any(bits[len(vis):])
    # merge lists: each query's slots in ascending chunk order; popcounts give path lengths
    qso, qs = pl["query_slot_offsets"], pl["query_slots"]
    for qi in range(nq):
        mine = qs[qso[qi]:qso[qi + 1]].tolist()
        assert mine == sorted(mine) and all(sq[s] == qi for s in mine)
        pop = sum(bin(int(w)).count("1") for s in mine for w in sm[s])
        assert pop == sum(seg[x] for x in anc[queries[qi]]) - seg[queries[qi]] + own_len[qi]
    assert qso[-1] == pl["num_slots"]


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("c", [1, 7, 16, 64, 100, 128])
def test_random_trees_against_closure(seed, c):
    rng = np.random.default_rng(seed * 31 + c)
    n = int(rng.integers(1, 40))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 3, 60])), int(rng.integers(1, 12)),
                             forest_prob=0.15)
    check_plan_invariants(ref_plan(p, s, qn, c), p, s, qn, c)


@pytest.mark.parametrize("seed", range(40))
@pytest.mark.parametrize("c", [1, 7, 32, 100])
def test_multi_token_plans_against_closure(seed, c):
    """Multi-token query nodes: the query sees its node's first query_lens
    tokens; groups hold only queries that see a token of the chunk."""
    rng = np.random.default_rng(7100 + seed * 13 + c)
    n = int(rng.integers(1, 30))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([2, 9, 70])), int(rng.integers(1, 12)),
                             forest_prob=0.15)
    ql = np.array([int(rng.integers(1, s[x] + 1)) for x in qn], dtype=np.int32)
    check_plan_invariants(ref_plan(p, s, qn, c, query_lens=ql), p, s, qn, c, query_lens=ql)


def test_multi_token_full_lengths_are_the_tree_plan():
    rng = np.random.default_rng(77)
    p, s, qn = W.random_tree(rng, 25, 1, 40, 9, forest_prob=0.1)
    a = ref_plan(p, s, qn, 16, query_lens=s[qn])
    b = ref_plan(p, s, qn, 16)
    for k in b:
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


def test_multi_token_workload_plan():
    wl = W.standard_workload(6)
    pl = ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, query_lens=wl.query_lens)
    check_plan_invariants(pl, wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens,
                          query_lens=wl.query_lens)


def test_multi_token_rejects_bad_lengths():
    for ql in ([0], [5], [1, 1]):
        with pytest.raises(PlanError):
            ref_plan([-1, 0], [3, 4], [1], 4, query_lens=ql)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_standard_workload_plans(cfg):
    wl = W.standard_workload(cfg)
    pl = ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
    if cfg in (1, 2, 3):
        check_plan_invariants(pl, wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
    assert pl["num_slots"] == pl["query_slot_offsets"][-1]


def test_rejects_bad_input():
    ok = ([-1, 0], [3, 4], [1])
    with pytest.raises(PlanError) as e:
        ref_plan([-1, 1], [3, 4], [1], 4)
    assert e.value.kind == "invalid_tree"
    with pytest.raises(PlanError) as e:
        ref_plan([-1, -2], [3, 4], [1], 4)
    assert e.value.kind == "invalid_tree"
    with pytest.raises(PlanError) as e:
        ref_plan(ok[0], [3, 0], ok[2], 4)
    assert e.value.kind == "invalid_tree"
    with pytest.raises(PlanError) as e:
        ref_plan(ok[0], ok[1], [2], 4)
    assert e.value.kind == "invalid_tree"
    with pytest.raises(PlanError) as e:
        ref_plan(*ok, 0)
    assert e.value.kind == "invalid_argument"
    with pytest.raises(PlanError) as e:
        ref_plan(ok[0], ok[1], [], 4)
    assert e.value.kind == "invalid_argument"


@pytest.mark.parametrize("seed", range(30))
def test_query_centric_plan_covers_each_path_once(seed):
    """Each query's run of the query-centric plan holds exactly the logical
    tokens it may see (ancestor sets by closure, not by walking paths), once
    each; every chunk is one full single-query slot within one run."""
    rng = np.random.default_rng(9100 + seed)
    n = int(rng.integers(1, 30))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 4, 40])), int(rng.integers(1, 9)),
                             forest_prob=float(rng.choice([0.0, 0.4])))
    c = int(rng.choice([1, 5, 32, 64]))
    plan = ref_plan_query_centric(p, s, qn, c)
    anc = _ancestor_sets(p)
    starts = np.concatenate([[0], np.cumsum(s)])
    f2l = plan["flat_to_logical"]
    cs = plan["chunk_start"]
    qso = plan["query_slot_offsets"]
    assert plan["num_slots"] == plan["num_chunks"] == len(cs) - 1
    assert (plan["chunk_full"] == 1).all()
    assert (plan["group_offsets"] == np.arange(plan["num_chunks"] + 1)).all()
    for qi, node in enumerate(qn):
        want = sorted(t for x in anc[int(node)] for t in range(starts[x], starts[x + 1]))
        ks = range(qso[qi], qso[qi + 1])
        assert all(plan["slot_query"][k] == qi for k in ks)
        got = [int(t) for k in ks for t in f2l[cs[k]:cs[k + 1]]]
        assert sorted(got) == want and len(got) == len(set(got))
        for k in ks:
            assert 1 <= cs[k + 1] - cs[k] <= c
            nbits = sum(bin(int(w)).count("1") for w in plan["slot_mask"][k])
            assert nbits == cs[k + 1] - cs[k]


@pytest.mark.parametrize("seed", range(30))
def test_node_chunk_plan_invariants(seed):
    """Node-granularity chunks: the tree plan's flat layout; no chunk crosses
    a node (each chunk lies in one node's flat interval, at most C long);
    every query's slots cover exactly its visible tokens (closure ancestor
    sets), once each; every slot row is all ones."""
    rng = np.random.default_rng(9300 + seed)
    n = int(rng.integers(1, 30))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 4, 40])), int(rng.integers(1, 9)),
                             forest_prob=float(rng.choice([0.0, 0.4])))
    c = int(rng.choice([1, 5, 32, 64]))
    plan = ref_plan_node_chunks(p, s, qn, c)
    tree = ref_plan(p, s, qn, c)
    assert (plan["flat_to_logical"] == tree["flat_to_logical"]).all()
    anc = _ancestor_sets(p)
    starts = np.concatenate([[0], np.cumsum(s)])
    cs, go, f2l = plan["chunk_start"], plan["group_offsets"], plan["flat_to_logical"]
    nfs = tree["node_flat_start"]
    for k in range(plan["num_chunks"]):
        a, b = int(cs[k]), int(cs[k + 1])
        assert 1 <= b - a <= c
        owners = [x for x in range(len(p)) if nfs[x] <= a and b <= nfs[x] + s[x]]
        assert len(owners) == 1
    for qi, node in enumerate(qn):
        want = sorted(t for x in anc[int(node)] for t in range(starts[x], starts[x + 1]))
        got = []
        for si in plan["query_slots"][plan["query_slot_offsets"][qi]:plan["query_slot_offsets"][qi + 1]]:
            k = int(np.searchsorted(go, si, side="right") - 1)
            assert plan["slot_query"][si] == qi
            got += [int(t) for t in f2l[cs[k]:cs[k + 1]]]
            assert sum(bin(int(w)).count("1") for w in plan["slot_mask"][si]) == cs[k + 1] - cs[k]
        assert sorted(got) == want and len(got) == len(set(got))
