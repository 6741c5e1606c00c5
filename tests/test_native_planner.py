"""The native planner against the reference planner (every array bit-exact),
its error paths, and the library's exported symbols.  Host-only: no GPU."""
import os
import re

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle.plan import PlanError, ref_plan, ref_plan_node_chunks, ref_plan_query_centric
from tree_structured_decode_amd import deft as D
from tree_structured_decode_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ("node_start", "flat_node_order", "node_flat_start", "flat_to_logical", "chunk_start",
        "group_offsets", "slot_query", "slot_mask", "chunk_full", "query_slot_offsets", "query_slots")
COUNTS = ("num_nodes", "num_queries", "chunk_tokens", "total_tokens", "num_chunks", "num_slots",
          "mask_words")


def assert_same_plan(native, ref):
    for k in COUNTS:
        assert native[k] == ref[k], k
    for k in KEYS:
        a, b = native[k], ref[k]
        assert a.dtype == b.dtype, k
        assert a.shape == b.shape, k
        assert np.array_equal(a, b), k


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "deft.h")).read()
    declared = set(re.findall(r"^\S.*?\b(deft_\w+)\(", header, flags=re.M))
    assert declared == set(D.EXPORTED_SYMBOLS)
    L = D.lib()
    for name in declared:
        assert getattr(L, name) is not None


def test_bench_library_exports_its_declared_symbols():
    """libdeft_bench.so (the benchmark's streaming-read calibration) exports
    what include/deft_bench.h declares; the sink size needs no GPU."""
    import ctypes
    header = open(os.path.join(ROOT, "include", "deft_bench.h")).read()
    declared = set(re.findall(r"^\S.*?\b(deft_bench_\w+)\(", header, flags=re.M))
    assert declared == {"deft_bench_stream_read", "deft_bench_stream_read_sink_floats"}
    D.lib()                        # the HIP runtime torch bundles, first
    B = ctypes.CDLL(os.path.join(ROOT, "tree_structured_decode_amd", "libdeft_bench.so"))
    for name in declared:
        assert getattr(B, name) is not None
    B.deft_bench_stream_read_sink_floats.restype = ctypes.c_size_t
    assert B.deft_bench_stream_read_sink_floats() > 0


def test_single_hip_runtime_in_process():
    D.lib()
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_standard_workloads_bit_exact(cfg):
    wl = W.standard_workload(cfg)
    for c in sorted({wl.chunk_tokens, 64, 128, 256}):
        native = D.deft_plan_export(D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, c))
        assert_same_plan(native, ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, c))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_query_centric_bit_exact(cfg):
    wl = W.standard_workload(cfg)
    for c in sorted({wl.chunk_tokens, 100, 512}):
        native = D.deft_plan_export(D.deft_plan_create_query_centric(wl.parents, wl.seg_lens,
                                                                     wl.query_nodes, c))
        assert_same_plan(native, ref_plan_query_centric(wl.parents, wl.seg_lens, wl.query_nodes, c))


@pytest.mark.parametrize("seed", range(20))
def test_query_centric_random_trees_bit_exact(seed):
    rng = np.random.default_rng(7000 + seed)
    n = int(rng.integers(1, 40))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 5, 70])), int(rng.integers(1, 12)),
                             forest_prob=float(rng.choice([0.0, 0.3])))
    c = int(rng.choice([1, 16, 33, 128]))
    native = D.deft_plan_export(D.deft_plan_create_query_centric(p, s, qn, c))
    assert_same_plan(native, ref_plan_query_centric(p, s, qn, c))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_node_chunks_bit_exact(cfg):
    wl = W.standard_workload(cfg)
    for c in sorted({wl.chunk_tokens, 100, 256}):
        native = D.deft_plan_export(D.deft_plan_create_node_chunks(wl.parents, wl.seg_lens,
                                                                   wl.query_nodes, c))
        assert_same_plan(native, ref_plan_node_chunks(wl.parents, wl.seg_lens, wl.query_nodes, c))


@pytest.mark.parametrize("seed", range(20))
def test_node_chunks_random_trees_bit_exact(seed):
    rng = np.random.default_rng(8000 + seed)
    n = int(rng.integers(1, 40))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 5, 70])), int(rng.integers(1, 12)),
                             forest_prob=float(rng.choice([0.0, 0.3])))
    c = int(rng.choice([1, 16, 33, 128]))
    native = D.deft_plan_export(D.deft_plan_create_node_chunks(p, s, qn, c))
    assert_same_plan(native, ref_plan_node_chunks(p, s, qn, c))


@pytest.mark.parametrize("seed", range(30))
def test_multi_token_random_trees_bit_exact(seed):
    rng = np.random.default_rng(8800 + seed)
    n = int(rng.integers(1, 40))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([2, 9, 70])), int(rng.integers(1, 14)),
                             forest_prob=float(rng.choice([0.0, 0.3])))
    ql = np.array([int(rng.integers(1, s[x] + 1)) for x in qn], dtype=np.int32)
    c = int(rng.choice([1, 16, 33, 128]))
    native = D.deft_plan_export(D.deft_plan_create_multi_token(p, s, qn, ql, c))
    assert_same_plan(native, ref_plan(p, s, qn, c, query_lens=ql))


def test_multi_token_workload_bit_exact():
    wl = W.standard_workload(6)
    for c in (wl.chunk_tokens, 64, 520):
        native = D.deft_plan_export(D.deft_plan_create_multi_token(wl.parents, wl.seg_lens, wl.query_nodes,
                                                                   wl.query_lens, c))
        assert_same_plan(native, ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, c,
                                          query_lens=wl.query_lens))


def test_multi_token_null_lengths_and_errors():
    wl = W.standard_workload(1)
    a = D.deft_plan_export(D.deft_plan_create_multi_token(wl.parents, wl.seg_lens, wl.query_nodes, None, 64))
    b = D.deft_plan_export(D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, 64))
    assert_same_plan(a, b)
    for ql in ([0], [5]):
        with pytest.raises(D.DeftError) as e:
            D.deft_plan_create_multi_token([-1, 0], [3, 4], [1], ql, 4)
        assert e.value.code == D.DEFT_ERR_INVALID_TREE
    with pytest.raises(ValueError):
        D.deft_plan_create_multi_token([-1, 0], [3, 4], [1], [1, 1], 4)


@pytest.mark.parametrize("c", [1, 7, 16, 64, 100, 128, 256, 512])
@pytest.mark.parametrize("seed", range(25))
def test_random_trees_bit_exact(seed, c):
    rng = np.random.default_rng(1000 + seed * 17 + c)
    n = int(rng.integers(1, 60))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 2, 5, 70, 300])), int(rng.integers(1, 20)),
                             forest_prob=float(rng.choice([0.0, 0.1, 0.5])))
    native = D.deft_plan_export(D.deft_plan_create(p, s, qn, c))
    assert_same_plan(native, ref_plan(p, s, qn, c))


@settings(max_examples=150, deadline=None)
@given(st.data())
def test_fuzzed_trees_bit_exact(data):
    n = data.draw(st.integers(1, 25))
    parents = [-1] + [data.draw(st.integers(-1, i - 1)) for i in range(1, n)]
    seg = [data.draw(st.integers(1, 40)) for _ in range(n)]
    nq = data.draw(st.integers(1, 10))
    queries = [data.draw(st.integers(0, n - 1)) for _ in range(nq)]
    c = data.draw(st.sampled_from([1, 2, 3, 16, 31, 32, 33, 64, 128]))
    native = D.deft_plan_export(D.deft_plan_create(parents, seg, queries, c))
    assert_same_plan(native, ref_plan(parents, seg, queries, c))


@pytest.mark.parametrize("args,kind", [
    (([-1, 1], [3, 4], [1], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, -2], [3, 4], [1], 4), D.DEFT_ERR_INVALID_TREE),
    (([0], [3], [0], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [3, 0], [1], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [3, -5], [1], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [3, 4], [2], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [3, 4], [-1], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [2**30, 2**30], [1], 4), D.DEFT_ERR_INVALID_TREE),
    (([-1, 0], [3, 4], [1], 0), D.DEFT_ERR_INVALID_ARGUMENT),
    (([-1, 0], [3, 4], [1], -3), D.DEFT_ERR_INVALID_ARGUMENT),
    (([-1, 0], [3, 4], [], 4), D.DEFT_ERR_INVALID_ARGUMENT),
    (([], [], [0], 4), D.DEFT_ERR_INVALID_ARGUMENT),
])
def test_plan_errors_match_reference(args, kind):
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_create(*args)
    assert e.value.code == kind
    assert D.deft_last_error()
    if kind == D.DEFT_ERR_INVALID_TREE and args[1] != [2**30, 2**30]:
        with pytest.raises(PlanError) as r:
            ref_plan(*args)
        assert r.value.kind == "invalid_tree"


def test_null_pointer_arguments():
    L = D.lib()
    import ctypes
    h = ctypes.c_void_p()
    assert L.deft_plan_create(None, None, 3, None, 1, 4, ctypes.byref(h)) == D.DEFT_ERR_INVALID_ARGUMENT
    p = np.array([-1], np.int32)
    assert L.deft_plan_create(D._ptr_i32(p), D._ptr_i32(np.array([3], np.int32)), 1,
                              D._ptr_i32(np.array([0], np.int32)), 1, 4, None) == D.DEFT_ERR_INVALID_ARGUMENT
    assert L.deft_plan_export(None, None) == D.DEFT_ERR_INVALID_ARGUMENT


def test_device_bytes_and_unsupported_shapes():
    plan = D.deft_plan_create([-1, 0], [100, 20], [1, 1, 0], 64)
    ok = D.make_desc(torch.bfloat16, 8, 2, 128, 100)
    pb, wb = D.deft_plan_device_bytes(plan, ok)
    slots = D.deft_plan_export(plan)["num_slots"]
    # bf16 inputs keep bf16 O / l plus fp32 m and l per (slot, head)
    assert pb > 0 and wb >= slots * 8 * (128 * 2 + 8)
    _, wb32 = D.deft_plan_device_bytes(plan, D.make_desc(torch.float32, 8, 2, 128, 100))
    assert wb32 >= slots * 8 * (128 + 2) * 4
    for desc, code in [
        (D.make_desc(torch.bfloat16, 8, 2, 96, 100), D.DEFT_ERR_UNSUPPORTED),
        (D.make_desc(torch.bfloat16, 8, 3, 128, 100), D.DEFT_ERR_UNSUPPORTED),
        (D.make_desc(torch.float16, 8, 2, 128, 100), D.DEFT_ERR_UNSUPPORTED),
        (D.make_desc(torch.bfloat16, 8, 2, 128, 100, page_size=32), D.DEFT_ERR_UNSUPPORTED),
        (D.make_desc(torch.bfloat16, 0, 2, 128, 100), D.DEFT_ERR_INVALID_ARGUMENT),
        (D.make_desc(torch.bfloat16, 8, 2, 128, 0), D.DEFT_ERR_INVALID_ARGUMENT),
    ]:
        with pytest.raises(D.DeftError) as e:
            D.deft_plan_device_bytes(plan, desc)
        assert e.value.code == code
    big = D.deft_plan_create([-1], [10000], [0], 8192)
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_device_bytes(big, ok)
    assert e.value.code == D.DEFT_ERR_UNSUPPORTED


def test_attention_rejects_plan_without_upload():
    import ctypes
    plan = D.deft_plan_create([-1, 0], [100, 20], [1], 64)
    desc = D.make_desc(torch.bfloat16, 8, 2, 128, 100)
    L = D.lib()
    fake = ctypes.c_void_p(256)
    rc = L.deft_tree_attention(fake, fake, fake, fake, plan.handle, fake, ctypes.byref(desc), fake,
                               1 << 20, None)
    assert rc == D.DEFT_ERR_INVALID_ARGUMENT
    assert "upload" in D.deft_last_error()
    rc = L.deft_plan_upload(plan.handle, ctypes.byref(desc), ctypes.c_void_p(100), 1 << 20, None)
    assert rc == D.DEFT_ERR_INVALID_ARGUMENT and "aligned" in D.deft_last_error()
    rc = L.deft_plan_upload(plan.handle, ctypes.byref(desc), None, 1 << 20, None)
    assert rc == D.DEFT_ERR_INVALID_ARGUMENT


def test_wide_mfma_item_rule(monkeypatch):
    """Work items of 128 rows are chosen when the 64-row items would fill the
    device's compute units twice (256 when no device can be queried): the
    32K-prefix tree takes them, the 4K-prefix tree does not.  The image holds
    8 ints per work item, so its size tells the two apart; DEFT_MFMA_WIDE
    forces either choice."""
    def plan_bytes(cfg, force):
        if force is None:
            monkeypatch.delenv("DEFT_MFMA_WIDE", raising=False)
        else:
            monkeypatch.setenv("DEFT_MFMA_WIDE", force)
        wl = W.standard_workload(cfg)
        plan = D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
        desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
        return D.deft_plan_device_bytes(plan, desc)[0]

    big_auto, big_wide, big_narrow = plan_bytes(5, None), plan_bytes(5, "1"), plan_bytes(5, "0")
    assert big_auto == big_wide < big_narrow
    small_auto, small_wide, small_narrow = plan_bytes(2, None), plan_bytes(2, "1"), plan_bytes(2, "0")
    assert small_auto == small_narrow > small_wide


def test_launch_size_limits():
    """Shapes whose rows or work-groups would not fit one launch's 32-bit
    grid are refused at sizing time, before anything reaches the device:
    num_queries * num_q_heads must stay below 2^28 (the merge covers 16 rows
    per 256-thread work-group), and the partial kernel's work items times
    the KV heads must stay within 2^23 - 1 work-groups of 512 threads."""
    plan = D.deft_plan_create([-1, 0], [16, 16], [1] * 65, 32)   # one chunk, 65 slots
    # 65 * 2^21 rows (below 2^28), two 64-row items per KV head: 2^22 work-groups
    D.deft_plan_device_bytes(plan, D.make_desc(torch.bfloat16, 1 << 21, 1 << 21, 64, 1))
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_device_bytes(plan, D.make_desc(torch.bfloat16, 1 << 22, 1 << 22, 64, 1))
    assert e.value.code == D.DEFT_ERR_UNSUPPORTED and "2^28" in str(e.value)
    # one query over 32 one-token chunks: 32 one-row VALU items per KV head
    small = D.deft_plan_create([-1], [32], [0], 1)
    D.deft_plan_device_bytes(small, D.make_desc(torch.float32, 1 << 17, 1 << 17, 64, 1))  # 2^22
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_device_bytes(small, D.make_desc(torch.float32, 1 << 18, 1 << 18, 64, 1))  # 2^23
    assert e.value.code == D.DEFT_ERR_UNSUPPORTED and "grid" in str(e.value)


def test_binding_checks_tensor_shapes():
    """The attention wrappers check every tensor against the plan and the
    descriptor before a pointer is taken: a wrong dtype, shape or size is a
    DeftError (INVALID_ARGUMENT) naming the argument; right-shaped host
    tensors get as far as the device-pointer conversion, which refuses them."""
    plan = D.deft_plan_create([-1, 0, 0], [40, 8, 9], [1, 2, 2], 32)   # 57 tokens: 4 pages
    desc = D.make_desc(torch.bfloat16, 8, 2, 64, 10)
    bf = torch.bfloat16
    good = dict(q=torch.zeros(3, 8, 64, dtype=bf), k=torch.zeros(10, 16, 2, 64, dtype=bf),
                v=torch.zeros(12, 16, 2, 64, dtype=bf), bt=torch.zeros(4, dtype=torch.int32),
                out=torch.zeros(3, 8, 64, dtype=bf), ws=torch.zeros(1 << 16, dtype=torch.uint8))

    def call(**kw):
        a = {**good, **kw}
        D.deft_tree_attention(a["q"], a["k"], a["v"], a["bt"], plan, a["out"], desc, a["ws"])

    for kw, name in [({"q": torch.zeros(3, 8, 64)}, "q"),                        # dtype
                     ({"q": torch.zeros(2, 8, 64, dtype=bf)}, "q"),              # queries
                     ({"out": torch.zeros(3, 8, 128, dtype=bf)}, "out"),
                     ({"k": torch.zeros(9, 16, 2, 64, dtype=bf)}, "k_cache"),   # fewer pages
                     ({"v": torch.zeros(10, 16, 4, 64, dtype=bf)}, "v_cache"),  # KV heads
                     ({"bt": torch.zeros(3, dtype=torch.int32)}, "block_table"),
                     ({"bt": torch.zeros(4, dtype=torch.int64)}, "block_table")]:
        with pytest.raises(D.DeftError) as e:
            call(**kw)
        assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT and str(e.value).split(": ")[1] == name
    with pytest.raises(ValueError, match="device tensor"):
        call()
    s = plan.num_slots
    for po, pm in [(torch.zeros(s, 8, 64), torch.zeros(s, 8)),                   # bf16 O expected
                   (torch.zeros(s + 1, 8, 64, dtype=bf), torch.zeros(s, 8))]:
        with pytest.raises(D.DeftError) as e:
            D.deft_lse_merge(plan, desc, po, pm, pm, good["out"], D.DEFT_PARTIAL_BF16_NORM)
        assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT and "part_o" in str(e.value)


def _rule_by_brute_force(parents, seg_lens, query_nodes, hq, hkv, bf16, cus, query_lens=None, min_rows=1):
    """The documented chunk-size rule, evaluated by building the reference
    planner's plan at every candidate size: the smallest multiple of 32 up to
    4096 whose work-groups (items of 64 rows for bf16 groups of >= min_rows
    rows, by default every bf16 group, 8 rows otherwise, times the KV heads)
    number at most `cus`; else 4096."""
    g = hq // hkv
    for c in range(32, 4097, 32):
        plan = ref_plan(parents, seg_lens, query_nodes, c, query_lens=query_lens)
        go = plan["group_offsets"].astype(np.int64)
        rows = (go[1:] - go[:-1]) * g
        blk = np.where(bf16 & (rows >= min_rows), 64, 8)
        if int(np.sum(-(-rows // blk))) * hkv <= cus:
            return c
    return 4096


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 6])
def test_auto_chunk_tokens_matches_the_rule(cfg):
    wl = W.standard_workload(cfg)
    bf16 = wl.dtype == torch.bfloat16
    for cus in (256, 80, 1024):
        desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
        got = D.deft_plan_auto_chunk_tokens(wl.parents, wl.seg_lens, wl.query_nodes, desc, cus,
                                            query_lens=wl.query_lens)
        want = _rule_by_brute_force(wl.parents, wl.seg_lens, wl.query_nodes, wl.num_q_heads, wl.num_kv_heads,
                                    bf16, cus, query_lens=wl.query_lens)
        assert got == want, (cfg, cus, got, want)


@pytest.mark.parametrize("cfg", [3, 4])
def test_auto_chunk_tokens_follows_the_matrix_core_threshold(monkeypatch, cfg):
    """DEFT_MFMA_MIN_ROWS=16 sends bf16 groups of fewer than 16 rows to the
    VALU body (8-row items), and the rule counts them that way."""
    monkeypatch.setenv("DEFT_MFMA_MIN_ROWS", "16")
    wl = W.standard_workload(cfg)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    got = D.deft_plan_auto_chunk_tokens(wl.parents, wl.seg_lens, wl.query_nodes, desc, 256)
    want = _rule_by_brute_force(wl.parents, wl.seg_lens, wl.query_nodes, wl.num_q_heads, wl.num_kv_heads,
                                True, 256, min_rows=16)
    assert got == want, (cfg, got, want)


def test_auto_chunk_tokens_known_choices():
    """On 256 compute units the rule gives 544 for the 4K-prefix tree (eight
    chunks x four 64-row items x eight KV heads = 256 work-groups; 520 would
    do too but is not a multiple of 32) and 4096 for the 32K-prefix tree
    (no size fits one round)."""
    wl = W.standard_workload(2)
    desc = D.make_desc(wl.dtype, 32, 8, 128, wl.num_pages)
    assert D.deft_plan_auto_chunk_tokens(wl.parents, wl.seg_lens, wl.query_nodes, desc, 256) == 544
    tree, _ = W.medusa_token_tree(np.random.default_rng(0), (8, 4, 2, 2, 1), 256)
    p, s, qn = W.prefix_plus_token_tree(32768, tree)
    desc5 = D.make_desc(torch.bfloat16, 64, 8, 128, 1)
    assert D.deft_plan_auto_chunk_tokens(p, s, qn, desc5, 256) == 4096


@pytest.mark.parametrize("seed", range(25))
def test_auto_chunk_tokens_random_trees(seed):
    rng = np.random.default_rng(9100 + seed)
    n = int(rng.integers(1, 40))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([5, 60, 300])), int(rng.integers(1, 30)),
                             forest_prob=float(rng.choice([0.0, 0.2])))
    hkv = int(rng.choice([1, 2, 8]))
    hq = hkv * int(rng.choice([1, 4, 8]))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    cus = int(rng.choice([4, 32, 256]))
    desc = D.make_desc(dtype, hq, hkv, 128, 10)
    got = D.deft_plan_auto_chunk_tokens(p, s, qn, desc, cus)
    assert got == _rule_by_brute_force(p, s, qn, hq, hkv, dtype == torch.bfloat16, cus)


def test_f32_partials_workspace_and_validation():
    """desc.f32_partials = 1 sizes the workspace for fp32 partial O for bf16
    inputs too (the image is unchanged), and values other than 0 and 1 are
    rejected."""
    wl = W.standard_workload(2)
    plan = D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
    s_ = D.deft_plan_export(plan)["num_slots"]
    dims = (wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    pb0, wb0 = D.deft_plan_device_bytes(plan, D.make_desc(torch.bfloat16, *dims))
    pb1, wb1 = D.deft_plan_device_bytes(plan, D.make_desc(torch.bfloat16, *dims, f32_partials=True))
    pbf, wbf = D.deft_plan_device_bytes(plan, D.make_desc(torch.float32, *dims))
    assert pb1 == pb0
    o_words = s_ * wl.num_q_heads * wl.head_dim
    def pad(w):
        return -(-w // 64) * 64
    ml = 2 * pad(s_ * wl.num_q_heads)
    assert wb0 == 4 * (pad(-(-o_words // 2)) + ml)
    assert wb1 == 4 * (pad(o_words) + ml) == wbf
    bad = D.make_desc(torch.bfloat16, *dims)
    bad.f32_partials = 2
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_device_bytes(plan, bad)
    assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT


def test_auto_chunk_tokens_errors():
    desc = D.make_desc(torch.bfloat16, 8, 2, 128, 10)
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_auto_chunk_tokens([-1, 5], [3, 3], [0], desc)
    assert e.value.code == D.DEFT_ERR_INVALID_TREE
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_auto_chunk_tokens([-1], [3], [0], D.make_desc(torch.bfloat16, 8, 2, 96, 10))
    assert e.value.code == D.DEFT_ERR_UNSUPPORTED
    with pytest.raises(D.DeftError) as e:
        D.deft_plan_auto_chunk_tokens([-1], [3], [0], desc, num_cus=-1)
    assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT
