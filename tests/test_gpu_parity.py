"""HIP path against the fp64 oracle, through the C ABI, on an MI355X.

Tolerance (per element, like allclose with atol = rtol = tol): 1e-5 for fp32
inputs, 2e-2 for bf16 inputs (fp32 accumulation).  Because 2e-2 is loose
next to the output magnitudes of some workloads, bf16 cases also check the
error against the output's own scale (_rms_check), and closed-form cases
(zero keys, constant values) check the mask and the gather where a stray
token would show.
"""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle.plan import ref_plan
from tree_structured_decode_amd import workloads as W
from tree_structured_decode_amd import deft as D
from tree_structured_decode_amd.runner import TreeAttention

from gpu_helpers import DEV, TOL, check_close, gpu_inputs, oracle_out, run_gpu, say

pytestmark = pytest.mark.gpu


def _rms_check(got, want, what):
    """Scale-aware check for bf16 outputs whose magnitude is far below 2e-2.

    Each rounding to bf16 (unit roundoff 2^-8) costs at most 2^-8 of the value
    and about a quarter of that on average.  The path rounds the probabilities
    before PV, each chunk's O / l (bf16 internal partials) and the output; the
    partial errors of different chunks are independent and shrink in the
    weighted mean, so the largest error stays below 2^-7 of the largest output
    and the mean error below 2^-8 of the mean output.  An all-zero or badly
    mixed output fails this at any scale.
    """
    err = np.abs(got - want)
    top, mean = float(np.abs(want).max()), float(np.abs(want).mean())
    assert err.max() <= 2 ** -7 * top, f"{what}: max err {err.max():.3e} above 2^-7 * {top:.3e}"
    assert err.mean() <= 2 ** -8 * mean, f"{what}: mean err {err.mean():.3e} above 2^-8 * {mean:.3e}"


@pytest.mark.parametrize("single_dispatch", [True, False])
@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_standard_workload_matches_oracle(cfg, single_dispatch):
    wl = W.standard_workload(cfg)
    say("standard", cfg, "C", wl.chunk_tokens, "single dispatch", single_dispatch)
    got, _ = run_gpu(wl, single_dispatch=single_dispatch)
    want = oracle_out(wl)
    check_close(got, want, TOL[wl.dtype], f"workload {cfg}")
    if wl.dtype == torch.bfloat16:
        _rms_check(got, want, f"workload {cfg}")


@pytest.mark.parametrize("c", [16, 64, 128, 256, 1024, 4096])
def test_spec_tree_chunk_sizes(c):
    wl = W.standard_workload(2, unscaled=True)
    say("spec tree unscaled C", c)
    got, _ = run_gpu(wl, chunk_tokens=c)
    want = oracle_out(wl)
    check_close(got, want, 2e-2, f"C={c}")
    _rms_check(got, want, f"C={c}")


def test_tiny_tree_shuffled_pages_and_chunk_sizes():
    for c in (1, 7, 16, 64, 100, 448, 4096):
        wl = W.standard_workload(1, placement="permuted")
        say("tiny permuted C", c)
        got, _ = run_gpu(wl, chunk_tokens=c)
        check_close(got, oracle_out(wl), 1e-5, f"C={c}")


@pytest.mark.parametrize("single_dispatch", [True, False])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("seed", range(6))
def test_random_trees(seed, dtype, single_dispatch):
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(1, 50))
    p, s, qn = W.random_tree(rng, n, 1, int(rng.choice([1, 9, 80, 300])), int(rng.integers(1, 40)),
                             forest_prob=float(rng.choice([0.0, 0.2])))
    hkv = int(rng.choice([1, 2, 8]))
    hq = hkv * int(rng.choice([1, 4, 8]))
    d = int(rng.choice([64, 128]))
    c = int(rng.choice([16, 32, 100, 128, 512]))
    wl = W.make_workload("rand", p, s, qn, chunk_tokens=c, hq=hq, hkv=hkv, d=d, dtype=dtype,
                         seed=seed, placement="scattered",
                         pool_pages=2 * (-(-int(s.sum()) // 16)) + 3)
    say("random", seed, str(dtype), f"N={n} Nq={len(qn)} Hq={hq} Hkv={hkv} d={d} C={c}", single_dispatch)
    got, _ = run_gpu(wl, single_dispatch=single_dispatch)
    want = oracle_out(wl)
    check_close(got, want, TOL[dtype], f"seed {seed}")
    if dtype == torch.bfloat16:
        _rms_check(got, want, f"seed {seed}")


@pytest.mark.parametrize("min_rows", ["1", "16"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("branches", [1, 2, 20])
def test_kernel_paths(monkeypatch, branches, d, dtype, min_rows):
    """Each body and row capacity on purpose: a 300-token prompt shared by
    `branches` queries, each on its own 90-token branch, 4 query heads per KV
    head.  The prompt's group has 4 * branches rows and every branch chunk 4.
    fp32 runs the VALU body (1 branch -> 4-row items, 2 -> 8-row items).  For
    bf16 the matrix-core body takes every chunk by default (few rows padded);
    with DEFT_MFMA_MIN_ROWS=16 chunks of fewer than 16 rows take the VALU body
    (4 rows: bf16 d=128 lanes hold 32 bytes; 8 rows) and 20 branches' prompt
    the matrix-core body."""
    monkeypatch.setenv("DEFT_MFMA_MIN_ROWS", min_rows)
    p, s, qn = W.shared_prompt_branches(300, branches, 90)
    wl = W.make_workload("paths", p, s, qn, chunk_tokens=96, hq=8, hkv=2, d=d, dtype=dtype,
                         seed=branches * 7 + d, placement="scattered",
                         pool_pages=2 * (-(-int(s.sum()) // 16)) + 5, value_scale=1.0 / np.sqrt(d))
    say("paths", branches, d, str(dtype))
    got, _ = run_gpu(wl)
    want = oracle_out(wl)
    check_close(got, want, TOL[dtype], f"paths {branches} {d}")
    if dtype == torch.bfloat16:
        _rms_check(got, want, f"paths {branches} {d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c", [16, 48, 144, 160, 176])
def test_mfma_step_remainders(c, d):
    """Chunk sizes whose 32-token step count leaves one or two steps after the
    last whole round of the MFMA body's four token splits (1, 2, 5, 5 and 6
    steps; partial last steps at 16, 48, 144 and 176).  20 branches on a
    300-token prompt give MFMA groups of 80 rows (a full and a partial row
    block), and the chunks across the prompt's end carry partial masks."""
    p, s, qn = W.shared_prompt_branches(300, 20, 90)
    wl = W.make_workload("tail", p, s, qn, chunk_tokens=c, hq=8, hkv=2, d=d, dtype=torch.bfloat16,
                         seed=c + d, placement="scattered",
                         pool_pages=2 * (-(-int(s.sum()) // 16)) + 5, value_scale=1.0 / np.sqrt(d))
    say("tail", c, d)
    got, _ = run_gpu(wl)
    want = oracle_out(wl)
    check_close(got, want, TOL[torch.bfloat16], f"tail {c} {d}")
    _rms_check(got, want, f"tail {c} {d}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_zero_keys_give_segment_weighted_mean(dtype):
    rng = np.random.default_rng(77)
    p, s, qn = W.random_tree(rng, 40, 1, 60, 30, forest_prob=0.05)
    d = 128
    wl = W.make_workload("zk", p, s, qn, chunk_tokens=64, hq=8, hkv=2, d=d, dtype=dtype, seed=3,
                         placement="scattered", pool_pages=3 * (-(-int(s.sum()) // 16)))
    wl.k_tokens.zero_()
    st = OA.node_starts(s)
    pattern = np.zeros((len(p), d))
    for node in range(len(p)):
        pattern[node, node % d] = node + 1.0
        wl.v_tokens[st[node]:st[node] + s[node]] = torch.from_numpy(pattern[node]).to(dtype)
    say("zero keys", str(dtype))
    got, _ = run_gpu(wl)
    for i, node in enumerate(qn):
        path = OA.path_nodes(p, node)
        want = sum(s[x] * pattern[x] for x in path) / sum(s[x] for x in path)
        # bf16: all contributions are positive, so each rounding to bf16 costs at
        # most its unit roundoff 2^-8 relative: once for a chunk's O / l in the
        # internal partial format, once for the output.
        rel = 1e-5 if dtype == torch.float32 else 2 ** -7 + 2 ** -12
        np.testing.assert_allclose(got[i], np.broadcast_to(want, got[i].shape), rtol=rel, atol=1e-6)


def test_constant_values_bf16():
    wl = W.standard_workload(4)
    wl.v_tokens[:] = torch.linspace(-2, 2, 128).to(torch.bfloat16)
    say("constant values")
    got, _ = run_gpu(wl)
    want = wl.v_tokens[0, 0].double().numpy()
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=2 ** -8, atol=0)


FORCE_WIDE = ("DEFT_MFMA_WIDE", "1")
FORCE_GROUP = ("DEFT_MFMA_GROUP", "1")
FORCE_VALU = ("DEFT_MFMA_MIN_ROWS", "16")    # bf16 chunks of < 16 rows on the VALU body


@pytest.mark.parametrize("cfg,c,force", [(1, 64, None), (3, 512, None), (3, 512, FORCE_VALU), (2, 256, None),
                                         (2, 256, FORCE_WIDE), (2, 96, FORCE_GROUP)])
def test_partials_match_oracle(monkeypatch, cfg, c, force):
    """Per-slot fp32 partials (m, l, unnormalised O) against the oracle's;
    `force` selects 128-row MFMA items or whole-group items (each with its
    own epilogue)."""
    if force is not None:
        monkeypatch.setenv(*force)
    wl = W.standard_workload(cfg, unscaled=True) if cfg == 2 else W.standard_workload(cfg)
    if cfg == 2:
        wl.q = wl.q[:, :8].contiguous()     # keep the oracle quick: 2 KV heads
        wl.k_tokens = wl.k_tokens[:, :2].contiguous()
        wl.v_tokens = wl.v_tokens[:, :2].contiguous()
        wl.num_q_heads, wl.num_kv_heads = 8, 2
    say("partials", cfg, c)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    from tree_structured_decode_amd.runner import TreeAttention
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, c, desc, device=DEV)
    po, pm, pl = ta.partials(q, kc, vc, bt)
    torch.cuda.synchronize()
    plan = ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, c)
    ids, kp, vp = W.compact_pool(wl)
    o, m, l = OA.chunk_partials(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens,
                                wl.query_nodes, plan, page_ids=ids)
    tol = TOL[wl.dtype]
    check_close(pm.double().cpu().numpy(), m, tol, "m")
    check_close(pl.double().cpu().numpy(), l, tol, "l")
    po = po.double().cpu().numpy()
    scale = np.maximum(l[:, :, None], 1.0)     # O is a sum of up to l-weighted values
    check_close(po / scale, o / scale, tol, "O / l")


@pytest.mark.parametrize("cfg,c,force", [(3, 512, None), (3, 512, FORCE_VALU), (2, 520, None),
                                         (2, 520, FORCE_WIDE), (2, 136, FORCE_GROUP)])
def test_bf16_normalised_partials_match_oracle(monkeypatch, cfg, c, force):
    """The internal partial format of bf16 inputs: O / l rounded to bf16."""
    if force is not None:
        monkeypatch.setenv(*force)
    wl = W.standard_workload(cfg, unscaled=True) if cfg == 2 else W.standard_workload(cfg)
    if cfg == 2:
        wl.q = wl.q[:, :8].contiguous()
        wl.k_tokens = wl.k_tokens[:, :2].contiguous()
        wl.v_tokens = wl.v_tokens[:, :2].contiguous()
        wl.num_q_heads, wl.num_kv_heads = 8, 2
    say("bf16 partials", cfg, c)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    from tree_structured_decode_amd.runner import TreeAttention
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, c, desc, device=DEV)
    po, pm, pl = ta.partials(q, kc, vc, bt, partial_format=D.DEFT_PARTIAL_BF16_NORM)
    torch.cuda.synchronize()
    plan = ref_plan(wl.parents, wl.seg_lens, wl.query_nodes, c)
    ids, kp, vp = W.compact_pool(wl)
    o, m, l = OA.chunk_partials(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens,
                                wl.query_nodes, plan, page_ids=ids)
    check_close(pm.double().cpu().numpy(), m, 2e-2, "m")
    check_close(pl.double().cpu().numpy(), l, 2e-2, "l")
    got = po.double().cpu().numpy()
    want = o / l[:, :, None]
    check_close(got, want, 2e-2, "O / l")
    _rms_check(got, want, "O / l")


def test_deterministic_and_writes_every_slot():
    wl = W.standard_workload(4)
    say("determinism")
    inputs = gpu_inputs(wl)
    a, _ = run_gpu(wl, inputs=inputs, poison_workspace=True)
    b, _ = run_gpu(wl, inputs=inputs, poison_workspace=False)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_two_kernel_and_fused_paths_match(cfg):
    """deft_partial_attention + deft_lse_merge (two dispatches) against the
    oracle, against deft_tree_attention_fused (the partial kernels merge each
    (query, head) row in the same dispatch; three calls on one plan, so its
    tickets must come back to zero after every call) and deft_tree_attention."""
    wl = W.standard_workload(cfg)
    say("two-kernel path", cfg)
    q, kc, vc, bt = inputs = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    from tree_structured_decode_amd.runner import TreeAttention
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV)
    bf16 = wl.dtype == torch.bfloat16
    fmt = D.DEFT_PARTIAL_BF16_NORM if bf16 else D.DEFT_PARTIAL_F32
    po, pm, pl = ta.partials(q, kc, vc, bt, partial_format=fmt)
    out2 = torch.full_like(q, float("nan"))
    D.deft_lse_merge(ta.plan, desc, po, pm, pl, out2, fmt)
    fused = []
    for _ in range(3):
        o = torch.full_like(q, float("nan"))
        D.deft_tree_attention_fused(q, kc, vc, bt, ta.plan, o, desc, ta.workspace)
        fused.append(o)
    o = torch.full_like(q, float("nan"))
    ta(q, kc, vc, bt, o)
    fused.append(o)
    torch.cuda.synchronize()
    got2 = out2.double().cpu().numpy()
    want = oracle_out(wl)
    check_close(got2, want, TOL[wl.dtype], "two-kernel path")
    for o in fused:
        # same partials, same merge arithmetic: identical bits
        assert torch.equal(o, out2)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_query_centric_baseline_matches_oracle(cfg):
    """The query-centric baseline plan (every query streams its own path) on
    the same kernels gives the same attention as the oracle."""
    wl = W.standard_workload(cfg)
    say("query-centric", cfg)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    from tree_structured_decode_amd.runner import TreeAttention
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                       query_centric=True)
    ta.workspace.view(torch.float32).fill_(float("nan"))
    out = torch.full_like(q, float("nan"))
    ta(q, kc, vc, bt, out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    want = oracle_out(wl)
    check_close(got, want, TOL[wl.dtype], "query-centric")
    if wl.dtype == torch.bfloat16:
        _rms_check(got, want, "query-centric")


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_node_granularity_plan_matches_oracle(cfg):
    """Node-granularity chunks (no chunk crosses a node) on the same kernels
    give the same attention as the oracle."""
    wl = W.standard_workload(cfg)
    say("node granularity", cfg)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    from tree_structured_decode_amd.runner import TreeAttention
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                       node_chunks=True)
    ta.workspace.view(torch.float32).fill_(float("nan"))
    out = torch.full_like(q, float("nan"))
    ta(q, kc, vc, bt, out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    want = oracle_out(wl)
    check_close(got, want, TOL[wl.dtype], "node granularity")
    if wl.dtype == torch.bfloat16:
        _rms_check(got, want, "node granularity")


@pytest.mark.parametrize("wide", [None, "1"])
def test_multi_token_workload_matches_oracle(monkeypatch, wide):
    """Multi-token query nodes (a query per draft token, causal inside its
    node): whole output, partials of the internal format, and the
    single-dispatch variant; wide = "1" forces 128-row MFMA items on (the
    prompt chunks' groups have 1024 rows)."""
    if wide is not None:
        monkeypatch.setenv("DEFT_MFMA_WIDE", wide)
    wl = W.standard_workload(6)
    say("multi-token workload", wide)
    q, kc, vc, bt = inputs = gpu_inputs(wl)
    got, ta = run_gpu(wl, inputs=inputs)
    want = oracle_out(wl)
    check_close(got, want, TOL[wl.dtype], "multi-token")
    _rms_check(got, want, "multi-token")
    out = torch.full_like(q, float("nan"))
    for _ in range(2):
        D.deft_tree_attention_fused(q, kc, vc, bt, ta.plan, out, ta.desc, ta.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(out.double().cpu().numpy(), got)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("seed", range(6))
def test_multi_token_random_trees(seed, dtype):
    """Random trees with random positions inside the query nodes; groups big
    enough for the matrix-core path at some chunks, single rows at others."""
    rng = np.random.default_rng(4200 + seed)
    n = int(rng.integers(2, 12))
    p, s, qn = W.random_tree(rng, n, 1, 60, int(rng.integers(1, 6)), forest_prob=0.2)
    # add a multi-token prefill of one node: a query on each of its tokens
    x = int(rng.integers(0, n))
    qn = np.concatenate([qn, np.full(int(s[x]), x)]).astype(np.int32)
    ql = np.array([int(rng.integers(1, s[v] + 1)) for v in qn[:-int(s[x])]] +
                  list(range(1, int(s[x]) + 1)), dtype=np.int32)
    c = int(rng.choice([16, 48, 128]))
    wl = W.make_workload("mt", p, s, qn, chunk_tokens=c, hq=8, hkv=2, d=128, dtype=dtype,
                         seed=seed, placement="permuted", value_scale=1.0 / np.sqrt(128),
                         query_lens=ql)
    say("multi-token random", seed, str(dtype), "queries", len(qn), "C", c)
    got, _ = run_gpu(wl)
    want = oracle_out(wl)
    check_close(got, want, TOL[dtype], "multi-token random")
    if dtype == torch.bfloat16:
        _rms_check(got, want, "multi-token random")


def test_single_node_single_query_and_duplicates():
    for parents, seg, qn in [([-1], [1], [0]), ([-1], [17], [0, 0, 0]), ([-1, 0, 0], [5, 1, 1], [0, 1, 2, 1])]:
        for dtype in (torch.float32, torch.bfloat16):
            wl = W.make_workload("edge", parents, seg, qn, chunk_tokens=16, hq=8, hkv=2, d=128,
                                 dtype=dtype, seed=1, placement="identity")
            say("edge", parents, seg, qn, str(dtype))
            got, _ = run_gpu(wl)
            check_close(got, oracle_out(wl), TOL[dtype], "edge")


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 64), (torch.float32, 128)])
def test_fused_merge_work_groups_many_rows(dtype, d):
    """161 queries x 16 heads = 2576 (query, head) rows: the single-dispatch
    path's merge work-groups take 32 rows, the last one ragged (16 rows).
    Output equals the two-dispatch path bit for bit, twice in a row (the
    tickets return to zero), and the oracle within tolerance."""
    p, s, qn = W.shared_prompt_branches(48, 161, 3)
    wl = W.make_workload("many-rows", p, s, qn, chunk_tokens=32, hq=16, hkv=4, d=d, dtype=dtype, seed=5,
                         placement="permuted")
    say("fused many rows", str(dtype), d)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV)
    ref = torch.full_like(q, float("nan"))
    D.deft_tree_attention(q, kc, vc, bt, ta.plan, ref, desc, ta.workspace)
    for rep in range(2):
        ta.workspace.view(torch.float32).fill_(float("nan"))
        o = torch.full_like(q, float("nan"))
        D.deft_tree_attention_fused(q, kc, vc, bt, ta.plan, o, desc, ta.workspace)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"rep {rep}: fused output differs from the two-dispatch path"
    check_close(ref.double().cpu().numpy(), oracle_out(wl), TOL[dtype], "many rows")


@pytest.mark.parametrize("cfg", [2, 3, 6])
def test_f32_partials_match_oracle(cfg):
    """bf16 inputs with desc.f32_partials = 1: the workspace holds fp32
    unnormalised partials.  The single dispatch and the two dispatches give
    the same bits, the oracle is met, and the output differs from the default
    bf16 partials' (the format took effect)."""
    wl = W.standard_workload(cfg)
    say("f32 partials", cfg)
    q, kc, vc, bt = gpu_inputs(wl)
    outs = {}
    for f32 in (False, True):
        desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages,
                           f32_partials=f32)
        ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                           query_lens=wl.query_lens)
        ta.workspace.view(torch.float32).fill_(float("nan"))
        one = torch.full_like(q, float("nan"))
        ta(q, kc, vc, bt, one)
        two = torch.full_like(q, float("nan"))
        D.deft_tree_attention(q, kc, vc, bt, ta.plan, two, desc, ta.workspace)
        torch.cuda.synchronize()
        assert torch.equal(one, two), f"f32_partials={f32}: single and two dispatches differ"
        outs[f32] = one
    assert not torch.equal(outs[False], outs[True])
    want = oracle_out(wl)
    got = outs[True].double().cpu().numpy()
    check_close(got, want, TOL[wl.dtype], f"f32 partials {cfg}")
    _rms_check(got, want, f"f32 partials {cfg}")


@pytest.mark.timeout(900)
def test_long_context_spec_tree_all_queries():
    """The 32K-prefix / 256-node tree in a pool filling ~60% of HBM, pages at
    random positions: every query and head against the oracle (computed once,
    about half a minute of host time), at long chunks (many pipeline steps
    per wave, several work-groups per CU in turn, 128-row items that cover
    every row block of every chunk), repeated because a stale-operand race
    would show up only in some runs."""
    total = torch.cuda.get_device_properties(0).total_memory
    pages = W.hbm_pool_pages(total)
    wl = W.standard_workload(5, pool_pages=pages)
    say("long context", "pool pages", pages)
    inputs = gpu_inputs(wl)
    say("long context", "oracle over", len(wl.query_nodes), "queries")
    want = oracle_out(wl)
    for c in (4096, 2048):
        for rep in range(2):
            say("long context C", c, "rep", rep)
            got, _ = run_gpu(wl, chunk_tokens=c, inputs=inputs)
            check_close(got, want, 2e-2, f"long context C={c} rep {rep}")
            _rms_check(got, want, f"long context C={c} rep {rep}")


def test_validate_block_table_host_check(monkeypatch):
    """With DEFT_VALIDATE=1 a block-table entry outside [0, num_pages) is
    reported before anything is launched, and a valid table runs as usual.
    The pool holds two pages more than desc declares, so the out-of-range
    entry still names memory that exists."""
    p, s, qn = W.shared_prompt_branches(64, 2, 32)
    n_lp = -(-int(s.sum()) // 16)
    wl = W.make_workload("validate", p, s, qn, chunk_tokens=32, hq=8, hkv=2, d=64,
                         dtype=torch.float32, seed=11, placement="identity", pool_pages=n_lp + 2)
    say("validate", n_lp)
    monkeypatch.setenv("DEFT_VALIDATE", "1")
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, 8, 2, 64, n_lp)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, 32, desc, device=DEV)
    bad = bt.clone()
    bad[1] = n_lp
    out = torch.full_like(q, float("nan"))
    with pytest.raises(D.DeftError) as err:
        ta(q, kc, vc, bad, out)
    assert err.value.code == D.DEFT_ERR_INVALID_ARGUMENT
    assert "block_table[1]" in str(err.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    ta(q, kc, vc, bt, out)
    torch.cuda.synchronize()
    check_close(out.double().cpu().numpy(), oracle_out(wl), TOL[torch.float32], "validate")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c", [48, 96, 544])
def test_wide_mfma_items_match_oracle(monkeypatch, c, d):
    """128-row MFMA items (two token splits of four 32-row waves, split 1
    merged into split 0 in registers), forced on: groups of 80 rows (a
    partial wide item) on the shared-prompt tree, at chunk sizes with one,
    three and seventeen 32-token steps."""
    monkeypatch.setenv("DEFT_MFMA_WIDE", "1")
    p, s, qn = W.shared_prompt_branches(300, 20, 90)
    wl = W.make_workload("wide", p, s, qn, chunk_tokens=c, hq=8, hkv=2, d=d, dtype=torch.bfloat16,
                         seed=3 * c + d, placement="scattered",
                         pool_pages=2 * (-(-int(s.sum()) // 16)) + 5, value_scale=1.0 / np.sqrt(d))
    say("wide", c, d)
    got, _ = run_gpu(wl)
    want = oracle_out(wl)
    check_close(got, want, TOL[torch.bfloat16], f"wide {c} {d}")
    _rms_check(got, want, f"wide {c} {d}")


def test_wide_mfma_items_standard_tree_and_fused(monkeypatch):
    """The 4K-prefix tree (256-row groups: two full 128-row items per chunk
    and KV head) with 128-row items forced on: against the oracle, and the
    single-dispatch path bit-identical to the two-dispatch one."""
    monkeypatch.setenv("DEFT_MFMA_WIDE", "1")
    wl = W.standard_workload(2)
    say("wide standard", wl.chunk_tokens)
    q, kc, vc, bt = gpu_inputs(wl)
    got, ta = run_gpu(wl, inputs=(q, kc, vc, bt))
    check_close(got, oracle_out(wl), TOL[torch.bfloat16], "wide cfg2")
    out2 = torch.full_like(q, float("nan"))
    D.deft_tree_attention_fused(q, kc, vc, bt, ta.plan, out2, ta.desc, ta.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(out2.double().cpu().numpy(), got)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c", [16, 48, 96, 144, 544])
@pytest.mark.parametrize("branches", [20, 70])
def test_group_items_match_oracle(monkeypatch, branches, c, d):
    """Whole-group MFMA items (up to 256 rows, no token split, a shared
    four-stage ring), forced on: 20 branches on a 300-token prompt give
    80-row groups (three of eight waves with rows, a partial row tile), 70
    branches give 280-row groups (a full 256-row item and a 24-row one), at
    chunk sizes of one, two, three, five and seventeen 32-token steps
    (ring reuse, partial last steps)."""
    monkeypatch.setenv("DEFT_MFMA_GROUP", "1")
    p, s, qn = W.shared_prompt_branches(300, branches, 90)
    wl = W.make_workload("group", p, s, qn, chunk_tokens=c, hq=8, hkv=2, d=d, dtype=torch.bfloat16,
                         seed=5 * c + d + branches, placement="scattered",
                         pool_pages=2 * (-(-int(s.sum()) // 16)) + 5, value_scale=1.0 / np.sqrt(d))
    say("group", branches, c, d)
    got, _ = run_gpu(wl)
    want = oracle_out(wl)
    check_close(got, want, TOL[torch.bfloat16], f"group {branches} {c} {d}")
    _rms_check(got, want, f"group {branches} {c} {d}")


def test_group_items_standard_tree_and_fused(monkeypatch):
    """The 4K-prefix tree at C = 128 (256-row groups, 33 chunks) with
    whole-group items forced on: against the oracle, and the single-dispatch
    path bit-identical to the two-dispatch one."""
    monkeypatch.setenv("DEFT_MFMA_GROUP", "1")
    wl = W.standard_workload(2, chunk_tokens=128)
    say("group standard", wl.chunk_tokens)
    q, kc, vc, bt = gpu_inputs(wl)
    got, ta = run_gpu(wl, inputs=(q, kc, vc, bt))
    check_close(got, oracle_out(wl), TOL[torch.bfloat16], "group cfg2")
    _rms_check(got, oracle_out(wl), "group cfg2")
    out2 = torch.full_like(q, float("nan"))
    D.deft_tree_attention_fused(q, kc, vc, bt, ta.plan, out2, ta.desc, ta.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(out2.double().cpu().numpy(), got)


@pytest.mark.parametrize("cfg,force", [(2, None), (4, None), (3, None), (6, None), (2, FORCE_WIDE),
                                       (2, FORCE_GROUP), (3, FORCE_VALU), (4, FORCE_VALU), (1, None)])
def test_fused_path_reads_fresh_partials(monkeypatch, cfg, force):
    """The single-dispatch path hands partials between work-groups (possibly
    on different XCDs) through device-coherent stores and loads and relaxed
    tickets.  Stale data would show here: calls alternate between two input
    sets (the second with Q negated and V permuted across the tree's tokens), the
    workspace is filled with NaN before each call, and every call's output is
    compared with the two-dispatch path's on the same inputs bit for bit (the
    first input set's also with the oracle)."""
    if force is not None:
        monkeypatch.setenv(*force)
    wl = W.standard_workload(cfg)
    say("fused fresh", cfg, force)
    q, kc, vc, bt = gpu_inputs(wl)
    q2 = (-q).contiguous()
    # V permuted across the tree's tokens (pages of the pool that hold none
    # stay poisoned, so the permutation stays among written rows)
    t = torch.arange(wl.total_tokens)
    pi, ri = bt.cpu().long()[t // 16].to(vc.device), (t % 16).to(vc.device)
    perm = torch.randperm(wl.total_tokens, generator=torch.Generator().manual_seed(cfg)).to(vc.device)
    vc2 = vc.clone()
    vc2[pi, ri] = vc[pi[perm], ri[perm]]
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                       query_lens=wl.query_lens)
    refs = []
    for qq, vv in ((q, vc), (q2, vc2)):
        o = torch.full_like(q, float("nan"))
        D.deft_tree_attention(qq, kc, vv, bt, ta.plan, o, desc, ta.workspace)
        refs.append(o)
    torch.cuda.synchronize()
    for rep in range(4):
        k = rep % 2
        qq, vv = ((q, vc), (q2, vc2))[k]
        ta.workspace.view(torch.float32).fill_(float("nan"))
        o = torch.full_like(q, float("nan"))
        D.deft_tree_attention_fused(qq, kc, vv, bt, ta.plan, o, desc, ta.workspace)
        torch.cuda.synchronize()
        assert torch.equal(o, refs[k]), f"rep {rep}: fused output differs from the two-dispatch path"
    check_close(refs[0].double().cpu().numpy(), oracle_out(wl), TOL[wl.dtype], "fused fresh, inputs 1")
