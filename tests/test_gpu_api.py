"""Host-side argument checks of the attention entry points on a GPU process.

Each call here is rejected before any kernel is launched; the library must
report the error code and leave the device untouched.
"""
import pytest
import torch

from tree_structured_decode_amd import deft as D
from tree_structured_decode_amd import workloads as W
from tree_structured_decode_amd.runner import TreeAttention

from gpu_helpers import DEV, check_close, gpu_inputs, oracle_out, say

pytestmark = pytest.mark.gpu


def _setup(cfg):
    wl = W.standard_workload(cfg)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV)
    return wl, desc, ta


def test_partial_format_checked():
    say("api: partial formats")
    wl, desc, ta = _setup(1)          # fp32 inputs
    q, kc, vc, bt = gpu_inputs(wl)
    s, hq, d = ta.plan_view_counts(), wl.num_q_heads, wl.head_dim
    po = torch.empty((s, hq, d), dtype=torch.float32, device=DEV)
    pm = torch.empty((s, hq), dtype=torch.float32, device=DEV)
    pl = torch.empty((s, hq), dtype=torch.float32, device=DEV)
    for fmt in (D.DEFT_PARTIAL_BF16_NORM, 7, -1):
        with pytest.raises(D.DeftError) as e:
            D.deft_partial_attention(q, kc, vc, bt, ta.plan, desc, po, pm, pl, fmt)
        assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT
        with pytest.raises(D.DeftError) as e:
            D.deft_lse_merge(ta.plan, desc, po, pm, pl, q, fmt)
        assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def test_workspace_and_desc_checked():
    say("api: workspace and desc")
    wl, desc, ta = _setup(2)
    q, kc, vc, bt = gpu_inputs(wl)
    out = torch.empty_like(q)
    small = torch.empty(ta.workspace_bytes - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(D.DeftError) as e:
        D.deft_tree_attention(q, kc, vc, bt, ta.plan, out, desc, small)
    assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT
    other = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads // 2, wl.head_dim, wl.num_pages)
    with pytest.raises(D.DeftError) as e:
        D.deft_tree_attention(q, kc, vc, bt, ta.plan, out, other, ta.workspace)
    assert e.value.code == D.DEFT_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()


def test_back_to_back_uploads_keep_each_image():
    """Uploads of one plan for two descs in a row, with no synchronisation
    between them: the second upload waits for the first copy before it
    rebuilds the plan's host staging buffer, so both device images are
    whole (each equals a fresh, synchronised upload of the same desc), and
    the attention call on the second image matches the oracle."""
    say("api: back-to-back uploads")
    wl = W.standard_workload(2)
    plan = D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
    d_bf16 = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    d_f32 = D.make_desc(torch.float32, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    images = []
    for desc in (d_f32, d_bf16):
        pb, _ = D.deft_plan_device_bytes(plan, desc)
        images.append(torch.zeros(pb // 4, dtype=torch.int32, device=DEV))
    D.deft_plan_upload(plan, d_f32, images[0])
    D.deft_plan_upload(plan, d_bf16, images[1])
    torch.cuda.synchronize()
    for desc, img in zip((d_f32, d_bf16), images):
        ref = torch.zeros_like(img)
        fresh = D.deft_plan_create(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens)
        D.deft_plan_upload(fresh, desc, ref)
        torch.cuda.synchronize()
        assert torch.equal(img, ref)
        D.deft_plan_destroy(fresh)
    q, kc, vc, bt = gpu_inputs(wl)
    _, wb = D.deft_plan_device_bytes(plan, d_bf16)
    ws = torch.empty(wb, dtype=torch.uint8, device=DEV)
    out = torch.full_like(q, float("nan"))
    D.deft_tree_attention(q, kc, vc, bt, plan, out, d_bf16, ws)
    torch.cuda.synchronize()
    sel = list(range(0, wl.num_queries, 8))
    got = out.double().cpu().numpy()[sel]
    from gpu_helpers import check_close, oracle_out, TOL
    check_close(got, oracle_out(wl, queries=sel), TOL[torch.bfloat16], "after back-to-back uploads")
    D.deft_plan_destroy(plan)


@pytest.mark.parametrize("single_dispatch", [True, False])
def test_bounded_wait_give_up_is_reported(monkeypatch, single_dispatch):
    """A partial kernel whose inter-wave waits may make no second check
    (DEFT_SPIN_LIMIT=0, forced from the host; every kernel still exits)
    reports through deft_plan_status; the status is cleared by the check,
    and normal calls leave it clear.  On the single-dispatch path the merge
    work-groups give up at once too, before their rows' partials are in:
    the tickets must still come back to zero, so the next normal call is
    exact."""
    wl = W.standard_workload(2)
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                       single_dispatch=single_dispatch)
    out = torch.empty_like(q)
    say("spin limit default")
    ta(q, kc, vc, bt, out)
    D.deft_plan_status(ta.plan)                 # no give-up
    say("spin limit 0")
    monkeypatch.setenv("DEFT_SPIN_LIMIT", "0")
    for _ in range(3):
        ta(q, kc, vc, bt, out)
    with pytest.raises(D.DeftError) as err:
        D.deft_plan_status(ta.plan)
    assert err.value.code == D.DEFT_ERR_HIP
    assert "bounded wait" in str(err.value)
    D.deft_plan_status(ta.plan)                 # cleared by the check
    monkeypatch.delenv("DEFT_SPIN_LIMIT")
    want = oracle_out(wl)
    for rep in range(2):
        ta.workspace.view(torch.float32).fill_(float("nan"))
        out.fill_(float("nan"))
        ta(q, kc, vc, bt, out)
        D.deft_plan_status(ta.plan)
        got = out.double().cpu().numpy()
        check_close(got, want, 2e-2, f"after the forced give-up, call {rep}")
