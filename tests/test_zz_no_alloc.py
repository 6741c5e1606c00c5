"""deft_tree_attention_noalloc against deft_tree_attention, through the C ABI.

The no-allocation entry point runs the same kernels on a library-owned device
scratch instead of a caller workspace, so its output must equal the
workspace path's bit for bit.  Two calls in a row, the second on a smaller
plan (the scratch keeps the first call's contents), then a plan whose
partials exceed the scratch, which must be refused before any launch.
"""
import numpy as np
import pytest
import torch

from tree_structured_decode_amd import deft as D
from tree_structured_decode_amd import workloads as W
from tree_structured_decode_amd.runner import TreeAttention

from gpu_helpers import DEV, TOL, check_close, gpu_inputs, oracle_out, say

pytestmark = pytest.mark.gpu


def _both(wl):
    """(no-alloc output, workspace-path output) on the same inputs."""
    q, kc, vc, bt = gpu_inputs(wl)
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, wl.chunk_tokens, desc, device=DEV,
                       query_lens=wl.query_lens)
    ta.workspace.view(torch.float32).fill_(float("nan"))
    ref = torch.full_like(q, float("nan"))
    D.deft_tree_attention(q, kc, vc, bt, ta.plan, ref, desc, ta.workspace)
    got = torch.full_like(q, float("nan"))
    D.deft_tree_attention_noalloc(q, kc, vc, bt, ta.plan, got, desc)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_workspace_path_twice_then_smaller():
    big = W.standard_workload(2)                      # 4K-prefix / 64-node tree, bf16
    p, s, qn = W.shared_prompt_branches(300, 3, 90)   # 3 branches on a 300-token prompt, fp32
    small = W.make_workload("noalloc-small", p, s, qn, chunk_tokens=64, hq=8, hkv=2, d=64,
                            dtype=torch.float32, seed=7, placement="scattered",
                            pool_pages=2 * (-(-int(s.sum()) // 16)) + 3)
    for wl in (big, small):
        say("noalloc", wl.name)
        got, ref = _both(wl)
        assert torch.equal(got, ref), f"{wl.name}: no-alloc output differs from the workspace path"
        want = oracle_out(wl)
        check_close(got.double().cpu().numpy(), want, TOL[wl.dtype], f"noalloc {wl.name}")


def test_noalloc_refuses_partials_beyond_the_scratch():
    """A root of 16384 tokens seen by 256 queries, 64 heads of d 128 at
    C = 64: 256 chunks x 256 slots x 64 heads of bf16 O is 1 GiB of partials,
    far above the scratch; the call fails before launching anything and
    leaves out untouched."""
    n = 256
    parents = np.array([-1] + [0] * n, dtype=np.int32)
    seg = np.array([16384] + [1] * n, dtype=np.int32)
    qn = np.arange(1, n + 1, dtype=np.int32)
    plan = D.deft_plan_create(parents, seg, qn, 64)
    desc = D.make_desc(torch.bfloat16, 64, 8, 128, 1)
    pb, wb = D.deft_plan_device_bytes(plan, desc)
    assert wb > D.DEFT_NOALLOC_SCRATCH_BYTES
    dev_plan = torch.empty(pb, dtype=torch.uint8, device=DEV)
    D.deft_plan_upload(plan, desc, dev_plan)
    q = torch.zeros((n, 64, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((1, 16, 8, 128), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    bt = torch.zeros(-(-int(seg.sum()) // 16), dtype=torch.int32, device=DEV)
    out = torch.full_like(q, float("nan"))
    say("noalloc refuse", wb)
    with pytest.raises(D.DeftError) as err:
        D.deft_tree_attention_noalloc(q, kc, vc, bt, plan, out, desc)
    assert err.value.code == D.DEFT_ERR_UNSUPPORTED
    assert "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
