"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compute the oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

from oracle import attention as OA
from tree_structured_decode_amd import deft as D
from tree_structured_decode_amd import workloads as W
from tree_structured_decode_amd.runner import TreeAttention

DEV = "cuda:0"
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def say(*msg):
    print("[gpu-case]", *msg, file=sys.stderr, flush=True)


def gpu_inputs(wl):
    kc, vc = W.build_pool(wl, DEV, poison=True)
    q = wl.q.to(DEV).contiguous()
    bt = torch.from_numpy(wl.block_table).to(DEV)
    return q, kc, vc, bt


def run_gpu(wl, chunk_tokens=None, poison_workspace=True, inputs=None, single_dispatch=True):
    """Tree attention through libdeft (the runner's single-dispatch call, or
    the partial and merge kernels); returns (out on CPU as float64, runner)."""
    c = chunk_tokens or wl.chunk_tokens
    desc = D.make_desc(wl.dtype, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.num_pages)
    q, kc, vc, bt = inputs if inputs is not None else gpu_inputs(wl)
    ta = TreeAttention(wl.parents, wl.seg_lens, wl.query_nodes, c, desc, device=DEV,
                       query_lens=wl.query_lens, single_dispatch=single_dispatch)
    if poison_workspace:
        ta.workspace.view(torch.float32).fill_(float("nan"))
    out = torch.full_like(q, float("nan"))
    ta(q, kc, vc, bt, out)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), ta


def oracle_out(wl, queries=None):
    ids, kp, vp = W.compact_pool(wl)
    return OA.tree_attention(wl.q, kp, vp, wl.block_table, wl.parents, wl.seg_lens, wl.query_nodes,
                             page_ids=ids, queries=queries, query_lens=wl.query_lens)


def check_close(got, want, tol, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = tol + tol * np.abs(want)
    bad = err > bound
    rms = float(np.sqrt(np.mean(want ** 2)))
    msg = (f"{what}: max abs err {err.max():.3e}, rms(oracle) {rms:.3e}, "
           f"{int(bad.sum())} of {bad.size} elements outside tol {tol}")
    assert not bad.any(), msg
    return float(err.max()), rms
