"""The entry points allocate nothing and enqueue one kernel each (two with
key splits: the split kernel and the merge), so they can be captured in a
HIP graph.  Each test captures a call with preallocated
outputs, replays the graph several times with eager GPU work and host
synchronisation in between, and checks every replay bit for bit against the
eager result (needs an MI355X)."""
import pytest
import torch

from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import (make_inputs, make_inputs_kv_fp8,
                                                       make_inputs_kv_int8)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("CASE", *what, flush=True)


def replay_and_check(call, o_ref, lse_ref, o, lse, replays=4):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call(o, lse)
    torch.cuda.synchronize()
    for r in range(replays):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), r


def test_graph_fwd():
    announce("graph fwd")
    q, k, v = (t.to(DEV) for t in make_inputs(1, 4, 1000, 128, "bf16", seed=2))
    o_ref, lse_ref = fa2.fwd(q, k, v)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    replay_and_check(lambda o, lse: fa2.fwd(q, k, v, out=o, lse=lse), o_ref, lse_ref, o, lse)


def test_graph_fwd_ext_causal_grouped():
    announce("graph fwd_ext")
    q, k, v = (t.to(DEV) for t in make_inputs(2, 8, 300, 64, "fp16", seed=3, Hkv=2, Nk=700))
    o_ref, lse_ref = fa2.fwd(q, k, v, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    replay_and_check(lambda o, lse: fa2.fwd(q, k, v, causal=True, out=o, lse=lse),
                     o_ref, lse_ref, o, lse)


def test_graph_fwd_kv_int8():
    announce("graph fwd_kv_int8")
    inputs = [t.to(DEV) for t in make_inputs_kv_int8(1, 4, 2, 500, 900, 128, "bf16", seed=4)]
    o_ref, lse_ref = fa2.fwd_kv_int8(*inputs, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    replay_and_check(lambda o, lse: fa2.fwd_kv_int8(*inputs, causal=True, out=o, lse=lse),
                     o_ref, lse_ref, o, lse)


def test_graph_fwd_kv_fp8():
    announce("graph fwd_kv_fp8")
    inputs = [t.to(DEV) for t in make_inputs_kv_fp8(1, 4, 2, 500, 900, 128, "fp16", seed=5)]
    o_ref, lse_ref = fa2.fwd_kv_fp8(*inputs, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    replay_and_check(lambda o, lse: fa2.fwd_kv_fp8(*inputs, causal=True, out=o, lse=lse),
                     o_ref, lse_ref, o, lse)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_graph_fwd_split(d):
    announce("graph fwd_split", d)
    q, k, v = (t.to(DEV) for t in make_inputs(2, 8, 2, d, "bf16", seed=6, Hkv=2, Nk=4000))
    ws = torch.empty(fa2.split_workspace_bytes(2, 8, 2, 2, 4000, d, True, fa2.BF16, 6),
                     dtype=torch.uint8, device=DEV)
    o_ref, lse_ref = fa2.fwd_split(q, k, v, causal=True, splits=6, workspace=ws)
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    replay_and_check(lambda o, lse: fa2.fwd_split(q, k, v, causal=True, splits=6, workspace=ws,
                                                  out=o, lse=lse),
                     o_ref, lse_ref, o, lse)
