"""fa2_fwd_split_noalloc (needs an MI355X): the allocation-free variant of
fa2_fwd_split, whose key-split partials live in a fixed scratch array in
the library's device memory instead of a caller's workspace.

Called through the C ABI, it must give exactly fa2_fwd_split's output (the
same kernels and split count, only the partials' address differs) on two
calls in a row, the second smaller than the first, so that a result cannot
lean on partials a previous call left behind; and a call whose partials
exceed the scratch is refused before any launch."""
import math

import pytest
import torch

from flashattention_forward_tile_amd import fa2
from flashattention_forward_tile_amd.workloads import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(*what):
    print("CASE", *what, flush=True)


def no_alloc(q, k, v, causal, splits):
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    code = fa2.lib().fa2_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                                           1.0 / math.sqrt(d), int(causal), fa2._DTYPE[q.dtype],
                                           splits, 0)
    assert code == fa2.OK, fa2.strerror(code)
    torch.cuda.synchronize()
    return o, lse


def test_no_alloc_matches_the_workspace_entry_point():
    # a large decode (library-chosen splits), then a smaller call
    for (B, Hq, Hkv, Nq, Nk, d, causal, splits) in ((4, 32, 8, 1, 32768, 128, True, 0),
                                                     (1, 8, 2, 3, 5000, 64, False, 5)):
        announce("no-alloc", B, Hq, Hkv, Nq, Nk, d, causal, splits)
        assert fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, causal, fa2.BF16, splits) > 0
        q, k, v = (t.to(DEV) for t in make_inputs(B, Hq, Nq, d, "bf16", seed=Nk, Hkv=Hkv,
                                                  Nk=Nk))
        o, lse = no_alloc(q, k, v, causal, splits)
        o_ref, lse_ref = fa2.fwd_split(q, k, v, causal=causal, splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_no_alloc_refuses_partials_beyond_its_scratch():
    announce("no-alloc limit")
    # 128 splits x 256 rows x 129 fp32 values = 16.9 MB > 16 MiB
    B, Hq, Hkv, Nq, Nk, d = 1, 64, 8, 4, 65536, 128
    assert fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, False, fa2.BF16, 128) > 16 << 20
    # full-size inputs, so that the call would stay in bounds even if it ran
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=DEV)
    code = fa2.lib().fa2_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d,
                                           0.1, 0, fa2.BF16, 128, 0)
    assert code == fa2.ERR_SCRATCH


def test_no_alloc_lowers_its_own_split_count_to_fit():
    """splits = 0 where the library's count (two parts: items of one query
    row each with 64 key tiles) needs more than the 16 MiB scratch: the call
    runs with the most parts that fit, here none, i.e. as fa2_fwd_ext."""
    B, Hq, Hkv, Nq, Nk, d = 256, 64, 1, 1, 2048, 128
    announce("no-alloc lowered count", B, Hq, Hkv, Nq, Nk, d)
    assert fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, True, fa2.BF16, 0) > 16 << 20
    assert fa2.split_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, True, fa2.BF16, 2) > 16 << 20
    q, k, v = (t.to(DEV) for t in make_inputs(B, Hq, Nq, d, "bf16", seed=7, Hkv=Hkv, Nk=Nk))
    o, lse = no_alloc(q, k, v, True, 0)
    o_ref, lse_ref = fa2.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
