"""verify_attn_full_noalloc (the verify entry point for callers that cannot allocate) against
verify_attn_full, through the C ABI: two calls in a row on one GPU, the second on a smaller,
ragged, shuffled-page input, so the library's scratch array still holds the first call's
partials when the second runs. The outputs must be bit-identical (same kernels, same split
plan), and the call must not allocate.
"""

import pytest
import torch

from kv_sparse_speculative_amd import kvss
from kv_sparse_speculative_amd.synth import generate
from kv_sparse_speculative_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

# (workload, reduced batch, prompt range): both plans split the key range, so both calls put
# their partials in the scratch array; the second needs less of it.
CALLS = [
    ("llama8b_ctx32k", 4, None),                  # 32 splits, 10.6 MB of partials
    ("qwen32b_ragged", 3, (16500, 18000)),        # 18 splits, 4.5 MB, G = 5, shuffled pages
]


def _case(name, batch, prompt):
    ns = generate(WORKLOADS[name], device="cuda", batch=batch, prompt=prompt, parts=("attn",))
    P = ns.prompt_lens_np
    kv = kvss.PagedKV(ns.k_cache, ns.v_cache, ns.block_table, ns.kv_lens_verify,
                      int(P.max()) + ns.T)
    return ns, kv


def _allocations():
    return torch.cuda.memory_stats().get("allocation.all.allocated", 0)


def test_noalloc_verify_equals_verify_on_two_calls():
    torch.cuda.set_device(0)
    needs = []
    for name, batch, prompt in CALLS:
        print(f"noalloc verify: {name} batch {batch} prompt {prompt}", flush=True)
        ns, kv = _case(name, batch, prompt)
        import ctypes
        need = kvss.lib().kvss_verify_workspace_bytes(ctypes.byref(kv.desc()),
                                                      ns.q_verify.shape[1], ns.T)
        assert 0 < need <= 32 << 20
        needs.append(need)
        ref_out, ref_lse = kvss.verify_attn_full(kv, ns.q_verify)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        torch.cuda.synchronize()
        before = _allocations()
        kvss.verify_attn_full_noalloc(kv, ns.q_verify, out=out, lse=lse)
        assert _allocations() == before
        torch.cuda.synchronize()
        assert torch.isfinite(ref_out).all()
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)
    assert needs[1] < needs[0]


def test_noalloc_verify_fp32_and_unsplit():
    """The fp32 path (split) and an unsplit bf16 plan (no scratch needed at all)."""
    torch.cuda.set_device(0)
    for name, batch, prompt in (("tiny_fp32", None, None), ("llama8b_ctx8k", 2, (3000, 3000))):
        print(f"noalloc verify: {name} batch {batch} prompt {prompt}", flush=True)
        ns, kv = _case(name, batch, prompt)
        ref_out, ref_lse = kvss.verify_attn_full(kv, ns.q_verify)
        out, lse = kvss.verify_attn_full_noalloc(kv, ns.q_verify)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)
