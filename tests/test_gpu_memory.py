"""Retained device memory across many sequence lengths (the multi-shape memory
regression test that the review of sglang PR "[diffusion] attention: add
fp8_fa_sm120 FP8 backend for SM120 GPUs" asks for): after attention calls on
many distinct shapes, every per-call buffer is released, the plan cache holds
at most PLAN_CACHE_SIZE plans, and once it is cleared the device's free memory
returns to where it was; a second pass over the same shapes does not grow it.
"""
import pytest
import torch

import fp8_flash_attention_amd as fa
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

MiB = 1 << 20


def _pass(lengths, H=4):
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    for S in lengths:
        q, k, v = (torch.randn((S, H, 128), generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(3))
        out = fa.attention(q, k, v)
        assert torch.isfinite(out.float()).all()
        del q, k, v, out
    torch.cuda.synchronize()


def test_memory_returns_to_baseline_across_shapes():
    lengths = [200 + 97 * i for i in range(40)]            # 40 distinct plans, more than the cache holds
    _pass([256])                                           # loads the kernels (and the library's static buffer)
    fa.clear_plan_cache()
    torch.cuda.empty_cache()
    alloc0 = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    log(f"memory baseline: torch allocated {alloc0} B, device free {free0 / MiB:.1f} MiB")
    _pass(lengths)
    assert len(fa._PLANS) <= fa.PLAN_CACHE_SIZE
    assert torch.cuda.memory_allocated() == alloc0         # workspaces and outputs released
    fa.clear_plan_cache()
    torch.cuda.empty_cache()
    free1, _ = torch.cuda.mem_get_info()
    _pass(lengths)
    fa.clear_plan_cache()
    torch.cuda.empty_cache()
    free2, _ = torch.cuda.mem_get_info()
    log(f"  device free after pass 1 {free1 / MiB:.1f} MiB, after pass 2 {free2 / MiB:.1f} MiB")
    assert free0 - free1 <= 16 * MiB                       # back to the baseline (allocator granularity)
    assert abs(free1 - free2) <= 2 * MiB                   # and no growth from one pass to the next
