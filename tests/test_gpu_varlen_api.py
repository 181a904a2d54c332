"""The pages' varlen calling convention (FlashInfer page, signature and
parameters): a device cu_seqlens with an optional host copy, an optional
preallocated out, the softmax scale, and a grow-only per-device workspace
shared by the FP8 and FP4 forms.  Results must equal the general entry
point's bit for bit (same plans, same kernels)."""
import pytest
import torch

import fp8_flash_attention_amd as fa
from workloads import generate, make_workload
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


def test_varlen_forms_match_the_general_entry_point():
    w = make_workload("varlen_api", 1500, 4, [0, 0, 1, 64, 700, 1500], seed=701, k_offset_var=2.0)
    q, k, v = generate(w, device="cuda")
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    log("varlen entry points vs fa.attention")
    a = fa.varlen_attention_fp8(q, k, v, cu)
    b = fa.varlen_attention_fp8(q, k, v, cu, cu_seqlens_host=w.cu_seqlens)
    o, l = fa.varlen_attention_fp8(q, k, v, cu, cu_seqlens_host=w.cu_seqlens, return_lse=True)
    ref, lref = fa.attention(q, k, v, cu_seqlens=w.cu_seqlens, return_lse=True)
    pre = torch.empty_like(q)
    c = fa.varlen_attention_fp8(q, k, v, cu, pre, cu_seqlens_host=w.cu_seqlens, softmax_scale=w.softmax_scale)
    m = fa.varlen_attention_mxfp4(q, k, v, cu, cu_seqlens_host=w.cu_seqlens)
    mref = fa.attention(q, k, v, cu_seqlens=w.cu_seqlens, fmt="mxfp4", q_centre=True)
    torch.cuda.synchronize()
    assert torch.equal(a, ref) and torch.equal(b, ref) and torch.equal(o, ref) and torch.equal(l, lref)
    assert c.data_ptr() == pre.data_ptr() and torch.equal(c, ref)
    assert torch.equal(m, mref)


def test_shared_workspace_grows_only():
    small = make_workload("ws_small", 300, 2, [0, 300], seed=702)
    large = make_workload("ws_large", 3000, 4, [0, 1000, 3000], seed=703)
    log("shared workspace: small, large, small")
    outs = []
    for w in (small, large, small):
        q, k, v = generate(w, device="cuda")
        cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
        outs.append((fa.varlen_attention_fp8(q, k, v, cu, cu_seqlens_host=w.cu_seqlens),
                     fa.workspace_bytes(0)))
    torch.cuda.synchronize()
    (o1, n1), (o2, n2), (o3, n3) = outs
    assert 0 < n1 < n2 and n3 == n2                  # grows to the larger plan, never shrinks
    assert torch.equal(o1, o3)                        # the same call gives the same result in the larger buffer
