"""The quantize + forward sequence under HIP graph capture (serving loops
replay a captured step).  The library allocates nothing and issues no memset
inside either call, so a captured step replays the same kernels on the same
buffers: every replay, with eager work and synchronizations between replays,
must reproduce the eager result (output and LSE) bit for bit.  Covered: the
default E4M3 plan, one whose work items are split along the keys (so the
combine pass is captured too), causal, a 96-channel head, the LSE output,
the allocation-free quantize entry point, an FP4 plan with Q centring, and
E4M3 plans with Q centring (its mean-term kernel captured with the
quantize), one of them split and quantized without allocation.
"""
import pytest
import torch

import fp8_flash_attention_amd as fa
from workloads import generate, make_workload
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

CASES = {
    "e4m3": dict(),
    "causal": dict(causal=True),
    "lse_noalloc": dict(lse=True, noalloc=True),
    "split_lse": dict(lse=True, split=True),
    "head_dim96_lse": dict(head_dim=96, lse=True),
    "mxfp4": dict(fmt="mxfp4", q_centre=True, lse=True),
    "e4m3_q_centre": dict(q_centre=True, lse=True),
    "e4m3_q_centre_split_noalloc": dict(q_centre=True, split=True, noalloc=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_step_replays_bit_identically(name):
    opts = dict(CASES[name])
    lse_on, noalloc, split = opts.pop("lse", False), opts.pop("noalloc", False), opts.pop("split", False)
    D = opts.get("head_dim", 128)
    if split:   # few items per XCD: the last round is split along the keys
        w = make_workload("graph_split", 4096, 2, [0, 4096], seed=602, k_offset_var=2.0)
    else:
        w = make_workload("graph", 2000, 8, [0, 700, 2000], seed=601, k_offset_var=2.0, head_dim=D)
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, **opts)
    ws = plan.new_workspace()
    out = torch.empty((w.tokens, w.heads, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.heads, w.tokens), dtype=torch.float32, device="cuda") if lse_on else None
    assert not split or plan.info()["partial_slots"] > 0
    quant = fa.quantize_noalloc if noalloc else fa.quantize
    log(f"graph capture {name}: {opts} lse={lse_on} noalloc={noalloc} pieces={plan.info()['partial_slots']}")
    quant(plan, q, k, v, ws)
    fa.forward(plan, ws, out, lse)
    torch.cuda.synchronize()
    eager = out.clone()
    eager_lse = lse.clone() if lse_on else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            quant(plan, q, k, v, ws, stream=s)
            fa.forward(plan, ws, out, lse, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        out.fill_(0)
        if lse_on:
            lse.fill_(0)
        ws.fill_(0xFF)                      # eager work on the same buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs"
        if lse_on:
            assert torch.equal(lse, eager_lse), f"replay {r}: LSE differs"
