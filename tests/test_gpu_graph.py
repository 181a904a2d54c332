"""The quantize + forward sequence under HIP graph capture (serving loops
replay a captured step).  The library allocates nothing and issues no memset
inside either call, so a captured step replays the same kernels on the same
buffers: every replay, with eager work and synchronizations between replays,
must reproduce the eager result bit for bit.
"""
import pytest
import torch

import fp8_flash_attention_amd as fa
from workloads import generate, make_workload
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("opts", [dict(), dict(causal=True), dict(fmt="mxfp4", q_centre=True)],
                         ids=["e4m3", "causal", "mxfp4"])
def test_captured_step_replays_bit_identically(opts):
    w = make_workload("graph", 2000, 8, [0, 700, 2000], seed=601, k_offset_var=2.0)
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, **opts)
    ws = plan.new_workspace()
    out = torch.empty((w.tokens, w.heads, 128), dtype=torch.bfloat16, device="cuda")
    log(f"graph capture {opts}")
    fa.quantize(plan, q, k, v, ws)
    fa.forward(plan, ws, out)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fa.quantize(plan, q, k, v, ws, stream=s)
            fa.forward(plan, ws, out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for r in range(4):
        out.fill_(0)
        ws.fill_(0xFF)                      # eager work on the same buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs"
