"""fp8attn_quantize_noalloc (statistics in the library's static device buffer)
against fp8attn_quantize: the code, scale and mean regions (with E4M3 Q
centring also the block means and the mean-term table) bit for bit and the
forward output from each workspace, on two calls in a row, the second with a
smaller input; the noalloc workspace stops where the statistics region would
begin and is poisoned first."""
import pytest
import torch

import fp8_flash_attention_amd as fa
from fp8_flash_attention_amd import _lib
from workloads import generate, make_workload
from tests.gpu_helpers import log

pytestmark = pytest.mark.gpu

E4M3_REGIONS = [_lib.REGION_Q, _lib.REGION_K, _lib.REGION_V, _lib.REGION_SCALES, _lib.REGION_MU]
MX_REGIONS = [_lib.REGION_Q, _lib.REGION_K, _lib.REGION_V, _lib.REGION_Q_BSCALES, _lib.REGION_K_BSCALES,
              _lib.REGION_V_BSCALES, _lib.REGION_QM_CODES, _lib.REGION_QM_SCALES, _lib.REGION_MU]


def _check(w, fmt="e4m3", q_centre=False):
    q, k, v = generate(w, device="cuda")
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0, fmt=fmt, q_centre=q_centre)
    n = plan.stats_offset()
    log(f"noalloc {w.name} T={w.tokens} H={w.heads} fmt={fmt}: workspace {plan.workspace_bytes} B, "
        f"noalloc workspace {n} B")
    assert 0 < n < plan.workspace_bytes
    ws_ref = plan.new_workspace()
    fa.quantize(plan, q, k, v, ws_ref)
    ws_na = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    fa.quantize_noalloc(plan, q, k, v, ws_na)
    torch.cuda.synchronize()
    regions = MX_REGIONS if fmt == "mxfp4" else E4M3_REGIONS + ([_lib.REGION_QMEAN, _lib.REGION_QM_TERM] if q_centre else [])
    for r in regions:
        a, b = plan.region(ws_ref, r), plan.region(ws_na, r)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), r
    log("  forward from both workspaces")
    o_ref = fa.forward(plan, ws_ref)
    o_na = fa.forward(plan, ws_na)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o_na)
    plan.close()


def test_noalloc_matches_quantize_on_two_calls_second_smaller():
    # the large call fills most of the static buffer (6720 of about 8000 chunk-heads);
    # the smaller one after it must not see anything the first left behind
    _check(make_workload("noalloc_large", 30272, 56, [0, 15104, 30208, 30208, 30271, 30272], seed=1201))
    _check(make_workload("noalloc_small", 700, 3, [0, 300, 700], seed=1202, k_offset_var=2.0))


def test_noalloc_fp4_plan_and_segment_edges():
    _check(make_workload("noalloc_mx", 1500, 4, [0, 0, 1, 64, 65, 1500], seed=1203, k_offset_var=2.0),
           fmt="mxfp4", q_centre=True)
    _check(make_workload("noalloc_tiny", 257, 2, [0, 1, 257], seed=1204))


def test_noalloc_e4m3_q_centre():
    # the Q block statistics go to the static buffer as well
    _check(make_workload("noalloc_qc", 1500, 3, [0, 0, 1, 64, 65, 193, 700, 700, 1500], seed=1205,
                         k_offset_var=2.0, q_offset_var=2.0), q_centre=True)
    _check(make_workload("noalloc_qc_small", 300, 2, [0, 300], seed=1206, q_offset_var=2.0), q_centre=True)


def test_noalloc_rejects_plans_beyond_the_static_buffer():
    T, H = 320_037, 56
    plan = fa.Plan(T, H, [0, T], device=0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    x = torch.empty((1, H, 128), dtype=torch.bfloat16, device="cuda").expand(T, H, 128)
    with pytest.raises(fa.Fp8AttnError) as e:
        fa.quantize_noalloc(plan, x, x, x, ws)
    assert e.value.status == _lib.EUNSUPPORTED and "static buffer" in str(e.value)
