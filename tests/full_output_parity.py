"""Full-output parity of the graded workloads: every output row of every head
against the float64 oracle, and the E4M3 codes, scales and K means of every
head against the CPU quantizer.  A script, not a pytest module (the oracle
needs minutes of host CPU per workload); it runs on a machine with the GPU:

    python -u -m tests.full_output_parity s4096_h56 s20440_h56_strided --out parity.json

Per workload it reports, over all T x H x 128 output elements: the relative
RMS error ||o - r|| / ||r|| (the reading of the pages' "relative RMS"), the
largest |o - r|, the largest excess over |o - r| <= 0.1 + 0.1 |r| (<= 0 means
every element is inside) and, on the rows that see fewer than 64 keys, the
same excess against the oracle on the dequantized operands; and the number of
code, scale and mean mismatches over all heads.  The launch is the one
``bench.py`` times (the default plan and workspace of the workload).
Progress is printed per head.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import fp8_flash_attention_amd as fa  # noqa: E402
from oracle import attention as A  # noqa: E402
from oracle import compare  # noqa: E402
from oracle import quantize as Qz  # noqa: E402
from tests.cases import FEW_KEYS, visible_keys  # noqa: E402
from tests.gpu_helpers import read_codes  # noqa: E402
from workloads import WORKLOADS, generate  # noqa: E402


def run(name: str) -> dict:
    w = WORKLOADS[name]
    t0 = time.time()
    print(f"[{name}] T={w.tokens} H={w.heads} cu={list(w.cu_seqlens)}", flush=True)
    qc, kc, vc = generate(w)
    q, k, v = (x.to("cuda:0") for x in (qc, kc, vc))
    plan = fa.Plan(w.tokens, w.heads, w.cu_seqlens, w.softmax_scale, device=0)
    ws = plan.new_workspace()
    fa.quantize(plan, q, k, v, ws)
    out = fa.forward(plan, ws)
    torch.cuda.synchronize()
    got_all = out.cpu()                                   # bf16 [T, H, 128]
    codes = read_codes(plan, ws)                          # every head, canonical order
    del q, k, v, out, ws
    torch.cuda.empty_cache()
    few = visible_keys(w.cu_seqlens, False) < FEW_KEYS
    num = den = 0.0
    max_abs = -np.inf
    excess = -np.inf
    excess_few_diag = -np.inf
    mismatches = {"q_codes": 0, "k_codes": 0, "v_codes": 0, "scales": 0, "mu": 0}
    per_head_rr = []
    for h in range(w.heads):
        hs = [h]
        qh, kh, vh = qc[:, hs], kc[:, hs], vc[:, hs]
        r = Qz.quantize(qh, kh, vh, w.cu_seqlens, w.softmax_scale)
        for key in ("q_codes", "k_codes", "v_codes"):
            mismatches[key] += int(np.count_nonzero(codes[key][:, hs] != r[key]))
        mismatches["scales"] += int(np.count_nonzero(
            np.asarray(codes["scales"])[:, hs].view(np.uint32) != r["scales"].view(np.uint32)))
        mismatches["mu"] += int(np.count_nonzero(codes["mu"][:, hs].view(np.uint32) != r["mu"].view(np.uint32)))
        ref = A.attention(qh, kh, vh, w.cu_seqlens, w.softmax_scale).numpy()
        got = got_all[:, hs].double().numpy()
        d = got - ref
        num += float(np.sum(d * d))
        den += float(np.sum(ref * ref))
        max_abs = max(max_abs, float(np.abs(d).max()))
        per_head_rr.append(float(np.sqrt(np.sum(d * d) / np.sum(ref * ref))))
        e = np.abs(d) - (compare.ATOL_BAR + compare.RTOL_BAR * np.abs(ref))
        excess = max(excess, float(e[~few].max()) if (~few).any() else -np.inf)
        if few.any():
            rows = list(np.nonzero(few)[0])
            dq, dk, dv = (Qz.dequantize(r[n], r["scales"][i])
                          for i, n in enumerate(("q_codes", "k_codes", "v_codes")))
            diag = A.attention_rows(dq, dk, dv, w.cu_seqlens, w.softmax_scale, rows).numpy()
            excess_few_diag = max(excess_few_diag, compare.allclose_excess(got[rows], diag))
        print(f"[{name}] head {h}: rel_rms {per_head_rr[-1]:.5f} max_abs {float(np.abs(d).max()):.5f} "
              f"({time.time() - t0:.0f} s)", flush=True)
    res = {"workload": name, "tokens": w.tokens, "heads": w.heads, "cu_seqlens": list(w.cu_seqlens),
           "elements": int(w.tokens * w.heads * 128),
           "rel_rms": float(np.sqrt(num / den)), "max_abs": max_abs,
           "allclose_excess_rows_ge_64_keys": excess,
           "rows_lt_64_keys": int(few.sum()),
           "allclose_excess_rows_lt_64_keys_vs_dequantized": (excess_few_diag if few.any() else None),
           "rel_rms_per_head_min": min(per_head_rr), "rel_rms_per_head_max": max(per_head_rr),
           "code_mismatches": mismatches, "host_threads": torch.get_num_threads(),
           "seconds": round(time.time() - t0, 1)}
    print(json.dumps(res), flush=True)
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="+")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    results = [run(n) for n in args.workloads]
    if args.out:
        with open(args.out, "w") as f:
            json.dump(results, f, indent=1)
    ok = all(r["rel_rms"] <= compare.REL_RMS_BAR and r["allclose_excess_rows_ge_64_keys"] <= 0
             and (r["allclose_excess_rows_lt_64_keys_vs_dequantized"] or -1) <= 0
             and not any(r["code_mismatches"].values()) for r in results)
    print("ALL WITHIN BARS" if ok else "SOME BAR MISSED", flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
