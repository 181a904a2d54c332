"""Host-side checks of bench.py and the committed profile summaries (no GPU)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_counter_entries_carry_what_the_bench_reads():
    with open(bench.COUNTERS_FILE) as f:
        d = json.load(f)
    for key in ("s30272_h56_koffset", "s30272_h56_koffset:mxfp4", "s30272_h56_koffset:mxfp4:qc"):
        e = d[key]
        assert len(e["kernel_hash"]) == 16
        assert e["hbm_bytes_per_launch"] == e["read_bytes"] + e["write_bytes"] > 0


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "fp8_flash_attention_amd", "csrc")
    csrc = tmp_path / "fp8_flash_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("attention.hip", "internal.h"):
        with open(os.path.join(src, f)) as fh:
            (csrc / f).write_text(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    (csrc / "attention.hip").write_text((csrc / "attention.hip").read_text() + "\n// a note\n\n/* more */\n")
    assert bench.kernel_source_hash() == h0
    (csrc / "attention.hip").write_text((csrc / "attention.hip").read_text() + "static int x;\n")
    assert bench.kernel_source_hash() != h0


def test_every_profile_summary_names_its_command():
    pdir = os.path.join(ROOT, "profiles")
    for f in sorted(os.listdir(pdir)):
        if f.endswith(".md"):
            with open(os.path.join(pdir, f)) as fh:
                t = fh.read()
            assert "rocprofv3 " in t and "bench.py" in t, f
            assert os.path.getsize(os.path.join(pdir, f)) < 64 * 1024, f
