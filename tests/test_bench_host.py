"""Host checks of bench.py: its flop counts against brute-force enumeration,
the parsing of the committed profile summaries it reads, its kernel names
against the C header, and its refusal of more than one GPU.  No GPU needed."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from replay_inputs import CaptureShape, ReplayShape  # noqa: E402


def test_replay_flops_match_enumerated_pairs():
    # 4d flops per visible (head, row, key) pair forward; backward 6d per prompt
    # pair (S, dP, dQ) and 10d per response pair (S, dP, dQ, dK, dV)
    sh = ReplayShape("t", 3, 1, 8, 7, 5, 1)
    prompt_pairs = resp_pairs = 0
    for _h in range(sh.hq):
        for i in range(sh.resp_len):
            prompt_pairs += sh.prompt_len
            resp_pairs += sum(1 for j in range(sh.resp_len) if j <= i)
    d = sh.head_dim
    assert bench.flops(sh) == {
        "fwd_prompt": 4 * d * prompt_pairs, "fwd_resp": 4 * d * resp_pairs,
        "bwd_prompt_dq": 6 * d * prompt_pairs, "bwd_resp": 10 * d * resp_pairs}


def test_capture_flops_match_enumerated_pairs():
    # position t of chunk [s, e) sees the captured positions [0, s) through the
    # pages and, causally, [s, t] of its own chunk
    sh = CaptureShape("c", 2, 1, 8, 700, 256, 2)
    prompt_pairs = resp_pairs = 0
    for s, e in sh.spans():
        for t in range(s, e):
            prompt_pairs += s
            resp_pairs += t - s + 1
    prompt_pairs *= sh.hq
    resp_pairs *= sh.hq
    assert bench.capture_flops(sh) == {"fwd_prompt": 4 * 8 * prompt_pairs,
                                       "fwd_resp": 4 * 8 * resp_pairs}


def test_summary_values_and_traffic_digest_guard(tmp_path, monkeypatch):
    f = tmp_path / "s.md"
    f.write_text("prose: not a value\n- source_digest: `abc123`\n- hbm_bytes_per_launch: `1.5e+10`\n")
    assert bench.summary_values(str(f)) == {"source_digest": "abc123",
                                            "hbm_bytes_per_launch": "1.5e+10"}
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(f))
    assert bench.read_traffic("abc123") == 1.5e10
    assert bench.read_traffic("other") is None  # counters of other kernel sources are not used
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.read_traffic("abc123") is None


def test_committed_summaries_are_machine_readable():
    vals = bench.summary_values(bench.TRAFFIC_SUMMARY)
    assert re.fullmatch(r"[0-9a-f]{16}", vals["source_digest"])
    assert float(vals["hbm_bytes_per_launch"]) > float(vals["algorithmic_bytes_per_launch"]) > 0
    for k in ("fwd_prompt", "bwd_prompt_dq"):
        assert 1.0 < bench.measured_clock_ghz(k) <= 2.4
    assert 1000 < bench.library_gemm_tflops() < bench.PEAK_BF16_TFLOPS
    assert bench.library_gemm_tflops() < bench.lds_fed_mfma_tflops() < bench.PEAK_BF16_TFLOPS


def test_timed_kernel_names_match_the_header():
    text = open(os.path.join(ROOT, "include", "ls_replay.h")).read()
    block = text[text.index("Kernel names:"):text.index("ls_timing_enable(0)")]
    assert sorted(re.findall(r'"(\w+)"', block)) == sorted(bench.KERNELS + ("resolve_pages",))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
