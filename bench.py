"""Benchmark of one replay step on one MI355X.

A step is one pass of the whole hot path over one synthetic member: the split
forward over the paged prompt, the causal response block, the exact LSE merge,
and the response-only backward (D = rowsum(dO*O), per-split dQ, response dQ,
response dK/dV, ordered dQ sum).  Inputs are resident in HBM before timing
starts, and the prompt's page table (host split + upload, once per prompt) is
built before it too.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--score]

The default workload is the 2,097,152-position prefix with R = 1024 (one member).  Any name in
``replay_inputs.WORKLOADS`` can be given; for the G = 8 group a step is the serial replay of all
eight members (R = 512 ... 4096) over the shared prompt, `prompt_keys_per_s` counts prompt keys
times members, and the line also carries each member's time from one extra, untimed pass.
``--score`` times forward-only scoring instead: all members in one pass over the prompt
(``ls_replay_attn_fwd_members``) and the merge, counting forward flops only.
``--blocks N`` replays the member as N token blocks, last block first (each block's forward,
merge and backward at its offset in the response, dK/dV added into one buffer); the flops are
those of the whole member.
A name in ``replay_inputs.CAPTURE_WORKLOADS`` times the chunked capture of one full-attention
layer instead: a step prefills the whole prompt chunk by chunk (each chunk's forward over the
pages before it and itself, the merge, and the append of its pages); flops are the forward's.

Prints one JSON line.  ``value`` is algorithmic TFLOP/s of the whole step
(only unmasked scores counted: 4d flops per (head,row,key) forward; 6d per
prompt key and 10d per response key backward, no prompt dK/dV work); the same
line carries prompt-keys/s, the roofline of the dominant kernel (measured with
HIP events on its launch stream over the timed region) and the float64 oracle
timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E (published)
DOMINANT = "bwd_prompt_dq"  # 60% of the algorithmic flops
KERNELS = ("fwd_prompt", "fwd_combine", "fwd_resp", "lse_merge", "bwd_dot", "bwd_prompt_dq",
           "bwd_resp_dq", "bwd_resp_dkdv", "kv_reduce", "dq_reduce", "page_append")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "bwd_prompt_dq_traffic_prefix2M.md")
CLOCK_SUMMARY = os.path.join(ROOT, "profiles", "prompt_kernels_clock_lds_prefix2M.md")
GEMM_SUMMARY = os.path.join(ROOT, "profiles", "library_gemm_bf16_ceiling.md")
PROBE_SUMMARY = os.path.join(ROOT, "profiles", "mfma_calibration_probes.md")
NOMINAL_CLOCK_GHZ = 2.4     # the clock of the published peak (256 CU x 4 SIMD x 1024 flop/clk)


def flops(shape) -> dict:
    d, hq, r, p = shape.head_dim, shape.hq, shape.resp_len, shape.prompt_len
    causal = r * (r + 1) // 2
    return {
        "fwd_prompt": 4 * d * hq * r * p,
        "fwd_resp": 4 * d * hq * causal,
        "bwd_prompt_dq": 6 * d * hq * r * p,
        "bwd_resp": 10 * d * hq * causal,
    }


def source_digest() -> str:
    """Hash of the kernel sources with comments and blank space taken out, so
    that a counter summary stays attached to the code it measured across
    edits that change no code.  The calibration probe (ls_calib.hip) is not
    part of the measured path and is left out."""
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "response_replay_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp", ".h")) and name != "ls_calib.hip":
            with open(os.path.join(csrc, name)) as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            text = " ".join(text.split())
            h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def read_traffic(digest: str):
    """Per-launch HBM bytes of the dominant kernel from the committed counter
    summary, or None if it is missing or was taken on other kernel sources."""
    vals = summary_values(TRAFFIC_SUMMARY)
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summary_values(path: str) -> dict:
    """The ``- key: `value` `` lines of a committed profile summary."""
    vals = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    return vals


def measured_clock_ghz(kernel: str):
    """Sustained shader clock during `kernel` from the committed counter
    summary (GRBM_GUI_ACTIVE per XCD over the dispatch's duration), or None."""
    try:
        return float(summary_values(CLOCK_SUMMARY)[f"{kernel}_clock_ghz"])
    except (KeyError, ValueError):
        return None


def lds_fed_mfma_tflops():
    """Sustained rate of the calibration probe whose MFMAs take their A
    operand from LDS at the attention kernels' ratio (`bench.py
    --mfma-probe`, mode 2) from the committed summary, or None."""
    try:
        return float(summary_values(PROBE_SUMMARY)["lds_fed_mfma_tflops"])
    except (KeyError, ValueError):
        return None


def library_gemm_tflops():
    """Sustained rate of the vendor library's square bf16 GEMM on this part
    (`bench.py --library-gemm`) from the committed summary, or None."""
    try:
        return float(summary_values(GEMM_SUMMARY)["library_gemm_tflops"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(shape, inp, seconds_hint: float = 20.0):
    """The float64 oracle on the host, on a bounded sample: KV head 0, its
    query heads, `rows` response rows each (always including the last rows,
    whose causal response block is the largest)."""
    import numpy as np
    import torch

    import oracle
    from replay_inputs import logical_prompt

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    g = shape.hq // shape.hkv
    # about 15 s of host work at the 2M prefix: ~1.2e7 (row x prompt-key)
    # pairs per second measured for forward + backward
    rows = max(1, min(64, shape.resp_len, (32 << 20) // max(shape.prompt_len, 1)))
    t0 = time.perf_counter()
    kp = logical_prompt(inp["k_pool"], inp["l2p"], shape.prompt_len, kv_heads=[0]).cpu()
    vp = logical_prompt(inp["v_pool"], inp["l2p"], shape.prompt_len, kv_heads=[0]).cpu()
    q = inp["q"][:g].cpu()
    do = inp["d_o"][:g].cpu()
    kr, vr = inp["k_resp"][:1].cpu(), inp["v_resp"][:1].cpu()
    R = shape.resp_len
    sel = np.tile(np.arange(R - rows, R), (g, 1))
    t1 = time.perf_counter()
    oracle.replay_forward(q, kp, vp, kr, vr, shape.scale, rows=sel)
    oracle.replay_backward(q, kp, vp, kr, vr, do, shape.scale, rows=sel)
    t2 = time.perf_counter()
    d, P = shape.head_dim, shape.prompt_len
    n = g * rows
    resp_keys = sum(i + 1 for i in range(R - rows, R)) * g
    algo = (4 + 6) * d * n * P + (4 + 10) * d * resp_keys
    secs = t2 - t1
    return {
        "value": algo / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 oracle forward+backward of {n} response rows (KV head 0: {g} query heads x "
                   f"the last {rows} rows) over the full {P}-position prompt; {secs:.1f} s compute "
                   f"(+{t1 - t0:.1f} s to gather inputs), scaled as algorithmic flops per second"),
        "prompt_keys_per_s_equiv": P * n / (shape.hq * R) / secs,
    }


def capture_flops(shape) -> dict:
    """Forward flops of the chunked capture: chunk [s, e) scores every earlier
    position and, causally, itself."""
    d, hq = shape.head_dim, shape.hq
    out = {"fwd_prompt": 0, "fwd_resp": 0}
    for s, e in shape.spans():
        tc = e - s
        out["fwd_prompt"] += 4 * d * hq * tc * s
        out["fwd_resp"] += 4 * d * hq * tc * (tc + 1) // 2
    return out


def cpu_baseline_capture(shape, inp):
    """The float64 oracle on the host: causal attention of the last rows of the
    prompt (query heads of KV head 0) over every position before them."""
    import numpy as np

    import oracle
    from replay_inputs import whole_prompt

    g = shape.hq // shape.hkv
    T = shape.total_len
    # about 10 s of host work: ~6e7 (row x key) pairs per second measured
    rows = max(1, min(512, (96 << 20) // T))
    t0 = time.perf_counter()
    q = whole_prompt([(c[0][:g], c[1][:1], c[2][:1]) for c in inp["chunks"]], 0)[:, T - rows:].cpu()
    k = whole_prompt([(None, c[1][:1], None) for c in inp["chunks"]], 1).cpu()
    v = whole_prompt([(None, None, c[2][:1]) for c in inp["chunks"]], 2).cpu()
    # the sampled rows are the last ones: give the oracle the sequence's keys
    # as the prompt and the sampled rows' own keys as the causal block
    kp, vp = k[:, : T - rows], v[:, : T - rows]
    kr, vr = k[:, T - rows:], v[:, T - rows:]
    sel = np.tile(np.arange(rows), (g, 1))
    t1 = time.perf_counter()
    oracle.replay_forward(q, kp, vp, kr, vr, shape.scale, rows=sel)
    t2 = time.perf_counter()
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    n = g * rows
    keys = sum(T - rows + i + 1 for i in range(rows)) * g
    secs = t2 - t1
    return {
        "value": 4 * shape.head_dim * keys / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"float64 oracle forward of {n} rows (KV head 0: {g} query heads x the last {rows} "
                   f"positions) over every earlier position of the {T}-position prompt; "
                   f"{secs:.1f} s compute (+{t1 - t0:.1f} s to gather inputs)"),
    }


def bench_library_gemm(args) -> int:
    """Calibration, not the workload: the vendor library's dense bf16 GEMM
    (torch.matmul, which dispatches to hipBLASLt) on square operands, timed
    with HIP events on the current stream.  Its sustained rate is the
    practical MFMA ceiling of the part: the clock it holds under a full
    matrix load is below the 2.4 GHz of the published peak."""
    import torch
    torch.manual_seed(args.seed)
    dev = torch.device("cuda:0")
    res = {}
    for n, iters in ((8192, 50), (16384, 8)):
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        res[str(n)] = {"ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / ms / 1e9, 1)}
        print(f"gemm {n}^3 bf16: {ms:.3f} ms, {res[str(n)]['tflops']} TFLOP/s", file=sys.stderr,
              flush=True)
        del a, b, c
    best = max(v["tflops"] for v in res.values())
    print(json.dumps({
        "metric": "library dense bf16 GEMM TFLOP/s (calibration)", "value": best,
        "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic", "config": {"workload": "torch.matmul square bf16", "sizes": res},
        "frac_of_bf16_peak": round(best / PEAK_BF16_TFLOPS, 4)}), flush=True)
    return 0


def bench_mfma_probe(args) -> int:
    """Calibration, not the workload: the library's MFMA probe
    (ls_calib_mfma) in its four modes, 2048 workgroups of 512 threads, three
    timed launches each after one warm-up launch, HIP events on the current
    stream.  Register operands give the rate the part sustains on the matrix
    units alone under its power limit; LDS operands at the attention kernels'
    1 KiB per 32768 flop add the cost of their operand stream."""
    import torch

    from response_replay_attention_amd import ls_calib_mfma
    dev = torch.device("cuda:0")
    wgs, iters = 2048, 100_000
    out_t = torch.empty(wgs * 512, dtype=torch.float32, device=dev)
    names = {0: "32x32x16 bf16, register operands", 1: "16x16x32 bf16, register operands",
             2: "32x32x16 bf16, A from LDS (1 KiB per MFMA)",
             3: "16x16x32 bf16, A from LDS (1 KiB per two MFMAs)"}
    res = {}
    for mode, name in names.items():
        ls_calib_mfma(mode, wgs, 8, out_t)
        rates = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fl = ls_calib_mfma(mode, wgs, iters, out_t)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            rates.append(fl / ms / 1e9)
            print(f"mode {mode} ({name}): {ms:.2f} ms, {rates[-1]:.1f} TFLOP/s", file=sys.stderr,
                  flush=True)
        res[str(mode)] = {"probe": name, "tflops": round(max(rates), 1),
                          "tflops_all": [round(r, 1) for r in rates]}
    print(json.dumps({
        "metric": "MFMA calibration probe TFLOP/s (power-limited ceiling)",
        "value": res["2"]["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ls_calib_mfma", "workgroups": wgs, "steps": iters, "modes": res}}),
        flush=True)
    return 0


def bench_capture(args, shape) -> int:
    import torch

    from replay_inputs import make_capture_inputs
    from response_replay_attention_amd import (capture_prefill, ls_timing_enable, ls_timing_read,
                                               ls_timing_reset)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_capture_inputs(shape, args.seed, device=dev)
    torch.cuda.synchronize()

    def step():
        capture_prefill(inp["chunks"], inp["k_pool"], inp["v_pool"], inp["slots"],
                        shape.num_splits, shape.policy, shape.block_pages, shape.scale,
                        consume=lambda i, o, lse: None)

    for _ in range(args.warmup):
        step()
    ls_timing_reset()
    ls_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ls_timing_enable(False)
    kern = {}
    for k in KERNELS:
        n, ms = ls_timing_read(k)
        if n:
            kern[k] = {"launches": n, "avg_ms": ms / n, "total_ms": ms}
    fl = capture_flops(shape)
    step_flops = sum(fl.values())
    tflops = step_flops * args.steps / elapsed / 1e12
    # launches of the dominant kernel differ in size (the prompt grows chunk by
    # chunk): its achieved rate is all its flops over all its time
    dom = kern.get("fwd_prompt", {"total_ms": float("nan"), "launches": 0})
    achieved = fl["fwd_prompt"] * args.steps / (dom["total_ms"] * 1e-3) / 1e12
    app = kern.get("page_append", {"avg_ms": float("nan")})
    chunk_bytes = 2 * shape.hkv * shape.chunk * shape.head_dim * 2  # K and V, bf16
    out = {
        "metric": "chunked capture (forward) TFLOP/s & positions/s; % bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": shape.name,
            "q_heads": shape.hq, "kv_heads": shape.hkv, "head_dim": shape.head_dim,
            "prompt_len": shape.total_len, "chunk": shape.chunk, "splits": shape.num_splits,
            "page_size": 256, "parallelism": "1 GPU; CP ranks emulated as page splits",
        },
        "positions_per_s": round(shape.total_len * args.steps / elapsed, 1),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {
            "kernel": "fwd_prompt",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "source_digest": source_digest(),
        },
        # the page writer is HBM-bound: K and V of a whole chunk read once and written once
        "page_append": {
            "avg_ms": round(app["avg_ms"], 4),
            "achieved_GBps": round(2 * chunk_bytes / (app["avg_ms"] * 1e-3) / 1e9, 1),
            "peak_GBps": PEAK_HBM_GBPS,
        },
        "kernels_avg_ms": {k: round(v["avg_ms"], 4) for k, v in kern.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_capture(shape, inp)
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefix_24x4_d256_p2097152_r1024_s8")
    ap.add_argument("--seed", type=int, default=20260002)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--score", action="store_true",
                    help="forward-only scoring of all members in one pass over the prompt "
                         "(merged O and LSE per member, no backward)")
    ap.add_argument("--blocks", type=int, default=1,
                    help="replay the member as this many token blocks, last block first")
    ap.add_argument("--late-dominant-keys", action="store_true",
                    help="every query row points near one direction and the last 64 prompt keys "
                         "of KV head 0 dominate it (the forward's exact recompute in the last "
                         "split); not a headline workload")
    ap.add_argument("--identity-pages", action="store_true",
                    help="place logical page p in pool slot p instead of a seeded random slot")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="calibration only: time the vendor library's square bf16 GEMM "
                         "(the practical MFMA ceiling) instead of a workload")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="calibration only: the MFMA rate the part sustains under its power "
                         "limit, with register operands and with an LDS operand stream")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (its page splits "
              "stand in for the context-parallel ranks on one device); run with --gpus 1",
              file=sys.stderr)
        return 2

    if args.library_gemm:
        return bench_library_gemm(args)
    if args.mfma_probe:
        return bench_mfma_probe(args)

    import torch

    from replay_inputs import (CAPTURE_WORKLOADS, FULL_2M, GROUP_2M, GROUP_2M_RESP_LENS,
                               WORKLOADS, make_inputs, make_response, plant_late_dominant_keys)
    if args.workload in CAPTURE_WORKLOADS:
        return bench_capture(args, CAPTURE_WORKLOADS[args.workload])
    from response_replay_attention_amd import (Member, PromptCache, block_bounds, ls_timing_enable,
                                               ls_timing_read, ls_timing_reset, replay_backward,
                                               replay_forward, replay_group, replay_token_blocks,
                                               score_group)

    shape = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    group = shape.name == GROUP_2M.name
    # the group replays G members of different lengths over one shared prompt;
    # every other workload is one member
    member_shapes = ([shape.with_(resp_len=r) for r in GROUP_2M_RESP_LENS] if group else [shape])
    inp = make_inputs(member_shapes[0], args.seed, device=dev, identity_pages=args.identity_pages)
    if args.late_dominant_keys:
        plant_late_dominant_keys(inp, member_shapes[0], args.seed, kv=0, n=64)
    members = [Member(inp["q"], inp["k_resp"], inp["v_resp"], inp["d_o"])]
    for i, sh in enumerate(member_shapes[1:], start=1):
        r = make_response(sh, args.seed + i, device=dev)
        members.append(Member(r["q"], r["k_resp"], r["v_resp"], r["d_o"]))
    if args.blocks > 1 and (group or args.score):
        print("--blocks applies to one member's replay", file=sys.stderr)
        return 2
    m0 = members[0]
    bounds = block_bounds(shape.resp_len, args.blocks) if args.blocks > 1 else []
    block_inputs = [(m0.q[:, s:e].contiguous(), m0.d_o[:, s:e].contiguous()) for s, e in bounds]
    torch.cuda.synchronize()

    def make_cache():
        return PromptCache(inp["k_pool"], inp["v_pool"], shape.prompt_len, inp["l2p"],
                           shape.num_splits, shape.policy, shape.block_pages)

    # the page table is built (host split) and uploaded once per prompt, before
    # the timed region: a step is the attention path proper, K1..K7
    cache = make_cache()

    def step():
        if args.score:
            score_group(cache, members, scale=shape.scale)
            return
        if group:
            replay_group(cache, members, scale=shape.scale)
            return
        if block_inputs:
            replay_token_blocks(cache, block_inputs, m0.k_resp, m0.v_resp, shape.scale,
                                consume=lambda b, fwd, dq: None)
            return
        m = members[0]
        fwd = replay_forward(cache, m.q, m.k_resp, m.v_resp, shape.scale)
        replay_backward(cache, m.q, m.k_resp, m.v_resp, fwd.o, fwd.lse, m.d_o, shape.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ls_timing_reset()
    ls_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ls_timing_enable(False)
    kern = {}
    for k in KERNELS:
        n, ms = ls_timing_read(k)
        if n:
            kern[k] = {"launches": n, "avg_ms": ms / n}

    per_member = [flops(sh) for sh in member_shapes]
    if args.score:  # forward work only
        per_member = [{k: v for k, v in f.items() if k.startswith("fwd")} for f in per_member]
    step_flops = sum(sum(f.values()) for f in per_member)
    ms_step = elapsed / args.steps * 1e3
    tflops = step_flops * args.steps / elapsed / 1e12
    dominant = "fwd_prompt" if args.score else DOMINANT
    dom = kern.get(dominant, {"avg_ms": float("nan")})
    # the dominant kernel's flops per launch: the members' mean (one launch per
    # member), or all members at once when scoring
    dom_flops = sum(f["fwd_prompt" if args.score else "bwd_prompt_dq"] for f in per_member)
    if not args.score:
        dom_flops /= len(per_member)
    if block_inputs:  # one dominant launch per block, each over its own rows
        dom_flops /= len(block_inputs)
    achieved = dom_flops / (dom["avg_ms"] * 1e-3) / 1e12
    digest = source_digest()
    # the counters were taken on the default workload (random page placement)
    traffic = (read_traffic(digest) if shape.name == FULL_2M.name and not args.score
               and not args.identity_pages and not block_inputs and not args.late_dominant_keys
               else None)

    out = {
        "metric": "replay-attn fwd+bwd TFLOP/s & prompt-keys/s at 2M prefix; % bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": shape.name,
            "q_heads": shape.hq, "kv_heads": shape.hkv, "head_dim": shape.head_dim,
            "prompt_len": shape.prompt_len, "resp_len": shape.resp_len,
            "splits": shape.num_splits, "page_size": shape.page_size,
            "parallelism": "1 GPU; CP ranks emulated as page splits",
        },
        "prompt_keys_per_s": round(shape.prompt_len * len(members) * args.steps / elapsed, 1),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "source_digest": digest,
        },
        # the same fraction against the peak at the shader clock measured under
        # this kernel (the published peak assumes 2.4 GHz)
        "frac_at_measured_clock": None,
        "kernels_avg_ms": {k: round(v["avg_ms"], 4) for k, v in kern.items()},
    }
    clk = measured_clock_ghz(dominant)
    if clk:
        out["frac_at_measured_clock"] = {
            "clock_ghz": clk, "peak": round(PEAK_BF16_TFLOPS * clk / NOMINAL_CLOCK_GHZ, 1),
            "frac": round(achieved / (PEAK_BF16_TFLOPS * clk / NOMINAL_CLOCK_GHZ), 4),
            "source": os.path.relpath(CLOCK_SUMMARY, ROOT)}
    gemm = library_gemm_tflops()
    if gemm:
        # the same kernel against what the vendor's own bf16 GEMM sustains here
        out["frac_of_library_gemm"] = {
            "library_gemm_tflops": gemm, "frac": round(achieved / gemm, 4),
            "step_frac": round(tflops / gemm, 4),
            "source": os.path.relpath(GEMM_SUMMARY, ROOT)}
    probe = lds_fed_mfma_tflops()
    if probe:
        # against the MFMA rate the part sustains with an LDS operand stream of
        # the same bytes per flop (no softmax, copies or barriers)
        out["frac_of_lds_fed_mfma_probe"] = {
            "probe_tflops": probe, "frac": round(achieved / probe, 4),
            "source": os.path.relpath(PROBE_SUMMARY, ROOT)}
    if args.identity_pages:
        out["config"]["page_layout"] = "identity"
    if args.late_dominant_keys:
        out["config"]["inputs"] = "late dominant keys (last 64 prompt keys of KV head 0)"
    if block_inputs:
        out["config"]["token_blocks"] = [list(b) for b in bounds]
        out["config"]["mode"] = "reverse token-block replay"
        out["roofline"]["traffic"] = None
    if args.score:
        out["metric"] = "group scoring (forward only) TFLOP/s & prompt-keys/s; % bf16 MFMA peak"
        out["config"]["mode"] = "score"
    if group and not args.score:
        out["config"]["members"] = len(members)
        out["config"]["resp_lens"] = list(GROUP_2M_RESP_LENS)
        # one more pass, outside the timed region, for the time of each member
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(members) + 1)]
        ev[0].record()
        for i, m in enumerate(members):
            replay_group(cache, [m], scale=shape.scale)
            ev[i + 1].record()
        torch.cuda.synchronize()
        out["per_member_ms"] = [round(ev[i].elapsed_time(ev[i + 1]), 3) for i in range(len(members))]
    if group and args.score:
        out["config"]["members"] = len(members)
        out["config"]["resp_lens"] = list(GROUP_2M_RESP_LENS)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(member_shapes[0], inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
