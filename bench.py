"""Benchmark of the hybrid layer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload cfg5] [--no-cpu-baseline]

A step is one hybrid_layer_step over one synthetic hybrid batch, inputs resident in HBM. The
default workload is the largest single-GPU one: a 70B-shaped layer (hidden 8192, 64/8 heads,
head_dim 128, d_ff 28672) with one 512-token prompt chunk at prefix 8192 plus 512 decodes whose
contexts are log-uniform in [1024, 32768] (seeded synthetic values; paged 16-token KV, about
19 GB of it, with a random block table). Prints ONE JSON line.

Besides the whole-step throughput it times every phase inside real steps (the same steps run
again with the library's phase marks, HIP events it records between its kernels) and through its
own entry point with HIP events on the launch stream (attention work lists built outside the
timed launches, as the step builds them in its first normalisation pass), reports the dominant
kernel against its roofline (HBM bytes for attention, matrix-core flops for a GEMM; its time
from the phase-marked steps), the GEMMs against the bf16 matrix-core
peak, the decode attention against HBM peak, and the fp64 oracle timed on the host cores over a
bounded sample of the same batch as a baseline.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak
SPIN_CYCLES = 2_000_000     # GPU spin between a phase's set-up and its timed launch
# the step's phases between consecutive marks of hl_batch_desc::events
STEP_PHASES = ("qkv_rope_append", "attention", "gemm_o", "rms_scale_mlp", "gemm_gate_up",
               "gemm_down")


def log(msg):
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"# {time.strftime('%H:%M:%S')} {msg}", file=sys.stderr, flush=True)


def algorithmic_counts(spec):
    """Work the method must do (no padding, causal-visible pairs only, KV read once per KV head)."""
    s = spec.shape
    T = spec.num_tokens
    d, hq, hkv = s.head_dim, s.n_q_heads, s.n_kv_heads
    gemm = {
        "qkv": 2.0 * T * s.hidden * s.qkv_cols,
        "o": 2.0 * T * hq * d * s.hidden,
        "gate_up": 2.0 * T * s.hidden * 2 * s.d_ff,
        "down": 2.0 * T * s.d_ff * s.hidden,
    }
    pairs = 0
    dec_bytes = 0
    for c, n in spec.seqs:
        if n > 1:
            pairs += n * c + n * (n + 1) // 2
        else:
            dec_bytes += (c + 1) * hkv * d * 2 * 2
    # every byte attention must move once: K and V of each sequence's keys (once per KV head),
    # its queries (decodes: two bf16 halves) and its output rows
    pre_kv, pre_io, dec_io = 0, 0, 0
    for c, n in spec.seqs:
        if n > 1:
            pre_kv += (c + n) * hkv * d * 2 * 2
            pre_io += 2 * n * hq * d * 2
        else:
            dec_io += 3 * hq * d * 2
    return {
        "gemm_flops": gemm,
        "weight_bytes": 2.0 * s.weight_params,
        "prefill_attn_flops": 4.0 * d * hq * pairs,
        "decode_kv_bytes": float(dec_bytes),
        "decode_attn_bytes": float(dec_bytes + dec_io),
        "prefill_attn_bytes": float(pre_kv + pre_io),
    }


ATTN_MODES = {"auto": 0, "fused": 1, "separate": 2}


def pct(v):
    """median, p10 and p90 of a sorted list of milliseconds"""
    if not v:
        return None
    q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
    return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4),
            "max": round(v[-1], 4), "n": len(v)}


def gpu_clocks():
    """Current SCLK / MCLK as rocm-smi reports them (a child process; None if unavailable)."""
    import shutil
    import subprocess
    exe = shutil.which("rocm-smi")
    if not exe:
        return None
    try:
        r = subprocess.run([exe, "--showclocks"], capture_output=True, text=True, timeout=20)
    except Exception:
        return None
    out = {}
    for line in r.stdout.splitlines():
        low = line.lower()
        for key in ("sclk", "mclk"):
            if key in low and "mhz" in low and key not in out:
                tok = [t for t in line.replace("(", " ").replace(")", " ").split() if t.lower().endswith("mhz")]
                if tok:
                    out[key] = tok[0]
    return out or None


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "hybrid_prefill_decode_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(profile_txt, src_hash):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", profile_txt)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.split(":")[0].strip() in ("source_hash", "hbm_bytes_per_launch"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src_hash or "hbm_bytes_per_launch" not in vals:
        return None
    return float(vals["hbm_bytes_per_launch"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--compare-split", action="store_true",
                    help="time the workload's mixed batch and its prefill-only and decode-only "
                         "halves (cfg2..cfg5)")
    ap.add_argument("--attention", default="auto", choices=sorted(ATTN_MODES),
                    help="how prefill and decode attention are launched (auto = the library's "
                         "choice)")
    ap.add_argument("--workload", default="cfg5",
                    help="cfg1..cfg5, cfgN_prefill_only / cfgN_decode_only (the batch split), or "
                         "p1_16dec_8k (16 decodes at 8K context, Qwen3-14B-shaped)")
    ap.add_argument("--model-layers", type=int, default=0,
                    help="time a whole model iteration instead of one layer: embedding, this many "
                         "layers of the workload's shape (own weights and KV pools each), final "
                         "norm + LM head on each sequence's last row, greedy (hl_model_step)")
    ap.add_argument("--vocab", type=int, default=0,
                    help="vocabulary of --model-layers (default: 151936 for the Qwen3 shapes, "
                         "128256 for the 70B shape)")
    ap.add_argument("--serve", default=None, choices=["replay", "chunks", "cliff"],
                    help="serving experiments with the native scheduler driving hl_model_step: "
                         "replay = Poisson arrivals through the token-budget scheduler, step times "
                         "against the step-time model; chunks = one 8192-token prompt in chunks of "
                         "128..8192; cliff = prefill steps at chunk sizes around tile multiples")
    ap.add_argument("--rate", type=float, default=40.0,
                    help="--serve replay: request arrival rate (requests per second)")
    ap.add_argument("--requests", type=int, default=200, help="--serve replay: requests")
    ap.add_argument("--mean-output", type=int, default=64,
                    help="--serve replay: mean output length (tokens)")
    ap.add_argument("--budgets", type=int, nargs="+", default=[512, 2048, 8192],
                    help="--serve replay: token budgets to replay")
    ap.add_argument("--chunks", type=int, nargs="+", default=[4096, 2048, 1024, 512, 256, 128],
                    help="--serve chunks: chunk sizes to compare with the one-shot prefill")
    ap.add_argument("--kv-blocks", type=int, default=16384,
                    help="--serve replay: KV blocks per layer (16 tokens each)")
    ap.add_argument("--graph", action="store_true",
                    help="with --model-layers: capture the iteration in a HIP graph and time replays")
    ap.add_argument("--phase-reps", type=int, default=20)
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="steps timed one at a time after overwriting 1 GiB (evicts the 256 MB "
                         "last-level cache), reported next to the warm steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-step-events", action="store_true",
                    help="skip the phase-marked steps (the roofline then times the dominant "
                         "kernel's phase launched on its own)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU-baseline budget: whole prompt chunks, then decodes until spent")
    ap.add_argument("--only-phase", default=None,
                    help="profiling aid: after set-up run only this phase --phase-reps times "
                         "(qkv_rope_append, attention_lists, prefill_attention, "
                         "decode_attention, hybrid_attention, gemm_o, rms_scale_mlp, "
                         "gemm_gate_up, gemm_down, kv_export, kv_import) and print its timing")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="profiling aid: run a plain elementwise copy (read N MiB, write N MiB) "
                         "--phase-reps times, to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures the hybrid layer step on one GPU; the library has no multi-GPU "
              "path (sharding is described, not implemented). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from hybrid_prefill_decode_amd import binding as B
    from hybrid_prefill_decode_amd import kvcache

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = "cuda"
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 19  # bf16 elements in N MiB
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.phase_reps):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 2 * n, "bytes_written": 2 * n,
                          "reps": args.phase_reps}), flush=True)
        return
    name = args.workload
    if args.serve:
        return serve_bench(args, dev)
    if args.compare_split:
        return split_bench(args, dev)
    spec = workloads.named_spec(name)
    if args.model_layers > 0:
        return model_bench(args, spec, dev)
    s = spec.shape
    T = spec.num_tokens
    table, pool = workloads.block_table(spec)
    cfg = B.layer_cfg(s)
    batch = B.Batch(spec.q_start, spec.num_cached, table, dev, attention=ATTN_MODES[args.attention])
    x = workloads.hidden_states(spec, dev)
    w = workloads.weights(spec, dev)
    kp, vp = kvcache.alloc_pools(pool, s.n_kv_heads, s.head_dim, dev, fill=0.0)
    for si, (c, _) in enumerate(spec.seqs):
        if c:
            k, v = workloads.cached_kv(spec, si, dev)
            kvcache.write_positions(kp, vp, table[si], range(c), k, v)
    out = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=dev)
    ws = B.alloc_workspace(cfg, batch, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"{name}: inputs resident ({T} tokens, {spec.num_seqs} sequences, KV pools "
        f"{2 * kp.numel() * 2 / 1e9:.1f} GB)")

    def step(events=None):
        B.hybrid_layer_step(cfg, batch, x, w, kp, vp, out, ws, stream=stream, events=events)

    if args.only_phase is None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
    else:
        args.steps = 0
    # K timed steps back to back; an event after every step gives the per-step distribution.
    # The collector stays off meanwhile: a collection pause of the launching thread leaves the
    # GPU idle between steps once the queued work runs out.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    gc.enable()
    ms_step = evs[0].elapsed_time(evs[-1]) / max(args.steps, 1)
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    clocks = gpu_clocks() if args.only_phase is None else None
    if args.only_phase is None:
        log(f"{args.steps} timed steps: {ms_step:.4f} ms per step")

    # The same K steps again, back to back, each with the library's phase marks
    # (hl_batch_desc::events: events it records on the launch stream between its kernels), for
    # the mean time of every phase inside real steps. A mark costs a few microseconds of the
    # stream, so `value` comes from the unmarked steps above.
    step_phase_us = None
    if args.only_phase is None and not args.no_step_events and args.steps > 0:
        marks = [[torch.cuda.Event(enable_timing=True) for _ in range(B.HL_STEP_EVENTS)]
                 for _ in range(args.steps)]
        for m in marks:
            for e in m:
                e.record(stream)  # torch creates an event's handle at its first record
        torch.cuda.synchronize()
        gc.disable()
        for m in marks:
            step(m)
        torch.cuda.synchronize()
        gc.enable()
        step_phase_us = {
            name: sum(m[j].elapsed_time(m[j + 1]) for m in marks) * 1000.0 / len(marks)
            for j, name in enumerate(STEP_PHASES)}
        log(f"in-step phases: { {k: round(v, 1) for k, v in step_phase_us.items()} }")

    # cold steps: the last-level cache holds nothing of the previous step
    cold = []
    if args.only_phase is None and args.cold_reps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for _ in range(args.cold_reps):
            scratch.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            cold.append(a.elapsed_time(b))
        del scratch
        cold.sort()
        log(f"{len(cold)} cold steps done")

    # ---- per-phase timing through the phase entry points (same kernels as the step)
    qd = s.n_q_heads * s.head_dim
    h1 = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=dev)
    rs = torch.empty(T, dtype=torch.float32, device=dev)
    q_rot = torch.empty(T, qd, dtype=torch.bfloat16, device=dev)
    # the low half of the step's two-part decode query (its values do not change the work)
    q_lo = (torch.randn(T, qd, device=dev) * 1e-3).to(torch.bfloat16)
    attn = torch.empty(T, qd, dtype=torch.bfloat16, device=dev)
    h2 = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=dev)
    mlp = torch.empty(T, s.d_ff, dtype=torch.bfloat16, device=dev)
    # the step hands every projection its workspace (split-K, stream-K, the few-row path)
    gws = torch.empty(B.gemm_workspace_bytes(T, s.hidden, s.d_ff, B.HL_EPI_RESIDUAL),
                      dtype=torch.uint8, device=dev)
    has_pre = any(n > 1 for _, n in spec.seqs)
    has_dec = any(n == 1 for _, n in spec.seqs)
    plan = B.attention_plan(cfg, batch)
    lists = lambda: B.attention_build_lists(cfg, batch, kp, vp, ws, stream)
    run = lambda paths: (lambda: B.attention_run(cfg, batch, q_rot, kp, vp, attn, ws, q_lo=q_lo,
                                                 paths=paths, stream=stream))
    # each attention path alone as the library runs it when the two are launched separately
    # (HL_ATTN_SEPARATE: the decode and prefill work lists sized for their own launches, as for a
    # decode-only or prefill-only batch); the fused launch's lists are sized for the fused launch
    batch_sep = B.Batch(spec.q_start, spec.num_cached, table, dev, attention=B.HL_ATTN_SEPARATE)
    ws_sep = B.alloc_workspace(cfg, batch_sep, dev)
    plan_sep = B.attention_plan(cfg, batch_sep)
    lists_sep = lambda: B.attention_build_lists(cfg, batch_sep, kp, vp, ws_sep, stream)
    run_sep = lambda paths: (lambda: B.attention_run(cfg, batch_sep, q_rot, kp, vp, attn, ws_sep,
                                                     q_lo=q_lo, paths=paths, stream=stream))
    # (name, launch, set-up launched before each timed launch, outside its events)
    phases = [
        ("qkv_rope_append", lambda: B.qkv_rope_append(cfg, batch, x, w, q_rot, kp, vp, ws, stream),
         None),
        ("attention_lists", lists, None),
    ]
    if has_pre:
        phases.append(("prefill_attention", run_sep(B.ATTN_PREFILL), lists_sep))
    if has_dec:
        phases.append(("decode_attention", run_sep(B.ATTN_DECODE), lists_sep))
    if has_pre and has_dec:
        # both paths as the step runs them: one fused launch when the plan fuses, else two
        phases.append(("hybrid_attention", run(B.ATTN_BOTH), lists))
    phases += [
        ("gemm_o", lambda: B.gemm_bf16_nt(attn, w["w_o"], h2, x, B.HL_EPI_RESIDUAL,
                                          workspace=gws, stream=stream), None),
        ("rms_scale_mlp", lambda: B.rms_scale(h2, w["mlp_norm"], h1, rs, s.rms_eps, stream), None),
        ("gemm_gate_up", lambda: B.gemm_bf16_nt(h1, w["w_gate_up"], mlp, None, B.HL_EPI_SWIGLU,
                                                workspace=gws, stream=stream, row_scale=rs),
         None),
        ("gemm_down", lambda: B.gemm_bf16_nt(mlp, w["w_down"], out, h2, B.HL_EPI_RESIDUAL,
                                             workspace=gws, stream=stream), None),
    ]
    # KV hand-off of the longest request (not part of the step): its whole span of this layer
    # out to the [L, 2, T, Hkv, d] transfer layout, and back in under another table and pool
    sl = max(range(len(spec.seqs)), key=lambda i: spec.seqs[i][0] + spec.seqs[i][1])
    span_len = spec.seqs[sl][0] + spec.seqs[sl][1]
    npg = (span_len + 15) // 16
    row_a = np.ascontiguousarray(table[sl][:npg], dtype=np.int32)
    row_b = np.random.default_rng(7).permutation(npg).astype(np.int32)
    ta, tb = torch.from_numpy(row_a).to(dev), torch.from_numpy(row_b).to(dev)
    xfer = torch.empty(1, 2, span_len, s.n_kv_heads, s.head_dim, dtype=torch.bfloat16, device=dev)
    kp2, vp2 = kvcache.alloc_pools(npg, s.n_kv_heads, s.head_dim, dev, fill=0.0)
    phases += [
        ("kv_export", lambda: B.kv_export(kp, vp, ta, row_a, 0, span_len, 0, xfer, stream), None),
        ("kv_import", lambda: B.kv_import(xfer, tb, row_b, 0, span_len, 0, kp2, vp2, stream),
         None),
    ]
    if args.only_phase is not None:
        names = [p[0] for p in phases]
        if args.only_phase not in names:
            raise SystemExit(f"no phase {args.only_phase} in this workload")
        # the phases before it run once, untimed, so that it reads the data a step gives it
        # (the rotated queries, the attention rows, the MLP activations)
        at = names.index(args.only_phase)
        for _, fn, pre in phases[:at]:
            if pre is not None:
                pre()
            fn()
        torch.cuda.synchronize()
        phases = [phases[at]]
    phase_us = {}
    for pname, fn, pre in phases:
        if pre is not None:
            pre()
        fn()
        torch.cuda.synchronize()
        # each timed launch bracketed by its own events, its set-up (if any) outside them; a GPU
        # spin before each one keeps the GPU busy while the host validates and enqueues it (the
        # block-table checks of the 70B-shaped batch take about 0.2 ms of host time), so the
        # events bracket the launch's kernels and no idle gap
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.phase_reps)]
        for a, b in evs:
            if pre is not None:
                pre()
            torch.cuda._sleep(SPIN_CYCLES)
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        total_ms = sum(a.elapsed_time(b) for a, b in evs)
        phase_us[pname] = 1000.0 * total_ms / args.phase_reps
        log(f"phase {pname}: {phase_us[pname]:.2f} us")
    if args.only_phase is not None:
        print(json.dumps({"only_phase": args.only_phase, "workload": name,
                          "reps": args.phase_reps, "avg_us": round(phase_us[args.only_phase], 2)}),
              flush=True)
        return

    # one traced fused launch: how the two paths shared the GPU (decode rate while prefill ran)
    trace_metrics = None
    if plan["fused"] and has_pre and has_dec:
        items = plan["prefill_parts"] * s.n_q_heads + plan["decode_units"] * s.n_kv_heads
        trace = torch.zeros(3 * items, dtype=torch.int64, device=dev)
        lists()
        torch.cuda._sleep(SPIN_CYCLES)
        B.attention_run_traced(cfg, batch, q_rot, kp, vp, attn, ws, trace, q_lo=q_lo,
                               paths=B.ATTN_BOTH, stream=stream)
        torch.cuda.synchronize()
        trace_metrics = fused_trace_metrics(spec, plan, trace.view(items, 3).cpu().numpy(),
                                            B.trace_clock_khz())
        if dec_gbps_alone := (algorithmic_counts(spec)["decode_kv_bytes"] /
                              (phase_us["decode_attention"] * 1e-6) / 1e9):
            trace_metrics["decode_alone_gbps"] = round(dec_gbps_alone, 1)
            trace_metrics["decode_in_prefill_window_over_alone"] = (
                round(trace_metrics["decode_gbps_in_prefill_window"] / dec_gbps_alone, 4)
                if trace_metrics["decode_gbps_in_prefill_window"] else None)
        log(f"fused trace: {trace_metrics}")

    cnt = algorithmic_counts(spec)
    # the QKV projection phase also holds its prep pass and the RoPE / append epilogue
    gemm_us = sum(phase_us[k] for k in ("qkv_rope_append", "gemm_o", "gemm_gate_up", "gemm_down"))
    gemm_tflops = sum(cnt["gemm_flops"].values()) / (gemm_us * 1e-6) / 1e12
    dec_gbps = (cnt["decode_kv_bytes"] / (phase_us["decode_attention"] * 1e-6) / 1e9
                if has_dec else None)
    pre_tflops = (cnt["prefill_attn_flops"] / (phase_us["prefill_attention"] * 1e-6) / 1e12
                  if has_pre else None)

    # the dominant kernel of the step and its roofline, its duration the mean inside the
    # phase-marked steps (with --no-step-events, the phase launched on its own)
    gu_flops = cnt["gemm_flops"]["gate_up"]
    gu_tflops = gu_flops / (phase_us["gemm_gate_up"] * 1e-6) / 1e12
    in_step = step_phase_us or {}
    timed_in = "phase-marked steps" if in_step else "own launches"
    gu_us = in_step.get("gemm_gate_up", phase_us["gemm_gate_up"])
    fused_alone = phase_us.get("hybrid_attention") if plan["fused"] else None
    fused_us = in_step.get("attention", fused_alone) if plan["fused"] else None
    if fused_us is not None and fused_us > gu_us:
        att_bytes = cnt["decode_attn_bytes"] + cnt["prefill_attn_bytes"]
        gbps = att_bytes / (fused_us * 1e-6) / 1e9
        src_hash = kernel_source_hash(["attention_hybrid.hip", "attn_prefill_core.h",
                                       "attn_decode_core.h", "attention_decode.hip", "common.h"])
        # the launch's bound is the larger of its two roofline terms: bytes at the HBM peak or
        # prefill flops at the matrix-core peak (decode-heavy batches: bytes; long prompt chunks:
        # flops), and `frac` is taken against that one
        tflops = cnt["prefill_attn_flops"] / (fused_us * 1e-6) / 1e12
        by_flops = cnt["prefill_attn_flops"] / PEAK_BF16_TFLOPS > att_bytes / PEAK_HBM_GBPS * 1e3
        roofline = {
            "kernel": "hybrid_attn_kernel (fused prefill + decode attention) and the decode "
                      "merge behind it: one hl_attention_run",
            **({"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "hbm_gbps": round(gbps, 1)} if by_flops else
               {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4)}),
            "traffic": read_traffic(f"hybrid_attention_{name}_pmc.txt", src_hash),
            "algorithmic_bytes_per_launch": att_bytes,
            "mfma_flops_per_launch": cnt["prefill_attn_flops"],
            "mfma_frac": round(cnt["prefill_attn_flops"] / (fused_us * 1e-6) / 1e12
                               / PEAK_BF16_TFLOPS, 4),
            "avg_launch_us": round(fused_us, 2),
            "avg_launch_us_alone": round(fused_alone, 2),
            "timed_in": timed_in,
        }
    else:
        src_hash = kernel_source_hash(["gemm.hip", "gemm_core.h", "gemm_swiglu.hip", "common.h"])
        roofline = {
            "kernel": "gemm_bf16_nt<SwiGLU> (gate/up projection)",
            "bound": "mfma", "achieved": round(gu_flops / (gu_us * 1e-6) / 1e12, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gu_flops / (gu_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": read_traffic(f"gemm_gate_up_{name}_pmc.txt", src_hash),
            "algorithmic_flops_per_launch": gu_flops,
            "avg_launch_us": round(gu_us, 2),
            "avg_launch_us_alone": round(phase_us["gemm_gate_up"], 2),
            "timed_in": timed_in,
        }
    roofline["source_hash"] = src_hash

    result = {
        "metric": "hybrid layer-step tokens/s; GEMM MFMA util % + decode-attn HBM GB/s vs peak",
        "value": round(T / (ms_step / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": pct(per_step),
        "cold_step_ms": pct(cold) if cold else None,
        "gpu_clocks_after_timed_steps": clocks,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and cached K/V, N(0,0.02^2) weights; random block table)",
        "config": {**workloads.describe(spec), "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "attention_plan": plan,
        "attention_plan_separate": plan_sep,
        "phases_us": {k: round(v, 2) for k, v in phase_us.items()},
        "step_phases_us": ({k: round(v, 2) for k, v in step_phase_us.items()}
                           if step_phase_us else None),
        "fused_attention_trace": trace_metrics,
        "gemm_mfma_util": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
        "gemm_tflops": round(gemm_tflops, 1),
        # the same four projections timed inside the phase-marked steps (their weights cold, the
        # first norm pass and the work lists in the QKV phase)
        "gemm_mfma_util_in_step": (round(sum(cnt["gemm_flops"].values()) / (sum(
            step_phase_us[k] for k in ("qkv_rope_append", "gemm_o", "gemm_gate_up", "gemm_down"))
            * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4) if step_phase_us else None),
        "gate_up_tflops": round(gu_tflops, 1),
        # decode attention alone (the step's two-part query; the separate path's work lists,
        # prebuilt)
        "decode_attn_hbm_gbps": None if dec_gbps is None else round(dec_gbps, 1),
        "decode_attn_hbm_frac": None if dec_gbps is None else round(dec_gbps / PEAK_HBM_GBPS, 4),
        "prefill_attn_tflops": None if pre_tflops is None else round(pre_tflops, 1),
        # weight bytes of the four projections over their phase time (phases repeat one layer, so
        # part of the weights may be served by the last-level cache)
        "gemm_weight_gbps": round(cnt["weight_bytes"] / (gemm_us * 1e-6) / 1e9, 1),
        "kv_transfer": {
            "tokens": span_len, "bytes_per_layer_slice": 2 * xfer.numel(),
            "export_gbps": round(2 * 2 * xfer.numel() / (phase_us["kv_export"] * 1e-6) / 1e9, 1),
            "import_gbps": round(2 * 2 * xfer.numel() / (phase_us["kv_import"] * 1e-6) / 1e9, 1),
            "note": "one layer slice of the longest request; GB/s counts bytes read + written",
        },
        "wall_s_timed": round(t_wall, 3),
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        del kp2, vp2, xfer
        result["cpu_baseline"] = cpu_baseline(spec, x, w, dev, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _union_us(iv):
    """Total length of the union of [start, end) intervals (sorted merge)."""
    total, cur_s, cur_e = 0.0, None, None
    for a, b in sorted(iv):
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                total += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    if cur_e is not None:
        total += cur_e - cur_s
    return total


def fused_trace_metrics(spec, plan, rec, khz):
    """How prefill and decode shared one fused attention launch, from its work-item trace
    (rec [items, 3] int64: start, end, workgroup; prefill items first). Decode bytes per item:
    the K and V of its pages' tokens for one KV head."""
    import numpy as np
    s = spec.shape
    n_pre = plan["prefill_parts"] * s.n_q_heads
    sp = plan["split_pages"]
    dec_bytes = []
    for c, n in spec.seqs:
        if n != 1:
            continue
        kv = c + 1
        pages = (kv + 15) // 16
        for u in range((pages + sp - 1) // sp):
            toks = min((u + 1) * sp * 16, kv) - u * sp * 16
            dec_bytes += [toks * s.head_dim * 2 * 2] * s.n_kv_heads
    dec_bytes = np.array(dec_bytes, dtype=np.float64)
    us = (rec[:, :2].astype(np.float64) - float(rec[:, 0].min())) * 1000.0 / khz
    pre, dec = us[:n_pre], us[n_pre:]
    assert dec.shape[0] == dec_bytes.shape[0], (dec.shape, dec_bytes.shape)
    span = float(us[:, 1].max())
    dec_active = _union_us(map(tuple, dec))
    pre_active = _union_us(map(tuple, pre)) if n_pre else 0.0
    win = float(pre[:, 1].max()) if n_pre else 0.0
    # decode bytes moved while prefill items still ran: each item's bytes prorated by the part of
    # its interval inside [0, win)
    frac = np.clip((np.minimum(dec[:, 1], win) - dec[:, 0]) / np.maximum(dec[:, 1] - dec[:, 0], 1e-9),
                   0.0, 1.0)
    in_win = float((dec_bytes * frac).sum())
    workers_pre = len(set(rec[:n_pre, 2].tolist())) if n_pre else 0
    return {
        "span_us": round(span, 1),
        "prefill_active_us": round(pre_active, 1),
        "decode_active_us": round(dec_active, 1),
        "decode_gbps_over_decode_active": round(dec_bytes.sum() / (dec_active * 1e-6) / 1e9, 1),
        "prefill_window_us": round(win, 1),
        "decode_gbps_in_prefill_window": round(in_win / (win * 1e-6) / 1e9, 1) if win > 0 else None,
        "decode_gbps_after_prefill": round((dec_bytes.sum() - in_win) / ((span - win) * 1e-6) / 1e9, 1)
                                     if span > win else None,
        "workgroups_running_prefill": workers_pre,
        "items": [n_pre, int(dec.shape[0])],
        "clock_khz": khz,
    }


def model_bench(args, spec, dev):
    """Whole-model iteration (hl_model_step) on the workload's batch: tokens/s and ms per step."""
    import numpy as np
    import torch

    import workloads
    from hybrid_prefill_decode_amd import binding as B
    from hybrid_prefill_decode_amd import kvcache

    s = spec.shape
    L = args.model_layers
    vocab = args.vocab or (128256 if s.hidden == 8192 else 151936)
    table, pool = workloads.block_table(spec)
    cfg = B.layer_cfg(s)
    batch = B.Batch(spec.q_start, spec.num_cached, table, dev, attention=ATTN_MODES[args.attention])
    # every layer has its own weights; the cached K/V of layer 0 is copied into every layer's
    # own pools (distinct memory, same values: the values do not change the work)
    kp0, vp0 = kvcache.alloc_pools(pool, s.n_kv_heads, s.head_dim, dev, fill=0.0)
    for si, (c, _) in enumerate(spec.seqs):
        if c:
            k, v = workloads.cached_kv(spec, si, dev)
            kvcache.write_positions(kp0, vp0, table[si], range(c), k, v)
    layers, pools = [], []
    for l in range(L):
        layers.append(workloads.weights(workloads.layer_spec(spec, l), dev))
        pools.append((kp0.clone(), vp0.clone()) if l else (kp0, vp0))
    t = workloads.model_tensors(spec, vocab, dev)
    model = B.ModelHandle(layers, pools, t["embed"], t["final_norm"], t["lm_head"])
    tokens = torch.from_numpy(t["tokens"]).to(dev)
    logits = torch.empty(spec.num_seqs, vocab, dtype=torch.bfloat16, device=dev)
    nxt = torch.empty(spec.num_seqs, dtype=torch.int32, device=dev)
    ws = B.alloc_model_workspace(cfg, batch, model, dev)
    stream = torch.cuda.current_stream()

    def step(st=None):
        B.model_step(cfg, batch, model, tokens, t["tokens"], logits, nxt, ws,
                     stream=st if st is not None else stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            step(gs)
        run = g.replay
        run()
        torch.cuda.synchronize()
    steps = max(args.steps // 5, 5)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    T = spec.num_tokens
    print(json.dumps({
        "metric": "model iteration tokens/s (embedding + layers + LM head + greedy)",
        "value": round(T / (ms / 1000.0), 1), "unit": "tokens/s", "n_gpus": 1,
        "ms_per_step": round(ms, 3), "step_ms": pct(per), "steps": steps, "warmup": args.warmup,
        "layers": L, "vocab": vocab, "graph": bool(args.graph), "dtype": "bf16",
        "data": "synthetic (seeded; random-init weights of the workload's layer shape)",
        "config": {**workloads.describe(spec), "parallelism": "none (1 GPU)"},
    }), flush=True)


def split_bench(args, dev):
    """The workload's mixed batch against the same data split into a prefill-only and a
    decode-only step (median step times, same process): what batching the decodes into the
    prefill's linear layers costs ("Chunked prefill (stall-free batching), explained", "The
    bottleneck: prefill-decode interference")."""
    import torch

    import workloads
    from hybrid_prefill_decode_amd import binding as B
    from hybrid_prefill_decode_amd import kvcache
    cfg_id = int(args.workload[3:].split("_")[0])
    res = {}
    for variant in ("mixed", "prefill_only", "decode_only"):
        spec = workloads.make_spec(cfg_id, variant)
        s = spec.shape
        table, pool = workloads.block_table(spec)
        cfg = B.layer_cfg(s)
        batch = B.Batch(spec.q_start, spec.num_cached, table, dev)
        x = workloads.hidden_states(spec, dev)
        w = workloads.weights(spec, dev)
        kp, vp = kvcache.alloc_pools(pool, s.n_kv_heads, s.head_dim, dev, fill=0.0)
        for si, (c, _) in enumerate(spec.seqs):
            if c:
                k, v = workloads.cached_kv(spec, si, dev)
                kvcache.write_positions(kp, vp, table[si], range(c), k, v)
        out = torch.empty(spec.num_tokens, s.hidden, dtype=torch.bfloat16, device=dev)
        ws = B.alloc_workspace(cfg, batch, dev)
        step = lambda: B.hybrid_layer_step(cfg, batch, x, w, kp, vp, out, ws)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record()
        for i in range(args.steps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        res[variant] = pct(sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)))
        print(f"# {variant}: {res[variant]}", file=sys.stderr, flush=True)
        del kp, vp, w, x, out, ws
        torch.cuda.empty_cache()
    mixed = res["mixed"]["median"]
    split = res["prefill_only"]["median"] + res["decode_only"]["median"]
    print(json.dumps({
        "experiment": "mixed_vs_split", "workload": args.workload,
        "step_ms": res, "mixed_ms": mixed, "prefill_plus_decode_ms": round(split, 4),
        "mixed_over_split": round(mixed / split, 4),
        "decode_alone_ms": res["decode_only"]["median"],
        "extra_for_decodes_in_mixed_ms": round(mixed - res["prefill_only"]["median"], 4),
        "data": "synthetic (seeded), the workload's batch and its two halves",
    }), flush=True)


def serve_bench(args, dev):
    """Serving experiments with the native scheduler driving hl_model_step; one JSON line each.
    Random-init weights of the Qwen3-8B layer shape, synthetic requests."""
    import numpy as np
    import torch

    import workloads
    from hybrid_prefill_decode_amd import binding as B
    from hybrid_prefill_decode_amd import serving as SV

    shape = workloads.SHAPES["qwen3_8b"]
    vocab = args.vocab or 151936

    def qs(v, p):
        return round(float(np.percentile(v, p)), 2) if len(v) else None

    if args.serve == "replay":
        L = args.model_layers or 8
        rng = np.random.default_rng(11)
        n_req = args.requests
        # Poisson arrivals, lognormal prompt lengths (mean 1000, at most 8192) and output lengths
        # (mean 250 on the page; --mean-output shortens them to bound the run time)
        sig = 1.0
        prompts = np.clip(rng.lognormal(np.log(1000) - sig * sig / 2, sig, n_req), 16, 8192)
        outs = np.clip(rng.lognormal(np.log(args.mean_output) - sig * sig / 2, sig, n_req), 1,
                       4 * args.mean_output)
        prompts, outs = prompts.astype(int), outs.astype(int)
        arrive = np.cumsum(rng.exponential(1000.0 / args.rate, n_req))  # ms
        mbs = (8192 + 4 * args.mean_output + 15) // 16 + 1
        eng = SV.Engine(shape, **workloads.engine_model(shape, L, vocab, args.kv_blocks, dev),
                        max_blocks_per_seq=mbs, device=dev, budget=args.budgets[0], max_seqs=256)
        kw = dict(layer_params=L * shape.weight_params, head_params=vocab * shape.hidden,
                  hidden=shape.hidden, layers=L,
                  kv_bytes_per_token=2 * L * shape.n_kv_heads * shape.head_dim * 2)
        for budget in args.budgets:
            eng.reset(budget=budget, max_seqs=256)
            clock, k, recs = 0.0, 0, []
            first, last, itl = {}, {}, []
            wall = time.perf_counter()
            while True:
                while k < n_req and arrive[k] <= clock:
                    eng.submit(k, int(prompts[k]), int(outs[k]))
                    k += 1
                r = eng.step()
                if r is None:
                    if k == n_req:
                        break
                    clock = float(arrive[k])
                    continue
                clock += r.ms
                recs.append(r)
                if len(recs) % 500 == 0:
                    print(f"# budget {budget}: {len(recs)} iterations, {k} arrived, "
                          f"clock {clock:.0f} ms", file=sys.stderr, flush=True)
                for rid in r.emitted:
                    if rid in last:
                        itl.append(clock - last[rid])
                    else:
                        first[rid] = clock - arrive[rid]
                    last[rid] = clock
            ms = np.array([r.ms for r in recs])
            fit_o = SV.fit_step_model(recs, overlap=True, **kw)
            fit_p = SV.fit_step_model(recs, overlap=False, **kw)
            emitted = sum(len(r.emitted) for r in recs)
            print(json.dumps({
                "experiment": "serve_replay", "layers": L, "budget": budget, "requests": n_req,
                "arrival_rate_per_s": args.rate, "mean_output": args.mean_output,
                "iterations": len(recs), "gpu_busy_s": round(float(ms.sum()) / 1e3, 3),
                "span_s": round(clock / 1e3, 3),
                "output_tokens_per_s": round(emitted / (clock / 1e3), 1),
                "step_ms": {"p50": qs(ms, 50), "p99": qs(ms, 99), "max": qs(ms, 100)},
                "ttft_ms": {"p50": qs(list(first.values()), 50),
                            "p99": qs(list(first.values()), 99)},
                "itl_ms": {"p50": qs(itl, 50), "p99": qs(itl, 99), "max": qs(itl, 100)},
                "step_model_fit_overlap": fit_o, "step_model_fit_serial": fit_p,
                "wall_s": round(time.perf_counter() - wall, 1),
                "data": "synthetic: Poisson arrivals, lognormal lengths, random-init weights",
            }), flush=True)
        return

    if args.serve == "chunks":
        L = args.model_layers or 36
        prompt = 8192
        eng = SV.Engine(shape, **workloads.engine_model(shape, L, vocab, prompt // 16 + 8, dev),
                        max_blocks_per_seq=prompt // 16 + 2, device=dev, budget=prompt,
                        max_seqs=4)
        res = {}
        for chunk in [prompt] + [c for c in args.chunks if c != prompt]:
            for rep in range(2):  # the first pass loads this chunk size's kernels
                eng.reset(budget=chunk, max_seqs=4)
                eng.submit(0, prompt, 1)
                recs = []
                while True:
                    r = eng.step()
                    if r is None:
                        break
                    recs.append(r)
            res[chunk] = recs
            print(f"# chunk {chunk}: {len(recs)} iterations, {sum(r.ms for r in recs):.2f} ms",
                  file=sys.stderr, flush=True)
        one = sum(r.ms for r in res[prompt])
        total = {c: sum(r.ms for r in v) for c, v in res.items()}
        print(json.dumps({
            "experiment": "chunked_prefill_overhead", "layers": L, "prompt": prompt,
            "total_ms": {str(c): round(t, 2) for c, t in total.items()},
            "iterations": {str(c): len(v) for c, v in res.items()},
            "overhead_vs_one_shot": {str(c): round(t / one - 1.0, 4) for c, t in total.items()},
            "data": "one synthetic prompt, random-init weights of the Qwen3-8B shape",
        }), flush=True)
        return

    # cliff: one prompt chunk at prefix 0 for sizes at and just past tile multiples, whole model
    # iteration, and the gate/up GEMM alone with the per-launch tile choice vs a fixed 256x256 tile
    L = args.model_layers or 36
    eng = SV.Engine(shape, **workloads.engine_model(shape, L, vocab, 160, dev),
                    max_blocks_per_seq=140, device=dev,
                    budget=4096, max_seqs=1)
    sizes = (256, 257, 512, 513, 1024, 1025, 2048, 2049)

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))[reps // 2]

    step, g_choice, g_fixed, choice = {}, {}, {}, {}
    w = eng.layer_w[0]["w_gate_up"]
    for c in sizes:
        table = np.arange(140, dtype=np.int32)[None, :]
        batch = B.Batch(np.array([0, c], np.int32), np.array([0], np.int32), table, dev)
        toks = (np.arange(c) * 7919 % vocab).astype(np.int32)
        tk = torch.from_numpy(toks).to(dev)
        ws = B.alloc_model_workspace(eng.cfg, batch, eng.model, dev)
        step[c] = timed(lambda: B.model_step(eng.cfg, batch, eng.model, tk, toks,
                                             eng.logits[:1], eng.next[:1], ws))
        a = torch.randn(c, shape.hidden, device=dev).to(torch.bfloat16)
        out = torch.empty(c, w.shape[0], dtype=torch.bfloat16, device=dev)
        gws = torch.empty(B.gemm_workspace_bytes(c, w.shape[0], shape.hidden), dtype=torch.uint8,
                          device=dev)
        g_choice[c] = timed(lambda: B.gemm_bf16_nt(a, w, out, workspace=gws))
        g_fixed[c] = timed(lambda: B.gemm_bf16_nt_tiled(a, w, out, 256, 256))
        choice[c] = B.gemm_tile_choice(c, w.shape[0], shape.hidden)
        print(f"# cliff {c}: step {step[c]:.3f} ms, gate/up {g_choice[c]:.4f} ms "
              f"(fixed 256x256 {g_fixed[c]:.4f} ms)", file=sys.stderr, flush=True)
    ratio = lambda d: {f"{c + 1}/{c}": round(d[c + 1] / d[c], 4) for c in sizes[::2]}
    print(json.dumps({
        "experiment": "tile_quantisation_cliff", "layers": L,
        "model_step_ms": {str(c): round(v, 3) for c, v in step.items()},
        "model_step_ratio": ratio(step),
        "gate_up_gemm_ms": {str(c): round(v, 4) for c, v in g_choice.items()},
        "gate_up_gemm_ratio": ratio(g_choice),
        "gate_up_tile_choice": {str(c): list(v) if isinstance(v, tuple) else v
                                for c, v in choice.items()},
        "gate_up_fixed_256x256_ms": {str(c): round(v, 4) for c, v in g_fixed.items()},
        "gate_up_fixed_256x256_ratio": ratio(g_fixed),
        "data": "one synthetic prompt chunk, random-init weights of the Qwen3-8B shape",
    }), flush=True)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(spec, x, w, dev, budget_s):
    """The fp64 oracle on the host cores over a bounded sample of the same batch.

    Inputs reach the host as bf16 (the copy from the device is not the oracle's work); the clock
    covers the bf16 -> fp64 upcasts and the oracle. Sample: every prompt chunk whole (its cached
    prefix streamed in with it), then decodes one request at a time in a seeded random order
    until the budget is spent (at least 4). The batch time is estimated as the weight upcast +
    the prompt chunks + the mean decode time x the batch's decode count; value = batch tokens /
    that estimate."""
    import numpy as np
    import torch

    import oracle.layer as OL
    import workloads

    s = spec.shape
    x_h = x.cpu()
    w_h = {k: v.cpu() for k, v in w.items()}
    up = lambda t: t.to(torch.float64).numpy()
    t0 = time.perf_counter()
    xh = up(x_h)
    wh = {k: up(v) for k, v in w_h.items()}
    t_upcast = time.perf_counter() - t0
    pre = [i for i, (c, n) in enumerate(spec.seqs) if n > 1]
    dec = [i for i, (c, n) in enumerate(spec.seqs) if n == 1]
    order = list(np.random.default_rng(spec.seed).permutation(dec)) if dec else []

    def one(si):
        c, n = spec.seqs[si]
        k, v = workloads.cached_kv(spec, si, dev)
        k, v = k.cpu(), v.cpu()
        r0 = int(spec.q_start[si])
        t = time.perf_counter()
        OL.sequence_step(s, xh[r0:r0 + n], wh, c, up(k), up(v))
        return time.perf_counter() - t

    log(f"cpu baseline: weights upcast in {t_upcast:.1f} s")
    t_pre = sum(one(si) for si in pre)
    log(f"cpu baseline: {len(pre)} prompt chunk(s) in {t_pre:.1f} s")
    t_dec = []
    spent = t_upcast + t_pre
    for si in order:
        if len(t_dec) >= 4 and spent >= budget_s:
            break
        t_dec.append(one(int(si)))
        spent += t_dec[-1]
    log(f"cpu baseline: {len(t_dec)} decodes in {sum(t_dec):.1f} s")
    est = t_upcast + t_pre + (float(np.mean(t_dec)) * len(dec) if dec else 0.0)
    cores = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            cores = max(blas)
    except Exception:
        pass
    return {"value": round(spec.num_tokens / est, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": _cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{spec.name}: every prompt chunk whole ({len(pre)}, {t_pre:.1f} s) and "
                      f"{len(t_dec)} of {len(dec)} decodes (seeded random order, mean "
                      f"{(np.mean(t_dec) if t_dec else 0):.3f} s each), weight upcast "
                      f"{t_upcast:.1f} s; batch estimate {est:.1f} s for {spec.num_tokens} "
                      f"tokens; fp64 numpy, bf16 -> fp64 upcasts inside the clock, cached K/V "
                      f"streamed one request at a time",
            "measured_s": round(spent, 2)}


if __name__ == "__main__":
    main()
