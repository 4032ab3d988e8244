"""Decoder token-steps/s of the recurrent decoder step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload refdepth]

Default workload: the reference-depth model (48 layers, d = 2048, 16 heads,
FFN 8192, window 512, one shared memory group, V = 32768, bf16) on 32
sequences: 2048 prompt tokens through rlt_run_sequence, then 512 single
rlt_decoder_step calls on the same state (no reset at the split).  A "step" is
one decoder step over the whole batch; --steps K times the first K steps of
that run (default: all 2560).  Inputs are synthetic (seeded, drawn on the GPU)
and resident in HBM before timing starts; logits of every step are written.

Printed: one JSON line with the throughput, the roofline figure of the
dominant kernel (cross-attention over the encoder memory), measured with HIP
events inside the timed region on the launch stream, and the CPU oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
KERNEL_SOURCE = os.path.join(ROOT, "recurrent_decode_step_amd", "csrc", "rlt_kernels.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k_attn_cross_refdepth_b32_counters.md")


def source_sha256(path=KERNEL_SOURCE):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(path=COUNTERS_FILE):
    """HBM bytes per launch of the cross-attention kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration), or None when the summary is missing or was taken on another
    version of the kernel source."""
    try:
        kv = {}
        for line in open(path):
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                kv[k.strip().strip("`")] = v.strip().strip("`")
        if kv.get("kernel_source_sha256") != source_sha256():
            return None
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def calibration_copy(dev, mib=256):
    """One plain streaming kernel of known size (reads and writes `mib` MiB),
    so hardware byte counters can be scaled against it."""
    import torch
    a = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def algorithmic_bytes_per_step(cfg, positions, es):
    """Bytes one decoder step must move: every weight once, the window cache
    (min(t, W) entries read incl. the new one), encoder memory 1..t per layer,
    e in, s in/out, logits out."""
    d, F, L, V, W = cfg.d_model, cfg.d_ffn, cfg.n_layers, cfg.vocab, cfg.window
    weights = es * (L * (6 * d * d + 2 * d * F + 3 * d) + 2 * d * d + d + V * d + 2 * d)
    swa = sum(L * 2 * d * es * min(t, W) for t in positions)
    mem = sum(L * 2 * d * es * t for t in positions)
    io = len(positions) * (d * es + 8 * d + 4 * V)
    return weights + swa + mem + io


def gemm_flops_per_step(cfg, n):
    d, F, L, V = cfg.d_model, cfg.d_ffn, cfg.n_layers, cfg.vocab
    return 2.0 * n * (L * (6 * d * d + 2 * d * F) + 2 * d * d + V * d)


def openblas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("internal_api") in
             ("openblas", "mkl", "blis")]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, params_gpu, e_gpu, mk_gpu, mv_gpu, budget_s=15.0, max_steps=64):
    """The oracle (fp32 NumPy, as it stands) on the host: the first steps of the
    same run, all sequences batched, until the time budget is spent."""
    import torch
    import oracle
    t_prep = time.time()
    params = {k: v.float().cpu() for k, v in params_gpu.items()}
    B = e_gpu.shape[0]
    om = oracle.Model(params=params, precision="fp32", d_model=cfg.d_model, n_heads=cfg.n_heads,
                      n_layers=cfg.n_layers, d_ffn=cfg.d_ffn, window=cfg.window,
                      mem_groups=cfg.mem_groups, vocab=cfg.vocab, rms_eps=cfg.rms_eps)
    del params
    steps_cap = max_steps
    e = e_gpu[:, :steps_cap].float().cpu()
    mk = mk_gpu[:, :, :, :steps_cap].float().cpu()
    mv = mv_gpu[:, :, :, :steps_cap].float().cpu()
    prep = time.time() - t_prep
    states = [oracle.initial_state(om) for _ in range(B)]
    t0 = time.time()
    done = 0
    while done < steps_cap:
        oracle.decoder_step(om, states, e[:, done], mk, mv)
        done += 1
        if time.time() - t0 >= budget_s and done >= 2:
            break
    el = time.time() - t0
    return {"value": B * done / el, "unit": "token-steps/s", "cores": openblas_threads(),
            "kind": "oracle",
            "sample": f"{B} sequences x the first {done} steps (t = 1..{done}) of the same run, "
                      f"NumPy fp32 oracle, weights read once per step for the batch "
                      f"({el:.1f} s timed, {prep:.1f} s input transfer untimed)"}


def run_refdepth(args):
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH

    wl = REFDEPTH
    cfg = wl.model
    B, T_total, prompt = wl.batch, wl.steps, wl.prompt
    K = T_total if args.steps is None else args.steps
    if not 1 <= K <= T_total:
        raise SystemExit(f"--steps must be in [1, {T_total}]")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    es = 2
    t_setup = time.time()
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, T_total, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T_total, device=dev)
    mem = binding.memory_view(mk, mv)
    e_by_step = e.transpose(0, 1).contiguous()       # [T][B][d]: one contiguous block per step
    state = binding.State(model, B, T_total)
    n_pre = min(K, prompt)
    logits_pre = torch.empty((B, n_pre, cfg.vocab), dtype=torch.float32, device=dev)
    logits_step = torch.empty((max(K - prompt, 1), B, cfg.vocab), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    if args.calibrate_copy:
        calibration_copy(dev)

    # warmup: W steps from H_0, then every slot back to H_0 (untimed)
    if args.warmup > 0:
        binding.rlt_run_sequence(model, state, e[:, :args.warmup], mem,
                                 logits_mode=binding.RLT_LOGITS_ALL)
        binding.rlt_state_reset(model, state, list(range(B)))
    torch.cuda.synchronize()

    stride = max(1, K // 64)
    classes = (binding.RLT_K_SETUP, binding.RLT_K_GEMM, binding.RLT_K_SWA, binding.RLT_K_CROSS)
    mask = (1 << binding.RLT_K_CROSS) if not args.breakdown else sum(1 << c for c in classes)
    binding.profile_begin(state, mask, 1 << 22, step_stride=stride)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    binding.rlt_run_sequence(model, state, e[:, :n_pre], mem, logits_mode=binding.RLT_LOGITS_ALL,
                             logits=logits_pre)
    if args.progress:
        print(f"prompt of {n_pre} steps enqueued", file=sys.stderr, flush=True)
    for j in range(prompt, K):
        binding.rlt_decoder_step(model, state, e_by_step[j], mem, logits=logits_step[j - prompt])
        if args.progress and (j + 1) % 128 == 0:
            print(f"step {j + 1} enqueued", file=sys.stderr, flush=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    prof = {c: binding.profile_collect(state, c) for c in classes}
    cross_ms, cross_n, cross_bytes = prof[binding.RLT_K_CROSS]
    binding.profile_begin(state, 0, 0)
    assert all(state.position(b) == K for b in range(B))
    if not torch.isfinite(logits_pre).all():
        raise RuntimeError("non-finite logits")

    positions_per_step = [[k + 1] * B for k in range(K)]
    bytes_run = sum(algorithmic_bytes_per_step(cfg, p, es) for p in positions_per_step)
    value = B * K / (ms / 1e3)
    cross_avg_ms = cross_ms / max(cross_n, 1)
    achieved = cross_bytes / max(cross_n, 1) / (cross_avg_ms / 1e3) / 1e9
    traffic = measured_traffic() if K == T_total else None
    out = {
        "metric": "decoder token-steps/sec at 1 GPU (48-layer, B=32/256); % HBM/MFMA roofline",
        "value": round(value, 2),
        "unit": "token-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "prompt": min(prompt, K),
                   "decode_steps": max(K - prompt, 0), "positions": f"1..{K}",
                   "logits": "every step, fp32"},
        "roofline": {"bound": "hbm", "kernel": "k_attn<bf16,128,1> (cross-attention, encoder memory)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes_per_launch": round(cross_bytes / max(cross_n, 1)),
                     "launches_timed": cross_n, "avg_launch_us": round(cross_avg_ms * 1e3, 2)},
        "step_roofline": {"bound": "hbm", "algorithmic_GB_per_step": round(bytes_run / K / 1e9, 3),
                          "achieved": round(bytes_run / (ms / 1e3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(bytes_run / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "setup_s": round(setup_s, 1),
    }
    if args.breakdown:
        names = {binding.RLT_K_SETUP: "setup", binding.RLT_K_GEMM: "gemm",
                 binding.RLT_K_SWA: "window_attention", binding.RLT_K_CROSS: "cross_attention"}
        n_prof_steps = len(range(0, K, stride))
        out["breakdown_ms_per_step"] = {
            names[c]: round(prof[c][0] / max(n_prof_steps, 1), 4) for c in classes}
        out["breakdown_GBps"] = {
            names[c]: round(prof[c][2] / (prof[c][0] / 1e3) / 1e9, 1) if prof[c][0] else None
            for c in classes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, e, mk, mv, budget_s=args.cpu_budget)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="refdepth", choices=["refdepth"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--progress", action="store_true",
                    help="print enqueue progress to stderr (long profiled runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB streaming kernel before warmup (counter scaling)")
    ap.add_argument("--breakdown", action="store_true",
                    help="time every kernel class on the sampled steps (adds event records)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decoder step shards by sequence with no "
              "communication, so N GPUs run N independent copies; run it with --gpus 1.",
              file=sys.stderr)
        raise SystemExit(2)
    out = run_refdepth(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
