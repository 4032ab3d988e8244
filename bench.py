"""Decoder token-steps/s of the recurrent decoder step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload refdepth]

Default workload: the reference-depth model (48 layers, d = 2048, 16 heads,
FFN 8192, window 512, one shared memory group, V = 32768, bf16) on 32
sequences: 2048 prompt tokens through rlt_run_sequence, then 512 single
rlt_decoder_step calls on the same state (no reset at the split).  A "step" is
one decoder step over the whole batch.  With no --steps the whole 2560-step
run is timed.  --steps K < 2560 times K steps at positions stratified over the
run instead: the run is cut into min(K, 20) equal strata of positions, a
resident state of all 32 sequences is imported (synthetic history, the
imported-state reading) at the middle of each stratum, and the K steps go
round those states in order, each consuming that state's next token; the K
steps are enqueued back to back and timed as one region, so their mean
position is the run's (about 1280) and the per-step work is the run's mean.
Inputs are synthetic (seeded, drawn on the GPU) and resident in HBM before
timing starts; logits of every step are written.

Printed: one JSON line with the throughput, the roofline figure of the
dominant kernel (cross-attention over the encoder memory), measured with HIP
events inside the timed region on the launch stream, and the CPU oracle timed
on a bounded sample of the same workload on the host cores.

Other measurements (each prints its own JSON line; not the default):
  --workload largebatch   256 sequences at ragged positions t ~ U{1..8192},
                          W = 1024: K consecutive batched steps from imported
                          states, MFMA utilisation of the GEMM kernels
  --workload tiny|small   the tiny fp32 and small bf16 configs, whole runs
                          (launch-bound; reported, not targeted); --fused:
                          the tiny run as one launch, one workgroup per sequence
  --workload longctx      d = 4096, 8 sequences, T = 32768: 64-step windows
                          from imported states at six start positions, per-step
                          time fitted as a + b min(t, W) + c t and summed
  --generate              generation at the reference depth: 512 tokens sampled
                          (temperature 1, top-k 50) after the 2048-token prompt
                          (--with-encoder: the causal encoder in the loop;
                          --fast-encoder: its short calls on the decoder's forms)
  --score                 replay scoring at the reference depth: every next
                          token's log-probability, read before it is consumed
  --counters-sample       reference-depth model, all sequences at the run's
                          mean sampled position: a few steps for hardware
                          counter passes (with --calibrate-copy)
  --peaks                 the device's achievable HBM read/copy and bf16 MFMA
                          rates (also added to the reference-depth line as
                          "achievable", measured after the timed region)
  --vendor-gemms          the step's GEMM sequence (reference-depth shapes,
                          weights per layer) through the vendor GEMM library
                          at --vendor-rows rows, for comparison with the
                          decoder's own GEMM kernels (kernel time by rocprofv3)
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
KERNEL_SOURCE = (os.path.join(ROOT, "recurrent_decode_step_amd", "csrc", "rlt_kernels.hip"),
                 os.path.join(ROOT, "recurrent_decode_step_amd", "csrc", "rlt_device.h"))
COUNTERS_FILE = os.path.join(ROOT, "profiles", "k_attn_cross_refdepth_b32_counters.md")


def source_sha256(paths=KERNEL_SOURCE):
    """sha256 over the cross-attention kernel's own source: the device helpers
    (rlt_device.h), the attention section of rlt_kernels.hip and its launcher
    functions (attn_dispatch, launch_attn, attn_chunk_max).  Edits to the
    GEMMs or other kernels leave it unchanged."""
    import hashlib
    import re
    kernels, device = paths
    text = open(kernels).read()
    a = text.index("// ---------------------------------------------------------------- attention")
    b = text.index("// ----------------------------------------------------------------", a + 10)
    parts = [open(device).read(), text[a:b]]
    for name in ("attn_dispatch", "launch_attn", "attn_chunk_max"):
        m = re.search(r"\n[^\n]*\b" + name + r"\([^)]*\) \{.*?\n\}\n", text, re.S)
        parts.append(m.group(0) if m else "")
    return hashlib.sha256("\0".join(parts).encode()).hexdigest()


def measured_traffic(algorithmic_per_launch, path=COUNTERS_FILE):
    """HBM bytes per launch of the cross-attention kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy
    calibration), taken on a sample of launches at the run's mean position and
    scaled by the ratio of algorithmic bytes per launch (run / sample); None
    when the summary is missing or was taken on another kernel source."""
    try:
        kv = {}
        for line in open(path):
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                kv[k.strip().strip("`")] = v.strip().strip("`")
        if kv.get("kernel_source_sha256") != source_sha256():
            return None
        sample = float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
        return sample * algorithmic_per_launch / float(kv["sample_algorithmic_bytes_per_launch"])
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


def synthetic_record(cfg, params, t, dev, index):
    """Decoder state about to consume token t: s and min(t-1, W-1) history
    entries per layer drawn N(0, 1); t = 1 is H_0 (s = s*, empty history)."""
    from recurrent_decode_step_amd import synth
    r = synth.imported_state(cfg, int(t), device=dev, index=index)
    if int(t) == 1:
        r["s"] = params["s_star"].clone()
    return r


def import_positions(model, state, cfg, params, positions, dev, chunk=8):
    """Import synthetic states so slot b is about to consume token positions[b]."""
    import torch
    from recurrent_decode_step_amd import binding
    B = len(positions)
    for b0 in range(0, B, chunk):
        idx = list(range(b0, min(B, b0 + chunk)))
        recs = [synthetic_record(cfg, params, positions[b], dev, b) for b in idx]
        snap = binding.build_snapshot(cfg, recs, version=model.version, device=dev)
        binding.rlt_state_import(model, state, snap, idx)
        del snap, recs
    torch.cuda.synchronize()


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


def cpu_baseline(cfg, params_gpu, e_gpu, mk_gpu, mv_gpu, t0, budget_s=15.0, max_steps=16,
                 where="the run's mean position"):
    """The oracle (fp32 NumPy, as it stands) on the host: all sequences of the
    workload batched, consuming tokens t0, t0+1, ... from synthetic states
    imported at t0 (the run's mean position), until the time budget is spent."""
    import torch
    import oracle
    t_prep = time.time()
    dev = e_gpu.device
    params = {k: v.float().cpu() for k, v in params_gpu.items()}
    B = e_gpu.shape[0]
    om = oracle.Model(params=params, precision="fp32", d_model=cfg.d_model, n_heads=cfg.n_heads,
                      n_layers=cfg.n_layers, d_ffn=cfg.d_ffn, window=cfg.window,
                      mem_groups=cfg.mem_groups, vocab=cfg.vocab, rms_eps=cfg.rms_eps)
    del params
    n_cap = min(max_steps, e_gpu.shape[1] - t0 + 1)
    states = []
    for b in range(B):
        r = synthetic_record(cfg, params_gpu, t0, dev, b)
        states.append(oracle.state_from_arrays(om, r["pos"], r["s"].float().cpu(),
                                               r["K"].float().cpu(), r["V"].float().cpu()))
        del r
    e = e_gpu[:, t0 - 1:t0 - 1 + n_cap].float().cpu()
    mk = mk_gpu[:, :, :, :t0 - 1 + n_cap].float().cpu()
    mv = mv_gpu[:, :, :, :t0 - 1 + n_cap].float().cpu()
    prep = time.time() - t_prep
    t_start = time.time()
    done = 0
    while done < n_cap:
        oracle.decoder_step(om, states, e[:, done], mk, mv)
        done += 1
        if time.time() - t_start >= budget_s:
            break
    el = time.time() - t_start
    return {"value": B * done / el, "unit": "token-steps/s", "cores": openblas_threads(),
            "kind": "oracle",
            "sample": f"{B} sequences x {done} steps (t = {t0}..{t0 + done - 1}, {where}) "
                      f"from synthetic states imported at t = {t0}, NumPy fp32 oracle, "
                      f"weights read once per step for the batch ({el:.1f} s timed, "
                      f"{prep:.1f} s state and input preparation untimed)"}


def measure_peaks(dev):
    """Achievable rates of this device, measured with the library's peak
    kernels outside any timed region: a streaming read and a copy of 1 GiB
    (16-byte non-temporal accesses, one contiguous 64 KiB span per workgroup)
    and dense bf16 MFMA loops of both instruction shapes; the fastest of 5
    launches each (events bound to the dispatch)."""
    import torch
    from recurrent_decode_step_amd import binding
    n = 1 << 30
    src = torch.zeros(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    read = binding.peak_bandwidth(src, dst, copy=False)
    copy = binding.peak_bandwidth(src, dst, copy=True)
    del src, dst
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(2 * cus * 256, dtype=torch.float32, device=dev)
    m32 = binding.peak_mfma(0, 4096, sink)
    m16 = binding.peak_mfma(1, 4096, sink)
    del sink
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(read, 1), "hbm_copy_GBps": round(copy, 1),
            "mfma_bf16_32x32x16_TFLOPs": round(m32, 1), "mfma_bf16_16x16x32_TFLOPs": round(m16, 1),
            "method": "rlt_peak_bandwidth (1 GiB read; copy counts read + written bytes) and "
                      "rlt_peak_mfma (dense loops), fastest of 5 launches"}


def with_peaks(out, dev):
    """Adds the measured achievable rates and the kernel's fraction of them."""
    pk = measure_peaks(dev)
    out["achievable"] = pk
    rf = out.get("roofline")
    if rf and rf.get("unit") == "GB/s" and rf.get("achieved"):
        rf["frac_of_achievable_read"] = round(rf["achieved"] / pk["hbm_read_GBps"], 4)
    return out


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
    classes = (binding.RLT_K_EXTRA, binding.RLT_K_GEMM, binding.RLT_K_SWA, binding.RLT_K_CROSS)
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
    traffic = measured_traffic(cross_bytes / max(cross_n, 1)) if K == T_total else None
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
        names = {binding.RLT_K_EXTRA: "extra", binding.RLT_K_GEMM: "gemm",
                 binding.RLT_K_SWA: "window_attention", binding.RLT_K_CROSS: "cross_attention"}
        n_prof_steps = len(range(0, K, stride))
        out["breakdown_ms_per_step"] = {
            names[c]: round(prof[c][0] / max(n_prof_steps, 1), 4) for c in classes}
        out["breakdown_GBps"] = {
            names[c]: round(prof[c][2] / (prof[c][0] / 1e3) / 1e9, 1) if prof[c][0] else None
            for c in classes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, e, mk, mv, t0=(K + 1) // 2,
                                           budget_s=args.cpu_budget)
    return with_peaks(out, dev)


def stratified_positions(T_total, K, n_states):
    """Strata of the positions 1..T_total: state j serves steps k = j, j + n,
    j + 2n, ... of the K timed steps and consumes r_j consecutive tokens
    from t_j, centred on the middle of stratum j."""
    starts, counts = [], []
    for j in range(n_states):
        r = len(range(j, K, n_states))
        mid = (j + 0.5) * T_total / n_states
        t0 = int(round(mid - (r - 1) / 2))
        t0 = max(1, min(t0, T_total - r + 1))
        starts.append(t0)
        counts.append(r)
    return starts, counts


def cpu_baseline_at(cfg, params_gpu, e_gpu, mk_gpu, mv_gpu, positions, budget_s=15.0):
    """The oracle (fp32 NumPy, as it stands) on the host: one batched step of
    all sequences at each sampled position, taken in pairs symmetric about the
    mean of `positions` (so the sample's mean position is the run's), each
    from synthetic states imported there, until the time budget is spent."""
    import oracle
    dev = e_gpu.device
    params = {k: v.float().cpu() for k, v in params_gpu.items()}
    B = e_gpu.shape[0]
    om = oracle.Model(params=params, precision="fp32", d_model=cfg.d_model, n_heads=cfg.n_heads,
                      n_layers=cfg.n_layers, d_ffn=cfg.d_ffn, window=cfg.window,
                      mem_groups=cfg.mem_groups, vocab=cfg.vocab, rms_eps=cfg.rms_eps)
    del params
    ps = sorted(positions)
    order = []
    lo, hi = 0, len(ps) - 1
    while lo <= hi:
        order.append(ps[lo])
        if hi != lo:
            order.append(ps[hi])
        lo, hi = lo + 1, hi - 1
    t_max = max(ps)
    mk = mk_gpu[:, :, :, :t_max].float().cpu().numpy()
    mv = mv_gpu[:, :, :, :t_max].float().cpu().numpy()
    spent, prep, done = 0.0, 0.0, []
    for t in order:
        t_prep = time.time()
        states = []
        for b in range(B):
            r = synthetic_record(cfg, params_gpu, t, dev, b)
            states.append(oracle.state_from_arrays(om, r["pos"], r["s"].float().cpu(),
                                                   r["K"].float().cpu(), r["V"].float().cpu()))
            del r
        e = e_gpu[:, t - 1].float().cpu()
        prep += time.time() - t_prep
        t0 = time.time()
        oracle.decoder_step(om, states, e, mk, mv)
        spent += time.time() - t0
        done.append(t)
        del states
        if spent >= budget_s and len(done) % 2 == 0:
            break
    return {"value": B * len(done) / spent, "unit": "token-steps/s", "cores": openblas_threads(),
            "kind": "oracle",
            "sample": f"{B} sequences x {len(done)} batched steps at t = "
                      f"{', '.join(str(t) for t in done)} (pairs symmetric about the run's mean "
                      f"position; mean t = {sum(done) / len(done):.0f}), each from synthetic "
                      f"states imported there, NumPy fp32 oracle, weights read once per step for "
                      f"the batch ({spent:.1f} s timed, {prep:.1f} s state preparation untimed)"}


def run_refdepth_stratified(args):
    """K timed steps of the reference-depth run at positions stratified over
    1..2560 (see the module docstring)."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH

    wl = REFDEPTH
    cfg = wl.model
    B, T_total = wl.batch, wl.steps
    K = args.steps
    n_states = min(K, args.strata)
    starts, counts = stratified_positions(T_total, K, n_states)
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
    states = []
    for j in range(n_states):
        st = binding.State(model, B, T_total)
        import_positions(model, st, cfg, params, [starts[j]] * B, dev)
        states.append(st)
        if args.progress:
            print(f"state {j} imported at t = {starts[j]}", file=sys.stderr, flush=True)
    logits = torch.empty((n_states, B, cfg.vocab), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    if args.calibrate_copy:
        calibration_copy(dev)

    # warmup: W steps on a separate state at the run's mean position (untimed)
    if args.warmup > 0:
        t_mid = T_total // 2
        ws = binding.State(model, B, T_total)
        import_positions(model, ws, cfg, params, [t_mid] * B, dev)
        for j in range(args.warmup):
            binding.rlt_decoder_step(model, ws, e_by_step[min(t_mid - 1 + j, T_total - 1)], mem,
                                     logits=logits[0])
        torch.cuda.synchronize()
        del ws
    torch.cuda.synchronize()

    # the kernel figure: every launch of the chosen class in the states of
    # the strata pairs (j, n-1-j) with j even, half the strata, symmetric about
    # the run's mean position; the launch carries its own timing events
    classes = (binding.RLT_K_EXTRA, binding.RLT_K_GEMM, binding.RLT_K_SWA, binding.RLT_K_CROSS)
    mask = (1 << binding.RLT_K_CROSS) if not args.breakdown else sum(1 << c for c in classes)
    profiled = [j for j in range(n_states) if min(j, n_states - 1 - j) % 2 == 0]
    for j in profiled:
        binding.profile_begin(states[j], mask, 1 << 16, step_stride=1)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    next_t = list(starts)
    positions = []
    ws = binding.StepWorkspace(model, B) if args.persistent else None
    if ws is not None:
        profiled = []                           # the persistent step has no per-kernel events
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(K):
        j = k % n_states
        t = next_t[j]
        if ws is None:
            binding.rlt_decoder_step(model, states[j], e_by_step[t - 1], mem, logits=logits[j])
        else:
            binding.rlt_run_sequence_persistent(model, states[j], e_by_step[t - 1].unsqueeze(1),
                                                mem, ws, logits=logits[j].unsqueeze(1))
        positions.append(t)
        next_t[j] = t + 1
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    prof = {c: [0.0, 0, 0.0] for c in classes}
    for j in profiled:
        for c in classes:
            a, n, b = binding.profile_collect(states[j], c)
            prof[c][0] += a
            prof[c][1] += n
            prof[c][2] += b
        binding.profile_begin(states[j], 0, 0)
    prof_steps = sum(counts[j] for j in profiled)
    for j, st in enumerate(states):
        assert all(st.position(b) == starts[j] - 1 + counts[j] for b in range(B))
    if not torch.isfinite(logits).all():
        raise RuntimeError("non-finite logits")

    if ws is not None:
        binding.rlt_persistent_check(ws)
    bytes_run = sum(algorithmic_bytes_per_step(cfg, [t] * B, es) for t in positions)
    cross_ms, cross_n, cross_bytes = prof[binding.RLT_K_CROSS]
    cross_avg_ms = cross_ms / max(cross_n, 1)
    achieved = cross_bytes / max(cross_n, 1) / (cross_avg_ms / 1e3) / 1e9 if cross_n else 0.0
    traffic = measured_traffic(cross_bytes / max(cross_n, 1)) if cross_n else None
    mean_t = sum(positions) / len(positions)
    out = {
        "metric": "decoder token-steps/sec at 1 GPU (48-layer, B=32/256); % HBM/MFMA roofline",
        "value": round(B * K / (ms / 1e3), 2),
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
        "config": {"workload": wl.name, "batch": B,
                   "method": f"{K} steps at positions stratified over 1..{T_total}: {n_states} "
                             f"resident states imported at the strata's middles, steps taken "
                             f"round the states back to back in one timed region",
                   "positions": f"{min(positions)}..{max(positions)} in {n_states} strata, "
                                f"mean t = {mean_t:.1f}",
                   "strata_starts": starts,
                   "logits": "every step, fp32",
                   "step": "persistent (one cooperative launch per step)" if ws is not None
                           else "launch chain (2 + 8L launches per step)"},
        "roofline": {"bound": "hbm", "kernel": "k_attn<bf16,128,1> (cross-attention, encoder memory)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes_per_launch": round(cross_bytes / max(cross_n, 1)),
                     "launches_timed": cross_n, "avg_launch_us": round(cross_avg_ms * 1e3, 2),
                     "timing": f"events bound to each launch's own dispatch, every launch of the "
                               f"{len(profiled)} strata {profiled} (pairs symmetric about the "
                               f"mean position)"},
        "step_roofline": {"bound": "hbm", "algorithmic_GB_per_step": round(bytes_run / K / 1e9, 3),
                          "achieved": round(bytes_run / (ms / 1e3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(bytes_run / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "setup_s": round(setup_s, 1),
    }
    if args.breakdown:
        names = {binding.RLT_K_EXTRA: "extra", binding.RLT_K_GEMM: "gemm",
                 binding.RLT_K_SWA: "window_attention", binding.RLT_K_CROSS: "cross_attention"}
        out["breakdown_ms_per_step"] = {names[c]: round(prof[c][0] / prof_steps, 4)
                                        for c in classes}
        out["breakdown_GBps"] = {
            names[c]: round(prof[c][2] / (prof[c][0] / 1e3) / 1e9, 1) if prof[c][0] else None
            for c in classes}
    del states
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_at(cfg, params, e, mk, mv, sorted(set(positions)),
                                              budget_s=args.cpu_budget)
    return with_peaks(out, dev)


def run_counters_sample(args):
    """Reference-depth model, all 32 sequences at the mean position of the
    stratified timed steps (20 strata of 1..2560: mean t = 1280), a few
    decoder steps, for rocprofv3 counter passes."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH
    wl = REFDEPTH
    cfg, B, T = wl.model, wl.batch, wl.steps
    n = args.sample_steps
    starts, _ = stratified_positions(T, 20, 20)
    t_mean = sum(starts) / len(starts)
    t0 = int(round(t_mean - (n - 1) / 2))
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, T, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    mem = binding.memory_view(mk, mv)
    state = binding.State(model, B, T)
    import_positions(model, state, cfg, params, [t0] * B, dev)
    print(f"counters sample: states imported at t = {t0}", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        calibration_copy(dev)
    binding.profile_begin(state, 1 << binding.RLT_K_CROSS, 1 << 16, step_stride=1)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device=dev)
    for j in range(n):
        binding.rlt_decoder_step(model, state, e[:, t0 - 1 + j].contiguous(), mem, logits=logits)
    torch.cuda.synchronize()
    ms, launches, nbytes = binding.profile_collect(state, binding.RLT_K_CROSS)
    return {"mode": "counters-sample", "workload": wl.name, "positions": f"{t0}..{t0 + n - 1}",
            "cross_launches": launches, "cross_algorithmic_bytes_per_launch": round(nbytes / launches),
            "cross_avg_launch_us": round(ms / launches * 1e3, 2),
            "calibration_copy_bytes": (256 << 20) if args.calibrate_copy else 0}


def run_score(args):
    """Replay scoring at the reference depth: all 32 sequences rebuilt from H_0
    over 2560 recorded tokens (realized tokens uniform in the vocabulary), the
    log-probability of every next token read from each step's logits before
    it is consumed; one rlt_score_sequence call, timed with HIP events."""
    import numpy as np
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH
    wl = REFDEPTH
    cfg, B, T_total = wl.model, wl.batch, wl.steps
    K = T_total if args.steps is None else args.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, T_total, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T_total, device=dev)
    mem = binding.memory_view(mk, mv)
    rng = np.random.default_rng([synth.SEED_POS, 1, 0, 0])
    tokens = torch.from_numpy(rng.integers(0, cfg.vocab, size=(B, K)).astype(np.int32)).to(dev)
    out = torch.empty((B, K), dtype=torch.float32, device=dev)
    state = binding.State(model, B, T_total)
    if args.warmup > 0:
        binding.rlt_score_sequence(model, state, e[:, :args.warmup], mem, tokens[:, :args.warmup])
        binding.rlt_state_reset(model, state, list(range(B)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    binding.rlt_score_sequence(model, state, e[:, :K], mem, tokens, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite scores")
    return {
        "metric": "replay-scored decoder token-steps/sec at 1 GPU (48-layer, B=32)",
        "value": round(B * K / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms / K, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + ", replay scoring", "batch": B, "positions": f"1..{K}",
                   "tokens": "uniform in the vocabulary (seed 3)",
                   "output": "log-probability of each realized next token, fp32"},
        "mean_logprob": round(float(out.double().mean()), 4),
    }


def run_full_sequence(args, wl):
    """A whole-run workload (tiny fp32 or small bf16): all sequences from H_0
    through T steps in one rlt_run_sequence call, logits of every step, timed
    with HIP events; the median of 5 repeats (state reset in between); the
    CPU oracle on the first steps of the same run beside it."""
    import statistics
    import torch
    from recurrent_decode_step_amd import binding, synth
    cfg, B, T = wl.model, wl.batch, wl.steps
    es = 2 if cfg.dtype == 1 else 4
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, T, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    mem = binding.memory_view(mk, mv)
    state = binding.State(model, B, T)
    logits = torch.empty((B, T, cfg.vocab), dtype=torch.float32, device=dev)
    ws = binding.StepWorkspace(model, B) if args.persistent else None

    if args.fused and not binding.fused_supported(cfg):
        raise SystemExit(f"--fused: {wl.name} does not fit one workgroup's LDS")

    def run(ee, lg=None):
        if ws is not None:
            return binding.rlt_run_sequence_persistent(model, state, ee, mem, ws, logits=lg)
        if args.fused:
            return binding.rlt_run_sequence_fused(model, state, ee, mem, logits=lg)
        return binding.rlt_run_sequence(model, state, ee, mem, logits=lg)

    run(e[:, :min(4, T)])                                               # warm-up
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(5):
        binding.rlt_state_reset(model, state, list(range(B)))
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        run(e, logits)
        ev1.record(stream)
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1))
    ms = statistics.median(times)
    bytes_run = sum(algorithmic_bytes_per_step(cfg, [k + 1] * B, es) for k in range(T))
    out = {
        "metric": f"decoder token-steps/sec at 1 GPU ({wl.name.split(' ')[0]})",
        "value": round(B * T / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": T,
        "ms_per_step": round(ms / T, 4), "higher_is_better": True,
        "dtype": "f32" if es == 4 else "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "positions": f"1..{T}",
                   "repeats": "median of 5 full runs", "logits": "every step, fp32",
                   "step": "persistent (one cooperative launch per step)" if ws is not None
                           else ("fused (the whole run in one launch, one workgroup per sequence)"
                                 if args.fused else "launch chain (2 + 8L launches per step)")},
        "step_roofline": {"bound": "hbm", "algorithmic_GB_per_step": round(bytes_run / T / 1e9, 5),
                          "achieved": round(bytes_run / (ms / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s",
                          "frac": round(bytes_run / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "launch-bound at this size; reported, not targeted"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, e, mk, mv, t0=1, budget_s=args.cpu_budget,
                                           max_steps=T, where="from the start of the same run")
    return out


def run_generate(args):
    """Generation at the reference depth: the 2048-token prompt of all 32
    sequences through rlt_run_sequence (last logits only, untimed), then 512
    tokens generated by rlt_generate (temperature 1, top-k 50; stand-in
    encoder tables write the memory entries of the generated positions),
    timed with HIP events around the generation."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH
    wl = REFDEPTH
    cfg, B, T, P = wl.model, wl.batch, wl.steps, wl.prompt
    n = T - P if args.steps is None else min(args.steps, T - P)
    temperature, top_k = 1.0, 50
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, P, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    te, tk, tv = synth.encoder_tables(cfg, device=dev)
    u = synth.uniforms((B, n), device=dev)
    state = binding.State(model, B, T)
    logits0 = binding.rlt_run_sequence(model, state, e, (mk, mv), logits_mode=binding.RLT_LOGITS_LAST)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    tok, lp, _ = binding.rlt_generate(model, state, logits0, te, tk, tv, (mk, mv), temperature,
                                      top_k, u)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    if not torch.isfinite(lp).all():
        raise RuntimeError("non-finite log-probabilities")
    return {
        "metric": "generated token-steps/sec at 1 GPU (48-layer, B=32, after a 2048-token prompt)",
        "value": round(B * n / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": n,
        "ms_per_step": round(ms / n, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + ", generation", "batch": B,
                   "positions": f"{P + 1}..{P + n}",
                   "sampling": f"temperature {temperature}, top-k {top_k}, uniforms seed 5",
                   "encoder": "stand-in tables (e and memory rows of the sampled token)"},
        "mean_behaviour_logprob": round(float(lp.double().mean()), 4),
        "distinct_tokens": int(torch.unique(tok).numel()),
    }


def run_generate_encoded(args):
    """Generation at the reference depth with the causal encoder in the loop:
    the 2048-token prompt of all 32 sequences encoded by rlt_encode and
    consumed by rlt_run_sequence (untimed), then 512 tokens generated by
    rlt_generate_encoded (temperature 1, top-k 50; each sampled token encoded
    from the encoder cache of its sequence, T = 1), timed with HIP events
    around the generation."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH
    wl = REFDEPTH
    cfg, B, T, P = wl.model, wl.batch, wl.steps, wl.prompt
    n = T - P if args.steps is None else min(args.steps, T - P)
    temperature, top_k = 1.0, 50
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    enc = binding.Encoder(model, synth.encoder_params(cfg, device=dev))
    es = binding.EncoderState(enc, B, T, B * P)
    sd = torch.bfloat16
    shape = (cfg.mem_groups, B, cfg.n_heads, T, cfg.head_dim)
    mk = torch.zeros(shape, dtype=sd, device=dev)
    mv = torch.zeros(shape, dtype=sd, device=dev)
    prompt = torch.from_numpy(synth.token_ids(B, P, cfg.vocab, index=0)).to(dev)
    e = binding.rlt_encode(enc, es, prompt, (mk, mv))
    u = synth.uniforms((B, n), device=dev)
    state = binding.State(model, B, T)
    logits0 = binding.rlt_run_sequence(model, state, e, (mk, mv), logits_mode=binding.RLT_LOGITS_LAST)
    del e
    if args.fast_encoder:
        binding.rlt_encoder_state_set_mode(es, binding.RLT_ENC_FAST)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    tok, lp, _ = binding.rlt_generate_encoded(model, state, logits0, enc, es, (mk, mv), temperature,
                                              top_k, u)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    if not torch.isfinite(lp).all():
        raise RuntimeError("non-finite log-probabilities")
    return {
        "metric": "generated token-steps/sec at 1 GPU (48-layer, B=32, after a 2048-token prompt, "
                  "causal encoder in the loop)",
        "value": round(B * n / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": n,
        "ms_per_step": round(ms / n, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + ", generation", "batch": B,
                   "positions": f"{P + 1}..{P + n}",
                   "sampling": f"temperature {temperature}, top-k {top_k}, uniforms seed 5",
                   "encoder": "the causal encoder, one token per sequence per step from its cache",
                   "encoder_mode": "fast (decoder kernel forms)" if args.fast_encoder
                                   else "exact (the prompt kernels' arithmetic)"},
        "mean_behaviour_logprob": round(float(lp.double().mean()), 4),
        "distinct_tokens": int(torch.unique(tok).numel()),
    }


def run_longctx_full(args):
    """The long-context workload run whole: 8 sequences from H_0 through all
    32768 steps (rlt_run_sequence in chunks of 1024 steps, no reset, logits of
    the last step of each chunk), timed with HIP events around the whole run."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import LONGCTX
    wl = LONGCTX
    cfg, B, T = wl.model, wl.batch, wl.steps
    chunk = 1024
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    e = synth.encoder_e(cfg, B, T, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    mem = binding.memory_view(mk, mv)
    state = binding.State(model, B, T)
    binding.rlt_run_sequence(model, state, e[:, :4], mem, logits_mode=binding.RLT_LOGITS_LAST)
    binding.rlt_state_reset(model, state, list(range(B)))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(T // chunk + 1)]
    ev[0].record(stream)
    for c in range(T // chunk):
        lg = binding.rlt_run_sequence(model, state, e[:, c * chunk:(c + 1) * chunk], mem,
                                      logits_mode=binding.RLT_LOGITS_LAST)
        ev[c + 1].record(stream)
        ev[c + 1].synchronize()
        print(f"longctx full run: {(c + 1) * chunk} of {T} steps, "
              f"{ev[c].elapsed_time(ev[c + 1]) / chunk:.3f} ms/step", file=sys.stderr, flush=True)
    ms = ev[0].elapsed_time(ev[-1])
    if not torch.isfinite(lg).all():
        raise RuntimeError("non-finite logits")
    bytes_total = sum(algorithmic_bytes_per_step(cfg, [t] * B, 2) for t in range(1, T + 1, 64)) * 64
    return {
        "metric": "decoder token-steps/sec at 1 GPU (48-layer, d=4096, B=8, T=32768)",
        "value": round(B * T / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": T,
        "ms_per_step": round(ms / T, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "method": "one full run of 32768 steps from H_0",
                   "logits": "last step of every 1024-step chunk"},
        "step_roofline": {"bound": "hbm", "algorithmic_GB_per_step": round(bytes_total / T / 1e9, 3),
                          "achieved": round(bytes_total / (ms / 1e3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(bytes_total / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
    }


def run_largebatch(args):
    """256 sequences at ragged positions t_b ~ U{1..8192} (W = 1024): states
    imported at t_b, one untimed step, then K batched steps timed with HIP
    events around the whole pass, then K more with every launch timed per
    kernel class (the GEMM time gives the MFMA utilisation).  Each pass moves
    every sequence on by K positions (K << mean t, so the per-step work is
    the same to within K / 4096)."""
    import numpy as np
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import LARGEBATCH
    wl = LARGEBATCH
    cfg, B = wl.model, wl.batch
    K = args.steps or 5
    n_steps = 2 * K + 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_setup = time.time()
    pos = synth.ragged_positions(B, wl.t_max)
    cap = wl.t_max + n_steps
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    # e rows of the consumed positions only: stream (sequence b, start t_b)
    e = torch.stack([synth.normal((n_steps, cfg.d_model), device=dev, seed=synth.SEED_E,
                                  index=b, layer=int(pos[b]), round_bf16=True,
                                  out_dtype=torch.bfloat16) for b in range(B)])
    e_by_step = e.transpose(0, 1).contiguous()       # [step][B][d]
    del e
    mk, mv = synth.encoder_memory(cfg, B, cap, device=dev)
    mem = binding.memory_view(mk, mv)
    state = binding.State(model, B, cap)
    import_positions(model, state, cfg, params, pos, dev)
    print(f"largebatch: {B} states imported ({time.time() - t_setup:.0f} s)", file=sys.stderr,
          flush=True)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device=dev)
    binding.rlt_decoder_step(model, state, e_by_step[0], mem, logits=logits)   # untimed
    torch.cuda.synchronize()
    classes = (binding.RLT_K_GEMM, binding.RLT_K_SWA, binding.RLT_K_CROSS)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    for j in range(1, K + 1):
        binding.rlt_decoder_step(model, state, e_by_step[j], mem, logits=logits)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    binding.profile_begin(state, sum(1 << c for c in classes), 1 << 20, step_stride=1)
    for j in range(K + 1, 2 * K + 1):
        binding.rlt_decoder_step(model, state, e_by_step[j], mem, logits=logits)
    torch.cuda.synchronize()
    prof = {c: binding.profile_collect(state, c) for c in classes}
    binding.profile_begin(state, 0, 0)
    if not torch.isfinite(logits).all():
        raise RuntimeError("non-finite logits")
    gemm_ms = prof[binding.RLT_K_GEMM][0] / K
    flops = gemm_flops_per_step(cfg, B)
    bytes_step = sum(algorithmic_bytes_per_step(cfg, [int(t) + j for t in pos], 2)
                     for j in range(1, K + 1)) / K
    names = {binding.RLT_K_GEMM: "gemm", binding.RLT_K_SWA: "window_attention",
             binding.RLT_K_CROSS: "cross_attention"}
    return {
        "metric": "decoder token-steps/sec at 1 GPU (48-layer, B=256); MFMA utilisation of the "
                  "GEMM kernels",
        "value": round(B * K / (ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1, "steps": K,
        "ms_per_step": round(ms / K, 4), "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B,
                   "positions": f"t_b ~ U{{1..{wl.t_max}}} (seed 3); timed steps consume "
                                f"t_b+1..t_b+{K}, profiled steps t_b+{K + 1}..t_b+{2 * K}",
                   "mean_t_b": round(float(np.mean(pos)), 1), "state": "imported synthetic"},
        "mfma": {"bound": "mfma", "gemm_flops_per_step": flops,
                 "gemm_ms_per_step": round(gemm_ms, 4),
                 "achieved": round(flops / (gemm_ms / 1e3) / 1e12, 1),
                 "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(flops / (gemm_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "step_roofline": {"bound": "hbm", "algorithmic_GB_per_step": round(bytes_step / 1e9, 3),
                          "achieved": round(bytes_step / (ms / K / 1e3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(bytes_step / (ms / K / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "breakdown_ms_per_step": {names[c]: round(prof[c][0] / K, 4) for c in classes},
        "breakdown_GBps": {names[c]: round(prof[c][2] / (prof[c][0] / 1e3) / 1e9, 1)
                           for c in classes},
    }


def run_longctx(args):
    """d = 4096, B = 8, T = 32768.  The full run is estimated from 64-step
    windows starting at imported states at t0 in {1, 4097, 8193, 16385, 24577,
    32705}: per-step time tau(t) = a + b min(t, W) + c t is fitted to the
    windows' per-step times (bytes per step are exactly affine in min(t, W)
    and t) and summed over t = 1..32768."""
    import numpy as np
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import LONGCTX
    wl = LONGCTX
    cfg, B, T = wl.model, wl.batch, wl.steps
    W = cfg.window
    n = args.steps or 64
    starts = [1, 4097, 8193, 16385, 24577, T - n + 1]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    mem = binding.memory_view(mk, mv)
    state = binding.State(model, B, T)
    rows = []
    cross = []                                  # per window: (ms, launches, bytes)
    stream = torch.cuda.current_stream()
    for t0 in starts:
        import_positions(model, state, cfg, params, [t0] * B, dev, chunk=2)
        e = torch.stack([synth.normal((n, cfg.d_model), device=dev, seed=synth.SEED_E, index=b,
                                      layer=t0, round_bf16=True, out_dtype=torch.bfloat16)
                         for b in range(B)])
        if t0 == starts[0]:
            binding.rlt_decoder_step(model, state, e[:, 0].contiguous(), mem)   # warm, untimed
            import_positions(model, state, cfg, params, [t0] * B, dev, chunk=2)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        binding.profile_begin(state, 1 << binding.RLT_K_CROSS, 1 << 16, step_stride=1)
        ev0.record(stream)
        binding.rlt_run_sequence(model, state, e, mem, logits_mode=binding.RLT_LOGITS_LAST)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1)
        cross.append(binding.profile_collect(state, binding.RLT_K_CROSS))
        binding.profile_begin(state, 0, 0)
        t_mid = t0 + (n - 1) / 2
        rows.append((t0, ms / n, float(np.mean([min(t, W) for t in range(t0, t0 + n)])), t_mid))
        print(f"longctx: window t0={t0}: {ms / n:.3f} ms/step", file=sys.stderr, flush=True)
    A = np.array([[1.0, r[2], r[3]] for r in rows])
    y = np.array([r[1] for r in rows])
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    ts = np.arange(1, T + 1, dtype=np.float64)
    total_ms = float(np.sum(coef[0] + coef[1] * np.minimum(ts, W) + coef[2] * ts))
    bytes_total = sum(algorithmic_bytes_per_step(cfg, [t] * B, 2) for t in range(1, T + 1, 64)) * 64
    c_ms = sum(c[0] for c in cross)
    c_n = sum(c[1] for c in cross)
    c_bytes = sum(c[2] for c in cross)
    out = {
        "metric": "decoder token-steps/sec at 1 GPU (48-layer, d=4096, B=8, T=32768)",
        "value": round(B * T / (total_ms / 1e3), 2), "unit": "token-steps/s", "n_gpus": 1,
        "steps": T, "ms_per_step": round(total_ms / T, 4), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "method":
                   f"{n}-step windows from imported states at t0 = {starts}; "
                   "tau(t) = a + b min(t,W) + c t least-squares fit, summed over t = 1..32768"},
        "windows_ms_per_step": {str(r[0]): round(r[1], 4) for r in rows},
        "fit_ms": {"a": float(coef[0]), "b_per_window_pos": float(coef[1]),
                   "c_per_memory_pos": float(coef[2])},
        "step_roofline": {"bound": "hbm",
                          "algorithmic_GB_per_step": round(bytes_total / T / 1e9, 3),
                          "achieved": round(bytes_total / (total_ms / 1e3) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(bytes_total / (total_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "k_attn<bf16,128,1> (cross-attention, encoder memory)",
                     "achieved": round(c_bytes / (c_ms / 1e3) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(c_bytes / (c_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "launches_timed": c_n,
                     "avg_launch_us": round(c_ms / max(c_n, 1) * 1e3, 2),
                     "per_window_GBps": {str(t0): round(c[2] / (c[0] / 1e3) / 1e9, 1)
                                         for t0, c in zip(starts, cross)},
                     "timing": "events bound to each launch's own dispatch, every launch of the "
                               "six windows"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_longctx(cfg, params, mk, mv, starts, W, T,
                                                   budget_s=max(args.cpu_budget, 60.0))
    return out


def cpu_baseline_longctx(cfg, params_gpu, mk_gpu, mv_gpu, starts, W, T, budget_s=60.0, rows=2):
    """The oracle (fp32 NumPy, as it stands) on the host for the long-context
    workload: `rows` sequences take one batched step from synthetic states
    imported at each window start (in the order 1, last, then inwards, until
    the budget is spent and at least three starts are done), per-step time
    fitted as a + b min(t, W) + c t (as on the GPU) and summed over the run.
    The fp32 weights (42.6 GiB) are converted once, untimed."""
    import numpy as np
    import oracle
    dev = mk_gpu.device
    t_prep = time.time()
    params = {k: v.float().cpu() for k, v in params_gpu.items()}
    om = oracle.Model(params=params, precision="fp32", d_model=cfg.d_model, n_heads=cfg.n_heads,
                      n_layers=cfg.n_layers, d_ffn=cfg.d_ffn, window=cfg.window,
                      mem_groups=cfg.mem_groups, vocab=cfg.vocab, rms_eps=cfg.rms_eps)
    del params
    prep = time.time() - t_prep
    order = [starts[0], starts[-1]] + [t for t in reversed(starts[1:-1])]
    pts, spent = [], 0.0
    for t in order:
        t_prep = time.time()
        st = []
        for b in range(rows):
            r = synthetic_record(cfg, params_gpu, t, dev, b)
            st.append(oracle.state_from_arrays(om, r["pos"], r["s"].float().cpu(),
                                               r["K"].float().cpu(), r["V"].float().cpu()))
            del r
        mk = mk_gpu[:, :rows, :, :t].float().cpu().numpy()
        mv = mv_gpu[:, :rows, :, :t].float().cpu().numpy()
        e = np.random.default_rng(t).standard_normal((rows, cfg.d_model)).astype(np.float32)
        prep += time.time() - t_prep
        t0 = time.time()
        oracle.decoder_step(om, st, e, mk, mv)
        el = time.time() - t0
        spent += el
        pts.append((t, el))
        print(f"longctx cpu baseline: t = {t}: {el:.2f} s per step", file=sys.stderr, flush=True)
        del st, mk, mv
        if spent >= budget_s and len(pts) >= 3:
            break
    A = np.array([[1.0, min(t, W), t] for t, _ in pts])
    y = np.array([el for _, el in pts])
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    ts = np.arange(1, T + 1, dtype=np.float64)
    total_s = float(np.sum(coef[0] + coef[1] * np.minimum(ts, W) + coef[2] * ts))
    return {"value": rows * T / total_s, "unit": "token-steps/s", "cores": openblas_threads(),
            "kind": "oracle",
            "sample": f"{rows} sequences x one batched step at t = "
                      f"{', '.join(str(t) for t, _ in pts)} (s per step "
                      f"{', '.join(f'{el:.2f}' for _, el in pts)}), each from synthetic states "
                      f"imported there, NumPy fp32 oracle; per-step time fitted as a + b min(t, W) "
                      f"+ c t and summed over t = 1..{T} ({spent:.1f} s timed, {prep:.1f} s weight "
                      f"conversion and state preparation untimed)"}


def run_encode(args):
    """The token-parallel causal encoder over the reference-depth prompt: 32
    sequences x 2048 tokens in one rlt_encode call (e rows, the encoder cache
    of every layer and the memory entries of all 2048 positions), repeated
    `steps` times from position 0.  Each kernel class is timed with HIP events
    on the launch stream; the GEMMs are the dominant, MFMA-bound kernels."""
    import numpy as np
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import REFDEPTH
    wl = REFDEPTH
    cfg, B, T = wl.model, wl.batch, wl.prompt
    K = 3 if args.steps is None else args.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_setup = time.time()
    params = synth.model_params(cfg, device=dev)
    eparams = synth.encoder_params(cfg, device=dev)
    model = binding.Model(cfg, params, version=1)
    enc = binding.Encoder(model, eparams)
    es = binding.EncoderState(enc, B, T, B * T)
    sd = torch.bfloat16
    mk = torch.zeros((cfg.mem_groups, B, cfg.n_heads, T, cfg.head_dim), dtype=sd, device=dev)
    mv = torch.zeros_like(mk)
    mem = binding.memory_view(mk, mv)
    tok_np = synth.token_ids(B, T, cfg.vocab, index=0)
    tok = torch.from_numpy(tok_np).to(dev)
    e = torch.empty((B, T, cfg.d_model), dtype=sd, device=dev)
    slots = list(range(B))
    setup_s = time.time() - t_setup
    if args.calibrate_copy:
        calibration_copy(dev)
    for _ in range(max(args.warmup, 0)):
        binding.rlt_encode(enc, es, tok, mem, e_out=e)
        binding.rlt_encoder_state_reset(es, slots)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(K):
        binding.rlt_encode(enc, es, tok, mem, e_out=e)
        binding.rlt_encoder_state_reset(es, slots)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / K
    if not torch.isfinite(e).all():
        raise RuntimeError("non-finite encoder output")
    # per-class kernel times of one more call, HIP events around every launch
    binding.encoder_profile_begin(es, 0b111, 100000)
    binding.rlt_encode(enc, es, tok, mem, e_out=e)
    binding.rlt_encoder_state_reset(es, slots)
    cls = {}
    for name, c in (("gemm", binding.RLT_E_GEMM), ("attention", binding.RLT_E_ATTN),
                    ("embed_norm", binding.RLT_E_OTHER)):
        tot, n, fl, by = binding.encoder_profile_collect(es, c)
        cls[name] = {"ms": tot, "launches": n, "flops": fl, "bytes": by}
    binding.encoder_profile_begin(es, 0, 0)
    g = cls["gemm"]
    a = cls["attention"]
    flops_total = g["flops"] + a["flops"]
    out = {
        "metric": "encoder prompt tokens/sec at 1 GPU (48-layer, B=32 x 2048-token prompt)",
        "value": round(B * T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + ", causal encoder over the prompt", "batch": B,
                   "prompt": T, "tokens": "uniform in the vocabulary (seed 7)",
                   "outputs": "e rows, encoder cache of 48 layers, memory K/V of 2048 positions"},
        "roofline": {"bound": "mfma", "kernel": "k_pgemm (token-parallel GEMMs)",
                     "achieved": round(g["flops"] / (g["ms"] / 1e3) / 1e12, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(g["flops"] / (g["ms"] / 1e3) / 2.5e15, 4),
                     "traffic": None, "flops_per_call": g["flops"], "launches": g["launches"],
                     "avg_launch_us": round(1e3 * g["ms"] / max(g["launches"], 1), 2)},
        "call_mfma": {"flops": flops_total, "achieved": round(flops_total / (ms / 1e3) / 1e12, 1),
                      "frac": round(flops_total / (ms / 1e3) / 2.5e15, 4)},
        "breakdown_ms": {k: round(v["ms"], 3) for k, v in cls.items()},
        "attention_TFLOPs": round(a["flops"] / (a["ms"] / 1e3) / 1e12, 1),
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_encoder_baseline(cfg, params, eparams, tok_np[0], args.cpu_budget)
    return out


def cpu_encoder_baseline(cfg, params_gpu, eparams_gpu, tokens, budget_s=15.0):
    """The oracle's encoder (fp32 NumPy, as it stands) over growing prefixes of
    one sequence until the time budget is spent; tokens/s of the longest."""
    import oracle
    t_prep = time.time()
    LAYER_KEYS = ("g1", "g2", "g3", "wq", "wk", "wv", "wo", "wqc", "woc", "w1", "w2")
    small = {k: params_gpu[k].float().cpu() for k in ("s_star", "wg", "bg", "go", "wout")}
    layers = [{k: params_gpu[k][l].float().cpu() for k in LAYER_KEYS} for l in range(cfg.n_layers)]
    om = oracle.Model(params=small, precision="fp32", d_model=cfg.d_model, n_heads=cfg.n_heads,
                      n_layers=cfg.n_layers, d_ffn=cfg.d_ffn, window=cfg.window,
                      mem_groups=cfg.mem_groups, vocab=cfg.vocab, rms_eps=cfg.rms_eps,
                      layer_source=lambda l: layers[l])
    oe = oracle.Encoder(om, {k: v.float().cpu() for k, v in eparams_gpu.items()})
    prep = time.time() - t_prep
    n, rate, el = 16, 0.0, 0.0
    spent = 0.0
    while spent < budget_s and n <= len(tokens):
        t0 = time.time()
        oracle.encode(oe, tokens[:n])
        el = time.time() - t0
        spent += el
        rate, done = n / el, n
        n *= 2
    return {"value": rate, "unit": "tokens/s", "cores": openblas_threads(), "kind": "oracle",
            "sample": f"1 sequence, its first {done} tokens in one oracle encode call "
                      f"(NumPy fp32, 48 layers; {el:.1f} s timed, {spent:.1f} s over the doubling "
                      f"prefixes, {prep:.1f} s weight conversion untimed)"}


def run_train(args):
    """Backpropagation through time in fp32: B sequences x T steps from H_0,
    loss on every next token, the full gradient of every parameter, e and the
    memory (one rlt_bptt call), repeated `steps` times.  Default: the small
    configuration (d = 512, H = 8, L = 12, F = 2048, W = 128, G = 12, V = 4096),
    B = 128, T = 128, every intermediate kept.  --train-workload refdepth: the
    reference-depth model (d = 2048, L = 48, F = 8192, W = 512, G = 1,
    V = 32768) in fp32, B = 8, T = 256, which fits only with activation
    checkpointing (--train-segment, default 16 there)."""
    import torch
    from recurrent_decode_step_amd import binding, synth
    from recurrent_decode_step_amd.configs import SMALL, REFDEPTH
    ref = args.train_workload == "refdepth"
    cfg = (REFDEPTH if ref else SMALL).model.with_(dtype=0)
    B = args.train_batch if args.train_batch else (8 if ref else 128)
    T = args.train_steps if args.train_steps else (256 if ref else 128)
    seg = args.train_segment if args.train_segment is not None else (16 if ref else 0)
    K = (1 if ref else 3) if args.steps is None else args.steps
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    params = synth.model_params(cfg, device=dev)
    e = synth.encoder_e(cfg, B, T, device=dev)
    mk, mv = synth.encoder_memory(cfg, B, T, device=dev)
    tg = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=0)).to(dev)
    L_ = binding.load_library()
    cc = binding.make_config(cfg)
    ws_bytes = L_.rlt_bptt_workspace_bytes_segmented(binding.C.byref(cc), B, T, seg)
    ws_full = L_.rlt_bptt_workspace_bytes(binding.C.byref(cc), B, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    for _ in range(1 if ref else max(args.warmup, 1)):
        loss, g, de, dm = binding.rlt_bptt(cfg, params, e, (mk, mv), tg, workspace=ws, segment=seg)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(K):
        loss, g, de, dm = binding.rlt_bptt(cfg, params, e, (mk, mv), tg, workspace=ws, segment=seg)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / K
    if not torch.isfinite(loss).all():
        raise RuntimeError("non-finite loss")
    d, L, F, V, W, H = cfg.d_model, cfg.n_layers, cfg.d_ffn, cfg.vocab, cfg.window, cfg.n_heads
    # GEMM FLOPs: forward, input gradients and weight gradients (3 x the forward products)
    fwd = 4 * d * d + L * (12 * d * d + 4 * d * F) + 2 * d * V
    gemm_flops = 3.0 * B * T * fwd
    # attention: 4 d per attended position forward, twice that backward
    pos = sum(min(t + 1, W) + (t + 1) for t in range(T))
    attn_flops = 3.0 * 4 * d * L * B * pos
    total = gemm_flops + attn_flops
    out = {
        "metric": f"BPTT training tokens/sec at 1 GPU (fp32, {L}-layer d={d}, B={B} x {T} steps)",
        "value": round(B * T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": 1 if ref else max(args.warmup, 1), "ms_per_step": round(ms, 3),
        "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": (f"{'refdepth' if ref else 'small'}-f32 model (V={V},d={d},H={H},L={L},F={F},"
                                f"W={W},G={cfg.mem_groups}), BPTT over B={B} sequences x T={T} steps"),
                   "batch": B, "steps_per_sequence": T, "loss": "next-token cross-entropy, all targets",
                   "gradients": "every parameter, e and memory; full BPTT",
                   "activation_checkpointing": (f"segments of {seg} steps (every step forward once, "
                                                f"then each segment recomputed before its backward)"
                                                if 0 < seg < T else "none: every intermediate kept"),
                   "workspace_GB": round(ws_bytes / 1e9, 2),
                   "workspace_GB_without_checkpointing": round(ws_full / 1e9, 2)},
        "roofline": {"bound": "mfma", "kernel": "whole rlt_bptt call (fp32 MFMA GEMMs, VALU attention)",
                     "achieved": round(total / (ms / 1e3) / 1e12, 2), "peak": 157.3,
                     "unit": "TFLOP/s", "frac": round(total / (ms / 1e3) / 157.3e12, 4),
                     "traffic": None, "gemm_flops": gemm_flops, "attention_flops": attn_flops},
        "loss_per_token": round(float(loss) / (B * T), 4),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_train_baseline(cfg, params, e, mk, mv, tg, args.cpu_budget)
    if 0 < seg < T:
        # forward FLOPs are spent twice for every segment but the last
        nseg = (T + seg - 1) // seg
        out["roofline"]["recomputed_forward_flops"] = round(
            (gemm_flops + attn_flops) / 3.0 * (nseg - 1) * seg / T)
    return out


def cpu_train_baseline(cfg, params, e, mk, mv, tg, budget_s=15.0):
    """The oracle's BPTT (torch autograd, float64 as it stands) on the host,
    one sequence over growing step counts until the budget is spent."""
    import torch
    from oracle import bptt
    host = {k: v.float().cpu() for k, v in params.items()}
    nthreads = torch.get_num_threads()
    n, rate, el, spent, done = 2, 0.0, 0.0, 0.0, 0
    while spent < budget_s and n <= e.shape[1]:
        t0 = time.time()
        bptt.gradients(host, e[:1, :n].cpu(), mk[:, :1, :, :n].cpu(), mv[:, :1, :, :n].cpu(),
                       tg[:1, :n].cpu().numpy(), n_heads=cfg.n_heads, window=cfg.window,
                       rms_eps=cfg.rms_eps)
        el = time.time() - t0
        spent += el
        rate, done = n / el, n
        n *= 2
    return {"value": rate, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"1 sequence x {done} steps in one oracle BPTT call (torch autograd, float64, "
                      f"12 layers; {el:.1f} s timed, {spent:.1f} s over the doubling lengths)"}


def run_vendor_gemms(args):
    """The decoder step's GEMM sequence (merge, then per layer QKV, O, Qc, Oc,
    FFN-up, FFN-down, then the head) at the reference-depth model with its own
    weights per layer, run through torch.nn.functional.linear in bf16 (the
    vendor GEMM library) at 32 or 256 rows: the library's rate on the same
    shapes and weight streams, beside the decoder's own GEMM kernels.  No
    norms, epilogues or attention: plain products only.  The wall time here
    includes the host's per-call cost; the kernel time comes from a
    rocprofv3 kernel trace of the same command."""
    import torch
    import torch.nn.functional as Fn
    from recurrent_decode_step_amd.configs import REFDEPTH
    cfg = REFDEPTH.model
    L, d, F, V = cfg.n_layers, cfg.d_model, cfg.d_ffn, cfg.vocab
    M = args.vendor_rows
    K = args.steps or 10
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    g = torch.Generator(device=dev).manual_seed(0)

    def w(n, k):
        return (torch.randn(n, k, device=dev, generator=g) * 0.02).to(torch.bfloat16).contiguous()
    layers = [(w(3 * d, d), w(d, d), w(d, d), w(d, d), w(F, d), w(d, F)) for _ in range(L)]
    wg, wout = w(d, 2 * d), w(V, d)
    xs = {k: torch.randn(M, k, device=dev, generator=g).to(torch.bfloat16) for k in (d, 2 * d, F)}

    def step():
        Fn.linear(xs[2 * d], wg)
        for qkv, o, qc, oc, up, down in layers:
            for wm in (qkv, o, qc, oc, up):
                Fn.linear(xs[d], wm)
            Fn.linear(xs[F], down)
        Fn.linear(xs[d], wout)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    flops = gemm_flops_per_step(cfg, M)
    return {"mode": "vendor GEMM sequence (torch.nn.functional.linear, bf16)", "rows": M,
            "steps": K, "warmup": args.warmup, "gemm_flops_per_step": flops,
            "wall_ms_per_step": round(ms, 4),
            "wall_TFLOPs": round(flops / (ms / 1e3) / 1e12, 1),
            "note": "wall time includes the host's per-call cost; take the kernel time from "
                    "rocprofv3 --kernel-trace --stats of this command"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="refdepth",
                    choices=["refdepth", "largebatch", "longctx", "tiny", "small"])
    ap.add_argument("--full", action="store_true",
                    help="longctx: one full 32768-step run instead of the window fit")
    ap.add_argument("--generate", action="store_true",
                    help="generation at the reference depth after the 2048-token prompt")
    ap.add_argument("--with-encoder", action="store_true",
                    help="--generate with the causal encoder in the loop instead of the tables")
    ap.add_argument("--fast-encoder", action="store_true",
                    help="--with-encoder: the encoder state in RLT_ENC_FAST mode")
    ap.add_argument("--train", action="store_true",
                    help="backpropagation through time (fp32, small config, B x 128 steps)")
    ap.add_argument("--train-batch", type=int, default=0,
                    help="sequences per BPTT call for --train (default 128; refdepth 8)")
    ap.add_argument("--train-steps", type=int, default=0,
                    help="steps per sequence for --train (default 128; refdepth 256)")
    ap.add_argument("--train-segment", type=int, default=None,
                    help="activation checkpointing for --train: steps held at once (0 = all)")
    ap.add_argument("--train-workload", default="small", choices=["small", "refdepth"],
                    help="model for --train")
    ap.add_argument("--encode", action="store_true",
                    help="the causal encoder over the reference-depth prompt (B = 32 x 2048 tokens)")
    ap.add_argument("--score", action="store_true",
                    help="replay scoring at the reference depth (log-probability of each next token)")
    ap.add_argument("--counters-sample", action="store_true",
                    help="a few reference-depth steps at the sampled mean position (counter passes)")
    ap.add_argument("--sample-steps", type=int, default=4)
    ap.add_argument("--strata", type=int, default=20,
                    help="reference depth --steps K: position strata (resident states), at most K")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--progress", action="store_true",
                    help="print enqueue progress to stderr (long profiled runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB streaming kernel before warmup (counter scaling)")
    ap.add_argument("--persistent", action="store_true",
                    help="tiny/small/refdepth --steps K: one persistent launch per decoder step")
    ap.add_argument("--fused", action="store_true",
                    help="tiny: the whole run in one launch (rlt_run_sequence_fused)")
    ap.add_argument("--peaks", action="store_true",
                    help="only the achievable HBM and MFMA rates of the device")
    ap.add_argument("--vendor-gemms", action="store_true",
                    help="the step's GEMM sequence through the vendor GEMM library (comparison)")
    ap.add_argument("--vendor-rows", type=int, default=256, help="rows for --vendor-gemms")
    ap.add_argument("--breakdown", action="store_true",
                    help="time every kernel class on the sampled steps (adds event records)")
    args = ap.parse_args()
    if args.strata < 1:
        ap.error("--strata must be >= 1")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decoder step shards by sequence with no "
              "communication, so N GPUs run N independent copies; run it with --gpus 1.",
              file=sys.stderr)
        raise SystemExit(2)
    if args.peaks:
        import torch
        out = {"mode": "peaks", **measure_peaks(torch.device("cuda", 0))}
    elif args.vendor_gemms:
        out = run_vendor_gemms(args)
    elif args.counters_sample:
        out = run_counters_sample(args)
    elif args.encode:
        out = run_encode(args)
    elif args.train:
        out = run_train(args)
    elif args.score:
        out = run_score(args)
    elif args.generate:
        out = run_generate_encoded(args) if args.with_encoder else run_generate(args)
    elif args.workload == "largebatch":
        out = run_largebatch(args)
    elif args.workload == "longctx":
        out = run_longctx_full(args) if args.full else run_longctx(args)
    elif args.workload in ("tiny", "small"):
        from recurrent_decode_step_amd.configs import TINY, SMALL
        out = run_full_sequence(args, TINY if args.workload == "tiny" else SMALL)
    elif args.steps is not None and args.steps < 2560:
        out = run_refdepth_stratified(args)
    else:
        out = run_refdepth(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
