"""The persistent step (one cooperative launch per decoder step, each work
item waiting on the ready flags of the items it reads) against the launch
chain, through the C ABI
(needs an MI355X).  Both run the same per-workgroup code with the same K
split and summation order, so logits and the exported states must be equal
bit for bit."""
from __future__ import annotations

import pytest
import torch

from _tiny import tiny_cfg, inputs
from recurrent_decode_step_amd import binding, synth
from recurrent_decode_step_amd.configs import DTYPE_BF16, DTYPE_FP32, SMALL

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


CASES = {
    # name: (config overrides, B, T, logits mode)
    "tiny-f32-dh16": (dict(), 4, 20, binding.RLT_LOGITS_ALL),
    "f32-dh32-B20": (dict(d_model=64, n_heads=2, d_ffn=256, vocab=40), 20, 10,
                     binding.RLT_LOGITS_ALL),
    "bf16-dh64-B20-W4": (dict(dtype=DTYPE_BF16, d_model=128, n_heads=2, d_ffn=512, window=4,
                              vocab=40), 20, 12, binding.RLT_LOGITS_ALL),
    "bf16-dh128-L3-G3-last": (dict(dtype=DTYPE_BF16, d_model=256, n_heads=2, d_ffn=512, window=5,
                                   n_layers=3, mem_groups=3, vocab=70), 6, 9,
                              binding.RLT_LOGITS_LAST),
    "bf16-dh32-none": (dict(dtype=DTYPE_BF16, d_model=64, n_heads=2, d_ffn=256, window=3,
                            vocab=24), 3, 7, binding.RLT_LOGITS_NONE),
}


def run_pair(cfg, B, T, mode, e, mem, imports=None):
    params = {k: v.to(DEV) for k, v in synth.model_params(cfg, device="cpu").items()}
    model = binding.Model(cfg, params, version=1)
    cap = mem[0].shape[3]
    sa = binding.State(model, B, cap)
    sb = binding.State(model, B, cap)
    if imports is not None:
        binding.rlt_state_import(model, sa, imports, list(range(B)))
        binding.rlt_state_import(model, sb, imports, list(range(B)))
    ws = binding.StepWorkspace(model, B)
    la = binding.rlt_run_sequence(model, sa, e, mem, logits_mode=mode)
    lb = binding.rlt_run_sequence_persistent(model, sb, e, mem, ws, logits_mode=mode)
    binding.rlt_persistent_check(ws)
    torch.cuda.synchronize()
    snap_a = binding.rlt_state_export(model, sa, list(range(B)))
    snap_b = binding.rlt_state_export(model, sb, list(range(B)))
    return model, sa, sb, la, lb, snap_a, snap_b


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_step_is_bitwise_the_launch_chain(name):
    kw, B, T, mode = CASES[name]
    cfg = tiny_cfg(**kw)
    say(f"[persistent] case={name} B={B} T={T} mode={mode}")
    e, mk, mv = inputs(cfg, B, T)
    e, mem = e.to(DEV), (mk.to(DEV), mv.to(DEV))
    model, sa, sb, la, lb, snap_a, snap_b = run_pair(cfg, B, T, mode, e, mem)
    for b in range(B):
        assert sa.position(b) == sb.position(b) == T
    if mode != binding.RLT_LOGITS_NONE:
        assert torch.isfinite(la).all()
        say(f"  max |d logit| = {float((la - lb).abs().max()):.3e}")
        assert torch.equal(la, lb)
    assert torch.equal(snap_a, snap_b)


def test_persistent_step_ragged_imported_states():
    """Slots at different positions (imported synthetic states): window and
    memory lengths differ by row within every attention phase."""
    cfg = tiny_cfg(dtype=DTYPE_BF16, d_model=128, n_heads=2, d_ffn=512, window=6, vocab=40)
    starts = [1, 3, 6, 7, 12, 20, 2, 9]
    B, T = len(starts), 5
    cap = max(starts) + T
    recs = []
    params_cpu = synth.model_params(cfg, device="cpu")
    for b, t in enumerate(starts):
        r = synth.imported_state(cfg, t, device="cpu", index=b)
        if t == 1:
            r["s"] = params_cpu["s_star"].clone()
        recs.append(r)
    snap = binding.build_snapshot(cfg, recs, version=1, device=DEV)
    e_all, mk, mv = inputs(cfg, B, cap)
    e = torch.stack([e_all[b, starts[b] - 1:starts[b] - 1 + T] for b in range(B)]).to(DEV)
    say(f"[persistent] ragged starts {starts}")
    _, sa, sb, la, lb, snap_a, snap_b = run_pair(cfg, B, T, binding.RLT_LOGITS_ALL, e,
                                                 (mk.to(DEV), mv.to(DEV)), imports=snap)
    assert torch.isfinite(la).all()
    assert torch.equal(la, lb)
    assert torch.equal(snap_a, snap_b)


def test_persistent_step_small_workload_shape():
    """The small bf16 workload's model and batch (d = 512, 8 heads, 12 layers,
    G = 12, W = 128, B = 64), 24 steps: K split over 2, 4 and 8 wavefronts,
    several GEMM workgroups per persistent workgroup."""
    cfg = SMALL.model
    B, T = SMALL.batch, 24
    say(f"[persistent] small workload B={B} T={T}")
    e = synth.encoder_e(cfg, B, T, device=DEV)
    mk, mv = synth.encoder_memory(cfg, B, T, device=DEV)
    _, sa, sb, la, lb, snap_a, snap_b = run_pair(cfg, B, T, binding.RLT_LOGITS_ALL, e, (mk, mv))
    assert torch.isfinite(la).all()
    say(f"  max |d logit| = {float((la - lb).abs().max()):.3e}")
    assert torch.equal(la, lb)
    assert torch.equal(snap_a, snap_b)


def test_persistent_step_rejects_a_short_workspace():
    cfg = tiny_cfg()
    params = {k: v.to(DEV) for k, v in synth.model_params(cfg, device="cpu").items()}
    model = binding.Model(cfg, params, version=1)
    st = binding.State(model, 2, 4)
    ws = binding.StepWorkspace(model, 2)
    short = binding.StepWorkspace.__new__(binding.StepWorkspace)
    short.buf = ws.buf[:ws.buf.numel() // 2]
    e, mk, mv = inputs(cfg, 2, 4)
    with pytest.raises(binding.RLTError) as ei:
        binding.rlt_run_sequence_persistent(model, st, e.to(DEV), (mk.to(DEV), mv.to(DEV)), short)
    assert ei.value.status == binding.RLT_ERR_SHAPE
    assert st.position(0) == 0


def test_persistent_step_wait_time_out_is_reported_and_cleared():
    """A wait that can never be satisfied, forced from the host (the waits look
    for an epoch no item stores), times out after its 0.2 s bound: the call's
    launches end, rlt_persistent_check reports RLT_ERR_DEVICE, and after a
    reset the next call on the same workspace runs normally, bitwise equal to
    the launch chain."""
    import time
    cfg = tiny_cfg()
    B, T = 4, 6
    e, mk, mv = inputs(cfg, B, T)
    e, mem = e.to(DEV), (mk.to(DEV), mv.to(DEV))
    params = {k: v.to(DEV) for k, v in synth.model_params(cfg, device="cpu").items()}
    model = binding.Model(cfg, params, version=1)
    st = binding.State(model, B, T)
    ws = binding.StepWorkspace(model, B)
    say("[persistent] forced time-out")
    binding.rlt_persistent_test_stall(True)
    try:
        t0 = time.time()
        binding.rlt_run_sequence_persistent(model, st, e, mem, ws)
        with pytest.raises(binding.RLTError) as ei:
            binding.rlt_persistent_check(ws)
        elapsed = time.time() - t0
    finally:
        binding.rlt_persistent_test_stall(False)
    assert ei.value.status == binding.RLT_ERR_DEVICE
    say(f"  reported after {elapsed:.2f} s")
    assert elapsed < 5.0                   # one bounded wait, then every later one returns at once
    binding.rlt_state_reset(model, st, list(range(B)))
    sa = binding.State(model, B, T)
    la = binding.rlt_run_sequence(model, sa, e, mem)
    lb = binding.rlt_run_sequence_persistent(model, st, e, mem, ws)
    binding.rlt_persistent_check(ws)
    torch.cuda.synchronize()
    assert torch.isfinite(la).all()
    assert torch.equal(la, lb)
    for b in range(B):
        assert st.position(b) == T
