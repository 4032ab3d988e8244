"""rlt_run_sequence_fused: the whole run of each slot in one workgroup (small
fp32 models), its memory held in LDS for the call or staged in chunks.
Checked against the CPU oracle (max |d logit| <= 1e-4, the
fp32 gate), for bitwise invariance to splitting a run into calls, for
continuing states the launch chain left (ragged positions included), for
its logits modes, and for its refusal of models it does not take."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _tiny import tiny_cfg, make_model, inputs
from recurrent_decode_step_amd import binding, synth
from recurrent_decode_step_amd.configs import DTYPE_BF16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def say(msg):
    print(msg, flush=True)


class Rig:
    def __init__(self, cfg, B, T):
        self.cfg, self.B, self.T = cfg, B, T
        self.params = synth.model_params(cfg)
        self.e, self.mk, self.mv = inputs(cfg, B, T, T)
        self.model = binding.Model(cfg, {k: v.to(DEV) for k, v in self.params.items()}, version=1)
        self.mem = (self.mk.to(DEV), self.mv.to(DEV))
        self.mk_np, self.mv_np = self.mk.float().numpy(), self.mv.float().numpy()
        self.ed = self.e.to(DEV)

    def state(self):
        return binding.State(self.model, self.B, self.T)

    def oracle_rows(self, lengths):
        """Logits of slot b over its first lengths[b] tokens, from H_0."""
        m, _ = make_model(self.cfg, params=self.params, precision="fp32")
        out = []
        for b, n in enumerate(lengths):
            st = [oracle.initial_state(m)]
            out.append(oracle.run_sequence(m, st, self.e[[b], :n], self.mk_np, self.mv_np,
                                           mem_index=[b])[0])
        return out


CASES = {
    "tiny": (dict(), 4, 64),                        # the tiny fp32 workload: B = 4, T = 64
    "window1": (dict(window=1), 3, 20),
    "window2": (dict(window=2), 3, 20),
    "window-over-T": (dict(window=24), 2, 20),
    "L3-G3-F32": (dict(n_layers=3, mem_groups=3, d_ffn=32), 3, 24),
    "H1-dh32": (dict(n_heads=1), 2, 20),
    "B64": (dict(), 64, 12),                        # one workgroup per slot, 64 of them
    # one memory group but too many positions to hold in LDS: staged in chunks
    "G1-staged": (dict(), 2, 120),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_run_matches_oracle(name):
    kw, B, T = CASES[name]
    cfg = tiny_cfg(**kw)
    assert binding.fused_supported(cfg)
    say(f"[fused parity] case={name} cfg={kw} B={B} T={T}")
    rig = Rig(cfg, B, T)
    st = rig.state()
    got = binding.rlt_run_sequence_fused(rig.model, st, rig.ed, rig.mem).cpu().numpy()
    ref = np.stack(rig.oracle_rows([T] * B))
    err = float(np.max(np.abs(got - ref)))
    say(f"  max|dlogit| = {err:.3e}")
    assert err <= 1e-4
    for b in range(B):
        assert st.position(b) == T


def test_fused_split_is_bitwise_invisible():
    """run(T) == run(k) + run(T - k), logits and the state left behind."""
    cfg = tiny_cfg()
    B, T = 4, 40
    rig = Rig(cfg, B, T)
    st = rig.state()
    full = binding.rlt_run_sequence_fused(rig.model, st, rig.ed, rig.mem).cpu()
    snap_full = binding.rlt_state_export(rig.model, st, list(range(B))).cpu()
    for k in (1, cfg.window - 1, cfg.window, 17):
        say(f"[fused split] k={k}")
        st2 = rig.state()
        a = binding.rlt_run_sequence_fused(rig.model, st2, rig.ed[:, :k], rig.mem).cpu()
        b = binding.rlt_run_sequence_fused(rig.model, st2, rig.ed[:, k:], rig.mem).cpu()
        assert torch.equal(torch.cat([a, b], 1), full)
        assert torch.equal(binding.rlt_state_export(rig.model, st2, list(range(B))).cpu(), snap_full)


def test_fused_continues_ragged_chain_states():
    """The launch chain takes every slot k steps and slots 0 and 2 r more
    (ragged positions); the fused run then takes T2 steps of every slot from
    where each stands; then the chain takes one more step.  All against the
    oracle run of each slot over its own tokens."""
    cfg = tiny_cfg()
    B, k, r, T2 = 4, 9, 5, 12
    T = k + r + T2 + 1
    rig = Rig(cfg, B, T)
    st = rig.state()
    binding.rlt_run_sequence(rig.model, st, rig.ed[:, :k], rig.mem,
                             logits_mode=binding.RLT_LOGITS_NONE)
    fast = [0, 2]
    for j in range(r):
        binding.rlt_decoder_step(rig.model, st, rig.ed[fast, k + j], rig.mem, slots=fast)
    start = [st.position(b) for b in range(B)]
    assert start == [k + r, k, k + r, k]
    e2 = torch.stack([rig.ed[b, start[b]:start[b] + T2] for b in range(B)])
    got = binding.rlt_run_sequence_fused(rig.model, st, e2, rig.mem).cpu().numpy()
    e3 = torch.stack([rig.ed[b, start[b] + T2] for b in range(B)])
    last = binding.rlt_decoder_step(rig.model, st, e3, rig.mem).cpu().numpy()
    ref = rig.oracle_rows([s + T2 + 1 for s in start])
    err = max(float(np.max(np.abs(got[b] - ref[b][start[b]:start[b] + T2]))) for b in range(B))
    err_last = max(float(np.max(np.abs(last[b] - ref[b][-1]))) for b in range(B))
    say(f"[fused after chain] starts={start} max|dlogit| fused {err:.3e}, chain after {err_last:.3e}")
    assert err <= 1e-4 and err_last <= 1e-4
    for b in range(B):
        assert st.position(b) == start[b] + T2 + 1


def test_fused_logits_modes():
    cfg = tiny_cfg()
    B, T = 3, 16
    rig = Rig(cfg, B, T)
    full = binding.rlt_run_sequence_fused(rig.model, rig.state(), rig.ed, rig.mem).cpu()
    last = binding.rlt_run_sequence_fused(rig.model, rig.state(), rig.ed, rig.mem,
                                          logits_mode=binding.RLT_LOGITS_LAST).cpu()
    assert torch.equal(last, full[:, -1])
    st = rig.state()
    out = binding.rlt_run_sequence_fused(rig.model, st, rig.ed, rig.mem,
                                         logits_mode=binding.RLT_LOGITS_NONE)
    assert out is None
    st_ref = rig.state()
    binding.rlt_run_sequence_fused(rig.model, st_ref, rig.ed, rig.mem)
    rows = list(range(B))
    assert torch.equal(binding.rlt_state_export(rig.model, st, rows).cpu(),
                       binding.rlt_state_export(rig.model, st_ref, rows).cpu())


def test_fused_rejects_unsupported_models_without_side_effects():
    cfg = tiny_cfg(dtype=DTYPE_BF16)
    assert not binding.fused_supported(cfg)
    rig = Rig(cfg, 2, 4)
    st = rig.state()
    with pytest.raises(binding.RLTError) as ei:
        binding.rlt_run_sequence_fused(rig.model, st, rig.ed, rig.mem)
    assert ei.value.status == binding.RLT_ERR_UNSUPPORTED
    assert st.position(0) == 0 and st.position(1) == 0
