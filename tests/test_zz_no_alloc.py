"""rlt_decoder_step_noalloc (per-step working memory in the library's static
per-device array) against rlt_decoder_step (working memory in the state),
through the C ABI (needs an MI355X).  Both run the same kernels on the same
launch shapes, so logits and states must agree bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from _tiny import tiny_cfg, inputs
from recurrent_decode_step_amd import binding, synth
from recurrent_decode_step_amd.configs import DTYPE_BF16, DTYPE_FP32

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def pair(cfg, B, T):
    params = {k: v.to(DEV) for k, v in synth.model_params(cfg).items()}
    model = binding.Model(cfg, params, version=1)
    e, mk, mv = inputs(cfg, B, T)
    return model, e.to(DEV), (mk.to(DEV), mv.to(DEV)), binding.State(model, B, T), \
        binding.State(model, B, T)


@pytest.mark.parametrize("dtype", [DTYPE_FP32, DTYPE_BF16])
def test_noalloc_step_matches_decoder_step(dtype):
    """Four calls in a row on two identical states, one through each entry
    point: all 20 rows (a ragged 16-row tail), then a smaller call of 5 rows
    with a slot list, then all rows again at ragged positions (the row-order
    staging), then a single row.  Logits and the exported states agree
    bitwise after every call."""
    cfg = tiny_cfg(dtype=dtype, d_model=128, n_heads=2, d_ffn=512, window=4, vocab=40)
    B, T = 20, 8
    say(f"[noalloc] dtype={dtype} B={B}")
    model, e, mem, sa, sb = pair(cfg, B, T)
    calls = [None, [7, 3, 19, 0, 12], None, [5]]
    pos = [0] * B
    for j, slots in enumerate(calls):
        rows = list(range(B)) if slots is None else slots
        er = torch.stack([e[r, pos[r]] for r in rows]).contiguous()
        la = binding.rlt_decoder_step(model, sa, er, mem, slots=slots)
        lb = torch.full_like(la, float("nan"))
        binding.rlt_decoder_step_noalloc(model, sb, er, mem, lb, slots=slots)
        torch.cuda.synchronize()
        say(f"  call {j}: {len(rows)} rows, max |d| = {float((la - lb).abs().max()):.3e}")
        assert torch.isfinite(la).all()
        assert torch.equal(la, lb), j
        for r in rows:
            pos[r] += 1
        for r in range(B):
            assert sa.position(r) == pos[r] == sb.position(r)
        snap_a = binding.rlt_state_export(model, sa, list(range(B)))
        snap_b = binding.rlt_state_export(model, sb, list(range(B)))
        assert torch.equal(snap_a, snap_b), j


def test_noalloc_rejects_more_rows_than_the_static_array_holds():
    """A call whose working memory exceeds the 16 MiB array fails with
    RLT_ERR_RANGE before any device work: positions and state unchanged."""
    cfg = tiny_cfg(dtype=DTYPE_BF16, d_model=128, n_heads=2, d_ffn=512, window=2, vocab=16)
    B, T = 8000, 2
    params = {k: v.to(DEV) for k, v in synth.model_params(cfg).items()}
    model = binding.Model(cfg, params, version=1)
    mk = torch.zeros((1, B, cfg.n_heads, T, cfg.head_dim), dtype=torch.bfloat16, device=DEV)
    st = binding.State(model, B, T)
    before = binding.rlt_state_export(model, st, [0, B - 1])
    e = torch.zeros((B, cfg.d_model), dtype=torch.bfloat16, device=DEV)
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.RLTError) as ei:
        binding.rlt_decoder_step_noalloc(model, st, e, (mk, mk.clone()), logits)
    assert ei.value.status == binding.RLT_ERR_RANGE
    say(f"[noalloc] {B} rows: {ei.value}")
    torch.cuda.synchronize()
    assert st.position(0) == 0 and st.position(B - 1) == 0
    assert torch.equal(before, binding.rlt_state_export(model, st, [0, B - 1]))
    # the same state then takes a call that fits
    n = 64
    binding.rlt_decoder_step_noalloc(model, st, e[:n].contiguous(), (mk, mk.clone()), logits[:n])
    torch.cuda.synchronize()
    assert st.position(0) == 1 and st.position(n) == 0
    assert torch.isfinite(logits[:n]).all()
