"""Pins of the CPU oracle's backpropagation through time (no GPU).

Titles of the pages cited:
  [Article]   Recurrent Looped Transformer: A New Architecture for Infinite Context
              Reasoning in Language Models
  [Tutorial]  Understanding and Applying the Recurrent Looped Transformer Architecture
  [Forget]    What If a Transformer Never Had to Forget? Meet the Recurrent Looped
              Transformer (RLT)
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import bptt
from _tiny import oracle_kwargs
from recurrent_decode_step_amd import synth
from recurrent_decode_step_amd.configs import ModelConfig


def micro(G=1, W=3, L=2):
    return ModelConfig(vocab=11, d_model=16, n_heads=2, n_layers=L, d_ffn=32, window=W,
                       mem_groups=G, dtype=0)


def inputs(cfg, B=2, T=6, seed=0):
    params = synth.model_params(cfg)
    # larger weights than the synthetic default so every path carries a visible gradient
    params = {k: (v * 10.0 if k.startswith("w") else v) for k, v in params.items()}
    e = synth.encoder_e(cfg, B, T)
    mk, mv = synth.encoder_memory(cfg, B, T)
    tg = synth.token_ids(B, T, cfg.vocab, index=seed)
    return params, e, mk, mv, tg


def grads(cfg, params, e, mk, mv, tg, **kw):
    return bptt.gradients(params, e, mk, mv, tg, n_heads=cfg.n_heads, window=cfg.window,
                          rms_eps=cfg.rms_eps, **kw)


def test_torch_forward_matches_numpy_oracle():
    """The differentiable forward is the decoder step of the NumPy oracle: logits of
    every step agree in float64 (ties the two implementations to each other)."""
    for G in (1, 2):
        cfg = micro(G=G)
        params, e, mk, mv, tg = inputs(cfg, T=7)
        P = {k: torch.as_tensor(v.numpy(), dtype=torch.float64) for k, v in params.items()}
        _, logits = bptt.forward_loss(P, torch.as_tensor(e.numpy(), dtype=torch.float64),
                                      torch.as_tensor(mk.numpy(), dtype=torch.float64),
                                      torch.as_tensor(mv.numpy(), dtype=torch.float64), tg,
                                      n_heads=cfg.n_heads, window=cfg.window, return_logits=True)
        om = oracle.Model(params=params, precision="fp64", **oracle_kwargs(cfg))
        states = [oracle.initial_state(om) for _ in range(2)]
        ref = oracle.run_sequence(om, states, e.numpy().astype(np.float64), mk.numpy(), mv.numpy())
        np.testing.assert_allclose(logits.detach().numpy(), ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("G", [1, 2])
def test_gradients_match_central_differences(G):
    """The gradient is the derivative: for random directions v in every parameter
    group, e and the memory, (L(x + eps v) - L(x - eps v)) / (2 eps) equals
    <grad, v> (float64, eps = 1e-6)."""
    cfg = micro(G=G)
    params, e, mk, mv, tg = inputs(cfg)
    loss, gp, de, dmk, dmv = grads(cfg, params, e, mk, mv, tg)
    rng = np.random.default_rng(11)
    base = {k: params[k].numpy().astype(np.float64) for k in bptt.PARAM_KEYS}
    X = {"e": e.numpy().astype(np.float64), "mk": mk.numpy().astype(np.float64),
         "mv": mv.numpy().astype(np.float64)}
    gx = {"e": de, "mk": dmk, "mv": dmv}

    def L_at(pp, xx):
        return grads(cfg, pp, xx["e"], xx["mk"], xx["mv"], tg)[0]

    eps = 1e-6
    for name in list(bptt.PARAM_KEYS) + ["e", "mk", "mv"]:
        src = base if name in base else X
        v = rng.standard_normal(src[name].shape)
        plus = {**src, name: src[name] + eps * v}
        minus = {**src, name: src[name] - eps * v}
        if src is base:
            fd = (L_at(plus, X) - L_at(minus, X)) / (2 * eps)
            an = float((gp[name] * v).sum())
        else:
            fd = (L_at(base, plus) - L_at(base, minus)) / (2 * eps)
            an = float((gx[name] * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
    assert loss > 0


def masked_late(tg, k):
    t = np.array(tg, copy=True)
    t[:, :k] = -1
    return t


def test_detaching_both_state_parts_cuts_every_cross_chunk_path():
    """Truncated BPTT with s and the cache both detached at the boundary after
    step 3: the loss of later steps has exactly zero gradient w.r.t. the e of
    steps 1..3 [Forget, truncated-BPTT note: a complete detach needs both parts]."""
    cfg = micro(W=3)
    params, e, mk, mv, tg = inputs(cfg, T=6)
    _, _, de, _, _ = grads(cfg, params, e, mk, mv, masked_late(tg, 3), chunk=3, detach=("s", "kv"))
    assert np.all(de[:, :3] == 0.0)
    assert np.abs(de[:, 3:]).max() > 0


@pytest.mark.parametrize("kept", ["s", "kv"])
def test_detaching_one_state_part_leaves_the_other_path(kept):
    """Detaching only s leaves the gradient path through the window cache, and
    detaching only the cache leaves the path through s [Article, "Training
    Methodology": cross terms through the key-value cache; Forget, truncated-BPTT
    note]."""
    cfg = micro(W=3)
    params, e, mk, mv, tg = inputs(cfg, T=6)
    cut = ("kv",) if kept == "s" else ("s",)
    _, _, de, _, _ = grads(cfg, params, e, mk, mv, masked_late(tg, 3), chunk=3, detach=cut)
    assert np.abs(de[:, :3]).max() > 1e-8


def test_window_one_has_no_cache_path():
    """With W = 1 the cache carries nothing across steps (the window is the
    current token), so detaching s alone already cuts every cross-chunk path."""
    cfg = micro(W=1)
    params, e, mk, mv, tg = inputs(cfg, T=6)
    _, _, de, _, _ = grads(cfg, params, e, mk, mv, masked_late(tg, 3), chunk=3, detach=("s",))
    assert np.all(de[:, :3] == 0.0)


def test_masked_targets_remove_the_loss_not_the_state_path():
    """Loss masking removes loss terms only [Article, "Training Methodology";
    Tutorial, "Pretraining and supervised fine-tuning"]:
    with the targets of steps 1..4 masked, their e still receive gradient from
    the later losses; with every target masked the loss and all gradients are 0."""
    cfg = micro()
    params, e, mk, mv, tg = inputs(cfg, T=6)
    loss, gp, de, _, _ = grads(cfg, params, e, mk, mv, masked_late(tg, 4))
    assert np.abs(de[:, :4]).max() > 1e-8
    loss0, gp0, de0, dmk0, _ = grads(cfg, params, e, mk, mv, np.full_like(tg, -1))
    assert loss0 == 0.0
    assert all(np.all(g == 0) for g in gp0.values()) and np.all(de0 == 0) and np.all(dmk0 == 0)


def test_memory_gradient_is_causal():
    """Step t reads memory positions 1..t only: with only the first 2 targets
    unmasked, memory positions 3.. get no gradient, and future e none either."""
    cfg = micro()
    params, e, mk, mv, tg = inputs(cfg, T=6)
    t = np.full_like(tg, -1)
    t[:, :2] = tg[:, :2]
    _, _, de, dmk, dmv = grads(cfg, params, e, mk, mv, t)
    assert np.all(dmk[:, :, :, 2:] == 0) and np.all(dmv[:, :, :, 2:] == 0)
    assert np.all(de[:, 2:] == 0)
    assert np.abs(dmk[:, :, :, :2]).max() > 0
