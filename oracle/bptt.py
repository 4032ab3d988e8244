"""Reference (oracle) backpropagation through time of the recurrent decoder.

TEST INFRASTRUCTURE (see the package header for who may import it).

The forward is the decoder step of rlt_oracle written once more with torch
tensors (float64 by default) so that torch's autograd gives the exact
gradient of the loss; the step's arithmetic and readings are those of
rlt_oracle.decoder_step (gated merge, pre-RMSNorm window self-attention with
the current token in the window, cross-attention to the memory through the
current position, GELU FFN, head on RMSNorm_o(s_t)).

What is differentiated [Article, "Training Methodology"; Tutorial, "Pretraining
and supervised fine-tuning"; Forget, the training passage and its note on
truncated BPTT]:
  loss = sum over sequences b and steps t with target[b][t] >= 0 of
         -log softmax(logits_{b,t})[target[b][t]]
  (full-sequence next-token prediction; a target < 0 removes the loss term
  only, never the state update, so gradients still flow through that step).
  Gradients flow through the recurrent output s_t, through the window cache
  entries (the cross terms of the state-to-state Jacobian) and into e_t and
  the encoder memory.
Truncated BPTT names every detached tensor: with chunk length k, at each
boundary between step k*j and k*j + 1 the listed parts of H = (s, C) are
detached: "s" (the recurrent output), "kv" (every cache entry carried across
the boundary) or both.  The forward values never change.
"""
from __future__ import annotations

import math

import numpy as np
import torch

LAYER_KEYS = ("g1", "g2", "g3", "wq", "wk", "wv", "wo", "wqc", "woc", "w1", "w2")
PARAM_KEYS = ("s_star", "wg", "bg", "go", "wout") + LAYER_KEYS


def _rms(x, g, eps):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g


def _attend(q, K, V, scale):
    """q [H][dh], K/V [n][H][dh] -> [H][dh] (softmax over the n entries)."""
    s = torch.einsum("hc,nhc->hn", q, K) * scale
    p = torch.softmax(s, dim=1)
    return torch.einsum("hn,nhc->hc", p, V)


def forward_loss(params, e, mem_k, mem_v, targets, *, n_heads, window, rms_eps=1e-6,
                 chunk=0, detach=(), return_logits=False):
    """Loss of B sequences run from H_0 over T steps.

    params  dict of torch tensors (canonical layout, see rlt_oracle.Model)
    e       [B][T][d]; mem_k/mem_v [G][B][H][T_cap][dh]; targets [B][T] ints
    chunk   truncation length (0: full BPTT); detach: subset of {"s", "kv"}"""
    P = params
    B, T, d = e.shape
    H = n_heads
    dh = d // H
    L = P["wq"].shape[0]
    G = mem_k.shape[0]
    scale = 1.0 / math.sqrt(dh)
    s = P["s_star"].expand(B, d)
    cacheK = [[[] for _ in range(B)] for _ in range(L)]   # per layer, per sequence: list of [H][dh]
    cacheV = [[[] for _ in range(B)] for _ in range(L)]
    loss = e.new_zeros(())
    all_logits = []
    for t in range(T):
        if chunk and t > 0 and t % chunk == 0:
            # boundary between step t and t + 1 (1-based): cut the named tensors
            if "s" in detach:
                s = s.detach()
            if "kv" in detach:
                cacheK = [[[k.detach() for k in seq] for seq in lay] for lay in cacheK]
                cacheV = [[[v.detach() for v in seq] for seq in lay] for lay in cacheV]
        et = e[:, t]
        z = torch.cat([et, s], dim=-1) @ P["wg"].T + P["bg"]
        g = torch.sigmoid(z)
        x = g * et + (1 - g) * s
        for l in range(L):
            a = _rms(x, P["g1"][l], rms_eps)
            q = (a @ P["wq"][l].T).reshape(B, H, dh)
            k = (a @ P["wk"][l].T).reshape(B, H, dh)
            v = (a @ P["wv"][l].T).reshape(B, H, dh)
            outs = []
            for b in range(B):
                cacheK[l][b].append(k[b])
                cacheV[l][b].append(v[b])
                cacheK[l][b] = cacheK[l][b][-window:]
                cacheV[l][b] = cacheV[l][b][-window:]
                outs.append(_attend(q[b], torch.stack(cacheK[l][b]), torch.stack(cacheV[l][b]), scale))
            o = torch.stack(outs).reshape(B, d)
            x = x + o @ P["wo"][l].T
            c = _rms(x, P["g2"][l], rms_eps)
            qc = (c @ P["wqc"][l].T).reshape(B, H, dh)
            grp = 0 if G == 1 else l
            oc = torch.stack([_attend(qc[b], mem_k[grp, b, :, :t + 1].transpose(0, 1),
                                      mem_v[grp, b, :, :t + 1].transpose(0, 1), scale)
                              for b in range(B)]).reshape(B, d)
            x = x + oc @ P["woc"][l].T
            f = _rms(x, P["g3"][l], rms_eps)
            h = torch.nn.functional.gelu(f @ P["w1"][l].T, approximate="none")
            x = x + h @ P["w2"][l].T
        s = x
        logits = _rms(s, P["go"], rms_eps) @ P["wout"].T
        if return_logits:
            all_logits.append(logits)
        tg = torch.as_tensor(np.asarray(targets)[:, t], dtype=torch.long)
        keep = tg >= 0
        if bool(keep.any()):
            lp = torch.log_softmax(logits, dim=-1)
            loss = loss - lp[keep, tg[keep]].sum()
    if return_logits:
        return loss, torch.stack(all_logits, dim=1)
    return loss


def gradients(params, e, mem_k, mem_v, targets, *, n_heads, window, rms_eps=1e-6, chunk=0,
              detach=(), dtype=torch.float64):
    """Loss and its gradient w.r.t. every parameter, e and the memory.

    Inputs may be numpy arrays or torch tensors; everything is converted to
    `dtype` on the CPU.  Returns (loss, {name: grad}, de, dmem_k, dmem_v)."""
    def leaf(x):
        t = torch.as_tensor(np.asarray(x.detach().cpu() if hasattr(x, "detach") else x)).to(dtype)
        return t.clone().requires_grad_(True)
    P = {k: leaf(params[k]) for k in PARAM_KEYS}
    E, MK, MV = leaf(e), leaf(mem_k), leaf(mem_v)
    loss = forward_loss(P, E, MK, MV, targets, n_heads=n_heads, window=window, rms_eps=rms_eps,
                        chunk=chunk, detach=detach)
    names = list(PARAM_KEYS)
    if not loss.requires_grad:          # every target masked: no loss term at all
        grads = [None] * (len(names) + 3)
    else:
        grads = torch.autograd.grad(loss, [P[k] for k in names] + [E, MK, MV], allow_unused=True)
    out = {}
    for k, gr in zip(names, grads[:len(names)]):
        out[k] = (torch.zeros_like(P[k]) if gr is None else gr).numpy()
    rest = [(torch.zeros_like(x) if gr is None else gr).numpy()
            for x, gr in zip((E, MK, MV), grads[len(names):])]
    return float(loss.detach()), out, rest[0], rest[1], rest[2]
