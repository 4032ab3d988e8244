"""Token-parallel sliding-window pass: the negative control for the recurrence.

TEST INFRASTRUCTURE (see the package header for who may import it).

The pages state that no exact parallel scan is known for the nonlinear decoder
recurrence and that an ordinary parallel sliding-window attention pass over the
same weights is not equivalent to it
[Article, "Principle 2: Co-Design Between Model and Hardware";
 Princeton, design principles paragraph].  They do not define that pass.
Reading: the same blocks evaluated for all tokens at once, self-attention under
a band-causal mask of width W (token t sees t-W+1..t), memory read causally
(1..t), and, because s_{t-1} does not exist before the pass has run, every
token merges its e_t with the start state s*.  When the gate is pinned to 1
(no feedback), this pass and the recurrence coincide.
"""
from __future__ import annotations

import numpy as np

from .rlt_oracle import Model, _to_np


def parallel_swa_pass(model: Model, e, mem_k, mem_v):
    """Logits [T][V] of one sequence, all T tokens in parallel.

    e [T][d]; mem_k/mem_v [G][H][T_cap][dh] (this sequence's memory)."""
    m = model
    dt = m.dt
    e = _to_np(e, dt)
    T = e.shape[0]
    MK, MV = _to_np(mem_k, dt), _to_np(mem_v, dt)
    x = m.merge(e, np.broadcast_to(m.s_star, e.shape).copy())
    idx = np.arange(T)
    band = (idx[None, :] <= idx[:, None]) & (idx[None, :] > idx[:, None] - m.W)
    causal = idx[None, :] <= idx[:, None]
    scale = dt(1.0 / np.sqrt(m.dh))

    def masked_attention(Q, K, V, mask):
        # Q [T][H][dh], K/V [S][H][dh], mask [T][S]
        sc = np.einsum("thc,shc->hts", Q, K) * scale
        sc = np.where(mask[None], sc, -np.inf)
        sc = sc - sc.max(axis=2, keepdims=True)
        p = np.exp(sc)
        o = np.einsum("hts,shc->thc", p, V) / p.sum(axis=2)[..., None].transpose(1, 0, 2)
        return o.reshape(T, m.d)

    for l in range(m.L):
        P = m.layer(l)
        a = m.R(m.rms(x, P["g1"]))
        Q = m.R(a @ P["wq"].T).reshape(T, m.H, m.dh)
        K = m.R(a @ P["wk"].T).reshape(T, m.H, m.dh)
        V = m.R(a @ P["wv"].T).reshape(T, m.H, m.dh)
        x = x + m.R(masked_attention(Q, K, V, band)) @ P["wo"].T
        c = m.R(m.rms(x, P["g2"]))
        Qc = m.R(c @ P["wqc"].T).reshape(T, m.H, m.dh)
        grp = 0 if m.G == 1 else l
        Km = MK[grp, :, :T, :].transpose(1, 0, 2)
        Vm = MV[grp, :, :T, :].transpose(1, 0, 2)
        x = x + m.R(masked_attention(Qc, Km, Vm, causal)) @ P["woc"].T
        f = m.R(m.rms(x, P["g3"]))
        x = x + m.R(m.gelu(f @ P["w1"].T)) @ P["w2"].T
    return m.R(m.rms(x, m.go)) @ m.wout.T
