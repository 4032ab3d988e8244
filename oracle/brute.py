"""Brute-force float64 transcription of the decoder recurrence (tiny inputs).

TEST INFRASTRUCTURE (see the package header for who may import it).

Written independently of the cached oracle in rlt_oracle.py, with no decoder
cache at all: it records the residual stream that entered every layer at every
past token, and at each step recomputes every key and value it needs from
those records, with the window and memory ranges written out as explicit
1-based index ranges and every softmax as a Python loop.  It therefore checks
the cache bookkeeping (append, trim, window length, memory bound) of the
cached oracle, and, via the tests, of everything downstream.

Equations followed, by page:
  [Tutorial] "Understanding and Applying the Recurrent Looped Transformer
  Architecture", "How the Architecture Works" (state, initial state, state
  transition, next-token distribution) and "Three forms of context" (window
  includes the current token; memory read through the current position).
  [Princeton] "Princeton Researcher Proposes Recurrent Looped Transformer to
  Carry Decoder State Across Tokens", architecture paragraph (gated merge, block
  contents, groups G = 1 / G = L_D).
Readings (gate, norm, GELU, block order) are the same as the cached oracle's.
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.array(x, dtype=np.float64)


def brute_force_run(cfg: dict, params: dict, e, mem_k, mem_v, T: int, start=None):
    """Logits [T][V] of one sequence consuming tokens 1..T from H_0.

    cfg: d_model, n_heads, n_layers, window, mem_groups, rms_eps
    e [T][d]; mem_k, mem_v [G][H][T_cap][dh] (this sequence's memory)."""
    d = cfg["d_model"]
    H = cfg["n_heads"]
    dh = d // H
    L = cfg["n_layers"]
    W = cfg["window"]
    G = cfg["mem_groups"]
    eps = cfg.get("rms_eps", 1e-6)
    P = {k: _f64(v) for k, v in params.items()}
    e = _f64(e)
    MK, MV = _f64(mem_k), _f64(mem_v)

    def norm(vec, gain):
        mean_sq = sum(float(c) * float(c) for c in vec) / len(vec)
        return vec / math.sqrt(mean_sq + eps) * gain

    def softmax_mix(query, keys, values):
        # query [dh]; keys/values: lists of [dh] vectors
        logit = [float(np.dot(query, kk)) / math.sqrt(dh) for kk in keys]
        top = max(logit)
        wts = [math.exp(z - top) for z in logit]
        tot = sum(wts)
        out = np.zeros(dh)
        for wj, vv in zip(wts, values):
            out += (wj / tot) * vv
        return out

    # layer_in[l][j] = residual stream entering layer l at token j (1-based)
    layer_in = [dict() for _ in range(L)]
    s = P["s_star"].copy()
    logits = np.zeros((T, P["wout"].shape[0]))
    for t in range(1, T + 1):
        et = e[t - 1]
        zz = P["wg"] @ np.concatenate([et, s]) + P["bg"]
        gate = np.array([1.0 / (1.0 + math.exp(-z)) if z > -700 else 0.0 for z in zz])
        x = gate * et + (1.0 - gate) * s
        for l in range(L):
            layer_in[l][t] = x.copy()
            g1, g2, g3 = P["g1"][l], P["g2"][l], P["g3"][l]
            qv = P["wq"][l] @ norm(x, g1)
            first = max(1, t - W + 1)
            sa = np.zeros(d)
            for h in range(H):
                sl = slice(h * dh, (h + 1) * dh)
                keys, vals = [], []
                for j in range(first, t + 1):           # positions first..t inclusive
                    aj = norm(layer_in[l][j], g1)
                    keys.append((P["wk"][l] @ aj)[sl])
                    vals.append((P["wv"][l] @ aj)[sl])
                sa[sl] = softmax_mix(qv[sl], keys, vals)
            x = x + P["wo"][l] @ sa
            qc = P["wqc"][l] @ norm(x, g2)
            grp = 0 if G == 1 else l
            ca = np.zeros(d)
            for h in range(H):
                sl = slice(h * dh, (h + 1) * dh)
                keys = [MK[grp, h, j - 1] for j in range(1, t + 1)]   # memory 1..t
                vals = [MV[grp, h, j - 1] for j in range(1, t + 1)]
                ca[sl] = softmax_mix(qc[sl], keys, vals)
            x = x + P["woc"][l] @ ca
            pre = P["w1"][l] @ norm(x, g3)
            hid = np.array([0.5 * u * (1.0 + math.erf(u / math.sqrt(2.0))) for u in pre])
            x = x + P["w2"][l] @ hid
        s = x
        logits[t - 1] = P["wout"] @ norm(s, P["go"])
    return logits
