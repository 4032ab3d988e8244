"""Reference (oracle) causal encoder and memory projection, on the CPU.

TEST INFRASTRUCTURE (see the package header for who may import it).

What it computes, for one sequence of tokens x_1..x_T:
  the encoder runs over all tokens at once under a causal mask (position i
  sees positions 1..i) and produces a representation e_t per token
      [Article, "Encoder-Decoder Pairing with Shared Weights" and "Principle 2:
       Co-Design Between Model and Hardware" (token-parallel); Tutorial, "How
       the Architecture Works"; Princeton, architecture paragraph]
  encoder and decoder have the same number of layers, and encoder layer l
  uses the attention and feed-forward weights of decoder layer l
      [Article, "Encoder-Decoder Pairing with Shared Weights"; Princeton,
       architecture paragraph: the tied configuration]
  the memory M_<=t is projected from e_1..e_t, one group shared by every
  decoder layer (G = 1) or one group per decoder layer (G = L)
      [Princeton, architecture paragraph]
  prompt prefill = the encoder over the prompt, then the decoder recurrence
  over every prompt token
      [Tutorial, "Prompt prefill"]

Readings where the pages leave a step open (also listed in the design notes):
  input     a learned token embedding emb [V][d]; no positional encoding (as
            in the decoder)
  blocks    the decoder block without its cross-attention: pre-RMSNorm causal
            self-attention then the GELU FFN, residual adds; the tied weights
            are g1, W_Q, W_K, W_V, W_O, g3, W_1, W_2 of decoder layer l
  mask      full causal (no window): position i attends to 1..i, itself
            included; scale 1/sqrt(dh)
  output    e_t = RMSNorm(x_L; g_e) with the encoder's own gain g_e
  memory    K^g_t = W_Km[g] e_t, V^g_t = W_Vm[g] e_t (no bias), split into H
            heads of dh, stored [G][H][T][dh] like the decoder's memory input
  precision the decoder's rounding points (normed GEMM inputs, q/k/v,
            attention outputs, FFN hidden) plus e_t and the memory entries,
            which a bf16 model stores in bf16
"""
from __future__ import annotations

import numpy as np

from .rlt_oracle import Model, _to_np


class Encoder:
    """Encoder-only parameters next to a decoder Model whose layers it reuses.

    params: emb [V][d], ge [d], wkm, wvm [G][d][d] (torch Linear convention)."""

    def __init__(self, model: Model, params):
        self.m = model
        dt = model.dt
        self.emb = _to_np(params["emb"], dt)
        self.ge = _to_np(params["ge"], dt)
        self.wkm = _to_np(params["wkm"], dt)
        self.wvm = _to_np(params["wvm"], dt)
        if self.wkm.shape[0] != model.G or self.wvm.shape[0] != model.G:
            raise ValueError("one K and one V projection per memory group")


def encode(enc: Encoder, tokens, trace=None):
    """Encode one sequence.  tokens [T] ints in 0..V-1.

    Returns e [T][d], mem_k, mem_v [G][H][T][dh] and the per-layer encoder
    keys/values cache_k, cache_v [L][T][H][dh].  Every position is computed
    from the whole prefix at once, so encoding x_1..x_T and encoding a longer
    sequence that starts with them give the same first T rows."""
    m = enc.m
    dt = m.dt
    tok = np.asarray(tokens, dtype=np.int64).reshape(-1)
    T = tok.size
    if T and (tok.min() < 0 or tok.max() >= m.V):
        raise ValueError("token id outside the vocabulary")
    x = enc.emb[tok].astype(dt).copy()                       # residual stream [T][d]
    cache_k = np.empty((m.L, T, m.H, m.dh), dtype=dt)
    cache_v = np.empty((m.L, T, m.H, m.dh), dtype=dt)
    for l in range(m.L):
        P = m.layer(l)
        # causal self-attention with decoder layer l's weights
        a = m.R(m.rms(x, P["g1"]))
        q = m.R(a @ P["wq"].T).reshape(T, m.H, m.dh)
        k = m.R(a @ P["wk"].T).reshape(T, m.H, m.dh)
        v = m.R(a @ P["wv"].T).reshape(T, m.H, m.dh)
        o = np.empty((T, m.H, m.dh), dtype=dt)
        for i in range(T):
            o[i] = m.attend(q[i], k[:i + 1], v[:i + 1])       # positions 1..i
        x = x + m.R(o.reshape(T, m.d)) @ P["wo"].T
        # feed-forward network with decoder layer l's weights
        f = m.R(m.rms(x, P["g3"]))
        h = m.R(m.gelu(f @ P["w1"].T))
        x = x + h @ P["w2"].T
        cache_k[l], cache_v[l] = k, v
        if trace is not None:
            trace.setdefault("q", []).append(q.copy())
            trace.setdefault("k", []).append(k.copy())
            trace.setdefault("v", []).append(v.copy())
            trace.setdefault("o", []).append(o.copy())
            trace.setdefault("x", []).append(x.copy())
    e = m.R(m.rms(x, enc.ge))
    mem_k = np.empty((m.G, m.H, T, m.dh), dtype=dt)
    mem_v = np.empty((m.G, m.H, T, m.dh), dtype=dt)
    for g in range(m.G):
        mem_k[g] = m.R(e @ enc.wkm[g].T).reshape(T, m.H, m.dh).transpose(1, 0, 2)
        mem_v[g] = m.R(e @ enc.wvm[g].T).reshape(T, m.H, m.dh).transpose(1, 0, 2)
    return {"e": e, "mem_k": mem_k, "mem_v": mem_v, "cache_k": cache_k, "cache_v": cache_v}


def prefill(enc: Encoder, states, tokens, capacity=None):
    """Prompt prefill [Tutorial, "Prompt prefill"]: the encoder over each
    sequence's prompt, then the decoder recurrence over every prompt token (no
    reset, the same transition as decoding).  tokens [n][T]; states are
    decoder states at position 0 (updated in place).  Returns (logits
    [n][T][V], e [n][T][d], mem_k, mem_v [G][n][H][capacity][dh])."""
    from .rlt_oracle import run_sequence
    m = enc.m
    tok = np.asarray(tokens)
    n, T = tok.shape
    cap = capacity or T
    mem_k = np.zeros((m.G, n, m.H, cap, m.dh), dtype=m.dt)
    mem_v = np.zeros((m.G, n, m.H, cap, m.dh), dtype=m.dt)
    e = np.empty((n, T, m.d), dtype=m.dt)
    for i in range(n):
        r = encode(enc, tok[i])
        e[i] = r["e"]
        mem_k[:, i, :, :T] = r["mem_k"]
        mem_v[:, i, :, :T] = r["mem_v"]
    logits = run_sequence(m, states, e, mem_k, mem_v)
    return logits, e, mem_k, mem_v


def generate_encoded(enc: Encoder, states, prompts, logits0, mem_k, mem_v, temperature, top_k, u,
                     follow=None):
    """Autoregressive generation with the causal encoder in the loop
    [Tutorial, "Autoregressive generation": sample from the preceding state's
    distribution, encode the sampled token incrementally, consume it through
    the decoder exactly once].  For every step and sequence: sample with
    uniform u[i][j] (or take follow[i][j]) and record the token and its
    log-probability; the token becomes the next position p of its sequence
    (p = the decoder state's position before the step): e_p and memory entry
    p of every group are the encoder's output at p given the sequence's
    tokens 0..p (the encoder over the whole list; by causality the earlier
    rows are those of the shorter list), written into mem_k/mem_v
    [G][n][H][cap][dh]; then one decoder step consumes e_p.  prompts [n][P]:
    the tokens already encoded and consumed (states at position P).  Returns
    (tokens, log-probs, logits of the last step)."""
    import math
    from .rlt_oracle import decoder_step, sample_token, sampling_weights
    m = enc.m
    n = len(states)
    steps = np.asarray(u).shape[1]
    seqs = [list(int(t) for t in p) for p in np.asarray(prompts)]
    toks = np.zeros((n, steps), dtype=np.int64)
    lps = np.zeros((n, steps), dtype=np.float64)
    logits = np.asarray(logits0, dtype=np.float64)
    for j in range(steps):
        for i in range(n):
            tok, lp = sample_token(logits[i], temperature, top_k, float(u[i][j]))
            if follow is not None:
                tok = int(follow[i][j])
                z = logits[i]
                w, _ = sampling_weights(z, temperature, top_k)
                lp = float((z[tok] - z.max()) / temperature - math.log(w.sum()))
            toks[i, j], lps[i, j] = tok, lp
        e_rows = np.empty((n, m.d), dtype=m.dt)
        for i, st in enumerate(states):
            seqs[i].append(int(toks[i, j]))
            p = len(seqs[i]) - 1
            if st.pos != p:
                raise ValueError("the decoder state must have consumed every encoded token")
            r = encode(enc, seqs[i])
            e_rows[i] = r["e"][p]
            mem_k[:, i, :, p] = r["mem_k"][:, :, p]
            mem_v[:, i, :, p] = r["mem_v"][:, :, p]
        logits = decoder_step(m, states, e_rows, mem_k, mem_v).astype(np.float64)
    return toks, lps, logits
