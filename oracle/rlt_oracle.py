"""Reference (oracle) implementation of the Recurrent Looped Transformer's
recurrent decoder step, on the CPU, in NumPy.

TEST INFRASTRUCTURE.  This module exists to check the HIP library.  Only the
test suite, the package entry file's smoke check and the benchmark's
CPU-baseline leg may import it; the library and its binding never do, and it
imports nothing of theirs.  It is deliberately plain and slow: one state per
sequence, the decoder cache kept as an explicit list of past keys/values in
logical order (no ring buffer), every attention taken over an explicit index
range.

Pages cited (by title):
  [Tutorial]  "Understanding and Applying the Recurrent Looped Transformer
              Architecture" (aiezz.com tutorial)
  [Princeton] "Princeton Researcher Proposes Recurrent Looped Transformer to
              Carry Decoder State Across Tokens" (ainewsfeed.tech)
  [Article]   "Recurrent Looped Transformer: A New Architecture for Infinite
              Context Reasoning in Language Models" (technologiesdigest.com)
  [Forget]    "What If a Transformer Never Had to Forget? Meet the Recurrent
              Looped Transformer (RLT)" (wpnews.pro)

What one step computes, for a sequence consuming token t (t = 1 is BOS):
  state H_{t-1} = (s_{t-1}, C_{t-1}); H_0 = (s*, empty cache)
      [Tutorial, "How the Architecture Works": the H_t and H_0 equations]
  (s_t, C_t) = D(Merge(e_t, s_{t-1}), M_<=t, C_{t-1}, t)
      [Tutorial, "How the Architecture Works": state-transition equation]
  Merge: a gate mixes e_t with s_{t-1}
      [Princeton, architecture paragraph; Forget, architecture section]
  each decoder block: causal sliding-window self-attention over decoder
  activations, cross-attention to encoder memory, feed-forward network
      [Princeton, architecture paragraph; Article, "The Recurrent Decoder State"]
  the window W counts the current token; W - 1 entries are carried on
      [Tutorial, "Three forms of context" and "Advanced Implementation Tips"]
  memory is read only through the current position t
      [Tutorial, "Three forms of context"]
  logits = W_o RMSNorm_o(s_t)
      [Tutorial, "How the Architecture Works": next-token distribution]

Readings where the pages leave a step open (each also listed in the design
notes of the repository):
  gate      g = sigmoid(W_g [e_t ; s_{t-1}] + b_g) per channel,
            u = g * e_t + (1 - g) * s_{t-1}
  blocks    pre-RMSNorm with residual adds, order SWA -> cross -> FFN (the
            order the pages list them in)
  RMSNorm   x * (mean(x^2) + eps)^(-1/2) * gamma, eps = 1e-6, learned gamma
  positions none beyond the window/memory bounds; attention scale 1/sqrt(dh)
  heads     H heads of dh = d/H for both attentions; memory arrives already
            split per head ([G][seq][H][T][dh]); the decoder owns W_Qc, W_Oc
  groups    G = 1: every layer reads group 0; G = L: layer l reads group l
  FFN       W_2 GELU(W_1 f), GELU in the exact erf form, no biases
  s_t       the residual stream after the last block, before RMSNorm_o
  precision "fp32": fp32 everywhere; "fp64": float64 everywhere;
            "bf16": fp32 arithmetic that rounds to bf16 (nearest even) exactly
            where a bf16 model stores a value: the GEMM inputs (bf16(s) in the
            gate input, the normed activations, attention outputs, FFN hidden),
            q, k, v and q_c.  Residual stream, s_t, softmax and logits stay fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf as _erf, expit as _expit

PRECISIONS = ("fp32", "fp64", "bf16")


def round_bf16(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even), returned as
    fp32.  bf16 keeps the top 16 bits of the fp32 encoding; rounding adds
    0x7FFF plus the lowest kept bit before truncating."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _to_np(x, dt):
    if hasattr(x, "detach"):  # a torch tensor: upcast on the torch side first
        x = x.detach().to("cpu")
        x = x.double() if dt == np.float64 else x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=dt)


class Model:
    """Decoder parameters and dimensions.

    params: mapping with s_star [d], wg [d][2d], bg [d], go [d], wout [V][d]
    and the per-layer stacks g1, g2, g3 [L][d], wq, wk, wv, wo, wqc, woc
    [L][d][d], w1 [L][F][d], w2 [L][d][F] (torch Linear convention W[out][in]).
    Values may be numpy arrays or torch tensors.  `layer_source(l)`, when
    given, returns one layer's mapping on demand instead (for models too large
    to hold as float32 at once)."""

    LAYER_KEYS = ("g1", "g2", "g3", "wq", "wk", "wv", "wo", "wqc", "woc", "w1", "w2")

    def __init__(self, *, d_model, n_heads, n_layers, d_ffn, window, mem_groups, vocab,
                 params=None, precision="fp32", rms_eps=1e-6, layer_source=None, **_ignored):
        if precision not in PRECISIONS:
            raise ValueError(precision)
        self.d, self.H, self.L, self.F = d_model, n_heads, n_layers, d_ffn
        self.dh = d_model // n_heads
        self.W, self.G, self.V = window, mem_groups, vocab
        if self.G not in (1, self.L):
            raise ValueError("memory groups must be 1 or n_layers")
        self.eps = rms_eps
        self.precision = precision
        self.dt = np.float64 if precision == "fp64" else np.float32
        self.bf16 = precision == "bf16"
        dt = self.dt
        self.s_star = _to_np(params["s_star"], dt)
        self.wg = _to_np(params["wg"], dt)
        self.bg = _to_np(params["bg"], dt)
        self.go = _to_np(params["go"], dt)
        self.wout = _to_np(params["wout"], dt)
        self._layer_source = layer_source
        self._layers = None
        if layer_source is None:
            self._layers = [{k: _to_np(params[k][l], dt) for k in self.LAYER_KEYS}
                            for l in range(self.L)]

    def layer(self, l):
        if self._layers is not None:
            return self._layers[l]
        return {k: _to_np(v, self.dt) for k, v in self._layer_source(l).items()}

    # --- elementwise pieces -------------------------------------------------
    # The storage rounding points of a bf16 model (reading: every value a bf16
    # model stores is a bf16 number; accumulation, softmax, the residual
    # stream, s_t and the logits stay fp32).  Each call site of R names its
    # point, so a test can trace every rounded value and drop one point.
    ROUNDING_POINTS = ("gate_s", "norm1", "q", "k", "v", "swa_out", "norm2", "qc",
                       "cross_out", "norm3", "ffn_hidden", "norm_out")

    def R(self, x, point=None):
        """Storage rounding point `point`: bf16 in the bf16 emulation, identity
        otherwise."""
        return round_bf16(x) if self.bf16 else x

    def rms(self, x, gamma):
        """RMSNorm over the last axis with gain gamma (reading: eps = 1e-6)."""
        ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float64).astype(self.dt)
        r = (1.0 / np.sqrt(ms + self.dt(self.eps))).astype(self.dt)
        return (x * r) * gamma

    def gelu(self, x):
        """Exact GELU: x * Phi(x) = x/2 (1 + erf(x / sqrt 2)) (reading)."""
        x64 = x.astype(np.float64)
        return (0.5 * x64 * (1.0 + _erf(x64 / math.sqrt(2.0)))).astype(self.dt)

    def attend(self, q, K, V):
        """Softmax attention of one query per head over explicit entries.

        q [H][dh]; K, V [n][H][dh] -> [H][dh]; scale 1/sqrt(dh)."""
        scale = self.dt(1.0 / math.sqrt(self.dh))
        s = np.einsum("hc,nhc->hn", q, K) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        return np.einsum("hn,nhc->hc", p, V) / p.sum(axis=1, keepdims=True)

    def merge(self, e, s_prev):
        """Gated merge (reading): g = sigmoid(W_g [e ; s] + b_g),
        u = g * e + (1 - g) * s.  The gate input takes bf16(s) in the bf16
        emulation; the mix uses s itself."""
        z = np.concatenate([e, self.R(s_prev, "gate_s")], axis=-1) @ self.wg.T + self.bg
        g = _expit(z).astype(self.dt)
        return g * e + (self.dt(1.0) - g) * s_prev


@dataclass
class SeqState:
    """H = (s, C) of one sequence plus its position (tokens consumed so far).

    K[l], V[l]: [n_hist][H][dh] history of layer l in logical order (oldest
    first), n_hist <= W - 1."""
    s: np.ndarray
    K: list
    V: list
    pos: int = 0
    meta: dict = field(default_factory=dict)


def initial_state(model: Model) -> SeqState:
    """H_0 = (s*, empty cache), set once before BOS
    [Tutorial, "How the Architecture Works"; Princeton, architecture paragraph]."""
    empty = np.zeros((0, model.H, model.dh), dtype=model.dt)
    return SeqState(s=model.s_star.copy(), K=[empty.copy() for _ in range(model.L)],
                    V=[empty.copy() for _ in range(model.L)], pos=0)


def state_from_arrays(model: Model, pos, s, K, V) -> SeqState:
    """A state that has consumed `pos` tokens: s [d], K/V [L][H][n_hist][dh]
    (oldest entry first, n_hist = min(pos, W - 1))."""
    n_hist = min(pos, model.W - 1)
    Kl = [_to_np(K[l], model.dt).transpose(1, 0, 2).copy() for l in range(model.L)]
    Vl = [_to_np(V[l], model.dt).transpose(1, 0, 2).copy() for l in range(model.L)]
    for l in range(model.L):
        if Kl[l].shape[0] != n_hist or Vl[l].shape[0] != n_hist:
            raise ValueError("history length must be min(pos, W-1)")
    return SeqState(s=_to_np(s, model.dt).copy(), K=Kl, V=Vl, pos=int(pos))


def copy_state(st: SeqState) -> SeqState:
    return SeqState(s=st.s.copy(), K=[k.copy() for k in st.K], V=[v.copy() for v in st.V],
                    pos=st.pos, meta=dict(st.meta))


def decoder_step(model: Model, states, e_rows, mem_k, mem_v, mem_index=None, trace=None):
    """Consume one token in each listed sequence; returns logits [n][V].

    states    list of SeqState (updated in place: s, cache, pos += 1)
    e_rows    [n][d] encoder representation e_t of each sequence's token
    mem_k/v   encoder memory [G][S][H][T_cap][dh]; row i reads sequence
              mem_index[i] (default i) at positions 1..t_i
    trace     optional dict collecting per-layer intermediates (for tests)

    Sequences never interact: every row is the same computation on its own
    state; the batch only shares the weight products
    [Princeton, design principles paragraph: batching independent sequences]."""
    m = model
    dt = m.dt
    n = len(states)
    if mem_index is None:
        mem_index = list(range(n))
    t = [st.pos + 1 for st in states]
    for i in range(n):
        if t[i] > mem_k.shape[3]:
            raise ValueError("memory capacity exceeded")
    e = _to_np(e_rows, dt).reshape(n, m.d)
    s_prev = np.stack([st.s for st in states]).astype(dt)
    x = m.merge(e, s_prev)
    if trace is not None:
        trace.setdefault("x0", []).append(x.copy())
    for l in range(m.L):
        P = m.layer(l)
        # (1) causal sliding-window self-attention, window = positions
        #     max(1, t-W+1) .. t, the current token's entry included
        a = m.R(m.rms(x, P["g1"]), "norm1")
        q = m.R(a @ P["wq"].T, "q").reshape(n, m.H, m.dh)
        k = m.R(a @ P["wk"].T, "k").reshape(n, m.H, m.dh)
        v = m.R(a @ P["wv"].T, "v").reshape(n, m.H, m.dh)
        o = np.empty((n, m.H, m.dh), dtype=dt)
        for i, st in enumerate(states):
            Kw = np.concatenate([st.K[l], k[i:i + 1]], axis=0)
            Vw = np.concatenate([st.V[l], v[i:i + 1]], axis=0)
            if not st.meta.get("cache_dropped"):
                assert Kw.shape[0] == min(t[i], m.W)
            o[i] = m.attend(q[i], Kw, Vw)
            # carry the newest W-1 entries into C_t
            first_kept = max(0, Kw.shape[0] - (m.W - 1))
            st.K[l] = Kw[first_kept:].copy()
            st.V[l] = Vw[first_kept:].copy()
        x = x + m.R(o.reshape(n, m.d), "swa_out") @ P["wo"].T
        # (2) cross-attention to encoder memory positions 1..t
        c = m.R(m.rms(x, P["g2"]), "norm2")
        qc = m.R(c @ P["wqc"].T, "qc").reshape(n, m.H, m.dh)
        grp = 0 if m.G == 1 else l
        oc = np.empty((n, m.H, m.dh), dtype=dt)
        for i in range(n):
            Km = _to_np(mem_k[grp, mem_index[i], :, :t[i], :], dt).transpose(1, 0, 2)
            Vm = _to_np(mem_v[grp, mem_index[i], :, :t[i], :], dt).transpose(1, 0, 2)
            oc[i] = m.attend(qc[i], Km, Vm)
        x = x + m.R(oc.reshape(n, m.d), "cross_out") @ P["woc"].T
        # (3) feed-forward network
        f = m.R(m.rms(x, P["g3"]), "norm3")
        h = m.R(m.gelu(f @ P["w1"].T), "ffn_hidden")
        x = x + h @ P["w2"].T
        if trace is not None:
            trace.setdefault("q", []).append(q.copy())
            trace.setdefault("k", []).append(k.copy())
            trace.setdefault("v", []).append(v.copy())
            trace.setdefault("swa", []).append(o.copy())
            trace.setdefault("cross", []).append(oc.copy())
            trace.setdefault("x", []).append(x.copy())
    for i, st in enumerate(states):
        st.s = x[i].copy()
        st.pos += 1
    # next-token logits from s_t [Tutorial, "How the Architecture Works"]
    return m.R(m.rms(x, m.go), "norm_out") @ m.wout.T


def run_sequence(model: Model, states, e, mem_k, mem_v, mem_index=None, steps=None,
                 trace=None):
    """Consume `steps` tokens per sequence with no reset anywhere (prompt and
    response are the same transition) [Article, "The Critical Boundary";
    Tutorial, "Prompt prefill"].  e [n][T][d] -> logits [n][steps][V]."""
    e = np.asarray(e) if not hasattr(e, "detach") else e
    n, T = e.shape[0], e.shape[1]
    steps = T if steps is None else steps
    out = np.empty((n, steps, model.V), dtype=model.dt)
    for j in range(steps):
        out[:, j] = decoder_step(model, states, e[:, j], mem_k, mem_v, mem_index, trace)
    return out


def token_log_prob(logits, token):
    """log p(token) under softmax(logits), in float64: logits[token] minus the
    log of the sum of exp(logits), the maximum taken out first.  A token < 0
    is not scored (0.0)."""
    if token < 0:
        return 0.0
    z = np.asarray(logits, dtype=np.float64)
    zmax = float(np.max(z))
    return float(z[token] - zmax - math.log(float(np.sum(np.exp(z - zmax)))))


def score_sequence(model: Model, states, e, mem_k, mem_v, tokens, mem_index=None):
    """Replay scoring of a recorded sequence under the model as it stands:
    step t consumes token t, and the log-probability of the realized next
    token tokens[i][t] is read from that step's logits, before the token is
    consumed by step t + 1 [Tutorial, "Current-Policy Reinforcement Learning
    Replay": rebuild the states from the start, evaluate an action from the
    preceding state, then consume it once].  e [n][T][d], tokens [n][T] int
    (< 0: not scored) -> log-probabilities [n][T] float64."""
    e = np.asarray(e) if not hasattr(e, "detach") else e
    tok = np.asarray(tokens)
    n, T = tok.shape
    out = np.zeros((n, T), dtype=np.float64)
    for j in range(T):
        lg = decoder_step(model, states, e[:, j], mem_k, mem_v, mem_index)
        for i in range(n):
            out[i, j] = token_log_prob(lg[i], int(tok[i, j]))
    return out


def sampling_weights(logits, temperature, top_k):
    """Weights of the sampling distribution, float64: exp((z - max z) / T) on
    the kept tokens -- those whose logit is at least the top_k-th largest
    (all when top_k >= V) -- and 0 elsewhere."""
    z = np.asarray(logits, dtype=np.float64)
    V = z.size
    keep = np.ones(V, dtype=bool) if top_k >= V else z >= np.sort(z)[::-1][top_k - 1]
    return np.where(keep, np.exp((z - z.max()) / temperature), 0.0), keep


def sample_token(logits, temperature, top_k, u):
    """Token drawn with uniform u by the inverse CDF in token order: the first
    v whose cumulative weight exceeds u times the total.  Returns (token,
    log-probability of it under the sampling distribution)
    [Tutorial, "Autoregressive generation": sample from the distribution;
    Princeton, design principles: record each action's behaviour
    log-probability under the temperature and truncation actually used]."""
    w, keep = sampling_weights(logits, temperature, top_k)
    c = np.cumsum(w)
    total = float(c[-1])
    tok = int(np.searchsorted(c, u * total, side="right"))
    tok = min(tok, int(np.nonzero(keep)[0][-1]))
    z = np.asarray(logits, dtype=np.float64)
    return tok, float((z[tok] - z.max()) / temperature - math.log(total))


def generate(model: Model, states, logits0, table_e, table_k, table_v, mem_k, mem_v, temperature,
             top_k, u, follow=None):
    """Autoregressive generation [Tutorial, "Autoregressive generation"]: for
    every step, sample from the preceding state's logits, record the token and
    its log-probability, encode it with the stand-in tables (e = table_e[x];
    memory entry t of each group = table_k/v[g][x], written into mem_k/mem_v,
    numpy arrays [G][S][H][T][dh]) and consume it once.  follow [n][steps]:
    tokens to take instead of the sampled ones (replaying another
    implementation's choices); the log-probability is then that of the
    followed token.  Returns (tokens, log-probs, logits of the last step)."""
    n = len(states)
    steps = np.asarray(u).shape[1]
    toks = np.zeros((n, steps), dtype=np.int64)
    lps = np.zeros((n, steps), dtype=np.float64)
    logits = np.asarray(logits0, dtype=np.float64)
    te, tk, tv = np.asarray(table_e), np.asarray(table_k), np.asarray(table_v)
    for j in range(steps):
        for i in range(n):
            tok, lp = sample_token(logits[i], temperature, top_k, float(u[i][j]))
            if follow is not None:
                tok = int(follow[i][j])
                z = logits[i]
                w, _ = sampling_weights(z, temperature, top_k)
                lp = float((z[tok] - z.max()) / temperature - math.log(w.sum()))
            toks[i, j], lps[i, j] = tok, lp
        e_rows = te[toks[:, j]]
        for i, st in enumerate(states):
            for g in range(mem_k.shape[0]):
                mem_k[g, i, :, st.pos, :] = tk[g, toks[i, j]]
                mem_v[g, i, :, st.pos, :] = tv[g, toks[i, j]]
        logits = decoder_step(model, states, e_rows, mem_k, mem_v).astype(np.float64)
    return toks, lps, logits
