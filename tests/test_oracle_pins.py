"""Pins of the CPU oracle to facts the pages and mathematics fix (no GPU).

Each test names the page passage (by title and section) or the mathematical
fact it checks.  Titles:
  [Tutorial]  Understanding and Applying the Recurrent Looped Transformer Architecture
  [Princeton] Princeton Researcher Proposes Recurrent Looped Transformer to Carry
              Decoder State Across Tokens
  [Article]   Recurrent Looped Transformer: A New Architecture for Infinite Context
              Reasoning in Language Models
  [Forget]    What If a Transformer Never Had to Forget? Meet the Recurrent Looped
              Transformer (RLT)
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle
from _tiny import tiny_cfg, make_model, inputs, np64, gate_pinned, oracle_kwargs
from recurrent_decode_step_amd import synth

def run_oracle(model, e, mk, mv, rows=None, steps=None, trace=None):
    n = e.shape[0] if rows is None else len(rows)
    rows = list(range(n)) if rows is None else rows
    states = [oracle.initial_state(model) for _ in rows]
    ee = e[rows]
    out = oracle.run_sequence(model, states, ee, mk, mv, mem_index=rows, steps=steps,
                              trace=trace)
    return out, states


# ---------------------------------------------------------------- rounding
def test_round_bf16_known_values_and_library():
    # exact ties go to even; halfway above rounds up; representable values stay
    one = np.float32(1.0)
    ulp = 2.0 ** -7                   # bf16 spacing at 1.0
    vals = np.array([1.0, 1.0 + ulp / 2, 1.0 + 3 * ulp / 2, 1.0 + ulp / 2 + 2 ** -20,
                     -2.5, 3.0e-3, 65504.0, 1e30], dtype=np.float32)
    want = np.array([1.0, 1.0, 1.0 + 2 * ulp, 1.0 + ulp, -2.5], dtype=np.float32)
    got = oracle.round_bf16(vals)
    np.testing.assert_array_equal(got[:5], want)
    # library routine: torch's fp32 -> bf16 conversion is round-to-nearest-even
    x = torch.randn(100000, generator=torch.Generator().manual_seed(5)) * 7.0
    ref = x.to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.numpy()), ref)
    assert got.dtype == np.float32 and one == 1.0


# -------------------------------------------------------- elementwise pieces
def test_rms_gelu_against_library():
    cfg = tiny_cfg()
    model, _ = make_model(cfg, precision="fp64")
    x = torch.randn(5, cfg.d_model, dtype=torch.float64, generator=torch.Generator().manual_seed(1))
    g = 1 + 0.1 * torch.randn(cfg.d_model, dtype=torch.float64, generator=torch.Generator().manual_seed(2))
    ref = F.rms_norm(x, (cfg.d_model,), weight=g, eps=1e-6).numpy()
    np.testing.assert_allclose(model.rms(x.numpy(), g.numpy()), ref, rtol=1e-13, atol=1e-14)
    # a constant vector c*1 with unit gain normalises to c / sqrt(c^2 + eps)
    c = -3.0
    got = model.rms(np.full((1, 8), c), np.ones(8))
    np.testing.assert_allclose(got, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    # exact (erf) GELU, not the tanh approximation
    u = torch.linspace(-6, 6, 97, dtype=torch.float64)
    np.testing.assert_allclose(model.gelu(u.numpy()), F.gelu(u, approximate="none").numpy(),
                               rtol=1e-14, atol=1e-15)
    assert np.max(np.abs(model.gelu(u.numpy()) - F.gelu(u, approximate="tanh").numpy())) > 1e-4


def test_attend_single_entry_and_uniform():
    cfg = tiny_cfg()
    model, _ = make_model(cfg, precision="fp64")
    H, dh = cfg.n_heads, cfg.head_dim
    rng = np.random.default_rng(0)
    q = rng.standard_normal((H, dh))
    K = rng.standard_normal((1, H, dh))
    V = rng.standard_normal((1, H, dh))
    np.testing.assert_array_equal(model.attend(q, K, V), V[0])
    # zero query: uniform weights -> the mean of the values
    K = rng.standard_normal((7, H, dh))
    V = rng.standard_normal((7, H, dh))
    np.testing.assert_allclose(model.attend(np.zeros((H, dh)), K, V), V.mean(axis=0), rtol=1e-13)


# ------------------------------------------------------------ brute force (P1)
@pytest.mark.parametrize("W,L,G,H,T", [
    (8, 2, 1, 2, 24),      # the tiny workload's model, three windows deep
    (1, 2, 1, 2, 10),
    (2, 3, 3, 2, 12),
    (3, 1, 1, 1, 12),
    (40, 2, 2, 2, 16),     # W >= T
])
def test_oracle_matches_brute_force(W, L, G, H, T):
    """Cached oracle vs the cache-free float64 transcription.

    [Tutorial, "How the Architecture Works" and "Three forms of context"]"""
    cfg = tiny_cfg(window=W, n_layers=L, mem_groups=G, n_heads=H)
    m64, params = make_model(cfg, precision="fp64")
    m32, _ = make_model(cfg, params=params, precision="fp32")
    e, mk, mv = inputs(cfg, 2, T)
    kw = dict(d_model=cfg.d_model, n_heads=H, n_layers=L, window=W, mem_groups=G,
              rms_eps=cfg.rms_eps)
    for b in range(2):
        ref = oracle.brute_force_run(kw, params, e[b], mk[:, b], mv[:, b], T)
        got64, _ = run_oracle(m64, e, mk, mv, rows=[b])
        got32, _ = run_oracle(m32, e, mk, mv, rows=[b])
        np.testing.assert_allclose(got64[0], ref, rtol=0, atol=1e-11)
        assert np.max(np.abs(got32[0] - ref)) <= 1e-5


def test_ragged_batch_matches_brute_force():
    """Sequences at different positions stepped in one batch (P1, ragged)."""
    cfg = tiny_cfg()
    m64, params = make_model(cfg, precision="fp64")
    T = 20
    e, mk, mv = inputs(cfg, 3, T)
    states = [oracle.initial_state(m64) for _ in range(3)]
    starts = [0, 5, 11]
    for b, k in enumerate(starts):          # advance each alone to its start
        for j in range(k):
            oracle.decoder_step(m64, [states[b]], e[b:b + 1, j], mk, mv, mem_index=[b])
    got = np.empty((3, T - max(starts), cfg.vocab))
    for j in range(T - max(starts)):
        rows = [e[b, starts[b] + j] for b in range(3)]
        got[:, j] = oracle.decoder_step(m64, states, torch.stack(rows), mk, mv)
    kw = oracle_kwargs(cfg)
    for b in range(3):
        ref = oracle.brute_force_run(kw, params, e[b], mk[:, b], mv[:, b], T)
        np.testing.assert_allclose(got[b], ref[starts[b]:starts[b] + T - max(starts)],
                                   rtol=0, atol=1e-11)


# ------------------------------------------- W >= T is full causal attention (P2)
def torch_causal_transformer(cfg, params, e, mk, mv):
    """Token-parallel pre-norm transformer built from torch library routines
    (rms_norm, linear, scaled_dot_product_attention with is_causal, exact gelu).
    Equal to the recurrence when the gate is 1 and the window covers the run."""
    d, H, dh, eps = cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.rms_eps
    P = {k: v.double() for k, v in params.items()}
    x = e.double()
    T = x.shape[0]

    def heads(y):
        return y.view(T, H, dh).transpose(0, 1)

    for l in range(cfg.n_layers):
        a = F.rms_norm(x, (d,), weight=P["g1"][l], eps=eps)
        q, k, v = (heads(F.linear(a, P[w][l])) for w in ("wq", "wk", "wv"))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        x = x + F.linear(o.transpose(0, 1).reshape(T, d), P["wo"][l])
        c = F.rms_norm(x, (d,), weight=P["g2"][l], eps=eps)
        grp = 0 if cfg.mem_groups == 1 else l
        km, vm = mk[grp, :, :T].double(), mv[grp, :, :T].double()
        oc = F.scaled_dot_product_attention(heads(F.linear(c, P["wqc"][l])), km, vm, is_causal=True)
        x = x + F.linear(oc.transpose(0, 1).reshape(T, d), P["woc"][l])
        f = F.rms_norm(x, (d,), weight=P["g3"][l], eps=eps)
        x = x + F.linear(F.gelu(F.linear(f, P["w1"][l]), approximate="none"), P["w2"][l])
    return F.linear(F.rms_norm(x, (d,), weight=P["go"], eps=eps), P["wout"]).numpy()


@pytest.mark.parametrize("G", [1, 2])
def test_full_window_equals_causal_sdpa(G):
    """With W >= T the window drops nothing, so with the gate pinned to 1 the
    decoder is a causal pre-norm transformer [Tutorial, "Three forms of context"]."""
    T = 16
    cfg = tiny_cfg(window=T, mem_groups=G)
    _, params = make_model(cfg)
    params = gate_pinned(params, 100.0)
    m64, _ = make_model(cfg, params=params, precision="fp64")
    e, mk, mv = inputs(cfg, 2, T)
    got, _ = run_oracle(m64, e, mk, mv)
    for b in range(2):
        ref = torch_causal_transformer(cfg, params, e[b], mk[:, b], mv[:, b])
        np.testing.assert_allclose(got[b], ref, rtol=0, atol=1e-12)
    # a larger window changes nothing once W >= T
    m64b, _ = make_model(cfg.with_(window=T + 9), params=params, precision="fp64")
    got_b, _ = run_oracle(m64b, e, mk, mv)
    np.testing.assert_array_equal(got, got_b)
    # a window shorter than the run does change the result (the pin can fail)
    m64c, _ = make_model(cfg.with_(window=4), params=params, precision="fp64")
    got_c, _ = run_oracle(m64c, e, mk, mv)
    assert np.max(np.abs(got_c - got)) > 1e-6


# --------------------------------------------------- window conventions (P3, P4)
def test_window_one_returns_current_value():
    """W = 1: the window is the current token alone, so self-attention returns
    v_t exactly [Tutorial, "Advanced Implementation Tips": window definition]."""
    cfg = tiny_cfg(window=1)
    model, _ = make_model(cfg)
    e, mk, mv = inputs(cfg, 2, 12)
    tr = {}
    run_oracle(model, e, mk, mv, trace=tr)
    for swa, v in zip(tr["swa"], tr["v"]):
        np.testing.assert_array_equal(swa, v)


def test_first_token_reads_one_entry():
    """t = 1 starts from H_0 (empty cache) and memory through position 1 only
    [Tutorial, "How the Architecture Works"; "Three forms of context"]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    e, mk, mv = inputs(cfg, 3, 4)
    tr = {}
    run_oracle(model, e, mk, mv, steps=1, trace=tr)
    for l in range(cfg.n_layers):
        np.testing.assert_array_equal(tr["swa"][l], tr["v"][l])
        grp = 0
        np.testing.assert_array_equal(tr["cross"][l], np64(mv[grp, :, :, 0]).astype(np.float32))


def test_window_retention_golden():
    """Retained history after step t is min(t, W - 1) entries per layer.
    Fixture: tests/golden/window_retention.txt."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "window_retention.txt")
    rows = [tuple(int(v) for v in ln.split()) for ln in open(path)
            if ln.strip() and not ln.startswith("#")]
    cfg0 = tiny_cfg(d_model=8, n_heads=1, n_layers=2, d_ffn=8, vocab=4)
    for W, t, kept in rows:
        cfg = cfg0.with_(window=W)
        model, _ = make_model(cfg)
        e, mk, mv = inputs(cfg, 1, t)
        _, states = run_oracle(model, e, mk, mv)
        for l in range(cfg.n_layers):
            assert states[0].K[l].shape[0] == kept and states[0].V[l].shape[0] == kept


def test_depth_table_golden():
    """Structural depth of the state path is t * L_D decoder blocks: the table
    of the [Forget] page (1 -> 48, 10 -> 480, 100 -> 4,800, 1,000 -> 48,000).
    The count is the number of block outputs on the path from s_0 to s_t."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "depth_table.txt")
    rows = [tuple(int(v) for v in ln.split()) for ln in open(path)
            if ln.strip() and not ln.startswith("#")]
    cfg = tiny_cfg(d_model=4, n_heads=1, n_layers=48, d_ffn=4, vocab=2, window=2)
    model, _ = make_model(cfg)
    for t, std_depth, rlt_depth in rows:
        assert std_depth == cfg.n_layers
        if t > 100:     # the 1,000-token row is the same count; checked by formula only
            assert rlt_depth == t * cfg.n_layers
            continue
        e, mk, mv = inputs(cfg, 1, t)
        tr = {}
        run_oracle(model, e, mk, mv, trace=tr)
        assert len(tr["x"]) == rlt_depth


# ---------------------------------------------------- split invariance (P5, P6)
def test_prompt_response_split_is_bitwise_invisible():
    """Proposition 3.1: moving the prompt/response split leaves the result
    unchanged [Forget, Proposition 3.1; Article, "The Critical Boundary"]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    T = 24
    e, mk, mv = inputs(cfg, 2, T)
    full, _ = run_oracle(model, e, mk, mv)
    W = cfg.window
    for k in (1, W - 1, W, W + 1, T // 2):
        st = [oracle.initial_state(model) for _ in range(2)]
        a = oracle.run_sequence(model, st, e[:, :k], mk, mv)
        b = np.stack([oracle.decoder_step(model, st, e[:, j], mk, mv) for j in range(k, T)], 1)
        np.testing.assert_array_equal(np.concatenate([a, b], 1), full)
        st = [oracle.initial_state(model) for _ in range(2)]
        a = oracle.run_sequence(model, st, e[:, :k], mk, mv)
        b = oracle.run_sequence(model, st, e[:, k:], mk, mv)
        np.testing.assert_array_equal(np.concatenate([a, b], 1), full)


def test_resume_needs_the_whole_state():
    """Snapshot = s and every layer's cache; restoring s alone is not the same
    state [Tutorial, "Advanced Implementation Tips": the state is indivisible]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    T, k = 20, 9
    e, mk, mv = inputs(cfg, 1, T)
    full, _ = run_oracle(model, e, mk, mv)
    st = [oracle.initial_state(model)]
    oracle.run_sequence(model, st, e[:, :k], mk, mv)
    snap = oracle.copy_state(st[0])
    fresh = [oracle.copy_state(snap)]
    rest = oracle.run_sequence(model, fresh, e[:, k:], mk, mv)
    np.testing.assert_array_equal(rest[0], full[0, k:])
    # s only, cache emptied: differs for the next steps within the window
    s_only = oracle.initial_state(model)
    s_only.s = snap.s.copy()
    s_only.pos = snap.pos
    s_only.meta["cache_dropped"] = True
    wrong = oracle.run_sequence(model, [s_only], e[:, k:], mk, mv)
    for j in range(cfg.window - 1):
        assert np.max(np.abs(wrong[0, j] - full[0, k + j])) > 1e-7


# -------------------------------------------- parallel SWA pass (P7)
def test_parallel_pass_is_not_the_recurrence():
    """A token-parallel SWA pass is not equivalent to the recurrence; it is
    when the feedback is switched off [Article, "Principle 2"]."""
    cfg = tiny_cfg()
    model, params = make_model(cfg)
    T = 16
    e, mk, mv = inputs(cfg, 1, T)
    rec, _ = run_oracle(model, e, mk, mv)
    par = oracle.parallel_swa_pass(model, e[0], mk[:, 0], mv[:, 0])
    scale = np.max(np.abs(rec))
    assert np.max(np.abs(par[0] - rec[0, 0])) <= 1e-6 * max(scale, 1)
    for t in range(1, T):
        assert np.max(np.abs(par[t] - rec[0, t])) > 1e-2 * scale, t
    # positive control: gate pinned to 1 (u_t = e_t) -> same result at every t
    p1 = gate_pinned(params, 100.0)
    m1, _ = make_model(cfg, params=p1)
    rec1, _ = run_oracle(m1, e, mk, mv)
    par1 = oracle.parallel_swa_pass(m1, e[0], mk[:, 0], mv[:, 0])
    np.testing.assert_allclose(par1, rec1[0], rtol=0, atol=1e-6 * np.max(np.abs(rec1)))


# ---------------------------------------------------- receptive field (P8)
def test_receptive_field_is_exactly_one_plus_L_times_W_minus_1():
    """With the gate pinned to 1, e_1 reaches logits_t only through the
    windows: iff t <= 1 + L (W - 1).  An off-by-one in the window moves this
    boundary.  With the learned gate, e_1 reaches every later step (no reset)
    [Tutorial, "Three forms of context"; Article, "The Critical Boundary"]."""
    cfg = tiny_cfg()
    L, W = cfg.n_layers, cfg.window
    edge = 1 + L * (W - 1)
    T = edge + 3
    _, params = make_model(cfg)
    e, mk, mv = inputs(cfg, 1, T)
    e2 = e.clone()
    e2[0, 0] += 0.5
    m1, _ = make_model(cfg, params=gate_pinned(params, 100.0))
    a, _ = run_oracle(m1, e, mk, mv)
    b, _ = run_oracle(m1, e2, mk, mv)
    for t in range(1, T + 1):
        same = np.array_equal(a[0, t - 1], b[0, t - 1])
        assert same == (t > edge), t
    mg, _ = make_model(cfg, params=params)
    a, _ = run_oracle(mg, e, mk, mv)
    b, _ = run_oracle(mg, e2, mk, mv)
    assert not np.array_equal(a[0, -1], b[0, -1])


# ---------------------------------------------------- memory causality (P9)
def test_memory_is_read_through_t_inclusive():
    """Cross-attention reads memory positions 1..t only
    [Tutorial, "Three forms of context"]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    T = 12
    e, mk, mv = inputs(cfg, 1, T)
    base, _ = run_oracle(model, e, mk, mv)
    for j in (3, 7):                 # perturb memory position j (1-based)
        for which in (0, 1):
            m2 = [mk.clone(), mv.clone()]
            m2[which][:, :, :, j - 1, :] += 0.25
            out, _ = run_oracle(model, e, m2[0], m2[1])
            for t in range(1, T + 1):
                same = np.array_equal(out[0, t - 1], base[0, t - 1])
                assert same == (t < j), (j, which, t)


# ------------------------------------------------------ gate pins (P10, closed forms)
def test_gate_zero_ignores_every_e():
    """g = 0 (W_g = 0, b_g = -200): u_t = s_{t-1}, so no e_t reaches the output."""
    cfg = tiny_cfg()
    _, params = make_model(cfg)
    m0, _ = make_model(cfg, params=gate_pinned(params, -200.0))
    e, mk, mv = inputs(cfg, 1, 10)
    a, _ = run_oracle(m0, e, mk, mv)
    b, _ = run_oracle(m0, torch.randn_like(e), mk, mv)
    np.testing.assert_array_equal(a, b)


def _identity_blocks(params):
    p = dict(params)
    for k in ("wo", "woc", "w2"):
        p[k] = torch.zeros_like(params[k])
    return p


def test_gate_direction_closed_form_ema():
    """Blocks that add nothing (W_O = W_Oc = W_2 = 0) and a constant gate
    g = sigmoid(c) turn the recurrence into an exponential moving average:
    s_T = (1-g)^T s* + g sum_k (1-g)^(T-k) e_k.  Pins which input the gate
    weighs, that s_t is the pre-norm residual stream and that s carries over."""
    cfg = tiny_cfg()
    _, params = make_model(cfg)
    c = float(np.float32(1.3))      # exactly the fp32 value stored in b_g
    p = _identity_blocks(gate_pinned(params, c))
    m, _ = make_model(cfg, params=p, precision="fp64")
    T = 9
    e, mk, mv = inputs(cfg, 1, T)
    out, st = run_oracle(m, e, mk, mv)
    g = 1.0 / (1.0 + math.exp(-c))
    E = np64(e[0])
    s = (1 - g) ** T * np64(p["s_star"]) + g * sum((1 - g) ** (T - k) * E[k - 1]
                                                     for k in range(1, T + 1))
    np.testing.assert_allclose(st[0].s, s, rtol=1e-12, atol=1e-14)
    ref = F.linear(F.rms_norm(torch.tensor(s), (cfg.d_model,), weight=p["go"].double(),
                              eps=cfg.rms_eps), p["wout"].double()).numpy()
    np.testing.assert_allclose(out[0, -1], ref, rtol=1e-12, atol=1e-14)


def test_gate_reads_e_then_s():
    """Concatenation order [e_t ; s_{t-1}]: with W_g = [0 | c I], b_g = 0,
    e_1 = 0 and blocks that add nothing, s_1 = (1 - sigmoid(c s*)) * s*.
    With the order swapped the gate would be sigmoid(0) = 1/2."""
    cfg = tiny_cfg()
    _, params = make_model(cfg)
    d = cfg.d_model
    c = 40.0
    p = _identity_blocks(params)
    wg = torch.zeros(d, 2 * d)
    wg[:, d:] = c * torch.eye(d)
    p["wg"] = wg
    p["bg"] = torch.zeros(d)
    m, _ = make_model(cfg, params=p, precision="fp64")
    e, mk, mv = inputs(cfg, 1, 1)
    e = torch.zeros_like(e)
    _, st = run_oracle(m, e, mk, mv)
    s0 = np64(p["s_star"])
    np.testing.assert_allclose(st[0].s, (1 - expit(c * s0)) * s0, rtol=1e-13, atol=1e-16)
    assert np.max(np.abs(st[0].s - 0.5 * s0)) > 1e-3


# ---------------------------------------------------------------- groups (P11)
def test_per_layer_groups():
    """G = L_D with identical groups equals G = 1; distinct groups differ
    [Princeton, architecture paragraph: G = 1 or G = L_D]."""
    cfg = tiny_cfg()
    cfgL = cfg.with_(mem_groups=cfg.n_layers)
    _, params = make_model(cfg)
    m1, _ = make_model(cfg, params=params)
    mL, _ = make_model(cfgL, params=params)
    e, mk, mv = inputs(cfg, 2, 10)
    a, _ = run_oracle(m1, e, mk, mv)
    mkL = mk.expand(cfg.n_layers, *mk.shape[1:]).contiguous()
    mvL = mv.expand(cfg.n_layers, *mv.shape[1:]).contiguous()
    b, _ = run_oracle(mL, e, mkL, mvL)
    np.testing.assert_array_equal(a, b)
    _, mk2, mv2 = inputs(cfgL, 2, 10)
    c, _ = run_oracle(mL, e, mk2, mv2)
    assert np.max(np.abs(c - a)) > 1e-4


# ------------------------------------------------------- batch invariance (P12)
def test_batch_composition_does_not_matter():
    """Independent sequences: a sequence's logits do not depend on which other
    sequences share its batch [Princeton, design principles paragraph]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    e, mk, mv = inputs(cfg, 4, 12)
    all4, _ = run_oracle(model, e, mk, mv)
    for rows in ([2], [3, 1], [1, 0, 3]):
        sub, _ = run_oracle(model, e, mk, mv, rows=rows)
        for i, r in enumerate(rows):
            np.testing.assert_allclose(sub[i], all4[r], rtol=0, atol=2e-7)


# ---------------------------------------------------------- bf16 emulation
def test_bf16_emulation_is_close_to_exact():
    """The bf16-storage emulation stays within bf16 rounding of the float64
    result on the tiny model (relative L2 of the logits)."""
    cfg = tiny_cfg()
    _, params = make_model(cfg)
    m64, _ = make_model(cfg, params=params, precision="fp64")
    mbf, _ = make_model(cfg, params=params, precision="bf16")
    e, mk, mv = inputs(cfg, 2, 16)
    a, _ = run_oracle(m64, e, mk, mv)
    b, _ = run_oracle(mbf, e, mk, mv)
    rel = np.linalg.norm(b - a) / np.linalg.norm(a)
    assert 1e-5 < rel < 3e-2, rel


# ------------------------------------------------- replay scoring (next row)
def test_token_log_prob_closed_forms():
    """log softmax at the token: two logits 0 and ln 3 give ln(1/4) and ln(3/4);
    V equal logits give -ln V; a shift of every logit by 1000 changes nothing
    (the maximum is taken out before exp); a negative token is not scored."""
    z = np.array([0.0, math.log(3.0)])
    assert abs(oracle.token_log_prob(z, 0) - math.log(0.25)) < 1e-15
    assert abs(oracle.token_log_prob(z, 1) - math.log(0.75)) < 1e-15
    assert abs(oracle.token_log_prob(np.full(37, 2.5), 11) + math.log(37.0)) < 1e-14
    rng = np.random.default_rng(5)
    w = rng.normal(size=50)
    assert abs(oracle.token_log_prob(w + 1000.0, 7) - oracle.token_log_prob(w, 7)) < 1e-9
    assert oracle.token_log_prob(w, -1) == 0.0


def test_token_log_probs_normalise():
    """exp of the log-probabilities of every token sums to one."""
    rng = np.random.default_rng(6)
    z = rng.normal(scale=3.0, size=200)
    total = sum(math.exp(oracle.token_log_prob(z, v)) for v in range(200))
    assert abs(total - 1.0) < 1e-12


def test_score_uses_the_logits_before_the_token_is_consumed():
    """Column t of the replay score is read from the logits of step t (after
    consuming token t, before token t+1) [Tutorial, "Current-Policy
    Reinforcement Learning Replay"]: it equals log softmax of run_sequence's
    logits at column t, and not at t-1 or t+1.  Unscored tokens (< 0) leave
    the other columns unchanged."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    B, T = 3, 10
    e, mk, mv = inputs(cfg, B, T)
    tokens = np.random.default_rng(7).integers(0, cfg.vocab, size=(B, T))
    logits, _ = run_oracle(model, e, mk, mv)
    got = oracle.score_sequence(model, [oracle.initial_state(model) for _ in range(B)],
                                e, mk, mv, tokens)
    for i in range(B):
        for t in range(T):
            z = logits[i, t].astype(np.float64)
            ref = z[tokens[i, t]] - z.max() - math.log(np.exp(z - z.max()).sum())
            assert abs(got[i, t] - ref) < 1e-12
    shifted = np.array([[oracle.token_log_prob(logits[i, t - 1], tokens[i, t]) for t in range(1, T)]
                        for i in range(B)])
    assert np.max(np.abs(shifted - got[:, 1:])) > 1e-3
    masked = tokens.copy()
    masked[:, ::3] = -1
    got2 = oracle.score_sequence(model, [oracle.initial_state(model) for _ in range(B)],
                                 e, mk, mv, masked)
    assert np.all(got2[:, ::3] == 0.0)
    keep = np.ones(T, bool)
    keep[::3] = False
    assert np.array_equal(got2[:, keep], got[:, keep])


# ------------------------------------------------------ generation (next row)
def test_sample_token_inverse_cdf_closed_forms():
    """Logits 0, ln 2, ln 3 give p = 1/6, 2/6, 3/6: u = 0.1, 0.2, 0.6 pick tokens
    0, 1, 2 (first token whose cumulative probability exceeds u) with
    log-probabilities ln p; top_k = 2 keeps tokens 1, 2 (p = 2/5, 3/5);
    top_k = 1 is the argmax for every u; temperature 2 takes square roots of
    the weights."""
    z = np.array([0.0, math.log(2.0), math.log(3.0)])
    for u, tok, p in ((0.1, 0, 1 / 6), (0.2, 1, 2 / 6), (0.6, 2, 3 / 6)):
        t, lp = oracle.sample_token(z, 1.0, 3, u)
        assert t == tok and abs(lp - math.log(p)) < 1e-12
    t, lp = oracle.sample_token(z, 1.0, 2, 0.3)
    assert t == 1 and abs(lp - math.log(0.4)) < 1e-12
    t, lp = oracle.sample_token(z, 1.0, 2, 0.5)
    assert t == 2 and abs(lp - math.log(0.6)) < 1e-12
    for u in (0.0, 0.3, 0.999):
        assert oracle.sample_token(z, 1.0, 1, u)[0] == 2
    w = np.sqrt(np.array([1.0, 2.0, 3.0]))
    t, lp = oracle.sample_token(z, 2.0, 3, 0.99)
    assert t == 2 and abs(lp - math.log(w[2] / w.sum())) < 1e-12


def test_sample_token_frequencies_and_ties():
    """Over a fine grid of u the share of each token is its probability (to
    the grid step); top_k keeps every token tied with the k-th largest logit."""
    rng = np.random.default_rng(8)
    z = rng.normal(size=12)
    w, _ = oracle.sampling_weights(z, 0.7, 5)
    p = w / w.sum()
    N = 20000
    counts = np.zeros(12)
    for j in range(N):
        counts[oracle.sample_token(z, 0.7, 5, (j + 0.5) / N)[0]] += 1
    assert np.max(np.abs(counts / N - p)) <= 1.0 / N + 1e-12
    assert np.count_nonzero(counts) == 5
    tie = np.array([1.0, 5.0, 5.0, 2.0])
    _, keep = oracle.sampling_weights(tie, 1.0, 1)
    assert keep.tolist() == [False, True, True, False]


def test_generate_consumes_each_token_once():
    """Generation with the stand-in encoder equals running the decoder over the
    table rows of the generated tokens, with the memory entries those tokens
    wrote: the sampled token is encoded and consumed exactly once per step
    [Tutorial, "Autoregressive generation"]."""
    cfg = tiny_cfg()
    model, _ = make_model(cfg)
    B, P, n = 3, 5, 7
    e, mk, mv = inputs(cfg, B, P + n)
    te, tk, tv = synth.encoder_tables(cfg)
    u = synth.uniforms((B, n))
    mk1, mv1 = np64(mk).copy(), np64(mv).copy()
    states = [oracle.initial_state(model) for _ in range(B)]
    pre = oracle.run_sequence(model, states, e[:, :P], mk1, mv1)
    toks, lps, last = oracle.generate(model, states, pre[:, -1], te, tk, tv, mk1, mv1, 0.8, 6, u)
    # replay: the same prompt, then the table rows of the generated tokens
    st2 = [oracle.initial_state(model) for _ in range(B)]
    oracle.run_sequence(model, st2, e[:, :P], mk1, mv1)
    e_gen = np64(te)[toks]                                 # [B][n][d]
    rep = oracle.run_sequence(model, st2, e_gen, mk1, mv1)
    np.testing.assert_array_equal(rep[:, -1], last.astype(rep.dtype))
    for i in range(B):
        for j in range(n):
            np.testing.assert_array_equal(mk1[0, i, :, P + j], np64(tk)[0, toks[i, j]])
        assert states[i].pos == P + n
    # log-probabilities are those of the sampling distribution at each step
    logits_steps = np.concatenate([pre[:, -1:], rep[:, :-1]], axis=1)
    for i in range(B):
        for j in range(n):
            w, _ = oracle.sampling_weights(logits_steps[i, j], 0.8, 6)
            z = logits_steps[i, j].astype(np.float64)
            assert abs(lps[i, j] - ((z[toks[i, j]] - z.max()) / 0.8 - math.log(w.sum()))) < 1e-9
