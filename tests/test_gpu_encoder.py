"""GPU parity of the causal encoder (rlt_encode) against the CPU oracle.

Pages (by title): the encoder runs all known tokens at once under a causal
mask with the decoder layers' weights and projects the memory from e_t
[Recurrent Looped Transformer: A New Architecture for Infinite Context
Reasoning in Language Models, "Encoder-Decoder Pairing with Shared Weights";
Princeton Researcher Proposes Recurrent Looped Transformer to Carry Decoder
State Across Tokens, architecture paragraph]; prefill is the encoder followed
by the decoder recurrence over every prompt token [Understanding and Applying
the Recurrent Looped Transformer Architecture, "Prompt prefill"].

Gates: fp32 max |delta| <= 1e-4 on e, memory and encoder cache (values of
order 1) and on logits after prefill; bf16 relative L2 <= 2e-2.  Chunking
and batch composition do not change any value (bitwise): every kernel's result
for a token depends only on that token's own row and the cache positions it
attends to, in a fixed order."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _tiny import oracle_kwargs
from recurrent_decode_step_amd import binding, synth
from recurrent_decode_step_amd.configs import ModelConfig, REFDEPTH

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def setup(cfg, B, cap, max_rows, seed_index=0):
    params = synth.model_params(cfg, device=DEV)
    eparams = synth.encoder_params(cfg, device=DEV)
    model = binding.Model(cfg, params, version=1)
    enc = binding.Encoder(model, eparams)
    es = binding.EncoderState(enc, B, cap, max_rows)
    sd = torch.bfloat16 if cfg.dtype == 1 else torch.float32
    shape = (cfg.mem_groups, B, cfg.n_heads, cap, cfg.head_dim)
    mk = torch.zeros(shape, dtype=sd, device=DEV)
    mv = torch.zeros(shape, dtype=sd, device=DEV)
    return params, eparams, model, enc, es, mk, mv


def oracle_encoder(cfg, params, eparams, precision):
    om = oracle.Model(params={k: v.float().cpu() for k, v in params.items()}, precision=precision,
                      **oracle_kwargs(cfg))
    return oracle.Encoder(om, {k: v.float().cpu() for k, v in eparams.items()})


def f64(t):
    return t.detach().float().cpu().double().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


CONFIGS_F32 = [
    # (d, H, L, F, V, G): dh = 32, 16 and 128, one and per-layer memory groups
    (64, 2, 2, 256, 100, 1),
    (128, 8, 2, 192, 77, 2),
    (256, 2, 1, 512, 300, 1),
    # d = 512: the RMSNorm form that keeps the row in registers
    (512, 4, 1, 512, 64, 1),
]


@pytest.mark.parametrize("dims", CONFIGS_F32, ids=lambda d: "d%d_H%d_L%d_G%d" % (d[0], d[1], d[2], d[5]))
def test_encode_fp32_matches_oracle(dims):
    """3 sequences x 150 tokens = 450 rows: four 128-row tiles with a ragged
    tail, three 64-query blocks per sequence with a ragged last one."""
    d, H, L, F, V, G = dims
    cfg = ModelConfig(vocab=V, d_model=d, n_heads=H, n_layers=L, d_ffn=F, window=8,
                      mem_groups=G, dtype=0)
    B, T = 3, 150
    say(f"[encoder f32] {dims} B={B} T={T}")
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, 160, B * T)
    tok = synth.token_ids(B, T, V, index=1)
    e = binding.rlt_encode(enc, es, torch.from_numpy(tok).to(DEV), (mk, mv))
    torch.cuda.synchronize()
    ck, cv = es.cache()
    ref_enc = oracle_encoder(cfg, params, eparams, "fp32")
    worst = 0.0
    for b in range(B):
        r = oracle.encode(ref_enc, tok[b])
        checks = [(f64(e[b]), r["e"]), (f64(mk[:, b, :, :T]), r["mem_k"]),
                  (f64(mv[:, b, :, :T]), r["mem_v"]),
                  (f64(ck[:, b, :, :T].transpose(1, 2)), r["cache_k"]),
                  (f64(cv[:, b, :, :T].transpose(1, 2)), r["cache_v"])]
        for got, want in checks:
            assert got.shape == want.shape
            worst = max(worst, float(np.abs(got - want).max()))
    say(f"[encoder f32] max |delta| {worst:.2e}")
    assert worst <= 1e-4
    for b in range(B):
        assert es.position(b) == T


def test_encode_chunks_and_batches_are_bitwise_invariant():
    """A prompt encoded in one call, in uneven chunks, or alone gives bitwise
    the same e, memory and cache (positions continue across calls)."""
    cfg = ModelConfig(vocab=120, d_model=128, n_heads=4, n_layers=2, d_ffn=256, window=8,
                      mem_groups=2, dtype=1)
    B, T = 4, 200
    tok = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=2)).to(DEV)
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, 256, B * T)
    e_all = binding.rlt_encode(enc, es, tok, (mk, mv))
    # same model, second state: chunks 1 + 63 + 136, sequences in another order / alone
    es2 = binding.EncoderState(enc, B, 256, B * T)
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    parts = []
    for lo, hi in ((0, 1), (1, 64), (64, 200)):
        parts.append(binding.rlt_encode(enc, es2, tok[[2, 0, 3, 1], lo:hi].contiguous(), (mk2, mv2),
                                        slots=[2, 0, 3, 1]))
    e_chunk = torch.cat(parts, dim=1)[[1, 3, 0, 2]]
    torch.cuda.synchronize()
    assert torch.equal(e_all, e_chunk)
    assert torch.equal(mk, mk2) and torch.equal(mv, mv2)
    k1, v1 = es.cache()
    k2, v2 = es2.cache()
    assert torch.equal(k1[:, :, :, :T], k2[:, :, :, :T]) and torch.equal(v1[:, :, :, :T], v2[:, :, :, :T])
    # one sequence alone in a fresh state
    es3 = binding.EncoderState(enc, B, 256, T)
    mk3, mv3 = torch.zeros_like(mk), torch.zeros_like(mv)
    e_one = binding.rlt_encode(enc, es3, tok[3:4], (mk3, mv3), slots=[3])
    torch.cuda.synchronize()
    assert torch.equal(e_one[0], e_all[3])
    assert torch.equal(mk3[:, 3, :, :T], mk[:, 3, :, :T])


@pytest.mark.parametrize("d,H,F", [(256, 2, 4096), (128, 4, 256), (128, 2, 320)],
                         ids=["dh128_longK", "dh32", "dh64_Kgroups_and_rest"])
def test_short_calls_are_bitwise_the_one_call_result(d, H, F):
    """Calls of few rows take their own kernel forms (GEMM tiles of 32 tokens x
    32 features, stages in groups of eight, with staging-only wavefronts when
    K >= 4096; attention with one query wavefront per (sequence, head) when a
    call has at most 32 tokens per sequence).  K = 128 runs only the stages
    after the last whole group, 320 one group and the rest, 4096 whole groups.  Encoding 70 tokens, then 12, then 32, then 20 one token at
    a time gives bitwise the e rows, memory and cache of one call over all
    134 tokens; so does a batch of 64 sequences (two row tiles) stepped one
    token at a time."""
    cfg = ModelConfig(vocab=120, d_model=d, n_heads=H, n_layers=1, d_ffn=F, window=8,
                      mem_groups=1, dtype=1)
    B, chunks = 5, [70, 12, 32] + [1] * 20
    T = sum(chunks)
    say(f"[encoder short calls] d={d} H={H} F={F} B={B} chunks 70+12+32+20x1")
    tok = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=11)).to(DEV)
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, 160, B * T)
    e_all = binding.rlt_encode(enc, es, tok, (mk, mv))
    es2 = binding.EncoderState(enc, B, 160, B * 70)
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    parts, lo = [], 0
    for n in chunks:
        parts.append(binding.rlt_encode(enc, es2, tok[:, lo:lo + n].contiguous(), (mk2, mv2)))
        lo += n
    torch.cuda.synchronize()
    assert torch.isfinite(e_all).all()
    assert torch.equal(torch.cat(parts, dim=1), e_all)
    assert torch.equal(mk, mk2) and torch.equal(mv, mv2)
    k1, v1 = es.cache()
    k2, v2 = es2.cache()
    assert torch.equal(k1[:, :, :, :T], k2[:, :, :, :T]) and torch.equal(v1[:, :, :, :T], v2[:, :, :, :T])
    # 64 sequences: a prompt of 9, then 3 single tokens (64 rows per call)
    B2, P2 = 64, 9
    tok2 = torch.from_numpy(synth.token_ids(B2, P2 + 3, cfg.vocab, index=12)).to(DEV)
    es3 = binding.EncoderState(enc, B2, 16, B2 * (P2 + 3))
    mk3 = torch.zeros((1, B2, H, 16, d // H), dtype=torch.bfloat16, device=DEV)
    mv3 = torch.zeros_like(mk3)
    e_ref = binding.rlt_encode(enc, es3, tok2, (mk3, mv3))
    es4 = binding.EncoderState(enc, B2, 16, B2 * P2)
    mk4, mv4 = torch.zeros_like(mk3), torch.zeros_like(mv3)
    got = [binding.rlt_encode(enc, es4, tok2[:, :P2].contiguous(), (mk4, mv4))]
    for j in range(P2, P2 + 3):
        got.append(binding.rlt_encode(enc, es4, tok2[:, j:j + 1].contiguous(), (mk4, mv4)))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(got, dim=1), e_ref)
    assert torch.equal(mk3, mk4) and torch.equal(mv3, mv4)
    say("[encoder short calls] bitwise ok")


def test_large_call_matches_per_sequence_calls_bitwise():
    """17100 token rows in one call (134 row tiles, the last one ragged; 384
    QKV features, so a ragged feature tile too) against the same prompts
    encoded one sequence at a time in two chunks: every e row, memory row and
    cache entry agrees bitwise, and one sequence's first rows agree with the
    bf16 oracle."""
    cfg = ModelConfig(vocab=120, d_model=128, n_heads=4, n_layers=2, d_ffn=256, window=8,
                      mem_groups=2, dtype=1)
    B, T = 9, 1900
    say(f"[encoder large call] B={B} T={T} rows={B * T}")
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, T, B * T)
    tok = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=8)).to(DEV)
    e_all = binding.rlt_encode(enc, es, tok, (mk, mv))
    es2 = binding.EncoderState(enc, B, T, T)
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    rows = []
    for b in range(B):
        a = binding.rlt_encode(enc, es2, tok[b:b + 1, :700].contiguous(), (mk2, mv2), slots=[b])
        c = binding.rlt_encode(enc, es2, tok[b:b + 1, 700:].contiguous(), (mk2, mv2), slots=[b])
        rows.append(torch.cat([a, c], dim=1))
    torch.cuda.synchronize()
    assert torch.isfinite(e_all).all()
    assert torch.equal(torch.cat(rows, dim=0), e_all)
    assert torch.equal(mk, mk2) and torch.equal(mv, mv2)
    k1, v1 = es.cache()
    k2, v2 = es2.cache()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    P = 24
    oe = oracle_encoder(cfg, params, eparams, "bf16")
    r = oracle.encode(oe, tok.cpu().numpy()[5, :P])
    rel = rel_l2(f64(e_all[5, :P]), r["e"])
    say(f"[encoder large call] bitwise ok; seq 5 e[:{P}] rel-L2 {rel:.2e}")
    assert rel <= 2e-2

def test_encode_bf16_matches_oracle():
    """bf16 storage (the bf16-emulating oracle): dh = 128, 64 and 256, two groups."""
    for d, H, G in ((256, 2, 1), (256, 4, 2), (512, 2, 1)):
        cfg = ModelConfig(vocab=500, d_model=d, n_heads=H, n_layers=2, d_ffn=512, window=8,
                          mem_groups=G, dtype=1)
        B, T = 2, 130
        say(f"[encoder bf16] d={d} H={H} G={G}")
        params, eparams, model, enc, es, mk, mv = setup(cfg, B, T, B * T)
        tok = synth.token_ids(B, T, cfg.vocab, index=3)
        e = binding.rlt_encode(enc, es, torch.from_numpy(tok).to(DEV), (mk, mv))
        torch.cuda.synchronize()
        ref_enc = oracle_encoder(cfg, params, eparams, "bf16")
        for b in range(B):
            r = oracle.encode(ref_enc, tok[b])
            for name, got, want in (("e", f64(e[b]), r["e"]), ("mem_k", f64(mk[:, b]), r["mem_k"]),
                                    ("mem_v", f64(mv[:, b]), r["mem_v"])):
                rel = rel_l2(got, want)
                say(f"[encoder bf16] seq {b} {name} rel-L2 {rel:.2e}")
                assert rel <= 2e-2, (name, rel)


def test_prefill_encoder_then_decoder_matches_oracle():
    """Prefill = rlt_encode over the prompt, then rlt_run_sequence over every
    prompt token with the encoder's e and memory; logits against the oracle's
    prefill (fp32, max |delta logit| <= 1e-4)."""
    cfg = ModelConfig(vocab=64, d_model=64, n_heads=2, n_layers=2, d_ffn=128, window=8,
                      mem_groups=2, dtype=0)
    B, T = 3, 40
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, T, B * T)
    tok = synth.token_ids(B, T, cfg.vocab, index=4)
    e = binding.rlt_encode(enc, es, torch.from_numpy(tok).to(DEV), (mk, mv))
    st = binding.State(model, B, T)
    logits = binding.rlt_run_sequence(model, st, e, (mk, mv))
    torch.cuda.synchronize()
    ref_enc = oracle_encoder(cfg, params, eparams, "fp32")
    states = [oracle.initial_state(ref_enc.m) for _ in range(B)]
    ref, _, _, _ = oracle.prefill(ref_enc, states, tok)
    err = float(np.abs(f64(logits) - ref).max())
    say(f"[prefill f32] max |delta logit| {err:.2e}")
    assert err <= 1e-4
    for b in range(B):
        assert st.position(b) == T and es.position(b) == T


def test_encode_argument_and_range_errors():
    cfg = ModelConfig(vocab=50, d_model=64, n_heads=2, n_layers=1, d_ffn=128, window=4,
                      mem_groups=1, dtype=0)
    params, eparams, model, enc, es, mk, mv = setup(cfg, 2, 16, 20)
    tok = torch.zeros((2, 10), dtype=torch.int32, device=DEV)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encode(enc, es, torch.zeros((2, 11), dtype=torch.int32, device=DEV), (mk, mv))
    assert ex.value.status == binding.RLT_ERR_SHAPE
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encode(enc, es, tok, (mk, mv), slots=[1, 1])
    assert ex.value.status == binding.RLT_ERR_INVALID_ARG
    with pytest.raises(binding.RLTError) as ex:          # zero tokens: nothing to encode
        binding.rlt_encode(enc, es, tok[:, :0], (mk, mv))
    assert ex.value.status == binding.RLT_ERR_INVALID_ARG
    assert es.position(0) == 0 and es.position(1) == 0
    binding.rlt_encode(enc, es, tok, (mk, mv))
    with pytest.raises(binding.RLTError) as ex:          # 20 > max_tokens 16
        binding.rlt_encode(enc, es, tok, (mk, mv))
    assert ex.value.status == binding.RLT_ERR_RANGE
    assert es.position(0) == 10 and es.position(1) == 10
    binding.rlt_encoder_state_reset(es, [0])
    assert es.position(0) == 0
    small = torch.zeros((1, 2, 2, 12, 32), dtype=torch.float32, device=DEV)
    with pytest.raises(binding.RLTError) as ex:          # memory capacity 12 < 10 + 10
        binding.rlt_encode(enc, es, tok[1:], (small, small.clone()), slots=[1])
    assert ex.value.status == binding.RLT_ERR_RANGE
    # a bf16 model with head_dim 16 is outside the encoder kernels
    cfg16 = ModelConfig(vocab=50, d_model=64, n_heads=4, n_layers=1, d_ffn=128, window=4,
                        mem_groups=1, dtype=1)
    m16 = binding.Model(cfg16, synth.model_params(cfg16, device=DEV))
    with pytest.raises(binding.RLTError) as ex:
        binding.Encoder(m16, synth.encoder_params(cfg16, device=DEV))
    assert ex.value.status == binding.RLT_ERR_UNSUPPORTED


def test_out_of_vocabulary_token_poisons_only_its_sequence():
    """A token outside 0..V-1 gives NaN at its position and, through causal
    attention, at every later position of its sequence; the other sequences of
    the call are bitwise untouched (no out-of-range read)."""
    cfg = ModelConfig(vocab=40, d_model=64, n_heads=2, n_layers=1, d_ffn=128, window=4,
                      mem_groups=1, dtype=0)
    params, eparams, model, enc, es, mk, mv = setup(cfg, 2, 12, 24)
    tok = torch.from_numpy(synth.token_ids(2, 12, cfg.vocab, index=5)).to(DEV)
    ref = binding.rlt_encode(enc, es, tok, (mk, mv))
    es2 = binding.EncoderState(enc, 2, 12, 24)
    bad = tok.clone()
    bad[1, 5] = cfg.vocab
    got = binding.rlt_encode(enc, es2, bad, (torch.zeros_like(mk), torch.zeros_like(mv)))
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0])
    assert torch.isnan(got[1, 5:]).all()


def test_refdepth_full_prompt_sampled_rows():
    """The reference-depth model (48 layers, d = 2048, H = 16, F = 8192, bf16)
    over the full 2048-token prompt of 32 sequences in one call (the launches
    the benchmark times).  Causality lets the oracle check the first 48
    positions of two sampled sequences exactly as computed in that launch; the
    last positions are checked by chunk invariance (the same sequence encoded
    alone in two calls gives bitwise the same rows)."""
    wl = REFDEPTH
    cfg = wl.model
    B, T = wl.batch, wl.prompt
    say(f"[encoder full] {wl.name}: B={B} T={T}")
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, T, B * T)
    tok = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=6)).to(DEV)
    e = binding.rlt_encode(enc, es, tok, (mk, mv))
    torch.cuda.synchronize()
    assert torch.isfinite(e).all()
    say("[encoder full] launch done")
    # chunk invariance of the tail: sequence 31 alone, 2000 + 48 tokens
    es2 = binding.EncoderState(enc, B, T, T)
    mk2 = torch.zeros((cfg.mem_groups, B, cfg.n_heads, T, cfg.head_dim), dtype=mk.dtype, device=DEV)
    mv2 = torch.zeros_like(mk2)
    a = binding.rlt_encode(enc, es2, tok[31:32, :2000].contiguous(), (mk2, mv2), slots=[31])
    b = binding.rlt_encode(enc, es2, tok[31:32, 2000:].contiguous(), (mk2, mv2), slots=[31])
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a, b], dim=1)[0], e[31])
    assert torch.equal(mk2[:, 31], mk[:, 31])
    say("[encoder full] chunk invariance ok")
    del es2, mk2, mv2
    # oracle on the first P positions of two sequences
    P = 48
    LAYER_KEYS = ("g1", "g2", "g3", "wq", "wk", "wv", "wo", "wqc", "woc", "w1", "w2")
    small = {k: params[k].float().cpu() for k in ("s_star", "wg", "bg", "go", "wout")}
    om = oracle.Model(params=small, precision="bf16", **oracle_kwargs(cfg),
                      layer_source=lambda l: {k: params[k][l].float().cpu() for k in LAYER_KEYS})
    oe = oracle.Encoder(om, {k: v.float().cpu() for k, v in eparams.items()})
    tok_np = tok.cpu().numpy()
    for bsel in (0, 17):
        r = oracle.encode(oe, tok_np[bsel, :P])
        for name, got, want in (("e", f64(e[bsel, :P]), r["e"]),
                                ("mem_k", f64(mk[:, bsel, :, :P]), r["mem_k"]),
                                ("mem_v", f64(mv[:, bsel, :, :P]), r["mem_v"])):
            rel = rel_l2(got, want)
            say(f"[encoder full] seq {bsel} {name}[:{P}] rel-L2 {rel:.2e}")
            assert rel <= 2e-2, (bsel, name, rel)


def _valid_draw(z, temperature, top_k, u, tok, rel=1e-3):
    """tok is a valid inverse-CDF draw for u under the float64 distribution:
    its weight is positive and u * total lies in [cum(tok - 1), cum(tok)] up to
    rel * total (the library accumulates in fp32)."""
    w, _ = oracle.sampling_weights(z, temperature, top_k)
    c = np.cumsum(w)
    tot = c[-1]
    lo = c[tok - 1] if tok > 0 else 0.0
    return w[tok] > 0 and lo - rel * tot <= u * tot <= c[tok] + rel * tot


def _prefilled(cfg, B, P, n, index=5):
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, P + n, B * (P + n))
    prompts = synth.token_ids(B, P, cfg.vocab, index=index)
    e = binding.rlt_encode(enc, es, torch.from_numpy(prompts).to(DEV), (mk, mv))
    st = binding.State(model, B, P + n)
    pre = binding.rlt_run_sequence(model, st, e, (mk, mv), logits_mode=binding.RLT_LOGITS_LAST)
    return params, eparams, model, enc, es, mk, mv, prompts, st, pre


def test_generate_encoded_matches_oracle_f32():
    """Prefill, then 8 tokens generated with the causal encoder in the loop
    [Tutorial, "Autoregressive generation": sample, encode the token
    incrementally, consume it once]: every GPU token is a valid draw under the
    oracle's logits (the oracle replays the GPU's tokens), log-probabilities
    agree within 2e-4 / temperature, the last logits and the memory entries the
    encoder wrote within 1e-4."""
    cfg = ModelConfig(vocab=64, d_model=64, n_heads=2, n_layers=2, d_ffn=128, window=4,
                      mem_groups=2, dtype=0)
    B, P, n, temp, topk = 3, 5, 8, 0.9, 10
    params, eparams, model, enc, es, mk, mv, prompts, st, pre = _prefilled(cfg, B, P, n)
    u = synth.uniforms((B, n), index=6)
    say("[generate encoded f32]")
    tok, lp, last = binding.rlt_generate_encoded(model, st, pre, enc, es, (mk, mv), temp, topk,
                                                 u.to(DEV))
    torch.cuda.synchronize()
    tok, lp, last = tok.cpu().numpy(), lp.cpu().numpy(), f64(last)
    for b in range(B):
        assert st.position(b) == P + n and es.position(b) == P + n
    ref_enc = oracle_encoder(cfg, params, eparams, "fp32")
    states = [oracle.initial_state(ref_enc.m) for _ in range(B)]
    ologits, _, rmk, rmv = oracle.prefill(ref_enc, states, prompts, capacity=P + n)
    logits = ologits[:, -1].astype(np.float64)
    seqs = prompts.copy()
    for j in range(n):
        for b in range(B):
            assert _valid_draw(logits[b], temp, topk, float(u[b, j]), int(tok[b, j])), (j, b)
        _, olp, logits = oracle.generate_encoded(ref_enc, states, seqs, logits, rmk, rmv, temp,
                                                 topk, u[:, j:j + 1].numpy(),
                                                 follow=tok[:, j:j + 1])
        seqs = np.concatenate([seqs, tok[:, j:j + 1]], axis=1)
        assert np.max(np.abs(olp[:, 0] - lp[:, j])) <= 2e-4 / temp
    err = float(np.abs(logits - last).max())
    merr = max(float(np.abs(f64(mk) - rmk).max()), float(np.abs(f64(mv) - rmv).max()))
    say(f"  last logits max |delta| {err:.2e}, memory entries {merr:.2e}")
    assert err <= 1e-4 and merr <= 1e-4


def test_generate_encoded_equals_encode_then_run_sequence_bitwise():
    """bf16: generating n tokens with the encoder in the loop leaves the
    decoder state, the last logits and the memory exactly where encoding those
    n tokens in one rlt_encode call and running rlt_run_sequence over their e
    rows leaves them (chunking never changes the encoder's values, and each
    token is consumed once)."""
    cfg = ModelConfig(vocab=96, d_model=128, n_heads=2, n_layers=2, d_ffn=256, window=4,
                      mem_groups=1, dtype=1)
    B, P, n = 4, 6, 5
    params, eparams, model, enc, es, mk, mv, prompts, st, pre = _prefilled(cfg, B, P, n)
    u = synth.uniforms((B, n), index=7).to(DEV)
    say("[generate encoded bf16 bitwise]")
    tok, lp, last = binding.rlt_generate_encoded(model, st, pre, enc, es, (mk, mv), 1.0, 40, u)
    assert torch.isfinite(lp).all()
    # the replay: a second encoder state and decoder state from the same prompt
    es2 = binding.EncoderState(enc, B, P + n, B * (P + n))
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    e_pre = binding.rlt_encode(enc, es2, torch.from_numpy(prompts).to(DEV), (mk2, mv2))
    st2 = binding.State(model, B, P + n)
    binding.rlt_run_sequence(model, st2, e_pre, (mk2, mv2), logits_mode=binding.RLT_LOGITS_NONE)
    e_gen = binding.rlt_encode(enc, es2, tok, (mk2, mv2))
    rep = binding.rlt_run_sequence(model, st2, e_gen, (mk2, mv2))
    torch.cuda.synchronize()
    assert torch.equal(rep[:, -1], last)
    assert torch.equal(mk, mk2) and torch.equal(mv, mv2)
    snap_a = binding.rlt_state_export(model, st, list(range(B)))
    snap_b = binding.rlt_state_export(model, st2, list(range(B)))
    assert torch.equal(snap_a, snap_b)


@pytest.mark.parametrize("d,H,F,dtype,B", [(256, 2, 4096, 1, 5), (1024, 8, 4096, 1, 5),
                                           (1024, 8, 4096, 1, 40), (128, 2, 256, 1, 5),
                                           (128, 4, 256, 1, 5), (128, 2, 4096, 0, 5)],
                         ids=["bf16_dh128_split4", "bf16_split2_and_4", "bf16_split_two_row_tiles",
                              "bf16_dh64", "bf16_dh32", "fp32_dh64"])
def test_fast_short_calls_match_exact_and_oracle(d, H, F, dtype, B):
    """RLT_ENC_FAST: one-token calls take the decoder's attention form, and
    bf16 GEMMs of at most 64 rows split K over 2 or 4 workgroups (as many as
    keep a launch near 256 workgroups, at least 16 packed k-steps each), the
    last of which adds the parts in part order; the split depends on N and K
    only.  At d = 1024 QKV and FFN-up split in two and FFN-down in four, with
    5 rows (one row tile) or 40 (two).  After a 70-token prompt (one exact
    call), 20 one-token calls per sequence:
    e rows and memory within rounding of the exact mode (bf16 rel-L2 <= 1e-2,
    fp32 max |delta| <= 1e-4) and of the oracle (bf16 2e-2, fp32 1e-4); the
    same bits on a second run; and a sequence stepped alone gets the same bits
    as inside the batch."""
    cfg = ModelConfig(vocab=120, d_model=d, n_heads=H, n_layers=2, d_ffn=F, window=8,
                      mem_groups=1, dtype=dtype)
    P, n = 70, 20
    T = P + n
    say(f"[encoder fast] d={d} H={H} F={F} dtype={dtype} B={B}")
    tok = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=13)).to(DEV)
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, 96, B * P)

    def run(slots, mode):
        st_ = binding.EncoderState(enc, B, 96, B * P)
        mk_, mv_ = torch.zeros_like(mk), torch.zeros_like(mv)
        binding.rlt_encode(enc, st_, tok[slots, :P].contiguous(), (mk_, mv_), slots=slots)
        binding.rlt_encoder_state_set_mode(st_, mode)
        rows = [binding.rlt_encode(enc, st_, tok[slots, j:j + 1].contiguous(), (mk_, mv_), slots=slots)
                for j in range(P, T)]
        torch.cuda.synchronize()
        return torch.cat(rows, dim=1), mk_, mv_

    slots = list(range(B))
    e_x, mk_x, mv_x = run(slots, binding.RLT_ENC_EXACT)
    e_f, mk_f, mv_f = run(slots, binding.RLT_ENC_FAST)
    e_f2, mk_f2, mv_f2 = run(slots, binding.RLT_ENC_FAST)
    assert torch.isfinite(e_f).all()
    assert torch.equal(e_f, e_f2) and torch.equal(mk_f, mk_f2) and torch.equal(mv_f, mv_f2)
    e_one, mk_one, _ = run([3], binding.RLT_ENC_FAST)
    assert torch.equal(e_one[0], e_f[3])
    assert torch.equal(mk_one[:, 3, :, :T], mk_f[:, 3, :, :T])
    if dtype == 1:
        rel = rel_l2(f64(e_f), f64(e_x))
        relm = rel_l2(f64(mk_f[:, :, :, P:T]), f64(mk_x[:, :, :, P:T]))
        say(f"[encoder fast] fast vs exact: e rel-L2 {rel:.2e}, memory k rel-L2 {relm:.2e}")
        assert rel <= 1e-2 and relm <= 1e-2
    else:
        worst = float((e_f - e_x).abs().max())
        say(f"[encoder fast] fast vs exact: e max |delta| {worst:.2e}")
        assert worst <= 1e-4
    oe = oracle_encoder(cfg, params, eparams, "bf16" if dtype == 1 else "fp32")
    r = oracle.encode(oe, tok.cpu().numpy()[1, :T])
    if dtype == 1:
        rel = rel_l2(f64(e_f[1]), r["e"][P:T])
        say(f"[encoder fast] seq 1 against the oracle: rel-L2 {rel:.2e}")
        assert rel <= 2e-2
    else:
        worst = float(np.abs(f64(e_f[1]) - r["e"][P:T]).max())
        say(f"[encoder fast] seq 1 against the oracle: max |delta| {worst:.2e}")
        assert worst <= 1e-4


def test_generate_encoded_fast_equals_token_calls_then_run_sequence_bitwise():
    """With RLT_ENC_FAST set, generation leaves the decoder state, last logits
    and memory exactly where encoding the generated tokens one call per token
    (fast) and running rlt_run_sequence over their e rows leaves them."""
    cfg = ModelConfig(vocab=96, d_model=256, n_heads=2, n_layers=2, d_ffn=4096, window=4,
                      mem_groups=1, dtype=1)
    B, P, n = 4, 6, 5
    params, eparams, model, enc, es, mk, mv, prompts, st, pre = _prefilled(cfg, B, P, n)
    binding.rlt_encoder_state_set_mode(es, binding.RLT_ENC_FAST)
    u = synth.uniforms((B, n), index=9).to(DEV)
    say("[generate encoded fast bitwise]")
    tok, lp, last = binding.rlt_generate_encoded(model, st, pre, enc, es, (mk, mv), 1.0, 40, u)
    assert torch.isfinite(lp).all()
    es2 = binding.EncoderState(enc, B, P + n, B * (P + n))
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    e_pre = binding.rlt_encode(enc, es2, torch.from_numpy(prompts).to(DEV), (mk2, mv2))
    st2 = binding.State(model, B, P + n)
    binding.rlt_run_sequence(model, st2, e_pre, (mk2, mv2), logits_mode=binding.RLT_LOGITS_NONE)
    binding.rlt_encoder_state_set_mode(es2, binding.RLT_ENC_FAST)
    e_gen = torch.cat([binding.rlt_encode(enc, es2, tok[:, j:j + 1].contiguous(), (mk2, mv2))
                       for j in range(n)], dim=1)
    rep = binding.rlt_run_sequence(model, st2, e_gen, (mk2, mv2))
    torch.cuda.synchronize()
    assert torch.equal(rep[:, -1], last)
    assert torch.equal(mk, mk2) and torch.equal(mv, mv2)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encoder_state_set_mode(es2, 2)
    assert ex.value.status == binding.RLT_ERR_INVALID_ARG


def test_generate_encoded_needs_matching_positions():
    """The encoder must hold exactly the tokens the decoder consumed: a slot
    whose decoder state is one token ahead is a range error, found before any
    device work."""
    cfg = ModelConfig(vocab=64, d_model=64, n_heads=2, n_layers=1, d_ffn=128, window=4,
                      mem_groups=1, dtype=0)
    B, P, n = 2, 3, 2
    params, eparams, model, enc, es, mk, mv, prompts, st, pre = _prefilled(cfg, B, P, n + 1)
    binding.rlt_decoder_step(model, st, torch.zeros((B, cfg.d_model), device=DEV), (mk, mv))
    u = synth.uniforms((B, n), index=8).to(DEV)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_generate_encoded(model, st, pre, enc, es, (mk, mv), 1.0, 5, u)
    assert ex.value.status == binding.RLT_ERR_RANGE
    assert es.position(0) == P and st.position(0) == P + 1


def test_encoder_snapshot_resumes_a_conversation_bitwise():
    """Exact prefix snapshot of a conversation [Article, "Multi-Turn Serving"]:
    the decoder records, the encoder-cache records and the memory entries of
    three sequences after a 7-token prompt, imported into other slots (a
    permutation) of fresh states, continue exactly like the originals: the
    next 5 tokens' e rows, memory entries and logits are bitwise equal, row by
    row.  (bf16, two memory groups.)"""
    cfg = ModelConfig(vocab=96, d_model=128, n_heads=2, n_layers=2, d_ffn=256, window=4,
                      mem_groups=2, dtype=1)
    B, P, n, cap = 3, 7, 5, 12
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, cap, B * cap)
    prompts = synth.token_ids(B, P, cfg.vocab, index=12)
    nxt = torch.from_numpy(synth.token_ids(B, n, cfg.vocab, index=13)).to(DEV)
    e = binding.rlt_encode(enc, es, torch.from_numpy(prompts).to(DEV), (mk, mv))
    st = binding.State(model, B, cap)
    binding.rlt_run_sequence(model, st, e, (mk, mv), logits_mode=binding.RLT_LOGITS_NONE)
    dec = binding.rlt_state_export(model, st, list(range(B)))
    encs = binding.rlt_encoder_state_export(enc, es, list(range(B)), P)
    perm = [2, 0, 1]                                   # record i goes to slot perm[i]
    es2 = binding.EncoderState(enc, B, cap, B * cap)
    st2 = binding.State(model, B, cap)
    binding.rlt_encoder_state_import(enc, es2, encs, perm, P)
    binding.rlt_state_import(model, st2, dec, perm)
    mk2, mv2 = torch.zeros_like(mk), torch.zeros_like(mv)
    for i, j in enumerate(perm):
        mk2[:, j], mv2[:, j] = mk[:, i], mv[:, i]
    for i, j in enumerate(perm):
        assert es2.position(j) == P and st2.position(j) == P
    say("[encoder snapshot resume]")
    e_a = binding.rlt_encode(enc, es, nxt, (mk, mv))
    la = binding.rlt_run_sequence(model, st, e_a, (mk, mv))
    nxt2 = torch.empty_like(nxt)
    for i, j in enumerate(perm):
        nxt2[j] = nxt[i]
    e_b = binding.rlt_encode(enc, es2, nxt2, (mk2, mv2))
    lb = binding.rlt_run_sequence(model, st2, e_b, (mk2, mv2))
    torch.cuda.synchronize()
    for i, j in enumerate(perm):
        assert torch.equal(e_a[i], e_b[j])
        assert torch.equal(la[i], lb[j])
        assert torch.equal(mk[:, i], mk2[:, j]) and torch.equal(mv[:, i], mv2[:, j])


def test_encoder_snapshot_checks_before_any_change():
    """Export refuses a capacity below a slot's position (RLT_ERR_RANGE);
    import refuses a record of another capacity, a decoder record and a
    record of another model version (RLT_ERR_CONVENTION), each before it
    changes the state."""
    cfg = ModelConfig(vocab=64, d_model=64, n_heads=2, n_layers=1, d_ffn=128, window=4,
                      mem_groups=1, dtype=0)
    B, P, cap = 2, 5, 8
    params, eparams, model, enc, es, mk, mv = setup(cfg, B, cap, B * cap)
    binding.rlt_encode(enc, es, torch.from_numpy(synth.token_ids(B, P, cfg.vocab, index=14)).to(DEV),
                       (mk, mv))
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encoder_state_export(enc, es, [0, 1], P - 1)
    assert ex.value.status == binding.RLT_ERR_RANGE
    good = binding.rlt_encoder_state_export(enc, es, [0, 1], P)
    es2 = binding.EncoderState(enc, B, cap, B * cap)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encoder_state_import(enc, es2, good, [0, 1], P + 1)
    assert ex.value.status == binding.RLT_ERR_CONVENTION
    st = binding.State(model, B, cap)
    dec = binding.rlt_state_export(model, st, [0, 1])
    need = binding.encoder_snapshot_bytes(cfg, P, 2)
    fake = torch.zeros(max(need, dec.numel()), dtype=torch.uint8, device=DEV)
    fake[:dec.numel()] = dec
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encoder_state_import(enc, es2, fake, [0, 1], P)
    assert ex.value.status == binding.RLT_ERR_CONVENTION
    model2 = binding.Model(cfg, params, version=2)
    enc2 = binding.Encoder(model2, eparams)
    es3 = binding.EncoderState(enc2, B, cap, B * cap)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_encoder_state_import(enc2, es3, good, [0, 1], P)
    assert ex.value.status == binding.RLT_ERR_CONVENTION
    assert es2.position(0) == 0 and es2.position(1) == 0 and es3.position(0) == 0
    binding.rlt_encoder_state_import(enc, es2, good, [1, 0], P)
    assert es2.position(0) == P and es2.position(1) == P
