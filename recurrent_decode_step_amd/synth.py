"""Seeded synthetic inputs for the recurrent decoder step.

This module only draws random numbers: decoder and encoder weights, token ids,
encoder outputs e_t, encoder memory K/V, ragged positions and imported decoder
states.  It holds no
part of the decoder's arithmetic and is shared by the tests, the benchmark and
the oracle's callers; neither the oracle nor the HIP library imports it.

Recipe (the same for every workload):

* every tensor comes from its own torch generator whose seed is derived from
  (seed, kind, layer, index) by numpy's SeedSequence, so any single tensor can
  be regenerated alone;
* seeds: weights 0, e_t 1, memory 2, positions 3, imported states 4, stand-in
  encoder tables and uniforms 5, encoder parameters 6, token ids 7;
* weight matrices, s*, b_g ~ N(0, 0.02); RMSNorm gains = 1 + N(0, 0.02);
  e_t, memory K/V and imported states ~ N(0, 1);
* bf16 models round every drawn value to bf16 (round to nearest even) before
  use, so the stored value is exactly the value every consumer sees.

Values depend on the device the generator runs on (torch's CPU and GPU
generators differ); each test draws all its inputs on one device.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import ModelConfig, DTYPE_BF16

SEED_WEIGHTS, SEED_E, SEED_MEM, SEED_POS, SEED_STATE = 0, 1, 2, 3, 4

# parameter kinds (stable ids: part of the seed derivation)
K_SSTAR, K_WG, K_BG, K_G1, K_G2, K_G3 = 1, 2, 3, 4, 5, 6
K_WQ, K_WK, K_WV, K_WO, K_WQC, K_WOC, K_W1, K_W2 = 7, 8, 9, 10, 11, 12, 13, 14
K_GO, K_WOUT = 15, 16

LAYER_MATS = (("wq", K_WQ), ("wk", K_WK), ("wv", K_WV), ("wo", K_WO),
              ("wqc", K_WQC), ("woc", K_WOC), ("w1", K_W1), ("w2", K_W2))
LAYER_GAINS = (("g1", K_G1), ("g2", K_G2), ("g3", K_G3))


def storage_dtype(cfg: ModelConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32


def _generator(device, seed: int, kind: int, layer: int, index: int) -> torch.Generator:
    ss = np.random.SeedSequence([int(seed), int(kind), int(layer), int(index)])
    s = int(ss.generate_state(1, np.uint64)[0]) & ((1 << 63) - 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal(shape, *, mean=0.0, std=1.0, device="cpu", seed=0, kind=0, layer=0, index=0,
           round_bf16=False, out_dtype=torch.float32) -> torch.Tensor:
    """N(mean, std^2) draw from the (seed, kind, layer, index) stream.

    With round_bf16 the fp32 draw is rounded to bf16 first; the result is then
    returned in out_dtype (bf16 storage, or fp32 holding bf16 values)."""
    g = _generator(device, seed, kind, layer, index)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    if round_bf16:
        x = x.to(torch.bfloat16)
    return x.to(out_dtype)


def model_params(cfg: ModelConfig, device="cpu", seed=SEED_WEIGHTS, layers=None) -> dict:
    """Canonical parameters, torch Linear convention W[out][in].

    Matrices are in the storage dtype (bf16 or fp32); vectors (s*, b_g, gains)
    are fp32 tensors holding storage-dtype values.  Per-layer tensors are
    stacked on a leading [L] axis.  `layers` restricts the per-layer tensors to
    the listed layer indices (for regenerating one layer at a time)."""
    d, F, V, L = cfg.d_model, cfg.d_ffn, cfg.vocab, cfg.n_layers
    bf = cfg.dtype == DTYPE_BF16
    sd = storage_dtype(cfg)
    kw = dict(device=device, seed=seed, round_bf16=bf)
    p = {
        "s_star": normal((d,), std=0.02, kind=K_SSTAR, **kw),
        "wg": normal((d, 2 * d), std=0.02, kind=K_WG, out_dtype=sd, **kw),
        "bg": normal((d,), std=0.02, kind=K_BG, **kw),
        "go": normal((d,), mean=1.0, std=0.02, kind=K_GO, **kw),
        "wout": normal((V, d), std=0.02, kind=K_WOUT, out_dtype=sd, **kw),
    }
    ls = list(range(L)) if layers is None else list(layers)
    shapes = {"wq": (d, d), "wk": (d, d), "wv": (d, d), "wo": (d, d),
              "wqc": (d, d), "woc": (d, d), "w1": (F, d), "w2": (d, F)}
    for name, kind in LAYER_MATS:
        p[name] = torch.stack([normal(shapes[name], std=0.02, kind=kind, layer=l,
                                      out_dtype=sd, **kw) for l in ls])
    for name, kind in LAYER_GAINS:
        p[name] = torch.stack([normal((d,), mean=1.0, std=0.02, kind=kind, layer=l, **kw)
                               for l in ls])
    return p


def encoder_e(cfg: ModelConfig, batch: int, steps: int, device="cpu", seed=SEED_E,
              first_seq: int = 0) -> torch.Tensor:
    """Encoder outputs e [batch][steps][d] in the storage dtype (row b drawn
    from stream index first_seq + b)."""
    bf = cfg.dtype == DTYPE_BF16
    return torch.stack([normal((steps, cfg.d_model), device=device, seed=seed, kind=0,
                               index=first_seq + b, round_bf16=bf,
                               out_dtype=storage_dtype(cfg)) for b in range(batch)])


def encoder_memory(cfg: ModelConfig, batch: int, capacity: int, device="cpu",
                   seed=SEED_MEM, first_seq: int = 0):
    """Encoder memory K, V, each [G][batch][H][capacity][dh] in the storage dtype."""
    G, H, dh = cfg.mem_groups, cfg.n_heads, cfg.head_dim
    bf = cfg.dtype == DTYPE_BF16
    sd = storage_dtype(cfg)
    out = []
    for kind in (0, 1):
        t = torch.empty((G, batch, H, capacity, dh), dtype=sd, device=device)
        for g in range(G):
            for b in range(batch):
                t[g, b] = normal((H, capacity, dh), device=device, seed=seed, kind=kind,
                                 layer=g, index=first_seq + b, round_bf16=bf, out_dtype=sd)
        out.append(t)
    return out[0], out[1]


def ragged_positions(batch: int, t_max: int, seed=SEED_POS) -> np.ndarray:
    """Token indices t_b ~ U{1..t_max}, i.i.d. over the batch (int64)."""
    rng = np.random.default_rng([seed, 0, 0, 0])
    return rng.integers(1, t_max + 1, size=batch).astype(np.int64)


def imported_state(cfg: ModelConfig, t: int, device="cpu", seed=SEED_STATE, index: int = 0):
    """A synthetic decoder state about to consume token t (so pos = t - 1).

    s ~ N(0,1) [d] fp32; history K, V [L][H][n_hist][dh] ~ N(0,1) in the
    storage dtype, oldest entry first, n_hist = min(t - 1, W - 1).  t = 1 is the
    initial state (the caller uses s* there)."""
    L, H, dh, W = cfg.n_layers, cfg.n_heads, cfg.head_dim, cfg.window
    bf = cfg.dtype == DTYPE_BF16
    sd = storage_dtype(cfg)
    n_hist = min(t - 1, W - 1)
    s = normal((cfg.d_model,), device=device, seed=seed, kind=0, index=index, round_bf16=bf)
    K = torch.empty((L, H, n_hist, dh), dtype=sd, device=device)
    V = torch.empty((L, H, n_hist, dh), dtype=sd, device=device)
    for l in range(L):
        K[l] = normal((H, n_hist, dh), device=device, seed=seed, kind=1, layer=l, index=index,
                      round_bf16=bf, out_dtype=sd)
        V[l] = normal((H, n_hist, dh), device=device, seed=seed, kind=2, layer=l, index=index,
                      round_bf16=bf, out_dtype=sd)
    return {"pos": t - 1, "s": s, "K": K, "V": V}


SEED_TABLES = 5


def encoder_tables(cfg: ModelConfig, device="cpu", seed=SEED_TABLES):
    """Stand-in incremental encoder for generation: e [V][d] and memory K, V
    [G][V][H][dh] rows per token, ~ N(0, 1), in the storage dtype."""
    bf = cfg.dtype == DTYPE_BF16
    sd = storage_dtype(cfg)
    V, d, G, H, dh = cfg.vocab, cfg.d_model, cfg.mem_groups, cfg.n_heads, cfg.head_dim
    e = normal((V, d), device=device, seed=seed, kind=0, round_bf16=bf, out_dtype=sd)
    k = torch.stack([normal((V, H, dh), device=device, seed=seed, kind=1, layer=g, round_bf16=bf,
                            out_dtype=sd) for g in range(G)])
    v = torch.stack([normal((V, H, dh), device=device, seed=seed, kind=2, layer=g, round_bf16=bf,
                            out_dtype=sd) for g in range(G)])
    return e, k, v


def uniforms(shape, device="cpu", seed=SEED_TABLES, index=0) -> torch.Tensor:
    """Uniform numbers in [0, 1) for sampling, from the (seed, 3, 0, index) stream."""
    g = _generator(device, seed, 3, 0, index)
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)


SEED_ENCODER, SEED_TOKENS = 6, 7
K_EMB, K_GE, K_WKM, K_WVM = 1, 2, 3, 4


def encoder_params(cfg: ModelConfig, device="cpu", seed=SEED_ENCODER) -> dict:
    """Encoder-only parameters (the encoder's blocks reuse the decoder's
    weights): token embedding emb [V][d] ~ N(0, 1) and memory projections
    wkm, wvm [G][d][d] ~ N(0, 0.02) in the storage dtype; the final RMSNorm
    gain ge [d] = 1 + N(0, 0.02) as fp32 holding storage-dtype values."""
    bf = cfg.dtype == DTYPE_BF16
    sd = storage_dtype(cfg)
    V, d, G = cfg.vocab, cfg.d_model, cfg.mem_groups
    kw = dict(device=device, seed=seed, round_bf16=bf)
    return {
        "emb": normal((V, d), kind=K_EMB, out_dtype=sd, **kw),
        "ge": normal((d,), mean=1.0, std=0.02, kind=K_GE, **kw),
        "wkm": torch.stack([normal((d, d), std=0.02, kind=K_WKM, layer=g, out_dtype=sd, **kw)
                            for g in range(G)]),
        "wvm": torch.stack([normal((d, d), std=0.02, kind=K_WVM, layer=g, out_dtype=sd, **kw)
                            for g in range(G)]),
    }


def token_ids(batch: int, steps: int, vocab: int, seed=SEED_TOKENS, index: int = 0) -> np.ndarray:
    """Token ids [batch][steps] ~ U{0..vocab-1} (int32)."""
    rng = np.random.default_rng([seed, index, 0, 0])
    return rng.integers(0, vocab, size=(batch, steps)).astype(np.int32)
