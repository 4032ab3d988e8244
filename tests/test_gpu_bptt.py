"""GPU parity of backpropagation through time (rlt_bptt, fp32) against the
oracle's autograd gradient (float64).

Pages (by title): full-sequence next-token prediction with backpropagation
through time, the loss masked per target but never the state update
[Recurrent Looped Transformer: A New Architecture for Infinite Context
Reasoning in Language Models, "Training Methodology"; Understanding and Applying
the Recurrent Looped Transformer Architecture, "Pretraining and supervised
fine-tuning"]; truncation names every detached tensor, and detaching s alone
leaves the path through the cache [What If a Transformer Never Had to Forget?
Meet the Recurrent Looped Transformer (RLT), its note on truncated BPTT].

Gate: for every gradient tensor, max |delta| <= 1e-4 * max |reference| (fp32
arithmetic over T steps against float64), or, where the recurrence itself
amplifies rounding, within 4x the error of the same oracle run in float32 on the
CPU (the conditioning of the problem, measured); the loss within 1e-5 relative.
Exact zeros the detach semantics fix are checked bitwise."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import bptt
from recurrent_decode_step_amd import binding, synth
from recurrent_decode_step_amd.configs import ModelConfig

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def case(cfg, B, T, scale=1.0, index=0, mask_first=0):
    params = synth.model_params(cfg, device=DEV)
    params = {k: (v * scale if k.startswith("w") else v) for k, v in params.items()}
    e = synth.encoder_e(cfg, B, T, device=DEV)
    mk, mv = synth.encoder_memory(cfg, B, T + 3, device=DEV)
    tg = torch.from_numpy(synth.token_ids(B, T, cfg.vocab, index=index))
    if mask_first:
        tg[:, :mask_first] = -1
    return params, e, mk, mv, tg


def compare(cfg, params, e, mk, mv, tg, chunk=0, detach=0, label="", segment=0):
    loss, g, de, (dmk, dmv) = binding.rlt_bptt(cfg, params, e, (mk, mv), tg, chunk=chunk,
                                               detach=detach, segment=segment)
    torch.cuda.synchronize()
    names = []
    if detach & binding.RLT_DETACH_S:
        names.append("s")
    if detach & binding.RLT_DETACH_KV:
        names.append("kv")
    kw = dict(n_heads=cfg.n_heads, window=cfg.window, rms_eps=cfg.rms_eps, chunk=chunk,
              detach=tuple(names))
    host = ({k: v.cpu() for k, v in params.items()}, e.cpu(), mk.cpu(), mv.cpu(), tg.numpy())
    rl, rg, rde, rdmk, rdmv = bptt.gradients(*host, **kw)
    # the same oracle in float32: how far fp32 rounding alone moves each gradient
    _, fg, fde, fdmk, fdmv = bptt.gradients(*host, dtype=torch.float32, **kw)
    assert abs(float(loss) - rl) <= 1e-5 * max(1.0, abs(rl)), (float(loss), rl)
    worst = 0.0
    pairs = ([(k, g[k], rg[k], fg[k]) for k in g] +
             [("e", de, rde, fde), ("mem_k", dmk, rdmk, fdmk), ("mem_v", dmv, rdmv, fdmv)])
    for name, got, want, f32 in pairs:
        got = got.double().cpu().numpy()
        scale = float(np.abs(want).max())
        err = float(np.abs(got - want).max())
        rel = err / scale if scale > 0 else err
        f32_rel = float(np.abs(f32.astype(np.float64) - want).max()) / scale if scale > 0 else 0.0
        worst = max(worst, rel)
        assert rel <= max(1e-4, 4.0 * f32_rel), (label, name, err, scale, f32_rel)
    say(f"[bptt] {label}: loss {float(loss):.6f} (ref {rl:.6f}), worst max-rel {worst:.2e}")
    return de, dmk


CONFIGS = [
    # (d, H, L, F, V, W, G): dh 16 and 32, one and per-layer memory groups
    ((32, 2, 2, 64, 11, 3, 1), 2, 6),
    ((32, 2, 2, 64, 11, 3, 2), 2, 6),
    ((128, 4, 2, 256, 200, 5, 1), 3, 20),
    # 128 sequences: per-step products over 128 rows (two register sets of loads)
    ((128, 4, 1, 256, 200, 4, 1), 128, 4),
    # 144 sequences: past 128 rows the per-step products keep one register set
    ((128, 4, 1, 256, 200, 4, 1), 144, 3),
    # F = V = 2048: the wide per-step product form (16 x 64 tiles) and, with V a
    # multiple of 16, the MFMA form of the head's input gradient
    ((128, 4, 1, 2048, 2048, 6, 1), 16, 4),
    # d = 512 (the benchmark's width): the RMSNorm forms that load the row into registers
    ((512, 8, 1, 512, 40, 3, 1), 3, 5),
]


@pytest.mark.parametrize("spec", CONFIGS, ids=lambda s: "d%d_L%d_W%d_G%d_B%d" % (s[0][0], s[0][2], s[0][5], s[0][6], s[1]))
def test_full_bptt_matches_oracle(spec):
    (d, H, L, F, V, W, G), B, T = spec
    cfg = ModelConfig(vocab=V, d_model=d, n_heads=H, n_layers=L, d_ffn=F, window=W, mem_groups=G,
                      dtype=0)
    for scale in (1.0, 10.0):
        params, e, mk, mv, tg = case(cfg, B, T, scale=scale, mask_first=2)
        compare(cfg, params, e, mk, mv, tg, label=f"d{d} G{G} weights x{scale}")


@pytest.mark.parametrize("detach", [1, 2, 3])
def test_truncated_bptt_matches_oracle(detach):
    """chunk 3 with s, the cache or both detached; with both, the e of steps
    1..3 get exactly zero gradient from the later losses."""
    cfg = ModelConfig(vocab=11, d_model=32, n_heads=2, n_layers=2, d_ffn=64, window=3,
                      mem_groups=1, dtype=0)
    params, e, mk, mv, tg = case(cfg, 2, 7, scale=10.0, mask_first=3)
    de, _ = compare(cfg, params, e, mk, mv, tg, chunk=3, detach=detach, label=f"detach {detach}")
    if detach == 3:
        assert torch.all(de[:, :3] == 0)
    else:
        assert float(de[:, :3].abs().max()) > 0


@pytest.mark.parametrize("segment", [1, 4, 7, 19])
def test_checkpointed_bptt_matches_full_bitwise_where_fixed(segment):
    """Activation checkpointing (segment S < T): every step runs forward once,
    then the segments in reverse are recomputed from their first state and run
    backward.  The recomputed steps repeat the same kernels on the same inputs,
    so the loss, the e gradients and the memory gradients are bitwise those of
    the run that keeps everything; the parameter gradients only regroup their
    sums over rows by segment (within 1e-5 of the full run's, relative to each
    tensor's largest entry), and all of it passes the oracle gate.  S = 7 and
    19 leave a ragged last segment (T = 20)."""
    cfg = ModelConfig(vocab=200, d_model=128, n_heads=4, n_layers=2, d_ffn=256, window=5,
                      mem_groups=1, dtype=0)
    params, e, mk, mv, tg = case(cfg, 3, 20, mask_first=2)
    full = binding.rlt_bptt(cfg, params, e, (mk, mv), tg)
    seg = binding.rlt_bptt(cfg, params, e, (mk, mv), tg, segment=segment)
    torch.cuda.synchronize()
    assert torch.equal(seg[0], full[0])                       # loss
    assert torch.equal(seg[2], full[2])                       # d e
    assert torch.equal(seg[3][0], full[3][0]) and torch.equal(seg[3][1], full[3][1])   # d memory
    worst = 0.0
    for k in full[1]:
        a, b = full[1][k].double(), seg[1][k].double()
        scale = float(a.abs().max())
        rel = float((a - b).abs().max()) / scale if scale > 0 else float((a - b).abs().max())
        worst = max(worst, rel)
        assert rel <= 1e-5, (k, rel)
    say(f"[bptt] segment {segment}: parameter gradients within {worst:.2e} of the full run")
    compare(cfg, params, e, mk, mv, tg, segment=segment, label=f"segment {segment}")


def test_checkpointed_truncated_bptt():
    """Segments that cut across truncation chunks (chunk 3, segment 2, s and
    the cache detached): the same exact zeros and the oracle gate."""
    cfg = ModelConfig(vocab=11, d_model=32, n_heads=2, n_layers=2, d_ffn=64, window=3,
                      mem_groups=2, dtype=0)
    params, e, mk, mv, tg = case(cfg, 2, 7, scale=10.0, mask_first=3)
    de, _ = compare(cfg, params, e, mk, mv, tg, chunk=3, detach=3, segment=2,
                    label="chunk 3, detach s and kv, segment 2")
    assert torch.all(de[:, :3] == 0)


def test_checkpointing_shrinks_the_workspace():
    """The reference-depth model (fp32 for training) at 8 sequences x 256
    steps: keeping every step needs about 28 GB, 16-step segments under 5 GB."""
    from recurrent_decode_step_amd.configs import REFDEPTH
    cfg = REFDEPTH.model.with_(dtype=0)
    L = binding.load_library()
    cc = binding.make_config(cfg)
    full = L.rlt_bptt_workspace_bytes(binding.C.byref(cc), 8, 256)
    seg = L.rlt_bptt_workspace_bytes_segmented(binding.C.byref(cc), 8, 256, 16)
    assert full == L.rlt_bptt_workspace_bytes_segmented(binding.C.byref(cc), 8, 256, 0)
    say(f"[bptt] workspace at reference depth, 8 x 256 steps: {full / 1e9:.1f} GB, "
        f"16-step segments {seg / 1e9:.1f} GB")
    assert seg < full / 3


def test_memory_with_unaligned_rows_is_rejected():
    """Memory rows must start on 16-byte boundaries (the attention kernels read
    16-byte pieces): a position stride of dh + 1 elements is a shape error,
    found before any work."""
    cfg = ModelConfig(vocab=11, d_model=32, n_heads=2, n_layers=2, d_ffn=64, window=3,
                      mem_groups=1, dtype=0)
    params, e, mk, mv, tg = case(cfg, 2, 6)
    G, B, H, cap, dh = mk.shape
    padded = torch.zeros((G, B, H, cap, dh + 1), dtype=mk.dtype, device=DEV)
    view = padded[..., :dh]
    assert view.stride(-2) == dh + 1
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_bptt(cfg, params, e, (view, view), tg)
    assert ex.value.status == binding.RLT_ERR_SHAPE


def test_bptt_rejects_bf16_and_bad_arguments():
    cfg = ModelConfig(vocab=11, d_model=32, n_heads=2, n_layers=1, d_ffn=64, window=3,
                      mem_groups=1, dtype=1)
    params, e, mk, mv, tg = case(cfg.with_(dtype=0), 1, 4)
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_bptt(cfg, params, e, (mk, mv), tg)
    assert ex.value.status == binding.RLT_ERR_UNSUPPORTED
    cfg32 = cfg.with_(dtype=0)
    short = (mk[:, :, :, :2].contiguous(), mv[:, :, :, :2].contiguous())
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_bptt(cfg32, params, e, short, tg)
    assert ex.value.status == binding.RLT_ERR_RANGE
    with pytest.raises(binding.RLTError) as ex:
        binding.rlt_bptt(cfg32, params, e, (mk, mv), tg, detach=4, chunk=2)
    assert ex.value.status == binding.RLT_ERR_INVALID_ARG
    with pytest.raises(binding.RLTError) as ex:          # zero steps
        binding.rlt_bptt(cfg32, params, e[:, :0], (mk, mv), tg[:, :0])
    assert ex.value.status == binding.RLT_ERR_INVALID_ARG
