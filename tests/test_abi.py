"""The C-ABI library loads, exports every symbol include/rlt.h declares, and
rejects bad arguments on the host before any device work (no GPU needed)."""
from __future__ import annotations

import ctypes as C
import os
import re

import pytest

from recurrent_decode_step_amd import binding
from recurrent_decode_step_amd.configs import TINY, SMALL, REFDEPTH, LARGEBATCH, LONGCTX

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("librlt.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "rlt.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rlt_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = lib()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.EXPORTED)
    assert L.rlt_abi_version() == binding.ABI_VERSION == 4


def test_status_strings():
    L = lib()
    for code in range(8):
        assert L.rlt_status_str(code).decode().startswith("RLT_")


def cfg_of(w, **kw):
    c = binding.make_config(w.model)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_size_queries():
    L = lib()
    # model bytes cover the packed weights
    for w in (TINY, SMALL, REFDEPTH, LONGCTX):
        m = w.model
        es = 2 if m.dtype == 1 else 4
        params = (2 * m.d_model ** 2 + m.n_layers * (6 * m.d_model ** 2 + 2 * m.d_model * m.d_ffn)
                  + m.vocab * m.d_model)
        got = L.rlt_model_bytes(C.byref(cfg_of(w)))
        assert params * es <= got <= params * es * 1.05 + (1 << 20), (w.name, got)
    # state bytes cover s, positions and the window cache [L][B][H][W][dh] x 2
    m = LARGEBATCH.model
    ring = 2 * m.n_layers * 256 * m.n_heads * m.window * m.head_dim * 2
    got = L.rlt_state_bytes(C.byref(cfg_of(LARGEBATCH)), 256, 8192)
    assert ring < got < ring * 1.2
    # snapshot record: header + s + 2 * [L][H][W-1][dh]
    m = TINY.model
    rec = L.rlt_snapshot_bytes(C.byref(cfg_of(TINY)), 1)
    assert rec == binding.snapshot_layout(m)[0]
    assert L.rlt_snapshot_bytes(C.byref(cfg_of(TINY)), 3) == 3 * rec


@pytest.mark.parametrize("field,value", [
    ("head_dim", 15), ("n_heads", 0), ("mem_groups", 3), ("dtype", 7), ("d_ffn", 100),
    ("window", 0), ("attn_chunk", -1)])
def test_bad_configs_are_rejected(field, value):
    L = lib()
    c = cfg_of(TINY, **{field: value})
    assert L.rlt_model_bytes(C.byref(c)) == 0
    out = C.c_void_p()
    p = binding.rlt_params()
    st = L.rlt_model_create(C.byref(c), C.byref(p), 1, None, 0, None, C.byref(out))
    assert st in (binding.RLT_ERR_INVALID_ARG, binding.RLT_ERR_SHAPE, binding.RLT_ERR_UNSUPPORTED)
    assert L.rlt_last_error().decode() != ""
    assert not out.value


def test_create_argument_checks_before_device_work():
    L = lib()
    c = cfg_of(TINY)
    out = C.c_void_p()
    p = binding.rlt_params()
    # NULL parameter pointers
    assert L.rlt_model_create(C.byref(c), C.byref(p), 1, None, 0, None,
                              C.byref(out)) == binding.RLT_ERR_INVALID_ARG
    # all pointers set but buffer misaligned / too small (fake addresses, never touched)
    for name, _ in binding.rlt_params._fields_:
        setattr(p, name, 0x1000)
    assert L.rlt_model_create(C.byref(c), C.byref(p), 1, C.c_void_p(0x1008), 1 << 30, None,
                              C.byref(out)) == binding.RLT_ERR_SHAPE
    assert L.rlt_model_create(C.byref(c), C.byref(p), 1, C.c_void_p(0x1000), 10, None,
                              C.byref(out)) == binding.RLT_ERR_SHAPE
    assert "required" in L.rlt_last_error().decode()


def test_null_handles():
    L = lib()
    out = C.c_void_p()
    assert L.rlt_state_init(None, 4, 64, None, 0, None, C.byref(out)) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_decoder_step(None, None, 1, None, None, None, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_run_sequence(None, None, 1, None, None, None, 0, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_score_sequence(None, None, 1, None, None, None, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_generate(None, None, 1, None, None, None, None, None, None, None, None,
                          None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_state_reset(None, None, 1, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_state_export(None, None, 1, None, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_state_import(None, None, 1, None, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_state_position(None, 0) == -1
    assert L.rlt_profile_begin(None, 1, 1, 1) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_profile_collect(None, 0, None, None, None) == binding.RLT_ERR_INVALID_ARG


def test_peak_measurement_argument_checks():
    """The peak calls reject bad arguments on the host, before any device work."""
    L = lib()
    out = C.c_double(0.0)
    big = 1 << 30
    assert L.rlt_peak_bandwidth(None, C.c_void_p(0x1000), big, 0, 1, C.byref(out),
                                None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_peak_bandwidth(C.c_void_p(0x1000), C.c_void_p(0x2000), big, 0, 0, C.byref(out),
                                None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_peak_bandwidth(C.c_void_p(0x1000), C.c_void_p(0x2000), 1 << 20, 0, 1,
                                C.byref(out), None) == binding.RLT_ERR_SHAPE      # under 64 MiB
    assert L.rlt_peak_bandwidth(C.c_void_p(0x1000), C.c_void_p(0x2000), big + 16, 0, 1,
                                C.byref(out), None) == binding.RLT_ERR_SHAPE      # not 64 KiB spans
    assert L.rlt_peak_bandwidth(C.c_void_p(0x1008), C.c_void_p(0x2000), big, 1, 1,
                                C.byref(out), None) == binding.RLT_ERR_SHAPE      # unaligned
    assert L.rlt_peak_mfma(0, 16, 1, None, 1 << 20, C.byref(out), None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_peak_mfma(2, 16, 1, C.c_void_p(0x1000), 1 << 20, C.byref(out),
                           None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_peak_mfma(0, 0, 1, C.c_void_p(0x1000), 1 << 20, C.byref(out),
                           None) == binding.RLT_ERR_INVALID_ARG


def test_encoder_null_handles_and_sizes():
    L = lib()
    out = C.c_void_p()
    assert L.rlt_encoder_bytes(None) == 0
    p = binding.rlt_encoder_params()
    assert L.rlt_encoder_create(None, C.byref(p), None, 0, None, C.byref(out)) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encoder_state_init(None, 2, 16, 8, None, 0, C.byref(out)) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encode(None, None, 1, None, 1, None, None, None, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encoder_state_reset(None, 1, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encoder_state_set_mode(None, binding.RLT_ENC_FAST) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encoder_position(None, 0) == -1
    assert L.rlt_encoder_profile_begin(None, 1, 1) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_encoder_profile_collect(None, 0, None, None, None, None) == binding.RLT_ERR_INVALID_ARG
    # the encoder state holds the cache [L][B][H][cap][dh] twice, per-row scratch
    # and the partial tiles of the fast short-call GEMMs (two 32-row tiles x
    # max(3d, F) / 32 feature tiles x 4 parts x 4 KiB, one counter per tile)
    for w in (TINY, SMALL, REFDEPTH):
        m = w.model
        es = 2 if m.dtype == 1 else 4
        B, cap, R = 4, 96, 40
        cache = 2 * m.n_layers * B * m.d_model * cap * es
        scratch = R * m.d_model * (4 + 4 * es) + R * m.d_ffn * es
        split = 2 * ((max(3 * m.d_model, m.d_ffn) + 31) // 32) * (4 * 4096 + 4)   # tiles, counters
        got = L.rlt_encoder_state_bytes(C.byref(cfg_of(w)), B, cap, R)
        assert cache + scratch + split <= got <= cache + scratch + split + 16 * 256
    assert L.rlt_encoder_state_bytes(C.byref(cfg_of(TINY)), 0, 16, 8) == 0
    assert L.rlt_encoder_state_bytes(C.byref(cfg_of(TINY)), 2, 16, 0) == 0
    # bf16 with head_dim 16 is outside the encoder kernels
    assert L.rlt_encoder_state_bytes(C.byref(cfg_of(SMALL, n_heads=32, head_dim=16)), 2, 16, 8) == 0


def test_bptt_host_checks():
    L = lib()
    c = cfg_of(TINY)
    # fp32 tiny config: a workspace size; bf16 or T beyond 4096: none
    assert L.rlt_bptt_workspace_bytes(C.byref(c), 2, 16) > 0
    assert L.rlt_bptt_workspace_bytes(C.byref(cfg_of(SMALL)), 2, 16) == 0
    assert L.rlt_bptt_workspace_bytes(C.byref(c), 2, 5000) == 0
    # NULL parameters and a bf16 config are rejected before any device work
    p = binding.rlt_params()
    assert L.rlt_bptt(C.byref(c), C.byref(p), 2, 4, None, None, None, None, C.byref(p), None, None,
                      None, None, 0, None) == binding.RLT_ERR_INVALID_ARG
    assert L.rlt_bptt(C.byref(cfg_of(SMALL)), C.byref(p), 2, 4, None, None, None, None, C.byref(p),
                      None, None, None, None, 0, None) == binding.RLT_ERR_UNSUPPORTED


def test_fused_run_support_rule():
    """rlt_fused_supported (host only): fp32 models whose weights, gains, one
    slot's window cache and activations fit in 160 KiB of LDS."""
    from _tiny import tiny_cfg
    from recurrent_decode_step_amd.configs import DTYPE_BF16, SMALL
    ok = [tiny_cfg(), tiny_cfg(window=1), tiny_cfg(window=24), tiny_cfg(n_heads=1),
          tiny_cfg(n_layers=3, mem_groups=3, d_ffn=32)]
    for cfg in ok:
        assert binding.fused_supported(cfg), cfg
    # W = 32, or three layers at d_ffn = 64: 163 and 161 KiB with a chunk of 64 memory positions
    no = [tiny_cfg(dtype=DTYPE_BF16), tiny_cfg(window=32), tiny_cfg(window=64),
          tiny_cfg(n_layers=3, mem_groups=3, d_ffn=64), tiny_cfg(n_layers=3, mem_groups=3),
          tiny_cfg(d_model=64, n_heads=2), SMALL.model]
    for cfg in no:
        assert not binding.fused_supported(cfg), cfg
