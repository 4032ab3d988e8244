"""Thin Python binding of librlt.so (ctypes).  Argument marshalling only:
torch supplies device memory and the current HIP stream; every step of the
decoder and the encoder runs in the library's HIP kernels.  The functions keep the C names
(rlt_decoder_step, rlt_run_sequence, ...); the classes wrap the handles.

Loading fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

from .configs import ModelConfig, DTYPE_BF16, DTYPE_FP32

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librlt.so")

RLT_OK, RLT_ERR_INVALID_ARG, RLT_ERR_SHAPE, RLT_ERR_RANGE, RLT_ERR_STALE, \
    RLT_ERR_CONVENTION, RLT_ERR_UNSUPPORTED, RLT_ERR_DEVICE = range(8)
RLT_LOGITS_ALL, RLT_LOGITS_LAST, RLT_LOGITS_NONE = 0, 1, 2
RLT_K_EXTRA, RLT_K_GEMM, RLT_K_SWA, RLT_K_CROSS = 0, 1, 2, 3
RLT_E_GEMM, RLT_E_ATTN, RLT_E_OTHER = 0, 1, 2
RLT_DETACH_S, RLT_DETACH_KV = 1, 2
ABI_VERSION = 4                      # include/rlt.h RLT_ABI_VERSION

EXPORTED = ("rlt_abi_version", "rlt_status_str", "rlt_last_error", "rlt_model_bytes",
            "rlt_model_create", "rlt_model_destroy", "rlt_state_bytes", "rlt_state_init",
            "rlt_state_destroy", "rlt_state_reset", "rlt_decoder_step", "rlt_decoder_step_noalloc",
            "rlt_run_sequence", "rlt_fused_supported", "rlt_run_sequence_fused",
            "rlt_persistent_workspace_bytes", "rlt_run_sequence_persistent",
            "rlt_persistent_check", "rlt_persistent_test_stall",
            "rlt_score_sequence", "rlt_generate", "rlt_generate_encoded",
            "rlt_state_position", "rlt_snapshot_bytes", "rlt_state_export", "rlt_state_import",
            "rlt_profile_begin", "rlt_profile_collect",
            "rlt_encoder_bytes", "rlt_encoder_create", "rlt_encoder_destroy",
            "rlt_encoder_state_bytes", "rlt_encoder_state_init", "rlt_encoder_state_destroy",
            "rlt_encoder_state_reset", "rlt_encoder_state_set_mode", "rlt_encoder_position", "rlt_encode",
            "rlt_encoder_profile_begin", "rlt_encoder_profile_collect",
            "rlt_encoder_snapshot_bytes", "rlt_encoder_state_export", "rlt_encoder_state_import",
            "rlt_bptt_workspace_bytes", "rlt_bptt_workspace_bytes_segmented", "rlt_bptt",
            "rlt_peak_bandwidth", "rlt_peak_mfma")


class RLTError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class rlt_config(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_layers", C.c_int32), ("d_ffn", C.c_int32),
                ("window", C.c_int32), ("mem_groups", C.c_int32), ("dtype", C.c_int32),
                ("rms_eps", C.c_float), ("attn_chunk", C.c_int32)]


class rlt_params(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("s_star", "wg", "bg", "g1", "g2", "g3", "wq", "wk",
                                          "wv", "wo", "wqc", "woc", "w1", "w2", "go", "wout")]


class rlt_memory(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("stride_group", C.c_int64),
                ("stride_seq", C.c_int64), ("stride_head", C.c_int64), ("stride_pos", C.c_int64),
                ("capacity", C.c_int32), ("n_seq", C.c_int32), ("n_groups", C.c_int32)]


class rlt_encoder_table(C.Structure):
    _fields_ = [("e", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p)]


class rlt_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("top_k", C.c_int32)]


class rlt_bptt_opts(C.Structure):
    _fields_ = [("chunk", C.c_int32), ("detach", C.c_int32), ("segment", C.c_int32)]


class rlt_encoder_params(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("emb", "ge", "wkm", "wvm")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load librlt.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"librlt.so not found at {path}: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    vp, i32, u64, sz = C.c_void_p, C.c_int32, C.c_uint64, C.c_size_t
    P = C.POINTER
    sig = {
        "rlt_abi_version": (i32, []),
        "rlt_status_str": (C.c_char_p, [i32]),
        "rlt_last_error": (C.c_char_p, []),
        "rlt_model_bytes": (sz, [P(rlt_config)]),
        "rlt_model_create": (i32, [P(rlt_config), P(rlt_params), u64, vp, sz, vp, P(vp)]),
        "rlt_model_destroy": (None, [vp]),
        "rlt_state_bytes": (sz, [P(rlt_config), i32, i32]),
        "rlt_state_init": (i32, [vp, i32, i32, vp, sz, vp, P(vp)]),
        "rlt_state_destroy": (None, [vp]),
        "rlt_state_reset": (i32, [vp, vp, i32, P(i32), vp]),
        "rlt_decoder_step": (i32, [vp, vp, i32, P(i32), vp, P(rlt_memory), vp, vp]),
        "rlt_decoder_step_noalloc": (i32, [vp, vp, i32, P(i32), vp, P(rlt_memory), vp, vp]),
        "rlt_run_sequence": (i32, [vp, vp, i32, vp, P(rlt_memory), vp, i32, vp]),
        "rlt_fused_supported": (i32, [P(rlt_config)]),
        "rlt_run_sequence_fused": (i32, [vp, vp, i32, vp, P(rlt_memory), vp, i32, vp]),
        "rlt_persistent_workspace_bytes": (sz, [P(rlt_config), i32]),
        "rlt_run_sequence_persistent": (i32, [vp, vp, i32, vp, P(rlt_memory), vp, i32, vp, sz, vp]),
        "rlt_persistent_check": (i32, [vp, vp]),
        "rlt_persistent_test_stall": (None, [i32]),
        "rlt_score_sequence": (i32, [vp, vp, i32, vp, P(rlt_memory), vp, vp, vp]),
        "rlt_generate_encoded": (i32, [vp, vp, i32, vp, vp, vp, P(rlt_memory), P(rlt_sampling),
                                       vp, vp, vp, vp, vp]),
        "rlt_generate": (i32, [vp, vp, i32, vp, P(rlt_encoder_table), P(rlt_memory), P(rlt_sampling),
                               vp, vp, vp, vp, vp]),
        "rlt_state_position": (i32, [vp, i32]),
        "rlt_snapshot_bytes": (sz, [P(rlt_config), i32]),
        "rlt_state_export": (i32, [vp, vp, i32, P(i32), vp, vp]),
        "rlt_state_import": (i32, [vp, vp, i32, P(i32), vp, vp]),
        "rlt_profile_begin": (i32, [vp, i32, i32, i32]),
        "rlt_profile_collect": (i32, [vp, i32, P(C.c_double), P(i32), P(C.c_double)]),
        "rlt_encoder_bytes": (sz, [vp]),
        "rlt_encoder_create": (i32, [vp, P(rlt_encoder_params), vp, sz, vp, P(vp)]),
        "rlt_encoder_destroy": (None, [vp]),
        "rlt_encoder_state_bytes": (sz, [P(rlt_config), i32, i32, i32]),
        "rlt_encoder_state_init": (i32, [vp, i32, i32, i32, vp, sz, P(vp)]),
        "rlt_encoder_state_destroy": (None, [vp]),
        "rlt_encoder_state_reset": (i32, [vp, i32, P(i32)]),
        "rlt_encoder_state_set_mode": (i32, [vp, i32]),
        "rlt_encoder_position": (i32, [vp, i32]),
        "rlt_encode": (i32, [vp, vp, i32, P(i32), i32, vp, vp, P(rlt_memory), vp]),
        "rlt_encoder_profile_begin": (i32, [vp, i32, i32]),
        "rlt_encoder_snapshot_bytes": (sz, [P(rlt_config), i32, i32]),
        "rlt_encoder_state_export": (i32, [vp, vp, i32, P(i32), i32, vp, vp]),
        "rlt_encoder_state_import": (i32, [vp, vp, i32, P(i32), i32, vp, vp]),
        "rlt_encoder_profile_collect": (i32, [vp, i32, P(C.c_double), P(i32), P(C.c_double),
                                              P(C.c_double)]),
        "rlt_bptt_workspace_bytes": (sz, [P(rlt_config), i32, i32]),
        "rlt_bptt_workspace_bytes_segmented": (sz, [P(rlt_config), i32, i32, i32]),
        "rlt_peak_bandwidth": (i32, [vp, vp, sz, i32, i32, P(C.c_double), vp]),
        "rlt_peak_mfma": (i32, [i32, i32, i32, vp, sz, P(C.c_double), vp]),
        "rlt_bptt": (i32, [P(rlt_config), P(rlt_params), i32, i32, vp, P(rlt_memory), vp,
                           P(rlt_bptt_opts), P(rlt_params), vp, P(rlt_memory), vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.rlt_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.rlt_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild the library")
    _lib = lib
    return lib


def _check(status: int):
    if status != RLT_OK:
        lib = load_library()
        raise RLTError(status, f"{lib.rlt_status_str(status).decode()}: "
                               f"{lib.rlt_last_error().decode()}")


def make_config(cfg: ModelConfig, attn_chunk: int = 0) -> rlt_config:
    return rlt_config(cfg.vocab, cfg.d_model, cfg.n_heads, cfg.head_dim, cfg.n_layers, cfg.d_ffn,
                      cfg.window, cfg.mem_groups, cfg.dtype, cfg.rms_eps, attn_chunk)


def _stream(stream=None) -> C.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _slots_arg(slots):
    if slots is None:
        return None, None
    arr = (C.c_int32 * len(slots))(*[int(s) for s in slots])
    return arr, len(slots)


def memory_view(k: torch.Tensor, v: torch.Tensor) -> rlt_memory:
    """rlt_memory over K, V tensors shaped [G][S][H][T][dh] (dh contiguous)."""
    if k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("K and V must have the same shape and strides")
    if k.stride(-1) != 1:
        raise ValueError("head_dim must be contiguous")
    sg, ss, sh, sp, _ = k.stride()
    return rlt_memory(k.data_ptr(), v.data_ptr(), sg, ss, sh, sp, k.shape[3], k.shape[1],
                      k.shape[0])


class Model:
    """Packed weights on the device (rlt_model_create)."""

    def __init__(self, cfg: ModelConfig, params: dict, version: int = 1, attn_chunk: int = 0,
                 stream=None):
        lib = load_library()
        self.cfg = cfg
        self.ccfg = make_config(cfg, attn_chunk)
        self.version = version
        nbytes = lib.rlt_model_bytes(C.byref(self.ccfg))
        if nbytes == 0:
            _check(RLT_ERR_INVALID_ARG)
        dev = torch.device("cuda", torch.cuda.current_device())
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        keep = {}
        sd = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
        for name in rlt_params._fields_:
            key = name[0]
            t = params[key]
            want = torch.float32 if key in ("s_star", "bg", "g1", "g2", "g3", "go") else sd
            keep[key] = t.to(device=dev, dtype=want).contiguous()
        p = rlt_params(*[keep[n[0]].data_ptr() for n in rlt_params._fields_])
        h = C.c_void_p()
        _check(lib.rlt_model_create(C.byref(self.ccfg), C.byref(p), version, self.buf.data_ptr(),
                                    nbytes, _stream(stream), C.byref(h)))
        self.handle = h
        # the canonical tensors are read by kernels already enqueued
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        del keep

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_model_destroy(self.handle)
            self.handle = None


class State:
    """Decoder states of `batch` slots (rlt_state_init)."""

    def __init__(self, model: Model, batch: int, max_tokens: int, stream=None):
        lib = load_library()
        self.model = model
        self.batch = batch
        self.max_tokens = max_tokens
        nbytes = lib.rlt_state_bytes(C.byref(model.ccfg), batch, max_tokens)
        if nbytes == 0:
            _check(RLT_ERR_INVALID_ARG)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=model.buf.device)
        h = C.c_void_p()
        _check(lib.rlt_state_init(model.handle, batch, max_tokens, self.buf.data_ptr(), nbytes,
                                  _stream(stream), C.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_state_destroy(self.handle)
            self.handle = None

    def position(self, slot: int) -> int:
        return load_library().rlt_state_position(self.handle, slot)


def rlt_decoder_step(model: Model, state: State, e: torch.Tensor, memory, logits=None,
                     slots=None, want_logits=True, stream=None):
    """One step for the rows of e ([n][d]); returns logits [n][V] fp32 (or None)."""
    lib = load_library()
    n = e.shape[0]
    if e.stride(-1) != 1 or e.stride(0) != e.shape[1]:
        e = e.contiguous()
    if logits is None and want_logits:
        logits = torch.empty((n, model.cfg.vocab), dtype=torch.float32, device=e.device)
    arr, _ = _slots_arg(slots)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_decoder_step(model.handle, state.handle, n, arr, e.data_ptr(), C.byref(mem),
                                logits.data_ptr() if logits is not None else None,
                                _stream(stream)))
    return logits


def rlt_decoder_step_noalloc(model: Model, state: State, e: torch.Tensor, memory, logits,
                             slots=None, stream=None):
    """rlt_decoder_step with the per-step working memory in the library's
    static per-device array: nothing is allocated here or in the library, so
    the caller passes the logits buffer ([n][V] fp32, or None for no logits)
    and e as a contiguous [n][d] tensor."""
    lib = load_library()
    n = e.shape[0]
    if e.stride(-1) != 1 or e.stride(0) != e.shape[1]:
        raise ValueError("e must be a contiguous [n][d] tensor")
    arr, _ = _slots_arg(slots)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_decoder_step_noalloc(model.handle, state.handle, n, arr, e.data_ptr(),
                                        C.byref(mem),
                                        logits.data_ptr() if logits is not None else None,
                                        _stream(stream)))
    return logits


def rlt_run_sequence(model: Model, state: State, e: torch.Tensor, memory,
                     logits_mode: int = RLT_LOGITS_ALL, logits=None, stream=None):
    """T steps for all slots, e [B][T][d]; returns logits per logits_mode."""
    lib = load_library()
    B, T = e.shape[0], e.shape[1]
    e = e.contiguous()
    if logits is None and logits_mode != RLT_LOGITS_NONE:
        shape = (B, T, model.cfg.vocab) if logits_mode == RLT_LOGITS_ALL else (B, model.cfg.vocab)
        logits = torch.empty(shape, dtype=torch.float32, device=e.device)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_run_sequence(model.handle, state.handle, T, e.data_ptr(), C.byref(mem),
                                logits.data_ptr() if logits is not None else None, logits_mode,
                                _stream(stream)))
    return logits


def fused_supported(cfg) -> bool:
    """Whether rlt_run_sequence_fused takes models of this configuration."""
    return bool(load_library().rlt_fused_supported(C.byref(make_config(cfg, 0))))


def rlt_run_sequence_fused(model: Model, state: State, e: torch.Tensor, memory,
                           logits_mode: int = RLT_LOGITS_ALL, logits=None, stream=None):
    """rlt_run_sequence as one launch (one workgroup per slot, weights in LDS;
    small fp32 models); same arguments and logits."""
    lib = load_library()
    B, T = e.shape[0], e.shape[1]
    e = e.contiguous()
    if logits is None and logits_mode != RLT_LOGITS_NONE:
        shape = (B, T, model.cfg.vocab) if logits_mode == RLT_LOGITS_ALL else (B, model.cfg.vocab)
        logits = torch.empty(shape, dtype=torch.float32, device=e.device)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_run_sequence_fused(model.handle, state.handle, T, e.data_ptr(), C.byref(mem),
                                      logits.data_ptr() if logits is not None else None,
                                      logits_mode, _stream(stream)))
    return logits


class StepWorkspace:
    """Device workspace of rlt_run_sequence_persistent for a state of `batch` slots."""

    def __init__(self, model: Model, batch: int):
        lib = load_library()
        nbytes = lib.rlt_persistent_workspace_bytes(C.byref(model.ccfg), batch)
        if nbytes == 0:
            _check(RLT_ERR_INVALID_ARG)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=model.buf.device)


def rlt_run_sequence_persistent(model: Model, state: State, e: torch.Tensor, memory,
                                workspace: StepWorkspace, logits_mode: int = RLT_LOGITS_ALL,
                                logits=None, stream=None):
    """rlt_run_sequence with one persistent launch per step; e [B][T][d]."""
    lib = load_library()
    B, T = e.shape[0], e.shape[1]
    e = e.contiguous()
    if logits is None and logits_mode != RLT_LOGITS_NONE:
        shape = (B, T, model.cfg.vocab) if logits_mode == RLT_LOGITS_ALL else (B, model.cfg.vocab)
        logits = torch.empty(shape, dtype=torch.float32, device=e.device)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_run_sequence_persistent(
        model.handle, state.handle, T, e.data_ptr(), C.byref(mem),
        logits.data_ptr() if logits is not None else None, logits_mode,
        workspace.buf.data_ptr(), workspace.buf.numel(), _stream(stream)))
    return logits


def rlt_persistent_check(workspace: StepWorkspace, stream=None):
    """Raises RLTError(RLT_ERR_DEVICE) if a wait of the last persistent call timed out."""
    _check(load_library().rlt_persistent_check(workspace.buf.data_ptr(), _stream(stream)))


def rlt_persistent_test_stall(on: bool):
    """Tests of the time-out path only: while on, every wait of later
    persistent calls looks for an epoch no item stores (see include/rlt.h)."""
    load_library().rlt_persistent_test_stall(1 if on else 0)


def rlt_score_sequence(model: Model, state: State, e: torch.Tensor, memory, tokens: torch.Tensor,
                       out=None, stream=None) -> torch.Tensor:
    """Replay scoring over T steps of all B slots: e [B][T][d], tokens [B][T]
    int32 (the token consumed at step t + 1; < 0: not scored) -> log-probs
    [B][T] fp32."""
    lib = load_library()
    B, T = e.shape[0], e.shape[1]
    e = e.contiguous()
    tokens = tokens.to(dtype=torch.int32).contiguous()
    if tokens.shape != (B, T):
        raise ValueError("tokens must be [B][T]")
    if out is None:
        out = torch.empty((B, T), dtype=torch.float32, device=e.device)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_score_sequence(model.handle, state.handle, T, e.data_ptr(), C.byref(mem),
                                  tokens.data_ptr(), out.data_ptr(), _stream(stream)))
    return out


def rlt_generate(model: Model, state: State, logits0: torch.Tensor, table_e: torch.Tensor,
                 table_k: torch.Tensor, table_v: torch.Tensor, memory, temperature: float,
                 top_k: int, u: torch.Tensor, stream=None):
    """Generate u.shape[1] tokens for all B slots from the preceding logits
    logits0 [B][V]; stand-in encoder tables e [V][d], k/v [G][V][H][dh];
    memory (K, V) [G][B][H][T][dh] tensors whose entries at the generated
    positions are written.  Returns (tokens [B][n] int32, log-probs [B][n]
    fp32, logits of the last step [B][V] fp32)."""
    lib = load_library()
    B, n = u.shape
    u = u.to(dtype=torch.float32).contiguous()
    logits0 = logits0.to(dtype=torch.float32).contiguous()
    dev = u.device
    tokens = torch.empty((B, n), dtype=torch.int32, device=dev)
    lp = torch.empty((B, n), dtype=torch.float32, device=dev)
    last = torch.empty((B, model.cfg.vocab), dtype=torch.float32, device=dev)
    enc = rlt_encoder_table(table_e.data_ptr(), table_k.data_ptr(), table_v.data_ptr())
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    smp = rlt_sampling(float(temperature), int(top_k))
    _check(lib.rlt_generate(model.handle, state.handle, n, logits0.data_ptr(), C.byref(enc),
                            C.byref(mem), C.byref(smp), u.data_ptr(), tokens.data_ptr(),
                            lp.data_ptr(), last.data_ptr(), _stream(stream)))
    return tokens, lp, last


def rlt_state_reset(model: Model, state: State, slots, stream=None):
    arr, n = _slots_arg(slots)
    _check(load_library().rlt_state_reset(model.handle, state.handle, n, arr, _stream(stream)))


def snapshot_bytes(model: Model, n: int) -> int:
    return load_library().rlt_snapshot_bytes(C.byref(model.ccfg), n)


def rlt_state_export(model: Model, state: State, slots, stream=None) -> torch.Tensor:
    lib = load_library()
    arr, n = _slots_arg(slots)
    snap = torch.empty(snapshot_bytes(model, n), dtype=torch.uint8, device=model.buf.device)
    _check(lib.rlt_state_export(model.handle, state.handle, n, arr, snap.data_ptr(),
                                _stream(stream)))
    return snap


def rlt_state_import(model: Model, state: State, snap: torch.Tensor, slots, stream=None):
    arr, n = _slots_arg(slots)
    _check(load_library().rlt_state_import(model.handle, state.handle, n, arr, snap.data_ptr(),
                                           _stream(stream)))


def snapshot_layout(cfg: ModelConfig):
    """(record bytes, offset of s, offset of K, offset of V) of one snapshot record."""
    es = 2 if cfg.dtype == DTYPE_BF16 else 4
    a256 = lambda x: (x + 255) // 256 * 256
    hist = cfg.n_layers * cfg.n_heads * (cfg.window - 1) * cfg.head_dim * es
    off_s = 256
    off_k = off_s + a256(cfg.d_model * 4)
    off_v = off_k + a256(hist)
    return off_v + a256(hist), off_s, off_k, off_v


def build_snapshot(cfg: ModelConfig, records, version: int, device) -> torch.Tensor:
    """Write snapshot records (the library's documented format) from
    {'pos', 's' [d], 'K'/'V' [L][H][n_hist][dh]} dicts."""
    rec, off_s, off_k, off_v = snapshot_layout(cfg)
    out = torch.zeros(rec * len(records), dtype=torch.uint8, device=device)
    sd = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
    L, H, dh, Wm1 = cfg.n_layers, cfg.n_heads, cfg.head_dim, cfg.window - 1
    for r, st in enumerate(records):
        base = r * rec
        hdr = torch.tensor([0x534C5452, 1], dtype=torch.int64).to(torch.int32)
        ints = torch.tensor([cfg.d_model, H, dh, L, cfg.window, cfg.dtype, int(st["pos"]), 0],
                            dtype=torch.int32)
        head = torch.cat([hdr.view(torch.uint8), ints.view(torch.uint8),
                          torch.tensor([version], dtype=torch.int64).view(torch.uint8)])
        out[base:base + head.numel()] = head.to(device)
        s = st["s"].to(device=device, dtype=torch.float32).contiguous()
        out[base + off_s: base + off_s + s.numel() * 4] = s.view(torch.uint8)
        n_hist = st["K"].shape[2]
        if Wm1 > 0 and n_hist > 0:
            for key, off in (("K", off_k), ("V", off_v)):
                full = torch.zeros((L, H, Wm1, dh), dtype=sd, device=device)
                full[:, :, :n_hist] = st[key].to(device=device, dtype=sd)
                b = full.contiguous().view(torch.uint8).reshape(-1)
                out[base + off: base + off + b.numel()] = b
    return out


def profile_begin(state: State, class_mask: int, max_launches: int, step_stride: int = 1):
    """Record launches of the kernel classes in class_mask (bit 1 << RLT_K_*)."""
    _check(load_library().rlt_profile_begin(state.handle, class_mask, max_launches, step_stride))


def profile_collect(state: State, kclass: int):
    """(total ms, launches, algorithmic bytes) recorded for one kernel class."""
    tot, n, b = C.c_double(), C.c_int32(), C.c_double()
    _check(load_library().rlt_profile_collect(state.handle, kclass, C.byref(tot), C.byref(n),
                                              C.byref(b)))
    return tot.value, n.value, b.value


# ---------------------------------------------------------------- encoder
class Encoder:
    """Encoder-only weights on the device (rlt_encoder_create); the layer
    weights are the model's (tied)."""

    def __init__(self, model: Model, params: dict, stream=None):
        lib = load_library()
        self.model = model
        cfg = model.cfg
        nbytes = lib.rlt_encoder_bytes(model.handle)
        if nbytes == 0:
            _check(RLT_ERR_UNSUPPORTED)
        dev = model.buf.device
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        sd = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
        keep = {k: params[k].to(device=dev, dtype=torch.float32 if k == "ge" else sd).contiguous()
                for k in ("emb", "ge", "wkm", "wvm")}
        p = rlt_encoder_params(*[keep[n[0]].data_ptr() for n in rlt_encoder_params._fields_])
        h = C.c_void_p()
        _check(lib.rlt_encoder_create(model.handle, C.byref(p), self.buf.data_ptr(), nbytes,
                                      _stream(stream), C.byref(h)))
        self.handle = h
        torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
        del keep

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_encoder_destroy(self.handle)
            self.handle = None


class EncoderState:
    """Encoder cache and scratch of `batch` slots (rlt_encoder_state_init)."""

    def __init__(self, encoder: Encoder, batch: int, max_tokens: int, max_rows: int):
        lib = load_library()
        self.encoder = encoder
        self.batch = batch
        self.max_tokens = max_tokens
        self.max_rows = max_rows
        nbytes = lib.rlt_encoder_state_bytes(C.byref(encoder.model.ccfg), batch, max_tokens,
                                             max_rows)
        if nbytes == 0:
            _check(RLT_ERR_INVALID_ARG)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=encoder.buf.device)
        h = C.c_void_p()
        _check(lib.rlt_encoder_state_init(encoder.handle, batch, max_tokens, max_rows,
                                          self.buf.data_ptr(), nbytes, C.byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.rlt_encoder_state_destroy(self.handle)
            self.handle = None

    def position(self, slot: int) -> int:
        return load_library().rlt_encoder_position(self.handle, slot)

    def cache(self):
        """Views (K, V) of the encoder cache, [L][B][H][max_tokens][dh]."""
        cfg = self.encoder.model.cfg
        sd = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
        shape = (cfg.n_layers, self.batch, cfg.n_heads, self.max_tokens, cfg.head_dim)
        n = 1
        for v in shape:
            n *= v
        flat = self.buf.view(sd)
        return flat[:n].view(shape), flat[_align_elems(n, sd):][:n].view(shape)


def _align_elems(n: int, dtype) -> int:
    es = 2 if dtype == torch.bfloat16 else 4
    return ((n * es + 255) // 256 * 256) // es


RLT_ENC_EXACT, RLT_ENC_FAST = 0, 1


def rlt_encoder_state_set_mode(es: EncoderState, mode: int):
    """Kernel forms of the state's short calls: RLT_ENC_EXACT (bitwise the
    prompt kernels' arithmetic) or RLT_ENC_FAST (the decoder's forms)."""
    _check(load_library().rlt_encoder_state_set_mode(es.handle, int(mode)))


def rlt_encoder_state_reset(es: EncoderState, slots):
    arr, n = _slots_arg(slots)
    _check(load_library().rlt_encoder_state_reset(es.handle, n, arr))


def rlt_encode(encoder: Encoder, es: EncoderState, tokens: torch.Tensor, memory, slots=None,
               e_out=None, want_e=True, stream=None):
    """Encode the next T tokens of each listed slot: tokens [n][T] int32 on the
    device; memory (K, V) [G][S][H][cap][dh] tensors (entries written).
    Returns e [n][T][d] in the model dtype (None with want_e=False)."""
    lib = load_library()
    cfg = encoder.model.cfg
    tokens = tokens.to(dtype=torch.int32).contiguous()
    n, T = tokens.shape
    if e_out is None and want_e:
        sd = torch.bfloat16 if cfg.dtype == DTYPE_BF16 else torch.float32
        e_out = torch.empty((n, T, cfg.d_model), dtype=sd, device=tokens.device)
    arr, _ = _slots_arg(slots)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    _check(lib.rlt_encode(encoder.handle, es.handle, n, arr, T, tokens.data_ptr(),
                          e_out.data_ptr() if e_out is not None else None, C.byref(mem),
                          _stream(stream)))
    return e_out


def encoder_profile_begin(es: EncoderState, class_mask: int, max_launches: int):
    """Record launches of the encoder kernel classes in class_mask (bit 1 << RLT_E_*)."""
    _check(load_library().rlt_encoder_profile_begin(es.handle, class_mask, max_launches))


def encoder_profile_collect(es: EncoderState, kclass: int):
    """(total ms, launches, algorithmic FLOPs, algorithmic bytes) of one encoder kernel class."""
    tot, n, fl, b = C.c_double(), C.c_int32(), C.c_double(), C.c_double()
    _check(load_library().rlt_encoder_profile_collect(es.handle, kclass, C.byref(tot), C.byref(n),
                                                      C.byref(fl), C.byref(b)))
    return tot.value, n.value, fl.value, b.value


# ---------------------------------------------------------------- training
PARAM_NAMES = tuple(n for n, _ in rlt_params._fields_)


def rlt_bptt(cfg: ModelConfig, params: dict, e: torch.Tensor, memory, targets: torch.Tensor,
             chunk: int = 0, detach: int = 0, want_de: bool = True, want_dmem: bool = True,
             workspace=None, stream=None, segment: int = 0):
    """Backpropagation through time over e [B][T][d] (fp32 model): returns
    (loss tensor [1], {name: gradient}, de [B][T][d] or None, (dmk, dmv) or None).
    params: canonical fp32 tensors; memory: (K, V) [G][B][H][cap][dh] fp32."""
    lib = load_library()
    if cfg.dtype != DTYPE_FP32:
        _check(RLT_ERR_UNSUPPORTED)
    ccfg = make_config(cfg)
    B, T = e.shape[0], e.shape[1]
    dev = e.device
    e = e.to(torch.float32).contiguous()
    tg = targets.to(device=dev, dtype=torch.int32).contiguous()
    P = {k: params[k].to(device=dev, dtype=torch.float32).contiguous() for k in PARAM_NAMES}
    grads = {k: torch.empty_like(P[k]) for k in PARAM_NAMES}
    cp = rlt_params(*[P[k].data_ptr() for k in PARAM_NAMES])
    cg = rlt_params(*[grads[k].data_ptr() for k in PARAM_NAMES])
    mk, mv = memory
    mem = memory_view(mk, mv)
    dmem = None
    dm = None
    if want_dmem:
        # the library takes the gradients with the memory's strides
        dm = tuple(torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device).zero_()
                   for t in (mk, mv))
        dmem = memory_view(*dm)
    de = torch.empty_like(e) if want_de else None
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    nbytes = lib.rlt_bptt_workspace_bytes_segmented(C.byref(ccfg), B, T, int(segment))
    if nbytes == 0:
        _check(RLT_ERR_INVALID_ARG)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    opts = rlt_bptt_opts(int(chunk), int(detach), int(segment))
    _check(lib.rlt_bptt(C.byref(ccfg), C.byref(cp), B, T, e.data_ptr(), C.byref(mem), tg.data_ptr(),
                        C.byref(opts), C.byref(cg), de.data_ptr() if de is not None else None,
                        C.byref(dmem) if dmem is not None else None, loss.data_ptr(),
                        workspace.data_ptr(), nbytes, _stream(stream)))
    return loss, grads, de, dm


def peak_bandwidth(src: torch.Tensor, dst: torch.Tensor, copy: bool, reps: int = 5,
                   stream=None) -> float:
    """GB/s of a streaming read (copy False) or copy of src's bytes (rlt_peak_bandwidth)."""
    out = C.c_double(0.0)
    _check(load_library().rlt_peak_bandwidth(src.data_ptr(), dst.data_ptr(),
                                             src.numel() * src.element_size(), 1 if copy else 0,
                                             reps, C.byref(out), _stream(stream)))
    return out.value


def peak_mfma(shape: int, iters: int, sink: torch.Tensor, reps: int = 5, stream=None) -> float:
    """TFLOP/s of a dense bf16 MFMA loop: shape 0 = 32x32x16, 1 = 16x16x32 (rlt_peak_mfma)."""
    out = C.c_double(0.0)
    _check(load_library().rlt_peak_mfma(shape, iters, reps, sink.data_ptr(),
                                        sink.numel() * sink.element_size(), C.byref(out),
                                        _stream(stream)))
    return out.value


def rlt_generate_encoded(model: Model, state: State, logits0: torch.Tensor, encoder: "Encoder",
                         enc_state: "EncoderState", memory, temperature: float, top_k: int,
                         u: torch.Tensor, stream=None):
    """Generate u.shape[1] tokens for all B slots with the causal encoder in
    the loop (rlt_generate_encoded): each sampled token is encoded from the
    encoder cache of its slot's earlier tokens.  The encoder state must have
    as many tokens encoded per slot as the decoder state has consumed.
    Returns (tokens [B][n] int32, log-probs [B][n] fp32, last logits [B][V])."""
    lib = load_library()
    B, n = u.shape
    u = u.to(dtype=torch.float32).contiguous()
    logits0 = logits0.to(dtype=torch.float32).contiguous()
    dev = u.device
    tokens = torch.empty((B, n), dtype=torch.int32, device=dev)
    lp = torch.empty((B, n), dtype=torch.float32, device=dev)
    last = torch.empty((B, model.cfg.vocab), dtype=torch.float32, device=dev)
    mem = memory if isinstance(memory, rlt_memory) else memory_view(*memory)
    smp = rlt_sampling(float(temperature), int(top_k))
    _check(lib.rlt_generate_encoded(model.handle, state.handle, n, logits0.data_ptr(),
                                    encoder.handle, enc_state.handle, C.byref(mem), C.byref(smp),
                                    u.data_ptr(), tokens.data_ptr(), lp.data_ptr(), last.data_ptr(),
                                    _stream(stream)))
    return tokens, lp, last


def encoder_snapshot_bytes(cfg: ModelConfig, capacity: int, n: int) -> int:
    return load_library().rlt_encoder_snapshot_bytes(C.byref(make_config(cfg)), capacity, n)


def rlt_encoder_state_export(encoder: "Encoder", es: "EncoderState", slots, capacity: int,
                             stream=None) -> torch.Tensor:
    """Encoder-cache records of the listed slots (rlt_encoder_state_export),
    `capacity` positions each; returns a uint8 device tensor."""
    lib = load_library()
    arr, n = _slots_arg(slots)
    nbytes = encoder_snapshot_bytes(encoder.model.cfg, capacity, n)
    snap = torch.empty(nbytes, dtype=torch.uint8, device=encoder.buf.device)
    _check(lib.rlt_encoder_state_export(encoder.handle, es.handle, n, arr, capacity,
                                        snap.data_ptr(), _stream(stream)))
    return snap


def rlt_encoder_state_import(encoder: "Encoder", es: "EncoderState", snap: torch.Tensor, slots,
                             capacity: int, stream=None):
    """Record i of snap into slot slots[i] (rlt_encoder_state_import)."""
    lib = load_library()
    arr, n = _slots_arg(slots)
    _check(lib.rlt_encoder_state_import(encoder.handle, es.handle, n, arr, capacity,
                                        snap.data_ptr(), _stream(stream)))
