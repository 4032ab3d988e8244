"""Model and workload configurations of the recurrent decoder step.

A model is fixed by (vocab V, d_model d, heads H, head_dim dh = d/H, decoder
layers L, FFN width F, window W, memory groups G, storage dtype).  G is 1
(one memory shared by every decoder layer) or L (one memory group per layer),
the two groupings the Recurrent Looped Transformer pages name in their
architecture paragraph.  The window W counts the current token, so at most
W - 1 history entries are carried to the next step.

The workloads are the five synthetic ones this library is tested and measured
on; their vocabularies for the 48-layer models are not given anywhere and are
read as 32768.
"""
from __future__ import annotations

from dataclasses import dataclass, field, asdict, replace

DTYPE_FP32 = 0
DTYPE_BF16 = 1
DTYPE_NAMES = {DTYPE_FP32: "f32", DTYPE_BF16: "bf16"}


@dataclass(frozen=True)
class ModelConfig:
    vocab: int
    d_model: int
    n_heads: int
    n_layers: int
    d_ffn: int
    window: int
    mem_groups: int
    dtype: int = DTYPE_BF16
    rms_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    def with_(self, **kw) -> "ModelConfig":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelConfig
    batch: int
    steps: int               # sequential decoder steps of the whole run
    prompt: int = 0          # prompt length (prefill part of `steps`)
    t_max: int = 0           # ragged positions t ~ U{1..t_max} (0: all start at t = 1)
    mem_capacity: int = 0    # encoder memory capacity T_cap (0: = steps)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def capacity(self) -> int:
        return self.mem_capacity or max(self.steps, self.t_max)


TINY = Workload(
    name="tiny-f32 (V=16,d=32,H=2,L=2,F=128,W=8,G=1,B=4,T=64)",
    model=ModelConfig(vocab=16, d_model=32, n_heads=2, n_layers=2, d_ffn=128,
                      window=8, mem_groups=1, dtype=DTYPE_FP32),
    batch=4, steps=64)

SMALL = Workload(
    name="small-bf16 (V=4096,d=512,H=8,L=12,F=2048,W=128,G=12,B=64,T=1024)",
    model=ModelConfig(vocab=4096, d_model=512, n_heads=8, n_layers=12, d_ffn=2048,
                      window=128, mem_groups=12, dtype=DTYPE_BF16),
    batch=64, steps=1024)

REFDEPTH = Workload(
    name="refdepth-bf16 (V=32768,d=2048,H=16,L=48,F=8192,W=512,G=1,B=32,T=2048+512)",
    model=ModelConfig(vocab=32768, d_model=2048, n_heads=16, n_layers=48, d_ffn=8192,
                      window=512, mem_groups=1, dtype=DTYPE_BF16),
    batch=32, steps=2560, prompt=2048)

LARGEBATCH = Workload(
    name="largebatch-bf16 (V=32768,d=2048,H=16,L=48,F=8192,W=1024,G=1,B=256,t~U[1,8192],1 step)",
    model=ModelConfig(vocab=32768, d_model=2048, n_heads=16, n_layers=48, d_ffn=8192,
                      window=1024, mem_groups=1, dtype=DTYPE_BF16),
    batch=256, steps=1, t_max=8192, mem_capacity=8192)

LONGCTX = Workload(
    name="longctx-bf16 (V=32768,d=4096,H=32,L=48,F=16384,W=4096,G=1,B=8,T=32768)",
    model=ModelConfig(vocab=32768, d_model=4096, n_heads=32, n_layers=48, d_ffn=16384,
                      window=4096, mem_groups=1, dtype=DTYPE_BF16),
    batch=8, steps=32768)

WORKLOADS = {"tiny": TINY, "small": SMALL, "refdepth": REFDEPTH,
             "largebatch": LARGEBATCH, "longctx": LONGCTX}
