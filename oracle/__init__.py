"""CPU oracle of the recurrent decoder step and the causal encoder (test
infrastructure only).

Only the test suite, the smoke check of the package entry file and the
benchmark's CPU-baseline leg may import anything from this package.  The HIP
library and its Python binding never do, and this package imports neither.
"""
from .rlt_oracle import (Model, SeqState, round_bf16, initial_state, state_from_arrays,
                         copy_state, decoder_step, run_sequence, token_log_prob, score_sequence,
                         sampling_weights, sample_token, generate)
from .brute import brute_force_run
from .encoder import Encoder, encode, prefill, generate_encoded
from . import bptt
from .parallel import parallel_swa_pass

__all__ = ["Model", "SeqState", "round_bf16", "initial_state", "state_from_arrays",
           "copy_state", "decoder_step", "run_sequence", "token_log_prob", "score_sequence",
           "sampling_weights", "sample_token", "generate",
           "brute_force_run", "Encoder", "encode", "prefill", "generate_encoded", "bptt",
           "parallel_swa_pass"]
