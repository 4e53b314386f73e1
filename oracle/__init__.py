"""CPU oracle of the decode attention block: test infrastructure only.

Importable by the tests, by the package's smoke check and by the benchmark's
CPU-baseline leg; never by the library.  `decode_step` is the fp64 numpy
oracle of the attention block, `ffn_step` that of the FFN half of the layer,
`mla_step` that of multi-head latent attention decode over a latent
cache, `brute` their 50-digit scalar twins for tiny shapes.
"""
from .decode_step import (  # noqa: F401
    decode_step_fp64, decode_step_from_inputs, to_f64, round_to_storage,
    rms_norm, qkv_project, rope, rope_angles, append_kv, attention, softmax, out_project,
)
from .ffn_step import ffn_step_fp64, ffn_step_from_inputs, silu  # noqa: F401
from .mla_step import mla_attention, mla_decode_fp64, mla_decode_from_inputs  # noqa: F401
