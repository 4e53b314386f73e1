"""CPU oracle of the decode attention block: test infrastructure only.

Importable by the tests, by the package's smoke check and by the benchmark's
CPU-baseline leg; never by the library.  `decode_step` is the fp64 numpy
oracle, `brute` its 50-digit scalar twin for tiny shapes.
"""
from .decode_step import (  # noqa: F401
    decode_step_fp64, decode_step_from_inputs, to_f64, round_to_storage,
    rms_norm, qkv_project, rope, rope_angles, append_kv, attention, softmax, out_project,
)
