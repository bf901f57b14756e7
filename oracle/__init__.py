"""CPU oracle of the convrot int8 linear layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package. See convrot_ref.py for the definitions it follows.
"""

from .convrot_ref import *  # noqa: F401,F403
from .convrot_ref import (  # noqa: F401
    bf16_to_f64, block_rotation, dequant_derotate, dequant_linear_reference_f64,
    dequant_reference_f64, derotation_integers, epilogue, f32_to_bf16, gemm_int32, hadamard,
    linear_int8, linear_int8_reference_f64, quantize_activations, quantize_weights,
    quantize_weights_per_channel, f16_to_f64, f32_to_f16, to_f64, from_f32,
    quantize_with_amax, rel_frobenius, rotate_rows, rotation_matrix, rotation_signs,
    round_exact_to_f32, splitmix64,
)
