"""CPU oracle of the int8 rowwise-quantized linear layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the library or its Python binding.
It shares no code with the HIP path.

Parity status: every function here is pinned by -m "not gpu" tests
(tests/test_oracle_formats.py, tests/test_oracle_layer.py) except
``mlp_forward_backward``'s comparison with the printed outputs of the
EasyDeL discussion #66 example, which is "parity unpinned": those numbers
come from JAX's random streams, Flax's initialiser and a different quantizer,
so they serve only as a magnitude check.
"""
from .formats import (bf16_bits_to_f64, f64_to_bf16_bits, from_f64, round_to_format, to_f64,
                      to_half, ulp)
from .layer import (dequant_weight, grad_bias, int_matmul, linear_backward_input,
                    linear_backward_input_int8, linear_backward_weight, linear_forward, mlp_forward_backward, outlier_columns,
                    page_bounds, quantize_rowwise, quantize_weight, quantize_weight_colwise, silu, silu_activation,
                    silu_grad, threshold_active)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "from_f64", "round_to_format", "to_f64", "to_half",
    "ulp", "dequant_weight", "grad_bias", "int_matmul", "linear_backward_input",
    "linear_backward_input_int8", "linear_backward_weight", "linear_forward", "mlp_forward_backward", "outlier_columns",
    "page_bounds", "quantize_rowwise", "quantize_weight", "quantize_weight_colwise", "silu", "silu_activation",
    "silu_grad", "threshold_active",
]
